"""Pins of the windowed-softmax oracle (Video DeltaNet's softmax branch).

FreeVideo page, section "Where Video DeltaNet comes in": each query chunk of
five latent frames sees itself and its two neighbouring chunks (a 15-frame
window); every frame sees the first and last latent frames, which see every
frame.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import attention as A
from test_oracle_pins import bf16_array


def brute_allowed(F, chunk, nb):
    """Pure-Python restatement: one boolean per (query frame, key frame)."""
    out = [[False] * F for _ in range(F)]
    for qf in range(F):
        for kf in range(F):
            near = abs(qf // chunk - kf // chunk) <= nb
            anchor = kf in (0, F - 1) or qf in (0, F - 1)
            out[qf][kf] = near or anchor
    return np.array(out, dtype=bool)


def check_frames_allowed(fn):
    for F in [1, 2, 3, 7, 12, 42, 72, 102]:
        for chunk, nb in [(5, 1), (5, 0), (3, 2), (1, 1)]:
            assert np.array_equal(fn(F, chunk, nb), brute_allowed(F, chunk, nb)), (F, chunk, nb)


def check_fifteen_frame_window(fn):
    # an interior chunk's frame sees 3 chunks x 5 frames = 15 frames of window
    # plus the two anchors; the anchors see every frame
    F = 72
    a = fn(F, 5, 1)
    for qf in range(10, 60):
        window = [kf for kf in range(F) if abs(kf // 5 - qf // 5) <= 1]
        assert len(window) == 15
        assert a[qf].sum() == 17
    assert a[0].all() and a[F - 1].all()
    assert a[:, 0].all() and a[:, F - 1].all()


def brute_tiles(N, ft, chunk, nb):
    F = -(-N // ft)
    allowed = brute_allowed(F, chunk, nb)
    T = -(-N // 128)
    lists = []
    for t in range(T):
        s = set()
        for i in range(t * 128, min(t * 128 + 128, N)):
            for j in range(N):
                if allowed[i // ft][j // ft]:
                    s.add(j // 128)
        lists.append(sorted(s))
    return lists


def check_window_tiles(fn):
    for N, ft, chunk, nb in [(1000, 64, 2, 1), (900, 100, 3, 1), (1300, 130, 2, 0), (128, 128, 5, 1)]:
        idx, count = fn(N, ft, chunk, nb)
        want = brute_tiles(N, ft, chunk, nb)
        assert len(count) == len(want)
        for t, w in enumerate(want):
            assert count[t] == len(w)
            assert list(idx[t, :count[t]]) == w
            assert np.all(idx[t, count[t]:] == -1)


def check_window_attention(fn):
    H, N, d, ft = 2, 700, 16, 64
    q, k, v = (bf16_array((H, N, d), 90 + t) for t in range(3))
    scale = 0.25
    F = -(-N // ft)
    # full window (every chunk a neighbour) is plain dense attention
    full = fn(q, k, v, scale, ft, 2, F)
    np.testing.assert_allclose(full, oracle.dense(q, k, v, scale), rtol=0, atol=1e-14)
    # brute force over the explicitly gathered keys
    out = fn(q, k, v, scale, ft, 2, 1)
    allowed = brute_allowed(F, 2, 1)
    for i in [0, 5, 63, 64, 200, 333, 640, 699]:
        keys = [j for j in range(N) if allowed[i // ft][j // ft]]
        for h in range(H):
            s = [scale * float(q[h, i] @ k[h, j]) for j in keys]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            want = sum(pj * v[h, j] for pj, j in zip(p, keys)) / sum(p)
            np.testing.assert_allclose(out[h, i], want, rtol=0, atol=1e-12)
    # Q = 0: the mean of V over the allowed keys
    z = fn(np.zeros_like(q), k, v, scale, ft, 2, 1)
    for i in [3, 300, 699]:
        keys = [j for j in range(N) if allowed[i // ft][j // ft]]
        np.testing.assert_allclose(z[:, i], v[:, keys].mean(axis=1), atol=1e-13)


def test_frames_allowed_brute_force():
    check_frames_allowed(oracle.window_frames_allowed)


def test_fifteen_frame_window_and_anchors():
    check_fifteen_frame_window(oracle.window_frames_allowed)


def test_window_tiles_brute_force():
    check_window_tiles(oracle.window_tiles)


def test_window_attention_pins():
    check_window_attention(oracle.window_attention)


def test_window_density_video_only():
    # video-only density of the mask at the pages' clip lengths; the page's
    # 42.1% / 20.0% also count the dense text and audio rows and columns
    for F, want in [(42, 0.40023), (102, 0.17743)]:
        assert abs(oracle.window_frames_allowed(F).mean() - want) < 1e-4


# ---------------------------------------------------------------- mutants

def _allowed_no_anchor(F, chunk=5, nb=1):
    c = np.arange(F) // chunk
    return np.abs(c[:, None] - c[None, :]) <= nb


def _allowed_wrong_chunk(F, chunk=5, nb=1):
    return A.window_frames_allowed(F, chunk + 1, nb)


def _allowed_one_sided(F, chunk=5, nb=1):
    a = A.window_frames_allowed(F, chunk, nb)
    c = np.arange(F) // chunk
    a &= (c[None, :] >= c[:, None] - nb) & (c[None, :] <= c[:, None]) | (np.arange(F)[None, :] == 0) \
        | (np.arange(F)[None, :] == F - 1) | (np.arange(F)[:, None] == 0) | (np.arange(F)[:, None] == F - 1)
    return a


@pytest.mark.parametrize("mut", [_allowed_no_anchor, _allowed_wrong_chunk, _allowed_one_sided],
                         ids=lambda f: f.__name__)
def test_allowed_mutants_caught(mut):
    with pytest.raises(AssertionError):
        check_frames_allowed(mut)


def _tiles_query_first_row_only(N, ft, chunk=5, nb=1):
    T = -(-N // 128)
    F = -(-N // ft)
    allowed = A.window_frames_allowed(F, chunk, nb)
    tf = np.arange(N) // ft
    idx = np.full((T, T), -1, dtype=np.int32)
    count = np.zeros(T, dtype=np.int32)
    for t in range(T):
        tiles = np.unique(np.nonzero(allowed[tf[t * 128]][tf])[0] // 128)
        idx[t, :len(tiles)] = tiles
        count[t] = len(tiles)
    return idx, count


def test_tiles_mutant_caught():
    with pytest.raises(AssertionError):
        check_window_tiles(_tiles_query_first_row_only)


def _attention_ignores_window(q, k, v, scale, ft, chunk=5, nb=1, rows=None):
    return oracle.dense(q, k, v, scale, rows=rows)


def test_attention_mutant_caught():
    with pytest.raises(AssertionError):
        check_window_attention(_attention_ignores_window)
