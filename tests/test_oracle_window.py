"""Pins of the windowed-softmax oracle (Video DeltaNet's softmax branch).

FreeVideo page, section "Where Video DeltaNet comes in": queries in a chunk of
five latent frames attend to their own chunk and the adjacent chunk on either
side (15 frames); the first and last latent frames are visible to every query
and attend to every frame themselves.
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


# ---------------------------------------------------------------- non-video prefix
# Text and audio tokens keep full softmax attention (FreeVideo page, "Where Video
# DeltaNet comes in"): with P non-video tokens ahead of the video, a prefix
# query sees every key and every query sees every prefix key.

def brute_token_allowed(N, P, ft, chunk, nb):
    """Pure-Python restatement at token level: allowed[i][j]."""
    F = -(-(N - P) // ft)
    fa = brute_allowed(F, chunk, nb)
    out = []
    for i in range(N):
        row = []
        for j in range(N):
            if i < P or j < P:
                row.append(True)
            else:
                row.append(bool(fa[(i - P) // ft][(j - P) // ft]))
        out.append(row)
    return out


def check_prefix_tiles(fn):
    for N, P, ft, chunk, nb in [(1000, 37, 64, 2, 1), (900, 300, 100, 3, 1), (1300, 128, 130, 2, 0),
                                (700, 1, 64, 1, 0), (640, 200, 64, 2, 0)]:
        allowed = brute_token_allowed(N, P, ft, chunk, nb)
        idx, count = fn(N, ft, chunk, nb, P)
        T = -(-N // 128)
        for t in range(T):
            want = sorted({j // 128 for i in range(t * 128, min(t * 128 + 128, N))
                           for j in range(N) if allowed[i][j]})
            assert count[t] == len(want), (N, P, t)
            assert list(idx[t, :count[t]]) == want
            assert np.all(idx[t, count[t]:] == -1)


def check_prefix_attention(fn):
    H, N, d, P, ft = 2, 520, 16, 72, 64
    q, k, v = (bf16_array((H, N, d), 190 + t) for t in range(3))
    scale = 0.25
    allowed = brute_token_allowed(N, P, ft, 2, 0)
    out = fn(q, k, v, scale, ft, 2, 0, prefix=P)
    for i in [0, 5, 71, 72, 73, 135, 136, 200, 333, 455, 456, 519]:
        keys = [j for j in range(N) if allowed[i][j]]
        for h in range(H):
            s = [scale * float(q[h, i] @ k[h, j]) for j in keys]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            want = sum(pj * v[h, j] for pj, j in zip(p, keys)) / sum(p)
            np.testing.assert_allclose(out[h, i], want, rtol=0, atol=1e-12)
    # prefix rows are dense rows, bit for bit
    dense = oracle.dense(q, k, v, scale, rows=np.arange(P))
    assert np.array_equal(out[:, :P], dense)
    # Q = 0: the mean of V over the allowed keys
    z = fn(np.zeros_like(q), k, v, scale, ft, 2, 0, prefix=P)
    for i in [3, 100, 300, 519]:
        keys = [j for j in range(N) if allowed[i][j]]
        np.testing.assert_allclose(z[:, i], v[:, keys].mean(axis=1), atol=1e-13)


def test_prefix_window_tiles_brute_force():
    check_prefix_tiles(oracle.window_tiles)


def test_prefix_window_attention_brute_force():
    check_prefix_attention(oracle.window_attention)


def test_prefix_zero_is_the_video_only_window():
    H, N, d = 1, 700, 16
    q, k, v = (bf16_array((H, N, d), 290 + t) for t in range(3))
    a = oracle.window_attention(q, k, v, 0.25, 64, 2, 1)
    b = oracle.window_attention(q, k, v, 0.25, 64, 2, 1, prefix=0)
    assert np.array_equal(a, b)


def test_window_density_counts_the_prefix():
    # brute-force count of the token-level mask against the closed form
    for P, F, ft, chunk, nb in [(0, 7, 3, 2, 1), (5, 7, 3, 2, 1), (11, 9, 4, 3, 0), (2, 12, 5, 5, 1)]:
        N = P + F * ft
        a = brute_token_allowed(N, P, ft, chunk, nb)
        want = sum(sum(r) for r in a) / (N * N)
        assert abs(oracle.window_density(P, F, ft, chunk, nb) - want) < 1e-15
    # prefix 0 reduces to the frame-level density pinned above
    assert abs(oracle.window_density(0, 42, 1008) - 0.40023) < 1e-4


def _prefix_hidden(q, k, v, scale, ft, chunk=5, nb=1, rows=None, prefix=0):
    # video rows lose the prefix keys
    H, N, d = q.shape
    out = oracle.window_attention(q, k, v, scale, ft, chunk, nb, rows=rows, prefix=prefix)
    vid = oracle.window_attention(q[:, prefix:], k[:, prefix:], v[:, prefix:], scale, ft, chunk, nb)
    out[:, prefix:] = vid
    return out


def _prefix_as_frames(q, k, v, scale, ft, chunk=5, nb=1, rows=None, prefix=0):
    # frames counted from token 0 instead of from the first video token
    return oracle.window_attention(q, k, v, scale, ft, chunk, nb, rows=rows, prefix=0)


@pytest.mark.parametrize("mut", [_prefix_hidden, _prefix_as_frames], ids=lambda f: f.__name__)
def test_prefix_attention_mutants_caught(mut):
    with pytest.raises(AssertionError):
        check_prefix_attention(mut)


def _prefix_tiles_ignored(N, ft, chunk=5, nb=1, prefix=0):
    return A.window_tiles(N, ft, chunk, nb, 0)


def test_prefix_tiles_mutant_caught():
    with pytest.raises(AssertionError):
        check_prefix_tiles(_prefix_tiles_ignored)
