"""Pins of the VSA-H3 packed-sequence oracle (oracle/vsa.py).

FastH3 page, section "Lever two: VSA-H3 makes each of the four calls cheaper":
only the generated-video part of the packed sequence is cut into 3D tiles over
its (t, h, w) latent grid ((4, 4, 4) = 64 tokens, or (4, 8, 8) = 256); pooled
tile scores and compute_topk pick the kept video tiles; non-video keys are
always included for video queries; non-video queries are dense.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import vsa as V
from test_oracle_pins import bf16_array


# ---------------------------------------------------------------- helpers (independent restatements)

def brute_tile_ids(frames, height, width, tile):
    """Tile id of every video token from its coordinates (pure Python)."""
    tt, th, tw = tile
    n_h = -(-height // th)
    n_w = -(-width // tw)
    ids = []
    for t in range(frames):
        for h in range(height):
            for w in range(width):
                ids.append((t // tt) * n_h * n_w + (h // th) * n_w + (w // tw))
    return ids


def brute_tiles(frames, height, width, tile):
    ids = brute_tile_ids(frames, height, width, tile)
    out = [[] for _ in range(max(ids) + 1)]
    for tok, j in enumerate(ids):
        out[j].append(tok)
    return out


def int_array(shape, seed, lo=-3, hi=4):
    return np.random.default_rng(seed).integers(lo, hi, size=shape).astype(np.float64)


# ---------------------------------------------------------------- checks (take the function under test)

def check_tiles(fn):
    for grid in [(8, 8, 8), (5, 24, 42), (3, 6, 10), (1, 1, 1), (9, 5, 7)]:
        for tile in [(4, 4, 4), (4, 8, 8), (2, 3, 5)]:
            got = [list(t) for t in fn(*grid, tile)]
            assert got == brute_tiles(*grid, tile), (grid, tile)


def check_pages_counts(fn):
    # 24 x 42 tokens per latent frame (FreeVideo page); 72 and 102 latent frames
    t72 = fn(72, 24, 42, (4, 4, 4))
    sizes = np.array([len(t) for t in t72])
    assert len(t72) == 18 * 6 * 11 == 1188
    assert (sizes == 64).sum() == 18 * 6 * 10 and (sizes == 32).sum() == 18 * 6
    assert oracle.keep_count(len(t72), 0.1) == 119
    t102 = fn(102, 24, 42, (4, 4, 4))
    assert len(t102) == 26 * 6 * 11 == 1716
    assert sizes.sum() == 72 * 1008 and sum(len(t) for t in t102) == 102 * 1008
    assert oracle.keep_count(len(t102), 0.1) == 172
    t256 = fn(72, 24, 42, (4, 8, 8))
    assert len(t256) == 18 * 3 * 6 == 324
    assert sorted(set(len(t) for t in t256)) == [64, 256]


def check_permutation_equivalence(select_fn, attn_fn):
    """With a grid the tile divides and no prefix, 3D tiles are a token
    permutation followed by the 1-D tiles of the same size."""
    for grid, tile, frac in [((8, 8, 8), (4, 4, 4), 0.25), ((8, 16, 16), (4, 8, 8), 0.3)]:
        size = tile[0] * tile[1] * tile[2]
        N = grid[0] * grid[1] * grid[2]
        q, k, v = (bf16_array((2, N, 16), 200 + t) for t in range(3))
        perm = np.concatenate(V.video_tiles(*grid, tile))
        qp, kp, vp = q[:, perm], k[:, perm], v[:, perm]
        idx1 = oracle.select_tiles(qp, kp, frac, tile=size)
        out1 = oracle.sparse(qp, kp, vp, 0.3, idx1, tile=size)
        idx = select_fn(q, k, 0, grid, tile, frac)
        assert np.array_equal(idx, idx1)
        out = attn_fn(q, k, v, 0.3, 0, grid, tile, frac)
        np.testing.assert_allclose(out[:, perm], out1, rtol=0, atol=1e-14)


def check_keep_all_and_text_rows(attn_fn):
    grid, tile, prefix = (5, 6, 10), (4, 4, 4), 7
    N = prefix + 5 * 6 * 10
    q, k, v = (bf16_array((2, N, 16), 210 + t) for t in range(3))
    dense = oracle.dense(q, k, v, 0.25)
    full = attn_fn(q, k, v, 0.25, prefix, grid, tile, 1.0)
    np.testing.assert_allclose(full, dense, rtol=0, atol=1e-13)
    part = attn_fn(q, k, v, 0.25, prefix, grid, tile, 0.2)
    np.testing.assert_allclose(part[:, :prefix], dense[:, :prefix], rtol=0, atol=1e-14)
    # the video rows really are sparse at 0.2
    assert np.abs(part[:, prefix:] - dense[:, prefix:]).max() > 1e-3


def check_q_zero(attn_fn):
    grid, tile, prefix, frac = (5, 6, 10), (4, 4, 4), 9, 0.25
    N = prefix + 5 * 6 * 10
    k, v = (bf16_array((2, N, 8), 220 + t) for t in range(2))
    q = np.zeros_like(k)
    out = attn_fn(q, k, v, 0.5, prefix, grid, tile, frac)
    tiles = brute_tiles(*grid, tile)
    kk = math.ceil(frac * len(tiles))
    keys = list(range(prefix)) + [prefix + t for j in range(kk) for t in tiles[j]]
    for i in [prefix, prefix + 1, prefix + 77, N - 1]:
        np.testing.assert_allclose(out[:, i], v[:, keys].mean(axis=1), rtol=0, atol=1e-13)
    # text rows: mean of every value
    np.testing.assert_allclose(out[:, 0], v.mean(axis=1), rtol=0, atol=1e-13)


def check_tile_constant_ranking(select_fn):
    """Keys constant inside each tile: the score of tile j is its constant, but
    only if a partial tile is divided by its own token count."""
    grid, tile, prefix = (4, 8, 6), (4, 4, 4), 3      # tiles of 64, 32, 64, 32 tokens
    tiles = brute_tiles(*grid, tile)
    assert [len(t) for t in tiles] == [64, 32, 64, 32]
    N = prefix + 4 * 8 * 6
    c = [3.0, 5.0, 4.0, 1.0]
    k = np.zeros((1, N, 4))
    k[0, :prefix, 0] = 100.0                           # the prefix never competes
    for j, toks in enumerate(tiles):
        k[0, [prefix + t for t in toks], 0] = c[j]
    q = np.zeros((1, N, 4))
    q[0, :, 0] = 1.0
    idx = select_fn(q, k, prefix, grid, tile, 0.5)
    assert idx.shape == (1, 4, 2)
    assert np.all(idx[0] == [1, 2])


def check_brute_force(select_fn, attn_fn):
    """Tiny case, every step written out with exact arithmetic."""
    grid, tile, prefix, frac, scale = (3, 3, 5), (2, 2, 2), 2, 0.34, 0.5
    F, Hh, W = grid
    N = prefix + F * Hh * W
    q, k, v = (int_array((1, N, 3), 230 + t) for t in range(3))
    tiles = brute_tiles(*grid, tile)
    T = len(tiles)
    kk = max(1, min(math.ceil(frac * T), T))

    def mean(x, toks):
        return [Fraction(sum(int(x[prefix + t, c]) for t in toks), len(toks)) for c in range(3)]

    qm = [mean(q[0], t) for t in tiles]
    km = [mean(k[0], t) for t in tiles]
    want_idx = []
    for i in range(T):
        score = [sum(a * b for a, b in zip(qm[i], km[j])) for j in range(T)]
        best = None
        for sub in itertools.combinations(range(T), kk):   # lexicographic order
            s = sum(score[j] for j in sub)
            if best is None or s > best[0]:
                best = (s, sub)
        want_idx.append(list(best[1]))
    idx = select_fn(q, k, prefix, grid, tile, frac)
    assert idx[0].tolist() == want_idx
    out = attn_fn(q, k, v, scale, prefix, grid, tile, frac)
    tile_of = brute_tile_ids(*grid, tile)
    for i in range(N):
        if i < prefix:
            keys = list(range(N))
        else:
            keys = list(range(prefix)) + [prefix + t for j in want_idx[tile_of[i - prefix]]
                                          for t in tiles[j]]
        s = [scale * sum(q[0, i, c] * k[0, j, c] for c in range(3)) for j in keys]
        m = max(s)
        p = [math.exp(x - m) for x in s]
        want = [sum(pj * v[0, j, c] for pj, j in zip(p, keys)) / sum(p) for c in range(3)]
        np.testing.assert_allclose(out[0, i], want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- pins

def test_tiles_against_coordinates():
    check_tiles(V.video_tiles)


def test_pages_tile_counts():
    check_pages_counts(V.video_tiles)


def test_permutation_equivalence_with_1d_tiles():
    check_permutation_equivalence(V.vsa_select, V.vsa_attention)


def test_keep_all_is_dense_and_text_rows_are_dense():
    check_keep_all_and_text_rows(V.vsa_attention)


def test_q_zero_gives_mean_over_prefix_and_first_tiles():
    check_q_zero(V.vsa_attention)


def test_tile_constant_ranking_uses_valid_counts():
    check_tile_constant_ranking(V.vsa_select)


def test_brute_force_tiny():
    check_brute_force(V.vsa_select, V.vsa_attention)


def test_means_exact_for_bf16_tiles():
    # the fp64 tile sums of bf16 values are exact: the mean is the exact
    # rational mean rounded once
    x = bf16_array((150, 8), 240)
    tiles = V.video_tiles(3, 5, 10, (2, 4, 4))
    got = V.video_tile_means(x, tiles)
    for j, toks in enumerate(tiles):
        for c in range(8):
            want = float(sum(Fraction(float(x[t, c])) for t in toks) / len(toks))
            assert got[j, c] == want


# ---------------------------------------------------------------- mutants

def _tiles_w_slowest(frames, height, width, tile=(4, 4, 4)):
    tt, th, tw = tile
    grid = np.arange(frames * height * width).reshape(frames, height, width)
    return [grid[a:a + tt, b:b + th, c:c + tw].reshape(-1)
            for c in range(0, width, tw) for b in range(0, height, th) for a in range(0, frames, tt)]


def _tiles_hw_swapped(frames, height, width, tile=(4, 4, 4)):
    tt, th, tw = tile
    grid = np.arange(frames * height * width).reshape(frames, width, height).transpose(0, 2, 1)
    return [grid[a:a + tt, b:b + th, c:c + tw].reshape(-1)
            for a in range(0, frames, tt) for b in range(0, height, th) for c in range(0, width, tw)]


@pytest.mark.parametrize("mut", [_tiles_w_slowest, _tiles_hw_swapped], ids=lambda f: f.__name__)
def test_tile_mutants_caught(mut, monkeypatch):
    with pytest.raises(AssertionError):
        check_tiles(mut)
    monkeypatch.setattr(V, "video_tiles", mut)
    with pytest.raises(AssertionError):
        check_q_zero(V.vsa_attention)


def _means_full_divisor(x, tiles):
    d = x.shape[1]
    full = max(len(t) for t in tiles)
    return np.array([x[t].sum(axis=0) / full for t in tiles]).reshape(len(tiles), d)


def test_means_mutant_caught(monkeypatch):
    monkeypatch.setattr(V, "video_tile_means", _means_full_divisor)
    with pytest.raises(AssertionError):
        check_tile_constant_ranking(V.vsa_select)


def _attn_variant(q, k, v, scale, prefix, grid, tile, keep_frac, rows=None, exempt=True,
                  text_dense=True, compete=False):
    H, N, d = q.shape
    tiles = V.video_tiles(*grid, tile)
    if compete:
        # prefix tokens join the competition as one more "tile" in front
        qm_all = []
        idx = []
        for h in range(H):
            qm = np.vstack([q[h, :prefix].mean(axis=0, keepdims=True),
                            V.video_tile_means(q[h, prefix:], tiles)])
            km = np.vstack([k[h, :prefix].mean(axis=0, keepdims=True),
                            V.video_tile_means(k[h, prefix:], tiles)])
            kk = oracle.keep_count(len(tiles) + 1, keep_frac)
            idx.append(oracle.top_tiles(oracle.tile_scores(qm, km), kk)[1:])
            qm_all.append(qm)
        groups = [np.arange(prefix)] + [prefix + t for t in tiles]
    else:
        idx = V.vsa_select(q, k, prefix, grid, tile, keep_frac)
        groups = None
    out = np.empty((H, N, d))
    tile_of = np.empty(N - prefix, dtype=int)
    for j, t in enumerate(tiles):
        tile_of[t] = j
    for h in range(H):
        for i in range(N):
            if i < prefix:
                keys = np.arange(N) if text_dense else np.arange(prefix)
            elif compete:
                keys = np.concatenate([groups[j] for j in idx[h][tile_of[i - prefix]]])
            else:
                sel = [prefix + tiles[j] for j in idx[h, tile_of[i - prefix]]]
                keys = np.concatenate(([np.arange(prefix)] if exempt else []) + sel)
            out[h, i] = oracle.attention_rows(q[h, i:i + 1], k[h, keys], v[h, keys], scale)[0]
    return out


def test_unmutated_variant_passes():
    # the mutant harness itself computes the oracle's result when nothing is planted
    check_q_zero(_attn_variant)
    check_keep_all_and_text_rows(_attn_variant)
    check_brute_force(V.vsa_select, _attn_variant)


@pytest.mark.parametrize("kw", [dict(exempt=False), dict(text_dense=False), dict(compete=True)],
                         ids=["prefix_not_exempt", "text_rows_sparse", "prefix_competes"])
def test_attention_mutants_caught(kw):
    def mut(*a, **k):
        return _attn_variant(*a, **k, **kw)
    caught = 0
    checks = (check_q_zero, check_keep_all_and_text_rows,
              lambda fn: check_brute_force(V.vsa_select, fn))
    for check in checks:
        try:
            check(mut)
        except AssertionError:
            caught += 1
    assert caught >= 1
