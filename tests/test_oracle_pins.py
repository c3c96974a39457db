"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each check is written as a function that takes the oracle routine under test,
so that tests/test_oracle_mutants.py can feed it deliberately broken variants
and show that the check catches them.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from video_diffusion_transformer_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_array(shape, seed, scale=1.0):
    """Random values that are exactly bfloat16, as float64."""
    rng = np.random.default_rng(seed)
    x = (scale * rng.standard_normal(shape)).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# pin helpers (each raises AssertionError on a mismatch)
# ----------------------------------------------------------------------------

def brute_force_attention(q, k, v, scale):
    """Pure-Python triple loop, straight from the softmax definition."""
    H, N, d = q.shape
    out = np.zeros((H, N, d))
    for h in range(H):
        for i in range(N):
            s = [scale * sum(q[h, i, c] * k[h, j, c] for c in range(d)) for j in range(N)]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            l = sum(p)
            for c in range(d):
                out[h, i, c] = sum(p[j] * v[h, j, c] for j in range(N)) / l
    return out


def check_dense_brute_force(dense_fn):
    for (H, N, d, seed) in [(1, 1, 2, 0), (2, 5, 2, 1), (1, 16, 8, 2), (2, 9, 3, 3)]:
        q, k, v = (bf16_array((H, N, d), seed + 10 * t) for t in range(3))
        scale = 1.0 / math.sqrt(d)
        got = dense_fn(q, k, v, scale)
        ref = brute_force_attention(q, k, v, scale)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def check_dense_vs_sdpa(dense_fn):
    q, k, v = (inputs.make_qkv(1008, 2, "iid", 0)[t].to(torch.float64) for t in range(3))
    scale = 1.0 / math.sqrt(128)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None], v[None], scale=scale, is_causal=False)[0].numpy()
    got = dense_fn(q.numpy(), k.numpy(), v.numpy(), scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def check_dense_invariants(dense_fn):
    H, N, d = 2, 300, 128
    q, k, v = (bf16_array((H, N, d), 40 + t) for t in range(3))
    scale = 1.0 / math.sqrt(d)
    base = dense_fn(q, k, v, scale)
    # rows of P sum to one: V = 1 gives exactly-one outputs
    ones = dense_fn(q, k, np.ones_like(v), scale)
    assert np.max(np.abs(ones - 1.0)) < 1e-12
    # Q = 0: uniform attention, output = mean of V over all keys
    zq = dense_fn(np.zeros_like(q), k, v, scale)
    np.testing.assert_allclose(zq, np.broadcast_to(v.mean(axis=1, keepdims=True), zq.shape), atol=1e-13)
    # constant V is reproduced
    cv = np.broadcast_to(v[:, :1, :], v.shape).copy()
    np.testing.assert_allclose(dense_fn(q, k, cv, scale), cv, atol=1e-13)
    # a vector added to every key shifts each score row by a constant
    c = bf16_array((H, 1, d), 99)
    np.testing.assert_allclose(dense_fn(q, k + c, v, scale), base, atol=1e-10)
    # permuting keys together with values changes nothing
    perm = np.random.default_rng(5).permutation(N)
    np.testing.assert_allclose(dense_fn(q, k[:, perm], v[:, perm], scale), base, atol=1e-13)
    # permuting queries permutes the output rows
    np.testing.assert_allclose(dense_fn(q[:, perm], k, v, scale), base[:, perm], atol=1e-13)
    # a dominant key: q_i = alpha * k_j makes o_i -> v_j
    qd = q.copy()
    qd[0, 7] = 40.0 * k[0, 123] / np.linalg.norm(k[0, 123])
    od = dense_fn(qd, k, v, scale)
    np.testing.assert_allclose(od[0, 7], v[0, 123], atol=1e-6)


def exact_mean_rounded(rows):
    """Exact rational mean of the rows, correctly rounded once to float64."""
    d = rows.shape[1]
    return np.array([float(sum(Fraction(x) for x in rows[:, c]) / len(rows)) for c in range(d)])


def check_tile_means_exact(means_fn):
    # 300 tokens: tiles of 128, 128 and a partial 44; 1008: last tile 112; 5040: last 48
    for N, seed in [(300, 1), (1008, 2), (5040, 3), (1, 4), (128, 5), (129, 6)]:
        x = bf16_array((N, 16), seed, scale=3.0)
        got = means_fn(x)
        T = -(-N // 128)
        assert got.shape == (T, 16)
        for t in range(T):
            ref = exact_mean_rounded(x[t * 128:min(t * 128 + 128, N)])
            assert np.array_equal(got[t], ref), (N, t)


def python_score(a, b):
    """The canonical score: +0.0, then d = 0.., one rounding per product and per sum."""
    acc = 0.0
    for x, y in zip(a.tolist(), b.tolist()):
        acc = acc + x * y
    return acc


def check_tile_scores_canonical(scores_fn):
    rng = np.random.default_rng(7)
    for T, d in [(5, 128), (9, 128), (3, 7)]:
        qm = rng.standard_normal((T, d))
        km = rng.standard_normal((T, d))
        got = scores_fn(qm, km)
        for i in range(T):
            for j in range(T):
                ref = python_score(qm[i], km[j])
                assert got[i, j] == ref, (i, j)
                # and within the forward error bound of the exact dot product
                exact = sum(Fraction(a) * Fraction(b) for a, b in zip(qm[i], km[j]))
                bound = d * 2.0 ** -52 * float(np.abs(qm[i]) @ np.abs(km[j]))
                assert abs(Fraction(got[i, j]) - exact) <= Fraction(bound)


def brute_force_topk(row, k):
    """Among all k-subsets with the largest exact sum, the lexicographically lowest."""
    best, best_sum = None, None
    for comb in itertools.combinations(range(len(row)), k):
        s = sum(Fraction(row[j]) for j in comb)
        if best_sum is None or s > best_sum:
            best, best_sum = comb, s
    return np.array(best)


def check_top_tiles_brute_force(top_fn):
    rng = np.random.default_rng(11)
    for T in [1, 2, 5, 8]:
        for k in range(1, T + 1):
            for trial in range(3):
                # quantized scores force exact ties
                sigma = np.round(rng.standard_normal((T, T)) * 2) / 2
                got = top_fn(sigma, k)
                assert got.dtype == np.int32 and got.shape == (T, k)
                for i in range(T):
                    assert np.array_equal(got[i], brute_force_topk(sigma[i], k)), (T, k, i, sigma[i])


def check_select_closed_forms(select_fn):
    # Q = 0: every score is +0.0, so the lowest k tiles win everywhere (tie rule)
    H, N, d = 2, 1000, 128
    k = bf16_array((H, N, d), 3)
    idx = select_fn(np.zeros((H, N, d)), k, 0.25)
    T = 8
    kk = 2
    assert idx.shape == (H, T, kk)
    assert np.array_equal(idx, np.broadcast_to(np.arange(kk, dtype=np.int32), (H, T, kk)))
    # a fraction that is not a whole number of tiles rounds up: 0.3 * 8 = 2.4 -> 3
    idx = select_fn(np.zeros((H, N, d)), k, 0.3)
    assert np.array_equal(idx, np.broadcast_to(np.arange(3, dtype=np.int32), (H, T, 3)))
    # tile-constant integer inputs: key tile j holds the value j in channel 0, so
    # sigma_ij = q0 * j exactly; positive q keeps the highest tiles, negative the lowest
    N = 1000
    kc = np.zeros((1, N, d))
    kc[0, :, 0] = np.arange(N) // 128
    qpos = np.zeros((1, N, d))
    qpos[0, :, 0] = 1.0
    qpos[0, 640:768, 0] = -2.0   # query tile 5 prefers low tiles
    idx = select_fn(qpos, kc, 0.375)  # ceil(0.375 * 8) = 3
    for t in range(8):
        want = [0, 1, 2] if t == 5 else [5, 6, 7]
        assert list(idx[0, t]) == want, (t, idx[0, t])
    # the partial last tile is averaged over its 104 valid tokens only: its keys
    # are 1.0 against 0.875 elsewhere; dividing by 128 would drop it to 0.8125
    kp = np.zeros((1, N, d))
    kp[0, :, 1] = 0.875
    kp[0, 896:, 1] = 1.0
    qp = np.zeros((1, N, d))
    qp[0, :, 1] = 1.0
    idx = select_fn(qp, kp, 0.125)      # one tile kept
    assert np.all(idx[0, :, 0] == 7)


def check_select_shift_invariance(select_fn):
    # small integers keep every mean, product and sum exact, so adding the same
    # vector to every key moves each score row by a constant and keeps the choice
    rng = np.random.default_rng(21)
    H, N, d = 2, 1024, 128
    q = rng.integers(-4, 5, (H, N, d)).astype(np.float64)
    k = rng.integers(-4, 5, (H, N, d)).astype(np.float64)
    c = 64.0 * rng.integers(-2, 3, (H, 1, d)).astype(np.float64)
    a = select_fn(q, k, 0.3)
    b = select_fn(q, k + c, 0.3)
    assert np.array_equal(a, b)


def check_sparse_pins(sparse_fn, dense_fn):
    H, N, d = 2, 300, 128
    q, k, v = (bf16_array((H, N, d), 60 + t) for t in range(3))
    scale = 1.0 / math.sqrt(d)
    T = 3
    # keep everything: identical to dense, bit for bit (same keys, same order)
    full = np.broadcast_to(np.arange(T, dtype=np.int32), (H, T, T))
    assert np.array_equal(sparse_fn(q, k, v, scale, full), dense_fn(q, k, v, scale))
    # Q = 0: mean of V over the kept tiles' valid keys
    idx = np.array([[[0], [2], [2]], [[1], [0], [2]]], dtype=np.int32)
    zo = sparse_fn(np.zeros_like(q), k, v, scale, idx)
    for h in range(H):
        for t in range(T):
            keys = oracle.kept_keys(idx[h, t], N)
            rows = np.arange(t * 128, min(t * 128 + 128, N))
            np.testing.assert_allclose(zo[h, rows], np.broadcast_to(v[h, keys].mean(0), (len(rows), d)),
                                       atol=1e-13)
    # brute force on the explicitly gathered keys, tiny width
    d2 = 2
    q2, k2, v2 = (bf16_array((1, N, d2), 70 + t) for t in range(3))
    idx2 = np.array([[[0, 2], [1, 2], [0, 1]]], dtype=np.int32)
    got = sparse_fn(q2, k2, v2, 0.7, idx2)
    for t in range(T):
        keys = oracle.kept_keys(idx2[0, t], N)
        rows = np.arange(t * 128, min(t * 128 + 128, N))
        for i in rows:
            s = [0.7 * (q2[0, i, 0] * k2[0, j, 0] + q2[0, i, 1] * k2[0, j, 1]) for j in keys]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            for c in range(d2):
                want = sum(pj * v2[0, j, c] for pj, j in zip(p, keys)) / sum(p)
                assert abs(got[0, i, c] - want) < 1e-12


# ----------------------------------------------------------------------------
# the tests
# ----------------------------------------------------------------------------

def test_dense_brute_force():
    check_dense_brute_force(oracle.dense)


def test_dense_matches_torch_sdpa_fp64():
    check_dense_vs_sdpa(oracle.dense)


def test_dense_invariants():
    check_dense_invariants(oracle.dense)


def test_dense_row_subset():
    q, k, v = (bf16_array((2, 500, 128), 80 + t) for t in range(3))
    rows = np.array([0, 17, 255, 499])
    full = oracle.dense(q, k, v, 0.1)
    np.testing.assert_allclose(oracle.dense(q, k, v, 0.1, rows=rows), full[:, rows], rtol=0, atol=1e-14)


def test_tile_means_exact():
    check_tile_means_exact(oracle.tile_means)


def test_tile_scores_canonical():
    check_tile_scores_canonical(oracle.tile_scores)


def test_top_tiles_brute_force():
    check_top_tiles_brute_force(oracle.top_tiles)


def test_select_closed_forms():
    check_select_closed_forms(oracle.select_tiles)


def test_select_shift_invariance():
    check_select_shift_invariance(oracle.select_tiles)


def test_sparse_pins():
    check_sparse_pins(oracle.sparse, oracle.dense)


def test_keep_count_rule():
    # compute_topk: max(1, min(ceil((1 - sparsity) * blocks), blocks))
    assert oracle.keep_count(567, 0.1) == 57
    assert oracle.keep_count(567, 1 - 0.9) == 57
    assert oracle.keep_count(804, 0.1) == 81
    assert oracle.keep_count(804, 1 - 0.9) == 81
    assert oracle.keep_count(8, 0.1) == 1
    assert oracle.keep_count(40, 0.1) == 4
    assert oracle.keep_count(1, 0.1) == 1
    assert oracle.keep_count(567, 1.0) == 567
    assert oracle.keep_count(567, 1e-9) == 1
    assert oracle.keep_count(0, 0.1) == 0
    # the IEEE double product decides: 0.07 * 100 rounds to 7.000000000000001
    assert oracle.keep_count(100, 0.07) == 8
    assert oracle.keep_count(50, 0.14) == 8


def test_geometry_matches_pages():
    with open(os.path.join(GOLDEN, "pages_geometry.json")) as f:
        g = json.load(f)
    assert inputs.TOKENS_PER_LATENT_FRAME == g["tokens_per_latent_frame"]["value"] == 24 * 42
    for frames, lat in g["clip_frames_to_latent"]["value"]:
        assert inputs.latent_frames(frames) == lat
    ch = g["vae_chunk"]
    for n in range(1, 30):   # every further 17-frame chunk adds 5 latent frames
        assert (inputs.latent_frames(17 * n + 5) - inputs.latent_frames(17 * (n - 1) + 5)
                == ch["latent_frames"])
        assert inputs.latent_frames(17 * n + 4) == inputs.latent_frames(17 * n + 5)  # rounds up
    for frames, tok in g["clip_tokens"]["value"]:
        assert inputs.video_tokens(frames) == tok
    assert inputs.TOTAL_HEADS * inputs.HEAD_DIM == g["heads"]["qkv_width"]
    qkv = 3 * 102816 * 7168 * 2 / 1e9
    assert round(qkv, 2) == g["qkv_all_heads_bytes_at_102816"]["value_gb"]
    assert round(102816 ** 2 * 2 / 1e9, 1) == g["dense_scores_one_head_bytes_at_102816"]["value_gb"]
    assert round(102816 * 4 * 128 * 2 / 1e6) == g["four_head_slice_bytes_at_102816"]["value_mb"]
    assert inputs.CONFIGS[3].tokens == 72576 and inputs.CONFIGS[5].tokens == 102816
    assert oracle.tile_count(72576) == 567 and oracle.tile_count(102816) == 804
    assert 102816 - 803 * 128 == 32   # the partial last tile of the 14.4 s clip
    f = g["compute_topk"]
    assert oracle.keep_count(567, 1 - f["trained_sparsity"]) == 57


def test_inputs_are_seeded_and_bf16():
    a = inputs.make_qkv(300, 2, "frame", 5)
    b = inputs.make_qkv(300, 2, "frame", 5)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (2, 300, 128) and x.is_contiguous()
        assert torch.equal(x, y)
    c = inputs.make_qkv(300, 3, "frame", 5)
    assert torch.equal(c[0][:2], a[0])        # fewer heads = a prefix of the same streams
    # frame correlation: same-frame q.k is large, cross-frame small
    q, k, _ = inputs.make_qkv(2016, 1, "frame", 1)
    qf, kf = q.float()[0], k.float()[0]
    same = (qf[:1008] * kf[:1008]).sum(1).mean()
    cross = (qf[:1008] * kf[1008:]).sum(1).mean()
    assert same > 80 and abs(cross) < 40
