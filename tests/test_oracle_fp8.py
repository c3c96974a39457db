"""Pins of the FP8 (E4M3) query-key score oracle (oracle/fp8.py).

FastH3 page, section "Update: consumer GPUs and Trim", subsection "Per device":
queries and keys quantized to 8 bits for the attention scores.  FP8 reading:
OCP E4M3 (bias 7, 3 mantissa bits, max 448, subnormal spacing 2^-9), scale =
max-abs / 448 per query row and per 64-key block, nearest value with ties to
the even mantissa, in float32.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import fp8 as F
from test_oracle_pins import bf16_array

TABLE = {c: F.e4m3_decode(c) for c in range(256)}
FINITE = sorted({v for v in TABLE.values() if v == v})


def brute_round(x):
    """Nearest finite E4M3 value by search over all codes; ties to the code
    with an even mantissa (its lowest bit clear)."""
    best = None
    for c, v in TABLE.items():
        if v != v:
            continue
        d = abs(v - x)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def test_code_table_from_the_format_definition():
    # 256 codes: two NaNs (S.1111.111), +-0, 2 x 126 nonzero finite values
    assert sum(1 for v in TABLE.values() if v != v) == 2
    assert TABLE[0x7F] != TABLE[0x7F] and TABLE[0xFF] != TABLE[0xFF]
    assert max(FINITE) == 448.0 and TABLE[0x7E] == 448.0
    assert min(v for v in FINITE if v > 0) == 2.0 ** -9           # smallest subnormal
    assert TABLE[0x08] == 2.0 ** -6 and TABLE[0x07] == 7 * 2.0 ** -9  # smallest normal, largest subnormal
    assert TABLE[0x38] == 1.0 and TABLE[0x3F] == 1.875 and TABLE[0x40] == 2.0
    assert len(FINITE) == 253                                          # -0 and +0 coincide


def check_rounding(rnd):
    # every finite value is its own rounding
    assert np.array_equal(rnd(np.array(FINITE)), np.array(FINITE))
    # random float32 values against the brute-force search
    rng = np.random.default_rng(70)
    xs = np.concatenate([rng.standard_normal(600) * 50, rng.standard_normal(300) * 0.01,
                         rng.uniform(-448, 448, 300)]).astype(np.float32).astype(np.float64)
    got = rnd(xs)
    for x, g in zip(xs, got):
        assert g == brute_round(x), (x, g, brute_round(x))
    # exact midpoints round to the even mantissa
    pos = [v for v in FINITE if v >= 0]
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    assert np.array_equal(rnd(np.array(mids)), np.array([brute_round(m) for m in mids]))
    assert rnd(np.array([1.0625]))[0] == 1.0 and rnd(np.array([1.1875]))[0] == 1.25
    assert rnd(np.array([3 * 2.0 ** -10]))[0] == 2 * 2.0 ** -9      # subnormal tie to even


def test_rounding_matches_brute_force_search():
    check_rounding(F.e4m3_round)


def check_quantizer(qrows, qblocks):
    x = bf16_array((300, 128), 71)
    vals, s = qrows(x)
    for r in range(300):
        assert s[r] == np.float32(np.float32(np.abs(x[r]).max()) / np.float32(448))
        y = (x[r].astype(np.float32) / s[r]).astype(np.float32).astype(np.float64)
        assert np.array_equal(vals[r], np.array([brute_round(t) for t in y]))
        assert np.abs(vals[r]).max() == 448.0                   # the largest magnitude maps to 448
    z = np.zeros((2, 128))
    zv, zs = qrows(z)
    assert not zv.any() and np.all(zs == 1.0)
    kv, ks = qblocks(x)
    assert ks.shape == (5,)                                     # 4 full blocks of 64 and one of 44
    for b in range(5):
        assert ks[b] == np.float32(np.float32(np.abs(x[64 * b:64 * b + 64]).max()) / np.float32(448))


def test_quantizer():
    check_quantizer(F.quantize_rows, F.quantize_blocks)


def check_on_grid(qrows, qblocks, attn):
    """E4M3 values times 2^e with a 448 in every group quantize back exactly
    (scale 2^e), and then FP8-score attention is dense attention."""
    rng = np.random.default_rng(72)
    H, N, d = 1, 192, 32
    pick = np.array([v for v in FINITE if abs(v) <= 448])
    vals = rng.choice(pick, size=(N, d))
    vals[:, 5] = 448.0
    e = rng.integers(-8, 2, size=N)
    x = vals * np.exp2(e)[:, None]
    c, s = qrows(x)
    assert np.array_equal(c, vals) and np.array_equal(s, np.exp2(e - 0.0).astype(np.float32) * np.float32(1))
    xb = vals * np.repeat(np.exp2(-np.arange(3.0)), 64)[:, None]
    cb, sb = qblocks(xb)
    assert np.array_equal(cb, vals) and np.array_equal(sb, np.exp2(-np.arange(3.0)).astype(np.float32))
    # keys on the per-block grid, queries on the per-row grid: FP8 scores are exact
    q = x[None] * 2.0 ** -6
    k = xb[None] * 2.0 ** -6
    v = bf16_array((H, N, d), 73)
    np.testing.assert_allclose(attn(q, k, v, 0.1), oracle.dense(q, k, v, 0.1), rtol=0, atol=1e-12)


def test_on_grid_inputs_are_exact():
    check_on_grid(F.quantize_rows, F.quantize_blocks, F.fp8_scores_attention)


def test_fp8_attention_is_close_to_dense():
    q, k, v = (bf16_array((2, 640, 128), 74 + t) for t in range(3))
    a = F.fp8_scores_attention(q, k, v, 1 / math.sqrt(128))
    b = oracle.dense(q, k, v, 1 / math.sqrt(128))
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 1e-3 < rel < 0.1


# ---------------------------------------------------------------- mutants

def _round_toward_zero(x):
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, e2 = np.frexp(mag)
    q = np.exp2(np.maximum(e2 - 1, -6) - 3)
    return np.sign(x) * np.trunc(mag / q) * q


def _round_fnuz_spacing(x):
    # bias 8 (the FNUZ variant): subnormal spacing 2^-10
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, e2 = np.frexp(mag)
    q = np.exp2(np.maximum(e2 - 1, -7) - 3)
    return np.sign(x) * np.rint(mag / q) * q


def _round_half_away(x):
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, e2 = np.frexp(mag)
    q = np.exp2(np.maximum(e2 - 1, -6) - 3)
    return np.sign(x) * np.floor(mag / q + 0.5) * q


@pytest.mark.parametrize("mut", [_round_toward_zero, _round_fnuz_spacing, _round_half_away],
                         ids=lambda f: f.__name__)
def test_rounding_mutants_caught(mut):
    with pytest.raises(AssertionError):
        check_rounding(mut)


def _rows_scale_240(x):
    out = np.empty(x.shape); s = np.empty(x.shape[0], dtype=np.float32)
    for r in range(x.shape[0]):
        m = np.float32(np.abs(x[r]).max())
        s[r] = np.float32(1) if m == 0 else np.float32(m / np.float32(240))
        out[r] = F.e4m3_round((x[r].astype(np.float32) / s[r]).astype(np.float32).astype(np.float64))
    return out, s


def _blocks_per_token(x, block=64):
    return F.quantize_rows(x)


@pytest.mark.parametrize("rows,blocks", [(_rows_scale_240, F.quantize_blocks), (F.quantize_rows, _blocks_per_token)],
                         ids=["scale_240", "per_token_keys"])
def test_quantizer_mutants_caught(rows, blocks):
    with pytest.raises(AssertionError):
        check_quantizer(rows, blocks)


def _attn_drops_key_scale(q, k, v, scale, rows=None, block=64):
    H, N, d = q.shape
    out = np.empty_like(q)
    for h in range(H):
        qc, sq = F.quantize_rows(q[h])
        kc, sk = F.quantize_blocks(k[h], block)
        out[h] = oracle.attention_rows(qc * sq.astype(np.float64)[:, None], kc, v[h], scale)
    return out


def test_attention_mutant_caught():
    with pytest.raises(AssertionError):
        check_on_grid(F.quantize_rows, F.quantize_blocks, _attn_drops_key_scale)
