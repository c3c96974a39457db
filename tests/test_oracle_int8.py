"""Pins of the INT8 query-key score oracle (oracle/int8.py).

FastH3 page, section "Update: consumer GPUs and Trim", subsection "Per device":
queries and keys quantized to INT8 for the attention scores.  Readings: per-token
query scales, per-64-key-block key scales, max-abs / 127, round half to even in
float32.
"""

import numpy as np
import pytest

import oracle
from oracle import int8 as I
from test_oracle_pins import bf16_array


def check_quantizer_bounds(qrows, qblocks):
    x = bf16_array((300, 128), 60)
    codes, s = qrows(x)
    assert codes.min() >= -127 and codes.max() <= 127
    for r in range(300):
        # every code reconstructs its value within half a step (plus the float32
        # rounding of x / s, at most 127 * 2^-24 of a step), the largest magnitude maps to 127
        err = np.abs(x[r] - codes[r] * np.float64(s[r]))
        assert err.max() <= np.float64(s[r]) * (0.5 + 127 * 2.0 ** -24)
        assert np.abs(codes[r]).max() == 127
    z = np.zeros((3, 128))
    zc, zs = qrows(z)
    assert not zc.any() and np.all(zs == 1.0)
    kc, ks = qblocks(x)
    assert ks.shape == (5,)                      # 300 rows: 4 full blocks of 64 and one of 44
    for b in range(5):
        blk = x[64 * b:64 * b + 64]
        assert ks[b] == np.float32(np.float32(np.abs(blk).max()) / np.float32(127))


def check_on_grid_codes(qrows, qblocks):
    """Values that are exactly code * 2^e with a 127 in every group quantize
    back to the same codes (scale = 2^e exactly)."""
    rng = np.random.default_rng(61)
    codes = rng.integers(-127, 128, size=(192, 16))
    codes[:, 3] = 127
    e_rows = rng.integers(-6, 3, size=192)
    x = codes * np.exp2(e_rows)[:, None]
    c, s = qrows(x)
    assert np.array_equal(c, codes) and np.array_equal(s, np.exp2(e_rows).astype(np.float32))
    # key blocks: block b scaled by 2^-b, its largest magnitude is 127 * 2^-b
    xb = codes * np.repeat(np.exp2(-np.arange(3.0)), 64)[:, None]
    cb, sb = qblocks(xb)
    assert np.array_equal(cb, codes) and np.array_equal(sb, np.exp2(-np.arange(3.0)).astype(np.float32))


def check_ties_round_to_even(qrows):
    # 127 * (k + 0.5) / 127 steps: halves go to the even code
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, 126.5, 3.25]])
    c, s = qrows(x)
    assert s[0] == 1.0
    assert c[0].tolist() == [127, 0, 2, 2, 0, -2, 126, 3]


def check_attention_on_grid(attn):
    """On-grid inputs dequantize exactly, so INT8 scores equal plain scores."""
    rng = np.random.default_rng(62)
    H, N, d = 2, 200, 16
    q = rng.integers(-127, 128, size=(H, N, d)).astype(np.float64)
    q[..., 0] = 127
    q *= np.exp2(rng.integers(-8, -4, size=(H, N, 1)))
    k = rng.integers(-127, 128, size=(H, N, d)).astype(np.float64)
    k[:, ::64, 1] = 127                      # each 64-key block holds a 127
    blocks = -(-N // 64)
    k *= np.repeat(np.exp2(rng.integers(-8, -4, size=(H, blocks))), 64, axis=1)[:, :N, None]
    v = bf16_array((H, N, d), 63)
    got = attn(q, k, v, 0.3)
    want = oracle.dense(q, k, v, 0.3)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def check_error_is_small(attn):
    q, k, v = (bf16_array((2, 1008, 128), 64 + t) for t in range(3))
    got = attn(q, k, v, 1 / np.sqrt(128))
    want = oracle.dense(q, k, v, 1 / np.sqrt(128))
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert 0 < rel < 0.02


def test_quantizer_bounds():
    check_quantizer_bounds(I.quantize_rows, I.quantize_blocks)


def test_on_grid_codes_exact():
    check_on_grid_codes(I.quantize_rows, I.quantize_blocks)


def test_ties_round_half_to_even():
    check_ties_round_to_even(I.quantize_rows)


def test_attention_on_grid_equals_dense():
    check_attention_on_grid(I.int8_scores_attention)


def test_error_against_dense_is_small():
    check_error_is_small(I.int8_scores_attention)


def test_rows_subset_matches_full():
    q, k, v = (bf16_array((2, 300, 32), 70 + t) for t in range(3))
    full = I.int8_scores_attention(q, k, v, 0.2)
    rows = np.array([0, 63, 64, 150, 299])
    np.testing.assert_allclose(I.int8_scores_attention(q, k, v, 0.2, rows=rows), full[:, rows],
                               rtol=0, atol=1e-15)


# ---------------------------------------------------------------- mutants

def _rows_floor(x):
    codes, s = I.quantize_rows(x)
    x32 = np.asarray(x, dtype=np.float32)
    return np.clip(np.floor(x32 / s[:, None]).astype(np.int64), -127, 127), s


def _rows_scale_255(x):
    x32 = np.asarray(x, dtype=np.float32)
    m = np.abs(x32).max(axis=1)
    s = np.where(m == 0, np.float32(1), m / np.float32(255)).astype(np.float32)
    return np.clip(np.rint(x32 / s[:, None]).astype(np.int64), -127, 127), s


def _blocks_128(x):
    return I.quantize_blocks(x, block=128)


def _blocks_per_token(x):
    return I.quantize_rows(x)


@pytest.mark.parametrize("mut", [_rows_floor, _rows_scale_255], ids=lambda f: f.__name__)
def test_row_quantizer_mutants_caught(mut):
    failed = 0
    for check in (lambda: check_quantizer_bounds(mut, I.quantize_blocks),
                  lambda: check_on_grid_codes(mut, I.quantize_blocks),
                  lambda: check_ties_round_to_even(mut)):
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed >= 1


@pytest.mark.parametrize("mut", [_blocks_128, _blocks_per_token], ids=lambda f: f.__name__)
def test_block_quantizer_mutants_caught(mut):
    with pytest.raises(AssertionError):
        check_on_grid_codes(I.quantize_rows, mut)


def _attn_no_key_scale(q, k, v, scale, rows=None):
    H, N, d = q.shape
    out = np.empty((H, N, d))
    for h in range(H):
        qc, sq = I.quantize_rows(q[h])
        kc, sk = I.quantize_blocks(k[h])
        out[h] = oracle.attention_rows(qc * sq[:, None].astype(np.float64), kc.astype(np.float64),
                                       v[h], scale)
    return out


def _attn_key_block_off_by_one(q, k, v, scale, rows=None):
    H, N, d = q.shape
    out = np.empty((H, N, d))
    for h in range(H):
        qc, sq = I.quantize_rows(q[h])
        kc, sk = I.quantize_blocks(k[h])
        sk_tok = np.repeat(sk.astype(np.float64), 64)[1:N + 1]
        sk_tok = np.concatenate([sk_tok, sk_tok[-1:]])[:N]
        out[h] = oracle.attention_rows(qc * sq[:, None].astype(np.float64), kc * sk_tok[:, None],
                                       v[h], scale)
    return out


@pytest.mark.parametrize("mut", [_attn_no_key_scale, _attn_key_block_off_by_one],
                         ids=lambda f: f.__name__)
def test_attention_mutants_caught(mut):
    with pytest.raises(AssertionError):
        check_attention_on_grid(mut)
