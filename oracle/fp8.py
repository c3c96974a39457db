"""fp64 CPU oracle for attention with FP8 (E4M3) query-key scores.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the HIP library and imports nothing from it.

What is computed: the FastH3 page ("FastH3 Preview v1: four calls,
one-tenth the attention...", section "Update: consumer GPUs and Trim",
subsection "Per device") reports attention scores taken from queries and keys
quantized to 8 bits, with values and the P V product kept in higher
precision.  This is the 8-bit floating-point reading of that step (the INT8
reading is oracle/int8.py).  The pages name no FP8 format or scale rule; the
readings taken here:

* the format is E4M3 of the OCP 8-bit floating-point specification: 1 sign
  bit, 4 exponent bits with bias 7, 3 mantissa bits; subnormals below 2^-6
  with spacing 2^-9; largest finite magnitude 448 (S.1111.110); S.1111.111 is
  NaN and there is no infinity;
* symmetric scaling: scale = max |x| / 448 over the group (a group of all
  zeros gets scale 1), queries per token, keys per block of 64 consecutive
  tokens of one head (the last block may be short), as for INT8;
* code = the E4M3 value nearest to x / scale, ties to the even mantissa; the
  scale and the division are IEEE float32 operations (the precision the
  kernel takes them in), so the codes are well defined bit for bit;
* the score of (i, j) is scale_attn * sq_i * sk_block(j) * sum_d qc_id kc_jd,
  the dot product of the E4M3 values taken exactly; softmax and P V are exact
  (fp64) with V as given.
"""

from __future__ import annotations

import numpy as np

KEY_BLOCK = 64
E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6     # smallest normal binade 2^-6
_MANT_BITS = 3


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Each value rounded to the nearest E4M3 value, ties to even mantissa.
    x: float64 array with |x| <= 448 (+ half a quantum below the overflow
    midpoint); returns float64."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    # binade exponent: 2^e <= |x| < 2^(e+1), clamped to the subnormal range
    _, e2 = np.frexp(mag)                     # mag = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2 - 1, _MIN_NORMAL_EXP)
    quantum = np.exp2(e - _MANT_BITS)         # spacing of the binade (2^-9 for subnormals)
    r = np.rint(mag / quantum) * quantum       # exact scaling by powers of two; rint = half to even
    if np.any(r > E4M3_MAX):
        raise ValueError("value beyond the E4M3 range")
    return np.where(x < 0, -r, r)


def e4m3_decode(code: int) -> float:
    """Value of an 8-bit E4M3 code (NaN for S.1111.111), from the format's definition."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** (-9)
    return s * (1 + m / 8.0) * 2.0 ** (e - 7)


def _quantize_group(x: np.ndarray):
    """E4M3 values (float64) and float32 scale of one group."""
    x32 = np.asarray(x, dtype=np.float32)
    m = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    s = np.float32(1.0) if m == 0 else np.float32(m / np.float32(E4M3_MAX))
    y = (x32 / s).astype(np.float32)           # correctly rounded float32 division
    return e4m3_round(y.astype(np.float64)), s


def quantize_rows(x: np.ndarray):
    """Per-row quantization.  x: [R, d] (values exact in float32).
    Returns (E4M3 values float64 [R, d], scales float32 [R])."""
    codes = np.empty(x.shape, dtype=np.float64)
    scales = np.empty(x.shape[0], dtype=np.float32)
    for r in range(x.shape[0]):
        codes[r], scales[r] = _quantize_group(x[r])
    return codes, scales


def quantize_blocks(x: np.ndarray, block: int = KEY_BLOCK):
    """Per-block quantization of consecutive rows.  x: [N, d].
    Returns (E4M3 values float64 [N, d], scales float32 [ceil(N / block)])."""
    N = x.shape[0]
    nb = -(-N // block)
    codes = np.empty(x.shape, dtype=np.float64)
    scales = np.empty(nb, dtype=np.float32)
    for b in range(nb):
        codes[b * block:(b + 1) * block], scales[b] = _quantize_group(x[b * block:(b + 1) * block])
    return codes, scales


def fp8_scores_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, rows=None,
                         block: int = KEY_BLOCK) -> np.ndarray:
    """Attention with E4M3 query-key scores, every head.

    q, k, v: [H, N, d] float64 holding bf16 values.  ``rows`` as in ``dense``.
    Returns [H, len(rows), d] float64.
    """
    H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((H, len(rows), d), dtype=np.float64)
    for h in range(H):
        qc, sq = quantize_rows(q[h, rows])
        kc, sk = quantize_blocks(k[h], block)
        # the dot products of E4M3 values are exact in fp64 (8-bit products,
        # magnitudes 2^-18 .. 2^17.6, at most 128 terms), then scaled
        dots = qc @ kc.T
        sk_key = np.repeat(sk.astype(np.float64), block)[:N]
        s = scale * (sq.astype(np.float64)[:, None] * sk_key[None, :]) * dots
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        out[h] = (p @ v[h]) / p.sum(axis=1, keepdims=True)
    return out
