"""fp64 CPU oracle for attention with INT8 query-key scores.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the HIP library and imports nothing from it.

What is computed: the FastH3 page ("FastH3 Preview v1: four calls,
one-tenth the attention...", section "Update: consumer GPUs and Trim",
subsection "Per device", the RTX 4090 paragraph) reports 8-bit integer codes
for the queries and keys that enter the score product, measured there at about
1.6x the speed with about 0.6% relative error; V and the P V product keep
higher precision.
The page does not give the quantization granularity, rounding or scale rule;
the readings taken here:

* symmetric INT8 with codes in [-127, 127]; scale = max |x| / 127 over the
  group (a group of all zeros gets scale 1 and codes 0);
* queries are quantized per token (one scale per query row); keys per block of
  64 consecutive tokens of one head (the last block may be short);
* code = round-half-to-even(x / scale).  Both the scale and the division are
  IEEE float32 operations, the precision the kernel takes these integer
  decisions in, so the codes are well defined bit for bit;
* the score of (i, j) is scale_attn * sq_i * sk_block(j) * sum_d qc_id kc_jd
  (an exact integer dot product); the softmax and the P V product are exact
  (fp64) with V as given.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_rows

KEY_BLOCK = 64


def _quantize_group(x: np.ndarray):
    """Codes (int64) and float32 scale of one group of values."""
    x32 = np.asarray(x, dtype=np.float32)
    m = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    s = np.float32(1.0) if m == 0 else np.float32(m / np.float32(127.0))
    codes = np.rint(x32 / s).astype(np.int64)
    return np.clip(codes, -127, 127), s


def quantize_rows(x: np.ndarray):
    """Per-row quantization.  x: [R, d] (values exact in float32).
    Returns (codes int64 [R, d], scales float32 [R])."""
    R = x.shape[0]
    codes = np.empty(x.shape, dtype=np.int64)
    scales = np.empty(R, dtype=np.float32)
    for r in range(R):
        codes[r], scales[r] = _quantize_group(x[r])
    return codes, scales


def quantize_blocks(x: np.ndarray, block: int = KEY_BLOCK):
    """Per-block quantization of consecutive rows.  x: [N, d].
    Returns (codes int64 [N, d], scales float32 [ceil(N / block)])."""
    N = x.shape[0]
    nb = -(-N // block)
    codes = np.empty(x.shape, dtype=np.int64)
    scales = np.empty(nb, dtype=np.float32)
    for b in range(nb):
        codes[b * block:(b + 1) * block], scales[b] = _quantize_group(x[b * block:(b + 1) * block])
    return codes, scales


def int8_scores_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, rows=None,
                          block: int = KEY_BLOCK) -> np.ndarray:
    """Attention with INT8 query-key scores, every head.

    q, k, v: [H, N, d] float64 holding bf16 values.  ``rows`` as in ``dense``.
    Returns [H, len(rows), d] float64.
    """
    H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((H, len(rows), d), dtype=np.float64)
    for h in range(H):
        qc, sq = quantize_rows(q[h, rows])
        kc, sk = quantize_blocks(k[h], block)
        # dequantized operands; their products are the exact integer dot scaled
        qd = qc.astype(np.float64) * sq.astype(np.float64)[:, None]
        kd = kc.astype(np.float64) * np.repeat(sk.astype(np.float64), block)[:N, None]
        out[h] = attention_rows(qd, kd, v[h], scale)
    return out
