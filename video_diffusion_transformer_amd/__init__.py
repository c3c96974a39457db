"""MI355X (gfx950) dense and block-sparse attention over video tokens.

A thin ctypes binding of the C ABI in include/fvattn.h, with the same names.
It only marshals arguments: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if libfvattn.so is missing or fails to load,
every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfvattn.so")

FVATTN_OK = 0
FVATTN_ERR_INVALID_ARG = 1
FVATTN_ERR_UNSUPPORTED = 2
FVATTN_ERR_ALLOC = 3
FVATTN_ERR_HIP = 4
FVATTN_DENSE = 0
FVATTN_BLOCK_SPARSE = 1
FVATTN_DENSE_INT8QK = 2
FVATTN_DENSE_FP8QK = 3
TILE = 128
HEAD_DIM = 128
MAX_TILES = 2048
PROBE_SINK = 262144
PROBE_WAVES = 4096
PROBE_FLOP_PER_ITER = PROBE_WAVES * 4 * 32768

_MODES = {"dense": FVATTN_DENSE, "sparse": FVATTN_BLOCK_SPARSE, "int8": FVATTN_DENSE_INT8QK,
          "fp8": FVATTN_DENSE_FP8QK,
          FVATTN_DENSE: FVATTN_DENSE, FVATTN_BLOCK_SPARSE: FVATTN_BLOCK_SPARSE,
          FVATTN_DENSE_INT8QK: FVATTN_DENSE_INT8QK, FVATTN_DENSE_FP8QK: FVATTN_DENSE_FP8QK}

_lib = None

# (name, restype, argtypes) of every exported function
_P, _I, _F, _D = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
SIGNATURES = {
    "fvattn_keep_count": (_I, [_I, _D]),
    "fvattn_forward": (_I, [_P, _P, _P, _P, _I, _I, _I, _F, _I, _D, _P]),
    "fvattn_select_tiles": (_I, [_P, _P, _I, _I, _I, _D, _P, _P]),
    "fvattn_forward_indexed": (_I, [_P, _P, _P, _P, _I, _P, _I, _I, _I, _F, _P]),
    "fvattn_forward_sparse_noalloc": (_I, [_P, _P, _P, _P, _I, _I, _I, _F, _D, _P]),
    "fvattn_forward_heads": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _D, _P]),
    "fvattn_tile_means": (_I, [_P, _I, _I, _I, _P, _P]),
    "fvattn_forward_window": (_I, [_P, _P, _P, _P, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    "fvattn_window_tiles": (_I, [_I, _I, _I, _I, _I, _P, _P, _P]),
    "fvattn_tile_scores": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "fvattn_forward_vsa": (_I, [_P, _P, _P, _P, _I, _I, _I, _F, _I, _I, _I, _I, _I, _I, _I, _D, _P]),
    "fvattn_vsa_select": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _D, _P, _P]),
    "fvattn_vsa_tile_count": (_I, [_I, _I, _I, _I, _I, _I]),
    "fvattn_quantize_k": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "fvattn_quantize_k_fp8": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "fvattn_vda_forward": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "fvattn_vda_states": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "fvattn_mfma_probe": (_I, [_P, _I, _I, _P]),
    "fvattn_status_string": (ctypes.c_char_p, [_I]),
}


class FvattnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(status_string(status))


def load(path: str = LIB_PATH):
    """Load libfvattn.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libfvattn.so is not built (%s); run `python -m video_diffusion_transformer_amd.build`"
            % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fvattn_status_string(int(status)).decode()


def _check(rc: int):
    if rc != FVATTN_OK:
        raise FvattnError(rc)


def keep_count(tokens: int, keep_frac: float) -> int:
    k = load().fvattn_keep_count(int(tokens), float(keep_frac))
    if k < 0:
        raise FvattnError(-k)
    return k


def tile_count(tokens: int) -> int:
    return -(-int(tokens) // TILE)


# ---------------------------------------------------------------- torch side

def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_qkv(*ts, shape=None):
    torch = _torch()
    ref = ts[0]
    if ref.dim() != 3:
        raise ValueError("expected [heads, tokens, head_dim] tensors")
    for t in ts:
        if t.dtype != torch.bfloat16:
            raise TypeError("expected bfloat16 tensors")
        if not t.is_cuda:
            raise ValueError("expected device tensors")
        if not t.is_contiguous():
            raise ValueError("expected contiguous tensors")
        if t.shape != ref.shape or t.device != ref.device:
            raise ValueError("q, k, v (and out) must share shape and device")
    return ref.shape


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def forward(q, k, v, scale: float | None = None, mode="dense", keep_frac: float = 0.1,
            out=None, stream=None):
    """fvattn_forward.  q, k, v: bf16 [heads, tokens, 128] device tensors."""
    torch = _torch()
    H, N, d = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(load().fvattn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), H, N, d, scale,
                                     _MODES[mode], float(keep_frac), _stream_ptr(stream)))
    return out


def forward_sparse_noalloc(q, k, v, scale: float | None = None, keep_frac: float = 0.1, out=None,
                           stream=None):
    """fvattn_forward_sparse_noalloc: block-sparse attention with the library's static
    scratch (no allocation inside the library; `out` may be passed in too)."""
    torch = _torch()
    H, N, d = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(load().fvattn_forward_sparse_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), H, N, d,
                                                    scale, float(keep_frac), _stream_ptr(stream)))
    return out


def forward_heads(q, k, v, group_heads: int, scale: float | None = None, mode="dense",
                  keep_frac: float = 0.1, out=None, stream=None):
    """fvattn_forward_heads: the same attention, launched in head groups of 16, 8 or 4."""
    torch = _torch()
    H, N, d = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(load().fvattn_forward_heads(_ptr(q), _ptr(k), _ptr(v), _ptr(out), H, int(group_heads),
                                           N, d, scale, _MODES[mode], float(keep_frac),
                                           _stream_ptr(stream)))
    return out


def select_tiles(q, k, keep_frac: float = 0.1, out=None, stream=None):
    """fvattn_select_tiles: int32 [heads, T, keep] kept key tiles per query tile."""
    torch = _torch()
    H, N, d = _check_qkv(q, k)
    kk = keep_count(N, keep_frac)
    if out is None:
        out = torch.empty((H, tile_count(N), kk), dtype=torch.int32, device=q.device)
    if out.dtype != torch.int32 or not out.is_contiguous() or tuple(out.shape) != (H, tile_count(N), kk):
        raise ValueError("idx out must be contiguous int32 [heads, T, keep]")
    with torch.cuda.device(q.device):
        _check(load().fvattn_select_tiles(_ptr(q), _ptr(k), H, N, d, float(keep_frac), _ptr(out),
                                          _stream_ptr(stream)))
    return out


def forward_indexed(q, k, v, idx, scale: float | None = None, out=None, stream=None):
    """fvattn_forward_indexed: sparse attention over caller-given tile lists idx [heads, T, keep]."""
    torch = _torch()
    H, N, d = _check_qkv(q, k, v)
    if idx.dtype != torch.int32 or not idx.is_contiguous() or idx.dim() != 3 \
            or idx.shape[0] != H or idx.shape[1] != tile_count(N) or idx.device != q.device:
        raise ValueError("idx must be contiguous int32 [heads, T, keep] on the device of q")
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(load().fvattn_forward_indexed(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), int(idx.shape[2]),
                                             _ptr(out), H, N, d, scale, _stream_ptr(stream)))
    return out


def tile_means(x, stream=None):
    """fvattn_tile_means: fp64 [heads, T, 128] tile means of a bf16 [heads, tokens, 128] tensor."""
    torch = _torch()
    H, N, d = _check_qkv(x)
    out = torch.empty((H, tile_count(N), d), dtype=torch.float64, device=x.device)
    with torch.cuda.device(x.device):
        _check(load().fvattn_tile_means(_ptr(x), H, N, d, _ptr(out), _stream_ptr(stream)))
    return out


def tile_scores(qm, km, stream=None):
    """fvattn_tile_scores: fp64 [heads, T, T] canonical scores of fp64 tile means."""
    torch = _torch()
    if qm.dtype != torch.float64 or km.dtype != torch.float64 or qm.shape != km.shape \
            or qm.dim() != 3 or not qm.is_contiguous() or not km.is_contiguous():
        raise ValueError("expected contiguous float64 [heads, T, 128] means")
    H, T, d = qm.shape
    out = torch.empty((H, T, T), dtype=torch.float64, device=qm.device)
    with torch.cuda.device(qm.device):
        _check(load().fvattn_tile_scores(_ptr(qm), _ptr(km), H, T, d, _ptr(out), _stream_ptr(stream)))
    return out


def forward_window(q, k, v, frame_tokens: int = 1008, chunk_frames: int = 5, neighbours: int = 1,
                   scale: float | None = None, prefix: int = 0, out=None, stream=None):
    """fvattn_forward_window: softmax restricted to the frame window and the anchor
    frames; `prefix` non-video tokens (text, audio) ahead of the video stay dense."""
    torch = _torch()
    H, N, d = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(load().fvattn_forward_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), H, N, d, scale,
                                            int(prefix), int(frame_tokens), int(chunk_frames),
                                            int(neighbours), _stream_ptr(stream)))
    return out


def window_tiles(tokens: int, frame_tokens: int = 1008, chunk_frames: int = 5, neighbours: int = 1,
                 prefix: int = 0, device="cuda", stream=None):
    """fvattn_window_tiles: (idx int32 [T, T] padded with -1, count int32 [T]) on the device."""
    torch = _torch()
    T = tile_count(tokens)
    idx = torch.empty((T, T), dtype=torch.int32, device=device)
    count = torch.empty((T,), dtype=torch.int32, device=device)
    with torch.cuda.device(idx.device):
        _check(load().fvattn_window_tiles(int(tokens), int(prefix), int(frame_tokens), int(chunk_frames),
                                          int(neighbours), _ptr(idx), _ptr(count), _stream_ptr(stream)))
    return idx, count


def vsa_tile_count(grid, tile=(4, 4, 4)) -> int:
    """fvattn_vsa_tile_count: video tiles of a (frames, height, width) grid."""
    n = load().fvattn_vsa_tile_count(*(int(x) for x in grid), *(int(x) for x in tile))
    if n < 0:
        raise FvattnError(-n)
    return n


def forward_vsa(q, k, v, prefix: int, grid, tile=(4, 4, 4), keep_frac: float = 0.1,
                scale: float | None = None, out=None, stream=None):
    """fvattn_forward_vsa: VSA-H3 attention over [prefix | video grid] packed tokens."""
    torch = _torch()
    H, N, d = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_qkv(q, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        _check(load().fvattn_forward_vsa(_ptr(q), _ptr(k), _ptr(v), _ptr(out), H, N, d, scale,
                                         int(prefix), *(int(x) for x in grid),
                                         *(int(x) for x in tile), float(keep_frac),
                                         _stream_ptr(stream)))
    return out


def vsa_select(q, k, prefix: int, grid, tile=(4, 4, 4), keep_frac: float = 0.1, stream=None):
    """fvattn_vsa_select: int32 [heads, Tv, keep] kept video key tiles per video query tile."""
    torch = _torch()
    H, N, d = _check_qkv(q, k)
    tv = vsa_tile_count(grid, tile)
    kk = keep_count(tv * TILE, keep_frac)    # the library's keep count of tv tiles
    out = torch.empty((H, tv, kk), dtype=torch.int32, device=q.device)
    with torch.cuda.device(q.device):
        _check(load().fvattn_vsa_select(_ptr(q), _ptr(k), H, N, d, int(prefix),
                                        *(int(x) for x in grid), *(int(x) for x in tile),
                                        float(keep_frac), _ptr(out), _stream_ptr(stream)))
    return out


def quantize_k(k, stream=None):
    """fvattn_quantize_k: (codes int8 [heads, tokens, 128], scales float32 [heads, ceil(tokens/64)])."""
    torch = _torch()
    H, N, d = _check_qkv(k)
    codes = torch.empty((H, N, d), dtype=torch.int8, device=k.device)
    scales = torch.empty((H, -(-N // 64)), dtype=torch.float32, device=k.device)
    with torch.cuda.device(k.device):
        _check(load().fvattn_quantize_k(_ptr(k), H, N, d, _ptr(codes), _ptr(scales), _stream_ptr(stream)))
    return codes, scales


def quantize_k_fp8(k, stream=None):
    """fvattn_quantize_k_fp8: (E4M3 codes uint8 [heads, tokens, 128], scales float32 [heads, ceil(tokens/64)])."""
    torch = _torch()
    H, N, d = _check_qkv(k)
    codes = torch.empty((H, N, d), dtype=torch.uint8, device=k.device)
    scales = torch.empty((H, -(-N // 64)), dtype=torch.float32, device=k.device)
    with torch.cuda.device(k.device):
        _check(load().fvattn_quantize_k_fp8(_ptr(k), H, N, d, _ptr(codes), _ptr(scales), _stream_ptr(stream)))
    return codes, scales


def _check_vda(q, k, v, beta, alpha, s_text, frame_tokens: int, out=None):
    """Shapes, dtypes, contiguity and device of the Video Delta Attention
    tensors (q may be None for the states call); returns (H, N, F)."""
    torch = _torch()
    ref = k
    if ref.dim() != 3 or ref.shape[2] != HEAD_DIM:
        raise ValueError("k must be [heads, tokens, 128]")
    H, N, d = ref.shape
    ft = int(frame_tokens)
    if ft <= 0 or N % ft:
        raise ValueError("tokens must be frames * frame_tokens")
    F = N // ft
    want = [(k, (H, N, d), torch.bfloat16, "k"), (v, (H, N, d), torch.bfloat16, "v"),
            (beta, (H, N), torch.float32, "beta"), (alpha, (H, F, d), torch.float32, "alpha"),
            (s_text, (H, d, d), torch.float32, "s_text")]
    if q is not None:
        want.insert(0, (q, (H, N, d), torch.bfloat16, "q"))
    if out is not None:
        want.append((out, (H, N, d), torch.float32, "out"))
    for t, shape, dtype, name in want:
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for t, _, _, name in want:
        if not t.is_cuda or t.device != ref.device:
            raise ValueError(f"{name} must be a device tensor on the device of k")
    return H, N, F


def vda_forward(q, k, v, beta, alpha, s_text, frame_tokens: int, chunk_frames: int = 5,
                neighbours: int = 1, out=None, stream=None):
    """fvattn_vda_forward: Video Delta Attention readout, float32 [heads, tokens, 128].
    Precondition (not checked on the device): every beta finite and >= 0."""
    torch = _torch()
    H, N, F = _check_vda(q, k, v, beta, alpha, s_text, frame_tokens, out)
    if out is None:
        out = torch.empty((H, N, HEAD_DIM), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        _check(load().fvattn_vda_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
                                         _ptr(s_text), _ptr(out), H, F, int(frame_tokens), HEAD_DIM,
                                         int(chunk_frames), int(neighbours), _stream_ptr(stream)))
    return out


def vda_states(k, v, beta, alpha, s_text, frame_tokens: int, stream=None):
    """fvattn_vda_states: (fwd, rev) float32 [heads, frames + 1, 128, 128].
    Precondition (not checked on the device): every beta finite and >= 0."""
    torch = _torch()
    H, N, F = _check_vda(None, k, v, beta, alpha, s_text, frame_tokens)
    d = HEAD_DIM
    fwd = torch.empty((H, F + 1, d, d), dtype=torch.float32, device=k.device)
    rev = torch.empty_like(fwd)
    with torch.cuda.device(k.device):
        _check(load().fvattn_vda_states(_ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(s_text), H, F,
                                        int(frame_tokens), d, _ptr(fwd), _ptr(rev), _stream_ptr(stream)))
    return fwd, rev


def mfma_probe(iters: int, sink=None, stream=None):
    """fvattn_mfma_probe: PROBE_FLOP_PER_ITER * iters FLOP of bf16 MFMAs on the
    current device; returns the float32 sink (time the call with events)."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(PROBE_SINK, dtype=torch.float32, device="cuda")
    if sink.dtype != torch.float32 or not sink.is_cuda or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous float32 device tensor")
    with torch.cuda.device(sink.device):
        _check(load().fvattn_mfma_probe(_ptr(sink), min(sink.numel(), 2**31 - 1), int(iters),
                                         _stream_ptr(stream)))
    return sink
