"""Seeded synthetic inputs for video-token attention.

This module only draws random numbers and fixes shapes. It holds none of the
attention arithmetic, so both the fp64 CPU oracle tests and the HIP path may
use it without sharing any of the method.

Shapes follow the MiniMax-H3 geometry on the FreeVideo page ("FreeVideo: a 66
GB video transformer on an 8 GB card...", section "What MiniMax H3 is,
briefly"): 56 heads of width 128, 1,008 tokens per latent frame at 1344x768
(a 24x42 latent grid), 72 latent frames (72,576 tokens) for a 10 s clip and 102
latent frames (102,816 tokens) for a 14.4 s clip.

Recipe (the pages give no activations, so these stand in for them):

* i.i.d. tensors: every element N(0, 1).
* frame-correlated Q and K: one shared N(0, 1) vector per (head, latent frame),
  used by both Q and K, plus independent N(0, 0.5^2) noise for Q and for K.
  This gives the within-frame locality of video tokens.  V is always N(0, 1).

Every tensor has its own counter-free numpy stream, ``default_rng([seed,
tag])``, so tensors can be drawn one head at a time (the draws of a stream are
consumed in C order, so head-by-head drawing equals drawing the whole array).
All draws are float32 and are rounded to bfloat16 with round-to-nearest-even.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

HEAD_DIM = 128
TOKENS_PER_LATENT_FRAME = 24 * 42  # 1344x768 with 16x spatial compression and 2x2 patches
TOTAL_HEADS = 56

# stream tags
_TAG_Q, _TAG_K, _TAG_V, _TAG_SHARED = 1, 2, 3, 4


def latent_frames(video_frames: int) -> int:
    """Latent frames for a clip: frames round up to 17n+5, each 17-frame chunk
    becomes 5 latent frames (FreeVideo page, "What MiniMax H3 is, briefly").
    17n+5 frames -> 5n+2 latent frames."""
    if video_frames < 1:
        raise ValueError("video_frames must be >= 1")
    n = max(0, math.ceil((video_frames - 5) / 17))
    return 5 * n + 2


def video_tokens(video_frames: int) -> int:
    return latent_frames(video_frames) * TOKENS_PER_LATENT_FRAME


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    tokens: int
    heads: int            # heads in the tensors of this workload
    group: int            # heads per launch for the head-group launcher
    dist: str             # "iid" or "frame"
    seed: int
    modes: tuple          # ("dense",), ("sparse", "dense") ...
    keep_frac: float = 0.1

    @property
    def frames(self) -> int:
        return self.tokens // TOKENS_PER_LATENT_FRAME

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)


CONFIGS = {
    1: Config("dense_1frame_1008tok_4h", 1008, 4, 4, "iid", 0, ("dense",)),
    2: Config("dense_5frame_5040tok_56h", 5040, 56, 56, "iid", 1, ("dense",)),
    3: Config("dense_10s_72576tok_16h", 72576, 16, 16, "frame", 2, ("dense",)),
    4: Config("sparse_10s_72576tok_56h", 72576, 56, 16, "frame", 3, ("sparse", "dense")),
    5: Config("dense_sparse_14s_102816tok_56h", 102816, 56, 8, "frame", 4, ("dense", "sparse")),
}


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([seed, tag])


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def make_qkv(tokens: int, heads: int, dist: str, seed: int, head_dim: int = HEAD_DIM,
             frame_tokens: int = TOKENS_PER_LATENT_FRAME):
    """Return (q, k, v) as contiguous CPU bfloat16 tensors [heads][tokens][head_dim]."""
    if dist not in ("iid", "frame"):
        raise ValueError(dist)
    rq, rk, rv, rs = (_rng(seed, t) for t in (_TAG_Q, _TAG_K, _TAG_V, _TAG_SHARED))
    q = torch.empty((heads, tokens, head_dim), dtype=torch.bfloat16)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    frames = -(-tokens // frame_tokens) if tokens else 0
    frame_of = np.arange(tokens) // frame_tokens
    for h in range(heads):
        nq = rq.standard_normal((tokens, head_dim), dtype=np.float32)
        nk = rk.standard_normal((tokens, head_dim), dtype=np.float32)
        nv = rv.standard_normal((tokens, head_dim), dtype=np.float32)
        if dist == "frame":
            s = rs.standard_normal((frames, head_dim), dtype=np.float32)
            shared = s[frame_of]
            nq = shared + np.float32(0.5) * nq
            nk = shared + np.float32(0.5) * nk
        q[h] = _to_bf16(nq)
        k[h] = _to_bf16(nk)
        v[h] = _to_bf16(nv)
    return q, k, v


def make_inputs(config_id: int, heads: int | None = None):
    """Inputs of one of the five workloads; ``heads`` may ask for fewer heads
    (the first ``heads`` of the same seeded streams)."""
    c = CONFIGS[config_id]
    return make_qkv(c.tokens, c.heads if heads is None else heads, c.dist, c.seed)


# Packed-sequence workload of VSA-H3 (FastH3 page, "Lever two"): a non-video
# prefix (text, condition keyframes, audio) ahead of the generated video.  The
# pages give no prefix length; 512 tokens is this stand-in's choice.
VSA_PREFIX = 512
VSA_GRID_72 = (72, 24, 42)       # 72,576 video tokens (10 s clip)


def make_packed_qkv(prefix: int, grid, heads: int, seed: int):
    """(q, k, v) CPU bf16 [heads][prefix + frames*height*width][128]: an i.i.d.
    prefix followed by frame-correlated video tokens in (t, h, w) raster order
    (the video part is make_qkv's "frame" recipe with frames of height*width
    tokens; the prefix draws from the streams of seed + 1000)."""
    frames, height, width = grid
    vq, vk, vv = make_qkv(frames * height * width, heads, "frame", seed,
                          frame_tokens=height * width)
    if prefix == 0:
        return vq, vk, vv
    pq, pk, pv = make_qkv(prefix, heads, "iid", seed + 1000)
    return tuple(torch.cat([a, b], dim=1).contiguous() for a, b in ((pq, vq), (pk, vk), (pv, vv)))



def make_vda_inputs(frames: int, heads: int, seed: int, frame_tokens: int = TOKENS_PER_LATENT_FRAME):
    """Inputs of the Video Delta Attention branch (synthetic; the pages give no
    activations): q, k unit-length directions (normalized N(0, I) draws, as the
    branch L2-normalizes them) and v N(0, 1), all bf16 [heads][frames *
    frame_tokens][128]; beta U(0.05, 0.95) per token, alpha U(0.8, 1.0) per
    frame and key dim, s_text 0.1 N(0, 1) [heads][128][128], all float32."""
    N = frames * frame_tokens
    rq, rk, rv, rs = (_rng(seed, t) for t in (_TAG_Q, _TAG_K, _TAG_V, _TAG_SHARED))
    out = []
    for r, unit in ((rq, True), (rk, True), (rv, False)):
        x = r.standard_normal((heads, N, HEAD_DIM), dtype=np.float32)
        if unit:
            x = x / np.linalg.norm(x, axis=2, keepdims=True)
        out.append(_to_bf16(x))
    beta = torch.from_numpy(rs.uniform(0.05, 0.95, (heads, N)).astype(np.float32))
    alpha = torch.from_numpy(rs.uniform(0.8, 1.0, (heads, frames, HEAD_DIM)).astype(np.float32))
    s_text = torch.from_numpy((0.1 * rs.standard_normal((heads, HEAD_DIM, HEAD_DIM))).astype(np.float32))
    return (*out, beta, alpha, s_text)
