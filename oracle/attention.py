"""fp64 CPU oracle for dense and block-sparse video-token attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the HIP library and imports nothing from it.

Inputs are the exact bfloat16 values widened to float64 (exact).  Everything is
plain numpy: a matmul serves as a step of the dense definition, nothing else is
blocked, fused or reordered.

Sources (the pages are the authority on what is computed):

* Dense attention: the joint attention of MiniMax H3 is one bidirectional
  (non-causal) softmax attention over the packed token sequence (FastH3 page,
  "FastH3 Preview v1: four calls, one-tenth the attention...", section "Lever
  two: VSA-H3 makes each of the four calls cheaper"); scores are streamed, never
  materialized (FreeVideo page, section "Why it does not fit: the arithmetic").
  The oracle is the plain definition, softmax(scale * Q K^T) V.
* Tile selection: pooled tile summaries give a cheap score for every (query
  tile, key tile) pair, then ``compute_topk`` keeps max(1, min(ceil((1 - sparsity) * blocks),
  blocks)) tiles (FastH3 page, "Lever two").  The pages do not fix the pooling
  operator, the score precision or the tie rule; the readings used here are:
  mean over the valid tokens of a contiguous 128-token tile, fp64 sums in token
  order, one correctly rounded division, an unscaled fp64 dot product summed in
  order d = 0..127 with every product and every sum rounded (no fused
  multiply-add), the k largest scores with ties going to the lower tile index,
  emitted in ascending tile order.
* Sparse attention: exact attention restricted to the kept tiles, with the
  compression branch contributing nothing, which is the base-weight behaviour
  (FastH3 page, "Lever two": the base loader zero-initializes
  ``to_gate_compress``).  Softmax is normalized over the kept keys only.

* Windowed softmax (the softmax branch of Video DeltaNet): exact attention
  restricted to a window of latent-frame chunks plus two anchor frames
  (FreeVideo page, section "Where Video DeltaNet comes in"); see the readings
  at ``window_frames_allowed``.

Parity pins for every function live in tests/test_oracle_pins.py and
tests/test_oracle_window.py.
"""

from __future__ import annotations

import math

import numpy as np

TILE = 128


# --------------------------------------------------------------------------
# dense attention (definition)
# --------------------------------------------------------------------------

def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q k^T) v for a block of query rows of one head.

    q: [R, d]; k, v: [N, d], all float64.  Returns [R, d] float64.
    Non-causal: every query sees every key.
    """
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / l


def dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, rows=None,
          block: int = 256) -> np.ndarray:
    """Dense attention of every head.

    q, k, v: [H, N, d] float64.  ``rows`` (optional) is a 1-D index array of
    query rows to compute (the same rows for every head); the result is then
    [H, len(rows), d].
    """
    H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((H, len(rows), d), dtype=np.float64)
    for h in range(H):
        for b in range(0, len(rows), block):
            r = rows[b:b + block]
            out[h, b:b + len(r)] = attention_rows(q[h, r], k[h], v[h], scale)
    return out


# --------------------------------------------------------------------------
# tile selection (algorithm, in the order the FastH3 page gives it:
# coarse pooled scores first, then compute_topk decides how many survive)
# --------------------------------------------------------------------------

def tile_count(tokens: int, tile: int = TILE) -> int:
    """Number of contiguous ``tile``-token tiles (128 by default) covering ``tokens`` tokens."""
    return -(-tokens // tile)


def keep_count(num_tiles: int, keep_frac: float) -> int:
    """compute_topk's rule with keep_frac = 1 - sparsity, in IEEE double.

    A sequence with no tiles keeps none.
    """
    if num_tiles == 0:
        return 0
    return max(1, min(math.ceil(keep_frac * num_tiles), num_tiles))


def tile_means(x: np.ndarray, tile: int = TILE) -> np.ndarray:
    """Mean of each tile's valid tokens, for one head.

    x: [N, d] float64.  Returns [T, d] float64.  Each tile sum runs in token
    order starting from +0.0; the mean is one correctly rounded division by the
    number of valid tokens in the tile.
    """
    N, d = x.shape
    T = tile_count(N, tile)
    starts = np.arange(T) * tile
    counts = np.minimum(starts + tile, N) - starts
    acc = np.zeros((T, d), dtype=np.float64)
    for i in range(tile):          # i-th token of every tile, in token order
        live = i < counts
        acc[live] = acc[live] + x[starts[live] + i]
    return acc / counts[:, None].astype(np.float64)


def tile_scores(qm: np.ndarray, km: np.ndarray) -> np.ndarray:
    """sigma[i, j] = sum_d qm[i, d] * km[j, d] (unscaled), for one head.

    qm: [T, d], km: [T, d] float64.  The sum starts at +0.0 and runs d = 0..d-1;
    every product and every sum is one IEEE double rounding (separate numpy
    multiply and add, no fused multiply-add).
    """
    T, d = qm.shape
    acc = np.zeros((T, km.shape[0]), dtype=np.float64)
    for c in range(d):
        acc = acc + np.multiply.outer(qm[:, c], km[:, c])
    return acc


def top_tiles(sigma: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k largest scores (ties -> lower column), ascending.

    sigma: [T, T] float64.  Returns int32 [T, k].
    """
    T = sigma.shape[0]
    out = np.empty((T, k), dtype=np.int32)
    for i in range(T):
        order = np.argsort(-sigma[i], kind="stable")  # descending, stable on ties
        out[i] = np.sort(order[:k])
    return out


def select_tiles(q: np.ndarray, k: np.ndarray, keep_frac: float, tile: int = TILE) -> np.ndarray:
    """Tile indices kept for every head and query tile.

    q, k: [H, N, d] float64.  Returns int32 [H, T, kk] with kk = keep_count(T, keep_frac).
    """
    H, N, _ = q.shape
    T = tile_count(N, tile)
    kk = keep_count(T, keep_frac)
    out = np.empty((H, T, kk), dtype=np.int32)
    for h in range(H):
        sigma = tile_scores(tile_means(q[h], tile), tile_means(k[h], tile))
        out[h] = top_tiles(sigma, kk)
    return out


# --------------------------------------------------------------------------
# sparse attention (exact attention over the kept tiles only)
# --------------------------------------------------------------------------

def kept_keys(tiles, tokens: int, tile: int = TILE) -> np.ndarray:
    """Token indices of the given tiles (valid tokens only), tile order kept."""
    return np.concatenate([np.arange(t * tile, min(t * tile + tile, tokens)) for t in tiles])


def sparse(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, idx: np.ndarray,
           rows=None, tile: int = TILE) -> np.ndarray:
    """Block-sparse attention: query i of tile t sees only the tokens of tiles idx[h, t].

    q, k, v: [H, N, d] float64; idx: int [H, T, kk].  ``rows`` as in ``dense``.
    """
    H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((H, len(rows), d), dtype=np.float64)
    tile_of = rows // tile
    for h in range(H):
        for t in np.unique(tile_of):
            sel = np.nonzero(tile_of == t)[0]
            keys = kept_keys(idx[h, t], N, tile)
            out[h, sel] = attention_rows(q[h, rows[sel]], k[h, keys], v[h, keys], scale)
    return out


# --------------------------------------------------------------------------
# windowed softmax of Video DeltaNet's softmax branch (definition)
#
# FreeVideo page, section "Where Video DeltaNet comes in": softmax stays exact
# but only inside a window.  Queries are grouped in chunks of five latent
# frames; a chunk attends to its own frames and to the adjacent chunk on either
# side (15 frames in all).  The first and the last latent frame are visible to
# every query, and their own queries attend to every frame.  Readings taken here: latent frame of token i = i // frame_tokens;
# chunk of frame f = f // chunk_frames, counted from frame 0 (the last chunk
# may be short); "neighbours" chunks on each side.
# --------------------------------------------------------------------------

def window_frames_allowed(frames: int, chunk_frames: int = 5, neighbours: int = 1) -> np.ndarray:
    """Boolean [F, F]: may a query in frame qf attend to a key in frame kf."""
    f = np.arange(frames)
    chunk = f // chunk_frames
    allowed = np.abs(chunk[:, None] - chunk[None, :]) <= neighbours
    if frames:
        for anchor in (0, frames - 1):
            allowed[:, anchor] = True
            allowed[anchor, :] = True
    return allowed


def _window_token_frames(tokens: int, frame_tokens: int, prefix: int):
    """Per token: -1 for the non-video prefix, else the latent frame of the
    video token (counted from the first video token).  Returns (frames of
    the video part, the per-token array)."""
    video = tokens - prefix
    frames = -(-video // frame_tokens)
    tf = np.full(tokens, -1, dtype=np.int64)
    tf[prefix:] = np.arange(video) // frame_tokens
    return frames, tf


def window_tiles(tokens: int, frame_tokens: int, chunk_frames: int = 5, neighbours: int = 1,
                 prefix: int = 0):
    """Key tiles each 128-token query tile must visit: every key tile holding a
    key that some query of the tile may attend to.  With a non-video prefix
    (text, audio) of ``prefix`` tokens ahead of the video, every prefix key is
    visible to every query and a prefix query sees every key.  Returns (idx
    [T, T] int32, padded with -1, ascending; count [T] int32)."""
    T = tile_count(tokens)
    frames, token_frame = _window_token_frames(tokens, frame_tokens, prefix)
    allowed = window_frames_allowed(frames, chunk_frames, neighbours)
    idx = np.full((T, T), -1, dtype=np.int32)
    count = np.zeros(T, dtype=np.int32)
    for t in range(T):
        qf = token_frame[t * TILE:min(t * TILE + TILE, tokens)]
        if (qf < 0).any():                       # a prefix query sees every key
            key_ok = np.ones(tokens, dtype=bool)
        else:
            kframes = np.nonzero(allowed[np.unique(qf)].any(axis=0))[0]
            key_ok = (token_frame < 0) | np.isin(token_frame, kframes)
        tiles = np.unique(np.nonzero(key_ok)[0] // TILE)
        idx[t, :len(tiles)] = tiles
        count[t] = len(tiles)
    return idx, count


def window_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, frame_tokens: int,
                     chunk_frames: int = 5, neighbours: int = 1, rows=None,
                     prefix: int = 0) -> np.ndarray:
    """Softmax attention restricted to the window and anchor frames, per head.

    The sequence is ``prefix`` non-video tokens (text, audio) followed by the
    video tokens.  Text and audio tokens keep full softmax attention (FreeVideo
    page, "Where Video DeltaNet comes in"): a prefix query attends to every
    key, and every query attends to every prefix key; a video query attends to
    the video keys of its window and of the anchor frames.

    q, k, v: [H, N, d] float64.  ``rows`` as in ``dense``.
    """
    H, N, d = q.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    frames, token_frame = _window_token_frames(N, frame_tokens, prefix)
    allowed = window_frames_allowed(frames, chunk_frames, neighbours)
    out = np.empty((H, len(rows), d), dtype=np.float64)
    qframe = token_frame[rows]
    for h in range(H):
        for f in np.unique(qframe):
            sel = np.nonzero(qframe == f)[0]
            if f < 0:
                keys = np.arange(N)
            else:
                keys = np.nonzero((token_frame < 0) | allowed[f, np.maximum(token_frame, 0)])[0]
            out[h, sel] = attention_rows(q[h, rows[sel]], k[h, keys], v[h, keys], scale)
    return out


def window_density(prefix: int, frames: int, frame_tokens: int, chunk_frames: int = 5,
                   neighbours: int = 1) -> float:
    """Fraction of (query, key) pairs the window attends to, prefix included:
    prefix rows see all N keys, video rows see the P prefix keys plus their
    allowed video frames (whole frames of frame_tokens tokens)."""
    allowed = window_frames_allowed(frames, chunk_frames, neighbours).astype(np.float64)
    video = frames * frame_tokens
    n = prefix + video
    pairs = prefix * n + video * prefix + frame_tokens * frame_tokens * allowed.sum()
    return pairs / (n * n)

