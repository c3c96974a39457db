"""fp64 CPU oracle for VSA-H3's packed-sequence attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It shares no code with
the HIP library and imports nothing from it.

What is computed (FastH3 page, "FastH3 Preview v1: four calls, one-tenth the
attention...", section "Lever two: VSA-H3 makes each of the four calls
cheaper"):

* The sequence is packed as [text | condition keyframes | audio | generated
  video]; everything before the generated video is the non-video prefix of
  ``prefix`` tokens.  The video part is a (t, h, w) latent grid, token index
  t * height * width + h * width + w after the prefix (24 x 42 = 1,008 tokens
  per latent frame at 1344x768: FreeVideo page, section "What MiniMax H3 is,
  briefly").
* Only the video part is cut into 3D tiles over that grid, (4, 4, 4) = 64
  tokens (FastH3's trained shape) or (4, 8, 8) = 256.
* A coarse pooled score ranks every video key tile against each video query
  tile, and compute_topk keeps max(1, min(ceil(keep_frac * tiles), tiles)) of
  them.
* Non-video keys are exempt: every video query sees all of them in addition to
  its kept tiles; they never compete for a slot.
* Non-video queries are dense: they see every key.
* The compression branch contributes nothing (base weights), so the softmax is
  exact over the keys a query sees.

Readings taken where the page is silent:

* Tiles are enumerated t-tile slowest, w-tile fastest; a tile's tokens are
  taken in (t, h, w) raster order, which is ascending token order.
* A grid extent that the tile does not divide (42 = 10 x 4 + 2) leaves partial
  tiles at that edge; they hold only their valid tokens.
* Pooling, score precision and ties follow the 1-D selection of
  ``attention.py``: fp64 mean over the tile's valid tokens (sum from +0.0 in
  the tile's token order, one division), unscaled fp64 dot product in order
  d = 0..127 without fused multiply-add, the k largest with ties to the lower
  tile index, kept tiles listed ascending.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_rows, keep_count, tile_scores, top_tiles


def video_tiles(frames: int, height: int, width: int, tile=(4, 4, 4)) -> list:
    """Video-relative token indices of every 3D tile, in tile order.

    Returns a list of int64 arrays; tile (a, b, c) covers latent frames
    [a tt, (a+1) tt), rows [b th, (b+1) th) and columns [c tw, (c+1) tw),
    clipped to the grid.
    """
    tt, th, tw = tile
    grid = np.arange(frames * height * width, dtype=np.int64).reshape(frames, height, width)
    out = []
    for a in range(0, frames, tt):
        for b in range(0, height, th):
            for c in range(0, width, tw):
                out.append(grid[a:a + tt, b:b + th, c:c + tw].reshape(-1))
    return out


def video_tile_means(x: np.ndarray, tiles: list) -> np.ndarray:
    """Mean of each tile's tokens, for one head.

    x: [Nv, d] float64 (the video part).  The sum of a tile runs over its
    tokens in the listed order starting from +0.0; the mean is one correctly
    rounded division by the tile's token count.
    """
    d = x.shape[1]
    size = max(len(t) for t in tiles)
    slot = np.full((len(tiles), size), -1, dtype=np.int64)   # i-th token of every tile
    for j, toks in enumerate(tiles):
        slot[j, :len(toks)] = toks
    acc = np.zeros((len(tiles), d), dtype=np.float64)
    for i in range(size):
        live = slot[:, i] >= 0
        acc[live] = acc[live] + x[slot[live, i]]
    counts = np.array([len(t) for t in tiles], dtype=np.float64)
    return acc / counts[:, None]


def vsa_select(q: np.ndarray, k: np.ndarray, prefix: int, grid, tile, keep_frac: float) -> np.ndarray:
    """Kept video key tiles of every head and video query tile.

    q, k: [H, N, d] float64 with N = prefix + frames * height * width.
    Returns int32 [H, Tv, kk], kk = keep_count(Tv, keep_frac), ascending.
    """
    H, N, _ = q.shape
    frames, height, width = grid
    assert N == prefix + frames * height * width
    tiles = video_tiles(frames, height, width, tile)
    Tv = len(tiles)
    kk = keep_count(Tv, keep_frac)
    out = np.empty((H, Tv, kk), dtype=np.int32)
    for h in range(H):
        qm = video_tile_means(q[h, prefix:], tiles)
        km = video_tile_means(k[h, prefix:], tiles)
        out[h] = top_tiles(tile_scores(qm, km), kk)
    return out


def vsa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, prefix: int, grid,
                  tile, keep_frac: float, rows=None, idx=None) -> np.ndarray:
    """VSA-H3 attention of every head, in the packed token order.

    q, k, v: [H, N, d] float64.  ``rows`` (optional): query rows to compute
    (same for every head).  ``idx``: kept tiles from ``vsa_select`` (computed
    here when not given).  Returns [H, len(rows), d] float64.
    """
    H, N, d = q.shape
    frames, height, width = grid
    tiles = video_tiles(frames, height, width, tile)
    if idx is None:
        idx = vsa_select(q, k, prefix, grid, tile, keep_frac)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    tile_of = np.empty(N - prefix, dtype=np.int64)
    for j, toks in enumerate(tiles):
        tile_of[toks] = j
    exempt = np.arange(prefix)
    out = np.empty((H, len(rows), d), dtype=np.float64)
    text_sel = np.nonzero(rows < prefix)[0]
    vid_sel = np.nonzero(rows >= prefix)[0]
    vid_tile = tile_of[rows[vid_sel] - prefix]
    for h in range(H):
        if len(text_sel):
            out[h, text_sel] = attention_rows(q[h, rows[text_sel]], k[h], v[h], scale)
        for a in np.unique(vid_tile):
            sel = vid_sel[vid_tile == a]
            keys = np.concatenate([exempt] + [prefix + tiles[j] for j in idx[h, a]])
            out[h, sel] = attention_rows(q[h, rows[sel]], k[h, keys], v[h, keys], scale)
    return out
