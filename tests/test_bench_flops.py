"""The effective-FLOP counts bench.py divides by, against brute-force counts of
the attended (query, key) pairs built from the oracle's own definitions.

Every figure bench.py reports as TFLOP/s is 4 * d * (attended query-key pairs)
/ time, so a miscount would misstate every rate.  CPU only.
"""

import numpy as np
import pytest

import bench
import oracle
from oracle import vsa as ovsa

D = 128


def _random_lists(rng, heads, rows, tiles, keep):
    idx = np.empty((heads, rows, keep), dtype=np.int32)
    for h in range(heads):
        for t in range(rows):
            idx[h, t] = np.sort(rng.choice(tiles, keep, replace=False))
    return idx


@pytest.mark.parametrize("N,keep", [(1000, 3), (128, 1), (129, 2), (2000, 16)])
def test_sparse_flops_counts_the_kept_keys_of_every_row(N, keep):
    rng = np.random.default_rng(N)
    T = oracle.tile_count(N)
    idx = _random_lists(rng, 2, T, T, keep)
    pairs = 0
    for h in range(2):
        for i in range(N):
            pairs += len(oracle.kept_keys(idx[h, i // 128], N))
    assert bench.sparse_flops(idx, N) == 4.0 * D * pairs


@pytest.mark.parametrize("N,ft,chunk,nb", [(1000, 64, 2, 1), (700, 100, 3, 0), (5040, 1008, 5, 1),
                                           (64, 64, 5, 1)])
def test_window_flops_counts_the_allowed_pairs(N, ft, chunk, nb):
    frames = -(-N // ft)
    allowed = oracle.window_frames_allowed(frames, chunk, nb)
    f = np.arange(N) // ft
    pairs = int(allowed[f][:, f].sum())
    assert bench.window_flops(N, ft, chunk, nb, heads=3) == 4.0 * D * 3 * pairs


@pytest.mark.parametrize("N,P,ft,chunk,nb", [(1000, 37, 64, 2, 1), (700, 300, 100, 3, 0), (5040, 128, 1008, 5, 1),
                                             (128, 64, 64, 5, 1)])
def test_window_flops_with_prefix_counts_the_allowed_pairs(N, P, ft, chunk, nb):
    frames = -(-(N - P) // ft)
    allowed = oracle.window_frames_allowed(frames, chunk, nb)
    f = np.arange(N - P) // ft
    pairs = int(allowed[f][:, f].sum()) + P * N + (N - P) * P
    assert bench.window_flops(N, ft, chunk, nb, heads=3, prefix=P) == 4.0 * D * 3 * pairs
    # the oracle's own output agrees on which keys a row sees: a window over a
    # whole-frame video part has the oracle's closed-form density
    if (N - P) % ft == 0:
        dens = oracle.window_density(P, frames, ft, chunk, nb)
        assert abs(bench.window_flops(N, ft, chunk, nb, heads=1, prefix=P) / (4.0 * D * N * N) - dens) < 1e-12


@pytest.mark.parametrize("prefix,grid,tile,keep", [(37, (5, 6, 7), (4, 4, 4), 3), (0, (4, 8, 8), (4, 8, 8), 1),
                                                  (100, (9, 10, 6), (4, 4, 4), 5)])
def test_vsa_flops_counts_prefix_rows_and_kept_tiles(prefix, grid, tile, keep):
    rng = np.random.default_rng(prefix + keep)
    tiles = ovsa.video_tiles(*grid, tile)
    Tv = len(tiles)
    idx = _random_lists(rng, 2, Tv, Tv, keep)
    n = prefix + grid[0] * grid[1] * grid[2]
    pairs = 0
    for h in range(2):
        pairs += prefix * n                       # non-video queries see every key
        for a, toks in enumerate(tiles):          # a video query of tile a
            keys = prefix + sum(len(tiles[j]) for j in idx[h, a])
            pairs += len(toks) * keys
    assert bench.vsa_flops(idx, prefix, grid, tile) == 4.0 * D * pairs
