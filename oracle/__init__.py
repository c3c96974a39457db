"""fp64 CPU oracle for video-token attention (dense, block-sparse, frame
window, VSA-H3 packed sequence, INT8 and FP8 query-key scores, Video Delta
Attention).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library or its binding.
"""

from .attention import (TILE, attention_rows, dense, keep_count, kept_keys, select_tiles,
                        sparse, tile_count, tile_means, tile_scores, top_tiles, window_attention,
                        window_density, window_frames_allowed, window_tiles)
from .int8 import KEY_BLOCK, int8_scores_attention, quantize_blocks, quantize_rows
from .fp8 import e4m3_decode, e4m3_round, fp8_scores_attention
from .vda import read_positions, scan_states, vda_attention
from .vsa import video_tile_means, video_tiles, vsa_attention, vsa_select
from .widen import widen

__all__ = ["e4m3_decode", "e4m3_round", "fp8_scores_attention", "read_positions", "scan_states", "vda_attention", "KEY_BLOCK", "int8_scores_attention", "quantize_blocks", "quantize_rows", "TILE", "attention_rows", "dense", "keep_count", "kept_keys", "select_tiles",
           "sparse", "tile_count", "tile_means", "tile_scores", "top_tiles", "widen",
           "video_tile_means", "video_tiles", "vsa_attention", "vsa_select",
           "window_attention", "window_density", "window_frames_allowed", "window_tiles"]
