// Internal launch interface between the C ABI (api.hip) and the gfx950 kernels.
// Not installed; every pointer here has already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fvattn {

constexpr int kHeadDim = 128;
constexpr int kTile = 128;        // selection tile (tokens)

// Frame-window description for the windowed softmax (latent frames of
// frame_tokens tokens, chunks of chunk_frames frames, `neighbours` chunks on
// each side, first and last frame as anchors); counts[t] = number of key tiles
// listed for query tile t.
struct WindowParams {
  const int32_t* counts = nullptr;
  int frame_tokens = 0;
  int chunk_frames = 1;
  int neighbours = 0;
  int frames = 0;
  // query block walked first within each head: the blocks from here to the
  // end (they hold the last frame, whose rows see every key) are the longest,
  // and starting with them keeps them out of the tail of the launch
  int first_block = 0;
};

// Dense (idx == nullptr) or tile-list (idx != nullptr, `keep` entries per query
// tile) attention forward over `heads` heads.
hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* out, const int32_t* idx, int keep, int heads, int tokens,
                            float scale, hipStream_t stream);

// Query rows per workgroup of the windowed softmax, and so per key-tile list.
constexpr int kWindowRows = 256;
// Bit set in an internal window-list entry when the key tile needs
// per-element masking for some row of the block (a disallowed frame, or keys
// past the sequence end).
constexpr int kMaskFlag = 1 << 30;

// Windowed softmax: key-tile lists idx [ceil(N / kWindowRows)][T] (row b lists
// counts[b] tiles, ascending; shared by every head).
hipError_t launch_attention_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* out, const int32_t* idx, const WindowParams& wp,
                                   int heads, int tokens, float scale, hipStream_t stream);

// Key-tile lists of the frame window for query blocks of q_rows rows (a
// multiple of 128): idx [ceil(N / q_rows)][T] (padded with -1), counts
// [ceil(N / q_rows)]; with `flags`, entries carry kMaskFlag.
hipError_t launch_window_tiles(int tokens, const WindowParams& wp, int q_rows, bool flags,
                               int32_t* idx, int32_t* counts, hipStream_t stream);

// S1: fp64 tile means.  transposed == false: out [heads][T][128];
// transposed == true: out [heads][128][T].
hipError_t launch_tile_means(const uint16_t* x, double* out, int heads, int tokens,
                             bool transposed, hipStream_t stream);

// S2 + S3: canonical fp64 scores of qm [heads][T][128] against kmT
// [heads][128][T]; with scores_out != nullptr the scores are written
// [heads][T][T] and no selection happens, otherwise the top `keep` tiles of
// every row go to idx_out [heads][T][keep], ascending.
hipError_t launch_score_select(const double* qm, const double* kmT, int heads, int tiles,
                               int keep, int32_t* idx_out, double* scores_out,
                               hipStream_t stream);

// [heads][T][128] -> [heads][128][T] (fp64), for the score diagnostic entry.
hipError_t launch_transpose_means(const double* in, double* out, int heads, int tiles,
                                  hipStream_t stream);

}  // namespace fvattn
