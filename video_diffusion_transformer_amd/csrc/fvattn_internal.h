// Internal launch interface between the C ABI (api.hip) and the gfx950 kernels.
// Not installed; every pointer here has already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fvattn {

constexpr int kHeadDim = 128;
constexpr int kTile = 128;        // selection tile (tokens)

// Geometry of a VSA-H3 packed sequence: `prefix` non-video tokens, then a
// frames x height x width latent grid of video tokens, cut into tt x th x tw
// tiles (size S = tt th tw in {64, 128, 256}).  The kernels work in a padded
// tile layout of npad slots: slots [0, ppad) hold the prefix (ppad = prefix
// rounded up to 256), then video tile j owns slots [ppad + j S, ppad + (j+1) S)
// with its valid tokens first, in (t, h, w) raster order.
struct VsaGeom {
  int prefix = 0, ppad = 0, frames = 0, height = 0, width = 0;
  int tt = 1, th = 1, tw = 1, nh = 1, nw = 1, size = 64, tiles = 0, npad = 0, tokens = 0;
};

// Tile j of the grid: first latent frame/row/column and extents (clipped at
// the grid edge).
struct VsaTile {
  int t0, h0, w0, et, eh, ew;
};

__host__ __device__ inline VsaTile vsa_tile(const VsaGeom& g, int j) {
  VsaTile r;
  const int a = j / (g.nh * g.nw), rem = j - a * g.nh * g.nw;
  const int b = rem / g.nw, c = rem - b * g.nw;
  r.t0 = a * g.tt;
  r.h0 = b * g.th;
  r.w0 = c * g.tw;
  r.et = g.frames - r.t0 < g.tt ? g.frames - r.t0 : g.tt;
  r.eh = g.height - r.h0 < g.th ? g.height - r.h0 : g.th;
  r.ew = g.width - r.w0 < g.tw ? g.width - r.w0 : g.tw;
  return r;
}

// Token (index in the packed sequence) held by padded slot `slot`, or -1 for a
// padding slot or a slot past npad.
__host__ __device__ inline int vsa_slot_token(const VsaGeom& g, int slot) {
  if (slot < 0 || slot >= g.npad) return -1;
  if (slot < g.ppad) return slot < g.prefix ? slot : -1;
  const int j = (slot - g.ppad) / g.size, r = slot - g.ppad - j * g.size;
  const VsaTile t = vsa_tile(g, j);
  if (r >= t.et * t.eh * t.ew) return -1;
  const int dt = r / (t.eh * t.ew), r2 = r - dt * t.eh * t.ew;
  const int dh = r2 / t.ew, dw = r2 - dh * t.ew;
  return g.prefix + ((t.t0 + dt) * g.height + (t.h0 + dh)) * g.width + (t.w0 + dw);
}

// Valid tokens among the 64 slots [64 s, 64 s + 64).
__host__ __device__ inline int vsa_sub_count(const VsaGeom& g, int s) {
  const int slot0 = 64 * s;
  int n;
  if (slot0 < g.ppad) {
    n = g.prefix - slot0;
  } else {
    const int j = (slot0 - g.ppad) / g.size, m = (slot0 - g.ppad - j * g.size) / 64;
    const VsaTile t = vsa_tile(g, j);
    n = t.et * t.eh * t.ew - 64 * m;
  }
  return n < 0 ? 0 : (n > 64 ? 64 : n);
}

// VSA list entry of one 64-key sub-tile: bits 0-15 sub-tile index, 16-21 valid
// keys - 1, 22-25 the 64-row query groups of the block that attend to it, and
// kMaskFlag when some group does not or some key is padding.
constexpr int kVsaCountShift = 16, kVsaGroupShift = 22;
// Query rows per VSA-H3 attention workgroup and per key list: a multiple of
// 64 (one group per 64 rows, at most four groups), one wave per 32 rows.
constexpr int kVsaRows = 128;

// Per-launch parameters of the list-driven modes.  Frame window: `prefix`
// non-video tokens, then latent frames of frame_tokens tokens, chunks of
// chunk_frames frames, `neighbours` chunks on each side, first and last frame
// as anchors; counts[b] = number of list entries of query block b.  VSA: the
// geometry above, and counts[h B + b].
struct ListParams {
  const int32_t* counts = nullptr;
  // Frame window: non-video tokens (text, audio) ahead of the video; they see
  // and are seen by every token, and video frames are counted after them
  int prefix = 0;
  int frame_tokens = 0;
  int chunk_frames = 1;
  int neighbours = 0;
  int frames = 0;
  // query block walked first within each head: the blocks from here to the
  // end (they hold the last frame, whose rows see every key) are the longest,
  // and starting with them keeps them out of the tail of the launch
  int first_block = 0;
  VsaGeom vsa;
  // INT8 query-key mode: per-64-key-block key scales [heads][ceil(N / 64)]
  const float* kscale = nullptr;
  // Frame window: the geometry of the list array the caller allocated, rows
  // per list (query rows one list covers), number of lists and int32 entries
  // per list.  The launcher refuses a layout the kernel would index past.
  int list_rows = 0, list_count = 0, list_stride = 0;
};

// hipSuccess when a frame-window list array of `wp` fits the attention
// kernel over `tokens` tokens (kWindowRows rows per list, one list per
// kWindowRows-row block, at least one entry per 128-token key tile per list),
// hipErrorInvalidValue otherwise.  Host arithmetic only.
hipError_t window_lists_fit(int tokens, const ListParams& wp);

// Dense (idx == nullptr) or tile-list (idx != nullptr, `keep` entries per query
// tile) attention forward over `heads` heads.
hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* out, const int32_t* idx, int keep, int heads, int tokens,
                            float scale, hipStream_t stream);

// Query rows per workgroup of the windowed softmax, and so per key-tile list.
constexpr int kWindowRows = 128;
// Bit set in an internal window-list entry when the key tile needs
// per-element masking for some row of the block (a disallowed frame, or keys
// past the sequence end).
constexpr int kMaskFlag = 1 << 30;

// Windowed softmax: key-tile lists idx [ceil(N / kWindowRows)][T] (row b lists
// counts[b] tiles, ascending; shared by every head).
hipError_t launch_attention_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* out, const int32_t* idx, const ListParams& wp,
                                   int heads, int tokens, float scale, hipStream_t stream);

// Key-tile lists of the frame window for query blocks of q_rows rows (a
// multiple of 128): idx [ceil(N / q_rows)][T] (padded with -1), counts
// [ceil(N / q_rows)]; with `flags`, entries carry kMaskFlag.
hipError_t launch_window_tiles(int tokens, const ListParams& wp, int q_rows, bool flags,
                               int32_t* idx, int32_t* counts, hipStream_t stream);

// VSA-H3: K and V into the padded tile layout (padding slots zeroed):
// kp, vp [heads][npad][128].
hipError_t launch_vsa_pack(const uint16_t* k, const uint16_t* v, uint16_t* kp, uint16_t* vp,
                           const VsaGeom& g, int heads, hipStream_t stream);

// VSA-H3: fp64 means of every video tile of q and of k (original layout),
// summed in the tile's token order, in one launch: qmT, kmT [heads][128][tiles].
hipError_t launch_vsa_means(const uint16_t* q, const uint16_t* k, double* qmT, double* kmT,
                            const VsaGeom& g, int heads, hipStream_t stream);

// VSA-H3: per (head, kVsaRows-row query block) the ascending list of 64-key
// sub-tiles its rows attend to, from the kept video tiles idx [heads][tiles][keep]:
// lists [heads][blocks][npad / 64], counts [heads][blocks].
hipError_t launch_vsa_lists(const int32_t* idx, int keep, const VsaGeom& g, int heads,
                            int32_t* lists, int32_t* counts, hipStream_t stream);

// VSA-H3 attention: q and out in the packed token order (the caller's
// layout), kp and vp in the padded tile layout, lists and lp.counts from
// launch_vsa_lists.
hipError_t launch_attention_vsa(const uint16_t* q, const uint16_t* kp, const uint16_t* vp,
                                uint16_t* out, const int32_t* lists, const ListParams& lp,
                                int heads, float scale, hipStream_t stream);

// INT8 (or, with fp8, OCP E4M3) keys: codes [heads][tokens][128] bytes and
// per-64-key-block scales [heads][ceil(tokens / 64)] float.
hipError_t launch_quantize_k(const uint16_t* k, uint8_t* codes, float* scales, int heads,
                             int tokens, bool fp8, hipStream_t stream);

// Dense attention with INT8 query-key scores: kq = codes from launch_quantize_k
// (lp.kscale = their scales); queries are quantized per row in the kernel.
hipError_t launch_attention_int8(const uint16_t* q, const uint8_t* kq, const uint16_t* v,
                                 uint16_t* out, const ListParams& lp, int heads, int tokens,
                                 float scale, hipStream_t stream);

// Dense attention with FP8 (E4M3) query-key scores: kq = E4M3 codes from
// launch_quantize_k with fp8 (lp.kscale = their scales); queries are
// quantized per row in the kernel.
hipError_t launch_attention_fp8(const uint16_t* q, const uint8_t* kq, const uint16_t* v,
                                uint16_t* out, const ListParams& lp, int heads, int tokens,
                                float scale, hipStream_t stream);

// Video Delta Attention: forward and reverse states [heads][frames + 1][128][128]
// (fp32) from k, v (bf16 [heads][frames * ft][128]), beta [heads][frames * ft],
// alpha [heads][frames][128] and s_text [heads][128][128]; scratch holds
// 5 * heads * frames * 128 * 128 floats.
hipError_t launch_vda_states(const uint16_t* k, const uint16_t* v, const float* beta,
                             const float* alpha, const float* s_text, int heads, int frames,
                             int ft, float* scratch, float* fwd, float* rev, hipStream_t stream);

// Video Delta Attention readout: out (fp32 [heads][frames * ft][128]) =
// (fwd[lo] + rev[hi]) q per query of each frame.
hipError_t launch_vda_readout(const uint16_t* q, const float* fwd, const float* rev, int heads,
                              int frames, int ft, int chunk, int nb, float* out, hipStream_t stream);

// S1: fp64 tile means out [heads][T][128].
hipError_t launch_tile_means(const uint16_t* x, double* out, int heads, int tokens,
                             hipStream_t stream);

// S1 for one selection: query and key means in one launch, both transposed:
// qmT, kmT [heads][128][T].
hipError_t launch_tile_means_qk(const uint16_t* q, const uint16_t* k, double* qmT, double* kmT,
                                int heads, int tokens, hipStream_t stream);

// S2: canonical fp64 scores of qmT against kmT (both [heads][128][T]) into
// scores_out [heads][T][T].
hipError_t launch_scores(const double* qmT, const double* kmT, int heads, int tiles,
                         double* scores_out, hipStream_t stream);

// S3: the top `keep` tiles of every row of scores [heads][T][T] into idx_out
// [heads][T][keep], ascending (T <= 2048).
hipError_t launch_select(const double* scores, int heads, int tiles, int keep, int32_t* idx_out,
                         hipStream_t stream);

// Matrix-core rate probe: kProbeBlocks workgroups of 256 threads, each wave
// `iters` iterations of four bf16 32x32x16 MFMAs; one float per thread into
// sink (kProbeBlocks * 256 floats).
constexpr int kProbeBlocks = 1024;
hipError_t launch_mfma_probe(float* sink, int iters, hipStream_t stream);

// [heads][T][128] -> [heads][128][T] (fp64), for the score diagnostic entry.
hipError_t launch_transpose_means(const double* in, double* out, int heads, int tiles,
                                  hipStream_t stream);

}  // namespace fvattn
