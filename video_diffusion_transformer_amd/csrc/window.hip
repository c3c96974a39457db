// Key-tile lists of the frame-window softmax (the softmax branch of Video
// DeltaNet, FreeVideo page, section "Where Video DeltaNet comes in": a chunk
// of latent frames sees its neighbouring chunks, and the first and last
// frames see and are seen by every frame).
//
// One wave per block of q_rows query tokens (128, the tile size, for both the
// public lists and the attention workgroups).  A key tile is listed when some query of the
// block may attend to some key of it.  Non-video tokens (text, audio) ahead of
// the video keep full softmax attention: a block holding a prefix row lists every
// tile, and a tile holding a prefix key is listed for every block.  Frames inside a tile are contiguous
// and chunks grow with frames, so this is a closed-form interval test: either
// tile holds an anchor frame, or the chunk ranges of the two tiles lie within
// `neighbours` of each other.  Listed tiles are compacted in ascending order
// with ballots; the rest of the row is filled with -1.
//
// For the attention kernel a listed tile is also flagged when some pair of a
// query of the block and a key of the tile is disallowed (or the tile is cut
// by the sequence end), so that only flagged tiles pay for per-element
// masking.  Every pair is allowed when one side's non-anchor frames are empty
// or the farthest pair of non-anchor chunks is within `neighbours`.

#include "fvattn_internal.h"

namespace fvattn {
namespace {

__global__ __launch_bounds__(64) void window_tiles_kernel(int N, ListParams wp, int q_rows,
                                                          bool flags, int T,
                                                          int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ counts) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int P = wp.prefix, ft = wp.frame_tokens, chunk = wp.chunk_frames, nb = wp.neighbours;
  const int last = wp.frames - 1;
  const int q_lo = t * q_rows, q_hi = (q_lo + q_rows < N ? q_lo + q_rows : N) - 1;
  // prefix rows see every key; the frame arithmetic below is for the
  // block's video rows [max(q_lo, P), q_hi] (none when q_hi < P)
  const bool q_pre = q_lo < P, q_vid = q_hi >= P;
  const int qf_lo = ((q_lo > P ? q_lo : P) - P) / ft, qf_hi = (q_hi - P) / ft;
  const bool q_anchor = qf_lo == 0 || qf_hi >= last;
  const int qc_lo = qf_lo / chunk, qc_hi = qf_hi / chunk;
  // non-anchor query frames [qa_lo, qa_hi] (empty when qa_lo > qa_hi)
  const int qa_lo = qf_lo > 1 ? qf_lo : 1, qa_hi = qf_hi < last - 1 ? qf_hi : last - 1;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* row = idx + (size_t)t * T;
  int base = 0;
  for (int j0 = 0; j0 < T; j0 += 64) {
    const int j = j0 + lane;
    bool need = false;
    int entry = j;
    if (j < T) {
      const int k_lo = j * kTile, k_hi = (k_lo + kTile < N ? k_lo + kTile : N) - 1;
      const bool k_pre = k_lo < P, k_vid = k_hi >= P;
      const int kf_lo = ((k_lo > P ? k_lo : P) - P) / ft, kf_hi = (k_hi - P) / ft;
      const bool k_anchor = kf_lo == 0 || kf_hi >= last;
      const int kc_lo = kf_lo / chunk, kc_hi = kf_hi / chunk;
      const bool video_need =
          q_vid && k_vid && (q_anchor || k_anchor || (kc_lo <= qc_hi + nb && kc_hi >= qc_lo - nb));
      need = q_pre || k_pre || video_need;
      const int ka_lo = kf_lo > 1 ? kf_lo : 1, ka_hi = kf_hi < last - 1 ? kf_hi : last - 1;
      const bool all_ok = !q_vid || !k_vid || qa_lo > qa_hi || ka_lo > ka_hi ||
                          (ka_hi / chunk - qa_lo / chunk <= nb && qa_hi / chunk - ka_lo / chunk <= nb);
      if (flags && (!all_ok || k_hi - k_lo + 1 < kTile)) entry |= kMaskFlag;
    }
    const uint64_t m = __ballot(need);
    if (need) row[base + __popcll(m & lt)] = entry;
    base += __popcll(m);
  }
  for (int p = base + lane; p < T; p += 64) row[p] = -1;
  if (lane == 0) counts[t] = base;
}

}  // namespace

hipError_t launch_window_tiles(int tokens, const ListParams& wp, int q_rows, bool flags,
                               int32_t* idx, int32_t* counts, hipStream_t stream) {
  const int T = (tokens + kTile - 1) / kTile;
  const int blocks = (tokens + q_rows - 1) / q_rows;
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(window_tiles_kernel, dim3(blocks), dim3(64), 0, stream, tokens, wp, q_rows,
                     flags, T, idx, counts);
  return hipGetLastError();
}

}  // namespace fvattn
