// Key-tile lists of the frame-window softmax (the softmax branch of Video
// DeltaNet, FreeVideo page, section "Where Video DeltaNet comes in": a chunk
// of latent frames sees its neighbouring chunks, and the first and last
// frames see and are seen by every frame).
//
// One wave per 128-token query tile.  A key tile is listed when some query of
// the tile may attend to some key of it.  Frames inside a tile are contiguous
// and chunks grow with frames, so this is a closed-form interval test: either
// tile holds an anchor frame, or the chunk ranges of the two tiles lie within
// `neighbours` of each other.  Listed tiles are compacted in ascending order
// with ballots; the rest of the row is filled with -1.

#include "fvattn_internal.h"

namespace fvattn {
namespace {

__global__ __launch_bounds__(64) void window_tiles_kernel(int N, WindowParams wp, int T,
                                                          int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ counts) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int ft = wp.frame_tokens, chunk = wp.chunk_frames, nb = wp.neighbours;
  const int last = wp.frames - 1;
  const int q_lo = t * kTile, q_hi = (q_lo + kTile < N ? q_lo + kTile : N) - 1;
  const int qf_lo = q_lo / ft, qf_hi = q_hi / ft;
  const bool q_anchor = qf_lo == 0 || qf_hi >= last;
  const int qc_lo = qf_lo / chunk, qc_hi = qf_hi / chunk;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* row = idx + (size_t)t * T;
  int base = 0;
  for (int j0 = 0; j0 < T; j0 += 64) {
    const int j = j0 + lane;
    bool need = false;
    if (j < T) {
      const int k_lo = j * kTile, k_hi = (k_lo + kTile < N ? k_lo + kTile : N) - 1;
      const int kf_lo = k_lo / ft, kf_hi = k_hi / ft;
      const bool k_anchor = kf_lo == 0 || kf_hi >= last;
      const int kc_lo = kf_lo / chunk, kc_hi = kf_hi / chunk;
      need = q_anchor || k_anchor || (kc_lo <= qc_hi + nb && kc_hi >= qc_lo - nb);
    }
    const uint64_t m = __ballot(need);
    if (need) row[base + __popcll(m & lt)] = j;
    base += __popcll(m);
  }
  for (int p = base + lane; p < T; p += 64) row[p] = -1;
  if (lane == 0) counts[t] = base;
}

}  // namespace

hipError_t launch_window_tiles(int tokens, const WindowParams& wp, int32_t* idx, int32_t* counts,
                               hipStream_t stream) {
  const int T = (tokens + kTile - 1) / kTile;
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(window_tiles_kernel, dim3(T), dim3(64), 0, stream, tokens, wp, T, idx, counts);
  return hipGetLastError();
}

}  // namespace fvattn
