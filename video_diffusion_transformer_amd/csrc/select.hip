// Tile selection for block-sparse attention on gfx950: the coarse stage of
// video sparse attention (FastH3 page, "FastH3 Preview v1: four calls,
// one-tenth the attention...", section "Lever two: VSA-H3 makes each of the
// four calls cheaper": pooled tiles are scored against the query tile, then
// compute_topk decides how many survive).
//
// S1  tile_means_kernel: mean of each contiguous 128-token tile of Q or K, in
//     fp64.  The sum runs in token order from +0.0 (one thread owns 8 head
//     dimensions of one tile and adds its tokens one after another), then one
//     IEEE-correct fp64 division by the number of valid tokens.  HBM-bound: it
//     reads Q and K once with 128-bit loads, 16 lanes per 256-byte token row.
// S2  score_select_kernel: sigma_ij = sum_d qm_i[d] * km_j[d] in fp64 from +0.0
//     in order d = 0..127, every product and every sum rounded on its own
//     (fp contraction is off in this file).  One workgroup owns 8 query tiles of
//     one head; their means sit in LDS and every thread walks one key tile
//     column of the transposed key means (coalesced), keeping 8 scores.
// S3  per query tile, the `keep` largest scores, ties to the lower key tile,
//     found by one wave with a most-significant-bit-first radix select on the
//     order-preserving 64-bit image of the doubles, then emitted in ascending
//     tile order with ballots.

#include "fvattn_internal.h"

#pragma clang fp contract(off)

namespace fvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMeansTiles = 16;   // tiles per workgroup in S1 (16 threads per tile)
constexpr int kRows = 8;          // query tiles per workgroup in S2/S3
constexpr int kMaxM = 32;         // FVATTN_MAX_TILES / 64 score slots per lane

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) {
  return (double)__uint_as_float(w & 0xffff0000u);
}

template <bool kTransposed>
__global__ __launch_bounds__(256) void tile_means_kernel(const uint16_t* __restrict__ X,
                                                         double* __restrict__ out, int N, int T) {
  __shared__ double stage[kHeadDim * kMeansTiles];
  const int h = blockIdx.y;
  const int tid = threadIdx.x, tt = tid >> 4, c = tid & 15;
  const int t = blockIdx.x * kMeansTiles + tt;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  if (t < T) {
    const int lo = t * kTile, hi = (lo + kTile < N) ? lo + kTile : N;
    const uint16_t* p = X + ((size_t)h * N + lo) * kHeadDim + 8 * c;
#pragma unroll 8
    for (int i = lo; i < hi; ++i, p += kHeadDim) {
      const u32x4 w = *(const u32x4*)p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = acc[2 * e] + bf16_lo(w[e]);
        acc[2 * e + 1] = acc[2 * e + 1] + bf16_hi(w[e]);
      }
    }
    const double n = (double)(hi - lo);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] / n;
  }
  if (!kTransposed) {
    if (t < T) {
      double* o = out + ((size_t)h * T + t) * kHeadDim + 8 * c;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = acc[e];
    }
    return;
  }
  // out[h][d][t]: stage through LDS so each row of the transposed result is
  // written as 16 consecutive doubles
#pragma unroll
  for (int e = 0; e < 8; ++e) stage[(8 * c + e) * kMeansTiles + tt] = acc[e];
  __syncthreads();
  const int d = tid >> 1, t0 = (tid & 1) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int t2 = blockIdx.x * kMeansTiles + t0 + e;
    if (t2 < T) out[((size_t)h * kHeadDim + d) * T + t2] = stage[d * kMeansTiles + t0 + e];
  }
}

// Order-preserving map of a double onto uint64 (larger double -> larger key).
__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// One wave: the `keep` largest of sc[0..T) (ties -> lower index), written
// ascending to out[0..keep).
__device__ void select_row(const double* sc, int T, int keep, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int M = (T + 63) >> 6;
  uint64_t u[kMaxM];
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) {
    const int j = 64 * m + lane;
    u[m] = (m < M && j < T) ? order_key(sc[j]) : 0ull;
  }
  // Radix select, most significant bit first.  Invariant: every valid key
  // whose bits above `b` exceed those of P is selected (keep - need of them),
  // `cand` keys share P's bits above `b`, and `need` of those are still wanted.
  uint64_t P = 0;
  int need = keep, cand = T, b = 64;
  while (need != cand && b > 0) {
    --b;
    const uint64_t hi_mask = (b == 63) ? 0ull : (~0ull << (b + 1));
    int c1 = 0;
#pragma unroll
    for (int m = 0; m < kMaxM; ++m) {
      if (m < M) {
        const bool valid = 64 * m + lane < T;
        const bool hit = valid && ((u[m] ^ P) & hi_mask) == 0 && ((u[m] >> b) & 1ull);
        c1 += popc(__ballot(hit));
      }
    }
    if (c1 >= need) {
      P |= (1ull << b);
      cand = c1;
    } else {
      need -= c1;
      cand -= c1;
    }
  }
  const bool all_tied = (need == cand);
  int base = 0, eqbase = 0;
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) {
    if (m < M) {
      const int j = 64 * m + lane;
      const bool valid = j < T;
      bool sel;
      if (all_tied) {
        sel = valid && (b == 64 || (u[m] >> b) >= (P >> b));
      } else {  // b == 0: keys equal to P compete, lowest index first
        const bool eq = valid && u[m] == P;
        const uint64_t eqb = __ballot(eq);
        const int rank = eqbase + popc(eqb & lt);
        eqbase += popc(eqb);
        sel = valid && (u[m] > P || (eq && rank < need));
      }
      const uint64_t sb = __ballot(sel);
      const int pos = base + popc(sb & lt);
      if (sel && pos < keep) out[pos] = j;
      base += popc(sb);
    }
  }
}

template <bool kWriteScores>
__global__ __launch_bounds__(256) void score_select_kernel(const double* __restrict__ qm,
                                                           const double* __restrict__ kmT, int T,
                                                           int keep, int32_t* __restrict__ idx,
                                                           double* __restrict__ scores) {
  extern __shared__ double sh[];
  double* qs = sh;                        // [128][kRows]
  double* sc = sh + kHeadDim * kRows;     // [kRows][T]
  const int h = blockIdx.y, i0 = blockIdx.x * kRows;
  const int nrows = (T - i0 < kRows) ? T - i0 : kRows;
  const int tid = threadIdx.x;
  for (int x = tid; x < kHeadDim * kRows; x += 256) {
    const int d = x / kRows, r = x - d * kRows;
    qs[x] = (r < nrows) ? qm[((size_t)h * T + i0 + r) * kHeadDim + d] : 0.0;
  }
  __syncthreads();
  const double* kh = kmT + (size_t)h * kHeadDim * T;
  for (int j = tid; j < T; j += 256) {
    double acc[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = 0.0;
#pragma unroll 8
    for (int d = 0; d < kHeadDim; ++d) {
      const double kv = kh[(size_t)d * T + j];
#pragma unroll
      for (int r = 0; r < kRows; ++r) acc[r] = acc[r] + qs[d * kRows + r] * kv;
    }
    if (kWriteScores) {
      for (int r = 0; r < nrows; ++r) scores[((size_t)h * T + i0 + r) * T + j] = acc[r];
    } else {
#pragma unroll
      for (int r = 0; r < kRows; ++r) sc[r * T + j] = acc[r];
    }
  }
  if (kWriteScores) return;
  __syncthreads();
  const int wave = tid >> 6;
  for (int r = wave; r < nrows; r += 4)
    select_row(sc + r * T, T, keep, idx + ((size_t)h * T + i0 + r) * keep);
}

__global__ void transpose_means_kernel(const double* __restrict__ in, double* __restrict__ out,
                                       int T) {
  const int h = blockIdx.y;
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= T * kHeadDim) return;
  const int t = x / kHeadDim, d = x - t * kHeadDim;
  out[((size_t)h * kHeadDim + d) * T + t] = in[((size_t)h * T + t) * kHeadDim + d];
}

}  // namespace

hipError_t launch_tile_means(const uint16_t* x, double* out, int heads, int tokens,
                             bool transposed, hipStream_t stream) {
  const int T = (tokens + kTile - 1) / kTile;
  if (heads <= 0 || T <= 0) return hipSuccess;
  const dim3 grid((T + kMeansTiles - 1) / kMeansTiles, heads);
  if (transposed)
    hipLaunchKernelGGL(tile_means_kernel<true>, grid, dim3(256), 0, stream, x, out, tokens, T);
  else
    hipLaunchKernelGGL(tile_means_kernel<false>, grid, dim3(256), 0, stream, x, out, tokens, T);
  return hipGetLastError();
}

hipError_t launch_score_select(const double* qm, const double* kmT, int heads, int tiles,
                               int keep, int32_t* idx_out, double* scores_out,
                               hipStream_t stream) {
  if (heads <= 0 || tiles <= 0) return hipSuccess;
  const dim3 grid((tiles + kRows - 1) / kRows, heads);
  if (scores_out) {
    const size_t lds = sizeof(double) * kHeadDim * kRows;
    hipLaunchKernelGGL(score_select_kernel<true>, grid, dim3(256), lds, stream, qm, kmT, tiles,
                       keep, idx_out, scores_out);
  } else {
    const size_t lds = sizeof(double) * ((size_t)kHeadDim * kRows + (size_t)kRows * tiles);
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute((const void*)score_select_kernel<false>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(score_select_kernel<false>, grid, dim3(256), lds, stream, qm, kmT, tiles,
                       keep, idx_out, scores_out);
  }
  return hipGetLastError();
}

hipError_t launch_transpose_means(const double* in, double* out, int heads, int tiles,
                                  hipStream_t stream) {
  if (heads <= 0 || tiles <= 0) return hipSuccess;
  const dim3 grid((tiles * kHeadDim + 255) / 256, heads);
  hipLaunchKernelGGL(transpose_means_kernel, grid, dim3(256), 0, stream, in, out, tiles);
  return hipGetLastError();
}

}  // namespace fvattn
