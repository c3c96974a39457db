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
//     reads Q and K once with 128-bit loads, 16 lanes per 256-byte token row,
//     Q and K in one launch, both written transposed for S2.
// S2  scores_kernel: sigma_ij = sum_d qm_i[d] * km_j[d] in fp64 from +0.0 in
//     order d = 0..127, every product and every sum rounded on its own (fp
//     contraction is off in this file).  A workgroup owns a 64 x 64 block of
//     (query tile, key tile) pairs; both mean sets arrive transposed
//     ([heads][128][T]), so a chunk of 32 dimensions is 32 runs of 64
//     consecutive doubles per side: coalesced loads, bank-conflict-free LDS
//     writes, and the next chunk's loads in flight while this one is summed.
//     Every thread keeps a 4 x 4 block of running sums in registers, each
//     summed in the canonical order.  The scores go to a stream-ordered
//     scratch matrix [heads][T][T].
// S3  select_kernel: per query tile, the `keep` largest scores, ties to the
//     lower key tile, found by one wave with a most-significant-bit-first radix
//     select on the order-preserving 64-bit image of the doubles, then emitted
//     in ascending tile order with ballots.

#include "fvattn_internal.h"

#pragma clang fp contract(off)

namespace fvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMeansTiles = 16;   // tiles per workgroup in S1 (16 threads per tile)
constexpr int kBlk = 64;          // S2: query and key tiles per workgroup
constexpr int kChunk = 32;        // S2: dimensions staged per pass

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) {
  return (double)__uint_as_float(w & 0xffff0000u);
}

template <bool kTransposed>
__device__ __forceinline__ void tile_means_body(const uint16_t* __restrict__ X,
                                                double* __restrict__ out, int N, int T, int h) {
  __shared__ double stage[kHeadDim * kMeansTiles];
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

// Means of one tensor, [heads][T][128] (the step-alone entry point).
__global__ __launch_bounds__(256) void tile_means_kernel(const uint16_t* __restrict__ X,
                                                         double* __restrict__ out, int N, int T) {
  tile_means_body<false>(X, out, N, T, blockIdx.y);
}

// Query and key means of one selection in one launch (blockIdx.z: 0 = Q,
// 1 = K), both transposed [heads][128][T] for the score kernel.
__global__ __launch_bounds__(256) void tile_means_qk_kernel(const uint16_t* __restrict__ Q,
                                                            const uint16_t* __restrict__ K,
                                                            double* __restrict__ qmT,
                                                            double* __restrict__ kmT, int N, int T) {
  if (blockIdx.z == 0)
    tile_means_body<true>(Q, qmT, N, T, blockIdx.y);
  else
    tile_means_body<true>(K, kmT, N, T, blockIdx.y);
}

// Order-preserving map of a double onto uint64 (larger double -> larger key).
__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// One wave: the `keep` largest of sc[0..T) (ties -> lower index), written
// ascending to out[0..keep).  T <= 64 kMaxM.
template <int kMaxM>
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

__global__ __launch_bounds__(256) void scores_kernel(const double* __restrict__ qmT,
                                                     const double* __restrict__ kmT, int T,
                                                     double* __restrict__ scores) {
  constexpr int kPer = kChunk * kBlk / 256;   // doubles per thread and side per chunk
  static_assert(kBlk == 64 && kPer * 256 == kChunk * kBlk && kHeadDim % kChunk == 0,
                "one 64-tile run per wave row, 4 rows per pass");
  __shared__ double qs[kChunk][kBlk];   // qs[d][i]: query means of the block, this chunk
  __shared__ double ks[kChunk][kBlk];   // ks[d][j]: key means of the block, this chunk
  const int h = blockIdx.z, i0 = blockIdx.y * kBlk, j0 = blockIdx.x * kBlk;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const double* qh = qmT + (size_t)h * kHeadDim * T;
  const double* kh = kmT + (size_t)h * kHeadDim * T;
  // element e of this thread: dimension d0 + (tid >> 6) + 4 e, tile (tid & 63)
  const int c = tid & 63, dr = tid >> 6;
  const bool qok = i0 + c < T, kok = j0 + c < T;
  double qreg[kPer], kreg[kPer];
  auto fetch = [&](int d0) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const size_t row = (size_t)(d0 + dr + 4 * e) * T;
      qreg[e] = qok ? qh[row + i0 + c] : 0.0;
      kreg[e] = kok ? kh[row + j0 + c] : 0.0;
    }
  };
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  fetch(0);
  for (int d0 = 0; d0 < kHeadDim; d0 += kChunk) {
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      qs[dr + 4 * e][c] = qreg[e];
      ks[dr + 4 * e][c] = kreg[e];
    }
    __syncthreads();
    if (d0 + kChunk < kHeadDim) fetch(d0 + kChunk);
#pragma unroll 4
    for (int d = 0; d < kChunk; ++d) {
      double qv[4], kv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qv[a] = qs[d][4 * ty + a];
#pragma unroll
      for (int b = 0; b < 4; ++b) kv[b] = ks[d][4 * tx + b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = acc[a][b] + qv[a] * kv[b];
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + 4 * ty + a;
    if (i >= T) continue;
    double* row = scores + ((size_t)h * T + i) * T;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (j0 + 4 * tx + b < T) row[j0 + 4 * tx + b] = acc[a][b];
  }
}

// One wave per (head, query tile) row of the score matrix; 4 rows per workgroup.
template <int kMaxM>
__global__ __launch_bounds__(256) void select_kernel(const double* __restrict__ scores, int T,
                                                     int rows, int keep, int32_t* __restrict__ idx) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  select_row<kMaxM>(scores + (size_t)row * T, T, keep, idx + (size_t)row * keep);
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
                             hipStream_t stream) {
  const int T = (tokens + kTile - 1) / kTile;
  if (heads <= 0 || T <= 0) return hipSuccess;
  const dim3 grid((T + kMeansTiles - 1) / kMeansTiles, heads);
  hipLaunchKernelGGL(tile_means_kernel, grid, dim3(256), 0, stream, x, out, tokens, T);
  return hipGetLastError();
}

hipError_t launch_tile_means_qk(const uint16_t* q, const uint16_t* k, double* qmT, double* kmT,
                                int heads, int tokens, hipStream_t stream) {
  const int T = (tokens + kTile - 1) / kTile;
  if (heads <= 0 || T <= 0) return hipSuccess;
  const dim3 grid((T + kMeansTiles - 1) / kMeansTiles, heads, 2);
  hipLaunchKernelGGL(tile_means_qk_kernel, grid, dim3(256), 0, stream, q, k, qmT, kmT, tokens, T);
  return hipGetLastError();
}

hipError_t launch_scores(const double* qmT, const double* kmT, int heads, int tiles,
                         double* scores_out, hipStream_t stream) {
  if (heads <= 0 || tiles <= 0) return hipSuccess;
  const int nb = (tiles + kBlk - 1) / kBlk;
  hipLaunchKernelGGL(scores_kernel, dim3(nb, nb, heads), dim3(256), 0, stream, qmT, kmT, tiles,
                     scores_out);
  return hipGetLastError();
}

hipError_t launch_select(const double* scores, int heads, int tiles, int keep, int32_t* idx_out,
                         hipStream_t stream) {
  if (heads <= 0 || tiles <= 0) return hipSuccess;
  const int rows = heads * tiles;
  const dim3 grid((rows + 3) / 4), block(256);
  // the smallest slot count that holds a row (register use grows with it)
  if (tiles <= 8 * 64)
    hipLaunchKernelGGL(select_kernel<8>, grid, block, 0, stream, scores, tiles, rows, keep, idx_out);
  else if (tiles <= 16 * 64)
    hipLaunchKernelGGL(select_kernel<16>, grid, block, 0, stream, scores, tiles, rows, keep, idx_out);
  else if (tiles <= 20 * 64)
    hipLaunchKernelGGL(select_kernel<20>, grid, block, 0, stream, scores, tiles, rows, keep, idx_out);
  else if (tiles <= 24 * 64)
    hipLaunchKernelGGL(select_kernel<24>, grid, block, 0, stream, scores, tiles, rows, keep, idx_out);
  else if (tiles <= 28 * 64)
    hipLaunchKernelGGL(select_kernel<28>, grid, block, 0, stream, scores, tiles, rows, keep, idx_out);
  else if (tiles <= 32 * 64)
    hipLaunchKernelGGL(select_kernel<32>, grid, block, 0, stream, scores, tiles, rows, keep, idx_out);
  else
    return hipErrorInvalidValue;
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
