// VSA-H3 packed-sequence support on gfx950 (FastH3 page, "FastH3 Preview v1:
// four calls, one-tenth the attention...", section "Lever two: VSA-H3 makes
// each of the four calls cheaper"): only the generated-video part of the
// packed sequence [text | condition keyframes | audio | video] is cut into 3D
// tiles over its (t, h, w) latent grid; non-video keys are exempt (seen by
// every video query) and non-video queries are dense.
//
// The attention kernel works on a padded tile layout (see VsaGeom): every 3D
// tile becomes a run of S slots, its valid tokens first.  Here:
// * vsa_pack_kernel: K and V into that layout (HBM copy, 16 B per lane,
//   coalesced 256-byte rows; padding slots written as zeros).
// * vsa_means_kernel: fp64 mean of every video tile of Q and of K (one launch,
//   blockIdx.z picks the tensor), read from the caller's layout and written
//   transposed [heads][128][tiles] for the score kernel; the sum walks the
//   tile's tokens in (t, h, w) raster order from +0.0, then one correctly
//   rounded division by the tile's token count.
//   Scores and top-k then run in select.hip over the video tiles only.
// * vsa_lists_kernel: per head and kVsaRows-row query block, the ascending list of
//   64-key sub-tiles that some query of the block attends to: every non-empty
//   sub-tile for a block of non-video queries; the non-video sub-tiles plus
//   the sub-tiles of the kept video tiles for a block of video queries.  Each
//   entry records which 64-row query groups of the block attend to it and how
//   many of its 64 slots hold tokens.

#include "fvattn_internal.h"

#pragma clang fp contract(off)

namespace fvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMeansTiles = 16;   // tiles per workgroup (16 threads per tile)
constexpr int kMaxSub = 8192;     // sub-tiles per list row held in LDS

__device__ __forceinline__ double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ __forceinline__ double bf16_hi(uint32_t w) {
  return (double)__uint_as_float(w & 0xffff0000u);
}

__global__ __launch_bounds__(256) void vsa_pack_kernel(const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V,
                                                       uint16_t* __restrict__ Kp,
                                                       uint16_t* __restrict__ Vp, VsaGeom g,
                                                       long long chunks) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= chunks) return;
  const int c = (int)(i & 15);
  const long long row = i >> 4;                 // h * npad + slot
  const int h = (int)(row / g.npad), slot = (int)(row - (long long)h * g.npad);
  const int tok = vsa_slot_token(g, slot);
  u32x4 kw = {0u, 0u, 0u, 0u}, vw = {0u, 0u, 0u, 0u};
  if (tok >= 0) {
    const size_t src = ((size_t)h * g.tokens + tok) * kHeadDim + 8 * c;
    kw = *(const u32x4*)(K + src);
    vw = *(const u32x4*)(V + src);
  }
  const size_t dst = (size_t)row * kHeadDim + 8 * c;
  *(u32x4*)(Kp + dst) = kw;
  *(u32x4*)(Vp + dst) = vw;
}

__global__ __launch_bounds__(256) void vsa_means_kernel(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ K,
                                                        double* __restrict__ qmT,
                                                        double* __restrict__ kmT, VsaGeom g) {
  __shared__ double stage[kHeadDim * kMeansTiles];
  const uint16_t* const X = blockIdx.z == 0 ? Q : K;
  double* const out = blockIdx.z == 0 ? qmT : kmT;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, tl = tid >> 4, c = tid & 15;
  const int j = blockIdx.x * kMeansTiles + tl;
  const int T = g.tiles;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  if (j < T) {
    const VsaTile t = vsa_tile(g, j);
    const uint16_t* base = X + ((size_t)h * g.tokens + g.prefix) * kHeadDim + 8 * c;
    for (int dt = 0; dt < t.et; ++dt)
      for (int dh = 0; dh < t.eh; ++dh) {
        const uint16_t* p =
            base + ((size_t)((t.t0 + dt) * g.height + t.h0 + dh) * g.width + t.w0) * kHeadDim;
        for (int dw = 0; dw < t.ew; ++dw, p += kHeadDim) {
          const u32x4 w = *(const u32x4*)p;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] = acc[2 * e] + bf16_lo(w[e]);
            acc[2 * e + 1] = acc[2 * e + 1] + bf16_hi(w[e]);
          }
        }
      }
    const double n = (double)(t.et * t.eh * t.ew);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = acc[e] / n;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) stage[(8 * c + e) * kMeansTiles + tl] = acc[e];
  __syncthreads();
  const int d = tid >> 1, j0 = (tid & 1) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j2 = blockIdx.x * kMeansTiles + j0 + e;
    if (j2 < T) out[((size_t)h * kHeadDim + d) * T + j2] = stage[d * kMeansTiles + j0 + e];
  }
}

__global__ __launch_bounds__(256) void vsa_lists_kernel(const int32_t* __restrict__ idx, int keep,
                                                        VsaGeom g, int blocks,
                                                        int32_t* __restrict__ lists,
                                                        int32_t* __restrict__ counts) {
  __shared__ uint8_t member[kMaxSub];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int nsub = g.npad / 64, psub = g.ppad / 64, per_tile = g.size / 64;
  for (int s = tid; s < nsub; s += 256) member[s] = 0;
  __syncthreads();
  int groups = 0;   // query groups of this block that hold slots (uniform)
  for (int grp = 0; grp < kVsaRows / 64; ++grp) {
    const int row0 = kVsaRows * b + 64 * grp;
    if (row0 >= g.npad) break;
    groups |= 1 << grp;
    const uint8_t bit = (uint8_t)(1 << grp);
    if (row0 < g.ppad) {
      // non-video queries: dense
      for (int s = tid; s < nsub; s += 256)
        if (vsa_sub_count(g, s) > 0) member[s] |= bit;
    } else {
      // video queries: every non-video key, plus the kept video tiles
      const int a = (row0 - g.ppad) / g.size;
      for (int s = tid; s < psub; s += 256)
        if (vsa_sub_count(g, s) > 0) member[s] |= bit;
      const int32_t* row = idx + ((size_t)h * g.tiles + a) * keep;
      for (int e = tid; e < keep * per_tile; e += 256) {
        const int jt = row[e / per_tile], m = e - (e / per_tile) * per_tile;
        const int s = psub + jt * per_tile + m;
        if (vsa_sub_count(g, s) > 0) member[s] |= bit;
      }
    }
    __syncthreads();
  }
  if (tid >= 64) return;
  // ascending compaction by one wave
  const int lane = tid;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int32_t* out = lists + ((size_t)h * blocks + b) * nsub;
  int base = 0;
  for (int s0 = 0; s0 < nsub; s0 += 64) {
    const int s = s0 + lane;
    const int mem = s < nsub ? member[s] : 0;
    const uint64_t m = __ballot(mem != 0);
    if (mem) {
      const int n = vsa_sub_count(g, s);
      int e = s | ((n - 1) << kVsaCountShift) | (mem << kVsaGroupShift);
      if (n < 64 || mem != groups) e |= kMaskFlag;
      out[base + __popcll(m & lt)] = e;
    }
    base += __popcll(m);
  }
  if (lane == 0) counts[(size_t)h * blocks + b] = base;
}

}  // namespace

hipError_t launch_vsa_pack(const uint16_t* k, const uint16_t* v, uint16_t* kp, uint16_t* vp,
                           const VsaGeom& g, int heads, hipStream_t stream) {
  const long long chunks = (long long)heads * g.npad * 16;
  if (chunks <= 0) return hipSuccess;
  const long long blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(vsa_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, k, v, kp, vp, g,
                     chunks);
  return hipGetLastError();
}

hipError_t launch_vsa_means(const uint16_t* q, const uint16_t* k, double* qmT, double* kmT,
                            const VsaGeom& g, int heads, hipStream_t stream) {
  if (heads <= 0 || g.tiles <= 0) return hipSuccess;
  const dim3 grid((g.tiles + kMeansTiles - 1) / kMeansTiles, heads, 2);
  hipLaunchKernelGGL(vsa_means_kernel, grid, dim3(256), 0, stream, q, k, qmT, kmT, g);
  return hipGetLastError();
}

hipError_t launch_vsa_lists(const int32_t* idx, int keep, const VsaGeom& g, int heads,
                            int32_t* lists, int32_t* counts, hipStream_t stream) {
  const int blocks = (g.npad + kVsaRows - 1) / kVsaRows;
  if (heads <= 0 || blocks <= 0) return hipSuccess;
  if (g.npad / 64 > kMaxSub) return hipErrorInvalidValue;
  hipLaunchKernelGGL(vsa_lists_kernel, dim3(blocks, heads), dim3(256), 0, stream, idx, keep, g,
                     blocks, lists, counts);
  return hipGetLastError();
}

}  // namespace fvattn
