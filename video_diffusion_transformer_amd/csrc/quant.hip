// INT8 keys for attention with INT8 query-key scores (FastH3 page, "FastH3
// Preview v1: four calls, one-tenth the attention...", section "Update:
// consumer GPUs and Trim", subsection "Per device": queries and keys quantized
// to INT8 for the scores).
//
// quantize_k_kernel: one workgroup per block of 64 consecutive keys of one
// head.  scale = max |k| / 127 over the block (1 for a block of zeros), code =
// round-half-to-even(k / scale) in [-127, 127]; the scale and the division are
// correctly rounded float32 operations.  Codes are written row-major, 128 bytes
// per key ([heads][tokens][128] int8), scales as float [heads][ceil(tokens/64)].
// Queries are quantized per row inside the attention kernel.
//
// The FP8 variant (quantize_k_kernel<true>) writes OCP E4M3 codes instead:
// scale = max |k| / 448, code = the E4M3 value nearest to k / scale (ties to
// the even mantissa) by the hardware conversion v_cvt_pk_fp8_f32, again with a
// correctly rounded float32 scale and division.

#include "fvattn_internal.h"

namespace fvattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQuantBlock = 64;

__device__ __forceinline__ float bf16_at(const u32x4& w, int e) {
  const uint32_t x = w[e >> 1];
  return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
}

__device__ __forceinline__ uint32_t code_byte(float x, float s) {
  float q = __builtin_rintf(__fdiv_rn(x, s));
  q = q > 127.f ? 127.f : (q < -127.f ? -127.f : q);
  return (uint32_t)((int)q & 0xff);
}

// Four FP8 E4M3 codes of x[0..3] / s packed little-endian into one word.
__device__ __forceinline__ uint32_t fp8_word(float x0, float x1, float x2, float x3, float s) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(x0, s), __fdiv_rn(x1, s), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__fdiv_rn(x2, s), __fdiv_rn(x3, s), w, true);
  return (uint32_t)w;
}

template <bool kFp8>
__global__ __launch_bounds__(256) void quantize_k_kernel(const uint16_t* __restrict__ K,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales, int N,
                                                         int nblk) {
  __shared__ float wmax[4];
  const int b = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int row = b * kQuantBlock + (tid >> 2), part = tid & 3;   // 4 threads per key, 32 dims each
  const bool live = row < N;
  u32x4 w[4];
  float m = 0.f;
  if (live) {
    const uint16_t* p = K + ((size_t)h * N + row) * kHeadDim + 32 * part;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[c] = *(const u32x4*)(p + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(bf16_at(w[c], e)));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = m == 0.f ? 1.f : __fdiv_rn(m, kFp8 ? 448.f : 127.f);
  if (tid == 0) scales[(size_t)h * nblk + b] = s;
  if (!live) return;
  u32x4 out[2];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t word = 0;
      if constexpr (kFp8) {
        word = fp8_word(bf16_at(w[c], 4 * j), bf16_at(w[c], 4 * j + 1), bf16_at(w[c], 4 * j + 2),
                        bf16_at(w[c], 4 * j + 3), s);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) word |= code_byte(bf16_at(w[c], 4 * j + e), s) << (8 * e);
      }
      out[c >> 1][2 * (c & 1) + j] = word;
    }
  uint8_t* o = codes + ((size_t)h * N + row) * kHeadDim + 32 * part;
  *(u32x4*)o = out[0];
  *(u32x4*)(o + 16) = out[1];
}

}  // namespace

hipError_t launch_quantize_k(const uint16_t* k, uint8_t* codes, float* scales, int heads,
                             int tokens, bool fp8, hipStream_t stream) {
  const int nblk = (tokens + kQuantBlock - 1) / kQuantBlock;
  if (heads <= 0 || nblk <= 0) return hipSuccess;
  if (fp8)
    hipLaunchKernelGGL(quantize_k_kernel<true>, dim3(nblk, heads), dim3(256), 0, stream, k, codes,
                       scales, tokens, nblk);
  else
    hipLaunchKernelGGL(quantize_k_kernel<false>, dim3(nblk, heads), dim3(256), 0, stream, k, codes,
                       scales, tokens, nblk);
  return hipGetLastError();
}

}  // namespace fvattn
