// Matrix-core rate probe for gfx950: how fast this GPU, at its present clock
// and power state, retires bf16 MFMAs with nothing else in the way.  The
// attention figures are reported against the 2.5 PFLOP/s dense bf16 peak of
// the MI355X data sheet, which assumes the 2.4 GHz peak clock; under a
// sustained matrix load the clock settles lower, and this probe measures the
// rate that is actually available, so a kernel's fraction of it can be
// compared across boxes.
//
// Each wave runs `iters` iterations of four independent accumulator chains of
// v_mfma_f32_32x32x16_bf16 (32,768 FLOP each); no memory traffic inside the
// loop.  Four waves per SIMD (1,024 workgroups of 4 waves on 256 CUs) keep the
// matrix pipe of every SIMD busy.  The accumulators are summed into one float
// per thread of `sink` so the loop cannot be removed.

#include "fvattn_internal.h"

namespace fvattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* __restrict__ sink, int iters) {
  const int tid = threadIdx.x, lane = tid & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((float)((lane + i) % 7 - 3) * 0.015625f);
    b[i] = (__bf16)((float)((lane * 3 + i) % 5 - 2) * 0.015625f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(size_t)blockIdx.x * 256 + tid] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* sink, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(kProbeBlocks), dim3(256), 0, stream, sink, iters);
  return hipGetLastError();
}

}  // namespace fvattn
