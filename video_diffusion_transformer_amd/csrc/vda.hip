// Video Delta Attention, the linear branch of Video DeltaNet, on gfx950
// (FreeVideo page, "FreeVideo: a 66 GB video transformer on an 8 GB card...",
// section "Where Video DeltaNet comes in").
//
// Per head, with d = 128 and a latent frame t of frame_tokens tokens:
//   A_t = sum_u beta_u k_u k_u^T,  B_t = sum_u beta_u v_u k_u^T,
//   S_t = (S_prev Diag(alpha_t) + B_t)(I + A_t)^-1 = S_prev P_t + C_t
// with M_t = (I + A_t)^-1, P_t = Diag(alpha_t) M_t and C_t = B_t M_t.  Everything
// but the last line is independent per frame, so it runs for all frames at
// once; only S_t = S_prev P_t + C_t is sequential.  The forward scan writes
// frames 1..F-2 in order, the reverse scan F-2..1, both from S_text / 2 (the
// first and last frames are softmax anchors and are not written).  A query of
// frame f reads o = fwd[lo(f)] q + rev[hi(f)] q, lo / hi the frames just
// before and after its softmax window (both seeds for the anchor frames).
//
// Every product is fp32 on the matrix cores (v_mfma_f32_32x32x2_f32: lane l
// holds A[l % 32][l / 32] and B[l / 32][l % 32]); the inverse is an in-place
// Gauss-Jordan elimination in LDS, which needs no pivoting because I + A_t is
// symmetric with eigenvalues >= 1.
//
// Kernels: vda_stats_kernel (A_t, B_t per frame), vda_inverse_kernel (M_t and
// P_t), vda_matmul_kernel (C_t = B_t M_t), vda_scan_kernel (one workgroup per
// head and direction, the state in LDS), vda_readout_kernel.

#include "fvattn_internal.h"

namespace fvattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = kHeadDim;           // 128
constexpr int kMat = kD * kD;          // one state-sized matrix
constexpr int kPad = kD + 1;           // LDS row pitch: a column walk by 32 lanes hits 32 banks

__device__ __forceinline__ float bf16f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ f32x16 mfma(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Accumulator register r of lane l holds row acc_row(r, l) and column l % 32
// of its 32 x 32 tile.
__device__ __forceinline__ int acc_row(int r, int l) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }

// Store four 32 x 32 tiles (row tile rt, column tiles 0..3) of a 128 x 128
// row-major matrix.
__device__ __forceinline__ void store_row_tile(float* __restrict__ m, int rt, const f32x16 (&acc)[4],
                                               int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) m[(32 * rt + acc_row(r, lane)) * kD + 32 * j + (lane & 31)] = acc[j][r];
}

// A_t and B_t of frame t of head h.  Wave w owns row tile w of both.
__global__ __launch_bounds__(256) void vda_stats_kernel(const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V,
                                                        const float* __restrict__ beta, int ft,
                                                        int frames, float* __restrict__ A,
                                                        float* __restrict__ B) {
  const int t = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, half = lane >> 5;
  const size_t N = (size_t)frames * ft;
  const size_t tok0 = (size_t)h * N + (size_t)t * ft;
  f32x16 acc_a[4], acc_b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc_a[j][r] = 0.f; acc_b[j][r] = 0.f; }
  for (int u0 = 0; u0 < ft; u0 += 2) {
    const int u = u0 + half;
    float kv[4], vw = 0.f, b = 0.f;
    if (u < ft) {
      const uint16_t* kr = K + (tok0 + u) * kD;
#pragma unroll
      for (int j = 0; j < 4; ++j) kv[j] = bf16f(kr[32 * j + l32]);
      vw = bf16f(V[(tok0 + u) * kD + 32 * w + l32]);
      b = beta[tok0 + u];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) kv[j] = 0.f;
    }
    const float ka = b * kv[w], va = b * vw;    // beta_u k_u[32 w + i], beta_u v_u[32 w + i]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc_a[j] = mfma(ka, kv[j], acc_a[j]);
      acc_b[j] = mfma(va, kv[j], acc_b[j]);
    }
  }
  const size_t off = ((size_t)h * frames + t) * kMat;
  store_row_tile(A + off, w, acc_a, lane);
  store_row_tile(B + off, w, acc_b, lane);
}

// M_t = (I + A_t)^-1 by Gauss-Jordan in place, and P_t = Diag(alpha_t) M_t.
// Thread (column j, parity p) keeps rows p, p + 2, ... of column j in
// registers.  Step k needs column k (published by its two owners) and row k
// (published by the owners of row k in every column) through LDS, double
// buffered by step parity so that one barrier per step suffices: a buffer is
// rewritten two steps later, after every thread has passed another barrier.
__global__ __launch_bounds__(256) void vda_inverse_kernel(const float* __restrict__ A,
                                                          const float* __restrict__ alpha,
                                                          float* __restrict__ M,
                                                          float* __restrict__ P) {
  __shared__ float colk[2][2][kD / 2];   // [buffer][row parity][row / 2]: a[row][k] before step k
  __shared__ float rowk[2][kD];          // [buffer][column]: a[k][column] before step k
  const size_t m = (size_t)blockIdx.y * gridDim.x + blockIdx.x;   // h * frames + t
  const int tid = threadIdx.x, j = tid & (kD - 1), p = tid >> 7;
  const float* src = A + m * kMat;
  float r[kD / 2];
#pragma unroll
  for (int i = 0; i < kD / 2; ++i) r[i] = src[(2 * i + p) * kD + j] + (2 * i + p == j ? 1.f : 0.f);
  for (int k = 0; k < kD; ++k) {
    const int buf = k & 1;
    if (j == k) {
#pragma unroll
      for (int i = 0; i < kD / 2; ++i) colk[buf][p][i] = r[i];
    }
    if (p == (k & 1)) {
      // this thread holds a[k][j] in r[k / 2]; select it without dynamic indexing
      float x = 0.f;
#pragma unroll
      for (int i = 0; i < kD / 2; ++i) x = (i == (k >> 1)) ? r[i] : x;
      rowk[buf][j] = x;
    }
    __syncthreads();
    const float piv_inv = 1.f / colk[buf][k & 1][k >> 1];
    const float rk = (j == k ? 1.f : rowk[buf][j]) * piv_inv;     // scaled row k, a[k][k] = 1 / pivot
#pragma unroll
    for (int i = 0; i < kD / 2; ++i) {
      const int row = 2 * i + p;
      r[i] = row == k ? rk : (j == k ? 0.f : r[i]) - colk[buf][p][i] * rk;
    }
  }
  const float* al = alpha + m * kD;
  float* mo = M + m * kMat;
  float* po = P + m * kMat;
#pragma unroll
  for (int i = 0; i < kD / 2; ++i) {
    const int row = 2 * i + p;
    mo[row * kD + j] = r[i];
    po[row * kD + j] = al[row] * r[i];
  }
}

// out[b] = X[b] Y[b] for batches of 128 x 128 matrices.  Wave w owns row tile w.
__global__ __launch_bounds__(256) void vda_matmul_kernel(const float* __restrict__ X,
                                                         const float* __restrict__ Y,
                                                         float* __restrict__ out) {
  __shared__ float xs[kD][kPad];
  const size_t b = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const float* x = X + b * kMat;
  const float* y = Y + b * kMat;
  for (int i = tid >> 7; i < kD; i += 2) xs[i][tid & (kD - 1)] = x[i * kD + (tid & (kD - 1))];
  __syncthreads();
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
#pragma unroll 4
  for (int s = 0; s < kD; s += 2) {
    const float av = xs[32 * w + l32][s + half];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma(av, y[(s + half) * kD + 32 * j + l32], acc[j]);
  }
  store_row_tile(out + b * kMat, w, acc, lane);
}

// One workgroup per (head, direction): S = S_text / 2, then S = S P_t + C_t over
// the written frames; states [head][frames + 1] of each direction.  Sixteen
// waves, one 32 x 32 output tile each (row tile w % 4, column tile w / 4): the
// chains are sequential, so each step is spread as wide as it goes.
__global__ __launch_bounds__(1024) void vda_scan_kernel(const float* __restrict__ P,
                                                        const float* __restrict__ C,
                                                        const float* __restrict__ s_text,
                                                        int frames, float* __restrict__ fwd,
                                                        float* __restrict__ rev) {
  __shared__ float S[kD][kPad];
  const int h = blockIdx.x, dir = blockIdx.y;   // 0 forward, 1 reverse
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const int rt = w & 3, ct = w >> 2;
  const int j0 = tid & (kD - 1), i0 = tid >> 7;   // copy pattern: 8 rows per pass
  float* states = (dir == 0 ? fwd : rev) + (size_t)h * (frames + 1) * kMat;
  const float* st = s_text + (size_t)h * kMat;
  const int first = dir == 0 ? 0 : frames;      // index of the seed state
  for (int i = i0; i < kD; i += 8) {
    const float x = 0.5f * st[i * kD + j0];
    S[i][j0] = x;
    states[(size_t)first * kMat + i * kD + j0] = x;
  }
  __syncthreads();
  for (int step = 0; step < frames; ++step) {
    const int t = dir == 0 ? step : frames - 1 - step;      // frame absorbed now
    const int dst = dir == 0 ? t + 1 : t;                   // state index written
    float* so = states + (size_t)dst * kMat;
    if (t >= 1 && t <= frames - 2) {
      const float* pm = P + ((size_t)h * frames + t) * kMat;
      const float* cm = C + ((size_t)h * frames + t) * kMat;
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = cm[(32 * rt + acc_row(r, lane)) * kD + 32 * ct + l32];
#pragma unroll 8
      for (int s2 = 0; s2 < kD; s2 += 2)
        acc = mfma(S[32 * rt + l32][s2 + half], pm[(s2 + half) * kD + 32 * ct + l32], acc);
      __syncthreads();   // every wave has read the old state
#pragma unroll
      for (int r = 0; r < 16; ++r) S[32 * rt + acc_row(r, lane)][32 * ct + l32] = acc[r];
      __syncthreads();
    }
    for (int i = i0; i < kD; i += 8) so[i * kD + j0] = S[i][j0];
  }
}

// out rows of frame f: o = (fwd[lo] + rev[hi]) q.  One workgroup per (frame,
// head): W = fwd[lo] + rev[hi] is staged once in LDS, then 128 query rows at a
// time pass through LDS (wave w owns 32 of them).
constexpr int kQPitch = kD + 2;   // bf16 row pitch of staged queries: 65 words, 32 rows -> 32 banks

__global__ __launch_bounds__(256) void vda_readout_kernel(const uint16_t* __restrict__ Q,
                                                          const float* __restrict__ fwd,
                                                          const float* __restrict__ rev, int ft,
                                                          int frames, int chunk, int nb,
                                                          float* __restrict__ out) {
  __shared__ float W[kD][kPad];
  __shared__ __attribute__((aligned(16))) uint16_t qs[kD][kQPitch];
  const int f = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  int lo = 0, hi = frames;
  if (f != 0 && f != frames - 1) {
    const int c = f / chunk;
    lo = (c - nb) * chunk;
    hi = (c + nb + 1) * chunk;
    lo = lo < 0 ? 0 : (lo > frames ? frames : lo);
    hi = hi < 0 ? 0 : (hi > frames ? frames : hi);
  }
  const float* wf = fwd + ((size_t)h * (frames + 1) + lo) * kMat;
  const float* wr = rev + ((size_t)h * (frames + 1) + hi) * kMat;
  for (int i = tid >> 7; i < kD; i += 2) {
    const int j = tid & (kD - 1);
    W[i][j] = wf[i * kD + j] + wr[i * kD + j];
  }
  const size_t N = (size_t)frames * ft;
  const uint16_t* qf = Q + ((size_t)h * N + (size_t)f * ft) * kD;
  float* of = out + ((size_t)h * N + (size_t)f * ft) * kD;
  for (int r0 = 0; r0 < ft; r0 += kD) {
    __syncthreads();   // W staged / previous rows consumed
    // 128 rows x 128 bf16: thread tid copies 4 B at (row, pair) for 16 passes
    for (int x = tid; x < kD * kD / 2; x += 256) {
      const int row = x >> 6, pr = x & 63;
      const uint32_t v =
          r0 + row < ft ? *(const uint32_t*)(qf + (size_t)(r0 + row) * kD + 2 * pr) : 0u;
      *(uint32_t*)&qs[row][2 * pr] = v;
    }
    __syncthreads();
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
#pragma unroll 4
    for (int s2 = 0; s2 < kD; s2 += 2) {
      const int d = s2 + half;
      const float av = bf16f(qs[32 * w + l32][d]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma(av, W[32 * j + l32][d], acc[j]);   // W^T[d][dv] = W[dv][d]
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = r0 + 32 * w + acc_row(r, lane);
        if (rr < ft) of[(size_t)rr * kD + 32 * j + l32] = acc[j][r];
      }
  }
}

}  // namespace

hipError_t launch_vda_states(const uint16_t* k, const uint16_t* v, const float* beta,
                             const float* alpha, const float* s_text, int heads, int frames,
                             int ft, float* scratch, float* fwd, float* rev, hipStream_t stream) {
  if (heads <= 0 || frames <= 0) return hipSuccess;
  const size_t per = (size_t)heads * frames * kMat;
  float* A = scratch;
  float* B = A + per;
  float* M = B + per;
  float* P = M + per;
  float* C = P + per;
  const dim3 grid(frames, heads);
  hipLaunchKernelGGL(vda_stats_kernel, grid, dim3(256), 0, stream, k, v, beta, ft, frames, A, B);
  hipLaunchKernelGGL(vda_inverse_kernel, grid, dim3(256), 0, stream, A, alpha, M, P);
  hipLaunchKernelGGL(vda_matmul_kernel, grid, dim3(256), 0, stream, B, M, C);
  hipLaunchKernelGGL(vda_scan_kernel, dim3(heads, 2), dim3(1024), 0, stream, P, C, s_text, frames, fwd,
                     rev);
  return hipGetLastError();
}

hipError_t launch_vda_readout(const uint16_t* q, const float* fwd, const float* rev, int heads,
                              int frames, int ft, int chunk, int nb, float* out, hipStream_t stream) {
  if (heads <= 0 || frames <= 0) return hipSuccess;
  hipLaunchKernelGGL(vda_readout_kernel, dim3(frames, heads), dim3(256), 0, stream, q, fwd, rev, ft,
                     frames, chunk, nb, out);
  return hipGetLastError();
}

}  // namespace fvattn
