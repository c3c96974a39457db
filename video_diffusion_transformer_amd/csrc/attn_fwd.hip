// Fused attention forward for gfx950 (MI355X): dense, or restricted to a list
// of 128-token key tiles per 128-token query tile (block-sparse).
//
// What it computes: out = softmax(scale * Q K^T) V per head, non-causal, the
// softmax taken over every key (dense) or over the keys of the listed tiles
// only (sparse); the scores are streamed tile by tile with an online softmax
// and never stored (FreeVideo page, section "Why it does not fit: the
// arithmetic"; FastH3 page, section "Lever two: VSA-H3 makes each of the four
// calls cheaper", fine stage: exact attention over the surviving tiles).
//
// Design (one workgroup = one head x one 128-row query tile, 4 waves of 32 rows):
// * Both products run on the bf16 matrix cores, v_mfma_f32_32x32x16_bf16, in
//   transposed form: S^T = K Q^T (A = K from LDS, B = Q^T held in registers for
//   the whole kernel) and O^T = V^T P^T (A = V^T from LDS, B = P^T taken
//   straight from the S^T accumulators).  With this orientation every lane owns
//   one query column of S^T and of O^T, so the softmax max/sum and the O
//   rescale are per-lane scalars plus one exchange between the two half-waves.
// * The key rows fed to the S^T product are permuted inside each 32-key block
//   so that half-wave g ends up holding keys 16g..16g+15 contiguously; P^T can
//   then be passed to the PV product without any data movement.
// * K and V stream through LDS in 64-key stages, double buffered: the next
//   stage's 128-bit global loads are in flight while the current stage is
//   multiplied.  K is stored row-major with an XOR swizzle on 16-byte chunks;
//   V is transposed on the way in (key-contiguous rows per head dimension),
//   also swizzled, so that every MFMA operand is one 128-bit LDS read.
// * fp32 online softmax in the exp2 domain (scale * log2 e folded into one
//   FMA per score), P rounded to bf16 for the PV product, out rounded to bf16.
// * Workgroups are remapped so each of the 8 XCDs walks a contiguous range of
//   (head, query tile) pairs, keeping one head's K/V hot in that XCD's L2.

#include <math.h>

#include "fvattn_internal.h"

namespace fvattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;                    // query rows per workgroup
constexpr int kBN = 64;                     // keys per LDS stage
constexpr int kThreads = 256;               // 4 waves x 32 query rows
constexpr int kRowBytes = kHeadDim * 2;     // 256 B per token row
constexpr int kKStage = kBN * kRowBytes;    // 16 KiB
constexpr int kVStage = kBN * kRowBytes;    // 16 KiB
constexpr int kStage = kKStage + kVStage;
constexpr int kLds = 2 * kStage;            // 64 KiB, two workgroups per CU
constexpr int kXcds = 8;

// K rows: chunk (16 B) swizzle; rows read together by one MFMA phase map to
// distinct chunk positions.
__device__ __forceinline__ int k_swz(int row) {
  return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
}
// V^T rows (one per head dimension, 64 keys = 8 chunks).
__device__ __forceinline__ int v_swz(int d) { return (d ^ (d >> 3)) & 7; }

// Key (within a 32-key block) fed as A-row m of the S^T product: output row m
// lands in half-wave (m>>2)&1 at accumulator 4*(m>>3) + (m&3), so this puts
// keys 16g..16g+15 in half-wave g, in accumulator order.
__device__ __forceinline__ int key_of_row(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// Hardware hands workgroup b to XCD b % 8; give every XCD a contiguous range.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = n / kXcds, rem = n % kXcds;
  const int x = b % kXcds, i = b / kXcds;
  return x * per + (x < rem ? x : rem) + i;
}

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <bool kSparse>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, const int32_t* __restrict__ idx,
    int keep, int N, int qtiles, float c) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int h = L / qtiles, qt = L - h * qtiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const size_t hoff = (size_t)h * (size_t)N * kHeadDim;
  const uint16_t* Qh = Q + hoff;
  const uint16_t* Kh = K + hoff;
  const uint16_t* Vh = V + hoff;

  // Q^T fragment of this lane's query row (B operand of S^T = K Q^T):
  // qf[dk][i] = Q[qrow][16 dk + 8 g + i].
  const int qrow = qt * kBM + wave * 32 + l32;
  bf16x8 qf[8];
#pragma unroll
  for (int dk = 0; dk < 8; ++dk) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (qrow < N) w = *(const u32x4*)(Qh + (size_t)qrow * kHeadDim + 16 * dk + 8 * g);
    qf[dk] = __builtin_bit_cast(bf16x8, w);
  }

  const int32_t* irow = kSparse ? idx + ((size_t)h * qtiles + qt) * keep : nullptr;
  const int nsub = kSparse ? 2 * keep : (N + kBN - 1) / kBN;
  auto kv_start = [&](int it) -> int {
    if (!kSparse) return it * kBN;
    int t = irow[it >> 1];
    t = t < 0 ? 0 : (t >= qtiles ? qtiles - 1 : t);
    return t * kTile + (it & 1) * kBN;
  };

  // Global -> register staging: K rows (tid>>4) + 16 rr, V rows 4 (tid>>4) + rr,
  // 16-byte chunk tid & 15 of each row; rows past N read as zero.
  const int ch = tid & 15, rg = tid >> 4;
  u32x4 kr[4], vr[4];
  auto load_kv = [&](int kv0) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int kk = kv0 + rg + 16 * rr;
      const int vk = kv0 + 4 * rg + rr;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (kk < N) a = *(const u32x4*)(Kh + (size_t)kk * kHeadDim + 8 * ch);
      if (vk < N) b = *(const u32x4*)(Vh + (size_t)vk * kHeadDim + 8 * ch);
      kr[rr] = a;
      vr[rr] = b;
    }
  };
  auto store_kv = [&](int buf) {
    unsigned char* Ks = smem + buf * kStage;
    unsigned char* Vt = Ks + kKStage;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = rg + 16 * rr;
      *(u32x4*)(Ks + row * kRowBytes + ((ch ^ k_swz(row)) << 4)) = kr[rr];
    }
    // transpose 4 keys x 8 dims into 8 rows of V^T (4 keys = 8 bytes each)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * ch + e;
      const int w = e >> 1;
      u32x2 val;
      if ((e & 1) == 0) {
        val[0] = pack_lo(vr[0][w], vr[1][w]);
        val[1] = pack_lo(vr[2][w], vr[3][w]);
      } else {
        val[0] = pack_hi(vr[0][w], vr[1][w]);
        val[1] = pack_hi(vr[2][w], vr[3][w]);
      }
      const int chunk = rg >> 1, half = rg & 1;
      *(u32x2*)(Vt + d * 128 + ((chunk ^ v_swz(d)) << 4) + half * 8) = val;
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int krow = key_of_row(l32);
  const int ksw = k_swz(krow);

  auto compute = [&](int buf, int kv0) {
    const unsigned char* Ks = smem + buf * kStage;
    const unsigned char* Vt = Ks + kKStage;
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
      const int cpos = ((2 * dk + g) ^ ksw) << 4;
      const bf16x8 a0 = *(const bf16x8*)(Ks + krow * kRowBytes + cpos);
      const bf16x8 a1 = *(const bf16x8*)(Ks + (krow + 32) * kRowBytes + cpos);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[dk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[dk], s1, 0, 0, 0);
    }
    // s0[r] = S[q][kv0 + 16 g + r], s1[r] = S[q][kv0 + 32 + 16 g + r]
    if (kv0 + kBN > N) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kv0 + 16 * g + r >= N) s0[r] = -INFINITY;
        if (kv0 + 32 + 16 * g + r >= N) s1[r] = -INFINITY;
      }
    }
    float mx = s0[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], c, -m_use));
      s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], c, -m_use));
      psum += s0[r] + s1[r];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    bf16x8 p[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[0][i] = (__bf16)s0[i];
      p[1][i] = (__bf16)s0[8 + i];
      p[2][i] = (__bf16)s1[i];
      p[3][i] = (__bf16)s1[8 + i];
    }
    // O^T += V^T P^T; step (kb, s) covers keys 32 kb + 16 g + 8 s + 0..7
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + l32;
      const unsigned char* vrow = Vt + d * 128;
      const int sw = v_swz(d);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int chunk = 4 * (st >> 1) + 2 * g + (st & 1);
        const bf16x8 a = *(const bf16x8*)(vrow + ((chunk ^ sw) << 4));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[st], oacc[db], 0, 0, 0);
      }
    }
  };

  load_kv(kv_start(0));
  store_kv(0);
  __syncthreads();
  for (int it = 0; it < nsub; ++it) {
    const int buf = it & 1;
    const int kv0 = kv_start(it);
    const bool more = it + 1 < nsub;
    if (more) load_kv(kv_start(it + 1));
    if (kv0 < N) compute(buf, kv0);
    if (more) store_kv(buf ^ 1);
    __syncthreads();
  }

  // O^T accumulators: oacc[db][4 j + i] = O[q][32 db + 8 j + 4 g + i]
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    uint16_t* orow = O + hoff + (size_t)qrow * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __bf16 b0 = (__bf16)(oacc[db][4 * j + 0] * inv);
        __bf16 b1 = (__bf16)(oacc[db][4 * j + 1] * inv);
        __bf16 b2 = (__bf16)(oacc[db][4 * j + 2] * inv);
        __bf16 b3 = (__bf16)(oacc[db][4 * j + 3] * inv);
        u32x2 w;
        w[0] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w[1] = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
               ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *(u32x2*)(orow + 32 * db + 8 * j + 4 * g) = w;
      }
  }
}

}  // namespace

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* out, const int32_t* idx, int keep, int heads, int tokens,
                            float scale, hipStream_t stream) {
  const int qtiles = (tokens + kBM - 1) / kBM;
  const long long blocks = (long long)heads * qtiles;
  if (blocks <= 0) return hipSuccess;
  const float c = scale * 1.4426950408889634f;  // scale * log2(e)
  if (idx)
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q,
                       k, v, out, idx, keep, tokens, qtiles, c);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, q,
                       k, v, out, idx, keep, tokens, qtiles, c);
  return hipGetLastError();
}

}  // namespace fvattn
