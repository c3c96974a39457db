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
//   rescale are per-lane scalars plus one swap between the two half-waves
//   (v_permlane32_swap, no LDS traffic).
// * The key rows fed to the S^T product are permuted inside each 32-key block
//   so that half-wave g ends up holding keys 16g..16g+15 contiguously; P^T can
//   then be passed to the PV product without any data movement.
// * K and V stream through LDS in 64-key stages, double buffered: the next
//   stage's 128-bit buffer loads are in flight while the current stage is
//   multiplied.  The buffer descriptor of each stage starts at the stage's first
//   key and ends at the last token, so the hardware range check zero-fills the
//   rows past the sequence end with no branches.  K and V are both stored
//   row-major with XOR swizzles on 16-byte chunks.  The V^T operand is read with
//   the gfx950 LDS transpose load (ds_read_b64_tr_b16), two per MFMA.
// * fp32 online softmax in the exp2 domain (scale * log2 e folded into one
//   FMA per score).  The running max is only raised, and O and the running sum
//   rescaled, when some row of the wave sees a score more than 2^8 above it
//   (wave-uniform branch); otherwise P may reach 2^8, which fp32 and bf16 hold
//   exactly as well as they hold 1.  P is rounded to bf16 for the PV product,
//   out to bf16.
// * Workgroups are remapped so each of the 8 XCDs walks a contiguous range of
//   (head, query tile) pairs, keeping one head's K/V hot in that XCD's L2.

#include <math.h>

#include <type_traits>

#include "fvattn_internal.h"

namespace fvattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBM = 128;                    // query rows per workgroup
constexpr int kBN = 64;                     // keys per LDS stage
constexpr int kThreads = 256;               // 4 waves x 32 query rows
constexpr int kRowBytes = kHeadDim * 2;     // 256 B per token row
constexpr int kKStage = kBN * kRowBytes;    // 16 KiB
constexpr int kVStage = kBN * kRowBytes;    // 16 KiB
constexpr int kStage = kKStage + kVStage;
constexpr int kLds = 2 * kStage;            // 64 KiB, two workgroups per CU
constexpr int kXcds = 8;
constexpr float kRescaleThreshold = 8.0f;   // log2 units
constexpr int kBufferFlags = 0x00020000;    // raw buffer, 32-bit data format

// K rows: chunk (16 B) swizzle; the 16 rows read by lanes 0..15 (and by 16..31)
// of one S^T operand load land on 16 distinct chunk positions.
__device__ __forceinline__ int k_swz(int row) {
  return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
}
// V rows: the 4 consecutive keys read by one 16-lane group of a transpose load
// land on distinct chunk positions.
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }

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

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes < 0 ? 0 : bytes,
                                           kBufferFlags);
}

// Combine x with its value in the other half-wave (lane l and lane l ^ 32).
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool kSparse>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, const int32_t* __restrict__ idx,
    int keep, int N, int qtiles, float c) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int h = L / qtiles, qt = L - h * qtiles;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const size_t hoff = (size_t)h * (size_t)N * kHeadDim;
  const uint16_t* Kh = K + hoff;
  const uint16_t* Vh = V + hoff;

  // Q^T fragment of this lane's query row (B operand of S^T = K Q^T):
  // qf[dk][i] = Q[qrow][16 dk + 8 g + i]; rows past N read as zero.
  const int q0 = qt * kBM + wave * 32;
  const int qrow = q0 + l32;
  bf16x8 qf[8];
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(Q + hoff + (size_t)q0 * kHeadDim, (N - q0) * kRowBytes);
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
      const u32x4 w =
          __builtin_amdgcn_raw_buffer_load_b128(rq, l32 * kRowBytes + 32 * dk + 16 * g, 0, 0);
      qf[dk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int32_t* irow = kSparse ? idx + ((size_t)h * qtiles + qt) * keep : nullptr;
  const int nsub = kSparse ? 2 * keep : (N + kBN - 1) / kBN;
  auto kv_start = [&](int it) -> int {
    if (!kSparse) return it * kBN;
    int t = irow[it >> 1];
    t = t < 0 ? 0 : (t >= qtiles ? qtiles - 1 : t);
    return t * kTile + (it & 1) * kBN;
  };

  // Global -> register staging: K and V rows rg + 16 rr, 16-byte chunk ch.
  const int ch = tid & 15, rg = tid >> 4;
  u32x4 kr[4], vr[4];
  auto load_kv = [&](int kv0) {
    const int rem = (N - kv0) * kRowBytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)kv0 * kHeadDim, rem);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)kv0 * kHeadDim, rem);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int off = (rg + 16 * rr) * kRowBytes + 16 * ch;
      kr[rr] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      vr[rr] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
    }
  };
  auto store_kv = [&](auto bufc) {
    unsigned char* Ks = smem + decltype(bufc)::value * kStage;
    unsigned char* Vs = Ks + kKStage;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = rg + 16 * rr;
      *(u32x4*)(Ks + row * kRowBytes + ((ch ^ k_swz(row)) << 4)) = kr[rr];
      *(u32x4*)(Vs + row * kRowBytes + ((ch ^ v_swz(row)) << 4)) = vr[rr];
    }
  };

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // S^T operand: row key_of_row(l32) (+32 for the second 32-key block), chunk
  // 2 dk + g; byte offsets within a stage, one per dk (the +32 rows and the
  // stage are immediate offsets).
  int koff[8];
  {
    const int krow = key_of_row(l32);
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) koff[dk] = krow * kRowBytes + (((2 * dk + g) ^ k_swz(krow)) << 4);
  }
  // V^T operand by transpose load: 16-lane group G = lane >> 4 covers head
  // dims 32 db + 16 (G & 1) + 0..15 and keys 32 kb + 16 (G >> 1) + 8 s + 0..7;
  // source lane s16 = lane & 15 reads 4 dims of key (s16 >> 2) (then + 4).
  // Byte offsets within a stage, one per db; the key steps (32 kb + 8 s, and
  // +4 for the second read) are whole rows and keep (key & 3), so they are
  // immediate offsets.
  int voff[4];
  {
    const int s16 = lane & 15, G = lane >> 4;
    const int vkey = 16 * (G >> 1) + (s16 >> 2);
    const int vdim = 16 * (G & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dim = vdim + 32 * db;
      voff[db] = kKStage + vkey * kRowBytes + (((dim >> 3) ^ v_swz(vkey)) << 4) + 8 * ((dim >> 2) & 1);
    }
  }

  auto compute = [&](auto bufc, int kv0) {
    const unsigned char* st_base = smem + decltype(bufc)::value * kStage;
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
      const bf16x8 a0 = *(const bf16x8*)(st_base + koff[dk]);
      const bf16x8 a1 = *(const bf16x8*)(st_base + koff[dk] + 32 * kRowBytes);
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
    mx = halfwave_max(mx) * c;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], c, -m_run));
      s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], c, -m_run));
      psum += s0[r] + s1[r];
    }
    l_run += psum;

    bf16x8 p[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[0][i] = (__bf16)s0[i];
      p[1][i] = (__bf16)s0[8 + i];
      p[2][i] = (__bf16)s1[i];
      p[3][i] = (__bf16)s1[8 + i];
    }
    // O^T += V^T P^T; step st = 2 kb + s covers keys 32 kb + 16 g + 8 s + 0..7
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const unsigned char* r0 = st_base + voff[db] + (32 * (st >> 1) + 8 * (st & 1)) * kRowBytes;
        const unsigned char* r1 = r0 + 4 * kRowBytes;
        const u32x2 lo =
            __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)r0));
        const u32x2 hi =
            __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)r1));
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), p[st],
                                                           oacc[db], 0, 0, 0);
      }
    }
  };

  // One stage: prefetch stage it+1 into registers, multiply stage it out of
  // LDS buffer `buf`, then park stage it+1 in the other buffer.  The loop is
  // unrolled by two so the buffer (and every LDS address offset) is a constant.
  auto step = [&](auto bufc, int it) {
    constexpr int buf = decltype(bufc)::value;
    const int kv0 = kv_start(it);
    const bool more = it + 1 < nsub;
    if (more) load_kv(kv_start(it + 1));
    if (kv0 < N) compute(bufc, kv0);
    if (more) store_kv(std::integral_constant<int, buf ^ 1>());
    __syncthreads();
  };
  load_kv(kv_start(0));
  store_kv(std::integral_constant<int, 0>());
  __syncthreads();
  for (int it = 0; it < nsub; it += 2) {
    step(std::integral_constant<int, 0>(), it);
    if (it + 1 < nsub) step(std::integral_constant<int, 1>(), it + 1);
  }

  // O^T accumulators: oacc[db][4 j + i] = O[q][32 db + 8 j + 4 g + i]
  const float inv = 1.f / halfwave_sum(l_run);
  if (qrow < N) {
    uint16_t* orow = O + hoff + (size_t)qrow * kHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const __bf16 b0 = (__bf16)(oacc[db][4 * j + 0] * inv);
        const __bf16 b1 = (__bf16)(oacc[db][4 * j + 1] * inv);
        const __bf16 b2 = (__bf16)(oacc[db][4 * j + 2] * inv);
        const __bf16 b3 = (__bf16)(oacc[db][4 * j + 3] * inv);
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
