// Fused attention forward for gfx950 (MI355X): dense, restricted to a list of
// 128-token key tiles per 128-token query tile (block-sparse), restricted to a
// frame window (Video DeltaNet's softmax branch), over VSA-H3's packed 3D-tile
// layout, or dense with INT8 or FP8 (E4M3) query-key scores.
//
// What it computes: out = softmax(scale * Q K^T) V per head, non-causal, the
// softmax taken over every key (dense), over the keys of the listed tiles only
// (sparse), or over the keys of the allowed frames (window); the scores are
// streamed tile by tile with an online softmax and never stored (FreeVideo
// page, section "Why it does not fit: the arithmetic"; FastH3 page, section
// "Lever two: VSA-H3 makes each of the four calls cheaper", fine stage: exact
// attention over the surviving tiles; FreeVideo page, section "Where Video
// DeltaNet comes in", for the window).
//
// Design (one workgroup = one head x kBM query rows, one wave per 32 rows;
// dense, sparse, window and VSA-H3: 4 waves, 128 rows (for sparse one
// selection tile), two workgroups per CU; INT8: 8 waves, 256 rows, one
// workgroup per CU; either way two waves per SIMD with 256 registers each):
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
// * K and V stream through LDS in 64-key stages, two slots each, written by the
//   buffer-load-to-LDS path (no registers involved); K runs two stages ahead
//   and V one.  The buffer descriptor of each stage starts at the stage's first
//   key and ends at the last token, so the hardware range check zero-fills rows
//   past the sequence end.  K and V are stored row-major with XOR swizzles on
//   16-byte chunks (each lane fetches the global chunk that belongs at its LDS
//   slot); the V^T operand is read with the gfx950 LDS transpose load
//   ds_read_b64_tr_b16; K and V operand reads run two MFMAs ahead of their
//   use.  Each slot is its own LDS array and the stage waits are explicit
//   vmcnt counts before a bare barrier, so no LDS read waits for loads it does
//   not consume.
// * Software pipeline per stage j: the S^T MFMAs of stage j+1 run while the
//   softmax of stage j (exp2, row sums, bf16 packing) runs on the vector ALU;
//   then the PV MFMAs of stage j run while the row max of stage j+1 is taken.
//   The interleaving is pinned with scheduling group barriers.  The scores
//   alternate between two register sets across two unrolled stages.  The wave
//   raises its issue priority for the PV region, so a SIMD shared with a wave
//   in its softmax keeps the matrix pipe busy.
// * fp32 online softmax in the exp2 domain (scale * log2 e folded into one
//   FMA per score).  The running max is only raised, and O and the running sum
//   rescaled, when some row of the wave sees a score more than 2^8 above it
//   (wave-uniform branch); otherwise P may reach 2^8, which fp32 and bf16 hold
//   exactly as well as they hold 1.  P is rounded to bf16 for the PV product,
//   out to bf16.
// * Workgroups are remapped so each of the 8 XCDs walks a contiguous range of
//   (head, query block) pairs, keeping one head's K/V hot in that XCD's L2.

#include <math.h>

#include <type_traits>

#include "fvattn_internal.h"

namespace fvattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowBytes = kHeadDim * 2;     // 256 B per token row
constexpr int kXcds = 8;
constexpr float kRescaleThreshold = 8.0f;   // log2 units
// LDS operand reads issued ahead of the MFMA that consumes them (two cover
// the read latency better than one; more gains nothing measurable).
constexpr int kReadAhead = 2;
constexpr int kBufferFlags = 0x00020000;    // raw buffer, 32-bit data format
// s_waitcnt immediates: vmcnt in bits 3:0, expcnt 6:4 (7 = no wait), lgkmcnt
// 11:8.  kWaitVm(n) waits until at most n buffer loads are in flight and every
// LDS access has completed.
constexpr int kWaitVmcnt0 = 0x0070;
constexpr int kWaitVm(int n) { return kWaitVmcnt0 | n; }

// K rows: chunk (16 B) swizzle; the 16 rows read by lanes 0..15 (and by 16..31)
// of one S^T operand load land on 16 distinct chunk positions.
__device__ __forceinline__ int k_swz(int row) {
  return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
}
// INT8 K rows (128 B): chunk swizzle; the 16 rows read by each 16-lane group of
// an S^T operand load fall on 16 distinct 16-byte bank groups (row parity
// selects the half of the 256-byte bank window, the swizzle the chunk).
__device__ __forceinline__ int k8_swz(int row) { return ((row >> 1) & 3) | (((row >> 4) & 1) << 2); }
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

// Buffer descriptor over `rows` rows of `row_bytes` bytes from `base` (fewer
// than 1 row: an empty range).  The byte count is the descriptor's 32-bit
// unsigned record count, formed in 64 bits: the host limits a head to fewer
// than 2^24 rows of at most 256 bytes, so it stays below 2^32.  (Only a
// lower clamp is applied: a min/max pair compiles to one vector med3, which
// would put the descriptor in vector registers and wrap every load through
// it in a readfirstlane loop.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int rows,
                                                            int row_bytes) {
  const long long bytes = rows > 0 ? (long long)rows * row_bytes : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFlags);
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

template <int B>
using Buf = std::integral_constant<int, B>;

// kWaves waves of 32 query rows (a workgroup covers kBM = 32 kWaves rows) and
// kStages LDS slots for each of K and V (loads run kStages - 1 stages ahead).
// The body lives in a __device__ template so that only the device compilation
// instantiates it; the __global__ wrapper below is all the host side sees.
// kMode: 0 dense, 1 per-head kept-tile lists of `keep` tiles, 2 frame-window
// lists shared by all heads (per-block counts, per-element frame mask), 3
// VSA-H3 per-head lists of 64-key sub-tiles over the padded tile layout (Q
// gathered from and O scattered to the packed token order), 4 dense with INT8
// query-key scores (K as int8 codes with per-64-key-block scales, Q quantized
// per row here; S^T on v_mfma_i32_32x32x32_i8, PV unchanged in bf16), 5 dense
// with FP8 (OCP E4M3) query-key scores (as 4, with E4M3 codes and S^T on the
// f8f6f4 matrix cores, v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation).
template <int kMode, int kWaves, int kStages, int kQB, int kBN>
__device__ __forceinline__ void attn_fwd_body(const uint16_t* __restrict__ Q,
                                              const uint16_t* __restrict__ K,
                                              const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                              const int32_t* __restrict__ idx, int keep, int N,
                                              int qtiles, float c, ListParams wp) {
  constexpr bool kI8 = kMode == 4;
  constexpr bool kF8 = kMode == 5;
  constexpr bool kQ8 = kI8 || kF8;                         // 8-bit Q and K codes
  constexpr bool kDenseWalk = kMode == 0 || kQ8;           // every key, no list
  constexpr int kKB = kBN / 32;               // 32-key MFMA blocks per stage
  constexpr int kTileBytes = kBN * kRowBytes; // one V (or bf16 K) stage
  constexpr int kKRowBytes = kQ8 ? kHeadDim : kRowBytes;      // K row in LDS: 8-bit or bf16
  constexpr int kKTileBytes = kBN * kKRowBytes;
  constexpr int kDK = kI8 ? 4 : (kF8 ? 2 : 8);   // MFMAs along the head dimension
  constexpr int kBM = 32 * kQB * kWaves;
  constexpr int kLoadsPerWave = kTileBytes / (1024 * kWaves);  // 1 KiB per wave-wide load
  constexpr int kKLoadsPerWave = kKTileBytes / (1024 * kWaves);
  static_assert(kKLoadsPerWave >= 1, "one wave-wide K load per wave at least");
  static_assert(!kQ8 || (kBN == 64 && kStages == 2), "8-bit key scales are per 64-key stage, loaded one stage ahead");
  constexpr int kPrefetch = kStages - 1;
  static_assert(kMode != 1 || kBM == kTile, "per-head lists cover one selection tile");
  static_assert(kMode != 3 || (kBN == 64 && kBM == kVsaRows),
                "VSA entries are 64-key stages of kVsaRows-row blocks");
  // One LDS array per slot: distinct objects let the compiler see that a read
  // of one slot cannot alias a buffer-to-LDS load still landing in another,
  // so it does not wait for every load in flight before each LDS read.
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[kKTileBytes], k_lds1[kKTileBytes],
      k_lds2[kStages > 2 ? kKTileBytes : 16];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[kTileBytes], v_lds1[kTileBytes],
      v_lds2[kStages > 2 ? kTileBytes : 16];
  unsigned char* const k_slots[3] = {k_lds0, k_lds1, k_lds2};
  unsigned char* const v_slots[3] = {v_lds0, v_lds1, v_lds2};

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int h = L / qtiles, qs = L - h * qtiles;
  const int qt = kMode != 2 ? qs : (qs + wp.first_block < qtiles ? qs + wp.first_block
                                                                 : qs + wp.first_block - qtiles);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const size_t hoff = (size_t)h * (size_t)N * kHeadDim;
  const unsigned char* Kh = (const unsigned char*)K + (size_t)h * N * kHeadDim * (kQ8 ? 1 : 2);
  const uint16_t* Vh = V + hoff;
  // VSA: N counts padded slots; Q and O keep the packed token order
  const int qn = kMode == 3 ? wp.vsa.tokens : N;
  const size_t qoff = (size_t)h * (size_t)qn * kHeadDim;

  // Q^T fragments of this lane's two query rows (B operands of S^T = K Q^T):
  // qf[qb][dk][i] = Q[q0 + 32 qb + l32][16 dk + 8 g + i]; rows past N read as 0.
  const int q0 = qt * kBM + wave * 32 * kQB;
  bf16x8 qf[kQB][8];
  i32x4 qf8[kQB][4];   // INT8 mode: codes of Q^T, 16 dims per lane per 32-dim block
  i32x8 qff[kQB][2];   // FP8 mode: E4M3 codes of Q^T, 32 dims per lane per 64-dim block
  float crow[kQB];     // INT8 mode: scale * log2(e) * (this row's query scale)
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) crow[qb] = c;
  if constexpr (kI8) {
    // lane (row l32, half g) holds dims 32 dk + 16 g + 0..15 of its row; the
    // row's scale is max |q| / 127 over both halves; rows past N read zeros
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(Q + hoff + (size_t)q0 * kHeadDim, N - q0, kRowBytes);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      u32x4 w[8];
      float m = 0.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        w[x] = __builtin_amdgcn_raw_buffer_load_b128(
            rq, (32 * qb + l32) * kRowBytes + 64 * (x >> 1) + 32 * g + 16 * (x & 1), 0, 0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t u = w[x][e >> 1];
          m = fmaxf(m, fabsf(__uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16))));
        }
      }
      m = halfwave_max(m);
      const float sq = m == 0.f ? 1.f : __fdiv_rn(m, 127.f);
      crow[qb] = c * sq;
#pragma unroll
      for (int dk = 0; dk < 4; ++dk) {
        i32x4 codes;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * wd + e;                       // dim 32 dk + 16 g + j
            const uint32_t u = w[2 * dk + (j >> 3)][(j & 7) >> 1];
            const float xv = __uint_as_float((j & 1) ? (u & 0xffff0000u) : (u << 16));
            float qv = __builtin_rintf(__fdiv_rn(xv, sq));
            qv = qv > 127.f ? 127.f : (qv < -127.f ? -127.f : qv);
            word |= (uint32_t)((int)qv & 0xff) << (8 * e);
          }
          codes[wd] = (int)word;
        }
        qf8[qb][dk] = codes;
      }
    }
  } else if constexpr (kF8) {
    // lane (row l32, half g) holds dims 64 dk + 32 g + 0..31 of its row; the
    // row's scale is max |q| / 448 over both halves; E4M3 codes nearest to
    // q / scale (correctly rounded float32 division, hardware conversion with
    // ties to even); rows past N read zeros
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(Q + hoff + (size_t)q0 * kHeadDim, N - q0, kRowBytes);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      u32x4 w[8];
      float m = 0.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        w[x] = __builtin_amdgcn_raw_buffer_load_b128(
            rq, (32 * qb + l32) * kRowBytes + 128 * (x >> 2) + 64 * g + 16 * (x & 3), 0, 0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t u = w[x][e >> 1];
          m = fmaxf(m, fabsf(__uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16))));
        }
      }
      m = halfwave_max(m);
      const float sq = m == 0.f ? 1.f : __fdiv_rn(m, 448.f);
      crow[qb] = c * sq;
      auto val = [&](int dk, int i) {   // dim 64 dk + 32 g + i
        const uint32_t u = w[4 * dk + (i >> 3)][(i & 7) >> 1];
        return __fdiv_rn(__uint_as_float((i & 1) ? (u & 0xffff0000u) : (u << 16)), sq);
      };
#pragma unroll
      for (int dk = 0; dk < 2; ++dk) {
        i32x8 codes;
#pragma unroll
        for (int wd = 0; wd < 8; ++wd) {
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(val(dk, 4 * wd), val(dk, 4 * wd + 1), 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(val(dk, 4 * wd + 2), val(dk, 4 * wd + 3), word, true);
          codes[wd] = word;
        }
        qff[qb][dk] = codes;
      }
    }
  } else if constexpr (kMode == 3) {
    // gather: the lane's slot holds token vsa_slot_token(slot); padding reads
    // past the end of the descriptor and gets zeros
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qoff, qn, kRowBytes);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int tok = vsa_slot_token(wp.vsa, q0 + 32 * qb + l32);
      const int row_off = (tok < 0 ? qn : tok) * kRowBytes;
#pragma unroll
      for (int dk = 0; dk < 8; ++dk) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rq, row_off + 32 * dk + 16 * g, 0, 0);
        qf[qb][dk] = __builtin_bit_cast(bf16x8, w);
      }
    }
  } else {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(Q + hoff + (size_t)q0 * kHeadDim, N - q0, kRowBytes);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int dk = 0; dk < 8; ++dk) {
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
            rq, (32 * qb + l32) * kRowBytes + 32 * dk + 16 * g, 0, 0);
        qf[qb][dk] = __builtin_bit_cast(bf16x8, w);
      }
  }

  const int ktiles = (N + kTile - 1) / kTile;
  const int32_t* irow = kMode == 1   ? idx + ((size_t)h * qtiles + qt) * keep
                        : kMode == 2 ? idx + (size_t)qt * wp.list_stride
                        : kMode == 3 ? idx + ((size_t)h * qtiles + qt) * (N / kBN)
                                     : nullptr;
  const int nsub = kDenseWalk   ? (N + kBN - 1) / kBN
                   : kMode == 3 ? wp.counts[(size_t)h * qtiles + qt]
                                : (kTile / kBN) * (kMode == 1 ? keep : wp.counts[qt]);
  // List entry of stage i (any i >= 0: past the end it repeats the last
  // entry, so the load never leaves the list), and the first key of stage i
  // from its entry.  Window lists flag (kMaskFlag) the key tiles that need
  // per-element masking for some row of this block; kv_of passes the flag on.
  constexpr int kSub = kMode == 3 ? 1 : kTile / kBN;   // stages per list entry
  const int nlist = kMode == 1 ? keep : kMode == 2 ? wp.counts[qt] : kMode == 3 ? nsub : 1;
  auto entry = [&](int i) -> int {
    const int j = i / kSub;
    return irow[j < nlist ? j : nlist - 1];
  };
  auto kv_of = [&](int e, int i) -> int {
    if (kDenseWalk) return i * kBN;
    if (kMode == 3) return (e & 0xffff) * kBN | (e & kMaskFlag);
    const int flag = kMode == 2 ? (e & kMaskFlag) : 0;
    int t = kMode == 2 ? (e & ~kMaskFlag) : e;
    t = t < 0 ? 0 : (t >= ktiles ? ktiles - 1 : t);
    return (t * kTile + (i % kSub) * kBN) | flag;
  };
  auto kv_start = [&](int i) -> int { return kv_of(kDenseWalk ? 0 : entry(i), i); };
  // Raw entries of stages it+1 .. it+kStages, loaded one stage before use and
  // decoded only where used, so no stage waits on a scalar list load it has
  // just issued.
  int ring[kStages];
#pragma unroll
  for (int j = 0; j < kStages; ++j) ring[j] = !kDenseWalk ? entry(1 + j) : 0;

  // Buffer-to-LDS loads: wave-wide load i of this wave fills LDS rows
  // 4 (kLoadsPerWave wave + i) + (lane >> 4), 16-byte slot lane & 15; the lane
  // fetches the global chunk that the swizzle places in that slot.
  int koffg[kKLoadsPerWave], voffg[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kKLoadsPerWave; ++i) {
    if constexpr (kQ8) {   // 8 rows of 128 B per wave-wide load
      const int row = 8 * (kKLoadsPerWave * wave + i) + (lane >> 3), slot = lane & 7;
      koffg[i] = row * kKRowBytes + ((slot ^ k8_swz(row)) << 4);
    } else {
      const int row = 4 * (kKLoadsPerWave * wave + i) + (lane >> 4), slot = lane & 15;
      koffg[i] = row * kKRowBytes + ((slot ^ k_swz(row)) << 4);
    }
  }
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int row = 4 * (kLoadsPerWave * wave + i) + (lane >> 4), slot = lane & 15;
    voffg[i] = row * kRowBytes + ((slot ^ v_swz(row)) << 4);
  }
  auto load_k = [&](int kv0, auto bufc) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(Kh + (size_t)kv0 * kKRowBytes, N - kv0, kKRowBytes);
    unsigned char* dst = k_slots[decltype(bufc)::value] + wave * kKLoadsPerWave * 1024;
#pragma unroll
    for (int i = 0; i < kKLoadsPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * 1024), 16, koffg[i], 0, 0, 0);
  };
  auto load_v = [&](int kv0, auto bufc) {
    const __amdgpu_buffer_rsrc_t r = make_rsrc(Vh + (size_t)kv0 * kHeadDim, N - kv0, kRowBytes);
    unsigned char* dst = v_slots[decltype(bufc)::value] + wave * kLoadsPerWave * 1024;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + i * 1024), 16, voffg[i], 0, 0, 0);
  };

  // S^T operand: row key_of_row(l32) (+32 for the second 32-key block), chunk
  // 2 dk + g; byte offsets within a stage, one per dk.  FP8 mode: 32 bytes per
  // lane, chunks 4 dk + 2 g and 4 dk + 2 g + 1 (koff, koff2).
  int koff[kDK], koff2[kDK];
  {
    const int krow = key_of_row(l32);
#pragma unroll
    for (int dk = 0; dk < kDK; ++dk) {
      if constexpr (kF8) {
        koff[dk] = krow * kKRowBytes + (((4 * dk + 2 * g) ^ k8_swz(krow)) << 4);
        koff2[dk] = krow * kKRowBytes + (((4 * dk + 2 * g + 1) ^ k8_swz(krow)) << 4);
      } else {
        koff[dk] = krow * kKRowBytes + (((2 * dk + g) ^ (kI8 ? k8_swz(krow) : k_swz(krow))) << 4);
        koff2[dk] = 0;
      }
    }
  }
  // V^T operand by transpose load: 16-lane group G = lane >> 4 covers head
  // dims 32 db + 16 (G & 1) + 0..15 and keys 32 kb + 16 (G >> 1) + 8 s + 0..7;
  // source lane s16 = lane & 15 reads 4 dims of key (s16 >> 2) (then + 4).
  // One byte offset per db; the key steps keep (key & 3) and are immediates.
  int voff[4];
  {
    const int s16 = lane & 15, G = lane >> 4;
    const int vkey = 16 * (G >> 1) + (s16 >> 2);
    const int vdim = 16 * (G & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dim = vdim + 32 * db;
      voff[db] = vkey * kRowBytes + (((dim >> 3) ^ v_swz(vkey)) << 4) + 8 * ((dim >> 2) & 1);
    }
  }

  f32x16 oacc[kQB][4];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
  float m_run[kQB], l_run[kQB];
#pragma unroll
  // VSA lists can open with stages a wave does not attend to (masked whole):
  // a finite start keeps exp2(S c - m) at exp2(-inf) = 0 there, where -inf
  // would give exp2(NaN).  The first real stage replaces it (alpha = 0).
  for (int qb = 0; qb < kQB; ++qb) {
    m_run[qb] = kMode == 3 ? -1e30f : -INFINITY;
    l_run[qb] = 0.f;
  }

  // S^T of one stage: S[qb][kb][r] = S[q0 + 32 qb + l32][kv0 + 32 kb + 16 g + r]
  auto qk = [&](auto bufc, f32x16 (&S)[kQB][kKB]) {
    const unsigned char* kb0 = k_slots[decltype(bufc)::value];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) S[qb][kb][r] = 0.f;
#pragma unroll
    for (int dk = 0; dk < kDK; ++dk)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        if constexpr (kF8) {
          // E4M3 x E4M3 on the f8f6f4 matrix cores (format 0 on both sides,
          // unit block scales: E8M0 127 = 2^0), fp32 accumulation
          const i32x4 a0 = *(const i32x4*)(kb0 + koff[dk] + kb * 32 * kKRowBytes);
          const i32x4 a1 = *(const i32x4*)(kb0 + koff2[dk] + kb * 32 * kKRowBytes);
          const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            S[qb][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qff[qb][dk], S[qb][kb], 0, 0,
                                                                         0, 127, 0, 127);
        } else if constexpr (kI8) {
          // int32 scores in the float registers (bit patterns); converted after
          const i32x4 a = *(const i32x4*)(kb0 + koff[dk] + kb * 32 * kKRowBytes);
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            S[qb][kb] = __builtin_bit_cast(
                f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            a, qf8[qb][dk], __builtin_bit_cast(i32x16, S[qb][kb]), 0, 0, 0));
        } else {
          const bf16x8 a = *(const bf16x8*)(kb0 + koff[dk] + kb * 32 * kKRowBytes);
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb)
            S[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][dk], S[qb][kb], 0, 0, 0);
        }
      }
  };
  // INT8 mode: the exact int32 scores to float (|S| < 2^24, exact).  The
  // whole accumulator is reinterpreted at once: a bit cast of one vector
  // element does not read that element.
  auto to_float = [&](f32x16 (&S)[kQB][kKB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
        S[qb][kb] = __builtin_convertvector(__builtin_bit_cast(i32x16, S[qb][kb]), f32x16);
  };
  // Keys past N: -inf scores.  Only stages that reach past the end need it.
  auto mask = [&](f32x16 (&S)[kQB][kKB], int kv0) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kv0 + 32 * kb + 16 * g + r >= N) {
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) S[qb][kb][r] = -INFINITY;
        }
  };
  // Frame window (kMode 2): a key frame is allowed for this lane's query frame
  // if their chunks are within wp.neighbours of each other or either frame is
  // the first or last one.  frame_tokens >= 64, so a 64-key stage spans at
  // most two frames; stages where every lane allows both skip the masking.
  // Frame 0 is an anchor and every list starts with key tile 0, so stage 0
  // (keys 0..63, all of frame 0) is open to every row: the running max is
  // finite from the prologue on, and a later stage masked whole for a row adds
  // exp2(-inf) = 0 to it.  Non-video tokens (text, audio) ahead of the video:
  // frames are counted from the first video token, a prefix query is treated
  // as an anchor (it sees every key), and a stage holding prefix keys can
  // only hold frame-0 keys besides them (frame_tokens >= 64), all open to
  // every query: the prefix keys fall in the stage's first frame (ok0).
  int q_chunk[kQB];
  bool q_anchor[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int qrow = q0 + 32 * qb + l32;
    const int qf = kMode == 2 && qrow >= wp.prefix ? (qrow - wp.prefix) / wp.frame_tokens : 0;
    q_chunk[qb] = kMode == 2 ? qf / wp.chunk_frames : 0;
    q_anchor[qb] = qrow < wp.prefix || qf == 0 || qf >= wp.frames - 1;
  }
  auto frame_ok = [&](int qb, int kf) {
    const int dc = q_chunk[qb] - kf / wp.chunk_frames;
    return q_anchor[qb] || kf == 0 || kf == wp.frames - 1 || (dc <= wp.neighbours && -dc <= wp.neighbours);
  };
  auto window_mask = [&](f32x16 (&S)[kQB][kKB], int kv0) {
    const int kf0 = (kv0 > wp.prefix ? kv0 - wp.prefix : 0) / wp.frame_tokens;
    const int next_frame = wp.prefix + (kf0 + 1) * wp.frame_tokens;   // first key of frame kf0 + 1
    bool ok0[kQB], ok1[kQB];
    bool need = kv0 + kBN > N;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      ok0[qb] = frame_ok(qb, kf0);
      ok1[qb] = next_frame >= kv0 + kBN || frame_ok(qb, kf0 + 1);
      need = need || !ok0[qb] || !ok1[qb];
    }
    if (!__builtin_amdgcn_ballot_w64(need)) return;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * kb + 16 * g + r;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          if (key >= N || !(key < next_frame ? ok0[qb] : ok1[qb])) S[qb][kb][r] = -INFINITY;
      }
  };
  // VSA (kMode 3), flagged entries only: a wave whose 64-row query group does
  // not attend to the sub-tile masks the whole stage; otherwise keys past the
  // sub-tile's valid count (padding slots) are masked.
  auto vsa_mask = [&](f32x16 (&S)[kQB][kKB], int e) {
    if (!((e >> (kVsaGroupShift + (wave >> 1))) & 1)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) S[qb][kb][r] = -INFINITY;
      return;
    }
    const int n = ((e >> kVsaCountShift) & 63) + 1;
    if (n == kBN) return;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + 16 * g + r >= n) {
#pragma unroll
          for (int qb = 0; qb < kQB; ++qb) S[qb][kb][r] = -INFINITY;
        }
  };
  // Row max of a stage, in scaled log2 units.
  // cm[qb]: the multiplier of this stage's scores (c, or in INT8 mode
  // crow * the stage's key scale).
  auto rowmax = [&](const f32x16 (&S)[kQB][kKB], float (&mx)[kQB], const float (&cm)[kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float m = S[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, S[qb][kb][r]);
      mx[qb] = halfwave_max(m) * cm[qb];
    }
  };
  // Raise the running max (and rescale O and the sums) when some row of the
  // wave exceeds it by more than 2^8.
  auto maybe_rescale = [&](const float (&mx)[kQB]) {
    bool up = false;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) up |= mx[qb] > m_run[qb] + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(up)) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const float m_new = fmaxf(m_run[qb], mx[qb]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);   // 0 on the first stage
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
      }
    }
  };
  // P = exp2(S c - m) as bf16 B-operands; P[qb][st] covers keys 32 kb + 16 g + 8 s + 0..7
  // with st = 2 kb + s.  The running sum adds the bf16 values of P, the ones
  // the PV product multiplies, two at a time with v_dot2_f32_bf16 (half the
  // vector instructions of adding the fp32 values one by one; 1% faster).
  auto softmax = [&](const f32x16 (&S)[kQB][kKB], bf16x8 (&P)[kQB][2 * kKB], const float (&cm)[kQB]) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 one = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float ps[2] = {0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[qb][kb][r], cm[qb], -m_run[qb]));
          P[qb][2 * kb + (r >> 3)][r & 7] = (__bf16)p;
        }
#pragma unroll
      for (int st = 0; st < 2 * kKB; ++st)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const bf16x2 pr = {P[qb][st][2 * w], P[qb][st][2 * w + 1]};
          ps[w & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, ps[w & 1], false);
        }
      l_run[qb] += ps[0] + ps[1];
    }
  };
  // O^T += V^T P^T for one stage.
  auto pv = [&](auto bufc, const bf16x8 (&P)[kQB][2 * kKB]) {
    const unsigned char* vb0 = v_slots[decltype(bufc)::value];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int st = 0; st < 2 * kKB; ++st) {
        const unsigned char* r0 = vb0 + voff[db] + (32 * (st >> 1) + 8 * (st & 1)) * kRowBytes;
        const u32x2 lo =
            __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)r0));
        const u32x2 hi = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r0 + 4 * kRowBytes)));
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[qb][st], oacc[qb][db], 0, 0, 0);
      }
  };

  f32x16 SA[kQB][kKB], SB[kQB][kKB];
  bf16x8 P[kQB][2 * kKB];

  // Stage `it` (k = it mod kUnroll): its scores are in Scur (max already
  // folded into m_run); K(it+1) is in K slot (k+1) mod kStages and V(it) in V
  // slot k mod kStages.  It starts K(it+kStages) and V(it+kStages-1) into the
  // slots stage it-1 finished with.  Two scheduling regions: (1) softmax of
  // stage it on the vector ALU interleaved with the S^T MFMAs of stage it+1
  // (into Snext), (2) the PV MFMAs of stage it interleaved with the row max of
  // stage it+1.  On the last stage the S^T product reads a stale slot and its
  // result is discarded.
  auto loads_at = [&](int i) {   // wave-wide loads a stage issues (uniform)
    return (i + kStages < nsub ? kKLoadsPerWave : 0) + (i + kPrefetch < nsub ? kLoadsPerWave : 0);
  };
  // INT8 mode: key scales of stages it (sk_cur), it+1 (sk_next) and it+2
  // (loaded during stage it with a vector load, so the stage-top vmcnt wait
  // covers it).  Other modes: the multiplier is c throughout.
  const __amdgpu_buffer_rsrc_t rks =
      make_rsrc(kQ8 ? wp.kscale + (size_t)h * nsub : nullptr, kQ8 ? nsub : 0, 4);
  auto key_scale = [&](int i) -> float {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, 4 * i, 0, 0));
  };
  float sk_cur = 1.f, sk_next = 1.f;
  auto multipliers = [&](float sk, float (&cm)[kQB]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) cm[qb] = kQ8 ? crow[qb] * sk : c;
  };
  auto stage = [&](auto kc, int it, f32x16 (&Scur)[kQB][kKB], f32x16 (&Snext)[kQB][kKB]) {
    constexpr int k = decltype(kc)::value;
    constexpr int kSlotK = (k + 1) % kStages, kSlotV = k % kStages;
    // K(it+1) and V(it) were started kPrefetch stages ago; only the loads of
    // the stages after that may still be in flight.
    const int newer = (kPrefetch >= 2 && it >= 1) ? loads_at(it - 1) : 0;
    if (newer == 2 * kLoadsPerWave)
      __builtin_amdgcn_s_waitcnt(kWaitVm(2 * kLoadsPerWave));
    else if (newer == kLoadsPerWave)
      __builtin_amdgcn_s_waitcnt(kWaitVm(kLoadsPerWave));
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm(0));
    // A bare barrier: the waits above cover every load this stage reads, and
    // every LDS read of the previous stage has completed (its results were
    // consumed), so no wave can still be reading the slots refilled below.
    __builtin_amdgcn_s_barrier();
    const bool has_next = it + 1 < nsub;
    // dense stages are plain arithmetic; list stages come from the ring
    const int kv_next = kv_of(ring[0], it + 1);
    if (it + kStages < nsub) load_k(kv_of(ring[kStages - 1], it + kStages) & ~kMaskFlag, Buf<k % kStages>());
    if (it + kPrefetch < nsub)
      load_v(kv_of(ring[kPrefetch - 1], it + kPrefetch) & ~kMaskFlag, Buf<(k + kStages - 1) % kStages>());
    const int ahead = !kDenseWalk ? entry(it + 1 + kStages) : 0;
    const float sk_ahead = kQ8 ? key_scale(it + 2) : 1.f;
    float cm_cur[kQB], cm_next[kQB];
    multipliers(sk_cur, cm_cur);
    multipliers(sk_next, cm_next);

    softmax(Scur, P, cm_cur);
    qk(Buf<kSlotK>(), Snext);
    // Region 1: one K-operand read per (dk, kb) feeds kQB MFMAs; the softmax's
    // ~56 kQB kKB VALU instructions are spread between the MFMAs.  Reads run
    // kReadAhead operands ahead.
    {
      constexpr int kOps = kDK * kKB, kValuPerMfma = (56 * kKB * kQB + kOps * kQB - 1) / (kOps * kQB);
      constexpr int kReads = kF8 ? 2 : 1;   // LDS reads per K operand
#pragma unroll
      for (int o = 0; o < kReadAhead; ++o) __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
      for (int o = 0; o < kOps; ++o) {
        if (o + kReadAhead < kOps) __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
        }
      }
    }

    if constexpr (kI8) to_float(Snext);
    if constexpr (kMode == 2) {
      if (has_next && (kv_next & kMaskFlag)) window_mask(Snext, kv_next & ~kMaskFlag);
    } else if constexpr (kMode == 3) {
      if (has_next && (kv_next & kMaskFlag)) vsa_mask(Snext, ring[0]);
    } else if (has_next && kv_next + kBN > N) {
      mask(Snext, kv_next);
    }

    float mx[kQB];
    // Raise this wave's issue priority for the MFMA-heavy PV region: when the
    // other wave on the SIMD is in its softmax, the matrix pipe stays fed.
    __builtin_amdgcn_s_setprio(1);
    pv(Buf<kSlotV>(), P);
    rowmax(Snext, mx, cm_next);
    // Region 2: two transpose reads per (db, st) V operand feed kQB MFMAs; the
    // row max of the next stage (and in INT8 mode the conversion of its
    // scores) fills the gaps: one vector instruction per MFMA (0.5% faster
    // than two), three in INT8 mode (0.8% faster than four); either way the
    // same instructions.  Reads run kReadAhead operands ahead.
    {
      constexpr int kOps = 4 * 2 * kKB, kValu = kI8 ? 3 : 1;
#pragma unroll
      for (int o = 0; o < kReadAhead; ++o) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
#pragma unroll
      for (int o = 0; o < kOps; ++o) {
        if (o + kReadAhead < kOps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x002, kValu, 1);
        }
      }
    }

    __builtin_amdgcn_s_setprio(0);
    if (has_next) maybe_rescale(mx);
    if constexpr (!kDenseWalk) {
#pragma unroll
      for (int j = 0; j + 1 < kStages; ++j) ring[j] = ring[j + 1];
      ring[kStages - 1] = ahead;
    }
    sk_cur = sk_next;
    sk_next = sk_ahead;
  };

  // prologue: K(0..kStages-1) and V(0..kStages-2) started, scores and max of stage 0
  {
    const int kv0e = kv_start(0), kv0 = kv0e & ~kMaskFlag;
    load_k(kv0, Buf<0>());
    const int kv1 = kv_of(ring[0], 1) & ~kMaskFlag;
    if (1 < nsub) load_k(kv1, Buf<1 % kStages>());
    if (kStages > 2 && 2 < nsub) load_k(kv_of(ring[1], 2) & ~kMaskFlag, Buf<2 % kStages>());
    load_v(kv0, Buf<0>());
    if (kStages > 2 && 1 < nsub) load_v(kv1, Buf<1 % kStages>());
    if constexpr (kQ8) {
      sk_cur = key_scale(0);
      sk_next = key_scale(1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm(0));
    __builtin_amdgcn_s_barrier();
    qk(Buf<0>(), SA);
    if constexpr (kI8) to_float(SA);
    if constexpr (kMode == 2) {
      if (kv0e & kMaskFlag) window_mask(SA, kv0);
    } else if constexpr (kMode == 3) {
      if (kv0e & kMaskFlag) vsa_mask(SA, entry(0));
    }
    else if (kv0 + kBN > N) mask(SA, kv0);
    float mx[kQB], cm0[kQB];
    multipliers(sk_cur, cm0);
    rowmax(SA, mx, cm0);
    maybe_rescale(mx);
  }
  // Unrolled so that every slot and score register set is a constant.
  constexpr int kUnroll = kStages % 2 ? 2 * kStages : kStages;
  for (int it = 0; it < nsub; it += kUnroll) {
    stage(Buf<0>(), it, SA, SB);
    if (it + 1 < nsub) stage(Buf<1>(), it + 1, SB, SA);
    if (kUnroll > 2 && it + 2 < nsub) stage(Buf<2 % kUnroll>(), it + 2, SA, SB);
    if (kUnroll > 3 && it + 3 < nsub) stage(Buf<3 % kUnroll>(), it + 3, SB, SA);
    if (kUnroll > 4 && it + 4 < nsub) stage(Buf<4 % kUnroll>(), it + 4, SA, SB);
    if (kUnroll > 5 && it + 5 < nsub) stage(Buf<5 % kUnroll>(), it + 5, SB, SA);
  }

  // O^T accumulators: oacc[qb][db][4 j + i] = O[q0 + 32 qb + l32][32 db + 8 j + 4 g + i]
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float inv = 1.f / halfwave_sum(l_run[qb]);
    const int qrow = q0 + 32 * qb + l32;
    const int orow_idx = kMode == 3 ? vsa_slot_token(wp.vsa, qrow) : (qrow < N ? qrow : -1);
    if (orow_idx >= 0) {
      uint16_t* orow = O + qoff + (size_t)orow_idx * kHeadDim;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const __bf16 b0 = (__bf16)(oacc[qb][db][4 * j + 0] * inv);
          const __bf16 b1 = (__bf16)(oacc[qb][db][4 * j + 1] * inv);
          const __bf16 b2 = (__bf16)(oacc[qb][db][4 * j + 2] * inv);
          const __bf16 b3 = (__bf16)(oacc[qb][db][4 * j + 3] * inv);
          u32x2 w;
          w[0] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
          w[1] = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
          *(u32x2*)(orow + 32 * db + 8 * j + 4 * g) = w;
        }
    }
  }
}

// kQB = 1: 32 query rows per wave, two waves per SIMD (256 registers each);
// kQB = 2: 64 rows per wave, one wave per SIMD with the whole register file.
template <int kMode, int kWaves, int kStages, int kQB, int kBN>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(3 - kQB, 3 - kQB))) void
attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                const int32_t* __restrict__ idx, int keep, int N, int qtiles, float c,
                ListParams wp) {
  attn_fwd_body<kMode, kWaves, kStages, kQB, kBN>(Q, K, V, O, idx, keep, N, qtiles, c, wp);
}

}  // namespace

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            uint16_t* out, const int32_t* idx, int keep, int heads, int tokens,
                            float scale, hipStream_t stream) {
  const float c = scale * 1.4426950408889634f;  // scale * log2(e)
  if (idx) {
    // one 128-row selection tile per workgroup (4 waves), 2 workgroups per CU
    const int qtiles = (tokens + kTile - 1) / kTile;
    const long long blocks = (long long)heads * qtiles;
    if (blocks <= 0) return hipSuccess;
    attn_fwd_kernel<1, 4, 2, 1, 64><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        q, k, v, out, idx, keep, tokens, qtiles, c, ListParams{});
  } else {
    // 128 query rows per workgroup (4 waves) share each K/V stage (two LDS
    // slots each for K and V); two workgroups per CU, so the two waves of a
    // SIMD belong to different workgroups and never wait at each other's
    // stage barrier (2-3% faster than one 8-wave workgroup of 256 rows)
    const int qtiles = (tokens + 127) / 128;
    const long long blocks = (long long)heads * qtiles;
    if (blocks <= 0) return hipSuccess;
    attn_fwd_kernel<0, 4, 2, 1, 64><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        q, k, v, out, idx, keep, tokens, qtiles, c, ListParams{});
  }
  return hipGetLastError();
}

hipError_t window_lists_fit(int tokens, const ListParams& wp) {
  const int blocks = (tokens + kWindowRows - 1) / kWindowRows;
  const int ktiles = (tokens + kTile - 1) / kTile;
  if (tokens < 0 || wp.list_rows != kWindowRows || wp.list_count < blocks || wp.list_stride < ktiles)
    return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_attention_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   uint16_t* out, const int32_t* idx, const ListParams& wp,
                                   int heads, int tokens, float scale, hipStream_t stream) {
  // kWindowRows query rows per workgroup (one wave per 32); idx and
  // wp.counts hold one list per kWindowRows-row block, wp.list_stride entries
  // apart; a list layout that does not match is refused before any launch
  const hipError_t fit = window_lists_fit(tokens, wp);
  if (fit != hipSuccess) return fit;
  const float c = scale * 1.4426950408889634f;  // scale * log2(e)
  const int qtiles = (tokens + kWindowRows - 1) / kWindowRows;
  const long long blocks = (long long)heads * qtiles;
  if (blocks <= 0) return hipSuccess;
  attn_fwd_kernel<2, kWindowRows / 32, 2, 1, 64>
      <<<dim3((unsigned)blocks), dim3(2 * kWindowRows), 0, stream>>>(
      q, k, v, out, idx, 0, tokens, qtiles, c, wp);
  return hipGetLastError();
}

hipError_t launch_attention_int8(const uint16_t* q, const uint8_t* kq, const uint16_t* v,
                                 uint16_t* out, const ListParams& lp, int heads, int tokens,
                                 float scale, hipStream_t stream) {
  // 128 query rows per workgroup (4 waves), two workgroups per CU, as dense
  // (2.2% faster than 8-wave, 256-row workgroups, same output)
  const float c = scale * 1.4426950408889634f;  // scale * log2(e)
  const int qtiles = (tokens + 127) / 128;
  const long long blocks = (long long)heads * qtiles;
  if (blocks <= 0) return hipSuccess;
  attn_fwd_kernel<4, 4, 2, 1, 64><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      q, (const uint16_t*)kq, v, out, nullptr, 0, tokens, qtiles, c, lp);
  return hipGetLastError();
}

hipError_t launch_attention_fp8(const uint16_t* q, const uint8_t* kq, const uint16_t* v,
                                uint16_t* out, const ListParams& lp, int heads, int tokens,
                                float scale, hipStream_t stream) {
  // 256 query rows per workgroup (8 waves: 3.2% faster than two 4-wave
  // workgroups per CU for this mode, same output)
  const float c = scale * 1.4426950408889634f;  // scale * log2(e)
  const int qtiles = (tokens + 255) / 256;
  const long long blocks = (long long)heads * qtiles;
  if (blocks <= 0) return hipSuccess;
  attn_fwd_kernel<5, 8, 2, 1, 64><<<dim3((unsigned)blocks), dim3(512), 0, stream>>>(
      q, (const uint16_t*)kq, v, out, nullptr, 0, tokens, qtiles, c, lp);
  return hipGetLastError();
}

hipError_t launch_attention_vsa(const uint16_t* q, const uint16_t* kp, const uint16_t* vp,
                                uint16_t* out, const int32_t* lists, const ListParams& lp,
                                int heads, float scale, hipStream_t stream) {
  // kVsaRows padded query slots per workgroup (one wave per 32), one list of
  // 64-key sub-tiles per (head, block)
  const float c = scale * 1.4426950408889634f;  // scale * log2(e)
  const int qtiles = (lp.vsa.npad + kVsaRows - 1) / kVsaRows;
  const long long blocks = (long long)heads * qtiles;
  if (blocks <= 0) return hipSuccess;
  attn_fwd_kernel<3, kVsaRows / 32, 2, 1, 64>
      <<<dim3((unsigned)blocks), dim3(2 * kVsaRows), 0, stream>>>(
      q, kp, vp, out, lists, 0, lp.vsa.npad, qtiles, c, lp);
  return hipGetLastError();
}

}  // namespace fvattn
