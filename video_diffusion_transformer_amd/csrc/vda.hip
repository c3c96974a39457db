// Video Delta Attention, the linear branch of Video DeltaNet, on gfx950
// (FreeVideo page, "FreeVideo: a 66 GB video transformer on an 8 GB card...",
// section "Where Video DeltaNet comes in").
//
// Per head, with d = 128 and a latent frame t of frame_tokens tokens:
//   A_t = sum_u beta_u k_u k_u^T,  B_t = sum_u beta_u v_u k_u^T,
//   S_t = (S_prev Diag(alpha_t) + B_t)(I + A_t)^-1 = S_prev P_t + C_t
// with M_t = (I + A_t)^-1, P_t = Diag(alpha_t) M_t and C_t = B_t M_t.  Everything
// but the last line is independent per frame, so it runs for all interior
// frames at once; only S_t = S_prev P_t + C_t is sequential.  The forward scan writes
// frames 1..F-2 in order, the reverse scan F-2..1, both from S_text / 2 (the
// first and last frames are softmax anchors and are not written).  A query of
// frame f reads o = fwd[lo(f)] q + rev[hi(f)] q, lo / hi the frames just
// before and after its softmax window (both seeds for the anchor frames).
//
// Every product runs on the matrix cores at fp32 accuracy.  Where one operand
// is bf16 already (k, v, q), the fp32 operand is split into bf16 hi + lo parts
// and the two products run on the bf16 MFMA with fp32 accumulation (A_t, B_t
// and the readout); the rest uses v_mfma_f32_32x32x2_f32 (lane l holds
// A[l % 32][l / 32] and B[l / 32][l % 32]).  The inverse is a Gauss-Jordan
// elimination held in the matrix-core accumulators, which needs no pivoting
// because I + A_t is symmetric with eigenvalues >= 1.
//
// Kernels: vda_stats_kernel (A_t, B_t per frame), vda_inverse_kernel (M_t and
// P_t^T), vda_matmul_kernel (C_t = B_t M_t), vda_scan_kernel (one workgroup per
// head, direction and 32-row band of the state), vda_readout_kernel.

#include "fvattn_internal.h"

namespace fvattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// A_t and B_t of frame t of head h on the bf16 matrix cores: with X = beta K
// and Y = beta V split into bf16 hi + lo parts (residual <= 2^-18 of each
// value), A_t = X_hi^T K + X_lo^T K and B_t = Y_hi^T K + Y_lo^T K, fp32
// accumulation (K is bf16 already).  The frame streams through LDS in 64-token
// chunks of five tiles (K, X_hi, X_lo, Y_hi, Y_lo), rows of 256 B with 16-byte
// chunks XOR-swizzled by v_swz.  Every MFMA operand is 8 tokens of one head
// dim, read with ds_read_b64_tr_b16; both operands use the same addressing,
// so they agree on which token each reduction index holds.  Wave w owns row
// tile w of A_t and of B_t (8 accumulator tiles).
typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2s __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kChunk = 64;               // tokens per LDS chunk
constexpr int kTileB = kChunk * kD * 2;  // bytes of one chunk tile

__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void vda_stats_kernel(const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V,
                                                        const float* __restrict__ beta, int ft,
                                                        int frames, float* __restrict__ A,
                                                        float* __restrict__ B) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[5][kTileB];   // K, X_hi, X_lo, Y_hi, Y_lo
  const int t = blockIdx.x + 1, h = blockIdx.y;   // interior frames only
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const size_t N = (size_t)frames * ft;
  const size_t tok0 = (size_t)h * N + (size_t)t * ft;
  // transpose-read offset of head-dim block db: lane group G = lane >> 4 covers
  // dims 32 db + 16 (G & 1) + 0..15 and tokens 16 (G >> 1) + 8 s + 0..7 of a
  // 32-token half; source lane s16 reads 4 dims of token (s16 >> 2) (then + 4)
  int voff[4];
  {
    const int s16 = lane & 15, G = lane >> 4;
    const int vkey = 16 * (G >> 1) + (s16 >> 2);
    const int vdim = 16 * (G & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int dim = vdim + 32 * db;
      voff[db] = vkey * kD * 2 + (((dim >> 3) ^ v_swz(vkey)) << 4) + 8 * ((dim >> 2) & 1);
    }
  }
  auto frag = [&](int tile, int db, int st) -> bf16x8s {
    const unsigned char* r0 = lds[tile] + voff[db] + (32 * (st >> 1) + 8 * (st & 1)) * kD * 2;
    const u32x2s lo = __builtin_bit_cast(u32x2s, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)r0));
    const u32x2s hi = __builtin_bit_cast(
        u32x2s, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(r0 + 4 * kD * 2)));
    const u32x4s x = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8s, x);
  };
  f32x16 acc_a[4], acc_b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc_a[j][r] = 0.f; acc_b[j][r] = 0.f; }
  // raw K, V and beta of a chunk, 64 tokens x 16 chunks of 8 dims, 4 per
  // thread; the next chunk's loads are in flight while this one is multiplied
  u32x4s kw[4], vw[4];
  float bw[4];
  auto fetch = [&](int u0) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int pos = tid + 256 * x, row = pos >> 4, c = pos & 15;
      const int u = u0 + row;
      kw[x] = u32x4s{0u, 0u, 0u, 0u};
      vw[x] = u32x4s{0u, 0u, 0u, 0u};
      bw[x] = 0.f;
      if (u < ft) {
        kw[x] = *(const u32x4s*)(K + (tok0 + u) * kD + 8 * c);
        vw[x] = *(const u32x4s*)(V + (tok0 + u) * kD + 8 * c);
        bw[x] = beta[tok0 + u];
      }
    }
  };
  fetch(0);
  for (int u0 = 0; u0 < ft; u0 += kChunk) {
    __syncthreads();   // the previous chunk has been consumed
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int pos = tid + 256 * x, row = pos >> 4, c = pos & 15;
      const float b = bw[x];
      bf16x8s xh, xl, yh, yl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t kk = kw[x][e >> 1], vv = vw[x][e >> 1];
        const float kf = __uint_as_float((e & 1) ? (kk & 0xffff0000u) : (kk << 16));
        const float vf = __uint_as_float((e & 1) ? (vv & 0xffff0000u) : (vv << 16));
        const float xk = b * kf, yv = b * vf;
        xh[e] = (__bf16)xk;
        xl[e] = (__bf16)(xk - (float)xh[e]);
        yh[e] = (__bf16)yv;
        yl[e] = (__bf16)(yv - (float)yh[e]);
      }
      const int off = row * kD * 2 + ((c ^ v_swz(row)) << 4);
      *(u32x4s*)(lds[0] + off) = kw[x];
      *(bf16x8s*)(lds[1] + off) = xh;
      *(bf16x8s*)(lds[2] + off) = xl;
      *(bf16x8s*)(lds[3] + off) = yh;
      *(bf16x8s*)(lds[4] + off) = yl;
    }
    __syncthreads();
    if (u0 + kChunk < ft) fetch(u0 + kChunk);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bf16x8s xh = frag(1, w, st), xl = frag(2, w, st), yh = frag(3, w, st), yl = frag(4, w, st);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8s kf = frag(0, j, st);
        acc_a[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, kf, acc_a[j], 0, 0, 0);
        acc_a[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, kf, acc_a[j], 0, 0, 0);
        acc_b[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yh, kf, acc_b[j], 0, 0, 0);
        acc_b[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yl, kf, acc_b[j], 0, 0, 0);
      }
    }
  }
  const size_t off = ((size_t)h * frames + t) * kMat;
  store_row_tile(A + off, w, acc_a, lane);
  store_row_tile(B + off, w, acc_b, lane);
}

// M_t = (I + A_t)^-1 by Gauss-Jordan elimination in place, four pivots per
// step, and P_t^T for P_t = Diag(alpha_t) M_t (M_t is symmetric, so P_t^T[i][j]
// = alpha_t[j] M_t[i][j]).  The matrix never leaves the fp32
// matrix-core accumulators: wave w holds tiles (w, 0..3).  Step q pivots on
// K = {4q..4q+3} with the 4 x 4 block P = a[K][K] and Pinv = P^-1:
//   a[K][j] <- Pinv a[K][j] (j not in K),   a[K][K] <- Pinv,
//   a[i][j] <- a[i][j] - a[i][K] Pinv a[K][j],   a[i][K] <- -a[i][K] Pinv   (i not in K),
// which is a single rank-4 update a <- a0 - C R, where a0 is a with row K and
// column K zeroed, C = a[:][K] except C[K][K] = -I, and R = Pinv a[K][:] except
// R[K][K] = Pinv (two v_mfma_f32_32x32x2_f32 per tile).  No pivoting: every P
// is a Schur complement of the symmetric I + A_t, so its eigenvalues stay >= 1.
// Row K reaches every wave through LDS (double buffered: one barrier per
// step); column K stays within each wave; every lane inverts P itself.
// Interior frames only (blockIdx.x + 1): the scans never read the anchors.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void vda_inverse_kernel(const float* __restrict__ A, const float* __restrict__ alpha, int frames,
                        float* __restrict__ M, float* __restrict__ PT) {
  __shared__ f32x4 rows[2][kD];       // rows[buf][col] = a[4q + 0..3][col]
  __shared__ float cols[4][32][5];    // wave w: a[32 w + row][4q + 0..3], pitch 5
  const size_t m = (size_t)blockIdx.y * frames + blockIdx.x + 1;   // h * frames + t
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const float* src = A + m * kMat;
  f32x16 acc[4];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * w + acc_row(r, lane), col = 32 * T + l32;
      acc[T][r] = src[row * kD + col] + (row == col ? 1.f : 0.f);
    }
#pragma unroll
  for (int q = 0; q < 32; ++q) {
    const int J = q >> 3, s = q & 7;            // tile / band holding K; 4-row group in it
    const int rr = 4 * (s >> 1), hs = s & 1;    // rows 4s..4s+3: registers rr.., half hs
    f32x4* rb = rows[q & 1];
    const int cm = l32 - 4 * s;                 // offset of this lane's column (row) in K
    const bool in_k = cm >= 0 && cm < 4;
    if (w == J && half == hs) {
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        const f32x4 v = {acc[T][rr], acc[T][rr + 1], acc[T][rr + 2], acc[T][rr + 3]};
        rb[32 * T + l32] = v;
      }
    }
    if (in_k) {
#pragma unroll
      for (int r = 0; r < 16; ++r) cols[w][acc_row(r, lane)][cm] = acc[J][r];
    }
    __syncthreads();
    // Pinv, in place: pv[i][j] = a[4q + i][4q + j] = rb[4q + j][i]
    float pv[4][4];
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
      const f32x4 c = rb[4 * q + j2];
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) pv[i2][j2] = c[i2];
    }
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) {
      const float d = 1.f / pv[p2][p2];
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2)
        if (j2 != p2) pv[p2][j2] *= d;
      pv[p2][p2] = d;
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        if (i2 == p2) continue;
        const float f = pv[i2][p2];
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2)
          if (j2 != p2) pv[i2][j2] = fmaf(-f, pv[p2][j2], pv[i2][j2]);
        pv[i2][p2] = -f * d;
      }
    }
    // B operands R[2 h + half][32 T + l32]; the columns of K read as the identity
    float pr[2][4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) pr[h2][i2] = half ? pv[2 * h2 + 1][i2] : pv[2 * h2][i2];
    float rv[4][2];
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      f32x4 raw = rb[32 * T + l32];
      if (T == J && in_k) {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) raw[i2] = cm == i2 ? 1.f : 0.f;
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        rv[T][h2] = pr[h2][0] * raw[0] + pr[h2][1] * raw[1] + pr[h2][2] * raw[2] + pr[h2][3] * raw[3];
    }
    // A operands -C[l32][2 h + half]; the rows of K read as +I
    float cv[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const float c = cols[w][l32][2 * h2 + half];
      cv[h2] = (w == J && in_k) ? (cm == 2 * h2 + half ? 1.f : 0.f) : -c;
    }
    if (in_k) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[J][r] = 0.f;
    }
    if (w == J && half == hs) {
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) acc[T][rr + i2] = 0.f;
    }
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      acc[T] = mfma(cv[0], rv[T][0], acc[T]);
      acc[T] = mfma(cv[1], rv[T][1], acc[T]);
    }
  }
  const float* al = alpha + m * kD;
  float* mo = M + m * kMat;
  float* po = PT + m * kMat;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const float ac = al[32 * T + l32];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * w + acc_row(r, lane), col = 32 * T + l32;
      mo[row * kD + col] = acc[T][r];
      po[row * kD + col] = ac * acc[T][r];
    }
  }
}

// C_t = B_t M_t for the interior frames (b = h * frames + t).  M_t is symmetric,
// so column j of M_t is row j: wave w computes column band w of C_t and holds
// M_t[32 w + l32][64 g .. 64 g + 63] (k = 64 g + i in product i, g the lane
// half) in registers from 16 vector loads; B_t is staged in LDS for the A
// operands of all four row tiles.
__global__ __launch_bounds__(256) void vda_matmul_kernel(const float* __restrict__ X,
                                                         const float* __restrict__ Y, int frames,
                                                         float* __restrict__ out) {
  __shared__ float xs[kD][kPad];
  const size_t b = (size_t)blockIdx.y * frames + blockIdx.x + 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  const float* x = X + b * kMat;
  const f32x4* yrow = (const f32x4*)(Y + b * kMat + (32 * w + l32) * kD + 64 * half);
  f32x4 yv[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) yv[j] = yrow[j];
  for (int i = tid >> 7; i < kD; i += 2) xs[i][tid & (kD - 1)] = x[i * kD + (tid & (kD - 1))];
  __syncthreads();
  float* o = out + b * kMat + 32 * w + l32;
#pragma unroll 1
  for (int I = 0; I < 4; ++I) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int k = 0; k < 64; ++k) acc = mfma(xs[32 * I + l32][64 * half + k], yv[k >> 2][k & 3], acc);
#pragma unroll
    for (int r = 0; r < 16; ++r) o[(32 * I + acc_row(r, lane)) * kD] = acc[r];
  }
}

// The scans: S_t = S_prev P_t + C_t over the interior frames, forward from
// fwd[0] = S_text / 2 and reverse from rev[F] = S_text / 2; every state is
// stored (anchor frames pass the state on unchanged).  Rows of S never mix, so
// a workgroup runs one head, one direction and one 32-row band of the state.
// Wave w owns column tile w: its B operands are rows 32 w.. of P_t^T (64
// consecutive k per lane) and its accumulator starts from C_t's tile, both
// loaded into registers one frame ahead; the band (the A operand) is in LDS.
// Lane half g takes k = 64 g + i in product i.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void vda_scan_kernel(const float* __restrict__ PT, const float* __restrict__ C,
                     const float* __restrict__ s_text, int frames, float* __restrict__ fwd,
                     float* __restrict__ rev) {
  __shared__ float S[32][kPad];
  const int rb = blockIdx.x, h = blockIdx.y, dir = blockIdx.z;   // dir 0 forward, 1 reverse
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, half = lane >> 5;
  float* states = (dir == 0 ? fwd : rev) + (size_t)h * (frames + 1) * kMat;
  const float* st = s_text + (size_t)h * kMat;
  auto frame_of = [&](int step) { return dir == 0 ? step : frames - 1 - step; };
  auto dst_of = [&](int step) { return dir == 0 ? step + 1 : frames - 1 - step; };
  // this lane's elements of its tile: rows 32 rb + acc_row(r), column 32 w + l32
  auto store = [&](int idx, const f32x16& x) {
    float* so = states + (size_t)idx * kMat + 32 * w + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) so[(32 * rb + acc_row(r, lane)) * kD] = x[r];
  };
  f32x16 cur;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * rb + acc_row(r, lane), col = 32 * w + l32;
    cur[r] = 0.5f * st[row * kD + col];
    S[acc_row(r, lane)][col] = cur[r];
  }
  store(dir == 0 ? 0 : frames, cur);
  store(dst_of(0), cur);                       // frame of step 0 is an anchor
  __syncthreads();
  f32x4 pa[16], pb[16];
  f32x16 ca, cb;
  auto load = [&](int t, f32x4 (&pt)[16], f32x16& c) {
    const size_t m = (size_t)h * frames + t;
    const f32x4* src = (const f32x4*)(PT + m * kMat + (32 * w + l32) * kD + 64 * half);
#pragma unroll
    for (int j = 0; j < 16; ++j) pt[j] = src[j];
    const float* cm = C + m * kMat + 32 * w + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) c[r] = cm[(32 * rb + acc_row(r, lane)) * kD];
  };
  auto step = [&](int i, const f32x4 (&pt)[16], const f32x16& c, f32x4 (&pt_next)[16], f32x16& c_next) {
    if (i + 1 <= frames - 2) load(frame_of(i + 1), pt_next, c_next);
    f32x16 acc = c;
#pragma unroll
    for (int k = 0; k < 64; ++k) acc = mfma(S[l32][64 * half + k], pt[k >> 2][k & 3], acc);
    __syncthreads();   // every wave has read the old band
#pragma unroll
    for (int r = 0; r < 16; ++r) S[acc_row(r, lane)][32 * w + l32] = acc[r];
    __syncthreads();
    cur = acc;
    store(dst_of(i), cur);
  };
  if (frames > 2) load(frame_of(1), pa, ca);
  for (int i = 1; i <= frames - 2; i += 2) {
    step(i, pa, ca, pb, cb);
    if (i + 1 <= frames - 2) step(i + 1, pb, cb, pa, ca);
  }
  if (frames > 1) store(dst_of(frames - 1), cur);   // the other anchor
}

// out rows of frame f: o = (fwd[lo] + rev[hi]) q on the bf16 matrix cores.  q is
// bf16 already; W = fwd[lo] + rev[hi] is split into W_hi = bf16(W) and W_lo =
// bf16(W - W_hi), |W - W_hi - W_lo| <= 2^-18 |W|, and o = W_hi q + W_lo q with
// fp32 accumulation.  In the product O = Q W^T both operands are
// row-contiguous: lane l of v_mfma_f32_32x32x16_bf16 takes 8 consecutive head
// dims of query l % 32 (A, from global) and of row l % 32 of W (B, from LDS),
// and each output register of a half-wave is 32 consecutive head dims of one
// query, so every store instruction writes two whole 128-byte segments.  One
// eight-wave workgroup per (frame, head); wave w covers query tiles w, w + 8, ...
constexpr int kWPitch = kD + 8;   // bf16 row pitch of the staged W halves: 16-byte chunks rotate per row

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(512) void vda_readout_kernel(const uint16_t* __restrict__ Q,
                                                          const float* __restrict__ fwd,
                                                          const float* __restrict__ rev, int ft,
                                                          int frames, int chunk, int nb,
                                                          float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) __bf16 w_hi[kD][kWPitch];
  __shared__ __attribute__((aligned(16))) __bf16 w_lo[kD][kWPitch];
  const int f = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
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
  for (int x = tid; x < kMat; x += 512) {
    const int i = x >> 7, j = x & (kD - 1);
    const float wv = wf[x] + wr[x];
    const __bf16 h16 = (__bf16)wv;
    w_hi[i][j] = h16;
    w_lo[i][j] = (__bf16)(wv - (float)h16);
  }
  __syncthreads();
  const size_t N = (size_t)frames * ft;
  const uint16_t* qf = Q + ((size_t)h * N + (size_t)f * ft) * kD;
  float* of = out + ((size_t)h * N + (size_t)f * ft) * kD;
  // ft * 256 < 2^31: the host rejects larger frames
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(qf), (short)0, ft * kD * 2, 0x00020000);
  const int ntiles = (ft + 31) / 32;
  for (int nt = w; nt < ntiles; nt += 8) {
    const int qrow = 32 * nt + l32;
    // A operand: query qrow, dims 16 kt + 8 g + 0..7 (rows past ft read zeros)
    bf16x8 qb[8];
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
      qb[kt] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, qrow * kD * 2 + 32 * kt + 16 * g, 0, 0));
#pragma unroll 1
    for (int mt = 0; mt < 4; ++mt) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        const bf16x8 ah = *(const bf16x8*)&w_hi[32 * mt + l32][16 * kt + 8 * g];
        const bf16x8 al = *(const bf16x8*)&w_lo[32 * mt + l32][16 * kt + 8 * g];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qb[kt], ah, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qb[kt], al, acc, 0, 0, 0);
      }
      // acc[r]: query 32 nt + acc_row(r, lane), head dim 32 mt + l32
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * nt + acc_row(r, lane);
        if (row < ft) of[(size_t)row * kD + 32 * mt + l32] = acc[r];
      }
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
  // frame statistics, inverses and C_t for the interior frames 1..frames-2
  // (the first and last frames are never written into a state)
  if (frames > 2) {
    const dim3 grid(frames - 2, heads);
    hipLaunchKernelGGL(vda_stats_kernel, grid, dim3(256), 0, stream, k, v, beta, ft, frames, A, B);
    hipLaunchKernelGGL(vda_inverse_kernel, grid, dim3(256), 0, stream, A, alpha, frames, M, P);
    hipLaunchKernelGGL(vda_matmul_kernel, grid, dim3(256), 0, stream, B, M, frames, C);
  }
  hipLaunchKernelGGL(vda_scan_kernel, dim3(4, heads, 2), dim3(256), 0, stream, P, C, s_text, frames,
                     fwd, rev);
  return hipGetLastError();
}

hipError_t launch_vda_readout(const uint16_t* q, const float* fwd, const float* rev, int heads,
                              int frames, int ft, int chunk, int nb, float* out, hipStream_t stream) {
  if (heads <= 0 || frames <= 0) return hipSuccess;
  hipLaunchKernelGGL(vda_readout_kernel, dim3(frames, heads), dim3(512), 0, stream, q, fwd, rev, ft,
                     frames, chunk, nb, out);
  return hipGetLastError();
}

}  // namespace fvattn
