// C ABI of the video-token attention library (declared in include/fvattn.h).
//
// Host side only: argument checks (all of them before any HIP call), the
// keep count of compute_topk, stream-ordered scratch for the sparse, INT8,
// window, VSA-H3 and Video Delta Attention paths, and the head-group loop.
// Every step of the computation runs in the kernels of attn_fwd.hip,
// select.hip, quant.hip, window.hip, vsa.hip and vda.hip (probe.hip: the
// matrix-core rate probe used to read the measurements).

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <cstdint>

#include "../../include/fvattn.h"
#include "fvattn_internal.h"

namespace {

using fvattn::kHeadDim;
using fvattn::kTile;

constexpr long long kMaxPerHead = (1LL << 31) - 1;   // elements of one head's tensor
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];        // 0 unknown, 1 gfx950, 2 other

int tiles_of(int tokens) { return tokens == 0 ? 0 : (tokens - 1) / kTile + 1; }

bool keep_frac_ok(double f) { return f > 0.0 && f <= 1.0; }   // false for NaN

bool scale_ok(float s) { return isfinite(s) && s > 0.0f; }

int keep_of(int tiles, double keep_frac) {
  if (tiles == 0) return 0;
  const double want = ceil(keep_frac * (double)tiles);
  if (want >= (double)tiles) return tiles;
  return want < 1.0 ? 1 : (int)want;
}

// Library-owned stream-ordered memory pool of each device (created on first
// use, never destroyed): freed scratch stays in it between calls, and the
// device's default pool, which other code in the process may use, is left
// with its own settings.
std::mutex g_pool_mutex;
hipMemPool_t g_pools[kMaxDevices];

// Scratch of fvattn_forward_sparse_noalloc: one array per GPU, in the code
// object's device memory, for callers that cannot allocate.  Host code never
// uses `scratch` itself (its host-side name is only a stand-in): it uses the
// device address from hipGetSymbolAddress, looked up once per device.
constexpr size_t kStaticScratchBytes = FVATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FVATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FVATTN_ERR_UNSUPPORTED;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    st = g_device_state[dev].load(std::memory_order_acquire);
    if (st != 0) return st == 1 ? FVATTN_OK : FVATTN_ERR_UNSUPPORTED;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return FVATTN_ERR_HIP;
    st = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (st == 1) {
      hipMemPoolProps props;
      memset(&props, 0, sizeof(props));
      props.allocType = hipMemAllocationTypePinned;
      props.handleTypes = hipMemHandleTypeNone;
      props.location.type = hipMemLocationTypeDevice;
      props.location.id = dev;
      hipMemPool_t pool = nullptr;
      if (hipMemPoolCreate(&pool, &props) != hipSuccess) {
        (void)hipGetLastError();
        return FVATTN_ERR_HIP;
      }
      uint64_t threshold = UINT64_MAX;
      (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &threshold);
      g_pools[dev] = pool;
    }
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? FVATTN_OK : FVATTN_ERR_UNSUPPORTED;
}

bool test_fail_alloc() {
  const char* e = getenv("FVATTN_TEST_FAIL_ALLOC");
  return e && e[0] == '1';
}

int hip_status(hipError_t e) { return e == hipSuccess ? FVATTN_OK : FVATTN_ERR_HIP; }

// Stream-ordered scratch from the current device's library pool (the device
// has passed check_device); release with hipFreeAsync on the same stream.
int scratch_malloc(void** p, size_t bytes, hipStream_t stream) {
  *p = nullptr;
  if (test_fail_alloc()) return FVATTN_ERR_ALLOC;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices || !g_pools[dev])
    return FVATTN_ERR_HIP;
  if (hipMallocFromPoolAsync(p, bytes, g_pools[dev], stream) != hipSuccess) {
    (void)hipGetLastError();
    *p = nullptr;
    return FVATTN_ERR_ALLOC;
  }
  return FVATTN_OK;
}

// Scratch of one sparse call: transposed tile means of Q and of K
// [H][128][T], the tile scores [H][T][T], and the kept tile lists [H][T][keep].
struct SparseScratch {
  void* base = nullptr;
  double* qmT = nullptr;
  double* kmT = nullptr;
  double* scores = nullptr;
  int32_t* idx = nullptr;
};

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Bytes of a sparse call's scratch, and its layout over `base`.
size_t sparse_scratch_bytes(int heads, int tiles, int keep, bool need_idx) {
  const size_t means = align256(sizeof(double) * (size_t)heads * tiles * kHeadDim);
  const size_t scoreb = align256(sizeof(double) * (size_t)heads * tiles * tiles);
  const size_t idxb = need_idx ? align256(sizeof(int32_t) * (size_t)heads * tiles * keep) : 0;
  return 2 * means + scoreb + idxb;
}

void sparse_scratch_carve(SparseScratch* s, void* base, int heads, int tiles, bool need_idx) {
  const size_t means = align256(sizeof(double) * (size_t)heads * tiles * kHeadDim);
  const size_t scoreb = align256(sizeof(double) * (size_t)heads * tiles * tiles);
  char* p = (char*)base;
  s->qmT = (double*)p;
  s->kmT = (double*)(p + means);
  s->scores = (double*)(p + 2 * means);
  s->idx = need_idx ? (int32_t*)(p + 2 * means + scoreb) : nullptr;
}

int scratch_alloc(SparseScratch* s, int heads, int tiles, int keep, bool need_idx,
                  hipStream_t stream) {
  const int rc =
      scratch_malloc(&s->base, sparse_scratch_bytes(heads, tiles, keep, need_idx), stream);
  if (rc != FVATTN_OK) return rc;
  sparse_scratch_carve(s, s->base, heads, tiles, need_idx);
  return FVATTN_OK;
}

// Device address of the current device's static scratch array, looked up
// once per device with that device current; nullptr on failure.
void* static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

int scratch_free(SparseScratch* s, hipStream_t stream) {
  if (!s->base) return FVATTN_OK;
  return hip_status(hipFreeAsync(s->base, stream));
}

// Selection into idx (S1-S3) for heads already validated.
int run_selection(const uint16_t* q, const uint16_t* k, int heads, int tokens, int keep,
                  const SparseScratch& s, int32_t* idx, hipStream_t stream) {
  const int T = tiles_of(tokens);
  hipError_t e = fvattn::launch_tile_means_qk(q, k, s.qmT, s.kmT, heads, tokens, stream);
  if (e == hipSuccess) e = fvattn::launch_scores(s.qmT, s.kmT, heads, T, s.scores, stream);
  if (e == hipSuccess) e = fvattn::launch_select(s.scores, heads, T, keep, idx, stream);
  return hip_status(e);
}

// INT8 or FP8 keys of one call: codes [H][N][128] (1 byte each) and block
// scales [H][ceil(N/64)], then the attention with 8-bit scores.
int forward_q8(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int heads,
               int tokens, float scale, bool fp8, hipStream_t stream) {
  const int nblk = (tokens + 63) / 64;
  const size_t codeb = align256((size_t)heads * tokens * kHeadDim);
  const size_t scaleb = align256(sizeof(float) * (size_t)heads * nblk);
  void* base = nullptr;
  const int ra = scratch_malloc(&base, codeb + scaleb, stream);
  if (ra != FVATTN_OK) return ra;
  uint8_t* codes = (uint8_t*)base;
  float* scales = (float*)((char*)base + codeb);
  hipError_t e = fvattn::launch_quantize_k(k, codes, scales, heads, tokens, fp8, stream);
  if (e == hipSuccess) {
    fvattn::ListParams lp;
    lp.kscale = scales;
    e = fp8 ? fvattn::launch_attention_fp8(q, codes, v, out, lp, heads, tokens, scale, stream)
            : fvattn::launch_attention_int8(q, codes, v, out, lp, heads, tokens, scale, stream);
  }
  const int rc = hip_status(e);
  const int rf = hip_status(hipFreeAsync(base, stream));
  return rc != FVATTN_OK ? rc : rf;
}

// Forward for one validated launch of `heads` heads.
int forward_one(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, int heads,
                int tokens, float scale, int mode, double keep_frac, hipStream_t stream) {
  if (mode == FVATTN_DENSE)
    return hip_status(fvattn::launch_attention(q, k, v, out, nullptr, 0, heads, tokens, scale, stream));
  if (mode == FVATTN_DENSE_INT8QK || mode == FVATTN_DENSE_FP8QK)
    return forward_q8(q, k, v, out, heads, tokens, scale, mode == FVATTN_DENSE_FP8QK, stream);
  const int T = tiles_of(tokens);
  const int keep = keep_of(T, keep_frac);
  SparseScratch s;
  int rc = scratch_alloc(&s, heads, T, keep, true, stream);
  if (rc != FVATTN_OK) return rc;
  rc = run_selection(q, k, heads, tokens, keep, s, s.idx, stream);
  if (rc == FVATTN_OK)
    rc = hip_status(fvattn::launch_attention(q, k, v, out, s.idx, keep, heads, tokens, scale, stream));
  const int rf = scratch_free(&s, stream);
  return rc != FVATTN_OK ? rc : rf;
}

// Checks shared by the forward entry points, in the documented order.  Returns
// FVATTN_OK and sets *empty when there is nothing to do.
int check_forward_args(const void* q, const void* k, const void* v, const void* out, int heads,
                       int tokens, int head_dim, float scale, int mode, double keep_frac,
                       bool* empty) {
  *empty = false;
  if (mode != FVATTN_DENSE && mode != FVATTN_BLOCK_SPARSE && mode != FVATTN_DENSE_INT8QK &&
      mode != FVATTN_DENSE_FP8QK)
    return FVATTN_ERR_INVALID_ARG;
  if (heads < 0 || tokens < 0) return FVATTN_ERR_INVALID_ARG;
  if (!scale_ok(scale)) return FVATTN_ERR_INVALID_ARG;
  if (mode == FVATTN_BLOCK_SPARSE && !keep_frac_ok(keep_frac)) return FVATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return FVATTN_ERR_UNSUPPORTED;
  if (heads == 0 || tokens == 0) {
    *empty = true;
    return FVATTN_OK;
  }
  if (!q || !k || !v || !out) return FVATTN_ERR_INVALID_ARG;
  if ((long long)tokens * kHeadDim > kMaxPerHead) return FVATTN_ERR_UNSUPPORTED;
  if (mode == FVATTN_BLOCK_SPARSE && tiles_of(tokens) > FVATTN_MAX_TILES)
    return FVATTN_ERR_UNSUPPORTED;
  return FVATTN_OK;
}

// Checks shared by the VSA-H3 entry points, in the documented order; fills the
// geometry.  Sets *empty when there is nothing to do.
int check_vsa_args(int heads, int tokens, int head_dim, int prefix, int frames, int height,
                   int width, int tt, int th, int tw, double keep_frac, fvattn::VsaGeom* g,
                   bool* empty) {
  *empty = false;
  if (heads < 0 || tokens < 0 || prefix < 0 || frames < 1 || height < 1 || width < 1 || tt < 1 ||
      th < 1 || tw < 1 || !keep_frac_ok(keep_frac))
    return FVATTN_ERR_INVALID_ARG;
  const long long video = (long long)frames * height * width;
  if ((long long)prefix + video != (long long)tokens) return FVATTN_ERR_INVALID_ARG;
  const long long size = (long long)tt * th * tw;
  if (head_dim != kHeadDim || (size != 64 && size != 128 && size != 256))
    return FVATTN_ERR_UNSUPPORTED;
  g->prefix = prefix;
  g->ppad = (prefix + 255) / 256 * 256;
  g->frames = frames;
  g->height = height;
  g->width = width;
  g->tt = tt;
  g->th = th;
  g->tw = tw;
  g->nh = (height + th - 1) / th;
  g->nw = (width + tw - 1) / tw;
  g->size = (int)size;
  const long long tiles = (long long)((frames + tt - 1) / tt) * g->nh * g->nw;
  const long long npad = g->ppad + tiles * size;
  if (tiles > FVATTN_MAX_TILES || npad / 64 > 8192 || npad * kHeadDim > kMaxPerHead)
    return FVATTN_ERR_UNSUPPORTED;
  g->tiles = (int)tiles;
  g->npad = (int)npad;
  g->tokens = tokens;
  if (heads == 0) *empty = true;
  return FVATTN_OK;
}

// Checks shared by the Video Delta Attention entry points.
int check_vda_args(int heads, int frames, int frame_tokens, int head_dim) {
  if (heads < 0 || frames < 0 || frame_tokens < 0) return FVATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return FVATTN_ERR_UNSUPPORTED;
  // one head's tensors below 2^31 elements; a frame's bf16 rows below 2^31
  // bytes (the readout addresses a frame through one buffer descriptor)
  if ((long long)frames * frame_tokens * kHeadDim > kMaxPerHead ||
      (long long)(frames + 1) * kHeadDim * kHeadDim > kMaxPerHead ||
      (long long)frame_tokens * kHeadDim * 2 > kMaxPerHead)
    return FVATTN_ERR_UNSUPPORTED;
  return FVATTN_OK;
}

}  // namespace

extern "C" {

int fvattn_keep_count(int tokens, double keep_frac) {
  if (tokens < 0 || !keep_frac_ok(keep_frac)) return -FVATTN_ERR_INVALID_ARG;
  return keep_of(tiles_of(tokens), keep_frac);
}

int fvattn_forward(const void* q, const void* k, const void* v, void* out, int heads, int tokens,
                   int head_dim, float scale, int mode, double keep_frac, void* stream) {
  bool empty;
  int rc = check_forward_args(q, k, v, out, heads, tokens, head_dim, scale, mode, keep_frac, &empty);
  if (rc != FVATTN_OK || empty) return rc;
  if (mode != FVATTN_DENSE && test_fail_alloc()) return FVATTN_ERR_ALLOC;
  rc = check_device();
  if (rc != FVATTN_OK) return rc;
  return forward_one((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)out,
                     heads, tokens, scale, mode, keep_frac, (hipStream_t)stream);
}

int fvattn_select_tiles(const void* q, const void* k, int heads, int tokens, int head_dim,
                        double keep_frac, int32_t* idx_out, void* stream) {
  if (heads < 0 || tokens < 0 || !keep_frac_ok(keep_frac)) return FVATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return FVATTN_ERR_UNSUPPORTED;
  if (heads == 0 || tokens == 0) return FVATTN_OK;
  if (!q || !k || !idx_out) return FVATTN_ERR_INVALID_ARG;
  if ((long long)tokens * kHeadDim > kMaxPerHead || tiles_of(tokens) > FVATTN_MAX_TILES)
    return FVATTN_ERR_UNSUPPORTED;
  if (test_fail_alloc()) return FVATTN_ERR_ALLOC;
  int rc = check_device();
  if (rc != FVATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int T = tiles_of(tokens);
  const int keep = keep_of(T, keep_frac);
  SparseScratch s;
  rc = scratch_alloc(&s, heads, T, keep, false, st);
  if (rc != FVATTN_OK) return rc;
  rc = run_selection((const uint16_t*)q, (const uint16_t*)k, heads, tokens, keep, s, idx_out, st);
  const int rf = scratch_free(&s, st);
  return rc != FVATTN_OK ? rc : rf;
}

int fvattn_forward_sparse_noalloc(const void* q, const void* k, const void* v, void* out,
                                  int heads, int tokens, int head_dim, float scale,
                                  double keep_frac, void* stream) {
  bool empty;
  int rc = check_forward_args(q, k, v, out, heads, tokens, head_dim, scale, FVATTN_BLOCK_SPARSE,
                              keep_frac, &empty);
  if (rc != FVATTN_OK || empty) return rc;
  const int T = tiles_of(tokens);
  const int keep = keep_of(T, keep_frac);
  if (sparse_scratch_bytes(heads, T, keep, true) > kStaticScratchBytes) return FVATTN_ERR_UNSUPPORTED;
  rc = check_device();
  if (rc != FVATTN_OK) return rc;
  void* base = static_scratch();
  if (!base) return FVATTN_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  SparseScratch s;
  sparse_scratch_carve(&s, base, heads, T, true);
  const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)k;
  rc = run_selection(qq, kk, heads, tokens, keep, s, s.idx, st);
  if (rc != FVATTN_OK) return rc;
  return hip_status(fvattn::launch_attention(qq, kk, (const uint16_t*)v, (uint16_t*)out, s.idx,
                                             keep, heads, tokens, scale, st));
}

int fvattn_forward_indexed(const void* q, const void* k, const void* v, const int32_t* idx,
                           int keep, void* out, int heads, int tokens, int head_dim, float scale,
                           void* stream) {
  if (heads < 0 || tokens < 0 || !scale_ok(scale)) return FVATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return FVATTN_ERR_UNSUPPORTED;
  if (heads == 0 || tokens == 0) return FVATTN_OK;
  if (!q || !k || !v || !idx || !out) return FVATTN_ERR_INVALID_ARG;
  if (keep < 1 || keep > tiles_of(tokens)) return FVATTN_ERR_INVALID_ARG;
  if ((long long)tokens * kHeadDim > kMaxPerHead) return FVATTN_ERR_UNSUPPORTED;
  int rc = check_device();
  if (rc != FVATTN_OK) return rc;
  return hip_status(fvattn::launch_attention((const uint16_t*)q, (const uint16_t*)k,
                                             (const uint16_t*)v, (uint16_t*)out, idx, keep, heads,
                                             tokens, scale, (hipStream_t)stream));
}

int fvattn_forward_heads(const void* q, const void* k, const void* v, void* out, int total_heads,
                         int group_heads, int tokens, int head_dim, float scale, int mode,
                         double keep_frac, void* stream) {
  bool empty;
  int rc = check_forward_args(q, k, v, out, total_heads, tokens, head_dim, scale, mode, keep_frac,
                              &empty);
  if (rc != FVATTN_OK) return rc;
  if (group_heads != 16 && group_heads != 8 && group_heads != 4) return FVATTN_ERR_UNSUPPORTED;
  if (empty) return FVATTN_OK;
  if (mode != FVATTN_DENSE && test_fail_alloc()) return FVATTN_ERR_ALLOC;
  rc = check_device();
  if (rc != FVATTN_OK) return rc;
  const size_t per_head = (size_t)tokens * kHeadDim;
  for (int h0 = 0; h0 < total_heads; h0 += group_heads) {
    const int n = (total_heads - h0 < group_heads) ? total_heads - h0 : group_heads;
    const size_t off = (size_t)h0 * per_head;
    rc = forward_one((const uint16_t*)q + off, (const uint16_t*)k + off, (const uint16_t*)v + off,
                     (uint16_t*)out + off, n, tokens, scale, mode, keep_frac, (hipStream_t)stream);
    if (rc != FVATTN_OK) return rc;
  }
  return FVATTN_OK;
}

// Video frames after a prefix of `prefix` tokens (the last may be partial).
int window_frames(int tokens, int prefix, int frame_tokens) {
  return tokens > prefix ? (tokens - prefix - 1) / frame_tokens + 1 : 0;
}

int fvattn_window_tiles(int tokens, int prefix_tokens, int frame_tokens, int chunk_frames,
                        int neighbours, int32_t* idx_out, int32_t* count_out, void* stream) {
  if (tokens < 0 || chunk_frames < 1 || neighbours < 0 || prefix_tokens < 0 ||
      prefix_tokens > tokens)
    return FVATTN_ERR_INVALID_ARG;
  if (frame_tokens < 64) return FVATTN_ERR_UNSUPPORTED;
  if (tokens == 0) return FVATTN_OK;
  if (!idx_out || !count_out) return FVATTN_ERR_INVALID_ARG;
  if (tiles_of(tokens) > FVATTN_MAX_TILES) return FVATTN_ERR_UNSUPPORTED;
  int rc = check_device();
  if (rc != FVATTN_OK) return rc;
  fvattn::ListParams wp;
  wp.prefix = prefix_tokens;
  wp.frame_tokens = frame_tokens;
  wp.chunk_frames = chunk_frames;
  wp.neighbours = neighbours;
  wp.frames = window_frames(tokens, prefix_tokens, frame_tokens);
  return hip_status(
      fvattn::launch_window_tiles(tokens, wp, kTile, false, idx_out, count_out, (hipStream_t)stream));
}

int fvattn_forward_window(const void* q, const void* k, const void* v, void* out, int heads,
                          int tokens, int head_dim, float scale, int prefix_tokens,
                          int frame_tokens, int chunk_frames, int neighbours, void* stream) {
  if (heads < 0 || tokens < 0 || !scale_ok(scale) || chunk_frames < 1 || neighbours < 0 ||
      prefix_tokens < 0 || prefix_tokens > tokens)
    return FVATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || frame_tokens < 64) return FVATTN_ERR_UNSUPPORTED;
  if (heads == 0 || tokens == 0) return FVATTN_OK;
  if (!q || !k || !v || !out) return FVATTN_ERR_INVALID_ARG;
  if ((long long)tokens * kHeadDim > kMaxPerHead || tiles_of(tokens) > FVATTN_MAX_TILES)
    return FVATTN_ERR_UNSUPPORTED;
  if (test_fail_alloc()) return FVATTN_ERR_ALLOC;
  int rc = check_device();
  if (rc != FVATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int T = tiles_of(tokens);
  const int blocks = (tokens - 1) / fvattn::kWindowRows + 1;
  void* mem = nullptr;
  const size_t idx_bytes = align256(sizeof(int32_t) * (size_t)blocks * T);
  rc = scratch_malloc(&mem, idx_bytes + align256(sizeof(int32_t) * (size_t)blocks), st);
  if (rc != FVATTN_OK) return rc;
  int32_t* idx = (int32_t*)mem;
  int32_t* counts = (int32_t*)((char*)mem + idx_bytes);
  fvattn::ListParams wp;
  wp.counts = counts;
  wp.prefix = prefix_tokens;
  wp.frame_tokens = frame_tokens;
  wp.chunk_frames = chunk_frames;
  wp.neighbours = neighbours;
  wp.frames = window_frames(tokens, prefix_tokens, frame_tokens);
  // the blocks of the last frame (rows that see every key) are walked first
  wp.first_block =
      wp.frames > 0
          ? (int)(((long long)prefix_tokens + (long long)(wp.frames - 1) * frame_tokens) /
                  fvattn::kWindowRows)
          : 0;
  // the layout allocated above: launch_window_tiles writes `blocks` lists of
  // kWindowRows rows, T entries apart; the attention launcher checks it again
  wp.list_rows = fvattn::kWindowRows;
  wp.list_count = blocks;
  wp.list_stride = T;
  hipError_t e = fvattn::launch_window_tiles(tokens, wp, fvattn::kWindowRows, true, idx, counts, st);
  if (e == hipSuccess)
    e = fvattn::launch_attention_window((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                        (uint16_t*)out, idx, wp, heads, tokens, scale, st);
  rc = hip_status(e);
  const int rf = hip_status(hipFreeAsync(mem, st));
  return rc != FVATTN_OK ? rc : rf;
}

int fvattn_tile_means(const void* x, int heads, int tokens, int head_dim, double* means_out,
                      void* stream) {
  if (heads < 0 || tokens < 0) return FVATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return FVATTN_ERR_UNSUPPORTED;
  if (heads == 0 || tokens == 0) return FVATTN_OK;
  if (!x || !means_out) return FVATTN_ERR_INVALID_ARG;
  if ((long long)tokens * kHeadDim > kMaxPerHead) return FVATTN_ERR_UNSUPPORTED;
  int rc = check_device();
  if (rc != FVATTN_OK) return rc;
  return hip_status(fvattn::launch_tile_means((const uint16_t*)x, means_out, heads, tokens,
                                              (hipStream_t)stream));
}

int fvattn_tile_scores(const double* qm, const double* km, int heads, int tiles, int head_dim,
                       double* scores_out, void* stream) {
  if (heads < 0 || tiles < 0) return FVATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return FVATTN_ERR_UNSUPPORTED;
  if (heads == 0 || tiles == 0) return FVATTN_OK;
  if (!qm || !km || !scores_out) return FVATTN_ERR_INVALID_ARG;
  if (tiles > FVATTN_MAX_TILES) return FVATTN_ERR_UNSUPPORTED;
  if (test_fail_alloc()) return FVATTN_ERR_ALLOC;
  int rc = check_device();
  if (rc != FVATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const size_t means = align256(sizeof(double) * (size_t)heads * tiles * kHeadDim);
  void* base = nullptr;
  rc = scratch_malloc(&base, 2 * means, st);
  if (rc != FVATTN_OK) return rc;
  double* qmT = (double*)base;
  double* kmT = (double*)((char*)base + means);
  hipError_t e = fvattn::launch_transpose_means(qm, qmT, heads, tiles, st);
  if (e == hipSuccess) e = fvattn::launch_transpose_means(km, kmT, heads, tiles, st);
  if (e == hipSuccess) e = fvattn::launch_scores(qmT, kmT, heads, tiles, scores_out, st);
  rc = hip_status(e);
  const int rf = hip_status(hipFreeAsync(base, st));
  return rc != FVATTN_OK ? rc : rf;
}

static int quantize_k_entry(const void* k, int heads, int tokens, int head_dim, void* codes_out,
                     float* scales_out, bool fp8, void* stream) {
  if (heads < 0 || tokens < 0) return FVATTN_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return FVATTN_ERR_UNSUPPORTED;
  if (heads == 0 || tokens == 0) return FVATTN_OK;
  if (!k || !codes_out || !scales_out) return FVATTN_ERR_INVALID_ARG;
  if ((long long)tokens * kHeadDim > kMaxPerHead) return FVATTN_ERR_UNSUPPORTED;
  int rc = check_device();
  if (rc != FVATTN_OK) return rc;
  return hip_status(fvattn::launch_quantize_k((const uint16_t*)k, (uint8_t*)codes_out, scales_out,
                                              heads, tokens, fp8, (hipStream_t)stream));
}

int fvattn_quantize_k(const void* k, int heads, int tokens, int head_dim, int8_t* codes_out,
                      float* scales_out, void* stream) {
  return quantize_k_entry(k, heads, tokens, head_dim, codes_out, scales_out, false, stream);
}

int fvattn_quantize_k_fp8(const void* k, int heads, int tokens, int head_dim, uint8_t* codes_out,
                          float* scales_out, void* stream) {
  return quantize_k_entry(k, heads, tokens, head_dim, codes_out, scales_out, true, stream);
}

int fvattn_vda_states(const void* k, const void* v, const float* beta, const float* alpha,
                      const float* s_text, int heads, int frames, int frame_tokens, int head_dim,
                      float* fwd_out, float* rev_out, void* stream) {
  int rc = check_vda_args(heads, frames, frame_tokens, head_dim);
  if (rc != FVATTN_OK) return rc;
  if (heads == 0 || frames == 0) return FVATTN_OK;
  if (frame_tokens == 0) return FVATTN_ERR_INVALID_ARG;
  if (!k || !v || !beta || !alpha || !s_text || !fwd_out || !rev_out) return FVATTN_ERR_INVALID_ARG;
  if (test_fail_alloc()) return FVATTN_ERR_ALLOC;
  rc = check_device();
  if (rc != FVATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  void* mem = nullptr;
  const size_t bytes = sizeof(float) * 5 * (size_t)heads * frames * kHeadDim * kHeadDim;
  rc = scratch_malloc(&mem, bytes, st);
  if (rc != FVATTN_OK) return rc;
  rc = hip_status(fvattn::launch_vda_states((const uint16_t*)k, (const uint16_t*)v, beta, alpha,
                                            s_text, heads, frames, frame_tokens, (float*)mem,
                                            fwd_out, rev_out, st));
  const int rf = hip_status(hipFreeAsync(mem, st));
  return rc != FVATTN_OK ? rc : rf;
}

int fvattn_vda_forward(const void* q, const void* k, const void* v, const float* beta,
                       const float* alpha, const float* s_text, float* out, int heads, int frames,
                       int frame_tokens, int head_dim, int chunk_frames, int neighbours,
                       void* stream) {
  int rc = check_vda_args(heads, frames, frame_tokens, head_dim);
  if (rc != FVATTN_OK) return rc;
  if (chunk_frames < 1 || neighbours < 0) return FVATTN_ERR_INVALID_ARG;
  if (heads == 0 || frames == 0) return FVATTN_OK;
  if (frame_tokens == 0) return FVATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !beta || !alpha || !s_text || !out) return FVATTN_ERR_INVALID_ARG;
  if (test_fail_alloc()) return FVATTN_ERR_ALLOC;
  rc = check_device();
  if (rc != FVATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const size_t mat = (size_t)kHeadDim * kHeadDim;
  const size_t work = 5 * (size_t)heads * frames * mat, states = (size_t)heads * (frames + 1) * mat;
  void* mem = nullptr;
  rc = scratch_malloc(&mem, sizeof(float) * (work + 2 * states), st);
  if (rc != FVATTN_OK) return rc;
  float* w = (float*)mem;
  float* fwd = w + work;
  float* rev = fwd + states;
  hipError_t e = fvattn::launch_vda_states((const uint16_t*)k, (const uint16_t*)v, beta, alpha,
                                           s_text, heads, frames, frame_tokens, w, fwd, rev, st);
  if (e == hipSuccess)
    e = fvattn::launch_vda_readout((const uint16_t*)q, fwd, rev, heads, frames, frame_tokens,
                                   chunk_frames, neighbours, out, st);
  rc = hip_status(e);
  const int rf = hip_status(hipFreeAsync(mem, st));
  return rc != FVATTN_OK ? rc : rf;
}

int fvattn_vsa_tile_count(int frames, int height, int width, int tile_t, int tile_h, int tile_w) {
  if (frames < 1 || height < 1 || width < 1 || tile_t < 1 || tile_h < 1 || tile_w < 1)
    return -FVATTN_ERR_INVALID_ARG;
  const long long t = (long long)((frames + tile_t - 1) / tile_t) * ((height + tile_h - 1) / tile_h) *
                      ((width + tile_w - 1) / tile_w);
  return t > 0x7fffffffLL ? -FVATTN_ERR_UNSUPPORTED : (int)t;
}

int fvattn_vsa_select(const void* q, const void* k, int heads, int tokens, int head_dim,
                      int prefix_tokens, int frames, int height, int width, int tile_t, int tile_h,
                      int tile_w, double keep_frac, int32_t* idx_out, void* stream) {
  fvattn::VsaGeom g;
  bool empty;
  int rc = check_vsa_args(heads, tokens, head_dim, prefix_tokens, frames, height, width, tile_t,
                          tile_h, tile_w, keep_frac, &g, &empty);
  if (rc != FVATTN_OK || empty) return rc;
  if (!q || !k || !idx_out) return FVATTN_ERR_INVALID_ARG;
  if (test_fail_alloc()) return FVATTN_ERR_ALLOC;
  rc = check_device();
  if (rc != FVATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int keep = keep_of(g.tiles, keep_frac);
  const size_t means = align256(sizeof(double) * (size_t)heads * g.tiles * kHeadDim);
  const size_t scoreb = align256(sizeof(double) * (size_t)heads * g.tiles * g.tiles);
  void* base = nullptr;
  rc = scratch_malloc(&base, 2 * means + scoreb, st);
  if (rc != FVATTN_OK) return rc;
  double* qmT = (double*)base;
  double* kmT = (double*)((char*)base + means);
  double* scores = (double*)((char*)base + 2 * means);
  hipError_t e = fvattn::launch_vsa_means((const uint16_t*)q, (const uint16_t*)k, qmT, kmT, g,
                                          heads, st);
  if (e == hipSuccess) e = fvattn::launch_scores(qmT, kmT, heads, g.tiles, scores, st);
  if (e == hipSuccess) e = fvattn::launch_select(scores, heads, g.tiles, keep, idx_out, st);
  rc = hip_status(e);
  const int rf = hip_status(hipFreeAsync(base, st));
  return rc != FVATTN_OK ? rc : rf;
}

int fvattn_forward_vsa(const void* q, const void* k, const void* v, void* out, int heads,
                       int tokens, int head_dim, float scale, int prefix_tokens, int frames,
                       int height, int width, int tile_t, int tile_h, int tile_w, double keep_frac,
                       void* stream) {
  if (!scale_ok(scale)) return FVATTN_ERR_INVALID_ARG;
  fvattn::VsaGeom g;
  bool empty;
  int rc = check_vsa_args(heads, tokens, head_dim, prefix_tokens, frames, height, width, tile_t,
                          tile_h, tile_w, keep_frac, &g, &empty);
  if (rc != FVATTN_OK || empty) return rc;
  if (!q || !k || !v || !out) return FVATTN_ERR_INVALID_ARG;
  if (test_fail_alloc()) return FVATTN_ERR_ALLOC;
  rc = check_device();
  if (rc != FVATTN_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  const int keep = keep_of(g.tiles, keep_frac);
  const int blocks = (g.npad + fvattn::kVsaRows - 1) / fvattn::kVsaRows, nsub = g.npad / 64;
  const size_t packed = align256(sizeof(uint16_t) * (size_t)heads * g.npad * kHeadDim);
  const size_t means = align256(sizeof(double) * (size_t)heads * g.tiles * kHeadDim);
  const size_t idxb = align256(sizeof(int32_t) * (size_t)heads * g.tiles * keep);
  const size_t listb = align256(sizeof(int32_t) * (size_t)heads * blocks * nsub);
  const size_t cntb = align256(sizeof(int32_t) * (size_t)heads * blocks);
  const size_t scoreb = align256(sizeof(double) * (size_t)heads * g.tiles * g.tiles);
  void* base = nullptr;
  rc = scratch_malloc(&base, 2 * packed + 2 * means + idxb + listb + cntb + scoreb, st);
  if (rc != FVATTN_OK) return rc;
  char* p = (char*)base;
  uint16_t* kp = (uint16_t*)p;
  uint16_t* vp = (uint16_t*)(p + packed);
  double* qmT = (double*)(p + 2 * packed);
  double* kmT = (double*)(p + 2 * packed + means);
  int32_t* idx = (int32_t*)(p + 2 * packed + 2 * means);
  int32_t* lists = (int32_t*)(p + 2 * packed + 2 * means + idxb);
  int32_t* counts = (int32_t*)(p + 2 * packed + 2 * means + idxb + listb);
  double* scores = (double*)(p + 2 * packed + 2 * means + idxb + listb + cntb);
  hipError_t e = fvattn::launch_vsa_pack((const uint16_t*)k, (const uint16_t*)v, kp, vp, g, heads, st);
  if (e == hipSuccess)
    e = fvattn::launch_vsa_means((const uint16_t*)q, (const uint16_t*)k, qmT, kmT, g, heads, st);
  if (e == hipSuccess) e = fvattn::launch_scores(qmT, kmT, heads, g.tiles, scores, st);
  if (e == hipSuccess) e = fvattn::launch_select(scores, heads, g.tiles, keep, idx, st);
  if (e == hipSuccess) e = fvattn::launch_vsa_lists(idx, keep, g, heads, lists, counts, st);
  if (e == hipSuccess) {
    fvattn::ListParams lp;
    lp.counts = counts;
    lp.vsa = g;
    e = fvattn::launch_attention_vsa((const uint16_t*)q, kp, vp, (uint16_t*)out, lists, lp, heads,
                                     scale, st);
  }
  rc = hip_status(e);
  const int rf = hip_status(hipFreeAsync(base, st));
  return rc != FVATTN_OK ? rc : rf;
}

int fvattn_mfma_probe(float* sink, int sink_floats, int iters, void* stream) {
  if (!sink || sink_floats < FVATTN_PROBE_SINK || iters < 1) return FVATTN_ERR_INVALID_ARG;
  static_assert(fvattn::kProbeBlocks * 256 == FVATTN_PROBE_SINK, "one float per probe thread");
  int rc = check_device();
  if (rc != FVATTN_OK) return rc;
  return hip_status(fvattn::launch_mfma_probe(sink, iters, (hipStream_t)stream));
}

// Not declared in the public header: the frame-window list-layout check of
// the attention launcher, exposed so host tests can run it without a GPU.
// Returns FVATTN_OK when `list_count` lists of `list_rows` rows, `list_stride`
// entries apart, fit the window attention over `tokens` tokens, else
// FVATTN_ERR_INVALID_ARG.
int fvattn_internal_window_lists_fit(int tokens, int list_rows, int list_count, int list_stride) {
  fvattn::ListParams wp;
  wp.list_rows = list_rows;
  wp.list_count = list_count;
  wp.list_stride = list_stride;
  return fvattn::window_lists_fit(tokens, wp) == hipSuccess ? FVATTN_OK : FVATTN_ERR_INVALID_ARG;
}

const char* fvattn_status_string(int status) {
  switch (status) {
    case FVATTN_OK: return "FVATTN_OK: success";
    case FVATTN_ERR_INVALID_ARG: return "FVATTN_ERR_INVALID_ARG: invalid argument";
    case FVATTN_ERR_UNSUPPORTED: return "FVATTN_ERR_UNSUPPORTED: unsupported shape, size or device";
    case FVATTN_ERR_ALLOC: return "FVATTN_ERR_ALLOC: scratch allocation failed";
    case FVATTN_ERR_HIP: return "FVATTN_ERR_HIP: HIP runtime or launch error";
    default: return "FVATTN: unknown status";
  }
}

}  // extern "C"
