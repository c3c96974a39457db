/*
 * fvattn.h - C ABI of the MI355X (gfx950) video-token attention library.
 *
 * What is computed
 * ----------------
 * Multi-head softmax attention over the packed video-token sequence of a
 * MiniMax-H3-shaped denoiser: 56 heads of width 128, 1,008 tokens per latent
 * frame (FreeVideo page "FreeVideo: a 66 GB video transformer on an 8 GB
 * card...", section "What MiniMax H3 is, briefly").  The attention is one
 * bidirectional (non-causal) softmax attention (FastH3 page "FastH3 Preview v1:
 * four calls, one-tenth the attention...", section "Lever two: VSA-H3 makes
 * each of the four calls cheaper"), streamed so that the score matrix is never
 * materialized (FreeVideo page, section "Why it does not fit: the
 * arithmetic").
 *
 * Four modes:
 *   FVATTN_DENSE         out = softmax(scale * Q K^T) V over every key.
 *   FVATTN_BLOCK_SPARSE  the sequence is cut into contiguous 128-token tiles;
 *                        tiles are mean-pooled, every query tile scores every
 *                        key tile with the pooled dot product, the top
 *                        k = max(1, min(ceil(keep_frac * T), T)) key tiles are
 *                        kept (compute_topk, FastH3 page, "Lever two"), and
 *                        exact attention runs over the kept tiles only, the
 *                        softmax normalized over the kept keys.
 *   FVATTN_DENSE_INT8QK  FVATTN_DENSE with the scores from INT8 queries and
 *                        keys (FastH3 page, section "Update: consumer GPUs
 *                        and Trim", subsection "Per device"): symmetric codes
 *                        in [-127, 127], scale = max |x| / 127 (1 for a group
 *                        of zeros) per query row and per block of 64
 *                        consecutive keys of a head, code = round-half-to-even
 *                        (x / scale) with a correctly rounded float32 scale
 *                        and division; score = scale * sq * sk * (exact
 *                        integer dot product).  V and P V stay bf16 as in
 *                        FVATTN_DENSE.  Uses stream-ordered scratch for the
 *                        key codes and scales (heads * tokens * 128 bytes).
 *   FVATTN_DENSE_FP8QK   FVATTN_DENSE_INT8QK with 8-bit floating-point codes
 *                        instead (the FP8 reading of the same page passage):
 *                        OCP E4M3 (bias 7, 3 mantissa bits, largest finite
 *                        448), scale = max |x| / 448 (1 for a group of zeros)
 *                        per query row and per block of 64 consecutive keys,
 *                        code = the E4M3 value nearest to x / scale with ties
 *                        to the even mantissa (float32 scale and division,
 *                        correctly rounded); score = scale * sq * sk * (dot
 *                        product of the E4M3 values, fp32 accumulation on the
 *                        f8f6f4 matrix cores).  Scratch as INT8.
 *
 * Selection rule, exactly (the pages leave these points open; this is the
 * library's definition): tile t covers tokens [128t, min(128t+128, N)) and has
 * n_t valid tokens; its mean is an fp64 sum in token order starting from +0.0
 * followed by one correctly rounded fp64 division by n_t; the score of (query
 * tile i, key tile j) is the unscaled fp64 dot product of the two means summed
 * from +0.0 in order d = 0..127 with every product and every sum rounded
 * separately (no fused multiply-add); a query tile keeps the k highest scores,
 * ties going to the lower key-tile index; kept indices are listed ascending.
 *
 * Conventions for every entry point
 * ---------------------------------
 * Layout: q, k, v and out are contiguous bfloat16 arrays [heads][tokens][128]
 *   (head-major), device pointers.  A head group is therefore a contiguous
 *   sub-array.  Index arrays are int32 [heads][T][k], T = ceil(tokens/128),
 *   device pointers, ascending within each row.
 * Ownership: the caller owns every buffer and the stream.  The library never
 *   frees caller memory.  Sparse mode allocates its scratch (tile means, the
 *   fp64 tile score matrix [heads][T][T] and index lists) stream-ordered on
 *   the caller's stream and releases it there.  Scratch comes from a memory
 *   pool the library creates per device on its first call there (release
 *   threshold: keep everything, so repeated calls do not return to the
 *   driver); the pool lives until the process ends and holds at most the
 *   largest scratch that calls overlapping in stream order have needed.  The
 *   device's default memory pool is not touched.
 * Stream: `stream` is a hipStream_t passed as void*; NULL means the default
 *   stream.  Every call only enqueues work and returns; no host
 *   synchronization happens inside.
 * Graph capture: dense-mode fvattn_forward and fvattn_forward_heads,
 *   fvattn_forward_indexed and fvattn_forward_sparse_noalloc allocate nothing
 *   and enqueue only kernels, so a caller can capture them into a HIP graph
 *   and replay it (after one call outside capture, which caches the device
 *   check and, for the last one, the address of its static scratch).  The
 *   other entry points allocate stream-ordered scratch inside the call.
 * Bounds: nothing is read or written past `tokens`; a partial last tile is
 *   masked (its missing keys get -inf scores, its missing query rows are never
 *   stored).
 * Empty input: heads == 0 or tokens == 0 is a valid call that does nothing.
 * Errors: arguments are checked on the host before any HIP call, and a failing
 *   check launches nothing.  No call aborts, throws or prints.  Status codes:
 *     FVATTN_ERR_INVALID_ARG  a NULL pointer, heads < 0, tokens < 0, a scale
 *                             that is not finite and > 0, an unknown mode, a
 *                             keep_frac that is NaN or outside (0, 1] (sparse
 *                             only; ignored in dense mode), keep outside [1, T].
 *     FVATTN_ERR_UNSUPPORTED  head_dim != 128, group_heads not in {16, 8, 4},
 *                             sparse mode with T > FVATTN_MAX_TILES, one
 *                             head's slice of a tensor with 2^31 or more
 *                             elements (tokens > 16,777,215 at head_dim 128;
 *                             larger head counts are fine, heads are
 *                             addressed in 64 bits), or a current device
 *                             that is not gfx950.
 *     FVATTN_ERR_ALLOC        a stream-ordered scratch allocation failed.
 *     FVATTN_ERR_HIP          a HIP call or kernel launch reported an error.
 * Numerics: QK^T and PV run as bf16 matrix-core products with fp32
 *   accumulation; the online softmax keeps an fp32 running max and sum; P is
 *   rounded to bf16 before the PV product and the running sum adds those
 *   bf16 values; out is rounded to bf16.
 */
#ifndef FVATTN_H
#define FVATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FVATTN_OK = 0,
  FVATTN_ERR_INVALID_ARG = 1,
  FVATTN_ERR_UNSUPPORTED = 2,
  FVATTN_ERR_ALLOC = 3,
  FVATTN_ERR_HIP = 4
} fvattn_status;

typedef enum {
  FVATTN_DENSE = 0,
  FVATTN_BLOCK_SPARSE = 1,
  FVATTN_DENSE_INT8QK = 2,
  FVATTN_DENSE_FP8QK = 3
} fvattn_mode;

#define FVATTN_TILE 128       /* tokens per selection tile */
#define FVATTN_HEAD_DIM 128   /* the only supported head width */
#define FVATTN_MAX_TILES 2048 /* sparse mode: at most 2048 tiles (262,144 tokens) */

/* Keep count of compute_topk (FastH3 page, "Lever two"):
 * k = max(1, min(ceil(keep_frac * T), T)) with T = ceil(tokens / 128), the
 * product taken in IEEE double.  tokens == 0 gives 0.  Returns k >= 0, or
 * -FVATTN_ERR_INVALID_ARG for tokens < 0 or keep_frac NaN or outside (0, 1].
 * Pure host arithmetic. */
int fvattn_keep_count(int tokens, double keep_frac);

/* Attention forward for `heads` heads of `tokens` tokens (see the header
 * comment for the three modes).  q, k, v: bf16 [heads][tokens][head_dim] in;
 * out: bf16 [heads][tokens][head_dim] out (every row written).  scale
 * multiplies QK^T (1/sqrt(128) for H3-shaped heads).  keep_frac is used in
 * FVATTN_BLOCK_SPARSE mode only. */
int fvattn_forward(const void* q, const void* k, const void* v, void* out, int heads, int tokens,
                   int head_dim, float scale, int mode, double keep_frac, void* stream);

/* The selection of FVATTN_BLOCK_SPARSE mode alone (the coarse pooled-score
 * stage and compute_topk of FastH3 page, "Lever two").  q, k: bf16
 * [heads][tokens][head_dim] in; idx_out: int32 [heads][T][k] out, with
 * k = fvattn_keep_count(tokens, keep_frac), ascending per row. */
int fvattn_select_tiles(const void* q, const void* k, int heads, int tokens, int head_dim,
                        double keep_frac, int32_t* idx_out, void* stream);

/* FVATTN_BLOCK_SPARSE attention of fvattn_forward (same kernels, same
 * results bit for bit) that allocates nothing, for callers that cannot call
 * hipMalloc: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Its scratch (tile means, tile scores and kept
 * lists) lives in one static device array of FVATTN_NOALLOC_SCRATCH_BYTES per
 * GPU, held until the process ends; the caller passes only inputs and outputs.
 * Limit: 16 H T 128 + 8 H T^2 + 4 H T k bytes (each of the four parts rounded
 * up to 256 bytes; T = ceil(tokens / 128), k the keep count) must fit in the
 * array, else FVATTN_ERR_UNSUPPORTED before anything is enqueued (72,576
 * tokens fit with 16 heads, 102,816 tokens with 8 heads).  Every call on one
 * GPU uses that GPU's one array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.
 * Nothing in the array needs clearing between calls (every byte read is
 * written first by the same call).  Other arguments and errors as
 * fvattn_forward in FVATTN_BLOCK_SPARSE mode. */
#define FVATTN_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
int fvattn_forward_sparse_noalloc(const void* q, const void* k, const void* v, void* out,
                                  int heads, int tokens, int head_dim, float scale,
                                  double keep_frac, void* stream);

/* Sparse attention from caller-given tile lists (the role of
 * block_sparse_attn_from_indices on the FastH3 page, section "What's actually
 * on the GPU: three kernels behind one switch").  idx: int32 [heads][T][keep]
 * in, every entry in [0, T), ascending and distinct within a row (not checked
 * on the device: an out-of-range entry is clamped to T-1 and a repeated one is
 * attended twice).  keep in [1, T]. */
int fvattn_forward_indexed(const void* q, const void* k, const void* v, const int32_t* idx,
                           int keep, void* out, int heads, int tokens, int head_dim, float scale,
                           void* stream);

/* Head-group launcher: runs fvattn_forward on consecutive groups of
 * group_heads heads (16, 8 or 4), the last group taking the remainder (56 in
 * groups of 16 is 16+16+16+8), in order on the one stream.  This mirrors the
 * planner's head grouping (FreeVideo page, section "The rest is placement",
 * item 1; FreeVideo Adaptive Execution Planner page, section "Plan", row
 * "Attention").  Arguments as fvattn_forward with total_heads heads. */
int fvattn_forward_heads(const void* q, const void* k, const void* v, void* out, int total_heads,
                         int group_heads, int tokens, int head_dim, float scale, int mode,
                         double keep_frac, void* stream);

/* Frame-window softmax, the softmax branch of Video DeltaNet (FreeVideo page,
 * section "Where Video DeltaNet comes in"): exact softmax attention over a
 * packed sequence of prefix_tokens non-video tokens (text, audio) followed by
 * the video tokens.  Text and audio tokens keep full softmax attention: a
 * non-video query sees every key and every query sees every non-video key.
 * A video query of latent frame qf sees a video key of latent frame kf only if
 * |qf / chunk_frames - kf / chunk_frames| <= neighbours (integer division;
 * chunks counted from frame 0) or kf or qf is the first or the last frame.
 * Latent frame of video token i = (i - prefix_tokens) / frame_tokens (1,008
 * at 1344x768; chunks of 5 frames with 1 neighbour on each side give the
 * page's 15-frame window); the last frame may be partial.  A sequence whose
 * non-video tokens sit elsewhere (say audio after the video) is a permutation
 * of this layout: the attention is permutation-equivariant, so the caller
 * packs it as [non-video | video].
 * q, k, v, out as in fvattn_forward.  0 <= prefix_tokens <= tokens (else
 * FVATTN_ERR_INVALID_ARG), frame_tokens >= 64 (else FVATTN_ERR_UNSUPPORTED),
 * chunk_frames >= 1, neighbours >= 0.  Uses stream-ordered scratch for the
 * key-tile lists (ceil(tokens/128) * (T + 1) int32). */
int fvattn_forward_window(const void* q, const void* k, const void* v, void* out, int heads,
                          int tokens, int head_dim, float scale, int prefix_tokens,
                          int frame_tokens, int chunk_frames, int neighbours, void* stream);

/* The key-tile lists fvattn_forward_window walks: for each 128-token query
 * tile t, the ascending indices of the key tiles holding at least one key that
 * some query of t may attend to (a tile holding a non-video query lists every
 * tile; a tile holding a non-video key is listed for every query tile).
 * idx_out: int32 [T][T] device, row t holds count_out[t] indices followed by
 * -1; count_out: int32 [T] device. */
int fvattn_window_tiles(int tokens, int prefix_tokens, int frame_tokens, int chunk_frames,
                        int neighbours, int32_t* idx_out, int32_t* count_out, void* stream);

/* VSA-H3 packed-sequence attention (FastH3 page, section "Lever two: VSA-H3
 * makes each of the four calls cheaper").  The sequence is packed as
 * [prefix_tokens non-video tokens (text, condition keyframes, audio) |
 * generated video], the video part a frames x height x width latent grid in
 * (t, h, w) raster order (24 x 42 per latent frame at 1344x768), so tokens =
 * prefix_tokens + frames * height * width.  The video part is cut into
 * tile_t x tile_h x tile_w tiles over that grid ((4, 4, 4) = 64 tokens, the
 * shape FastH3 is trained on, or (4, 8, 8) = 256; the tile size must be 64,
 * 128 or 256), enumerated t-tile slowest, w-tile fastest; tiles at a grid
 * edge the tile does not divide are partial.  Each video query tile keeps the
 * k = max(1, min(ceil(keep_frac * Tv), Tv)) video key tiles of highest pooled
 * score (Tv = number of video tiles; means over each tile's valid tokens,
 * summed in (t, h, w) order; scores, ties and order as in the selection rule
 * above).  A video query attends to every non-video key plus the tokens of
 * its kept tiles; a non-video query attends to every key.  Softmax is exact
 * over the keys a query attends to.
 * q, k, v, out: bf16 [heads][tokens][128] in packed order, device pointers.
 * INVALID_ARG also for tokens != prefix_tokens + frames*height*width, a
 * non-positive grid or tile extent, or keep_frac outside (0, 1];
 * UNSUPPORTED for another tile size or Tv > FVATTN_MAX_TILES.  Uses
 * stream-ordered scratch: K and V in a padded tile layout (2 x heads x npad x
 * 256 B, npad = prefix rounded up to 256 + Tv * tile size), tile means, the
 * fp64 score matrix (heads x Tv x Tv), kept lists and per-block key lists. */
int fvattn_forward_vsa(const void* q, const void* k, const void* v, void* out, int heads,
                       int tokens, int head_dim, float scale, int prefix_tokens, int frames,
                       int height, int width, int tile_t, int tile_h, int tile_w,
                       double keep_frac, void* stream);

/* The selection of fvattn_forward_vsa alone: idx_out int32 [heads][Tv][k]
 * (device), the kept video key tiles of every video query tile, ascending. */
int fvattn_vsa_select(const void* q, const void* k, int heads, int tokens, int head_dim,
                      int prefix_tokens, int frames, int height, int width, int tile_t, int tile_h,
                      int tile_w, double keep_frac, int32_t* idx_out, void* stream);

/* Number of video tiles Tv of a frames x height x width grid cut into
 * tile_t x tile_h x tile_w tiles; -FVATTN_ERR_INVALID_ARG for a non-positive
 * extent.  Pure host arithmetic. */
int fvattn_vsa_tile_count(int frames, int height, int width, int tile_t, int tile_h, int tile_w);

/* The key quantization of FVATTN_DENSE_INT8QK alone, for checking: k bf16
 * [heads][tokens][128] in; codes_out int8 [heads][tokens][128] and
 * scales_out float [heads][ceil(tokens / 64)] out (device pointers). */
int fvattn_quantize_k(const void* k, int heads, int tokens, int head_dim, int8_t* codes_out,
                      float* scales_out, void* stream);

/* The key quantization of FVATTN_DENSE_FP8QK alone, for checking: k bf16
 * [heads][tokens][128] in; codes_out E4M3 bytes [heads][tokens][128] and
 * scales_out float [heads][ceil(tokens / 64)] out (device pointers). */
int fvattn_quantize_k_fp8(const void* k, int heads, int tokens, int head_dim, uint8_t* codes_out,
                          float* scales_out, void* stream);

/* Video Delta Attention, the linear branch of Video DeltaNet (FreeVideo page,
 * section "Where Video DeltaNet comes in"), before its learned gate, norm and
 * projection.  Per head, latent frame t (tokens [t*frame_tokens,
 * (t+1)*frame_tokens)) writes the state S (d_v x d_k = 128 x 128) as
 *   S_t = (S_prev Diag(alpha_t) + B_t)(I + A_t)^-1,
 *   A_t = sum_u beta_u k_u k_u^T, B_t = sum_u beta_u v_u k_u^T,
 * the closed-form minimizer of 1/2||S - S_prev Diag(alpha_t)||^2 +
 * 1/2 sum_u beta_u ||S k_u - v_u||^2.  A forward scan writes frames 1..F-2 in
 * order and a reverse scan F-2..1, both from S_text / 2 (the first and last
 * frames are the softmax anchors and are never written).  A query of frame f,
 * chunk c = f / chunk_frames, reads out = fwd[lo] q + rev[hi] q with
 * lo = clamp((c - neighbours) * chunk_frames, 0, F) and hi = clamp((c +
 * neighbours + 1) * chunk_frames, 0, F) (the frames before and after its
 * softmax window, see fvattn_forward_window); a query of an anchor frame reads
 * fwd[0] q + rev[F] q = S_text q.
 * q, k, v: bf16 [heads][frames * frame_tokens][128]; beta: float
 * [heads][frames * frame_tokens]; alpha: float [heads][frames][128]; s_text:
 * float [heads][128][128] (row = value dim); out: float
 * [heads][frames * frame_tokens][128].  All device pointers.  Products and
 * the inverse run in fp32 (matrix cores, Gauss-Jordan without pivoting on the
 * symmetric I + A_t, eigenvalues >= 1 for beta >= 0).  Uses stream-ordered
 * scratch of (5 * heads * frames + 2 * heads * (frames + 1)) * 64 KiB.
 * PRECONDITION: every beta is finite and >= 0 (the page's write weights).
 * The values live on the device and are not checked: a negative beta can
 * make I + A_t singular or indefinite, where the unpivoted elimination has
 * no guarantee, and a NaN or infinite beta propagates; the output is then
 * undefined (no fault, but no meaningful numbers).  UNSUPPORTED also for
 * frame_tokens > 8,388,607 (one frame's bf16 rows reach 2^31 bytes). */
int fvattn_vda_forward(const void* q, const void* k, const void* v, const float* beta,
                       const float* alpha, const float* s_text, float* out, int heads, int frames,
                       int frame_tokens, int head_dim, int chunk_frames, int neighbours,
                       void* stream);

/* The two scans of fvattn_vda_forward alone: fwd_out, rev_out float
 * [heads][frames + 1][128][128]; fwd[t] has absorbed the written frames
 * before t, rev[t] those from t on; fwd[0] = rev[frames] = s_text / 2.
 * Same PRECONDITION as fvattn_vda_forward: every beta finite and >= 0. */
int fvattn_vda_states(const void* k, const void* v, const float* beta, const float* alpha,
                      const float* s_text, int heads, int frames, int frame_tokens, int head_dim,
                      float* fwd_out, float* rev_out, void* stream);

/* Step S1 alone, for checking: fp64 tile means of x, bf16 [heads][tokens][128]
 * in, means_out fp64 [heads][T][128] out (device pointers). */
int fvattn_tile_means(const void* x, int heads, int tokens, int head_dim, double* means_out,
                      void* stream);

/* Step S2 alone, for checking: fp64 scores [heads][T][T] of the tile means
 * qm, km (fp64 [heads][T][128], device pointers) by the canonical rule. */
int fvattn_tile_scores(const double* qm, const double* km, int heads, int tiles, int head_dim,
                       double* scores_out, void* stream);

/* Matrix-core rate probe, for reading the attention figures against what this
 * GPU sustains at its present clock rather than against the data-sheet peak
 * (2.5 PFLOP/s dense bf16 at 2.4 GHz): 4,096 waves each run `iters`
 * iterations of four independent v_mfma_f32_32x32x16_bf16 chains, no memory
 * traffic, i.e. 4096 * iters * 4 * 32768 FLOP; time the call with events on
 * `stream`.  sink: float device buffer of at least FVATTN_PROBE_SINK floats
 * (one sum per thread, written so the loop cannot be removed).
 * INVALID_ARG for a NULL sink, sink_floats < FVATTN_PROBE_SINK or iters < 1. */
#define FVATTN_PROBE_SINK 262144
int fvattn_mfma_probe(float* sink, int sink_floats, int iters, void* stream);

/* Static description of a status code; never NULL. */
const char* fvattn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FVATTN_H */
