/*
 * rcc.h — C ABI of the Causal-RoPE + chunk-causal attention hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * [YL] C. Yuan, P. Li, "Accelerating Video Generation Inference with
 *      Sequential-Parallel 3D Positional Encoding Using a Global Time
 *      Index" (arXiv 2603.06664).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named *_dev / tensors are DEVICE pointers owned by the caller.
 *   The library allocates no device memory and frees none.
 * - Tensors are contiguous, row-major:
 *     activations  [batch, tokens, n_heads, head_dim]
 *     KV cache     [batch, cache_tokens, n_heads, head_dim]
 *   Tokens of a chunk are flattened in row-major (frame, row, column)
 *   order; cache row r holds the token whose index, counted over all
 *   frames from global frame 0, is r (the *_ring calls use the
 *   rolling-window layout described at rcc_ring instead).
 * - Every tensor pointer must be 16-byte aligned (RCC_ERR_ALIGN).
 * - Arguments are checked on the host before anything is launched; a call
 *   that returns anything but RCC_OK has launched nothing and written
 *   nothing.  Launches are asynchronous on `stream` (0 = the null stream);
 *   a failed launch returns RCC_ERR_HIP.  Sizes whose launch grid would
 *   exceed 2^32 work-items return RCC_ERR_SHAPE without launching.  No call
 *   synchronises the host.
 * - rcc_last_error() returns a human-readable detail of the last non-OK
 *   status returned on the calling thread.
 */
#ifndef RCC_H
#define RCC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define RCC_API __attribute__((visibility("default")))
#else
#define RCC_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RCC_OK = 0,
  RCC_ERR_NULL = 1,   /* a required pointer is NULL                         */
  RCC_ERR_SHAPE = 2,  /* inconsistent or unsupported sizes                  */
  RCC_ERR_RANGE = 3,  /* a position, token range or cache row out of range  */
  RCC_ERR_DTYPE = 4,  /* unknown dtype code                                 */
  RCC_ERR_ALIGN = 5,  /* a tensor pointer is not 16-byte aligned            */
  RCC_ERR_HIP = 6     /* the HIP runtime reported an error                  */
} rcc_status;

typedef enum { RCC_F32 = 0, RCC_BF16 = 1 } rcc_dtype;

/*
 * RoPE band layout.  head_dim = d_t + d_h + d_w; each band dim is even and
 * positive; the bands sit in t, h, w order along head_dim ([YL] §3.3.1:
 * temporal, height and width frequency parts; Algorithm 2 concatenates the
 * three per-axis tables in that order).  Band b, pair j (0 <= j < d_b/2)
 * turns at theta^(-2j/d_b) radians per unit of that axis's coordinate.
 * max_t/max_h/max_w are the table lengths: the largest global frame index,
 * row and column + 1 that any later call may use.
 */
typedef struct {
  int32_t d_t, d_h, d_w;
  double theta;
  int32_t max_t, max_h, max_w;
} rcc_rope3d_cfg;

/*
 * Where a call's tokens sit.  frames/height/width: the chunk's grid
 * (F = tau latent frames, H x W patches); start_frame: s = k * tau for
 * chunk k ([YL] §3.3.2 item 1); token_offset: Delta, the index of the
 * call's first token inside the chunk — r * L_local for sequence-parallel
 * rank r ([YL] §3.3.3, Algorithm 3 step 2).
 */
typedef struct {
  int32_t frames, height, width;
  int32_t start_frame;
  int64_t token_offset;
} rcc_grid;

/*
 * Number of floats of the device table buffer for `cfg`, or -1 if cfg is
 * NULL or invalid (including tables of more than 2^30 floats, 4 GiB).
 * Layout (float2 = {cos, sin}): [max_t][d_t/2] float2, then
 * [max_h][d_h/2] float2, then [max_w][d_w/2].
 */
RCC_API int64_t rcc_rope3d_tables_floats(const rcc_rope3d_cfg* cfg);

/*
 * The cos/sin tables of one band layout: a descriptor that binds the cfg to
 * the device buffer built for it.  The caller owns both the descriptor and
 * the buffer (`data`, at least rcc_rope3d_tables_floats(&cfg) floats, 16-byte
 * aligned); the library allocates nothing.  Only rcc_rope3d_tables_init
 * writes a descriptor: it seals the fields, and every later call checks the
 * seal and rejects (RCC_ERR_SHAPE, nothing launched) a descriptor that was
 * not made by init or whose cfg, data or floats changed since, so a call can
 * never index the buffer with a layout it was not sized for.  The buffer is
 * immutable after rcc_rope3d_tables_build; one descriptor may serve any
 * number of threads and streams.
 */
typedef struct {
  rcc_rope3d_cfg cfg;
  float* data;
  int64_t floats;
  uint64_t seal;
} rcc_rope3d_tables;

/*
 * rope3d_tables_init — host only, launches nothing: check `cfg` and the
 * buffer and write the sealed descriptor `*out`.
 * Errors: NULL (cfg, buf_dev or out); SHAPE (odd or non-positive band dim,
 * non-positive table length, tables of more than 2^30 floats, theta not
 * positive and finite, buf_floats < rcc_rope3d_tables_floats(cfg)); ALIGN
 * (buf_dev not 16-byte aligned).
 * On error *out is zeroed (an unsealed descriptor).
 */
RCC_API rcc_status rcc_rope3d_tables_init(const rcc_rope3d_cfg* cfg, float* buf_dev,
                                          int64_t buf_floats, rcc_rope3d_tables* out);

/*
 * rope3d_tables_build — fill the descriptor's buffer with cos/sin of
 * p * theta_{b,j} for every axis b, position p < max_b and pair j.  Angles
 * and cos/sin are evaluated in fp64 on the device and stored rounded to
 * fp32.  Done once; later calls only read it ([YL] §3.4.1 item 2: cos/sin
 * precomputed into contiguous memory instead of per-call caching;
 * Algorithm 2's `freqs`).
 * Errors: NULL; SHAPE (descriptor not sealed by init, or changed); HIP.
 */
RCC_API rcc_status rcc_rope3d_tables_build(const rcc_rope3d_tables* tables,
                                           hipStream_t stream);

/*
 * rope3d_positions — write int32 [n_tokens][4] = {t_global, h, w,
 * cache_row} for the call's tokens, computed by the same device function
 * the RoPE kernel uses ([YL] §3.3.3 and Algorithm 3 step 3:
 * i_global = Delta + i, t_global = s + floor(i_global / (H*W)); h and w in
 * row-major order; cache_row = s*H*W + i_global).  A check/debug export.
 * Errors: NULL, SHAPE (non-positive grid), RANGE (Delta < 0, Delta + n >
 * F*H*W, a cache row >= 2^31), ALIGN, HIP.
 */
RCC_API rcc_status rcc_rope3d_positions(const rcc_grid* grid, int64_t n_tokens,
                                int32_t* thw_dev, hipStream_t stream);

/*
 * rope3d_apply_append — Causal-RoPE SP on one token range, fused with the
 * KV-cache write ([YL] Algorithm 3 steps 2, 3 and 5; rotation of
 * Algorithm 2 and the §3.3.2 item 2 equation).
 *   q, k, v   [batch, n_tokens, n_heads, D] in `in_dtype`
 *   q_out     [batch, n_tokens, n_heads, D] in `out_dtype`; may equal q
 *             when the dtypes match.
 *   k_cache, v_cache [batch, cache_tokens, n_heads, D] in `out_dtype`.
 * Per token at (t, h, w) and pair j of band b, (x_2j + i x_2j+1) is
 * multiplied by cos + i sin of that band's table at that axis's
 * coordinate (fp32 arithmetic).  q_out gets rotated q; cache rows
 * s*H*W + Delta + [0, n_tokens) get rotated k and the unrotated v
 * (overwriting them); no other cache row is touched.
 * The band layout (D = d_t + d_h + d_w) is the one `tables` was made for.
 * Errors: NULL; DTYPE; SHAPE (tables not sealed by rcc_rope3d_tables_init
 * or changed since, D % 8 != 0, batch outside [1, 65535], n_heads or grid
 * non-positive, n_tokens < 0, n_tokens * n_heads * D / 8 >= 2^31); RANGE
 * (Delta < 0,
 * Delta + n_tokens > F*H*W, s < 0, s + F > max_t, H > max_h, W > max_w,
 * s*H*W + Delta + n_tokens > cache_tokens); ALIGN; HIP.
 */
RCC_API rcc_status rcc_rope3d_apply_append(
    const rcc_rope3d_tables* tables, const rcc_grid* grid,
    rcc_dtype in_dtype, rcc_dtype out_dtype,
    int32_t batch, int64_t n_tokens, int32_t n_heads,
    const void* q, const void* k, const void* v,
    void* q_out, void* k_cache, void* v_cache, int64_t cache_tokens,
    hipStream_t stream);

/*
 * chunk_causal_attn — attention of a query chunk over the KV cache
 * ([YL] Algorithm 3 step 6, with the causal consistency across blocks of
 * §3.2 read as block (chunk) causal visibility).
 *   q        [batch, q_tokens, n_heads, head_dim] in `in_dtype`; query row
 *            i sits at cache position q_pos + i.
 *   k_cache, v_cache [batch, cache_tokens, n_heads, head_dim] in `in_dtype`.
 *   out      [batch, q_tokens, n_heads, head_dim] in `out_dtype`.
 * Key j is visible to query i iff j < kv_tokens and
 * floor(j / chunk_tokens) <= floor((q_pos + i) / chunk_tokens).
 * out = softmax(scale * q k^T over visible keys) v, scale > 0.  Operands are rounded
 * to bf16 (nearest-even) for the matrix cores; accumulation and softmax
 * state are fp32.  With bf16 inputs and head_dim 128, q is multiplied by
 * scale * log2(e) in fp32 before that rounding (the scores then leave the
 * matrix cores in base-2 units, ready for the exponential).
 * Errors: NULL; DTYPE; SHAPE (head_dim not a multiple of 8 in [8, 128],
 * batch/n_heads/chunk_tokens non-positive, q_tokens < 0, scale not positive
 * and finite); RANGE
 * (q_pos < 0, q_pos + q_tokens > kv_tokens, kv_tokens > cache_tokens,
 * sizes >= 2^31); ALIGN; HIP.
 */
RCC_API rcc_status rcc_chunk_causal_attn(
    rcc_dtype in_dtype, rcc_dtype out_dtype,
    int32_t batch, int32_t n_heads, int32_t head_dim,
    int64_t q_tokens, int64_t q_pos, int64_t kv_tokens, int64_t chunk_tokens,
    float scale,
    const void* q, const void* k_cache, const void* v_cache, int64_t cache_tokens,
    void* out, hipStream_t stream);

/*
 * qkv_rope_append — the local QKV projection fused with Causal-RoPE and the
 * KV-cache write ([YL] §3.4.1 item 3: QKV projection and Causal-RoPE in one
 * kernel; Algorithm 3 steps 1-3 and 5).  All tensors bf16 except the bias.
 *   x        [batch, n_tokens, model_dim]: the call's token slice.
 *   w_qkv    [3 * n_heads * D, model_dim], D = d_t + d_h + d_w of the
 *            tables' band layout: the rows of
 *            the q, k and v projections stacked in that order, each group
 *            head-major then head_dim (a fused Linear's weight).
 *   bias     fp32 [3 * n_heads * D], or NULL for none.
 *   q_out    [batch, n_tokens, n_heads, D].
 *   k_cache, v_cache [batch, cache_tokens, n_heads, D].
 * y = x w_qkv^T + bias is accumulated in fp32 from bf16 operands; its q and
 * k parts are rotated in fp32 exactly as rope3d_apply_append rotates them
 * (tables, grid, rows s*H*W + Delta + [0, n_tokens)) and rounded to bf16
 * (nearest-even) once, at the store.  q_out gets rotated q; the cache rows
 * of the slice get rotated k and the unrotated v; nothing else is written.
 * Errors: NULL (bias may be NULL); SHAPE (tables not sealed or changed,
 * D % 32 != 0, model_dim not a positive multiple of 32, batch, n_heads or grid
 * non-positive, n_tokens < 0, x or w_qkv of 4 GiB or more); RANGE (as
 * rope3d_apply_append); ALIGN (16 bytes; bias 4 bytes); HIP.
 */
RCC_API rcc_status rcc_qkv_rope_append(
    const rcc_rope3d_tables* tables, const rcc_grid* grid,
    int32_t batch, int64_t n_tokens, int32_t n_heads, int32_t model_dim,
    const void* x, const void* w_qkv, const float* bias,
    void* q_out, void* k_cache, void* v_cache, int64_t cache_tokens,
    hipStream_t stream);

/*
 * Rolling-window KV cache ([YL] §2.1: Self-Forcing reaches any video length
 * with a KV cache and a rolling window; [SF] = "Sparse Forcing: Native
 * Trainable Sparse Attention for Real-time Autoregressive Diffusion Video
 * Generation", §3.2: a full cache grows without bound, §3.3: a bounded
 * memory of persistent sink blocks plus a local window of the newest
 * blocks, §4.3: sink frames under a fixed KV budget).
 *
 * The cache keeps global frames 0 .. sink_frames-1 for good and the
 * window_frames most recent frames after them, in a ring of
 * (sink_frames + window_frames) * H*W rows per batch entry:
 *   frame slot(t) = t                                        if t < sink_frames
 *                 = sink_frames + (t - sink_frames) mod window_frames   otherwise
 *   token (t, h, w) -> ring row slot(t) * H*W + h*W + w.
 * Keys keep the rotation of their global time index t; nothing is
 * re-rotated when a frame leaves.  sink_frames >= 0; window_frames >= the
 * chunk's frames (a chunk never evicts its own frames).
 *
 * Once chunk [s, s+F) is written the ring holds its sink frames below s+F
 * and the last window_frames frames ending at s+F-1, and these occupy
 * exactly ring rows [0, min(s+F, sink+window) * H*W): the visible memory is
 * always a prefix of the ring, so attention over it needs no gather.
 *
 * block_h, block_w > 0 store each frame block-contiguously ([SF] §3.3
 * blockify, blocks one frame deep): the frame's (H/block_h) x (W/block_w)
 * blocks in row-major order, each block's block_h x block_w tokens in
 * row-major order, so token (h, w) is row slot(t) * H*W + b * block_h *
 * block_w + (h % block_h) * block_w + w % block_w with b = (h / block_h) *
 * (W / block_w) + w / block_w.  Block j of the held memory is then rows
 * [j * block_h * block_w, (j+1) * block_h * block_w): the key blocks of
 * rcc_block_sparse_attn with block_tokens = block_h * block_w.  Both 0
 * (the default) keep the frame row-major.  A window that never wraps
 * (window_frames >= every frame written) gives a blockified plain cache.
 */
typedef struct {
  int32_t sink_frames;
  int32_t window_frames;
  int32_t block_h;
  int32_t block_w;
} rcc_ring;

/*
 * Ring rows the chunk described by `grid` attends once it is written:
 * min(s + F, sink + window) * H*W.  Host-only.  Returns -1 if grid or ring
 * is NULL or invalid (non-positive grid, s < 0, sink < 0,
 * window < F, (sink + window) * H*W >= 2^31, or block dims that are
 * negative, only one of them zero, or not dividing H and W).
 */
RCC_API int64_t rcc_ring_held_tokens(const rcc_grid* grid, const rcc_ring* ring);

/*
 * ring_positions — rcc_rope3d_positions with the ring row in column 3:
 * int32 [n_tokens][4] = {t_global, h, w, ring_row}.  A check/debug export.
 * Errors: as rcc_rope3d_positions, plus NULL ring and SHAPE (sink < 0,
 * window < F, (sink + window) * H*W >= 2^31, invalid block dims).
 */
RCC_API rcc_status rcc_ring_positions(const rcc_grid* grid, const rcc_ring* ring,
                                      int64_t n_tokens, int32_t* thw_dev, hipStream_t stream);

/*
 * rope3d_apply_append_ring — rcc_rope3d_apply_append writing the ring:
 * q and k are rotated at their global (t, h, w) exactly as there; the
 * rotated k and the unrotated v overwrite the ring rows of the slice's
 * tokens (evicting the frames that held those slots).  k_cache and
 * v_cache are [batch, cache_tokens, n_heads, D] with
 * cache_tokens >= (sink + window) * H*W.
 * Errors: as rcc_rope3d_apply_append, with the RANGE rule on cache rows
 * replaced by cache_tokens < (sink + window) * H*W; NULL ring; SHAPE
 * (sink < 0, window < F, ring of 2^31 rows or more, invalid block dims).
 */
RCC_API rcc_status rcc_rope3d_apply_append_ring(
    const rcc_rope3d_tables* tables, const rcc_grid* grid,
    const rcc_ring* ring, rcc_dtype in_dtype, rcc_dtype out_dtype,
    int32_t batch, int64_t n_tokens, int32_t n_heads,
    const void* q, const void* k, const void* v,
    void* q_out, void* k_cache, void* v_cache, int64_t cache_tokens,
    hipStream_t stream);

/*
 * qkv_rope_append_ring — rcc_qkv_rope_append writing the ring rows of the
 * slice (same projection, rotation and rounding).
 * Errors: as rcc_qkv_rope_append, with the ring rules of
 * rcc_rope3d_apply_append_ring.
 */
RCC_API rcc_status rcc_qkv_rope_append_ring(
    const rcc_rope3d_tables* tables, const rcc_grid* grid,
    const rcc_ring* ring, int32_t batch, int64_t n_tokens, int32_t n_heads,
    int32_t model_dim, const void* x, const void* w_qkv, const float* bias,
    void* q_out, void* k_cache, void* v_cache, int64_t cache_tokens,
    hipStream_t stream);

/*
 * chunk_causal_attn_ring — attention of (a slice of) the chunk described
 * by `grid` over the memory the ring holds once that chunk is written
 * ([YL] Algorithm 3 step 6 over [SF] §3.3's bounded memory): every query
 * sees every held row, i.e. ring rows [0, rcc_ring_held_tokens(grid, ring)).
 *   q   [batch, q_tokens, n_heads, head_dim], q_tokens <= F*H*W
 *       (grid->token_offset does not matter here).
 *   k_cache, v_cache [batch, cache_tokens, n_heads, head_dim].
 *   out [batch, q_tokens, n_heads, head_dim].
 * Numerics as rcc_chunk_causal_attn (bf16 matrix-core operands, fp32
 * softmax and accumulation).  The keys are visited in ring order, not in
 * global time order; softmax does not depend on the order.
 * Errors: as rcc_chunk_causal_attn; NULL grid or ring; SHAPE (invalid grid
 * or ring); RANGE (q_tokens > F*H*W, held rows > cache_tokens).
 */
RCC_API rcc_status rcc_chunk_causal_attn_ring(
    const rcc_grid* grid, const rcc_ring* ring, rcc_dtype in_dtype, rcc_dtype out_dtype,
    int32_t batch, int32_t n_heads, int32_t head_dim, int64_t q_tokens, float scale,
    const void* q, const void* k_cache, const void* v_cache, int64_t cache_tokens,
    void* out, hipStream_t stream);

/*
 * block_sparse_attn — attention of each query block over a persistent +
 * local block memory ([SF] §3.3: the memory is the persistent set P, sink
 * blocks plus blocks kept from history, and the local window L, with
 * K = [K_P; K_L]; inside the local window each query block keeps its own
 * Top-K blocks Omega(q); §3.4: one kernel attends every query block to P
 * and to its Omega(q)).  The selection is an input; choosing it (block
 * scores, Top-C, Top-K) is the caller's.
 *   q        bf16 [batch, q_tokens, n_heads, 128], block-contiguous: query
 *            block i is rows [i*B, (i+1)*B) (the last one may be short).
 *   k_cache, v_cache bf16 [batch, cache_tokens, n_heads, 128]: key block j
 *            is rows [j*B, (j+1)*B); blocks j < kv_tokens / B exist.
 *   persist  int32 [batch, n_heads, n_persist] device: key blocks every
 *            query block of that (batch, head) attends.
 *   local    int32 [batch, n_heads, ceil(q_tokens / B), n_local] device:
 *            the key blocks each query block adds.
 *   out      [batch, q_tokens, n_heads, 128] in `out_dtype`.
 * B = block_tokens: 32, 48, 64, 128 or 256 (48 is [SF]'s [3,4,4] block and
 * 64 its [1,8,8]; a block is B consecutive rows whatever its shape).  Query
 * block i attends the union of its two lists:
 * repeated entries count once and entries outside [0, kv_tokens / B)
 * are ignored (-1 pads a list).  out = softmax(scale * q k^T) v over the
 * union's keys, fp32 softmax and accumulation, bf16 matrix-core operands;
 * a query block with an empty union gets zeros.  The order in which keys
 * are visited depends only on the two sets (persistent blocks ascending,
 * then the other local blocks ascending), never on the lists' order or
 * padding, so neither changes a bit of the result.
 * Errors: NULL (a tensor, or a list whose length is non-zero); DTYPE
 * (in_dtype not bf16, unknown out_dtype); SHAPE (head_dim != 128,
 * block_tokens not 32, 48, 64, 128 or 256, batch/n_heads non-positive,
 * q_tokens/kv_tokens/n_persist/n_local negative, n_persist + n_local >
 * 1024, kv_tokens / B > 32768, scale not positive and finite); RANGE
 * (kv_tokens > cache_tokens);
 * ALIGN (tensors 16 bytes, lists 4 bytes); HIP.
 */
RCC_API rcc_status rcc_block_sparse_attn(
    rcc_dtype in_dtype, rcc_dtype out_dtype, int32_t batch, int32_t n_heads, int32_t head_dim,
    int64_t q_tokens, int64_t kv_tokens, int32_t block_tokens, float scale,
    const void* q, const void* k_cache, const void* v_cache, int64_t cache_tokens,
    const int32_t* persist, int32_t n_persist, const int32_t* local, int32_t n_local,
    void* out, hipStream_t stream);

/* Static string naming a status code. */
RCC_API const char* rcc_status_string(rcc_status s);

/* Detail of the last non-OK status on this thread ("" if none). */
RCC_API const char* rcc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RCC_H */
