// C ABI: argument checks, then asynchronous launches on the caller's stream.
// Every check runs before any launch, so a non-OK return has touched no
// memory.  See include/rcc.h for the contract of each entry point.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "rcc_internal.h"

namespace {

thread_local char g_last_error[512] = "";

rcc_status fail(rcc_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

rcc_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return RCC_OK;
  // The launchers' own refusal of a grid beyond 32-bit work-item counts
  // (nothing launched): the sizes are too large for one call.
  if (e == hipErrorInvalidConfiguration)
    return fail(RCC_ERR_SHAPE, "%s: the launch grid would exceed 2^32 work-items", what);
  return fail(RCC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool valid_dtype(rcc_dtype d) { return d == RCC_F32 || d == RCC_BF16; }
constexpr int64_t kI32Max = 2147483647;

int64_t table_floats(const rcc_rope3d_cfg& c) {
  return (int64_t)c.max_t * c.d_t + (int64_t)c.max_h * c.d_h + (int64_t)c.max_w * c.d_w;
}

rcc_status check_cfg(const rcc_rope3d_cfg* c) {
  if (!c) return fail(RCC_ERR_NULL, "cfg is NULL");
  if (c->d_t <= 0 || c->d_h <= 0 || c->d_w <= 0 || (c->d_t | c->d_h | c->d_w) & 1)
    return fail(RCC_ERR_SHAPE, "band dims must be even and positive (got %d/%d/%d)",
                c->d_t, c->d_h, c->d_w);
  if (c->max_t <= 0 || c->max_h <= 0 || c->max_w <= 0)
    return fail(RCC_ERR_SHAPE, "table lengths must be positive");
  if (!(c->theta > 0.0) || !isfinite(c->theta))
    return fail(RCC_ERR_SHAPE, "theta must be positive and finite");
  // Kernels address the tables with 32-bit byte offsets.
  if (table_floats(*c) > (int64_t)1 << 30)
    return fail(RCC_ERR_SHAPE, "tables of %lld floats; at most 2^30 (4 GiB)",
                (long long)table_floats(*c));
  return RCC_OK;
}

// FNV-1a over the descriptor's fields (not its padding bytes): a descriptor
// whose cfg, buffer or length changed after init no longer matches its seal.
uint64_t seal_of(const rcc_rope3d_tables& t) {
  uint64_t h = 0xcbf29ce484222325ull;
  auto mix = [&h](const void* p, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 0x100000001b3ull;
  };
  const rcc_rope3d_cfg& c = t.cfg;
  mix(&c.d_t, 4); mix(&c.d_h, 4); mix(&c.d_w, 4); mix(&c.theta, 8);
  mix(&c.max_t, 4); mix(&c.max_h, 4); mix(&c.max_w, 4);
  const uintptr_t data = (uintptr_t)t.data;
  mix(&data, sizeof(data));
  mix(&t.floats, 8);
  return h ^ 0x52434354424c5345ull;
}

// A descriptor is usable only as rcc_rope3d_tables_init sealed it; its
// buffer then holds the layout of its cfg.
rcc_status check_tables(const rcc_rope3d_tables* t) {
  if (!t) return fail(RCC_ERR_NULL, "tables is NULL");
  if (t->seal != seal_of(*t))
    return fail(RCC_ERR_SHAPE,
                "tables descriptor not made by rcc_rope3d_tables_init, or changed since");
  rcc_status st = check_cfg(&t->cfg);
  if (st != RCC_OK) return st;
  if (!t->data || t->floats < table_floats(t->cfg))
    return fail(RCC_ERR_SHAPE, "tables buffer of %lld floats, the cfg needs %lld",
                (long long)t->floats, (long long)table_floats(t->cfg));
  return RCC_OK;
}

// Grid + token range checks shared by positions and apply_append.
rcc_status check_grid(const rcc_grid* g, int64_t n_tokens, rcc::GridArgs* out) {
  if (!g) return fail(RCC_ERR_NULL, "grid is NULL");
  if (g->frames <= 0 || g->height <= 0 || g->width <= 0)
    return fail(RCC_ERR_SHAPE, "grid dims must be positive");
  const int64_t hw = (int64_t)g->height * g->width;
  const int64_t L = hw * g->frames;
  if (L > kI32Max) return fail(RCC_ERR_SHAPE, "F*H*W must be < 2^31");
  if (n_tokens < 0) return fail(RCC_ERR_SHAPE, "n_tokens < 0");
  if (g->start_frame < 0) return fail(RCC_ERR_RANGE, "start_frame < 0");
  if (g->token_offset < 0 || g->token_offset + n_tokens > L)
    return fail(RCC_ERR_RANGE, "token range [%lld, %lld) outside the chunk of %lld tokens",
                (long long)g->token_offset, (long long)(g->token_offset + n_tokens),
                (long long)L);
  if ((int64_t)g->start_frame * hw + g->token_offset + n_tokens > kI32Max)
    return fail(RCC_ERR_RANGE, "cache rows must be < 2^31");
  out->height = g->height;
  out->width = g->width;
  out->hw = (int32_t)hw;
  out->start_frame = g->start_frame;
  out->token_offset = (int32_t)g->token_offset;
  out->sink = 0;
  out->window = 0;
  out->block_h = 0;
  out->block_w = 0;
  out->blocks_w = 0;
  out->div_hw = rcc::make_fastdiv((uint32_t)hw);
  out->div_w = rcc::make_fastdiv((uint32_t)g->width);
  out->div_window = rcc::make_fastdiv(1);
  out->div_bh = rcc::make_fastdiv(1);
  out->div_bw = rcc::make_fastdiv(1);
  return RCC_OK;
}

// Ring layout checks; on success fills the ring fields of `out` (whose grid
// part check_grid has already validated) and the ring's row count.
rcc_status check_ring(const rcc_grid* g, const rcc_ring* r, rcc::GridArgs* out,
                      int64_t* ring_rows) {
  if (!r) return fail(RCC_ERR_NULL, "ring is NULL");
  if (r->sink_frames < 0) return fail(RCC_ERR_SHAPE, "sink_frames < 0");
  if (r->window_frames < g->frames)
    return fail(RCC_ERR_SHAPE, "window_frames %d is smaller than the chunk's %d frames",
                r->window_frames, g->frames);
  const int64_t rows = ((int64_t)r->sink_frames + r->window_frames) * out->hw;
  if (rows > kI32Max) return fail(RCC_ERR_SHAPE, "ring rows must be < 2^31");
  if (r->block_h || r->block_w) {
    if (r->block_h <= 0 || r->block_w <= 0 || g->height % r->block_h || g->width % r->block_w)
      return fail(RCC_ERR_SHAPE, "blocks %dx%d must be positive and divide the %dx%d frame",
                  r->block_h, r->block_w, g->height, g->width);
    out->block_h = r->block_h;
    out->block_w = r->block_w;
    out->blocks_w = g->width / r->block_w;
    out->div_bh = rcc::make_fastdiv((uint32_t)r->block_h);
    out->div_bw = rcc::make_fastdiv((uint32_t)r->block_w);
  }
  out->sink = r->sink_frames;
  out->window = r->window_frames;
  out->div_window = rcc::make_fastdiv((uint32_t)r->window_frames);
  *ring_rows = rows;
  return RCC_OK;
}

// Rows of the ring held once the chunk is written: min(s + F, sink + window) frames.
int64_t held_rows(const rcc_grid* g, const rcc_ring* r) {
  const int64_t end = (int64_t)g->start_frame + g->frames;
  const int64_t cap = (int64_t)r->sink_frames + r->window_frames;
  return (end < cap ? end : cap) * ((int64_t)g->height * g->width);
}

rcc_status check_tables_cover(const rcc_rope3d_cfg* cfg, const rcc_grid* grid) {
  if ((int64_t)grid->start_frame + grid->frames > cfg->max_t)
    return fail(RCC_ERR_RANGE, "frames [%d, %d) exceed the time table (max_t %d)",
                grid->start_frame, grid->start_frame + grid->frames, cfg->max_t);
  if (grid->height > cfg->max_h || grid->width > cfg->max_w)
    return fail(RCC_ERR_RANGE, "grid %dx%d exceeds the h/w tables (%d, %d)",
                grid->height, grid->width, cfg->max_h, cfg->max_w);
  return RCC_OK;
}

// Cache-row range of a write: the plain cache needs rows up to
// s*H*W + Delta + n; the ring needs (sink + window) * H*W rows.
rcc_status check_cache_rows(const rcc_grid* grid, const rcc::GridArgs& g, int64_t n_tokens,
                            int64_t ring_rows, int64_t cache_tokens) {
  if (g.window > 0) {
    if (ring_rows > cache_tokens)
      return fail(RCC_ERR_RANGE, "the ring needs %lld rows, cache_tokens is %lld",
                  (long long)ring_rows, (long long)cache_tokens);
    return RCC_OK;
  }
  const int64_t last_row = (int64_t)grid->start_frame * g.hw + grid->token_offset + n_tokens;
  if (last_row > cache_tokens)
    return fail(RCC_ERR_RANGE, "cache rows up to %lld exceed cache_tokens %lld",
                (long long)last_row, (long long)cache_tokens);
  return RCC_OK;
}

rcc_status rope_append(const rcc_rope3d_tables* tables, const rcc_grid* grid,
                       const rcc_ring* ring, bool use_ring, rcc_dtype in_dtype,
                       rcc_dtype out_dtype, int32_t batch, int64_t n_tokens, int32_t n_heads,
                       const void* q, const void* k, const void* v, void* q_out,
                       void* k_cache, void* v_cache, int64_t cache_tokens,
                       hipStream_t stream) {
  rcc_status st = check_tables(tables);
  if (st != RCC_OK) return st;
  const rcc_rope3d_cfg* cfg = &tables->cfg;
  const float* tables_dev = tables->data;
  rcc::GridArgs g;
  st = check_grid(grid, n_tokens, &g);
  if (st != RCC_OK) return st;
  int64_t ring_rows = 0;
  if (use_ring && (st = check_ring(grid, ring, &g, &ring_rows)) != RCC_OK) return st;
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(RCC_ERR_DTYPE, "unknown dtype code");
  const int64_t D = (int64_t)cfg->d_t + cfg->d_h + cfg->d_w;
  if (D % 8) return fail(RCC_ERR_SHAPE, "head_dim %lld is not a multiple of 8", (long long)D);
  if (batch <= 0 || batch > 65535) return fail(RCC_ERR_SHAPE, "batch must be in [1, 65535]");
  if (n_heads <= 0) return fail(RCC_ERR_SHAPE, "n_heads must be positive");
  if ((int64_t)n_heads * D > kI32Max || n_tokens * n_heads * (D / 8) > kI32Max)
    return fail(RCC_ERR_SHAPE, "sizes must be < 2^31");
  if ((st = check_tables_cover(cfg, grid)) != RCC_OK) return st;
  if ((st = check_cache_rows(grid, g, n_tokens, ring_rows, cache_tokens)) != RCC_OK) return st;
  if (n_tokens == 0) return RCC_OK;
  if (!q || !k || !v || !q_out || !k_cache || !v_cache)
    return fail(RCC_ERR_NULL, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) ||
      !aligned16(q_out) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(RCC_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
  if (q_out == (const void*)q && in_dtype != out_dtype)
    return fail(RCC_ERR_DTYPE, "in-place q_out needs in_dtype == out_dtype");

  rcc::RopeArgs a;
  a.div_row_chunks = rcc::make_fastdiv((uint32_t)(n_heads * (D / 8)));
  a.div_slots = rcc::make_fastdiv((uint32_t)(D / 8));
  a.tables = tables_dev;
  a.pt = cfg->d_t / 2;
  a.ph = cfg->d_h / 2;
  a.pw = cfg->d_w / 2;
  a.off_h = (int64_t)cfg->max_t * a.pt;
  a.off_w = a.off_h + (int64_t)cfg->max_h * a.ph;
  a.grid = g;
  a.batch = batch;
  a.n_tokens = (int32_t)n_tokens;
  a.n_heads = n_heads;
  a.head_dim = (int32_t)D;
  a.cache_tokens = cache_tokens;
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  return from_hip(rcc::launch_rope3d_apply_append(a, in_dtype, out_dtype, stream),
                  "rope3d_apply_append launch");
}

rcc_status qkv_append(const rcc_rope3d_tables* tables, const rcc_grid* grid,
                      const rcc_ring* ring, bool use_ring, int32_t batch, int64_t n_tokens,
                      int32_t n_heads, int32_t model_dim, const void* x, const void* w_qkv,
                      const float* bias, void* q_out, void* k_cache, void* v_cache,
                      int64_t cache_tokens, hipStream_t stream) {
  rcc_status st = check_tables(tables);
  if (st != RCC_OK) return st;
  const rcc_rope3d_cfg* cfg = &tables->cfg;
  const float* tables_dev = tables->data;
  rcc::GridArgs g;
  st = check_grid(grid, n_tokens, &g);
  if (st != RCC_OK) return st;
  int64_t ring_rows = 0;
  if (use_ring && (st = check_ring(grid, ring, &g, &ring_rows)) != RCC_OK) return st;
  const int64_t D = (int64_t)cfg->d_t + cfg->d_h + cfg->d_w;
  if (D % 32) return fail(RCC_ERR_SHAPE, "head_dim %lld is not a multiple of 32", (long long)D);
  if (batch <= 0 || batch > 65535) return fail(RCC_ERR_SHAPE, "batch must be in [1, 65535]");
  if (n_heads <= 0) return fail(RCC_ERR_SHAPE, "n_heads must be positive");
  if (model_dim <= 0 || model_dim % 32)
    return fail(RCC_ERR_SHAPE, "model_dim must be a positive multiple of 32 (got %d)", model_dim);
  const int64_t n_feat = 3 * (int64_t)n_heads * D;
  const int64_t n_tok = (int64_t)batch * n_tokens;
  if (n_feat > kI32Max || n_tok > kI32Max) return fail(RCC_ERR_SHAPE, "sizes must be < 2^31");
  // Operand loads use 32-bit byte offsets.
  if (n_feat * model_dim * 2 > (int64_t)UINT32_MAX || n_tok * model_dim * 2 > (int64_t)UINT32_MAX)
    return fail(RCC_ERR_SHAPE, "x and w_qkv must each be smaller than 4 GiB");
  if ((st = check_tables_cover(cfg, grid)) != RCC_OK) return st;
  if ((st = check_cache_rows(grid, g, n_tokens, ring_rows, cache_tokens)) != RCC_OK) return st;
  if (n_tokens == 0) return RCC_OK;
  if (!x || !w_qkv || !q_out || !k_cache || !v_cache)
    return fail(RCC_ERR_NULL, "a tensor pointer is NULL");
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q_out) ||
      !aligned16(k_cache) || !aligned16(v_cache) || ((uintptr_t)bias & 3u))
    return fail(RCC_ERR_ALIGN, "tensor pointers must be 16-byte aligned (bias 4-byte)");

  rcc::QkvArgs a;
  a.tables = tables_dev;
  a.pt = cfg->d_t / 2;
  a.ph = cfg->d_h / 2;
  a.pw = cfg->d_w / 2;
  a.off_h = (int64_t)cfg->max_t * a.pt;
  a.off_w = a.off_h + (int64_t)cfg->max_h * a.ph;
  a.grid = g;
  a.batch = batch;
  a.n_tokens = (int32_t)n_tokens;
  a.n_heads = n_heads;
  a.head_dim = (int32_t)D;
  a.model_dim = model_dim;
  a.cache_tokens = cache_tokens;
  a.x = x;
  a.w = w_qkv;
  a.bias = bias;
  a.q_out = q_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  return from_hip(rcc::launch_qkv_rope_append(a, stream), "qkv_rope_append launch");
}

}  // namespace

extern "C" {

const char* rcc_status_string(rcc_status s) {
  switch (s) {
    case RCC_OK: return "RCC_OK";
    case RCC_ERR_NULL: return "RCC_ERR_NULL";
    case RCC_ERR_SHAPE: return "RCC_ERR_SHAPE";
    case RCC_ERR_RANGE: return "RCC_ERR_RANGE";
    case RCC_ERR_DTYPE: return "RCC_ERR_DTYPE";
    case RCC_ERR_ALIGN: return "RCC_ERR_ALIGN";
    case RCC_ERR_HIP: return "RCC_ERR_HIP";
  }
  return "RCC_ERR_UNKNOWN";
}

const char* rcc_last_error(void) { return g_last_error; }

int64_t rcc_rope3d_tables_floats(const rcc_rope3d_cfg* cfg) {
  if (check_cfg(cfg) != RCC_OK) return -1;
  return table_floats(*cfg);
}

rcc_status rcc_rope3d_tables_init(const rcc_rope3d_cfg* cfg, float* buf_dev, int64_t buf_floats,
                                  rcc_rope3d_tables* out) {
  if (!out) return fail(RCC_ERR_NULL, "out is NULL");
  memset(out, 0, sizeof(*out));
  rcc_status st = check_cfg(cfg);
  if (st != RCC_OK) return st;
  if (!buf_dev) return fail(RCC_ERR_NULL, "buf_dev is NULL");
  if (!aligned16(buf_dev)) return fail(RCC_ERR_ALIGN, "buf_dev not 16-byte aligned");
  if (buf_floats < table_floats(*cfg))
    return fail(RCC_ERR_SHAPE, "buffer of %lld floats, the cfg needs %lld",
                (long long)buf_floats, (long long)table_floats(*cfg));
  out->cfg = *cfg;
  out->data = buf_dev;
  out->floats = buf_floats;
  out->seal = seal_of(*out);
  return RCC_OK;
}

rcc_status rcc_rope3d_tables_build(const rcc_rope3d_tables* tables, hipStream_t stream) {
  rcc_status st = check_tables(tables);
  if (st != RCC_OK) return st;
  return from_hip(rcc::launch_rope3d_tables(tables->cfg, tables->data, stream),
                  "rope3d_tables launch");
}

rcc_status rcc_rope3d_positions(const rcc_grid* grid, int64_t n_tokens, int32_t* thw_dev,
                                hipStream_t stream) {
  rcc::GridArgs g;
  rcc_status st = check_grid(grid, n_tokens, &g);
  if (st != RCC_OK) return st;
  if (n_tokens == 0) return RCC_OK;
  if (!thw_dev) return fail(RCC_ERR_NULL, "thw_dev is NULL");
  if (!aligned16(thw_dev)) return fail(RCC_ERR_ALIGN, "thw_dev not 16-byte aligned");
  return from_hip(rcc::launch_rope3d_positions(g, (int32_t)n_tokens, thw_dev, stream),
                  "rope3d_positions launch");
}

rcc_status rcc_ring_positions(const rcc_grid* grid, const rcc_ring* ring, int64_t n_tokens,
                              int32_t* thw_dev, hipStream_t stream) {
  rcc::GridArgs g;
  rcc_status st = check_grid(grid, n_tokens, &g);
  if (st != RCC_OK) return st;
  int64_t ring_rows = 0;
  if ((st = check_ring(grid, ring, &g, &ring_rows)) != RCC_OK) return st;
  if (n_tokens == 0) return RCC_OK;
  if (!thw_dev) return fail(RCC_ERR_NULL, "thw_dev is NULL");
  if (!aligned16(thw_dev)) return fail(RCC_ERR_ALIGN, "thw_dev not 16-byte aligned");
  return from_hip(rcc::launch_rope3d_positions(g, (int32_t)n_tokens, thw_dev, stream),
                  "ring_positions launch");
}

int64_t rcc_ring_held_tokens(const rcc_grid* grid, const rcc_ring* ring) {
  rcc::GridArgs g;
  int64_t ring_rows = 0;
  if (check_grid(grid, 0, &g) != RCC_OK || check_ring(grid, ring, &g, &ring_rows) != RCC_OK)
    return -1;
  return held_rows(grid, ring);
}

rcc_status rcc_rope3d_apply_append(
    const rcc_rope3d_tables* tables, const rcc_grid* grid,
    rcc_dtype in_dtype, rcc_dtype out_dtype,
    int32_t batch, int64_t n_tokens, int32_t n_heads,
    const void* q, const void* k, const void* v,
    void* q_out, void* k_cache, void* v_cache, int64_t cache_tokens,
    hipStream_t stream) {
  return rope_append(tables, grid, nullptr, false, in_dtype, out_dtype, batch,
                     n_tokens, n_heads, q, k, v, q_out, k_cache, v_cache, cache_tokens, stream);
}

rcc_status rcc_rope3d_apply_append_ring(
    const rcc_rope3d_tables* tables, const rcc_grid* grid,
    const rcc_ring* ring, rcc_dtype in_dtype, rcc_dtype out_dtype,
    int32_t batch, int64_t n_tokens, int32_t n_heads,
    const void* q, const void* k, const void* v,
    void* q_out, void* k_cache, void* v_cache, int64_t cache_tokens,
    hipStream_t stream) {
  return rope_append(tables, grid, ring, true, in_dtype, out_dtype, batch,
                     n_tokens, n_heads, q, k, v, q_out, k_cache, v_cache, cache_tokens, stream);
}

rcc_status rcc_qkv_rope_append(
    const rcc_rope3d_tables* tables, const rcc_grid* grid,
    int32_t batch, int64_t n_tokens, int32_t n_heads, int32_t model_dim,
    const void* x, const void* w_qkv, const float* bias,
    void* q_out, void* k_cache, void* v_cache, int64_t cache_tokens,
    hipStream_t stream) {
  return qkv_append(tables, grid, nullptr, false, batch, n_tokens, n_heads, model_dim,
                    x, w_qkv, bias, q_out, k_cache, v_cache, cache_tokens, stream);
}

rcc_status rcc_qkv_rope_append_ring(
    const rcc_rope3d_tables* tables, const rcc_grid* grid,
    const rcc_ring* ring, int32_t batch, int64_t n_tokens, int32_t n_heads,
    int32_t model_dim, const void* x, const void* w_qkv, const float* bias,
    void* q_out, void* k_cache, void* v_cache, int64_t cache_tokens,
    hipStream_t stream) {
  return qkv_append(tables, grid, ring, true, batch, n_tokens, n_heads, model_dim,
                    x, w_qkv, bias, q_out, k_cache, v_cache, cache_tokens, stream);
}

rcc_status rcc_chunk_causal_attn(
    rcc_dtype in_dtype, rcc_dtype out_dtype,
    int32_t batch, int32_t n_heads, int32_t head_dim,
    int64_t q_tokens, int64_t q_pos, int64_t kv_tokens, int64_t chunk_tokens,
    float scale,
    const void* q, const void* k_cache, const void* v_cache, int64_t cache_tokens,
    void* out, hipStream_t stream) {
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(RCC_ERR_DTYPE, "unknown dtype code");
  if (head_dim < 8 || head_dim > 128 || head_dim % 8)
    return fail(RCC_ERR_SHAPE, "head_dim must be a multiple of 8 in [8, 128] (got %d)", head_dim);
  if (batch <= 0 || batch > 65535) return fail(RCC_ERR_SHAPE, "batch must be in [1, 65535]");
  if (n_heads <= 0 || n_heads > 65535) return fail(RCC_ERR_SHAPE, "n_heads must be in [1, 65535]");
  if (chunk_tokens <= 0) return fail(RCC_ERR_SHAPE, "chunk_tokens must be positive");
  if (q_tokens < 0) return fail(RCC_ERR_SHAPE, "q_tokens < 0");
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(RCC_ERR_SHAPE, "scale must be positive and finite");
  if (q_pos < 0 || q_pos + q_tokens > kv_tokens)
    return fail(RCC_ERR_RANGE, "query rows [%lld, %lld) not inside the %lld visible keys",
                (long long)q_pos, (long long)(q_pos + q_tokens), (long long)kv_tokens);
  if (kv_tokens > cache_tokens)
    return fail(RCC_ERR_RANGE, "kv_tokens %lld > cache_tokens %lld", (long long)kv_tokens,
                (long long)cache_tokens);
  if (kv_tokens + chunk_tokens > kI32Max || (int64_t)n_heads * head_dim > kI32Max)
    return fail(RCC_ERR_RANGE, "sizes must be < 2^31");
  if (q_tokens == 0) return RCC_OK;
  if (!q || !k_cache || !v_cache || !out) return fail(RCC_ERR_NULL, "a tensor pointer is NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return fail(RCC_ERR_ALIGN, "tensor pointers must be 16-byte aligned");

  rcc::AttnArgs a;
  a.batch = batch;
  a.n_heads = n_heads;
  a.head_dim = head_dim;
  a.q_tokens = (int32_t)q_tokens;
  a.q_pos = (int32_t)q_pos;
  a.kv_tokens = (int32_t)kv_tokens;
  a.chunk_tokens = (int32_t)chunk_tokens;
  a.cache_tokens = cache_tokens;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  return from_hip(rcc::launch_chunk_causal_attn(a, in_dtype, out_dtype, stream),
                  "chunk_causal_attn launch");
}

rcc_status rcc_chunk_causal_attn_ring(
    const rcc_grid* grid, const rcc_ring* ring, rcc_dtype in_dtype, rcc_dtype out_dtype,
    int32_t batch, int32_t n_heads, int32_t head_dim, int64_t q_tokens, float scale,
    const void* q, const void* k_cache, const void* v_cache, int64_t cache_tokens,
    void* out, hipStream_t stream) {
  rcc::GridArgs g;
  rcc_status st = check_grid(grid, 0, &g);
  if (st != RCC_OK) return st;
  int64_t ring_rows = 0;
  if ((st = check_ring(grid, ring, &g, &ring_rows)) != RCC_OK) return st;
  const int64_t held = held_rows(grid, ring);
  if (q_tokens > (int64_t)grid->frames * g.hw)
    return fail(RCC_ERR_RANGE, "q_tokens %lld exceed the chunk's %lld tokens",
                (long long)q_tokens, (long long)grid->frames * g.hw);
  if (held > cache_tokens)
    return fail(RCC_ERR_RANGE, "the ring holds %lld rows, cache_tokens is %lld",
                (long long)held, (long long)cache_tokens);
  // Every query sees every held row, and the held rows are the ring's
  // prefix [0, held): one key block that all queries share.
  return rcc_chunk_causal_attn(in_dtype, out_dtype, batch, n_heads, head_dim, q_tokens, 0, held,
                               held, scale, q, k_cache, v_cache, cache_tokens, out, stream);
}

rcc_status rcc_block_sparse_attn(
    rcc_dtype in_dtype, rcc_dtype out_dtype, int32_t batch, int32_t n_heads, int32_t head_dim,
    int64_t q_tokens, int64_t kv_tokens, int32_t block_tokens, float scale,
    const void* q, const void* k_cache, const void* v_cache, int64_t cache_tokens,
    const int32_t* persist, int32_t n_persist, const int32_t* local, int32_t n_local,
    void* out, hipStream_t stream) {
  if (in_dtype != RCC_BF16 || !valid_dtype(out_dtype))
    return fail(RCC_ERR_DTYPE, "block-sparse attention takes bf16 inputs");
  if (head_dim != 128) return fail(RCC_ERR_SHAPE, "head_dim must be 128 (got %d)", head_dim);
  if (block_tokens != 32 && block_tokens != 48 && block_tokens != 64 && block_tokens != 128 &&
      block_tokens != 256)
    return fail(RCC_ERR_SHAPE, "block_tokens must be 32, 48, 64, 128 or 256 (got %d)",
                block_tokens);
  if (batch <= 0 || batch > 65535) return fail(RCC_ERR_SHAPE, "batch must be in [1, 65535]");
  if (n_heads <= 0 || n_heads > 65535) return fail(RCC_ERR_SHAPE, "n_heads must be in [1, 65535]");
  if (q_tokens < 0 || kv_tokens < 0 || n_persist < 0 || n_local < 0)
    return fail(RCC_ERR_SHAPE, "negative size");
  if ((int64_t)n_persist + n_local > rcc::block_sparse_max_entries())
    return fail(RCC_ERR_SHAPE, "n_persist + n_local must be at most %d",
                rcc::block_sparse_max_entries());
  if (kv_tokens / block_tokens > 32768)
    return fail(RCC_ERR_SHAPE, "at most 32768 key blocks");
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(RCC_ERR_SHAPE, "scale must be positive and finite");
  if (kv_tokens > cache_tokens)
    return fail(RCC_ERR_RANGE, "kv_tokens %lld > cache_tokens %lld", (long long)kv_tokens,
                (long long)cache_tokens);
  const int64_t n_qb = (q_tokens + block_tokens - 1) / block_tokens;
  if (q_tokens > kI32Max || n_qb * n_heads * batch > kI32Max)
    return fail(RCC_ERR_SHAPE, "sizes must be < 2^31");
  if (q_tokens == 0) return RCC_OK;
  if (!q || !k_cache || !v_cache || !out || (n_persist && !persist) || (n_local && !local))
    return fail(RCC_ERR_NULL, "a tensor or list pointer is NULL");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      ((uintptr_t)persist & 3u) || ((uintptr_t)local & 3u))
    return fail(RCC_ERR_ALIGN, "tensors must be 16-byte aligned, lists 4-byte");

  rcc::SparseArgs a;
  a.batch = batch;
  a.n_heads = n_heads;
  a.q_tokens = (int32_t)q_tokens;
  a.kv_tokens = (int32_t)kv_tokens;
  a.block_tokens = block_tokens;
  a.n_qblocks = (int32_t)n_qb;
  a.n_kblocks = (int32_t)(kv_tokens / block_tokens);
  a.n_persist = n_persist;
  a.n_local = n_local;
  a.cache_tokens = cache_tokens;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.persist = persist;
  a.local = local;
  a.out = out;
  return from_hip(rcc::launch_block_sparse_attn(a, out_dtype, stream), "block_sparse_attn launch");
}

}  // extern "C"
