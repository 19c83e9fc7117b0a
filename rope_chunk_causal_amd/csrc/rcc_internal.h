// Internal declarations shared by the kernel files and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rcc.h"

namespace rcc {

// A one-dimensional dispatch carries groups * threads work-items in 32 bits.
// Launchers refuse larger grids with hipErrorInvalidConfiguration instead of
// letting the cast to the launch's grid size truncate them (which would
// leave outputs unwritten).
inline bool grid_fits(int64_t groups, int threads) {
  return groups * threads <= (int64_t)UINT32_MAX;
}

// Division by a divisor fixed for a launch (Granlund and Montgomery,
// "Division by Invariant Integers using Multiplication", PLDI 1994): with
// l = ceil(log2 d) and m = ceil(2^(32+l) / d) - 2^32, the quotient of any
// n < 2^31 by d is (mulhi(n, m) + n) >> l (the sum stays below 2^32).  The
// host makes it; kernels divide with one multiply-high, an add and a shift.
struct FastDiv {
  uint32_t m, s;
};
inline FastDiv make_fastdiv(uint32_t d) {  // d >= 1
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << (32 + l)) + d - 1) / d;
  return FastDiv{(uint32_t)(m - (1ull << 32)), l};
}
__host__ __device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return ((uint32_t)(((uint64_t)n * f.m) >> 32) + n) >> f.s;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Word 3 of the buffer resources the kernels' LDS-DMA loads go through
// (raw buffers, stride 0): data format 32 bits.  The kernels move K/V and
// GEMM tiles into LDS with buffer_load ... lds rather than global_load_lds:
// the compiler's wait-count model then treats LDS reads as completing in
// order, so a fragment read waits only for itself (lgkmcnt(n)) and not for
// every LDS read in flight.
constexpr int kRawBufferFlags = 0x00020000;

// Position of a call's token inside the video ([YL] §3.3.3).  All values
// fit in 32 bits: the host checks F*H*W < 2^31 and cache rows < 2^31.
// window == 0: the cache keeps every frame in global order.  window > 0:
// a rolling-window ring that keeps frames [0, sink) and the `window` most
// recent frames (Sparse Forcing §3.3's sink blocks plus local window).
struct GridArgs {
  int32_t height, width, hw;  // H, W, H*W
  int32_t start_frame;        // s
  int32_t token_offset;       // Delta
  int32_t sink, window;       // ring layout (window 0 = no ring)
  int32_t block_h, block_w;   // blockified frames (0 = row-major)
  int32_t blocks_w;           // W / block_w
  FastDiv div_hw, div_w;      // by H*W and by W
  FastDiv div_window;         // by window (ring), by block_h and block_w
  FastDiv div_bh, div_bw;     //   (blockified frames); divisor 1 when unused
};

struct TokenPos {
  int32_t t, h, w, row;
};

// i_global = Delta + i; frame in chunk = i_global / HW; t_global = s + frame;
// h, w in row-major order.  Cache row = slot(t_global) * HW + frame row, with
// slot(t) = t for the plain cache (so row = s*HW + i_global) and, for the
// ring, t below the sinks or sink + (t - sink) mod window; the frame row is
// h*W + w, or for blockified frames the block's index times block_h*block_w
// plus the token's row-major index inside its block.
__device__ __forceinline__ TokenPos token_position(const GridArgs& g, int32_t i) {
  const uint32_t ig = (uint32_t)(g.token_offset + i);
  const uint32_t f = fdiv(ig, g.div_hw);
  const uint32_t rem = ig - f * (uint32_t)g.hw;
  const uint32_t h = fdiv(rem, g.div_w);
  TokenPos p;
  p.t = g.start_frame + (int32_t)f;
  p.h = (int32_t)h;
  p.w = (int32_t)(rem - h * (uint32_t)g.width);
  int32_t slot = p.t;
  if (g.window > 0 && p.t >= g.sink) {
    const uint32_t x = (uint32_t)(p.t - g.sink);
    slot = g.sink + (int32_t)(x - fdiv(x, g.div_window) * (uint32_t)g.window);
  }
  uint32_t frow = rem;
  if (g.block_h > 0) {
    const uint32_t hb = fdiv(h, g.div_bh), wb = fdiv((uint32_t)p.w, g.div_bw);
    const uint32_t dh = h - hb * (uint32_t)g.block_h, dw = (uint32_t)p.w - wb * (uint32_t)g.block_w;
    frow = ((hb * (uint32_t)g.blocks_w + wb) * (uint32_t)g.block_h + dh) * (uint32_t)g.block_w + dw;
  }
  p.row = slot * g.hw + (int32_t)frow;
  return p;
}

// Launchers (argument checks are done by the C-ABI layer before these run).
hipError_t launch_rope3d_tables(const rcc_rope3d_cfg& cfg, float* tables, hipStream_t s);
hipError_t launch_rope3d_positions(const GridArgs& g, int32_t n, int32_t* thw, hipStream_t s);

struct RopeArgs {
  FastDiv div_row_chunks, div_slots;  // by n_heads * head_dim / 8 and by head_dim / 8
  const float* tables;
  int32_t pt, ph, pw;         // pairs per band
  int64_t off_h, off_w;       // float2 offsets of the h and w tables
  GridArgs grid;
  int32_t batch, n_tokens, n_heads, head_dim;
  int64_t cache_tokens;
  const void* q;
  const void* k;
  const void* v;
  void* q_out;
  void* k_cache;
  void* v_cache;
};
hipError_t launch_rope3d_apply_append(const RopeArgs& a, rcc_dtype in, rcc_dtype out,
                                      hipStream_t s);

struct QkvArgs {
  const float* tables;
  int32_t pt, ph, pw;         // pairs per band
  int64_t off_h, off_w;       // float2 offsets of the h and w tables
  GridArgs grid;
  int32_t batch, n_tokens, n_heads, head_dim, model_dim;
  int64_t cache_tokens;
  const void* x;              // [batch, n_tokens, model_dim] bf16
  const void* w;              // [3 * n_heads * head_dim, model_dim] bf16
  const float* bias;          // [3 * n_heads * head_dim] or nullptr
  void* q_out;
  void* k_cache;
  void* v_cache;
};
hipError_t launch_qkv_rope_append(const QkvArgs& a, hipStream_t s);

struct AttnArgs {
  int32_t batch, n_heads, head_dim;
  int32_t q_tokens, q_pos, kv_tokens, chunk_tokens;
  int64_t cache_tokens;
  float scale_log2;           // scale * log2(e)
  const void* q;
  const void* k;
  const void* v;
  void* out;
};
hipError_t launch_chunk_causal_attn(const AttnArgs& a, rcc_dtype in, rcc_dtype out,
                                    hipStream_t s);
// bf16, head_dim 128 fast path (attn_d128.hip).
bool attn_d128_supported(const AttnArgs& a, rcc_dtype in);
hipError_t launch_attn_d128(const AttnArgs& a, rcc_dtype out, hipStream_t s);

// Block-sparse attention over a persistent + local block memory
// (attn_sparse.hip; bf16, head_dim 128).
struct SparseArgs {
  int32_t batch, n_heads;
  int32_t q_tokens, kv_tokens, block_tokens;  // block_tokens in {32, 48, 64, 128, 256}
  int32_t n_qblocks, n_kblocks;               // ceil(q_tokens / B), kv_tokens / B
  int32_t n_persist, n_local;                 // list lengths
  int64_t cache_tokens;
  float scale_log2;                           // scale * log2(e)
  const void* q;
  const void* k;
  const void* v;
  const int32_t* persist;                     // [batch, n_heads, n_persist]
  const int32_t* local;                       // [batch, n_heads, n_qblocks, n_local]
  void* out;
};
int block_sparse_max_entries();               // n_persist + n_local limit
hipError_t launch_block_sparse_attn(const SparseArgs& a, rcc_dtype out, hipStream_t s);

}  // namespace rcc
