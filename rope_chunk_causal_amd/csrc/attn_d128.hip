// Chunk-causal flash attention, bf16, head_dim 128: the production shape.
//
// [YL] Yuan & Li, "Accelerating Video Generation Inference with
// Sequential-Parallel 3D Positional Encoding Using a Global Time Index",
// Algorithm 3 step 6 with block-causal visibility (§3.2, §3.3); the
// visibility rule and the MFMA formulation are those of attn.hip (S^T = K Q^T
// and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, P^T kept in registers).
//
// What this kernel adds for the bf16 / head_dim-128 shape:
// * One workgroup of 8 waves (256 query rows, two waves per SIMD) per CU, so
//   each K/V tile moves from L2 into LDS once per 256 rows.
// * K and V move global -> LDS with global_load_lds_dwordx4 (no VGPR
//   staging) in 32-key tiles through a ring of four LDS stages: tile t is
//   computed while tiles t+1 and t+2 are in flight and tile t+3 starts into
//   the stage tile t-1 used.  One workgroup barrier per tile; the wait before
//   it counts only the loads of tile t.  (A two-stage ring that waits for the
//   next tile each step leaves the MFMAs idle for much of the L2 latency.)
// * Both tiles stay row-major (256 B per key) with an XOR swizzle of the
//   16-byte chunk index chosen per use, so every LDS read is bank-conflict
//   free: K chunk c of key r sits at c ^ (r % 16) (ds_read_b128 of 16 keys at
//   one chunk), V chunk c at c ^ 4 (r % 4) (ds_read_b64_tr_b16 of 4 keys x 64 B).
// * V^T operands come from ds_read_b64_tr_b16: in each 16-lane group, lane i
//   receives element i%4 of the 8-byte chunk addressed by lane 4e + i/4, so
//   16 lanes that address a 4-key x 16-dim block get that block transposed.
// * Lazy rescaling: a row's reference max moves only when the tile max
//   exceeds it by more than 2^8; P stays <= 256 and the final O / l is exact.
// * Workgroups are renumbered so each XCD (dispatch is round-robin over the
//   8 XCDs) gets a contiguous range of (batch, head, query-tile) work: query
//   tiles of one head run on one XCD and share its L2 for K/V.
#include "rcc_internal.h"

namespace rcc {

namespace {

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;      // query rows per workgroup
constexpr int kBN = 32;               // keys per tile
constexpr int kRowBytes = kD * 2;     // 256 B per key row
constexpr int kTileBytes = kBN * kRowBytes;  // 8 KB
constexpr int kXcds = 8;
constexpr int kStages = 4;            // K/V tiles resident in LDS
constexpr float kLazy = 8.0f;         // log2 headroom before a rescale

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DMA layout of a tile: wave w moves 1 KB = key rows 4 w + (0..3) into LDS
// bytes [w KB, +1 KB); lane -> (row 4 w + lane/16, LDS chunk slot lane%16).
struct Dma {
  uint32_t k, v;      // lane's byte offset inside its key row (swizzled chunk)
};

__device__ __forceinline__ Dma dma_offsets(int64_t rs, int wave, int lane) {
  const int sub = lane >> 4;
  const int cpos = lane & 15;
  const int r = 4 * wave + sub;       // 0..31
  Dma d;
  d.k = (uint32_t)((cpos ^ (r & 15)) << 4);
  d.v = (uint32_t)((cpos ^ (sub << 2)) << 4);
  return d;
}

// Issue this wave's share of one K and one V tile (keys j0 .. j0+31).  Key
// indices are clamped to kv_end - 1: a ragged last tile re-reads the last key
// for rows past kv_end (their scores are masked), and a tile past the end (the
// pipeline always runs three tiles ahead) re-reads it into a stage no step
// reads again.  Branch-free, so the compiler tracks which stage each load
// writes.  Offsets are 32-bit from the (batch, head) base: the host limits a
// batch's cache to 4 GiB.
__device__ __forceinline__ void issue_tile(const __bf16* kg, const __bf16* vg, int64_t rs,
                                           int j0, int kv_end, const Dma& d, char* ks,
                                           char* vs, int wave, int lane) {
  j0 = __builtin_amdgcn_readfirstlane(j0);
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  const int key = min(j0 + 4 * wave + (lane >> 4), kv_end - 1);
  const uint32_t row = (uint32_t)key * row_bytes;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(kg) + (row + d.k),
                                   (lds_void*)(ks + wave * 1024), 16, 0, 0);
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(vg) + (row + d.v),
                                   (lds_void*)(vs + wave * 1024), 16, 0, 0);
}

// Wait until at most n of this wave's DMA instructions are in flight (n is
// 2 per tile: 1 K + 1 V), then a workgroup barrier.  The barrier carries no
// memory fence: a fence would also wait for the later tiles' loads.
template <int n>
__device__ __forceinline__ void tile_ready() {
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Per-wave state carried across key tiles.
struct WaveState {
  f32x16 oacc[4];
  float m_run, l_run;
};

// Per-lane constants of one workgroup.
struct Lane {
  int koff[8];      // K-fragment byte offsets in a tile
  int voff[4];      // V^T-fragment byte offsets in a tile (+ kq*16 rows, +8 rows)
  int g, lim;
};

// One 32-key tile read from stage buffers (ks, vs); later tiles are already
// being loaded into other stages.  Each stage is a distinct __shared__ object,
// so the compiler does not order these LDS reads after the other stages' DMA
// writes.
__device__ __forceinline__ void tile_step(WaveState& w, const Lane& L, const bf16x8 (&qf)[8],
                                          const char* ks, const char* vs, int j0, int lim_lo,
                                          float c2) {
  // S^T = K Q^T, fragment reads kept ahead of the MFMAs that consume them.
  f32x16 s0 = f32x16{};
  bf16x8 ka[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) ka[kk] = *reinterpret_cast<const bf16x8*>(ks + L.koff[kk]);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) s0 = mfma32(ka[kk], qf[kk], s0);

  if (j0 + kBN > lim_lo) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + (r >> 2) * 8 + L.g * 4 + (r & 3);
      s0[r] = key < L.lim ? s0[r] : -INFINITY;
    }
  }

  auto vread = [&](int kq, int dt) {
    const int base = kq * 16 * kRowBytes + L.voff[dt];
    // Whole-vector form: building the operand element by element from the
    // v4i16 variant was mis-packed by the compiler.
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vs + base));
    const bf16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vs + base + 8 * kRowBytes));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  bf16x8 vf[2][4];
#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) vf[kq][dt] = vread(kq, dt);

  float mx = s0[0];
#pragma unroll
  for (int r = 1; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s0[r]), s0[r + 1]);  // v_max3_f32
  mx = fmaxf(mx, s0[15]);
  mx = xhalf_max(mx) * c2;
  // Lazy rescale: move the reference max only when it would grow by > 2^8.
  const float m_use = (mx - w.m_run > kLazy) ? mx : w.m_run;
  if (__ballot(m_use != w.m_run)) {
    const float alpha = __builtin_amdgcn_exp2f(w.m_run - m_use);
    w.l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) w.oacc[dt][r] *= alpha;
    w.m_run = m_use;
  }

  float rsum = 0.f;
  bf16x8 pf[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, -w.m_run));
    rsum += p;
    pf[r >> 3][r & 7] = (__bf16)p;
  }
  w.l_run += xhalf_sum(rsum);

#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.oacc[dt] = mfma32(vf[kq][dt], pf[kq], w.oacc[dt]);
}

template <typename Tout>
__global__ __launch_bounds__(kThreads, 1) void attn_d128_kernel(AttnArgs a, int n_qt) {
  // One object per stage: K tile at +0, V tile at +8 KB.  All stages lie
  // below 64 KB, so every fragment read addresses its stage with the 16-bit
  // immediate offset of ds_read.
  __shared__ __align__(1024) char sS0[2 * kTileBytes];
  __shared__ __align__(1024) char sS1[2 * kTileBytes];
  __shared__ __align__(1024) char sS2[2 * kTileBytes];
  __shared__ __align__(1024) char sS3[2 * kTileBytes];
  char* const sK0 = sS0; char* const sV0 = sS0 + kTileBytes;
  char* const sK1 = sS1; char* const sV1 = sS1 + kTileBytes;
  char* const sK2 = sS2; char* const sV2 = sS2 + kTileBytes;
  char* const sK3 = sS3; char* const sV3 = sS3 + kTileBytes;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // XCD-aware renumbering of the 1-D grid.
  const int total = (int)gridDim.x;
  const int bid = blockIdx.x;
  const int per = (total + kXcds - 1) / kXcds;
  const int rem = total % kXcds;
  const int xcd = bid % kXcds;
  const int id = xcd * per - (rem && xcd > rem ? xcd - rem : 0) + bid / kXcds;
  const int qt = id % n_qt;
  const int bh = id / n_qt;
  const int h = bh % a.n_heads;
  const int b = bh / a.n_heads;

  const int64_t rs = (int64_t)a.n_heads * kD;
  const __bf16* qg = reinterpret_cast<const __bf16*>(a.q) + (int64_t)b * a.q_tokens * rs + h * kD;
  const __bf16* kg = reinterpret_cast<const __bf16*>(a.k) + (int64_t)b * a.cache_tokens * rs + h * kD;
  const __bf16* vg = reinterpret_cast<const __bf16*>(a.v) + (int64_t)b * a.cache_tokens * rs + h * kD;
  Tout* og = reinterpret_cast<Tout*>(a.out) + (int64_t)b * a.q_tokens * rs + h * kD;

  const int q0 = qt * kBM;
  const int qrow = q0 + wave * 32 + l32;
  const int qclamp = qrow < a.q_tokens ? qrow : a.q_tokens - 1;
  const int C = a.chunk_tokens;
  const int qlast = min(q0 + kBM, a.q_tokens) - 1;
  const int lim_lo = min(a.kv_tokens, ((a.q_pos + q0) / C + 1) * C);
  const int kv_end = min(a.kv_tokens, ((a.q_pos + qlast) / C + 1) * C);
  const int n_tiles = (kv_end + kBN - 1) / kBN;

  // Q^T operand fragments (rows past q_tokens read the last row; never stored),
  // loaded before the first K/V tiles so the per-tile waits below count only
  // tile loads.
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(qg + (int64_t)qclamp * rs + kk * 16 + g * 8);

  const Dma dma = dma_offsets(rs, wave, lane);
  issue_tile(kg, vg, rs, 0, kv_end, dma, sK0, sV0, wave, lane);
  issue_tile(kg, vg, rs, kBN, kv_end, dma, sK1, sV1, wave, lane);
  issue_tile(kg, vg, rs, 2 * kBN, kv_end, dma, sK2, sV2, wave, lane);

  Lane L;
  L.g = g;
  L.lim = min(a.kv_tokens, ((a.q_pos + qclamp) / C + 1) * C);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) L.koff[kk] = l32 * kRowBytes + (((kk * 2 + g) ^ (l32 & 15)) << 4);
  {
    const int G = lane >> 4, j = lane & 15;
    const int vrow = (G >> 1) * 4 + (j >> 2);
    const int vsw = (j >> 2) << 2;  // 4 * (row % 4)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int c = dt * 4 + 2 * (G & 1) + ((j & 3) >> 1);
      L.voff[dt] = vrow * kRowBytes + ((c ^ vsw) << 4) + ((j & 1) << 3);
    }
  }

  WaveState w;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) w.oacc[dt] = f32x16{};
  w.m_run = -INFINITY;
  w.l_run = 0.f;
  const float c2 = a.scale_log2;

  // Tile t lives in stage t % 4; tiles t+1 and t+2 are in flight while it is
  // computed, and tile t+3 starts into the stage that tile t-1 used.
  auto step = [&](int t, const char* ks, const char* vs, char* kn, char* vn) {
    tile_ready<4>();
    issue_tile(kg, vg, rs, (t + 3) * kBN, kv_end, dma, kn, vn, wave, lane);
    tile_step(w, L, qf, ks, vs, t * kBN, lim_lo, c2);
  };
  int t = 0;
  for (; t + kStages <= n_tiles; t += kStages) {
    step(t, sK0, sV0, sK3, sV3);
    step(t + 1, sK1, sV1, sK0, sV0);
    step(t + 2, sK2, sV2, sK1, sV1);
    step(t + 3, sK3, sV3, sK2, sV2);
  }
  if (t < n_tiles) step(t, sK0, sV0, sK3, sV3);
  if (t + 1 < n_tiles) step(t + 1, sK1, sV1, sK0, sV0);
  if (t + 2 < n_tiles) step(t + 2, sK2, sV2, sK1, sV1);
  // No load may still be writing this workgroup's LDS when it exits.
  __builtin_amdgcn_s_waitcnt(0);

  if (qrow < a.q_tokens) {
    const float inv = 1.f / w.l_run;
    Tout* orow = og + (int64_t)qrow * rs;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d0 = dt * 32 + jq * 8 + g * 4;
        const float x0 = w.oacc[dt][jq * 4] * inv, x1 = w.oacc[dt][jq * 4 + 1] * inv;
        const float x2 = w.oacc[dt][jq * 4 + 2] * inv, x3 = w.oacc[dt][jq * 4 + 3] * inv;
        if constexpr (sizeof(Tout) == 2) {
          bf16x4 v;
          v[0] = (__bf16)x0; v[1] = (__bf16)x1; v[2] = (__bf16)x2; v[3] = (__bf16)x3;
          *reinterpret_cast<bf16x4*>(orow + d0) = v;
        } else {
          *reinterpret_cast<float4*>(orow + d0) = make_float4(x0, x1, x2, x3);
        }
      }
  }
}

}  // namespace

bool attn_d128_supported(const AttnArgs& a, rcc_dtype in) {
  // K/V loads use 32-bit byte offsets inside one batch entry's cache.
  const int64_t cache_bytes = (int64_t)a.cache_tokens * a.n_heads * kRowBytes;
  return in == RCC_BF16 && a.head_dim == kD && cache_bytes <= (int64_t)UINT32_MAX;
}

hipError_t launch_attn_d128(const AttnArgs& a, rcc_dtype out, hipStream_t s) {
  const int n_qt = (a.q_tokens + kBM - 1) / kBM;
  const int64_t total = (int64_t)n_qt * a.n_heads * a.batch;
  if (out == RCC_BF16)
    hipLaunchKernelGGL((attn_d128_kernel<__bf16>), dim3((uint32_t)total), dim3(kThreads), 0, s, a, n_qt);
  else
    hipLaunchKernelGGL((attn_d128_kernel<float>), dim3((uint32_t)total), dim3(kThreads), 0, s, a, n_qt);
  return hipGetLastError();
}

}  // namespace rcc
