// Chunk-causal flash attention, bf16, head_dim 128: the production shape.
//
// [YL] Yuan & Li, "Accelerating Video Generation Inference with
// Sequential-Parallel 3D Positional Encoding Using a Global Time Index",
// Algorithm 3 step 6 with block-causal visibility (§3.2, §3.3); the
// visibility rule and the MFMA formulation are those of attn.hip (S^T = K Q^T
// and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, P^T kept in registers).
//
// What this kernel adds for the bf16 / head_dim-128 shape:
// * K and V tiles move global -> LDS with global_load_lds_dwordx4 (no VGPR
//   staging), double-buffered: the loads of tile j+1 are in flight while
//   tile j is computed, with one workgroup barrier per tile.
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
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;      // query rows per workgroup
constexpr int kBN = 64;               // keys per tile
constexpr int kRowBytes = kD * 2;     // 256 B per key row
constexpr int kTileBytes = kBN * kRowBytes;  // 16 KB
constexpr int kXcds = 8;
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

// DMA layout of a tile: instruction i (0..3) of wave w moves 1 KB = key rows
// 16 i + 4 w + (0..3) into LDS bytes [(4 i + w) KB, +1 KB); lane -> (row
// 16 i + 4 w + lane/16, LDS chunk slot lane%16).  With this assignment the
// swizzle of every lane is the same for all four instructions, so a lane
// needs one K and one V byte offset; instruction i adds 16 rows.
struct Dma {
  uint32_t k, v;      // lane's byte offset inside the tile for instruction 0
  uint32_t step;      // bytes of 16 key rows
};

__device__ __forceinline__ Dma dma_offsets(int64_t rs, int wave, int lane) {
  const int sub = lane >> 4;
  const int cpos = lane & 15;
  const int r = 4 * wave + sub;       // row of instruction 0; r % 16 == r, r % 4 == sub
  Dma d;
  d.k = (uint32_t)(r * rs * 2 + ((cpos ^ r) << 4));
  d.v = (uint32_t)(r * rs * 2 + ((cpos ^ (sub << 2)) << 4));
  d.step = (uint32_t)(16 * rs * 2);
  return d;
}

// Issue this wave's share of one K tile and one V tile (keys j0 .. j0+63).
// Full tiles use a uniform base pointer plus the per-lane offsets; a ragged
// last tile clamps rows past kv_end to the last key (their scores are masked
// and their P is 0).
__device__ __forceinline__ void issue_tile(const __bf16* kg, const __bf16* vg, int64_t rs,
                                           int j0, int kv_end, const Dma& d, char* ks,
                                           char* vs, int wave, int lane) {
  if (j0 + kBN <= kv_end) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* kb = reinterpret_cast<const char*>(kg + (int64_t)j0 * rs) + i * d.step;
      const char* vb = reinterpret_cast<const char*>(vg + (int64_t)j0 * rs) + i * d.step;
      __builtin_amdgcn_global_load_lds(kb + d.k, (lds_void*)(ks + (4 * i + wave) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vb + d.v, (lds_void*)(vs + (4 * i + wave) * 1024), 16, 0, 0);
    }
    return;
  }
  const int sub = lane >> 4;
  const int cpos = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * i + 4 * wave + sub;
    int key = j0 + r;
    key = key < kv_end ? key : kv_end - 1;
    const int ck = cpos ^ (r & 15);
    const int cv = cpos ^ ((r & 3) << 2);
    __builtin_amdgcn_global_load_lds(kg + (int64_t)key * rs + ck * 8,
                                     (lds_void*)(ks + (4 * i + wave) * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vg + (int64_t)key * rs + cv * 8,
                                     (lds_void*)(vs + (4 * i + wave) * 1024), 16, 0, 0);
  }
}

// Per-wave state carried across key tiles.
struct WaveState {
  f32x16 oacc[4];
  float m_run, l_run;
};

// Per-lane constants of one workgroup.
struct Lane {
  int koff[2][8];   // K-fragment byte offsets in a tile
  int voff[4];      // V^T-fragment byte offsets in a tile (+ kq*16 rows, +8 rows)
  int g, lim;
};

// One key tile read from stage buffers (ks, vs); the tile after it is already
// being loaded into the other stage.  ks/vs are distinct __shared__ objects
// per stage, so the compiler does not order these LDS reads after the other
// stage's DMA writes.
__device__ __forceinline__ void tile_step(WaveState& w, const Lane& L, const bf16x8 (&qf)[8],
                                          const char* ks, const char* vs, int j0, int lim_lo,
                                          float c2) {
  // S^T = K Q^T: the two 32-key blocks interleaved; the schedule below keeps
  // the fragment reads two k-steps ahead of the MFMAs that consume them.
  f32x16 s0 = f32x16{}, s1 = f32x16{};
  bf16x8 ka[8], kb[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    ka[kk] = *reinterpret_cast<const bf16x8*>(ks + L.koff[0][kk]);
    kb[kk] = *reinterpret_cast<const bf16x8*>(ks + L.koff[1][kk]);
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    s0 = mfma32(ka[kk], qf[kk], s0);
    s1 = mfma32(kb[kk], qf[kk], s1);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // DS reads, k-steps 0-1
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); // DS reads, k-step i+2
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0); // MFMAs, k-step i
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // MFMAs, k-steps 6-7

  if (j0 + kBN > lim_lo) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + (r >> 2) * 8 + L.g * 4 + (r & 3);
      s0[r] = key < L.lim ? s0[r] : -INFINITY;
      s1[r] = key + 32 < L.lim ? s1[r] : -INFINITY;
    }
  }

  // V^T fragments of the first 16-key block, read before the softmax math.
  auto vread = [&](int kq, int dt) {
    const int base = kq * 16 * kRowBytes + L.voff[dt];
    // Whole-vector form: building the operand element by element from the
    // v4i16 variant was mis-packed by the compiler.
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vs + base));
    const bf16x4 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vs + base + 8 * kRowBytes));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  bf16x8 vcur[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) vcur[dt] = vread(0, dt);

  float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);  // v_max3_f32
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
  bf16x8 pf[4];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, -w.m_run));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s1[r], c2, -w.m_run));
    rsum += p0 + p1;
    pf[r >> 3][r & 7] = (__bf16)p0;
    pf[2 + (r >> 3)][r & 7] = (__bf16)p1;
  }
  w.l_run += xhalf_sum(rsum);

  // O^T += V^T P^T, next block's V^T fragments read one block ahead.
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    bf16x8 vnext[4];
    if (kq + 1 < 4) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vnext[dt] = vread(kq + 1, dt);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.oacc[dt] = mfma32(vcur[dt], pf[kq], w.oacc[dt]);
    if (kq + 1 < 4) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vcur[dt] = vnext[dt];
    }
  }
}

template <typename Tout>
__global__ __launch_bounds__(kThreads, 2) void attn_d128_kernel(AttnArgs a, int n_qt) {
  __shared__ __align__(1024) char sK0[kTileBytes];
  __shared__ __align__(1024) char sV0[kTileBytes];
  __shared__ __align__(1024) char sK1[kTileBytes];
  __shared__ __align__(1024) char sV1[kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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

  const Dma dma = dma_offsets(rs, wave, lane);
  issue_tile(kg, vg, rs, 0, kv_end, dma, sK0, sV0, wave, lane);

  // Q^T operand fragments (rows past q_tokens read the last row; never stored).
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(qg + (int64_t)qclamp * rs + kk * 16 + g * 8);

  Lane L;
  L.g = g;
  L.lim = min(a.kv_tokens, ((a.q_pos + qclamp) / C + 1) * C);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r = kb * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) L.koff[kb][kk] = r * kRowBytes + (((kk * 2 + g) ^ (r & 15)) << 4);
  }
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

  for (int t = 0; t < n_tiles; t += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < n_tiles) issue_tile(kg, vg, rs, (t + 1) * kBN, kv_end, dma, sK1, sV1, wave, lane);
    tile_step(w, L, qf, sK0, sV0, t * kBN, lim_lo, c2);
    if (t + 1 < n_tiles) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 2 < n_tiles) issue_tile(kg, vg, rs, (t + 2) * kBN, kv_end, dma, sK0, sV0, wave, lane);
      tile_step(w, L, qf, sK1, sV1, (t + 1) * kBN, lim_lo, c2);
    }
  }

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
  return in == RCC_BF16 && a.head_dim == kD;
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
