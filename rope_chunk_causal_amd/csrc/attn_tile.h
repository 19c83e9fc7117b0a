// Per-tile machinery of the bf16 / head_dim-128 attention kernels
// (attn_d128.hip: chunk-causal over a contiguous key range;
// attn_sparse.hip: block-sparse over a list of key blocks).
//
// Formulation: S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16; a
// wave owns 32 query rows, P^T stays in registers, online softmax in base 2
// with lazy rescaling.  K/V tiles are 32 keys x 256 B, row-major in LDS with
// an XOR swizzle of the 16-byte chunk index per use, so every LDS read is
// bank-conflict free: K chunk c of key r sits at c ^ (r % 16) (ds_read_b128
// of 16 keys at one chunk), V chunk c at c ^ 4 (r % 4) (ds_read_b64_tr_b16
// of 4 keys x 64 B).  V^T operands come from ds_read_b64_tr_b16: in each
// 16-lane group, lane i receives element i%4 of the 8-byte chunk addressed by
// lane 4e + i/4, so 16 lanes that address a 4-key x 16-dim block get that
// block transposed.  Softmax bookkeeping (WaveState): a row's reference
// moves only when its scores rise well above it (lazy rescaling), or, in
// the sweeps the kernels run by default, only on the first tile, with the
// row's sum and output certified at the end (row_certified).
#pragma once

#include "rcc_internal.h"

namespace rcc {
namespace attn128 {

constexpr int kD = 128;
constexpr int kBN = 32;                      // keys per tile
constexpr int kRowBytes = kD * 2;            // 256 B per key row
constexpr int kTileBytes = kBN * kRowBytes;  // 8 KB
constexpr int kXcds = 8;
constexpr float kLazy = 8.0f;                // log2 headroom before a rescale (classic)
// Base-2 scheme (scores are base-2 exponents): the reference moves when a
// tile's max exceeds it by more than 48, i.e. a probability passes 2^48; a
// lane's 16 probabilities of a tile are checked through their sum, which
// stays below 2^56 unless one of them passed 2^52.
constexpr float kMoveT = 48.0f;
constexpr float kSumCap = 72057594037927936.0f;  // 2^56

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

// Global byte offset, inside its key row, of the 16-byte chunk that a DMA
// lane moves so that LDS chunk slot `cpos` of tile row r holds the swizzled
// chunk (K: slot c ^ (r % 16); V: slot c ^ 4 (r % 4)).
__device__ __forceinline__ uint32_t k_chunk(int r, int cpos) {
  return (uint32_t)((cpos ^ (r & 15)) << 4);
}
__device__ __forceinline__ uint32_t v_chunk(int r, int cpos) {
  return (uint32_t)((cpos ^ ((r & 3) << 2)) << 4);
}

// Wait until at most n of this wave's DMA instructions are in flight, then a
// workgroup barrier.  The barrier carries no memory fence: a fence would also
// wait for the later tiles' loads.
template <int n>
__device__ __forceinline__ void tile_ready() {
  static_assert(n >= 0 && n < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Per-wave state carried across key tiles.
//
// Two bookkeeping schemes for the scores, chosen per kernel (kBase2):
// * classic: S^T = K Q^T from the bf16 q; a score's probability is
//   exp2(s * c2 - m_run) with c2 = scale * log2(e) (one fma per score); the
//   reference max moves when a tile's max exceeds it by more than 2^8, and
//   l_run is the row's sum.
// * base-2 accumulation: q is pre-multiplied by c2 (load_q<true>) and the
//   S^T accumulation starts from negm = -m_run, so the MFMA results are
//   already s * c2 - m_run and a score's probability is exp2 of it, with
//   no VALU op before the exponential.  It needs 16 more VGPRs (negm).  No
//   tile max is taken in the common case: the reference is set from the
//   first tile that gives the row weight, and afterwards moves only when a
//   lane's probability sum of a tile leaves [0, 2^56] (a probability above
//   2^52, i.e. a score more than 52 above the reference, or a NaN/inf) and
//   the tile max is then more than 48 above it.  Probabilities thus stay
//   below 2^56 (finite in bf16 and in the fp32 sums), and the reference never
//   exceeds the row max, so the row's largest probability is at least 1.  l_run is the lane's half
//   of the row sum (its 16 keys of each tile); finish_rows adds the halves.
//   A sweep may also run its steps past the first unchecked (kChecked
//   false: the first tile's max stays the reference and no test is made)
//   and certify each row at the end (row_certified), falling back to a
//   checked sweep for the rows' workgroup when one fails.
struct WaveState {
  f32x16 oacc[4];
  f32x16 negm;          // -m_run in every element (base-2 scheme only)
  float m_run, l_run;
};

// Per-lane constants.
struct Lane {
  int koff[8];      // K-fragment byte offsets in a tile
  int voff[4];      // V^T-fragment byte offsets in a tile (+ kq*16 rows, +8 rows)
  int g, lim;
};

__device__ __forceinline__ void lane_setup(Lane& L, int lane) {
  const int l32 = lane & 31;
  L.g = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) L.koff[kk] = l32 * kRowBytes + (((kk * 2 + L.g) ^ (l32 & 15)) << 4);
  const int G = lane >> 4, j = lane & 15;
  const int vrow = (G >> 1) * 4 + (j >> 2);
  const int vsw = (j >> 2) << 2;  // 4 * (row % 4)
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int c = dt * 4 + 2 * (G & 1) + ((j & 3) >> 1);
    L.voff[dt] = vrow * kRowBytes + ((c ^ vsw) << 4) + ((j & 1) << 3);
  }
}

template <bool kBase2>
__device__ __forceinline__ void wave_init(WaveState& w) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) w.oacc[dt] = f32x16{};
  w.negm = f32x16{};
  // The base-2 scheme needs a finite reference from the start (it enters the
  // MFMA accumulation); the first tile with weight moves it to that tile's
  // max.
  w.m_run = kBase2 ? 0.f : -INFINITY;
  w.l_run = 0.f;
}

// Q^T operand fragments of query row `qrow` (the lane's column of S^T); for
// the base-2 scheme multiplied by c2 = scale * log2(e) in fp32 and rounded
// to bf16 (nearest even) once.
template <bool kBase2>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[8], const __bf16* qg, int64_t rs, int qrow,
                                       int g, float c2) {
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(qg + (int64_t)qrow * rs + kk * 16 + g * 8);
    if constexpr (kBase2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kk][e] = (__bf16)((float)x[e] * c2);
    } else {
      qf[kk] = x;
    }
  }
}

// One 32-key tile read from stage buffers (ks, vs); later tiles are already
// being loaded into other stages.  Each stage is a distinct __shared__ object,
// so the compiler does not order these LDS reads after the other stages' DMA
// writes.  kMask: keys at or past L.lim get no weight (only tiles that reach
// lim_lo test it).  kBase2: the score bookkeeping (see WaveState).
// kChecked = false: the reference never moves and no test is made (no tile
// max in the classic scheme), so the exponentials and the O^T MFMAs form one
// straight-line block; the caller certifies the row afterwards
// (row_certified) and redoes the sweep with checked steps if a row fails.
template <bool kMask, bool kBase2, bool kChecked = true>
__device__ __forceinline__ void tile_step(WaveState& w, const Lane& L, const bf16x8 (&qf)[8],
                                          const char* ks, const char* vs, int j0, int lim_lo,
                                          float c2) {
  // S^T = K Q^T (base 2: K (c2 Q)^T - m_run), fragment reads kept ahead of
  // the MFMAs that consume them.
  bf16x8 ka[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) ka[kk] = *reinterpret_cast<const bf16x8*>(ks + L.koff[kk]);
  f32x16 s0 = mfma32(ka[0], qf[0], kBase2 ? w.negm : f32x16{});
#pragma unroll
  for (int kk = 1; kk < 8; ++kk) s0 = mfma32(ka[kk], qf[kk], s0);

  // V^T fragments, read before the masking branch so that they share the
  // S^T MFMAs' basic block and the scheduler can issue them under that chain
  // (after the branch they waited for the exponentials' block).
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

  if constexpr (kMask) {
    if (j0 + kBN > lim_lo) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + (r >> 2) * 8 + L.g * 4 + (r & 3);
        s0[r] = key < L.lim ? s0[r] : -INFINITY;
      }
    }
  }

  bf16x8 pf[2];
  if constexpr (kBase2) {
    float p[16];
    float rsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(s0[r]);
      rsum += p[r];
    }
    // Rare path: a probability may pass 2^52 (or is not finite), or the row
    // has no weight yet; then take the tile max and move the reference if
    // it is more than 48 above it, or if the row has no weight (to the
    // first finite max, so that uniformly very negative scores do not all
    // underflow).  Lanes l and l + 32 hold the same row and decide alike.
    if (kChecked && __ballot(!(rsum <= kSumCap) || w.l_run == 0.f)) {
      float mx = s0[0];
#pragma unroll
      for (int r = 1; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s0[r]), s0[r + 1]);
      mx = fmaxf(mx, s0[15]);
      mx = xhalf_max(mx);
      const float l_row = xhalf_sum(w.l_run);
      const bool move = mx > kMoveT || (l_row == 0.f && mx > -INFINITY);
      const float shift = move ? mx : 0.f;
      const float alpha = l_row == 0.f ? 0.f : __builtin_amdgcn_exp2f(-shift);
      w.l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) w.oacc[dt][r] *= alpha;
      rsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = __builtin_amdgcn_exp2f(s0[r] - shift);
        rsum += p[r];
      }
      w.m_run += shift;
#pragma unroll
      for (int r = 0; r < 16; ++r) w.negm[r] = -w.m_run;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (__bf16)p[r];
    w.l_run += rsum;
  } else {
    if constexpr (kChecked) {
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
    }
    float rsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s0[r], c2, -w.m_run));
      rsum += p;
      pf[r >> 3][r & 7] = (__bf16)p;
    }
    w.l_run += xhalf_sum(rsum);
  }

#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) w.oacc[dt] = mfma32(vf[kq][dt], pf[kq], w.oacc[dt]);
}

// Base-2 scheme: l_run becomes the row's sum (both lanes of the row take
// part; call it with every lane of the wave active).
template <bool kBase2>
__device__ __forceinline__ void finish_rows(WaveState& w) {
  if constexpr (kBase2) w.l_run = xhalf_sum(w.l_run);
}

// After a sweep whose steps past the first were unchecked (the row's whole
// sum in l_run: finish_rows done in the base-2 scheme): the row's result is
// the checked scheme's up to rounding when its sum lies in [2^-20, 2^64] and
// the lane's O^T accumulators are finite.  Every probability is at most the
// sum, so none passed 2^64 (finite in bf16 and in the fp32 sums); the largest
// is at least the sum over the number of keys (below 2^31), at least 2^-51,
// so a probability that underflows (below 2^-126) is below 2^-75 of it; and
// O^T, at most the sum times max |v|, overflows only for |v| past 2^64 (the
// checked scheme lets the sum reach ~2^69), which the finiteness test
// catches.  The tests compare bit patterns, so NaN and inf fail whatever
// the compiler assumes about NaNs.
__device__ __forceinline__ bool row_certified(const WaveState& w) {
  const uint32_t lb = __float_as_uint(w.l_run);
  uint32_t e = 0;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) e = max(e, __float_as_uint(w.oacc[dt][r]) & 0x7f800000u);
  return lb >= 0x35800000u && lb <= 0x5f800000u && e != 0x7f800000u;  // 2^-20, 2^64
}

// O / l for the lane's query row (column of O^T), stored to orow.  A row that
// saw no key (l = 0) is written as zeros.
template <typename Tout>
__device__ __forceinline__ void store_row(const WaveState& w, Tout* orow, int g) {
  const float inv = w.l_run > 0.f ? 1.f / w.l_run : 0.f;
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

// XCD-aware renumbering of a 1-D grid: dispatch is round-robin over the 8
// XCDs, so consecutive ids of the result land on one XCD and share its L2.
// XCD x receives the blocks x, x + 8, ...: per of them if x < rem (or rem is
// 0), per - 1 otherwise.  Its ids form one contiguous range, and the ranges
// are laid out in the XCD order 0, 4, 1, 5, 2, 6, 3, 7, so that where the
// first rem XCDs hold one block more, each pair of neighbouring ranges holds
// 2 per - 1 ids: for 19 query tiles x 12 heads (228 blocks, rem 4) every
// range boundary then falls inside a head or on a head boundary such that
// each XCD holds two heads, where the order 0, 1, ..., 7 left three XCDs
// with parts of three heads.
__device__ __forceinline__ int xcd_major_id() {
  const int total = (int)gridDim.x;
  const int bid = blockIdx.x;
  const int per = (total + kXcds - 1) / kXcds;
  const int rem = total % kXcds;
  const int xcd = bid % kXcds;
  const int pos = 2 * (xcd & 3) + (xcd >> 2);
  int start = 0;
#pragma unroll
  for (int y = 0; y < kXcds; ++y) {
    if (2 * (y & 3) + (y >> 2) < pos) start += (rem == 0 || y < rem) ? per : per - 1;
  }
  return start + bid / kXcds;
}

}  // namespace attn128
}  // namespace rcc
