// Fused QKV projection + Causal-RoPE + KV-cache write, bf16.
//
// [YL] Yuan & Li, "Accelerating Video Generation Inference with
// Sequential-Parallel 3D Positional Encoding Using a Global Time Index",
// §3.4.1 item 3 (QKV projection and Causal-RoPE fused into one kernel) and
// Algorithm 3 steps 1-3 and 5: y = x W^T (+ b) for the rank's token slice,
// q and k rotated at the token's global (t, h, w), the rotated k and the
// unrotated v written to the cache rows of the slice.
//
// GEMM formulation on v_mfma_f32_32x32x16_bf16: C^T = W x^T, so an
// accumulator block has 32 output features as rows and 32 tokens as columns.
// In that layout lane l holds token l%32 and features 8(j/4) + 4(l/32) + j%4
// (j = 0..15): every rotary pair (2p, 2p+1) of a token sits in one lane, and
// the epilogue rotates it in fp32 straight from the accumulator (no bf16
// rounding of q and k before the rotation, unlike a projection followed by a
// separate RoPE kernel).
//
// * Workgroups are numbered so that each XCD's share is a compact
//   (features x tokens) rectangle of tiles: its L2 then serves the W rows of
//   a few feature tiles and the x rows of a few token tiles.
// * Workgroup = 8 waves = 256 features x BT tokens (BT = 256 or 384); wave
//   (wf, wt) owns 128 features x BT/4 tokens (4 x TB accumulator blocks,
//   TB = BT/128): per 16-deep k-step, 4 + TB fragment reads feed 4 TB MFMAs.
//   The host picks BT per call so that the grid fills the 256 CUs in the
//   fewest rounds: a 4680-token chunk is 13 x 18 = 234 workgroups of 384
//   tokens (one round) against 19 x 18 = 342 of 256 (two rounds).
// * W and x stream through a ring of LDS stages of 32 K-columns each (W tile
//   at +0, x tile after it) with buffer_load_dwordx4 ... lds from raw
//   buffers over W and x (exact LDS wait counts, see kRawBufferFlags): with
//   S stages, tile t is computed while the next S - 2 are in flight and tile
//   t + S - 1 starts into the stage t - 1 used.  Loads are branch-free (row and k
//   indices clamped), so the compiler tracks which stage each load writes.
// * Both operands are K-contiguous rows (64 B per row per stage) with the
//   16-byte chunk swizzle c ^ ((row / 4) % 4), which makes the ds_read_b128
//   fragment reads bank-conflict free.
// * Epilogue, one 32-token block at a time: bias (staged in LDS once) and
//   rotation in registers, bf16 results staged through the (then free) LDS
//   ring so that 16 lanes write each token's 256 B of a wave's 128 features
//   with one 16-byte store each.  The stores are non-temporal: the outputs
//   are written once and not read again by this kernel.
#include "rcc_internal.h"

namespace rcc {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBF = 256;                 // features per workgroup
constexpr int kBK = 32;                  // K columns per stage
constexpr int kRowBytes = kBK * 2;       // 64 B per row per stage
constexpr int kWTile = kBF * kRowBytes;  // 16 KB of W per stage
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int BT>
struct Tile {
  static constexpr int kTB = BT / 128;            // 32-token blocks per wave
  static constexpr int kXTile = BT * kRowBytes;   // x bytes per stage
  static constexpr int kStage = kWTile + kXTile;  // 32 or 40 KB
  static constexpr int kStages = BT == 256 ? 4 : 3;
  static constexpr int kXInstr = BT / 128;        // x DMA instructions per wave per stage
  static constexpr int kInstr = 2 + kXInstr;      // all DMA instructions per wave per stage
};

// Wave w loads W rows 32 w .. 32 w + 31 (two instructions of 16 rows) and x
// rows (BT/8) w .. (BT/8) (w + 1) - 1 (BT/128 instructions) of K-columns
// [k0, k0 + 32): lane l -> row base + 16 i + l/4, LDS chunk slot l%4, global
// chunk (l%4) ^ ((row / 4) % 4).  Rows past the matrix re-read its last row
// (their outputs are not stored); k0 past the end re-reads the last
// K-columns into a stage no step reads again.
template <int BT>
__device__ __forceinline__ void issue_stage(const __bf16* w, const __bf16* x, int f0, int t0,
                                            int n_feat, int n_tok, int K, int k0, char* ws,
                                            int wave, int lane) {
  using T = Tile<BT>;
  k0 = __builtin_amdgcn_readfirstlane(min(k0, K - kBK));
  char* xs = ws + kWTile;
  const uint32_t row_bytes = (uint32_t)(K * 2);
  // Buffer resources over W and x (each under 4 GiB, checked by the host):
  // the byte offsets stay 32-bit, and the hardware range check covers the
  // whole matrix.
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(w), 0, (int)((uint32_t)n_feat * row_bytes), kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(x), 0, (int)((uint32_t)n_tok * row_bytes), kRawBufferFlags);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 32 * wave + 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const uint32_t wrow = (uint32_t)min(f0 + r, n_feat - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(ws + (2 * wave + i) * 1024), 16,
                                             wrow * row_bytes + (uint32_t)(k0 * 2 + c * 16), 0,
                                             0, 0);
  }
#pragma unroll
  for (int i = 0; i < T::kXInstr; ++i) {
    const int r = 16 * (T::kXInstr * wave + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    const uint32_t xrow = (uint32_t)min(t0 + r, n_tok - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(xs + (T::kXInstr * wave + i) * 1024),
                                             16, xrow * row_bytes + (uint32_t)(k0 * 2 + c * 16),
                                             0, 0, 0);
  }
}

// At most n of this wave's loads in flight, then a barrier without a memory
// fence (a fence would also wait for the later stages).
template <int n>
__device__ __forceinline__ void stage_ready() {
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// kWan: head_dim 128 with rotary bands of 22 / 21 / 21 pairs (t / h / w);
// each 32-feature block then starts at a known place in its head, so every
// pair's band is a compile-time fact (up to the lane half).
template <int BT, bool kWan>
__global__ __launch_bounds__(kThreads, 1) void qkv_rope_kernel(QkvArgs a, int n_ft, int n_tt,
                                                               int gf) {
  using T = Tile<BT>;
  constexpr int S = T::kStages;
  constexpr int TB = T::kTB;
  // One object per stage, so the compiler does not order a stage's LDS reads
  // after another stage's DMA writes; each lies below 64 KB.
  __shared__ __align__(1024) char sS0[T::kStage];
  __shared__ __align__(1024) char sS1[T::kStage];
  __shared__ __align__(1024) char sS2[T::kStage];
  __shared__ __align__(1024) char sS3[S > 3 ? T::kStage : 16];
  auto stage = [&](int u) -> char* {
    return u == 0 ? sS0 : u == 1 ? sS1 : u == 2 ? sS2 : sS3;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int wf = wave >> 2;   // 128-feature half
  const int wt = wave & 3;    // token quarter

  // XCD-major numbering: an XCD's workgroups take consecutive ids.  Ids
  // run over groups of gf feature tiles; inside a group, token tile by token
  // tile, and the group's feature tiles inside that.  A range of consecutive
  // ids is then a compact (features x tokens) rectangle, so an XCD's L2
  // holds the W rows of a few feature tiles and the x rows of a few token
  // tiles, instead of all of W for every token tile.
  const int total = (int)gridDim.x;
  const int per = (total + kXcds - 1) / kXcds;
  const int rem = total % kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int id = xcd * per - (rem && xcd > rem ? xcd - rem : 0) + blockIdx.x / kXcds;
  const int grp = id / (gf * n_tt);
  const int in_grp = id - grp * gf * n_tt;
  const int gsz = min(gf, n_ft - grp * gf);  // the last group may be narrower
  const int f0 = (grp * gf + in_grp % gsz) * kBF;
  const int t0 = (in_grp / gsz) * BT;

  const int K = a.model_dim;
  const int hd = a.n_heads * a.head_dim;
  const int n_feat = 3 * hd;
  const int n_tok = a.batch * a.n_tokens;
  // Bias of the workgroup's 256 features, staged in LDS once (read in the
  // epilogue, after its barrier): per-block global bias loads exposed their
  // latency 4 TB times per wave.
  __shared__ __align__(16) float sBias[kBF];
  if (threadIdx.x < kBF)
    sBias[threadIdx.x] = (a.bias && f0 + (int)threadIdx.x < n_feat) ? a.bias[f0 + threadIdx.x] : 0.f;
  const __bf16* w = reinterpret_cast<const __bf16*>(a.w);
  const __bf16* x = reinterpret_cast<const __bf16*>(a.x);
  const int steps = K / kBK;

#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    issue_stage<BT>(w, x, f0, t0, n_feat, n_tok, K, u * kBK, stage(u), wave, lane);

  // chunk 2 kk + g of row r sits in slot (2 kk + g) ^ ((r / 4) % 4)
  const int sw0 = (g ^ ((l32 >> 2) & 3)) << 4;
  const int sw1 = ((2 + g) ^ ((l32 >> 2) & 3)) << 4;
  const int aoff0 = (wf * 128 + l32) * kRowBytes + sw0, aoff1 = aoff0 - sw0 + sw1;
  const int boff0 = kWTile + (wt * 32 * TB + l32) * kRowBytes + sw0, boff1 = boff0 - sw0 + sw1;

  f32x16 acc[4][TB];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[fb][tb] = f32x16{};

  auto step = [&](int t, int u) {
    stage_ready<(S - 2) * T::kInstr>();
    issue_stage<BT>(w, x, f0, t0, n_feat, n_tok, K, (t + S - 1) * kBK, stage((u + S - 1) % S),
                    wave, lane);
    const char* sp = stage(u);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ao = kk ? aoff1 : aoff0, bo = kk ? boff1 : boff0;
      bf16x8 af[4], bfr[TB];
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) af[fb] = *reinterpret_cast<const bf16x8*>(sp + ao + fb * 32 * kRowBytes);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) bfr[tb] = *reinterpret_cast<const bf16x8*>(sp + bo + tb * 32 * kRowBytes);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[fb][tb] = mfma32(af[fb], bfr[tb], acc[fb][tb]);
    }
  };
  int t = 0;
  for (; t + S <= steps; t += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) step(t + u, u);
  }
#pragma unroll
  for (int u = 0; u < S - 1; ++u)
    if (t + u < steps) step(t + u, u);
  // Every load has landed and every wave is done with the stages: they now
  // hold the output tiles.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Epilogue, per 32-token block of the wave: (1) registers -> LDS: bias
  // and the rotation of q and k in fp32, rounded to bf16, into this wave's
  // 32 x 128 staging tile (token-major, 256 B per token; 16-byte chunk c of
  // token t at slot c ^ (t % 16)); (2) LDS -> global: 16 lanes write one
  // token's 256 B, 4 tokens per instruction.  A wave reads back only what it
  // wrote, and its LDS operations complete in order: no barrier.
  char* tile = stage(wave >> 2) + (wave & 3) * 8192;
  // Cache row of each of the wave's 32 tokens of the current block, written
  // by the lane that owns the token and read back by the lanes storing it
  // (a wave's LDS operations complete in order).
  __shared__ int64_t sRow[kWaves][32];
  const float2* tab = reinterpret_cast<const float2*>(a.tables);
  const int c = lane & 15;
  const int fc = f0 + wf * 128 + c * 8;
  const int which_c = fc / hd;
  const int fr = fc - which_c * hd;
  const int head = fr / a.head_dim;
  const int dcol = head * a.head_dim + (fr - head * a.head_dim);
  __bf16* obase = reinterpret_cast<__bf16*>(which_c == 0 ? a.q_out : which_c == 1 ? a.k_cache : a.v_cache);
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int m = min(t0 + wt * 32 * TB + tb * 32 + l32, n_tok - 1);
    const int mb = m / a.n_tokens;
    const TokenPos pos = token_position(a.grid, m - mb * a.n_tokens);
    // This lane's token's cache row (the store phase takes it from the lane
    // that owns the token instead of recomputing the position), and the
    // float2 index shift of each band's row for the table lookups.
    if (g == 0) sRow[wave][l32] = (int64_t)mb * a.cache_tokens + pos.row;
    const int pt = kWan ? 22 : a.pt, ph = kWan ? 21 : a.ph, pw = kWan ? 21 : a.pw;
    const int sh_t = pos.t * pt;
    const int sh_h = (int)a.off_h + pos.h * ph - pt;
    const int sh_w = (int)a.off_w + pos.w * pw - pt - ph;
    // Per 32-feature block, the cos/sin of its 8 rotary pairs for the lane's
    // token are all loaded before any is used.
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const int f = f0 + wf * 128 + fb * 32;  // first feature of the block (wave-uniform)
      if (f >= n_feat) continue;
      const int which = f / hd;
      const int d0 = kWan ? fb * 32 : (f - which * hd) % a.head_dim;
      f32x4 bias[4];
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4)
        bias[j4] = *reinterpret_cast<const f32x4*>(sBias + wf * 128 + fb * 32 + j4 * 8 + g * 4);
      float2 cs[4][2];
      if (which < 2) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int pr = ((d0 + j4 * 8 + g * 4) >> 1) + e;  // rotary pair inside the head
            cs[j4][e] = tab[pr + (pr < pt ? sh_t : pr < pt + ph ? sh_h : sh_w)];
          }
      }
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[fb][tb][j4 * 4 + e] + bias[j4][e];
        if (which < 2) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float2 c2 = cs[j4][e];
            const float x0 = y[2 * e], x1 = y[2 * e + 1];
            y[2 * e] = x0 * c2.x - x1 * c2.y;
            y[2 * e + 1] = x0 * c2.y + x1 * c2.x;
          }
        }
        bf16x4 v;
        v[0] = (__bf16)y[0];
        v[1] = (__bf16)y[1];
        v[2] = (__bf16)y[2];
        v[3] = (__bf16)y[3];
        const int cc = fb * 4 + j4;  // 16-byte chunk of the 128 features
        *reinterpret_cast<bf16x4*>(tile + l32 * 256 + ((cc ^ (l32 & 15)) << 4) + g * 8) = v;
      }
    }
    // Chunk c of the wave's features is one 8-feature run of one head of q,
    // k or v.
    if (fc < n_feat) {
#pragma unroll 4
      for (int it = 0; it < 8; ++it) {
        const int tl = it * 4 + (lane >> 4);
        const int mm = t0 + wt * 32 * TB + tb * 32 + tl;
        if (mm >= n_tok) break;
        int64_t row;
        if (which_c == 0) {
          row = mm;
        } else {
          row = sRow[wave][tl];
        }
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(tile + tl * 256 + ((c ^ (tl & 15)) << 4));
        __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(obase + row * hd + dcol));
      }
    }
  }
}

// Feature tiles per group of the workgroup order (see the kernel).  Six
// (1536 features, 4.7 MB of W at model dim 1536) measured best among 3, 6, 9
// and 18 on the 480P chunk and close to best on the 64-chunk SP batch:
// reads beyond L2 fell from 136.5 to 96.9 MB and from 1.36 to 0.68 GB.
constexpr int kGroupTiles = 6;
int feature_group(int n_ft) { return n_ft < kGroupTiles ? n_ft : kGroupTiles; }

template <int BT>
hipError_t launch_bt(const QkvArgs& a, int n_ft, int64_t n_tok, hipStream_t s) {
  const int64_t n_tt = (n_tok + BT - 1) / BT;
  if (!grid_fits(n_ft * n_tt, kThreads)) return hipErrorInvalidConfiguration;
  const bool wan = a.head_dim == 128 && a.pt == 22 && a.ph == 21 && a.pw == 21;
  if (wan)
    hipLaunchKernelGGL((qkv_rope_kernel<BT, true>), dim3((uint32_t)(n_ft * n_tt)), dim3(kThreads),
                       0, s, a, n_ft, (int)n_tt, feature_group(n_ft));
  else
    hipLaunchKernelGGL((qkv_rope_kernel<BT, false>), dim3((uint32_t)(n_ft * n_tt)), dim3(kThreads),
                       0, s, a, n_ft, (int)n_tt, feature_group(n_ft));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_rope_append(const QkvArgs& a, hipStream_t s) {
  const int n_feat = 3 * a.n_heads * a.head_dim;
  const int64_t n_tok = (int64_t)a.batch * a.n_tokens;
  const int n_ft = (n_feat + kBF - 1) / kBF;
  // Token tile that fills the CUs in the fewest rounds, counting a round of
  // 384-token tiles as 1.5 rounds of 256-token ones.
  constexpr int64_t kCUs = 256;
  auto cost = [&](int64_t bt) {
    const int64_t tiles = n_ft * ((n_tok + bt - 1) / bt);
    return ((tiles + kCUs - 1) / kCUs) * bt;
  };
  return cost(384) < cost(256) ? launch_bt<384>(a, n_ft, n_tok, s) : launch_bt<256>(a, n_ft, n_tok, s);
}

}  // namespace rcc
