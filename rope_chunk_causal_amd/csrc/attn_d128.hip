// Chunk-causal flash attention, bf16, head_dim 128: the production shape.
//
// [YL] Yuan & Li, "Accelerating Video Generation Inference with
// Sequential-Parallel 3D Positional Encoding Using a Global Time Index",
// Algorithm 3 step 6 with block-causal visibility (§3.2, §3.3); the
// visibility rule and the MFMA formulation are those of attn.hip; the
// per-tile work (MFMA S^T and O^T, swizzled LDS reads, online softmax) is in
// attn_tile.h.
//
// What this kernel adds for the bf16 / head_dim-128 shape:
// * One workgroup of 8 waves (256 query rows, two waves per SIMD) per CU, so
//   each K/V tile moves from L2 into LDS once per 256 rows.
// * K and V move global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//   staging) in 32-key tiles through a ring of four LDS stages: tile t is
//   computed while tiles t+1 and t+2 are in flight and tile t+3 starts into
//   the stage tile t-1 used.  One workgroup barrier per tile; the wait before
//   it counts only the loads of tile t.  (A two-stage ring that waits for the
//   next tile each step leaves the MFMAs idle for much of the L2 latency.)
// * Workgroups are renumbered so each XCD (dispatch is round-robin over the
//   8 XCDs) gets a contiguous range of (batch, head, query-tile) work: query
//   tiles of one head run on one XCD and share its L2 for K/V.
// * Only the first tile's softmax step is checked: it sets each row's
//   reference, and the other tiles' steps make no test, so a tile's
//   exponentials and O^T MFMAs run as one straight-line block.  Each row's
//   sum and output then certify the sweep (row_certified); a workgroup with
//   a row that fails sweeps again with every step checked.
#include <type_traits>

#include "attn_tile.h"

namespace rcc {

namespace {

using namespace attn128;

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;      // query rows per workgroup
constexpr int kStages = 4;            // K/V tiles resident in LDS

// DMA layout of a tile: wave w moves 1 KB = key rows 4 w + (0..3) into LDS
// bytes [w KB, +1 KB); lane -> (row 4 w + lane/16, LDS chunk slot lane%16).
struct Dma {
  uint32_t k, v;      // lane's byte offset inside its key row (swizzled chunk)
};

__device__ __forceinline__ Dma dma_offsets(int wave, int lane) {
  const int r = 4 * wave + (lane >> 4);  // 0..31
  Dma d;
  d.k = k_chunk(r, lane & 15);
  d.v = v_chunk(r, lane & 15);
  return d;
}

// Issue this wave's share of one K and one V tile (keys j0 .. j0+31).  Key
// indices are clamped to kv_end - 1: a ragged last tile re-reads the last key
// for rows past kv_end (their scores are masked), and a tile past the end (the
// pipeline always runs three tiles ahead) re-reads it into a stage no step
// reads again.  Branch-free, so the compiler tracks which stage each load
// writes.  The tile's first key (clamped) gives a wave-uniform 64-bit base;
// each lane adds a 32-bit offset of at most 31 rows, so a batch entry's cache
// may exceed 4 GiB.
__device__ __forceinline__ void issue_tile(const char* kg, const char* vg, uint32_t row_bytes,
                                           int j0, int kv_end, const Dma& d, char* ks,
                                           char* vs, int wave, int lane) {
  const int jb = __builtin_amdgcn_readfirstlane(min(j0, kv_end - 1));
  const int64_t base = (int64_t)jb * row_bytes;
  const int key = min(j0 + 4 * wave + (lane >> 4), kv_end - 1);
  const uint32_t row = (uint32_t)(key - jb) * row_bytes;
  // Raw buffers over the tile's 32 key rows (wave-uniform base): LDS-DMA
  // through buffer loads, so the LDS fragment reads get exact wait counts.
  const int32_t span = (int32_t)(kBN * row_bytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kg + base), 0, span, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vg + base), 0, span, kRawBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(ks + wave * 1024), 16, row + d.k, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vs + wave * 1024), 16, row + d.v, 0, 0, 0);
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

  const int id = xcd_major_id();
  const int qt = id % n_qt;
  const int bh = id / n_qt;
  const int h = bh % a.n_heads;
  const int b = bh / a.n_heads;

  const int64_t rs = (int64_t)a.n_heads * kD;
  const __bf16* qg = reinterpret_cast<const __bf16*>(a.q) + (int64_t)b * a.q_tokens * rs + h * kD;
  const char* kg = reinterpret_cast<const char*>(
      reinterpret_cast<const __bf16*>(a.k) + (int64_t)b * a.cache_tokens * rs + h * kD);
  const char* vg = reinterpret_cast<const char*>(
      reinterpret_cast<const __bf16*>(a.v) + (int64_t)b * a.cache_tokens * rs + h * kD);
  const uint32_t row_bytes = (uint32_t)(rs * 2);
  Tout* og = reinterpret_cast<Tout*>(a.out) + (int64_t)b * a.q_tokens * rs + h * kD;

  const int q0 = qt * kBM;
  const int qrow = q0 + wave * 32 + l32;
  // A wave whose 32 rows all lie past q_tokens (the last query tile of a
  // ragged chunk) still moves its share of every K/V tile and meets every
  // barrier, but runs no matrix or softmax work.
  const bool has_rows = q0 + wave * 32 < a.q_tokens;
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
  load_q<true>(qf, qg, rs, qclamp, g, a.scale_log2);

  const Dma dma = dma_offsets(wave, lane);
  auto prologue = [&]() {
    issue_tile(kg, vg, row_bytes, 0, kv_end, dma, sK0, sV0, wave, lane);
    issue_tile(kg, vg, row_bytes, kBN, kv_end, dma, sK1, sV1, wave, lane);
    issue_tile(kg, vg, row_bytes, 2 * kBN, kv_end, dma, sK2, sV2, wave, lane);
  };
  prologue();

  Lane L;
  lane_setup(L, lane);
  L.lim = min(a.kv_tokens, ((a.q_pos + qclamp) / C + 1) * C);

  WaveState w;
  const float c2 = a.scale_log2;

  // Tile t lives in stage t % 4; tiles t+1 and t+2 are in flight while it is
  // computed, and tile t+3 starts into the stage that tile t-1 used.  The
  // first tile sets each row's reference (a checked step); the others run
  // unchecked (kChecked false) unless `checked`, the fallback sweep.  The
  // loop is instantiated for each and, for a wave with no query rows, as DMA
  // and barriers only, so no copy branches per tile.
  auto sweep = [&](auto work, auto checked) {
    wave_init<true>(w);
    auto step = [&](auto first, int t, const char* ks, const char* vs, char* kn, char* vn) {
      tile_ready<4>();
      issue_tile(kg, vg, row_bytes, (t + 3) * kBN, kv_end, dma, kn, vn, wave, lane);
      if constexpr (decltype(work)::value)
        tile_step<true, true, decltype(first)::value || decltype(checked)::value>(
            w, L, qf, ks, vs, t * kBN, lim_lo, c2);
    };
    const std::true_type head;
    const std::false_type body;
    if (n_tiles > 0) step(head, 0, sK0, sV0, sK3, sV3);
    int t = 1;
    for (; t + kStages <= n_tiles; t += kStages) {
      step(body, t, sK1, sV1, sK0, sV0);
      step(body, t + 1, sK2, sV2, sK1, sV1);
      step(body, t + 2, sK3, sV3, sK2, sV2);
      step(body, t + 3, sK0, sV0, sK3, sV3);
    }
    if (t < n_tiles) step(body, t, sK1, sV1, sK0, sV0);
    if (t + 1 < n_tiles) step(body, t + 1, sK2, sV2, sK1, sV1);
    if (t + 2 < n_tiles) step(body, t + 2, sK3, sV3, sK2, sV2);
    // No load may still be writing this workgroup's LDS after the sweep.
    __builtin_amdgcn_s_waitcnt(0);
    finish_rows<true>(w);
  };
  if (has_rows)
    sweep(std::true_type{}, std::false_type{});
  else
    sweep(std::false_type{}, std::false_type{});

  // Certificate of the unchecked steps (row_certified); a workgroup with a
  // row that fails sweeps again with every step checked (only for scores
  // that rise far above the first tile's, or rows with almost no weight).
  // Rows past q_tokens repeat the last row and decide like it.
  if (__syncthreads_or(n_tiles > 0 && has_rows && !row_certified(w))) {
    prologue();
    if (has_rows)
      sweep(std::true_type{}, std::true_type{});
    else
      sweep(std::false_type{}, std::true_type{});
  }

  if (qrow < a.q_tokens) store_row(w, og + (int64_t)qrow * rs, g);
}

}  // namespace

bool attn_d128_supported(const AttnArgs& a, rcc_dtype in) {
  return in == RCC_BF16 && a.head_dim == kD;
}

hipError_t launch_attn_d128(const AttnArgs& a, rcc_dtype out, hipStream_t s) {
  const int n_qt = (a.q_tokens + kBM - 1) / kBM;
  const int64_t total = (int64_t)n_qt * a.n_heads * a.batch;
  if (!grid_fits(total, kThreads)) return hipErrorInvalidConfiguration;
  if (out == RCC_BF16)
    hipLaunchKernelGGL((attn_d128_kernel<__bf16>), dim3((uint32_t)total), dim3(kThreads), 0, s, a, n_qt);
  else
    hipLaunchKernelGGL((attn_d128_kernel<float>), dim3((uint32_t)total), dim3(kThreads), 0, s, a, n_qt);
  return hipGetLastError();
}

}  // namespace rcc
