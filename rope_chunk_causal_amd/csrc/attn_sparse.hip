// Block-sparse attention over a persistent + local block memory, bf16,
// head_dim 128.
//
// [SF] "Sparse Forcing: Native Trainable Sparse Attention for Real-time
// Autoregressive Diffusion Video Generation", §3.3 (memory M = P u L,
// K = [K_P; K_L], block-contiguous layout, Top-K blocks Omega(q) per query
// block inside the local window) and §3.4 (one kernel that attends each
// query block to the persistent blocks and its own local blocks).  The
// selection is an input: the persistent list per (batch, head), the local
// list per (batch, head, query block).
//
// Design for gfx950:
// * Blocks of 64, 128 or 256 rows (attn_sparse_grouped_kernel): one 8-wave
//   workgroup per G = 8 / (B / 32) query blocks of one (batch, head); blocks
//   of 48 rows: one 4-wave workgroup per two query blocks.  The
//   persistent blocks, common to every query block, stream once for the
//   whole workgroup: all 8 waves share each K/V tile (four LDS stages, three
//   tiles in flight), so a tile moves into LDS once per 256 query rows, as in
//   the dense kernel.  Then each query block streams its own local blocks,
//   minus those already persistent, through stages of its own; the blocks
//   step together (one workgroup barrier per tile).
// * Blocks of 32 rows (attn_sparse_kernel): one single-wave workgroup per
//   query block over the union of its two lists.
// * Setup: the key sets are built in LDS as bitmaps over key blocks (LDS
//   atomics; repeats and entries outside [0, kv_tokens / B) drop out) and
//   compacted in ascending order with a wave-level scan.  The visit order
//   thus depends only on the sets, never on how the lists are ordered or
//   padded.
// * A list's blocks are read as one key stream of 32-row tiles.  For B a
//   multiple of 32 every tile lies inside one block: no partial tiles and no
//   masking.  For B = 48 a tile may span two blocks (three tiles per two
//   blocks) and only a list's last tile can be partial (its keys past the
//   stream are masked).  The per-tile MFMA and softmax work is attn_tile.h's,
//   shared with the dense kernel.
// * K/V tiles stream global -> LDS, branch-free (the tile index is clamped
//   to the last tile, so the wait counts stay exact), into one __shared__
//   object per stage.  A tile inside one block goes through buffer_load
//   ... lds from a raw buffer at the tile's wave-uniform 64-bit base with
//   32-bit lane offsets (exact LDS wait counts, see kRawBufferFlags).  A
//   48-row tile can span two blocks: while a (batch, head)'s cache rows lie
//   within 4 GiB of its base, each lane's 32-bit offset goes into one raw
//   buffer over them; past that, global_load_lds_dwordx4 with each lane's
//   own 64-bit offset.  So a batch entry's cache may exceed 4 GiB.
// * Workgroups are numbered XCD-major: the query blocks of one head run on
//   one XCD and share its L2.
// * In the grouped kernels only a wave's first key tile takes the checked
//   softmax step (it sets each row's reference); the other tiles take no
//   tile max and no test, and each stored row's sum and output certify the
//   result at the end (row_certified).  A workgroup with a row that fails
//   streams both phases again with every step checked, from the lists still
//   in LDS.
#include <type_traits>

#include "attn_tile.h"

namespace rcc {

namespace {

using namespace attn128;

constexpr int kMaxSel = 1024;  // list entries per query block (persistent + local)

template <int NW, int S>
struct Sparse {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kInstr = 8 / NW;      // DMA instructions per wave per tensor per tile
  static constexpr int kWait = (S - 2) * 2 * kInstr;  // loads of tiles t+1 .. t+S-2
  static_assert(NW == 1 || NW == 2 || NW == 4 || NW == 8, "block of 32, 64, 128 or 256 rows");
  static_assert(S >= 2 && S <= 4, "two to four stages");
};

// Issue this wave's share of tile t (clamped to the last tile: the pipeline
// runs S - 1 tiles ahead and re-reads the last one into a stage no step reads
// again).  Instruction i moves key rows 4 i .. 4 i + 3 of the tile into LDS
// bytes [i KB, +1 KB); lane -> (row 4 i + lane/16, chunk slot lane%16).
template <int NW>
__device__ __forceinline__ void issue_sparse(const char* kg, const char* vg, uint32_t row_bytes,
                                             const int* list, int t, int n_tiles, char* ks,
                                             char* vs, int wave, int lane) {
  constexpr int kInstr = 8 / NW;
  t = __builtin_amdgcn_readfirstlane(min(t, n_tiles - 1));
  const int blk = __builtin_amdgcn_readfirstlane(list[t / NW]);
  const int64_t base = (int64_t)(blk * (32 * NW) + (t % NW) * 32) * row_bytes;
  // Raw buffers over the tile's 32 key rows (see kRawBufferFlags).
  const int32_t span = (int32_t)(32 * row_bytes);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kg + base), 0, span, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t vr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vg + base), 0, span, kRawBufferFlags);
#pragma unroll
  for (int j = 0; j < kInstr; ++j) {
    const int i = wave + NW * j;
    const int r = 4 * i + (lane >> 4);
    const uint32_t off = (uint32_t)r * row_bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(ks + i * 1024), 16,
                                             off + k_chunk(r, lane & 15), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(vs + i * 1024), 16,
                                             off + v_chunk(r, lane & 15), 0, 0, 0);
  }
}

template <typename Tout, int NW, int S>
__global__ __launch_bounds__(64 * NW, NW > 1 ? 2 : 1) void attn_sparse_kernel(SparseArgs a) {
  using P = Sparse<NW, S>;
  // One object per stage (K tile at +0, V at +8 KB), so the compiler does not
  // order a stage's LDS reads after another stage's DMA writes.
  __shared__ __align__(1024) char sS0[2 * kTileBytes];
  __shared__ __align__(1024) char sS1[2 * kTileBytes];
  __shared__ __align__(1024) char sS2[S > 2 ? 2 * kTileBytes : 16];
  __shared__ __align__(1024) char sS3[S > 3 ? 2 * kTileBytes : 16];
  __shared__ int s_list[kMaxSel];
  __shared__ int s_wave_total[NW];
  auto stage = [&](int u) -> char* {
    return u == 0 ? sS0 : u == 1 ? sS1 : u == 2 ? sS2 : sS3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int id = xcd_major_id();
  const int qb = id % a.n_qblocks;
  const int bh = id / a.n_qblocks;
  const int h = bh % a.n_heads;
  const int b = bh / a.n_heads;

  const int64_t rs = (int64_t)a.n_heads * kD;
  const __bf16* qg = reinterpret_cast<const __bf16*>(a.q) + (int64_t)b * a.q_tokens * rs + h * kD;
  const char* kg = reinterpret_cast<const char*>(
      reinterpret_cast<const __bf16*>(a.k) + (int64_t)b * a.cache_tokens * rs + h * kD);
  const char* vg = reinterpret_cast<const char*>(
      reinterpret_cast<const __bf16*>(a.v) + (int64_t)b * a.cache_tokens * rs + h * kD);
  Tout* og = reinterpret_cast<Tout*>(a.out) + (int64_t)b * a.q_tokens * rs + h * kD;

  const int qrow = qb * (32 * NW) + wave * 32 + l32;
  const int qclamp = qrow < a.q_tokens ? qrow : a.q_tokens - 1;
  bf16x8 qf[8];
  load_q<false>(qf, qg, rs, qclamp, g, a.scale_log2);

  // ---- the query block's key set: bitmap over key blocks, then compaction
  uint32_t* bm = reinterpret_cast<uint32_t*>(sS0);
  const int words = (a.n_kblocks + 31) >> 5;
  for (int i = tid; i < words; i += P::kThreads) bm[i] = 0u;
  __syncthreads();
  const int* pl = a.persist + (int64_t)bh * a.n_persist;
  const int* ll = a.local + ((int64_t)bh * a.n_qblocks + qb) * a.n_local;
  const int n_entries = a.n_persist + a.n_local;
  for (int e = tid; e < n_entries; e += P::kThreads) {
    const int x = e < a.n_persist ? pl[e] : ll[e - a.n_persist];
    if ((unsigned)x < (unsigned)a.n_kblocks) atomicOr(&bm[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  const int wpt = (words + P::kThreads - 1) / P::kThreads;  // words per thread
  const int w0 = tid * wpt;
  int cnt = 0;
  for (int i = 0; i < wpt; ++i)
    if (w0 + i < words) cnt += __popc(bm[w0 + i]);
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wave_total[wave] = incl;
  __syncthreads();
  int pos = incl - cnt, n_sel = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) {
    const int tot = s_wave_total[w2];
    pos += w2 < wave ? tot : 0;
    n_sel += tot;
  }
  for (int i = 0; i < wpt; ++i) {
    if (w0 + i >= words) break;
    uint32_t word = bm[w0 + i];
    while (word) {
      const int bit = __builtin_ctz(word);
      s_list[pos++] = (w0 + i) * 32 + bit;
      word &= word - 1u;
    }
  }
  __syncthreads();  // visit list complete; the bitmap's stage is free again
  n_sel = __builtin_amdgcn_readfirstlane(n_sel);
  const int n_tiles = n_sel * NW;

  Lane L;
  lane_setup(L, lane);
  WaveState w;
  wave_init<false>(w);
  const float c2 = a.scale_log2;
  const uint32_t row_bytes = __builtin_amdgcn_readfirstlane((uint32_t)(rs * 2));

  if (n_tiles > 0) {
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
      issue_sparse<NW>(kg, vg, row_bytes, s_list, u, n_tiles, stage(u), stage(u) + kTileBytes,
                       wave, lane);
    // Tile t lives in stage t % S; tile t + S - 1 starts into the stage that
    // tile t - 1 used once every wave is past tile t - 1.
    auto step = [&](int t, int u) {
      tile_ready<P::kWait>();
      const int un = (u + S - 1) % S;
      issue_sparse<NW>(kg, vg, row_bytes, s_list, t + S - 1, n_tiles, stage(un),
                       stage(un) + kTileBytes, wave, lane);
      tile_step<false, false>(w, L, qf, stage(u), stage(u) + kTileBytes, 0, 0, c2);
    };
    int t = 0;
    for (; t + S <= n_tiles; t += S) {
#pragma unroll
      for (int u = 0; u < S; ++u) step(t + u, u);
    }
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
      if (t + u < n_tiles) step(t + u, u);
    // No load may still be writing this workgroup's LDS when it exits.
    __builtin_amdgcn_s_waitcnt(0);
  }

  if (qrow < a.q_tokens) store_row(w, og + (int64_t)qrow * rs, g);
}

// Compact a bitmap over key blocks into an ascending list (all 64 * NW
// threads of the workgroup take part); returns the number of set bits.
template <int NW>
__device__ __forceinline__ int compact_list(const uint32_t* bm, int words, int* out, int tid,
                                            int lane, int wave, int* s_tot) {
  constexpr int kT = 64 * NW;
  const int wpt = (words + kT - 1) / kT;
  const int w0 = tid * wpt;
  int cnt = 0;
  for (int i = 0; i < wpt; ++i)
    if (w0 + i < words) cnt += __popc(bm[w0 + i]);
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_tot[wave] = incl;
  __syncthreads();
  int pos = incl - cnt, total = 0;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) {
    const int tot = s_tot[w2];
    pos += w2 < wave ? tot : 0;
    total += tot;
  }
  for (int i = 0; i < wpt; ++i) {
    if (w0 + i >= words) break;
    uint32_t word = bm[w0 + i];
    while (word) {
      out[pos++] = (w0 + i) * 32 + __builtin_ctz(word);
      word &= word - 1u;
    }
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(total);
}

// Issue DMA instructions i = i0, i0 + di, ... (NI of them) of tile t of a
// list of n >= 1 key blocks.  The list's blocks are read as one key stream,
// laid end to end: tile t is stream rows 32 t .. 32 t + 31, and rows past the
// stream's end repeat its last row (their scores are masked).  t is clamped
// to the last tile (the pipeline runs ahead).  Instruction i moves tile rows
// 4 i .. 4 i + 3 into LDS bytes [i KB, +1 KB); lane -> (row 4 i + lane/16,
// chunk slot lane%16).  For B a multiple of 32 a tile lies inside one block
// and a wave-uniform 64-bit base plus 32-bit lane offsets address it; for
// B = 48 a tile spans at most two blocks and each lane forms its row's 64-bit
// offset itself.
template <int B, int NI, bool kBuf>
__device__ __forceinline__ void issue_list(const char* kg, const char* vg, uint32_t row_bytes,
                                           const int* list, int n, int t, char* ks, int i0,
                                           int di, int lane, __amdgpu_buffer_rsrc_t kall,
                                           __amdgpu_buffer_rsrc_t vall) {
  const int n_tiles = (n * B + 31) / 32;
  t = __builtin_amdgcn_readfirstlane(min(t, n_tiles - 1));
  if constexpr (B % 32 == 0) {
    constexpr int kPer = B / 32;
    const int blk = __builtin_amdgcn_readfirstlane(list[t / kPer]);
    const int64_t base = (int64_t)(blk * B + (t % kPer) * 32) * row_bytes;
    // Raw buffers over the tile's 32 key rows (see kRawBufferFlags).
    const int32_t span = (int32_t)(32 * row_bytes);
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kg + base), 0, span, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vg + base), 0, span, kRawBufferFlags);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = i0 + di * j;
      const int r = 4 * i + (lane >> 4);
      const uint32_t off = (uint32_t)r * row_bytes;
      const uint32_t ok = off + k_chunk(r, lane & 15), ov = off + v_chunk(r, lane & 15);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(ks + i * 1024), 16, ok, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(ks + kTileBytes + i * 1024), 16, ov,
                                               0, 0, 0);
    }
  } else {
    static_assert(B > 32 && B < 64, "a tile spans at most two blocks");
    const int g0 = 32 * t;
    const int last = n * B - 1;
    const int b_lo = g0 / B;
    const int b_hi = min(g0 + 31, last) / B;
    const int blk_lo = __builtin_amdgcn_readfirstlane(list[b_lo]);
    const int blk_hi = __builtin_amdgcn_readfirstlane(list[b_hi]);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int i = i0 + di * j;
      const int r = 4 * i + (lane >> 4);
      const int gr = min(g0 + r, last);
      const int bi = gr / B;
      const int row = (bi == b_lo ? blk_lo : blk_hi) * B + (gr - bi * B);
      if constexpr (kBuf) {
        // The (batch, head)'s whole cache lies within 4 GiB of its base
        // (checked by the host): 32-bit offsets into one raw buffer.
        const uint32_t off = (uint32_t)row * row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kall, (lds_void*)(ks + i * 1024), 16,
                                                 off + k_chunk(r, lane & 15), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vall, (lds_void*)(ks + kTileBytes + i * 1024),
                                                 16, off + v_chunk(r, lane & 15), 0, 0, 0);
      } else {
        const int64_t off = (int64_t)row * row_bytes;
        __builtin_amdgcn_global_load_lds(kg + off + k_chunk(r, lane & 15),
                                         (lds_void*)(ks + i * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vg + off + v_chunk(r, lane & 15),
                                         (lds_void*)(ks + kTileBytes + i * 1024), 16, 0, 0);
      }
    }
  }
}

// Grouped variant for blocks of 48, 64, 128 or 256 rows: one NW-wave
// workgroup takes G = NW / NWB query blocks of one (batch, head), NWB =
// ceil(B / 32) waves per block.  The persistent blocks, common to all of
// them, stream once for the whole workgroup (every wave shares each tile;
// four LDS stages, three tiles in flight, as in the dense kernel).  Then
// every query block streams its own local blocks, minus those already in the
// persistent set, through SL stages of its own; the blocks advance in
// lockstep (one workgroup barrier per tile), and a block with fewer tiles
// idles at the barriers.
//
// Blocks of 48 rows ([SF]'s [3,4,4]) run 4-wave workgroups of two query
// blocks (64 KB of stages, two workgroups per CU: a 12-head chunk of 112
// blocks per head is 672 of them over 512 slots, a smaller last round than
// 336 eight-wave workgroups over 256), and
// read each list as a key stream of 32-row tiles across block boundaries:
// three tiles per two blocks, only a list's last tile partial and masked.  A
// block's second wave holds its rows 32 .. 47; its other 16 rows are
// computed but not stored.
template <typename Tout, int NW, int NWB, int B, bool kBuf>
__global__ __launch_bounds__(64 * NW, NW == 8 ? 1 : 2) void attn_sparse_grouped_kernel(
    SparseArgs a, int n_groups, uint32_t span) {
  static_assert(NW == 8 || NW == 4, "4 or 8 waves");
  static_assert(B == 32 * NWB || (B == 48 && NWB == 2), "block of 48, 64, 128 or 256 rows");
  constexpr int kT = 64 * NW;
  constexpr int G = NW / NWB;
  constexpr int kObjs = NW == 8 ? 8 : 4;              // 16 KB stage objects
  constexpr int SL = kObjs / G < 4 ? kObjs / G : 4;   // local stages per query block
  constexpr bool kGather = B % 32 != 0;
  constexpr int kPI = 8 / NW;                         // DMA instructions per wave per tensor
  constexpr int kLI = 8 / NWB;                        //   (persistent, local phase)
  constexpr int kPWait = 2 * 2 * kPI;                 // loads of tiles t+1, t+2
  constexpr int kLWait = (SL - 2) * 2 * kLI;          // loads of tiles t+1 .. t+SL-2
  static_assert(SL >= 2 && 1 + G <= kObjs, "stages for the lists' bitmaps and the local phase");
  __shared__ __align__(1024) char sS0[2 * kTileBytes];
  __shared__ __align__(1024) char sS1[2 * kTileBytes];
  __shared__ __align__(1024) char sS2[2 * kTileBytes];
  __shared__ __align__(1024) char sS3[2 * kTileBytes];
  __shared__ __align__(1024) char sS4[kObjs > 4 ? 2 * kTileBytes : 16];
  __shared__ __align__(1024) char sS5[kObjs > 5 ? 2 * kTileBytes : 16];
  __shared__ __align__(1024) char sS6[kObjs > 6 ? 2 * kTileBytes : 16];
  __shared__ __align__(1024) char sS7[kObjs > 7 ? 2 * kTileBytes : 16];
  __shared__ int s_plist[kMaxSel];
  __shared__ int s_llist[G][kMaxSel];
  __shared__ int s_tot[NW];
  auto stage = [&](int u) -> char* {
    return u == 0 ? sS0 : u == 1 ? sS1 : u == 2 ? sS2 : u == 3 ? sS3
         : u == 4 ? sS4 : u == 5 ? sS5 : u == 6 ? sS6 : sS7;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const int id = xcd_major_id();
  const int grp = id % n_groups;
  const int bh = id / n_groups;
  const int h = bh % a.n_heads;
  const int b = bh / a.n_heads;
  const int qb0 = grp * G;
  const int jw = wave / NWB;            // this wave's query block in the group
  const int wq = wave % NWB;            // this wave's 32-row slice of it

  const int64_t rs = (int64_t)a.n_heads * kD;
  const __bf16* qg = reinterpret_cast<const __bf16*>(a.q) + (int64_t)b * a.q_tokens * rs + h * kD;
  const char* kg = reinterpret_cast<const char*>(
      reinterpret_cast<const __bf16*>(a.k) + (int64_t)b * a.cache_tokens * rs + h * kD);
  const char* vg = reinterpret_cast<const char*>(
      reinterpret_cast<const __bf16*>(a.v) + (int64_t)b * a.cache_tokens * rs + h * kD);
  Tout* og = reinterpret_cast<Tout*>(a.out) + (int64_t)b * a.q_tokens * rs + h * kD;
  // Raw buffers over the (batch, head)'s whole cache (used by 48-row tiles
  // when it spans under 4 GiB: span = its byte extent from kg).
  const __amdgpu_buffer_rsrc_t kall =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kg), 0, (int)span, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t vall =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vg), 0, (int)span, kRawBufferFlags);

  const int brow = wq * 32 + l32;       // the lane's row inside its query block
  const int qrow = (qb0 + jw) * B + brow;
  const int qclamp = qrow < a.q_tokens ? qrow : a.q_tokens - 1;
  bf16x8 qf[8];
  load_q<false>(qf, qg, rs, qclamp, g, a.scale_log2);

  // ---- key sets: persistent bitmap, then per query block the local blocks
  // not already persistent; compacted into ascending lists.
  const int words = (a.n_kblocks + 31) >> 5;
  uint32_t* pbm = reinterpret_cast<uint32_t*>(sS0);
  auto lbm = [&](int jj) { return reinterpret_cast<uint32_t*>(stage(1 + jj)); };
  for (int i = tid; i < words; i += kT) {
    pbm[i] = 0u;
#pragma unroll
    for (int jj = 0; jj < G; ++jj) lbm(jj)[i] = 0u;
  }
  __syncthreads();
  const int* pl = a.persist + (int64_t)bh * a.n_persist;
  for (int e = tid; e < a.n_persist; e += kT) {
    const int x = pl[e];
    if ((unsigned)x < (unsigned)a.n_kblocks) atomicOr(&pbm[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  for (int e = tid; e < G * a.n_local; e += kT) {
    const int jj = e / a.n_local;
    const int qbj = qb0 + jj;
    if (qbj >= a.n_qblocks) continue;
    const int x = a.local[((int64_t)bh * a.n_qblocks + qbj) * a.n_local + (e - jj * a.n_local)];
    if ((unsigned)x < (unsigned)a.n_kblocks && !((pbm[x >> 5] >> (x & 31)) & 1u))
      atomicOr(&lbm(jj)[x >> 5], 1u << (x & 31));
  }
  __syncthreads();
  const int n_p = compact_list<NW>(pbm, words, s_plist, tid, lane, wave, s_tot);
  int n_l[G];
#pragma unroll
  for (int jj = 0; jj < G; ++jj)
    n_l[jj] = compact_list<NW>(lbm(jj), words, s_llist[jj], tid, lane, wave, s_tot);

  Lane L;
  lane_setup(L, lane);
  WaveState w;
  const float c2 = a.scale_log2;
  const uint32_t row_bytes = __builtin_amdgcn_readfirstlane((uint32_t)(rs * 2));
  // Tile t of a key stream of n_rows rows (only a 48-row block's stream has a
  // partial last tile: keys at or past L.lim = n_rows get no weight).  chk:
  // a checked softmax step (see tile_step's kChecked).
  auto compute = [&](auto chk, int t, const char* ks, int n_rows) {
    constexpr bool C = decltype(chk)::value;
    if constexpr (kGather)
      tile_step<true, false, C>(w, L, qf, ks, ks + kTileBytes, 32 * t, n_rows, c2);
    else
      tile_step<false, false, C>(w, L, qf, ks, ks + kTileBytes, 0, 0, c2);
  };
  const std::true_type checked;

  const int np_rows = n_p * B;
  const int n_pt = (np_rows + 31) / 32;
  auto issue_p = [&](int t, char* ks) {
    issue_list<B, kPI, kBuf>(kg, vg, row_bytes, s_plist, n_p, t, ks, wave, NW, lane, kall, vall);
  };
  int n_it = 0;
#pragma unroll
  for (int jj = 0; jj < G; ++jj) n_it = max(n_it, (n_l[jj] * B + 31) / 32);

  // Both phases.  The wave's first key tile (the persistent stream's first,
  // or its block's first local tile when there is no persistent block) is a
  // checked step that sets each row's reference; the others are checked
  // only in the fallback sweep (all_checked).
  auto sweep = [&](auto all_checked) {
    const std::integral_constant<bool, decltype(all_checked)::value> rest;
    wave_init<false>(w);
    // ---- phase 1: the persistent blocks, every tile shared by all waves.
    // Tile t lives in stage t % 4.
    if (n_pt > 0) {
      L.lim = np_rows;
      issue_p(0, sS0);
      issue_p(1, sS1);
      issue_p(2, sS2);
      auto step = [&](auto chk, int t, int u) {
        tile_ready<kPWait>();
        issue_p(t + 3, stage((u + 3) & 3));
        compute(chk, t, stage(u), np_rows);
      };
      step(checked, 0, 0);
      int t = 1;
      for (; t + 4 <= n_pt; t += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) step(rest, t + u, (1 + u) & 3);
      }
#pragma unroll
      for (int u = 0; u < 3; ++u)
        if (t + u < n_pt) step(rest, t + u, (1 + u) & 3);
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();  // every wave is done with the shared stages

    // ---- phase 2: each query block's own local blocks, SL stages per
    // block (tile t in the block's stage t % SL), all blocks stepping
    // together.
    auto local_phase = [&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int nl_rows = n_l[J] * B;
      const int my = (nl_rows + 31) / 32;
      auto issue_l = [&](int t, char* ks) {
        issue_list<B, kLI, kBuf>(kg, vg, row_bytes, s_llist[J], n_l[J], t, ks, wq, NWB, lane,
                                  kall, vall);
      };
      // This block's my tiles, then idle barriers up to the group's n_it, so
      // every wave passes the same number of barriers.
      if (my > 0) {
        L.lim = nl_rows;
#pragma unroll
        for (int u = 0; u < SL - 1; ++u) issue_l(u, stage(J * SL + u));
        auto step = [&](auto chk, int t, int u) {
          tile_ready<kLWait>();
          issue_l(t + SL - 1, stage(J * SL + (u + SL - 1) % SL));
          compute(chk, t, stage(J * SL + u), nl_rows);
        };
        if (n_pt > 0)
          step(rest, 0, 0);
        else
          step(checked, 0, 0);
        int t = 1;
        for (; t + SL <= my; t += SL) {
#pragma unroll
          for (int u = 0; u < SL; ++u) step(rest, t + u, (1 + u) % SL);
        }
#pragma unroll
        for (int u = 0; u < SL - 1; ++u)
          if (t + u < my) step(rest, t + u, (1 + u) % SL);
      }
      for (int t = my; t < n_it; ++t) tile_ready<kLWait>();
    };
    switch (jw) {
      case 0: local_phase(std::integral_constant<int, 0>{}); break;
      case 1: if constexpr (G > 1) local_phase(std::integral_constant<int, 1>{}); break;
      case 2: if constexpr (G > 2) local_phase(std::integral_constant<int, 2>{}); break;
      default: if constexpr (G > 3) local_phase(std::integral_constant<int, 3>{}); break;
    }
    __builtin_amdgcn_s_waitcnt(0);
  };
  sweep(std::false_type{});

  // Certificate of the unchecked steps (row_certified) for every stored row
  // that saw a key; a workgroup with a row that fails sweeps again with
  // every step checked.  The lists stay in LDS, so the setup is not redone.
  int my_tiles = n_pt;
#pragma unroll
  for (int jj = 0; jj < G; ++jj)
    if (jj == jw) my_tiles += (n_l[jj] * B + 31) / 32;
  const bool stored = brow < B && qrow < a.q_tokens;
  if (__syncthreads_or(stored && my_tiles > 0 && !row_certified(w))) sweep(checked);

  if (brow < B && qrow < a.q_tokens) store_row(w, og + (int64_t)qrow * rs, g);
}

template <typename Tout, int NW, int NWB, int B>
hipError_t launch_grouped(const SparseArgs& a, hipStream_t s) {
  constexpr int G = NW / NWB;
  const int n_groups = (a.n_qblocks + G - 1) / G;
  const int64_t total = (int64_t)n_groups * a.n_heads * a.batch;
  if (!grid_fits(total, 64 * NW)) return hipErrorInvalidConfiguration;
  // Byte extent of one (batch, head)'s cache rows from its base.  48-row
  // tiles (which can span two key blocks) load through one raw buffer over
  // it when it fits 32-bit offsets, else with 64-bit global addresses; the
  // other block sizes always use per-tile buffers.
  const int64_t extent = (int64_t)(a.cache_tokens - 1) * a.n_heads * kRowBytes + kRowBytes;
  const bool narrow = extent <= (int64_t)UINT32_MAX;
  const uint32_t span = narrow ? (uint32_t)extent : UINT32_MAX;
  if constexpr (B % 32 != 0) {
    if (!narrow) {
      hipLaunchKernelGGL((attn_sparse_grouped_kernel<Tout, NW, NWB, B, false>),
                         dim3((uint32_t)total), dim3(64 * NW), 0, s, a, n_groups, span);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((attn_sparse_grouped_kernel<Tout, NW, NWB, B, true>),
                     dim3((uint32_t)total), dim3(64 * NW), 0, s, a, n_groups, span);
  return hipGetLastError();
}

template <typename Tout, int NW, int S>
hipError_t launch_nw(const SparseArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.n_qblocks * a.n_heads * a.batch;
  if (!grid_fits(total, 64 * NW)) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_sparse_kernel<Tout, NW, S>), dim3((uint32_t)total), dim3(64 * NW), 0,
                     s, a);
  return hipGetLastError();
}

template <typename Tout>
hipError_t launch_t(const SparseArgs& a, hipStream_t s) {
  switch (a.block_tokens) {
    case 32: return launch_nw<Tout, 1, 2>(a, s);
    case 48: return launch_grouped<Tout, 4, 2, 48>(a, s);
    case 64: return launch_grouped<Tout, 8, 2, 64>(a, s);
    case 128: return launch_grouped<Tout, 8, 4, 128>(a, s);
    default: return launch_grouped<Tout, 8, 8, 256>(a, s);
  }
}

}  // namespace

int block_sparse_max_entries() { return kMaxSel; }

hipError_t launch_block_sparse_attn(const SparseArgs& a, rcc_dtype out, hipStream_t s) {
  return out == RCC_BF16 ? launch_t<__bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace rcc
