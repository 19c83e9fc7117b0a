// Chunk-causal flash attention over the KV cache for gfx950 (CDNA4).
//
// [YL] Yuan & Li, "Accelerating Video Generation Inference with
// Sequential-Parallel 3D Positional Encoding Using a Global Time Index",
// Algorithm 3 step 6 (queries attend to the keys/values read back from the
// cache) with block-causal visibility (§3.2, §3.3): query i at cache
// position q_pos + i sees key j iff j < kv_tokens and
// floor(j / C) <= floor((q_pos + i) / C).  Because chunks are contiguous,
// the visible keys of a query are the prefix [0, lim) with
// lim = min(kv_tokens, (floor((q_pos + i) / C) + 1) * C).
//
// Design (one workgroup = 4 waves = 128 query rows of one (batch, head)):
// * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K (A operand) streams from LDS,
//   Q^T (B operand) stays in registers.  In the 32x32 accumulator layout a
//   lane holds one query column and 16 key rows, so the softmax row max and
//   row sum are in-register reductions plus one exchange between the two
//   32-lane halves.
// * O^T = V^T P^T on the same MFMA: P^T comes straight from the S^T
//   registers (rounded to bf16) as the B operand; V^T (A operand) is read
//   from an LDS copy of V stored transposed ([d][key]) with the keys of
//   each 16-key block permuted so that a lane's 8 key slots are one 16-byte
//   LDS read.
// * Online softmax in base 2 with fp32 state per query row; scale*log2(e)
//   is applied to the fp32 scores.
#include "rcc_internal.h"

namespace rcc {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup
constexpr int kBN = 64;           // keys per LDS tile
constexpr int kKPad = 8;          // bf16 padding per K row in LDS
constexpr int kVPad = 8;          // bf16 padding per V^T row in LDS

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive elements -> bf16x8 (RNE for fp32 input), or zeros.
__device__ __forceinline__ bf16x8 load8_bf16(const __bf16* p, bool ok) {
  if (!ok) return bf16x8{};
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16x8 load8_bf16(const float* p, bool ok) {
  bf16x8 r{};
  if (ok) {
    const float4 lo = reinterpret_cast<const float4*>(p)[0];
    const float4 hi = reinterpret_cast<const float4*>(p)[1];
    r[0] = (__bf16)lo.x; r[1] = (__bf16)lo.y; r[2] = (__bf16)lo.z; r[3] = (__bf16)lo.w;
    r[4] = (__bf16)hi.x; r[5] = (__bf16)hi.y; r[6] = (__bf16)hi.z; r[7] = (__bf16)hi.w;
  }
  return r;
}

__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Position, inside a 16-key block, of local key kl in the permuted V^T rows:
// lane half g, slot s of the P^T operand holds key (s/4)*8 + g*4 + s%4.
__device__ __forceinline__ int vperm(int kl) {
  return ((kl >> 2) & 1) * 8 + (kl >> 3) * 4 + (kl & 3);
}

template <int DP, typename Tin, typename Tout>
__global__ __launch_bounds__(kThreads) void chunk_causal_attn_kernel(AttnArgs a) {
  constexpr int KS = DP + kKPad;   // K row stride in LDS (elements)
  constexpr int VS = kBN + kVPad;  // V^T row stride in LDS (elements)
  constexpr int KK = DP / 16;      // MFMA k-steps over head_dim
  constexpr int DT = DP / 32;      // 32-wide output tiles over head_dim
  __shared__ __align__(16) __bf16 Ks[kBN * KS];
  __shared__ __align__(16) __bf16 Vt[DP * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int q0 = blockIdx.x * kBM;
  const int D = a.head_dim;
  const int64_t rs = (int64_t)a.n_heads * D;  // token row stride (elements)

  const Tin* qg = reinterpret_cast<const Tin*>(a.q) + ((int64_t)b * a.q_tokens) * rs + (int64_t)h * D;
  const Tin* kg = reinterpret_cast<const Tin*>(a.k) + ((int64_t)b * a.cache_tokens) * rs + (int64_t)h * D;
  const Tin* vg = reinterpret_cast<const Tin*>(a.v) + ((int64_t)b * a.cache_tokens) * rs + (int64_t)h * D;
  Tout* og = reinterpret_cast<Tout*>(a.out) + ((int64_t)b * a.q_tokens) * rs + (int64_t)h * D;

  // This lane's query row and its visible-key limit.
  const int qrow = q0 + wave * 32 + l32;
  const int qclamp = qrow < a.q_tokens ? qrow : a.q_tokens - 1;
  const int C = a.chunk_tokens;
  const int lim = min(a.kv_tokens, ((a.q_pos + qclamp) / C + 1) * C);
  // Workgroup-uniform bounds: keys below lim_lo are visible to every row,
  // keys at or above kv_end to none.
  const int qlast = min(q0 + kBM, a.q_tokens) - 1;
  const int lim_lo = min(a.kv_tokens, ((a.q_pos + q0) / C + 1) * C);
  const int kv_end = min(a.kv_tokens, ((a.q_pos + qlast) / C + 1) * C);

  // Q^T operand fragments: lane supplies row qrow, head-dim slots kk*16 + g*8 .. +7.
  bf16x8 qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int d0 = kk * 16 + g * 8;
    qf[kk] = load8_bf16(qg + (int64_t)qclamp * rs + d0, qrow < a.q_tokens && d0 < D);
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int j0 = 0; j0 < kv_end; j0 += kBN) {
    __syncthreads();
    // K tile -> Ks[key][d]
    for (int u = tid; u < kBN * (DP / 8); u += kThreads) {
      const int key = u / (DP / 8), c = u % (DP / 8);
      const int kj = j0 + key;
      const bf16x8 val = load8_bf16(kg + (int64_t)kj * rs + c * 8, kj < kv_end && c * 8 < D);
      *reinterpret_cast<bf16x8*>(&Ks[key * KS + c * 8]) = val;
    }
    // V tile -> Vt[d][perm(key)], 4 keys x 8 dims per unit
    for (int u = tid; u < (kBN / 4) * (DP / 8); u += kThreads) {
      const int kq = u / (DP / 8), c = u % (DP / 8);
      bf16x8 r[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int kj = j0 + kq * 4 + x;
        r[x] = load8_bf16(vg + (int64_t)kj * rs + c * 8, kj < kv_end && c * 8 < D);
      }
      const int kl = kq * 4;
      const int pos = (kl & ~15) + vperm(kl & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 w;
        w[0] = r[0][e]; w[1] = r[1][e]; w[2] = r[2][e]; w[3] = r[3][e];
        *reinterpret_cast<bf16x4*>(&Vt[(c * 8 + e) * VS + pos]) = w;
      }
    }
    __syncthreads();

    // S^T = K Q^T for two 32-key blocks.
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 kf =
            *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + l32) * KS + kk * 16 + g * 8]);
        sacc[kb] = mfma32(kf, qf[kk], sacc[kb]);
      }
    }

    // Scale to base-2 logits; mask keys at or beyond this row's limit.
    const bool need_mask = j0 + kBN > lim_lo;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float s = sacc[kb][j] * a.scale_log2;
        if (need_mask) {
          const int key = j0 + kb * 32 + (j >> 2) * 8 + g * 4 + (j & 3);
          s = key < lim ? s : -INFINITY;
        }
        sacc[kb][j] = s;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rsum = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(sacc[kb][j] - m_new);
        rsum += p;
        pf[kb][j >> 3][j & 7] = (__bf16)p;
      }
    }
    rsum += __shfl_xor(rsum, 32);
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[dt][j] *= alpha;

    // O^T += V^T P^T over the four 16-key blocks of the tile.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const bf16x8 vf =
            *reinterpret_cast<const bf16x8*>(&Vt[(dt * 32 + l32) * VS + kq * 16 + g * 8]);
        oacc[dt] = mfma32(vf, pf[kq >> 1][kq & 1], oacc[dt]);
      }
    }
  }

  if (qrow < a.q_tokens) {
    const float inv = 1.f / l_run;
    Tout* orow = og + (int64_t)qrow * rs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d0 = dt * 32 + jq * 8 + g * 4;
        if (d0 < D)
          store4(orow + d0, oacc[dt][jq * 4] * inv, oacc[dt][jq * 4 + 1] * inv,
                 oacc[dt][jq * 4 + 2] * inv, oacc[dt][jq * 4 + 3] * inv);
      }
    }
  }
}

template <int DP>
hipError_t launch_dp(const AttnArgs& a, rcc_dtype in, rcc_dtype out, hipStream_t s) {
  const dim3 grid((uint32_t)((a.q_tokens + kBM - 1) / kBM), (uint32_t)a.n_heads,
                  (uint32_t)a.batch);
  if (in == RCC_BF16 && out == RCC_BF16)
    hipLaunchKernelGGL((chunk_causal_attn_kernel<DP, __bf16, __bf16>), grid, dim3(kThreads), 0, s, a);
  else if (in == RCC_BF16 && out == RCC_F32)
    hipLaunchKernelGGL((chunk_causal_attn_kernel<DP, __bf16, float>), grid, dim3(kThreads), 0, s, a);
  else if (in == RCC_F32 && out == RCC_BF16)
    hipLaunchKernelGGL((chunk_causal_attn_kernel<DP, float, __bf16>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((chunk_causal_attn_kernel<DP, float, float>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_causal_attn(const AttnArgs& a, rcc_dtype in, rcc_dtype out,
                                    hipStream_t s) {
  if (a.q_tokens == 0) return hipSuccess;
  if (attn_d128_supported(a, in)) return launch_attn_d128(a, out, s);
  if (a.head_dim <= 32) return launch_dp<32>(a, in, out, s);
  if (a.head_dim <= 64) return launch_dp<64>(a, in, out, s);
  return launch_dp<128>(a, in, out, s);
}

}  // namespace rcc
