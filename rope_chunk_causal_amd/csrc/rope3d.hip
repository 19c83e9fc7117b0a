// 3D RoPE with a global time index, fused with the KV-cache write, for gfx950.
//
// [YL] Yuan & Li, "Accelerating Video Generation Inference with
// Sequential-Parallel 3D Positional Encoding Using a Global Time Index":
//   tables        §3.4.1 item 2 and Algorithm 2 (`freqs`, one per axis)
//   positions     §3.3.2 item 1, §3.3.3, Algorithm 3 steps 2-3
//   rotation      §3.3.1 equation, §3.3.2 item 2, Algorithm 2 (adjacent pairs
//                 viewed as complex numbers, multiplied by cos + i sin)
//   cache write   Algorithm 3 step 5
//
// The apply kernel is HBM-bound: per token it reads q, k, v and writes
// q', k-cache and v-cache rows (6 * n_heads * D elements).  Threads are laid
// along the [token, head, D] rows: one thread owns one 16-byte chunk (8
// elements, 4 rotary pairs) of a row, so every wave-wide access covers 1 KB
// of consecutive bytes of q, k, v and of the cache rows (4.6-5.8% more HBM
// bandwidth than a thread per (token, slot) looping over heads, whose
// accesses were 256-byte pieces 3 KB apart).  The 4 (cos, sin) pairs of a
// chunk come from the L2-resident tables.  All loads of a thread are issued
// before its first store (in-place q_out == q stays correct).  Streamed data is read and written with
// non-temporal hints: each byte is touched once here, and keeping it out of
// the caches measured ~15% more HBM bandwidth than plain accesses.
#include "rcc_internal.h"

namespace rcc {

namespace {

constexpr int kBlock = 256;

// ---------------------------------------------------------------- tables

__global__ __launch_bounds__(kBlock) void rope3d_tables_kernel(
    float2* __restrict__ out, double theta, int32_t pt, int32_t ph, int32_t pw,
    int32_t max_t, int32_t max_h, int32_t max_w) {
  const int64_t nt = (int64_t)max_t * pt, nh = (int64_t)max_h * ph,
                nw = (int64_t)max_w * pw;
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= nt + nh + nw) return;
  int64_t r = idx;
  int32_t pairs;
  if (r < nt) {
    pairs = pt;
  } else if (r < nt + nh) {
    r -= nt;
    pairs = ph;
  } else {
    r -= nt + nh;
    pairs = pw;
  }
  const int64_t p = r / pairs;
  const int32_t j = (int32_t)(r - p * pairs);
  // theta_{b,j} = theta^(-2j/d_b), d_b = 2 * pairs; evaluated in fp64.
  const double freq = pow(theta, -(2.0 * (double)j) / (double)(2 * pairs));
  const double ang = (double)p * freq;
  double s, c;
  sincos(ang, &s, &c);
  out[idx] = make_float2((float)c, (float)s);
}

// ------------------------------------------------------------- positions

__global__ __launch_bounds__(kBlock) void rope3d_positions_kernel(
    GridArgs g, int32_t n, int4* __restrict__ out) {
  const int32_t i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  const TokenPos p = token_position(g, i);
  out[i] = make_int4(p.t, p.h, p.w, p.row);
}

// ----------------------------------------------------------------- apply

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec8;

template <> struct Vec8<__bf16> {
  u32x4 raw;
  __device__ __forceinline__ void load(const __bf16* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ void to_float(float f[8]) const {
    const uint32_t w[4] = {raw[0], raw[1], raw[2], raw[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <> struct Vec8<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
  }
  __device__ __forceinline__ void to_float(float f[8]) const {
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  }
};

// Round-to-nearest-even fp32 -> bf16 (v_cvt_pk_bf16_f32) and 16-byte store.
__device__ __forceinline__ void store8(__bf16* p, const float f[8]) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)f[i];
  __builtin_nontemporal_store(v, reinterpret_cast<bf16x8*>(p));
}

__device__ __forceinline__ void store8(float* p, const float f[8]) {
  __builtin_nontemporal_store(f32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store(f32x4{f[4], f[5], f[6], f[7]}, reinterpret_cast<f32x4*>(p) + 1);
}

// Same-type copy of v is a bit copy; otherwise it goes through fp32.
template <typename Tin, typename Tout>
__device__ __forceinline__ void copy8(Tout* dst, const Vec8<Tin>& v) {
  float f[8];
  v.to_float(f);
  store8(dst, f);
}
template <>
__device__ __forceinline__ void copy8<__bf16, __bf16>(__bf16* dst, const Vec8<__bf16>& v) {
  __builtin_nontemporal_store(v.raw, reinterpret_cast<u32x4*>(dst));
}
template <>
__device__ __forceinline__ void copy8<float, float>(float* dst, const Vec8<float>& v) {
  __builtin_nontemporal_store(v.lo, reinterpret_cast<f32x4*>(dst));
  __builtin_nontemporal_store(v.hi, reinterpret_cast<f32x4*>(dst) + 1);
}

// (x0 + i x1) * (c + i s) for 4 pairs.
__device__ __forceinline__ void rotate8(float x[8], const float c[4], const float s[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x0 = x[2 * q], x1 = x[2 * q + 1];
    x[2 * q] = x0 * c[q] - x1 * s[q];
    x[2 * q + 1] = x0 * s[q] + x1 * c[q];
  }
}

// grid: x = ceil(n_tokens * n_heads * D/8 / kBlock), z = batch; a wave covers
// 1 KB of consecutive bytes of the [token, head, D] rows.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(kBlock) void rope3d_apply_append_kernel(RopeArgs a) {
  const uint32_t slots = (uint32_t)a.head_dim >> 3;
  const uint32_t row_chunks = (uint32_t)a.n_heads * slots;
  const uint32_t tid = blockIdx.x * kBlock + threadIdx.x;
  if (tid >= (uint32_t)a.n_tokens * row_chunks) return;
  const int32_t i = (int32_t)fdiv(tid, a.div_row_chunks);
  const uint32_t chunk = tid - (uint32_t)i * row_chunks;
  const int32_t c = (int32_t)(chunk - fdiv(chunk, a.div_slots) * slots);
  const int32_t b = blockIdx.z;
  const TokenPos p = token_position(a.grid, i);
  const char* tab = reinterpret_cast<const char*>(a.tables);
  const int32_t sh_t = p.t * a.pt;
  const int32_t sh_h = (int32_t)a.off_h + p.h * a.ph - a.pt;
  const int32_t sh_w = (int32_t)a.off_w + p.w * a.pw - a.pt - a.ph;
  float cs[4], sn[4];
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int32_t j = 4 * c + qq;
    const uint32_t idx = (uint32_t)(j + (j < a.pt ? sh_t : j < a.pt + a.ph ? sh_h : sh_w));
    const float2 v = *reinterpret_cast<const float2*>(tab + idx * 8u);
    cs[qq] = v.x;
    sn[qq] = v.y;
  }
  const int64_t row_stride = (int64_t)a.n_heads * a.head_dim;
  const int64_t in_off = ((int64_t)b * a.n_tokens + i) * row_stride + 8 * (int64_t)chunk;
  const int64_t c_off = ((int64_t)b * a.cache_tokens + p.row) * row_stride + 8 * (int64_t)chunk;
  Vec8<Tin> vq, vk, vv;
  vq.load(reinterpret_cast<const Tin*>(a.q) + in_off);
  vk.load(reinterpret_cast<const Tin*>(a.k) + in_off);
  vv.load(reinterpret_cast<const Tin*>(a.v) + in_off);
  float x[8];
  vq.to_float(x);
  rotate8(x, cs, sn);
  store8(reinterpret_cast<Tout*>(a.q_out) + in_off, x);
  vk.to_float(x);
  rotate8(x, cs, sn);
  store8(reinterpret_cast<Tout*>(a.k_cache) + c_off, x);
  copy8<Tin, Tout>(reinterpret_cast<Tout*>(a.v_cache) + c_off, vv);
}
}  // namespace

hipError_t launch_rope3d_tables(const rcc_rope3d_cfg& cfg, float* tables, hipStream_t s) {
  const int32_t pt = cfg.d_t / 2, ph = cfg.d_h / 2, pw = cfg.d_w / 2;
  const int64_t total = (int64_t)cfg.max_t * pt + (int64_t)cfg.max_h * ph +
                        (int64_t)cfg.max_w * pw;
  const uint32_t blocks = (uint32_t)((total + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(rope3d_tables_kernel, dim3(blocks), dim3(kBlock), 0, s,
                     reinterpret_cast<float2*>(tables), cfg.theta, pt, ph, pw,
                     cfg.max_t, cfg.max_h, cfg.max_w);
  return hipGetLastError();
}

hipError_t launch_rope3d_positions(const GridArgs& g, int32_t n, int32_t* thw, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint32_t blocks = (uint32_t)((n + kBlock - 1) / kBlock);
  hipLaunchKernelGGL(rope3d_positions_kernel, dim3(blocks), dim3(kBlock), 0, s, g, n,
                     reinterpret_cast<int4*>(thw));
  return hipGetLastError();
}

hipError_t launch_rope3d_apply_append(const RopeArgs& a, rcc_dtype in, rcc_dtype out,
                                      hipStream_t s) {
  if (a.n_tokens == 0) return hipSuccess;
  const int64_t threads = (int64_t)a.n_tokens * a.n_heads * (a.head_dim / 8);
  const dim3 grid((uint32_t)((threads + kBlock - 1) / kBlock), 1, (uint32_t)a.batch);
  if (in == RCC_BF16 && out == RCC_BF16)
    hipLaunchKernelGGL((rope3d_apply_append_kernel<__bf16, __bf16>), grid, dim3(kBlock), 0, s, a);
  else if (in == RCC_BF16 && out == RCC_F32)
    hipLaunchKernelGGL((rope3d_apply_append_kernel<__bf16, float>), grid, dim3(kBlock), 0, s, a);
  else if (in == RCC_F32 && out == RCC_BF16)
    hipLaunchKernelGGL((rope3d_apply_append_kernel<float, __bf16>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((rope3d_apply_append_kernel<float, float>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace rcc
