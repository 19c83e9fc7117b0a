// Matrix-core ceiling probe: v_mfma_f32_32x32x16_bf16 throughput and shader
// clock with zero, N(0,1) and constant operands.
//
// Each 4-wave workgroup runs 4 independent accumulator chains over 8 operand
// fragments per lane (so the multiplier inputs change every instruction) and
// times itself with s_memtime (shader clock) against s_memrealtime (100 MHz),
// which gives the clock the chip actually ran at.  With random operands the
// chip lowers its clock to stay in its power budget, which sets the
// practical MFMA ceiling for data like the workload's.
//
// Build and run (not part of librcc):
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       rope_chunk_causal_amd/probes/mfma_clock.hip -o /tmp/mfma_clock && /tmp/mfma_clock
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                    \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);         \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

constexpr int kThreads = 256;
constexpr int kFrags = 16;  // 8 A and 8 B fragments per lane

// src: kFrags fragments of kThreads lanes each.
__global__ __launch_bounds__(kThreads) void mfma_loop(const bf16x8* src, float* out,
                                                      unsigned long long* clk, int iters) {
  bf16x8 a[8], b[8];
  for (int i = 0; i < 8; ++i) {
    a[i] = src[i * kThreads + threadIdx.x];
    b[i] = src[(8 + i) * kThreads + threadIdx.x];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i + 1], b[i], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i + 1], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i + 1], b[i + 1], c3, 0, 0, 0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * kThreads + threadIdx.x] = s;  // keeps the chains live
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

static unsigned short f32_to_bf16(float f) {
  unsigned u;
  memcpy(&u, &f, 4);
  u += 0x7fff + ((u >> 16) & 1);
  return (unsigned short)(u >> 16);
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const int max_blocks = cus * 8;
  const int n = kFrags * kThreads * 8;  // bf16 elements
  std::vector<unsigned short> h(n);
  void* src;
  float* out;
  unsigned long long* clk;
  CHECK(hipMalloc(&src, n * 2));
  CHECK(hipMalloc(&out, (size_t)max_blocks * kThreads * 4));
  CHECK(hipMalloc(&clk, (size_t)max_blocks * 16));
  printf("device %s, %d CUs\n", prop.gcnArchName, cus);
  const char* names[3] = {"zeros", "normal", "ones"};
  for (int mode = 0; mode < 3; ++mode) {
    srand(3);
    for (int i = 0; i < n; ++i) {
      float x = 0.f;
      if (mode == 1) {  // Box-Muller N(0,1)
        const float u1 = (rand() + 1.f) / (RAND_MAX + 2.f), u2 = rand() / (float)RAND_MAX;
        x = sqrtf(-2.f * logf(u1)) * cosf(6.2831853f * u2);
      } else if (mode == 2) {
        x = 1.f;
      }
      h[i] = f32_to_bf16(x);
    }
    CHECK(hipMemcpy(src, h.data(), n * 2, hipMemcpyHostToDevice));
    for (int occ : {2, 8}) {  // workgroups per CU
      const int blocks = cus * occ, iters = 4000;
      hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(kThreads), 0, 0, (const bf16x8*)src, out, clk, 100);
      CHECK(hipDeviceSynchronize());
      hipEvent_t e0, e1;
      CHECK(hipEventCreate(&e0));
      CHECK(hipEventCreate(&e1));
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(kThreads), 0, 0, (const bf16x8*)src, out, clk, iters);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      std::vector<unsigned long long> hc((size_t)blocks * 2);
      CHECK(hipMemcpy(hc.data(), clk, (size_t)blocks * 16, hipMemcpyDeviceToHost));
      double cyc = 0, real = 0;
      for (int b = 0; b < blocks; ++b) {
        cyc += (double)hc[2 * b];
        real += (double)hc[2 * b + 1];
      }
      const double flop = (double)blocks * 4 * iters * 16 * 32768.0;  // 4 waves x 16 MFMAs
      printf("%-6s %d WG/CU: %.3f ms  %.1f TFLOP/s  shader clock %.0f MHz\n", names[mode], occ, ms,
             flop / ms / 1e9, cyc / real * 100.0);
      CHECK(hipEventDestroy(e0));
      CHECK(hipEventDestroy(e1));
    }
  }
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  CHECK(hipFree(clk));
  return 0;
}
