// Issue-rate probe for gfx950: how many cycles one wave per SIMD spends per
// iteration of a fixed mix of matrix (16x16x32 bf16 MFMA), transcendental
// (v_exp_f32, v_rcp_f32) and plain fp32 VALU instructions. It measures the
// ceiling of the recurrence's step: the state update applies tanh to every
// state element (exp2, add, reciprocal, two fused multiply-adds), so a step
// costs at least that element work plus the issue of its MFMAs, whatever the
// matrix core could do.
//
// Every wave keeps its operands in registers; the only memory traffic is one
// float per thread and one cycle count per wave at the end. Cycle counts come
// from the shader clock (clock64) read before and after the loop.
//
// Build: hipcc --offload-arch=gfx950 -O3 (the library's flags) issue_probe.hip
// Run:   ./issue_probe        (prints one line per mix, then "done")
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                 \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

constexpr int kBlocks = 256, kThreads = 256, kIters = 20000;

// Per iteration: NM MFMAs on 4 independent accumulators, NT transcendental
// instructions (reciprocals, or exp2 when EXP) on 16 independent registers,
// NV fused multiply-adds on 32 independent registers, and NE state elements
// updated as the recurrence does (exp2, 1 + e, reciprocal, two fmas).
template <int NM, int NT, int NV, int NE, bool EXP>
__global__ __launch_bounds__(kThreads, 1) void probe(float* out, long long* cyc, int iters, float z) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  float t[16], v[32], g[32];
  for (int i = 0; i < 16; ++i) t[i] = 1.0f + 0.001f * (threadIdx.x + i);
  for (int i = 0; i < 32; ++i) v[i] = 0.5f + 0.001f * (threadIdx.x + i);
  for (int i = 0; i < 32; ++i) g[i] = 0.25f - 0.001f * (threadIdx.x % 13 + i);
  f4 acc[4];
  for (int i = 0; i < 4; ++i) acc[i] = f4{0, 0, 0, 0};
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.01f * i);
    b[i] = static_cast<__bf16>(0.02f * (threadIdx.x % 7));
  }
  // constants the compiler cannot fold (z is a zero passed at launch)
  const float c1 = z + 0.999f, c2 = z + 0.0001f;
  const float fg = z + 0.9f, av = z + 0.2885f, m2a = z - 0.577f;
  __syncthreads();
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m % 4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[m % 4], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if constexpr (EXP) t[i % 16] = __builtin_amdgcn_exp2f(t[i % 16]) * 0.5f;
      else t[i % 16] = __builtin_amdgcn_rcpf(t[i % 16]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i % 32] = fmaf(v[i % 32], c1, c2);
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const float e = __builtin_amdgcn_exp2f(g[i]);
      const float r = __builtin_amdgcn_rcpf(1.0f + e);
      g[i] = fmaf(m2a, r, fmaf(fg, g[i], av));
    }
  }
  const long long t1 = clock64();
  float s = 0;
  for (int i = 0; i < 16; ++i) s += t[i];
  for (int i = 0; i < 32; ++i) s += v[i] + g[i];
  for (int i = 0; i < 4; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[tid] = s;
  if (threadIdx.x % 64 == 0) cyc[tid / 64] = t1 - t0;
}

template <int NM, int NT, int NV, int NE, bool EXP>
void run(const char* what, float* out, long long* cyc) {
  const int nwaves = kBlocks * kThreads / 64;
  for (int rep = 0; rep < 2; ++rep) {  // the first launch warms the clock
    hipLaunchKernelGGL((probe<NM, NT, NV, NE, EXP>), dim3(kBlocks), dim3(kThreads), 0, 0, out, cyc, kIters, 0.0f);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
  }
  std::vector<long long> h(nwaves);
  CHECK(hipMemcpy(h.data(), cyc, nwaves * sizeof(long long), hipMemcpyDeviceToHost));
  std::sort(h.begin(), h.end());
  std::printf("%-34s mfma %2d  trans %2d  fma %2d  elements %2d : %7.1f cycles per iteration (median wave; max %.1f)\n",
              what, NM, NT, NV, NE, static_cast<double>(h[nwaves / 2]) / kIters,
              static_cast<double>(h[nwaves - 1]) / kIters);
}

}  // namespace

int main() {
  float* out = nullptr;
  long long* cyc = nullptr;
  CHECK(hipMalloc(&out, kBlocks * kThreads * sizeof(float)));
  CHECK(hipMalloc(&cyc, kBlocks * kThreads / 64 * sizeof(long long)));
  std::printf("one wave per SIMD (%d workgroups x %d threads), %d iterations\n", kBlocks, kThreads, kIters);
  run<0, 0, 0, 0, false>("empty loop", out, cyc);
  run<0, 16, 0, 0, false>("reciprocal", out, cyc);
  run<0, 32, 0, 0, false>("reciprocal", out, cyc);
  run<0, 16, 0, 0, true>("exp2 (and a multiply)", out, cyc);
  run<0, 0, 16, 0, false>("fma", out, cyc);
  run<0, 0, 32, 0, false>("fma", out, cyc);
  run<4, 0, 0, 0, false>("mfma", out, cyc);
  run<8, 0, 0, 0, false>("mfma", out, cyc);
  run<4, 16, 0, 0, false>("mfma under reciprocals", out, cyc);
  run<4, 0, 32, 0, false>("mfma under fmas", out, cyc);
  run<0, 16, 16, 0, false>("reciprocals and fmas", out, cyc);
  run<0, 0, 0, 32, false>("state elements", out, cyc);
  run<44, 0, 0, 32, false>("state elements + one step's mfma", out, cyc);
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  std::printf("done\n");
  return 0;
}
