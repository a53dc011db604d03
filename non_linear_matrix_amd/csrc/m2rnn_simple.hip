// Simple M²RNN forward kernel: one workgroup per (batch, head) unit, the state
// and the transition matrix held in LDS as fp32, plain fp32 FMA loops and the
// device library's tanhf. It covers every supported shape and both input
// types, and is the fp32 path.
//
// Per step (gist.science M²RNN technical summary, zh §2.1 update equations):
//   Z_t = tanh(H_{t-1} W + k_t v_t^T),  H_t = f_t H_{t-1} + (1 - f_t) Z_t,
// then the readout y_t = H_t^T q_t.
#include <hip/hip_runtime.h>

#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPerThread = 128 * 128 / kThreads;  // K, V <= 128

__device__ __forceinline__ float load_in(const void* p, long long i, int bf16) {
  if (bf16) {
    unsigned int u = static_cast<const unsigned short*>(p)[i];
    return __uint_as_float(u << 16);
  }
  return static_cast<const float*>(p)[i];
}

__global__ __launch_bounds__(kThreads) void simple_fwd_kernel(FwdArgs a) {
  extern __shared__ float smem[];
  const int K = a.K, V = a.V, T = a.T;
  const int KV = K * V;
  float* Hs = smem;        // [K][V]
  float* Ws = Hs + KV;     // [V][V]
  float* ks = Ws + V * V;  // [K]
  float* qs = ks + K;      // [K]
  float* vs = qs + K;      // [V]
  float* fs = vs + V;      // [1]
  const int tid = threadIdx.x;
  const long long unit = blockIdx.x;  // b * H + h
  const int h = static_cast<int>(unit % a.H);
  // this sequence's length; y rows past it are left to the launcher's fill
  const int Tb = a.lens ? min(max(a.lens[unit / a.H], 0), T) : T;

  for (int e = tid; e < V * V; e += kThreads) Ws[e] = load_in(a.W, (long long)h * V * V + e, a.bf16);
  for (int e = tid; e < KV; e += kThreads) Hs[e] = a.H0 ? a.H0[unit * KV + e] : 0.0f;

  const long long ld = a.ld > 0 ? a.ld : T;  // row stride of the per-step arrays
  const long long seqK = unit * ld * K;
  const long long seqV = unit * ld * V;
  for (int t = 0; t < Tb; ++t) {
    __syncthreads();  // previous readout finished with ks/qs/vs; W and H0 staged
    for (int e = tid; e < K; e += kThreads) {
      ks[e] = load_in(a.k, seqK + (long long)t * K + e, a.bf16);
      qs[e] = load_in(a.q, seqK + (long long)t * K + e, a.bf16);
    }
    for (int e = tid; e < V; e += kThreads) vs[e] = load_in(a.v, seqV + (long long)t * V + e, a.bf16);
    if (tid == 0) fs[0] = load_in(a.f, unit * ld + t, a.bf16);
    __syncthreads();
    const float ft = fs[0];
    float nv[kMaxPerThread];
#pragma unroll
    for (int r = 0; r < kMaxPerThread; ++r) {
      const int e = tid + r * kThreads;
      if (e < KV) {
        const int i = e / V, j = e - i * V;
        float acc = 0.0f;
        for (int l = 0; l < V; ++l) acc = fmaf(Hs[i * V + l], Ws[l * V + j], acc);
        const float z = tanhf(acc + ks[i] * vs[j]);
        nv[r] = ft * Hs[e] + (1.0f - ft) * z;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kMaxPerThread; ++r) {
      const int e = tid + r * kThreads;
      if (e < KV) Hs[e] = nv[r];
    }
    __syncthreads();
    for (int j = tid; j < V; j += kThreads) {
      float s = 0.0f;
      for (int i = 0; i < K; ++i) s = fmaf(Hs[i * V + j], qs[i], s);
      float* yp = a.y + seqV + (long long)t * V + j;
      *yp = a.accumulate ? *yp + s : s;
    }
  }
  if (a.HT) {
    __syncthreads();
    for (int e = tid; e < KV; e += kThreads) a.HT[unit * KV + e] = Hs[e];
  }
}

}  // namespace

Plan plan_simple(int B, int H, int K, int V) {
  const long long units = (long long)B * H;
  const size_t lds = sizeof(float) * ((size_t)K * V + (size_t)V * V + 2 * K + V + 1);
  return Plan{units > 0x7fffffffLL ? -1 : (int)units, kThreads, K, 1, 0, (int)lds};
}

hipError_t launch_simple(const FwdArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)plan_simple(a.B, a.H, a.K, a.V).lds_bytes;
  if (a.lens && !a.accumulate) {  // rows past a sequence's length read as zero
    if (a.ld > 0 && a.ld != a.T) return hipErrorInvalidValue;  // a window of y: the caller clears it
    hipError_t e = fill_zero(a.y, (long long)a.B * a.H * a.T * a.V, stream);
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(simple_fwd_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const long long units = (long long)a.B * a.H;
  if (units > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(simple_fwd_kernel, dim3((unsigned)units), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace m2rnn
