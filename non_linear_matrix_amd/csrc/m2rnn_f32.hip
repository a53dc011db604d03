// fp32 matrix-core M²RNN forward: every operand of the step in fp32, the state
// product on v_mfma_f32_16x16x4_f32.
//
// Per step (gist.science M²RNN technical summary, zh §2.1 update equations):
//   Z_t = tanh(H_{t-1} W + k_t v_t^T),  H_t = f_t H_{t-1} + (1 - f_t) Z_t,
// then the readout y_t = H_t^T q_t. The pages tie K and V, in multiples of 16,
// to the matrix units (zh §2.2, hardware-utilisation bullet); this kernel is
// that mapping for fp32 inputs, where the bf16 kernels' operand rounding would
// spend the fp32 bar.
//
// Work split: one workgroup per (batch, head) unit, one wave per 16-row tile of
// the K x V state (K / 16 waves). The state lives in registers for all T steps.
//
// Register layout (the same permuted-contraction idea as the bf16 kernels, for
// the 16x16x4 fp32 shape). The wave computes D = W^T G^T per 16-column tile co:
// lane l = 16 g + i holds, in accumulator register r, the element
// (row i, column 16 co + 4 g + r) of the tile. Contraction block (c, r) takes the
// state columns {16 c + 4 g + r : g = 0..3}; its B operand, lane l's value
// G[i][16 c + 4 g + r], is exactly register r of that lane's state tile c, so a
// step's result feeds the next step's products with no data movement. The A
// operand of block (c, r) for output tile co is W[16 c + 4 g + r][16 co + i]: a
// constant per lane, kept in registers for V <= 64 and read from LDS (stored in
// that order, one 16-byte read per (co, c)) for V = 128.
//
// Nonlinearity: the device library's tanhf on the fp32 pre-activation. The bf16
// kernels' 1 - 2 / (1 + 2^u) form has an absolute error near one ulp of 1,
// which is a large relative error on the small state elements of workloads with
// scaled inputs, and trajectories that amplify perturbations carry it to H_T;
// tanhf keeps every element's error relative. The gate blend is
// H_t = f H_{t-1} + (1 - f) Z_t as one FMA after the product (1 - f) Z_t.
//
// Readout: each lane multiplies its state elements by q_t[row], a 16-lane
// DPP butterfly sums the tile's rows (every lane of a row ends with the same
// sum), the per-wave partials go to LDS, and at the end of every 16-step chunk
// the waves' partials are added in wave order and written once: y has one fixed
// summation order, so it is bitwise repeatable and needs no clearing.
//
// Inputs k, q, v, f are staged through LDS 16 steps at a time; the next chunk's
// loads are issued one chunk ahead into registers.
#include <hip/hip_runtime.h>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

using namespace dev;

constexpr int kChunk = 16;        // steps staged at once
constexpr int kMaxThreads = 512;  // K = 128: 8 waves

// D = A B + C on a 16x16 fp32 tile, A and B fp32 with 4-deep contraction
__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS (floats): W fragments (V = 128 only: [co][c][lane] f4) | staged chunk
// k [16][K], q [16][K], v [16][V], f [16] | y partials [waves][16][V].
template <int V>
struct Lds {
  static constexpr bool WREG = V <= 64;
  static constexpr int W_FLOATS = WREG ? 0 : V * V;
  __host__ __device__ static int stage_off() { return W_FLOATS; }
  __host__ __device__ static int f_off(int K) { return stage_off() + kChunk * (2 * K + V); }
  __host__ __device__ static int y_off(int K) { return f_off(K) + kChunk; }
  __host__ __device__ static int total_bytes(int K) { return 4 * (y_off(K) + (K / 16) * kChunk * V); }
};

template <int V>
__global__ __launch_bounds__(kMaxThreads) void mfma_f32_fwd_kernel(FwdArgs a) {
  constexpr int CT = V / 16;  // 16-column tiles
  constexpr bool WREG = Lds<V>::WREG;
  constexpr int kSlots = 2 + CT;  // >= (8 K + 4 V) / (4 K): 16-byte chunk loads per thread
  extern __shared__ __align__(16) float smem[];
  const int K = a.K, T = a.T, NW = K / 16, NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const long long unit = blockIdx.x;  // b * H + h
  const int h = static_cast<int>(unit % a.H);
  // this sequence's length; y rows past it are left to the launcher's fill
  const int Tb = a.lens ? min(max(a.lens[unit / a.H], 0), T) : T;
  const long long ld = a.ld > 0 ? a.ld : T;  // row stride of the per-step arrays

  f4* Wl = reinterpret_cast<f4*>(smem);
  float* st = smem + Lds<V>::stage_off();
  float* fs = smem + Lds<V>::f_off(K);
  float* yp = smem + Lds<V>::y_off(K);
  const float* ks = st;
  const float* qs = st + kChunk * K;
  const float* vs = st + 2 * kChunk * K;

  // W as A fragments: (co, c) holds W[16 c + 4 g + r][16 co + i], r = 0..3
  const float* Wg = static_cast<const float*>(a.W) + (long long)h * V * V;
  f4 wreg[WREG ? CT * CT : 1];
  if constexpr (WREG) {
#pragma unroll
    for (int co = 0; co < CT; ++co)
#pragma unroll
      for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) wreg[co * CT + c][r] = Wg[(16 * c + 4 * grp + r) * V + 16 * co + row];
  } else {
    for (int idx = tid; idx < CT * CT * 64; idx += NT) {
      const int ln = idx & 63, pc = idx >> 6, co = pc / CT, c = pc % CT;
      f4 x;
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = Wg[(16 * c + 4 * (ln >> 4) + r) * V + 16 * co + (ln & 15)];
      Wl[idx] = x;
    }
  }

  // the state of rows 16 w + i, columns 16 co + 4 g .. + 3
  const long long sbase = unit * K * V + (long long)(16 * w + row) * V + 4 * grp;
  f4 g[CT];
#pragma unroll
  for (int co = 0; co < CT; ++co)
    g[co] = a.H0 ? *reinterpret_cast<const f4*>(a.H0 + sbase + 16 * co) : f4{0.0f, 0.0f, 0.0f, 0.0f};

  // chunk staging: the 16 k rows, then q, then v are contiguous in memory and in
  // LDS, so one flat index of 16-byte pieces covers all three
  const float* kg = static_cast<const float*>(a.k) + unit * ld * K;
  const float* qg = static_cast<const float*>(a.q) + unit * ld * K;
  const float* vg = static_cast<const float*>(a.v) + unit * ld * V;
  const float* fg = static_cast<const float*>(a.f) + unit * ld;
  const int nk4 = 4 * K, n4 = 8 * K + 4 * V;  // 16-byte pieces: k (and q) per chunk, all
  f4 pre[kSlots];
  float pf = 0.0f;
  auto fetch = [&](int t0, int n) {  // steps t0 .. t0 + n - 1 into registers
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      int i = tid + j * NT;
      if (i < n4) {
        const float* src;
        int rw, rl;
        if (i < 2 * nk4) {
          const int ii = i < nk4 ? i : i - nk4;
          rw = ii / (K / 4);
          rl = ii - rw * (K / 4);
          src = (i < nk4 ? kg : qg) + (long long)(t0 + rw) * K + 4 * rl;
        } else {
          const int ii = i - 2 * nk4;
          rw = ii / (V / 4);
          rl = ii - rw * (V / 4);
          src = vg + (long long)(t0 + rw) * V + 4 * rl;
        }
        if (rw < n) pre[j] = *reinterpret_cast<const f4*>(src);
      }
    }
    if (tid < n) pf = fg[t0 + tid];
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const int i = tid + j * NT;
      if (i < n4) reinterpret_cast<f4*>(st)[i] = pre[j];
    }
    if (tid < kChunk) fs[tid] = pf;
  };

  if (Tb > 0) {
    fetch(0, min(kChunk, Tb));
    stage();
    if (Tb > kChunk) fetch(kChunk, min(kChunk, Tb - kChunk));
  }
  __syncthreads();  // W fragments and chunk 0 staged

  float* yg = a.y + unit * ld * V;
  for (int t0 = 0; t0 < Tb; t0 += kChunk) {
    const int n = min(kChunk, Tb - t0);
    for (int s = 0; s < n; ++s) {
      const float kr = ks[s * K + 16 * w + row];
      const float qr = qs[s * K + 16 * w + row];
      const float f = fs[s];
      const float omf = 1.0f - f;
      f4 acc[CT];
#pragma unroll
      for (int co = 0; co < CT; ++co) acc[co] = kr * *reinterpret_cast<const f4*>(vs + s * V + 16 * co + 4 * grp);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        f4 wf[CT];
#pragma unroll
        for (int co = 0; co < CT; ++co) {
          if constexpr (WREG)
            wf[co] = wreg[co * CT + c];
          else
            wf[co] = Wl[(co * CT + c) * 64 + lane];
        }
        // consecutive products go to different output tiles
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int co = 0; co < CT; ++co) acc[co] = mfma4(wf[co][r], g[c][r], acc[co]);
      }
#pragma unroll
      for (int co = 0; co < CT; ++co) {
        f4 p;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          g[co][r] = fmaf(f, g[co][r], omf * tanhf(acc[co][r]));
          p[r] = row_sum16(g[co][r] * qr);
        }
        if (row == 0) *reinterpret_cast<f4*>(yp + (w * kChunk + s) * V + 16 * co + 4 * grp) = p;
      }
    }
    __syncthreads();  // the chunk's partials are in LDS; every wave is done with the staged inputs
    for (int i = tid; i < n * (V / 4); i += NT) {
      const int s = i / (V / 4), c4 = i - s * (V / 4);
      f4 sum = *reinterpret_cast<const f4*>(yp + s * V + 4 * c4);
      for (int u = 1; u < NW; ++u) sum += *reinterpret_cast<const f4*>(yp + (u * kChunk + s) * V + 4 * c4);
      f4* dst = reinterpret_cast<f4*>(yg + (long long)(t0 + s) * V + 4 * c4);
      *dst = a.accumulate ? *dst + sum : sum;
    }
    if (t0 + kChunk < Tb) stage();
    __syncthreads();  // partials read, next chunk staged
    if (t0 + 2 * kChunk < Tb) fetch(t0 + 2 * kChunk, min(kChunk, Tb - t0 - 2 * kChunk));
  }

  if (a.HT) {
#pragma unroll
    for (int co = 0; co < CT; ++co) *reinterpret_cast<f4*>(a.HT + sbase + 16 * co) = g[co];
  }
}

template <int V>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  const int lds = Lds<V>::total_bytes(a.K);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(mfma_f32_fwd_kernel<V>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mfma_f32_fwd_kernel<V>, dim3((unsigned)((long long)a.B * a.H)), dim3(4 * a.K), lds, stream,
                     a);
  return hipGetLastError();
}

int lds_bytes(int K, int V) {
  switch (V) {
    case 16: return Lds<16>::total_bytes(K);
    case 32: return Lds<32>::total_bytes(K);
    case 48: return Lds<48>::total_bytes(K);
    case 64: return Lds<64>::total_bytes(K);
    case 80: return Lds<80>::total_bytes(K);
    case 96: return Lds<96>::total_bytes(K);
    case 112: return Lds<112>::total_bytes(K);
    case 128: return Lds<128>::total_bytes(K);
    default: return -1;
  }
}

}  // namespace

bool mfma_f32_supports(int K, int V) {
  return K >= 16 && K <= 128 && K % 16 == 0 && V >= 16 && V <= 128 && V % 16 == 0;
}

Plan plan_mfma_f32(int B, int H, int K, int V) {
  const long long units = (long long)B * H;
  if (!mfma_f32_supports(K, V) || units > 0x7fffffffLL) return Plan{-1, 0, 0, 0, 0, 0};
  return Plan{(int)units, 4 * K, K, 1, 0, lds_bytes(K, V)};
}

hipError_t launch_mfma_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.bf16 || a.saved || !a.y || !mfma_f32_supports(a.K, a.V) || (long long)a.B * a.H > 0x7fffffffLL)
    return hipErrorInvalidValue;
  if (a.lens && !a.accumulate) {  // rows past a sequence's length read as zero
    if (a.ld > 0 && a.ld != a.T) return hipErrorInvalidValue;  // a window of y: the caller clears it
    hipError_t e = fill_zero(a.y, (long long)a.B * a.H * a.T * a.V, stream);
    if (e != hipSuccess) return e;
  }
  switch (a.V) {
    case 16: return launch_t<16>(a, stream);
    case 32: return launch_t<32>(a, stream);
    case 48: return launch_t<48>(a, stream);
    case 64: return launch_t<64>(a, stream);
    case 80: return launch_t<80>(a, stream);
    case 96: return launch_t<96>(a, stream);
    case 112: return launch_t<112>(a, stream);
    case 128: return launch_t<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace m2rnn
