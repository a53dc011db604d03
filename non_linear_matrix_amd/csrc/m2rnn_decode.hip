// One step of the M²RNN recurrence for many units at once: the decoding step,
// latency-oriented (gist.science M²RNN technical summary, zh §2.1 update
// equations; readout y_t = H_t^T q_t):
//   Z = tanh(H W + k v^T),  H' = f H + (1 - f) Z,  y = H'^T q.
//
// With T = 1 there is nothing to pipeline over time: the work is one K x V
// state read from HBM, a (K, V, V) product, the elementwise update and the
// state written back, per unit. The multi-step kernel's per-workgroup set-up
// (a 156 KB LDS layout, chunk staging, one workgroup per CU) would dominate, so
// this kernel is built for throughput over units instead:
//   * one workgroup (4 waves) walks a contiguous range of batch rows of one
//     head, so the head's W is staged into LDS once and serves every unit;
//   * a unit's K rows are 16-row tiles, one per wave at a time; a wave reads its
//     tile from HBM straight into the output layout of v_mfma_f32_16x16x32_bf16
//     (orientation D = W^T G^T, as the multi-step kernel: lane (g, n) holds row
//     n, columns 16 c + 4 g .. +3 of every 16-column tile c), so the same
//     registers are the bf16 B fragments of the product, through a permuted
//     contraction index in W's fragments (read from LDS with transposing reads);
//   * the state operand is split into bf16 hi + lo (two MFMA passes), ~16
//     significant bits: a decoding loop applies this step many times;
//   * the rank-1 term c k_n v_j is the accumulators' fp32 initial value;
//   * epilogue as the multi-step kernel: e = exp2(u), r = 1 / (1 + e),
//     G <- f G + a - 2 a r with G = c H, a = (1 - f) c, c = 2 / ln 2;
//   * readout: each lane's products H'[n][j] q_n summed over the 16 rows of the
//     tile with four DPP steps inside each 16-lane row, the tiles of a unit
//     summed in LDS in a fixed order: deterministic, fp32 throughout.
// Three workgroups per CU (LDS 43 KB, 128 VGPRs each) keep enough state reads in flight.
#include <hip/hip_runtime.h>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kMaxItems = 8;                   // 16-row tiles handled per workgroup iteration

template <int V>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(FwdArgs a, int nsplit) {
  constexpr int CT = V / 16, KB = V / 32, WROW = V + 8;
  __shared__ __attribute__((aligned(16))) unsigned short wst[V * WROW];
  __shared__ __attribute__((aligned(16))) float part[2][kMaxItems * V];
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64, g = l / 16, n = l % 16;
  const int h = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
  const int tpu = a.K / 16;                        // tiles per unit
  const int upi = tpu >= 4 ? 1 : 4 / tpu;          // units per iteration
  const int items = upi * tpu;
  const int b0 = static_cast<int>((long long)a.B * split / nsplit);
  const int b1 = static_cast<int>((long long)a.B * (split + 1) / nsplit);
  const long long ld = a.ld > 0 ? a.ld : a.T;      // row stride (in steps) of k, v, q, f, y
  const unsigned short* kin = static_cast<const unsigned short*>(a.k);
  const unsigned short* qin = static_cast<const unsigned short*>(a.q);
  const unsigned short* vin = static_cast<const unsigned short*>(a.v);
  const unsigned short* fin = static_cast<const unsigned short*>(a.f);

  {  // the head's W, row-major with padded rows
    const u4* Wg = reinterpret_cast<const u4*>(static_cast<const unsigned short*>(a.W) + (long long)h * V * V);
    for (int i = tid; i < V * V / 8; i += kThreads)
      *reinterpret_cast<u4*>(wst + (i / (V / 8)) * WROW + 8 * (i % (V / 8))) = Wg[i];
  }
  __syncthreads();
  // A fragment (c, b): lane (g, n) = W[32 b + 16 (j / 4) + 4 g + j % 4][16 c + n], j < 8
  auto wfrag = [&](int c, int b) {
    const unsigned short* src = wst + (32 * b + 4 * g + n / 4) * WROW + 16 * c + 4 * (n % 4);
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)src);
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * WROW));
    return __builtin_bit_cast(bf16x8, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };

  for (int it = 0, bb0 = b0; bb0 < b1; ++it, bb0 += upi) {
    const int par = it & 1;
    for (int i = w; i < items; i += 4) {
      const int bu = bb0 + i / tpu, rt = i % tpu;
      float* pdst = &part[par][i * V];
      if (bu >= b1) continue;
      const long long unit = (long long)bu * a.H + h;
      const int row = 16 * rt + n;
      const int len = a.lens ? min(max(a.lens[bu], 0), 1) : 1;
      // this lane's state values: row `row`, columns 16 c + 4 g .. +3
      f4 hv[CT];
      const float* H0 = a.H0 ? a.H0 + (unit * a.K + row) * V + 4 * g : nullptr;
#pragma unroll
      for (int c = 0; c < CT; ++c) hv[c] = H0 ? *reinterpret_cast<const f4*>(H0 + 16 * c) : f4{0, 0, 0, 0};
      float* HT = a.HT ? a.HT + (unit * a.K + row) * V + 4 * g : nullptr;
      if (len == 0) {  // empty sequence: H_T = H0 exactly, no readout
        if (HT) {
#pragma unroll
          for (int c = 0; c < CT; ++c) *reinterpret_cast<f4*>(HT + 16 * c) = hv[c];
        }
        if (n == 0) {
#pragma unroll
          for (int c = 0; c < CT; ++c) *reinterpret_cast<f4*>(pdst + 16 * c + 4 * g) = f4{0, 0, 0, 0};
        }
        continue;
      }
      const long long srow = unit * ld;  // this unit's (only) step
      const float ck = kC * bf16_to_f32(kin[srow * a.K + row]);
      const float qn = bf16_to_f32(qin[srow * a.K + row]);
      const float fg = bf16_to_f32(fin[srow]);
      const float av = (1.0f - fg) * kC, m2a = -2.0f * av;
      // rank-1 term as the initial accumulators: acc[c][i] = c k_row v[16 c + 4 g + i]
      f4 acc[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const u2 vv = *reinterpret_cast<const u2*>(vin + srow * V + 16 * c + 4 * g);
        acc[c] = f4{ck * bf16_to_f32(vv[0] & 0xffffu), ck * bf16_to_f32(vv[0] >> 16),
                    ck * bf16_to_f32(vv[1] & 0xffffu), ck * bf16_to_f32(vv[1] >> 16)};
      }
      f4 G[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) G[c] = hv[c] * kC;
      // products with the operand blocks (tiles 2b, 2b+1) as bf16 hi + lo
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        f8 x;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) { x[i4] = G[2 * b][i4]; x[4 + i4] = G[2 * b + 1][i4]; }
        const bf16x8 hi = __builtin_convertvector(x, bf16x8);
        const u4 hb = __builtin_bit_cast(u4, hi);
        f8 r;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          r[2 * p] = x[2 * p] - __uint_as_float(hb[p] << 16);
          r[2 * p + 1] = x[2 * p + 1] - __uint_as_float(hb[p] & 0xffff0000u);
        }
        const bf16x8 lo = __builtin_convertvector(r, bf16x8);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const bf16x8 wf = wfrag(c, b);
          acc[c] = mfma(wf, hi, acc[c]);
          acc[c] = mfma(wf, lo, acc[c]);
        }
      }
      // update, new state out, readout partial over the tile's 16 rows
      f4 ys[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        f4 hn;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float e = __builtin_amdgcn_exp2f(acc[c][i4]);
          const float rr = __builtin_amdgcn_rcpf(1.0f + e);
          hn[i4] = fmaf(m2a, rr, fmaf(fg, G[c][i4], av)) * kInvC;
        }
        if (HT) *reinterpret_cast<f4*>(HT + 16 * c) = hn;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) ys[c][i4] = row_sum16(hn[i4] * qn);
      }
      if (n == 0) {
#pragma unroll
        for (int c = 0; c < CT; ++c) *reinterpret_cast<f4*>(pdst + 16 * c + 4 * g) = ys[c];
      }
    }
    __syncthreads();
    // y of this iteration's units: the tiles' partials in a fixed order
    if (a.y) {
      for (int t = tid; t < upi * V; t += kThreads) {
        const int uo = t / V, col = t % V, bu = bb0 + uo;
        if (bu >= b1) continue;
        float s = 0.0f;
        for (int rt = 0; rt < tpu; ++rt) s += part[par][(uo * tpu + rt) * V + col];
        float* dst = a.y + ((long long)bu * a.H + h) * ld * V + col;
        *dst = a.accumulate ? *dst + s : s;
      }
    }
    // the next iteration writes the other partial buffer; this one is rewritten
    // only after the next barrier, which every thread reaches after its sums
  }
}

}  // namespace

bool decode_supports(const FwdArgs& a) {
  return a.T == 1 && a.saved == nullptr && a.bf16 && (a.V == 64 || a.V == 128) &&
         (a.K == 32 || a.K == 64 || a.K == 128);
}

int decode_splits(int B, int H) {
  // about three workgroups per CU (256 CUs; LDS allows three) over the heads,
  // at least one batch row each
  long long s = (768 + H - 1) / H;
  if (s > B) s = B;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

hipError_t launch_decode(const FwdArgs& a, hipStream_t stream) {
  if (!decode_supports(a)) return hipErrorInvalidValue;
  const int ns = decode_splits(a.B, a.H);
  const long long grid = (long long)a.H * ns;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.V == 128)
    hipLaunchKernelGGL(decode_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a, ns);
  else
    hipLaunchKernelGGL(decode_kernel<64>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a, ns);
  return hipGetLastError();
}

}  // namespace m2rnn
