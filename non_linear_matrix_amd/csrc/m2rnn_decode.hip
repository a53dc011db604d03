// One step of the M²RNN recurrence for many units at once: the decoding step,
// latency-oriented (gist.science M²RNN technical summary, zh §2.1 update
// equations; readout y_t = H_t^T q_t):
//   Z = tanh(H W + k v^T),  H' = f H + (1 - f) Z,  y = H'^T q.
//
// With T = 1 there is nothing to pipeline over time: the work is one K x V
// state read from HBM, a (K, V, V) product, the elementwise update and the
// state written back, per unit. This kernel is built for throughput over units:
//   * one workgroup (4 waves) walks a contiguous range of batch rows of one
//     head; the head's W is read once, through LDS, into the waves' matrix
//     registers (permuted A fragments, as the multi-step kernel), and serves
//     every unit;
//   * a unit's K rows are 16-row tiles, one per wave at a time. The state tile
//     moves between HBM and the wave's LDS tile with whole-row accesses (each
//     load or store instruction covers whole rows of the tile) marked
//     non-temporal, since the state streams through once; and between LDS and
//     the registers in the output layout of
//     v_mfma_f32_16x16x32_bf16 (orientation D = W^T G^T: lane (g, n) holds row
//     n, columns 16 c + 4 g .. +3 of every 16-column tile c), whose registers
//     are the bf16 B fragments of the product through the permuted
//     contraction index;
//   * the state operand is split into bf16 hi + lo (two MFMA passes), ~16
//     significant bits: a decoding loop applies this step many times;
//   * the rank-1 term c k_n v_j is the accumulators' fp32 initial value;
//   * epilogue as the multi-step kernel: e = exp2(u), r = 1 / (1 + e),
//     G <- f G + a - 2 a r with G = c H, a = (1 - f) c, c = 2 / ln 2;
//   * the new state goes back through the LDS tile; each lane then holds whole
//     columns of it, stores them row by row, and sums its columns' readout
//     H'[i][j] q_i over the tile's 16 rows in row order; the tiles of a unit are
//     summed in LDS in a fixed order: deterministic, fp32 throughout.
// Two workgroups per CU (W in the matrix registers, 128 per wave at V = 128).
#include <hip/hip_runtime.h>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kMaxItems = 8;                   // 16-row tiles handled per workgroup iteration
constexpr int kBlocksPerCu = 2;

template <int V>
struct DecodeLayout {
  static constexpr int WROW = V + 8;           // bf16 per W staging row (padded)
  static constexpr int TROW = V + 4;           // floats per state-tile row (padded)
  static constexpr int WST_BYTES = V * WROW * 2;
  static constexpr int TILE_FLOATS = 16 * TROW;
  static constexpr int TILES_BYTES = 4 * TILE_FLOATS * 4;
  static constexpr int PART_OFF = WST_BYTES > TILES_BYTES ? WST_BYTES : TILES_BYTES;  // W staging is the prologue's only
  static constexpr int TOTAL = PART_OFF + 2 * kMaxItems * V * 4;
  // whole-row global accesses: lanes per row, rows per instruction, instructions per tile
  static constexpr int LPR = V / 4;
  static constexpr int RPI = 64 / LPR;
  static constexpr int NPC = 16 / RPI;
  static constexpr int CPL = V / 64;           // columns per lane in the column pass
};

template <int V>
__global__ __launch_bounds__(kThreads, kBlocksPerCu) void decode_kernel(FwdArgs a, int nsplit) {
  using L = DecodeLayout<V>;
  constexpr int CT = V / 16, KB = V / 32, WROW = L::WROW, TROW = L::TROW, CPL = L::CPL;
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];
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
  float* const tile = reinterpret_cast<float*>(lds) + w * L::TILE_FLOATS;
  float* const part_all = reinterpret_cast<float*>(lds + L::PART_OFF);

  // A fragment (c, b): lane (g, n) = W[32 b + 16 (j / 4) + 4 g + j % 4][16 c + n], j < 8,
  // kept in the matrix registers for the whole launch
  bf16x8 Wf[CT][KB];
  {
    unsigned short* wst = reinterpret_cast<unsigned short*>(lds);
    const u4* Wg = reinterpret_cast<const u4*>(static_cast<const unsigned short*>(a.W) + (long long)h * V * V);
    for (int i = tid; i < V * V / 8; i += kThreads)
      *reinterpret_cast<u4*>(wst + (i / (V / 8)) * WROW + 8 * (i % (V / 8))) = Wg[i];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        const unsigned short* src = wst + (32 * b + 4 * g + n / 4) * WROW + 16 * c + 4 * (n % 4);
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)src);
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * WROW));
        s8 wa = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        asm volatile("" : "=a"(wa) : "0"(wa));
        Wf[c][b] = __builtin_bit_cast(bf16x8, wa);
      }
    __syncthreads();  // the staging region becomes the waves' state tiles
  }
  // this lane's place in the whole-row accesses: row RPI p + rr, columns cc .. cc + 3
  const int rr = l / L::LPR, cc = 4 * (l % L::LPR);

  for (int it = 0, bb0 = b0; bb0 < b1; ++it, bb0 += upi) {
    float* const part = part_all + (it & 1) * kMaxItems * V;
    for (int i = w; i < items; i += 4) {
      const int bu = bb0 + i / tpu, rt = i % tpu;
      float* pdst = part + i * V;
      if (bu >= b1) continue;
      const long long unit = (long long)bu * a.H + h;
      const int row0 = 16 * rt;
      const int len = a.lens ? min(max(a.lens[bu], 0), 1) : 1;
      const float* H0t = a.H0 ? a.H0 + (unit * a.K + row0) * V : nullptr;
      float* HTt = a.HT ? a.HT + (unit * a.K + row0) * V : nullptr;
      // the state tile, whole rows per instruction
      f4 hw[L::NPC];
#pragma unroll
      for (int p = 0; p < L::NPC; ++p)
        hw[p] = H0t ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(H0t + (L::RPI * p + rr) * V + cc))
                    : f4{0, 0, 0, 0};
      if (len == 0) {  // empty sequence: H_T = H0 exactly, no readout
        if (HTt) {
#pragma unroll
          for (int p = 0; p < L::NPC; ++p)
            __builtin_nontemporal_store(hw[p], reinterpret_cast<f4*>(HTt + (L::RPI * p + rr) * V + cc));
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j) pdst[CPL * l + j] = 0.0f;
        continue;
      }
#pragma unroll
      for (int p = 0; p < L::NPC; ++p) *reinterpret_cast<f4*>(tile + (L::RPI * p + rr) * TROW + cc) = hw[p];
      __builtin_amdgcn_wave_barrier();
      f4 G[CT];  // lane (g, n): row n, columns 16 c + 4 g .. +3, scaled by c
#pragma unroll
      for (int c = 0; c < CT; ++c) G[c] = *reinterpret_cast<const f4*>(tile + n * TROW + 16 * c + 4 * g) * kC;
      const long long srow = unit * ld;  // this unit's (only) step
      const float ck = kC * bf16_to_f32(kin[srow * a.K + row0 + n]);
      const float fg = bf16_to_f32(fin[srow]);
      const float av = (1.0f - fg) * kC, m2a = -2.0f * av;
      // q of the tile's 16 rows, for the column pass
      const u4 q0 = *reinterpret_cast<const u4*>(qin + srow * a.K + row0);
      const u4 q1 = *reinterpret_cast<const u4*>(qin + srow * a.K + row0 + 8);
      // rank-1 term as the initial accumulators: acc[c][i] = c k_row v[16 c + 4 g + i]
      f4 acc[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const u2 vv = *reinterpret_cast<const u2*>(vin + srow * V + 16 * c + 4 * g);
        acc[c] = f4{ck * bf16_to_f32(vv[0] & 0xffffu), ck * bf16_to_f32(vv[0] >> 16),
                    ck * bf16_to_f32(vv[1] & 0xffffu), ck * bf16_to_f32(vv[1] >> 16)};
      }
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
        for (int c = 0; c < CT; ++c) acc[c] = mfma(Wf[c][b], hi, acc[c]);
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c] = mfma(Wf[c][b], lo, acc[c]);
      }
      // update, new state back into the LDS tile
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        f4 hn;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float e = __builtin_amdgcn_exp2f(acc[c][i4]);
          const float rr2 = __builtin_amdgcn_rcpf(1.0f + e);
          hn[i4] = fmaf(m2a, rr2, fmaf(fg, G[c][i4], av)) * kInvC;
        }
        *reinterpret_cast<f4*>(tile + n * TROW + 16 * c + 4 * g) = hn;
      }
      __builtin_amdgcn_wave_barrier();
      // column pass: lane l holds columns CPL l .. +CPL-1 of every row; stores
      // whole rows, and sums the readout over the 16 rows in row order
      float ys[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) ys[j] = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const unsigned int qp = (r < 8 ? q0 : q1)[(r % 8) / 2];
        const float qv = bf16_to_f32((r % 2) ? qp >> 16 : qp & 0xffffu);
        if constexpr (CPL == 2) {
          const f2 hv = *reinterpret_cast<const f2*>(tile + r * TROW + 2 * l);
          if (HTt) __builtin_nontemporal_store(hv, reinterpret_cast<f2*>(HTt + r * V + 2 * l));
          ys[0] = fmaf(hv[0], qv, ys[0]);
          ys[1] = fmaf(hv[1], qv, ys[1]);
        } else {
          const float hv = tile[r * TROW + l];
          if (HTt) __builtin_nontemporal_store(hv, HTt + r * V + l);
          ys[0] = fmaf(hv, qv, ys[0]);
        }
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) pdst[CPL * l + j] = ys[j];
      // the next tile's first LDS write follows these reads in the wave's order
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // y of this iteration's units: the tiles' partials in a fixed order
    if (a.y) {
      for (int t = tid; t < upi * V; t += kThreads) {
        const int uo = t / V, col = t % V, bu = bb0 + uo;
        if (bu >= b1) continue;
        float s = 0.0f;
        for (int rt = 0; rt < tpu; ++rt) s += part[(uo * tpu + rt) * V + col];
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
  // two workgroups per CU (256 CUs) over the heads, at least one batch row each
  long long s = (256 * kBlocksPerCu + H - 1) / H;
  if (s > B) s = B;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

Plan plan_decode(int B, int H, int K, int V) {
  const long long grid = (long long)H * decode_splits(B, H);
  const int lds = V == 128 ? DecodeLayout<128>::TOTAL : DecodeLayout<64>::TOTAL;
  return Plan{grid > 0x7fffffffLL ? -1 : (int)grid, kThreads, 16, K / 16, 0, lds};
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
