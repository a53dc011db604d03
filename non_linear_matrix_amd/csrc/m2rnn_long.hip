// M²RNN forward recurrence, latency-oriented variant for workloads with few
// 16-row tiles (small batch x heads, long sequences), on gfx950 matrix cores.
//
// Same computation as the multi-step kernel (gist.science M²RNN technical
// summary, zh §2.1 update equations; readout y_t = H_t^T q_t):
//   Z_t = tanh(H_{t-1} W + k_t v_t^T),  H_t = f_t H_{t-1} + (1 - f_t) Z_t.
//
// The multi-step kernel gives each 16-row tile to one wave, so a step costs one
// wave's whole product and epilogue (~1900 cycles at V = 128) and a workload
// with fewer tiles than the GPU has SIMDs leaves most of them idle. Here a tile
// is one workgroup of V/32 waves, each owning 32 columns (two 16-column output
// tiles, one 32-wide contraction block), or at V = 64 of V/16 waves, each
// owning one 16-column output tile (half a block):
//   * a wave's products are its two output tiles against all V/32 operand
//     blocks (W^T fragments of its columns only, in AGPRs); the epilogue covers
//     its 8 elements per lane;
//   * after the epilogue each wave writes its bf16 operand block (and the low
//     half with SPLIT) into a shared LDS state tile; one LDS barrier; each wave
//     reads the other blocks back as its next B fragments. The next step's
//     rank-1 term and the wave's own block are multiplied before the barrier;
//   * the state layout, the permuted contraction index, the scaled state
//     G = c H (c = 2 / ln 2), the rank-1 MFMA and the epilogue are those of the
//     multi-step kernel, so both give the same rounding per step;
//   * readout: the shared bf16 state tiles come back through transposing LDS
//     reads, one MFMA per 16 columns per step pair against q; every 16 steps a
//     wave adds its columns' sums over the tile's 16 rows into y with atomic
//     adds. The K/16 row tiles of a unit are separate workgroups, so y receives
//     K/16 contributions per element in an order that varies between runs. Each
//     contribution is first rounded to a grid of spacing 2^(E_t - 23), where
//     2^E_t bounds |y_t| from quantities every workgroup of the unit computes
//     identically: ||q_t||_1 over all K rows times M, a bound on |H_t| that the
//     gated convex update gives (|tanh| <= 1, so M_t = f_t M_{t-1} + 1 - f_t
//     from M_0 = max(1, max |H0|) bounds it; M_t never grows, so the bound at a
//     chunk's start serves all its steps). Every sum of such values is a
//     multiple of the spacing below 2^(E_t + 1), so it is exact in fp32 and the
//     order of the adds cannot change y (onto a cleared y). The grid adds at
//     most 2^-23 ||q_t||_1 M per row tile to an element's error.
// Inputs k, v, q, f are staged per 16-step chunk into LDS (two stage buffers),
// fetched from HBM a chunk ahead.
#include <hip/hip_runtime.h>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

using namespace dev;

constexpr int kChunk = 16;

// GRID: the y grid of the plain forward (the training forward keeps its y adds
// unrounded and stages only its own rows of q, which keeps it within the
// registers of two workgroups per CU).
// TW: 16-column output tiles per wave (2: V/32 waves, each owning a 32-wide
// contraction block; 1: V/16 waves, two per block, so a step's epilogue and
// products are split over twice the waves).
template <int V, bool GRID, int TW = 2>
struct LongLayout {
  static_assert(TW == 1 || TW == 2, "one or two output tiles per wave");
  static constexpr int S = V / (16 * TW);  // waves per workgroup
  static constexpr int CT = V / 16;       // 16-column tiles
  static constexpr int THREADS = 64 * S;
  static constexpr int HROW = V + 8;      // bf16 per state-tile row (padded)
  // dwords per (step, column-in-tile) of rank-1 A records: one (v, v) pair per
  // column tile, padded by two so that the 16 rows a 16-lane group reads fall
  // on distinct banks
  static constexpr int NVX = CT + 2;
  // state-tile slots, for the high and for the low halves: the readout of the
  // step pair (s - 1, s) runs after step s's barrier, and the next write into
  // step s - 1's slot, at step s + 3, comes two barriers later
  static constexpr int NHS = 4;
  static constexpr int KX_BYTES = 2 * kChunk * 16 * 4;
  static constexpr int QS_BYTES = 2 * kChunk * 16 * 2;
  static constexpr int FS_BYTES = 2 * kChunk * 4 * 4;
  static constexpr int VX_BYTES = 2 * kChunk * 16 * NVX * 4;
  static constexpr int XB_BYTES = NHS * 16 * HROW * 2;
  static constexpr int XL_BYTES = NHS * 16 * HROW * 2;
  static constexpr int KX_OFF = 0;
  static constexpr int QS_OFF = KX_OFF + KX_BYTES;
  static constexpr int FS_OFF = QS_OFF + QS_BYTES;
  static constexpr int VX_OFF = FS_OFF + FS_BYTES;
  static constexpr int XB_OFF = VX_OFF + VX_BYTES;
  static constexpr int XL_OFF = XB_OFF + XB_BYTES;
  static constexpr int YS_ROW = 33;       // floats per row of a wave's y transpose tile
  static constexpr int YS_BYTES = S * 16 * YS_ROW * 4;
  static constexpr int YS_OFF = XL_OFF + XL_BYTES;
  // the y-grid inputs of the last four staged chunks (index chunk & 3): ||q_t||_1
  // over all K rows per step, and the state bound M for the chunk's steps
  static constexpr int YB_SLOTS = 4;
  static constexpr int YB_PER = kChunk + 4;
  static constexpr int YB_BYTES = YB_SLOTS * YB_PER * 4;
  static constexpr int YB_OFF = YS_OFF + YS_BYTES;
  static constexpr int Z_OFF = YB_OFF + YB_BYTES;
  static constexpr int TOTAL = Z_OFF + 16;
  static_assert(V * HROW * 2 <= VX_BYTES + XB_BYTES + XL_BYTES,
                "W fits in the rank-1 and state-tile regions during the prologue");
  static_assert(2 * TOTAL <= 160 * 1024, "two workgroups per CU");
  // 16-byte global pieces of one chunk: k of the tile's 16 rows, q of them
  // (without GRID), v
  static constexpr int P_K = kChunk * 2;
  static constexpr int P_Q = GRID ? 0 : kChunk * 2;
  static constexpr int P_V = kChunk * V / 8;
  static constexpr int PIECES = P_K + P_Q + P_V;
  static constexpr int PPT = (PIECES + THREADS - 1) / THREADS;
  // GRID: q of every row (K <= 128: 16 pieces per step), its own registers. Piece
  // i = tid + j THREADS is step i / 16, part i % 16, so a step's pieces fill one
  // 16-lane DPP row.
  // (with more than 256 threads the first 256 take one piece each)
  static constexpr int QPT = GRID ? (kChunk * 16 + THREADS - 1) / THREADS : 0;
  static_assert(!GRID || QPT * THREADS == kChunk * 16 || (QPT == 1 && THREADS % (kChunk * 16) == 0),
                "whole q pieces per thread");
};

// Product over the 16 lanes of a DPP row; every lane of the row ends with it
// (each stage multiplies a lane by its partner: x y and y x are the same float).
__device__ __forceinline__ float row_prod16(float x) {
  x *= __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // lane ^ 1
  x *= __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // lane ^ 2
  x *= __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // half mirror
  x *= __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // mirror
  return x;
}

// One chunk of per-step inputs for the tile's 16 rows: loaded to registers, then
// stored into a stage buffer in the forms the MFMAs read.
// F16: q is staged as fp16 (the readout's operand type)
template <int V, bool GRID, bool F16 = false, int TW = 2>
struct LongStager {
  using L = LongLayout<V, GRID, TW>;
  // 8 staged q values (bf16 bit patterns) as stored in LDS
  static __device__ __forceinline__ u4 q_out(const u4& r) {
    if constexpr (F16) return __builtin_bit_cast(u4, bf16x8_to_f16(__builtin_bit_cast(s8, r)));
    return r;
  }
  u4 reg[L::PPT];
  u4 qreg[L::QPT > 0 ? L::QPT : 1];
  unsigned short freg;

  __device__ __forceinline__ void load(const FwdArgs& a, long long unit, int row0, int chunk, int Tb,
                                       long long ld) {
    const int tid = threadIdx.x;
    const int t0 = chunk * kChunk;
    const unsigned short* k = static_cast<const unsigned short*>(a.k);
    const unsigned short* q = static_cast<const unsigned short*>(a.q);
    const unsigned short* v = static_cast<const unsigned short*>(a.v);
    const unsigned short* f = static_cast<const unsigned short*>(a.f);
#pragma unroll
    for (int p = 0; p < L::PPT; ++p) {
      const int slot = tid + p * L::THREADS;
      reg[p] = u4{0, 0, 0, 0};
      if (slot < L::P_K + L::P_Q) {
        const bool isq = slot >= L::P_K;
        const int s2 = isq ? slot - L::P_K : slot;
        const int s = s2 / 2, part = s2 % 2, t = t0 + s;
        if (t < Tb) reg[p] = *reinterpret_cast<const u4*>((isq ? q : k) + (unit * ld + t) * a.K + row0 + 8 * part);
      } else if (slot < L::PIECES) {
        const int s2 = slot - L::P_K - L::P_Q;
        const int s = s2 / (V / 8), part = s2 % (V / 8), t = t0 + s;
        if (t < Tb) reg[p] = *reinterpret_cast<const u4*>(v + (unit * ld + t) * V + 8 * part);
      }
    }
    if constexpr (GRID) {
#pragma unroll
      for (int j = 0; j < L::QPT; ++j) {
        const int i = tid + j * L::THREADS, t = t0 + i / 16, col = 8 * (i % 16);
        qreg[j] = u4{0, 0, 0, 0};
        if (i < kChunk * 16 && t < Tb && col < a.K)
          qreg[j] = *reinterpret_cast<const u4*>(q + (unit * ld + t) * a.K + col);
      }
    }
    freg = 0x3f80u;  // gate 1 past the end: the padding steps keep the state
    if (tid < kChunk && t0 + tid < Tb) freg = f[unit * ld + t0 + tid];
  }

  // Publish chunk `chunk` into stage buffer chunk & 1, and with GRID its y-grid
  // inputs into slot chunk & 3: ||q_t||_1 per step (each step's 16 pieces summed
  // over one DPP row in a fixed order) and the state bound M for the chunk's
  // steps; m carries the bound from chunk to chunk (wave 0). Every workgroup of
  // the unit computes the same values.
  __device__ __forceinline__ void store(char* lds, int chunk, int row0, float& m) const {
    const int tid = threadIdx.x;
    const int buf = chunk & 1;
    float* yb = reinterpret_cast<float*>(lds + L::YB_OFF) + (chunk & (L::YB_SLOTS - 1)) * L::YB_PER;
    if constexpr (GRID) {
    unsigned short* qsg = reinterpret_cast<unsigned short*>(lds + L::QS_OFF) + buf * kChunk * 16;
#pragma unroll
    for (int j = 0; j < L::QPT; ++j) {
      const int i = tid + j * L::THREADS, st = i / 16, own = i % 16 - row0 / 8;
      if (i >= kChunk * 16) break;  // whole waves past the chunk's pieces
      float qa = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        qa += fabsf(bf16_to_f32(qreg[j][d] & 0xffffu)) + fabsf(bf16_to_f32(qreg[j][d] >> 16));
      qa = row_sum16(qa);
      if (i % 16 == 0) yb[st] = qa;
      // the tile's own rows are the readout's q
      if (own == 0 || own == 1) *reinterpret_cast<u4*>(qsg + st * 16 + 8 * own) = q_out(qreg[j]);
    }
    if (tid < 64) {
      // M_t - 1 = f_t (M_{t-1} - 1) and M >= 1, so M is non-increasing: the bound
      // at the chunk's start holds for all its steps, and after the chunk it is
      // 1 + (f_0 ... f_15)(M - 1). The product runs over the DPP row of lanes
      // 0 .. 15, which hold the chunk's gates (1 past the sequence's end).
      float pf = row_prod16(bf16_to_f32(freg));
      pf = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pf), 0));
      if (tid == 0) yb[kChunk] = m;
      m = fmaf(pf, m - 1.0f, 1.0f);
    }
    }
    unsigned int* kx = reinterpret_cast<unsigned int*>(lds + L::KX_OFF) + buf * kChunk * 16;
    unsigned short* qs = reinterpret_cast<unsigned short*>(lds + L::QS_OFF) + buf * kChunk * 16;
    float* fs = reinterpret_cast<float*>(lds + L::FS_OFF) + buf * kChunk * 4;
    unsigned int* vx = reinterpret_cast<unsigned int*>(lds + L::VX_OFF) + buf * kChunk * 16 * L::NVX;
#pragma unroll
    for (int p = 0; p < L::PPT; ++p) {
      const int slot = tid + p * L::THREADS;
      const u4 r = reg[p];
      if (slot < L::P_K) {
        const int s = slot / 2, part = slot % 2;
        // c k as a (hi, lo) bf16 pair per row: the rank-1 MFMA's B operand
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float ck0 = kC * bf16_to_f32(r[d] & 0xffffu), ck1 = kC * bf16_to_f32(r[d] >> 16);
          const unsigned int hp = pack_bf16(ck0, ck1);
          const unsigned int lp = pack_bf16(ck0 - __uint_as_float(hp << 16), ck1 - __uint_as_float(hp & 0xffff0000u));
          kx[s * 16 + 8 * part + 2 * d] = (hp & 0xffffu) | (lp << 16);
          kx[s * 16 + 8 * part + 2 * d + 1] = (hp >> 16) | (lp & 0xffff0000u);
        }
      } else if (slot < L::P_K + L::P_Q) {
        const int s2 = slot - L::P_K, s = s2 / 2, part = s2 % 2;
        *reinterpret_cast<u4*>(qs + s * 16 + 8 * part) = q_out(r);
      } else if (slot < L::PIECES) {
        const int s2 = slot - L::P_K - L::P_Q;
        const int s = s2 / (V / 8), part = s2 % (V / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int col = 8 * part + i;
          const unsigned int raw = (r[i / 2] >> (16 * (i % 2))) & 0xffffu;
          const int tile = col / 16;
          vx[(s * 16 + col % 16) * L::NVX + tile] = raw | (raw << 16);
        }
      }
    }
    if (tid < kChunk) {
      const float fg = bf16_to_f32(freg);
      const float av = (1.0f - fg) * kC;
      fs[tid * 4 + 0] = fg;
      fs[tid * 4 + 1] = av;
      fs[tid * 4 + 2] = -2.0f * av;
      fs[tid * 4 + 3] = 0.0f;
    }
  }
};

template <int V, bool SPLIT, bool SAVE, bool F16, int TW>
__global__ __launch_bounds__(64 * V / (16 * TW), 1) void mfma_fwd_long_kernel(FwdArgs a) {
  constexpr bool GRID = !SAVE;
  static_assert(TW == 2 || !SAVE, "the saving forward keeps two tiles per wave (whole saved blocks)");
  // the state operand's type: bf16, or fp16 (F16: one operand, no saved data)
  static_assert(!F16 || (!SPLIT && !SAVE), "the fp16 operand is a single-operand forward");
  using Op = std::conditional_t<F16, f16x8, bf16x8>;
  using L = LongLayout<V, GRID, TW>;
  static_assert(L::THREADS == 64 * V / (16 * TW), "launch bounds");
  constexpr int KB = V / 32, HROW = L::HROW, NHS = L::NHS;
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];

  const int tid = threadIdx.x;
  const int w = tid / 64, l = tid % 64, g = l / 16, n = l % 16;
  const int tiles = a.K / 16;
  const long long unit = blockIdx.x / tiles;
  const int row0 = (blockIdx.x % tiles) * 16;
  const int h = static_cast<int>(unit % a.H);
  const int T = a.T;
  const long long LD = a.ld > 0 ? a.ld : a.T;
  const int Tb = a.lens ? min(max(a.lens[unit / a.H], 0), T) : T;
  const int nchunks = (Tb + kChunk - 1) / kChunk;
  const int my_row = row0 + n;
  // this wave's output tiles TW w .. TW w + TW - 1, in contraction block ob (with
  // TW = 1, half hw of it)
  const int ob = TW * w / 2, hw = TW == 1 ? w % 2 : 0;

  unsigned short* xb = reinterpret_cast<unsigned short*>(lds + L::XB_OFF);
  unsigned short* xl = reinterpret_cast<unsigned short*>(lds + L::XL_OFF);
  const unsigned int* kx_all = reinterpret_cast<const unsigned int*>(lds + L::KX_OFF);
  const unsigned short* qs_all = reinterpret_cast<const unsigned short*>(lds + L::QS_OFF);
  const float* fs_all = reinterpret_cast<const float*>(lds + L::FS_OFF);
  const unsigned int* vx_all = reinterpret_cast<const unsigned int*>(lds + L::VX_OFF);
  const unsigned int* zero_lds = reinterpret_cast<const unsigned int*>(lds + L::Z_OFF);

  // ---- prologue: chunk 0/1 inputs, W, H0 requested before the first wait
  LongStager<V, GRID, F16, TW> st, st1;
  st.load(a, unit, row0, 0, Tb, LD);
  if (nchunks > 1) st1.load(a, unit, row0, 1, Tb, LD);
  constexpr int WLOADS = V * V / 8 / L::THREADS;
  static_assert(WLOADS * 8 * L::THREADS == V * V, "W splits evenly");
  u4 wreg[WLOADS];
  {
    const u4* Wg = reinterpret_cast<const u4*>(static_cast<const unsigned short*>(a.W) + (long long)h * V * V);
#pragma unroll
    for (int p = 0; p < WLOADS; ++p) wreg[p] = Wg[tid + p * L::THREADS];
  }
  // the y grid's state bound M_0 = max(1, max |H0|) over the unit's whole H0
  // (every workgroup of the unit reads all of it: max does not round, so all
  // get the same value); four loads in flight per thread
  float hmax = 0.0f;
  if (GRID && a.H0 && a.y) {
    const f4* h0u = reinterpret_cast<const f4*>(a.H0 + unit * a.K * V);
    const int n4 = a.K * V / 4;
    for (int i = tid; i < n4; i += 4 * L::THREADS) {
      f4 hv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) hv[u] = i + u * L::THREADS < n4 ? h0u[i + u * L::THREADS] : f4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        hmax = fmaxf(hmax, fmaxf(fmaxf(fabsf(hv[u][0]), fabsf(hv[u][1])), fmaxf(fabsf(hv[u][2]), fabsf(hv[u][3]))));
    }
  }
  float* const ybt = reinterpret_cast<float*>(lds + L::YB_OFF);
  if constexpr (GRID) {
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) hmax = fmaxf(hmax, __shfl_xor(hmax, off));
    if (l == 0) ybt[w] = hmax;  // read after the W-staging barrier below
  }
  f4 G[TW];  // own output tiles TW w + j: lane (g, n) holds G[n][16 c + 4 g + i]
  {
    const float* H0 = a.H0 ? a.H0 + (unit * a.K + my_row) * V : nullptr;
#pragma unroll
    for (int j = 0; j < TW; ++j)
      G[j] = H0 ? *reinterpret_cast<const f4*>(H0 + 16 * (TW * w + j) + 4 * g) * kC : f4{0, 0, 0, 0};
    if constexpr (F16) {
      // an initial state beyond the fp16 operand's range is NaN from the start;
      // with gates in [0, 1] the state never grows past max(1, max |H0|) after it
#pragma unroll
      for (int j = 0; j < TW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) G[j][i] = f16_range_or_nan(G[j][i]);
    }
  }
  // W^T fragments of this wave's output tiles, every contraction block, via
  // LDS. Register arrays over the blocks are indexed o = 0 .. KB - 1 for block
  // (ob + o) mod KB (o = 0: the wave's own block), so that every register index
  // is a compile-time constant; only LDS addresses depend on the wave.
  Op Wf[TW][KB];
  {
    unsigned short* wst = reinterpret_cast<unsigned short*>(lds + L::VX_OFF);
#pragma unroll
    for (int p = 0; p < WLOADS; ++p) {
      const int i = tid + p * L::THREADS;
      *reinterpret_cast<u4*>(wst + (i / (V / 8)) * HROW + 8 * (i % (V / 8))) = wreg[p];
    }
    __syncthreads();
    if constexpr (GRID)
      for (int ww = 0; ww < L::S; ++ww) hmax = fmaxf(hmax, ybt[ww]);
#pragma unroll
    for (int j = 0; j < TW; ++j)
#pragma unroll
      for (int o = 0; o < KB; ++o) {
        const int c = TW * w + j, b = (ob + o) % KB;
        const unsigned short* src = wst + (32 * b + 4 * g + n / 4) * HROW + 16 * c + 4 * (n % 4);
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)src);
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * HROW));
        s8 wa = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (F16) wa = __builtin_bit_cast(s8, bf16x8_to_f16(wa));
        asm volatile("" : "=a"(wa) : "0"(wa));
        Wf[j][o] = __builtin_bit_cast(Op, wa);
      }
    lds_barrier();  // the regions are the rank-1 stage buffers and state tiles from here on
  }
  // zeroed state-tile slots: the readout of an odd final step multiplies a slot
  // that step never wrote (by zero q), which must not hold NaN patterns
  for (int i = tid; i < (L::XB_BYTES + L::XL_BYTES) / 4; i += L::THREADS)
    reinterpret_cast<unsigned int*>(lds + L::XB_OFF)[i] = 0u;
  // LDS init: the zero word; chunks 0, 1
  if (tid < 4) reinterpret_cast<unsigned int*>(lds + L::Z_OFF)[tid] = 0u;
  // the y grid's state bound: after the last staged chunk (wave 0), and per step
  // of that chunk (lanes 0 .. 15)
  float mbound = fmaxf(1.0f, hmax);
  if (nchunks > 0) st.store(lds, 0, row0, mbound);
  if (nchunks > 1) st1.store(lds, 1, row0, mbound);
  if (nchunks > 2) st.load(a, unit, row0, 2, Tb, LD);

  // operand blocks: Bf[o] lane (g, n) = bf16 G[n][32 b + 16 (j / 4) + 4 g + j % 4],
  // b = (ob + o) mod KB. With TW = 1 the wave makes half of its own block (its
  // tile's four elements, in the other half zeros that are never stored) and
  // reads every block, its own included, back after the exchange.
  Op Bf[KB], Bl[KB];
  auto make_own = [&]() {
    f8 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = G[0][i]; x[4 + i] = TW == 2 ? G[TW - 1][i] : 0.0f; }
    Bf[0] = __builtin_convertvector(x, Op);
    if constexpr (SPLIT) {
      const u4 hb = __builtin_bit_cast(u4, Bf[0]);
      f8 r;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        r[2 * p] = x[2 * p] - __uint_as_float(hb[p] << 16);
        r[2 * p + 1] = x[2 * p + 1] - __uint_as_float(hb[p] & 0xffff0000u);
      }
      Bl[0] = __builtin_convertvector(r, bf16x8);
    }
  };
  // the shared state tile slot of step s: row n, block b at columns 32 b + 8 g
  auto publish_own = [&](int slot) {
    if constexpr (TW == 2) {
      *reinterpret_cast<Op*>(xb + slot * 16 * HROW + n * HROW + 32 * w + 8 * g) = Bf[0];
      if constexpr (SPLIT) *reinterpret_cast<Op*>(xl + slot * 16 * HROW + n * HROW + 32 * w + 8 * g) = Bl[0];
    } else {
      // the tile's four elements: half hw of the block's fragment
      const int off = slot * 16 * HROW + n * HROW + 32 * ob + 8 * g + 4 * hw;
      *reinterpret_cast<u2*>(xb + off) = __builtin_bit_cast(u4, Bf[0]).xy;
      if constexpr (SPLIT) *reinterpret_cast<u2*>(xl + off) = __builtin_bit_cast(u4, Bl[0]).xy;
    }
  };
  auto fetch_others = [&](int slot) {
#pragma unroll
    for (int o = TW == 2 ? 1 : 0; o < KB; ++o) {
      const int b = (ob + o) % KB;
      Bf[o] = *reinterpret_cast<const Op*>(xb + slot * 16 * HROW + n * HROW + 32 * b + 8 * g);
      if constexpr (SPLIT) Bl[o] = *reinterpret_cast<const Op*>(xl + slot * 16 * HROW + n * HROW + 32 * b + 8 * g);
    }
  };
  // rank-1 term of step s of the chunk in stage buffer sb: acc[j] = (v, tile TW w + j) x (hi, lo of c k)
  auto rank1 = [&](int sb, int s, f4 (&acc)[TW]) {
    const unsigned int* kx = kx_all + sb * kChunk * 16;
    const unsigned int* vx = vx_all + sb * kChunk * 16 * L::NVX;
    const unsigned int kp = *((g == 0) ? kx + s * 16 + n : zero_lds);
    // 16x16x32: A the (v, v) pairs of tiles 2w, 2w + 1 and zeros, B the (hi, lo)
    // pair of c k in the slots of the tile. Not the
    // 16x16x16 form: on gfx950 a 16x16x32 product that took a 16x16x16 result as
    // its accumulator a few instructions later read it before the result was
    // there, and here the compiler places the rank-1 write within a few
    // instructions of the first product into the same accumulator.
    if constexpr (TW == 2) {
      const uint2 win = *reinterpret_cast<const uint2*>(vx + (s * 16 + n) * L::NVX + 2 * w);
      const bf16x8 av = __builtin_bit_cast(bf16x8, u4{win.x, win.y, 0u, 0u});
      acc[0] = mfma(av, __builtin_bit_cast(bf16x8, u4{kp, 0u, 0u, 0u}), f4{0, 0, 0, 0});
      acc[TW - 1] = mfma(av, __builtin_bit_cast(bf16x8, u4{0u, kp, 0u, 0u}), f4{0, 0, 0, 0});
    } else {
      const unsigned int win = vx[(s * 16 + n) * L::NVX + w];
      acc[0] = mfma(__builtin_bit_cast(bf16x8, u4{win, 0u, 0u, 0u}), __builtin_bit_cast(bf16x8, u4{kp, 0u, 0u, 0u}),
                    f4{0, 0, 0, 0});
    }
  };
  auto products = [&](int o, f4 (&acc)[TW]) {
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      acc[j] = mfma(Wf[j][o], Bf[o], acc[j]);
      if constexpr (SPLIT) acc[j] = mfma(Wf[j][o], Bl[o], acc[j]);
    }
  };

  // readout partials: Dr[j] lane (g, n) accumulates y_{t0 + n}[position 16 (TW w + j) + 4 g + i]
  // over the tile's 16 rows (positions are the permuted order of the state tiles:
  // position 32 b + 8 g' + e holds column 32 b + 16 (e / 4) + 4 g' + e % 4)
  f4 Dr[TW];
#pragma unroll
  for (int j = 0; j < TW; ++j) Dr[j] = f4{0, 0, 0, 0};
  // in two parts, so that the LDS reads go out with the exchange's and the
  // MFMAs follow the step's products
  // with SPLIT the low halves of the state are read out too (their tiles are
  // exchanged anyway), so y carries the split operand's precision
  struct ReadoutOps {
    Op q, s[TW], sl[SPLIT ? TW : 1];
  };
  auto readout_load = [&](int sb, int s0, int nvalid) {
    ReadoutOps r;
    const int p = g / 2, rr = 8 * (g % 2), s = s0 + p;
    // (q_s in column s of the operand, zero elsewhere). With two tiles per wave
    // every lane loads and the others' q is masked to zero afterwards: the load
    // under a lane condition compiled into a branch around it, 1-1.6 % of C4 and
    // C5; with one tile per wave (V = 64) the branch measured faster (C2 1-4 %).
    const u4* qsrc = reinterpret_cast<const u4*>(qs_all + sb * kChunk * 16 + s * 16 + rr);
    const bool use = n == s && p < nvalid;
    u4 qv;
    if constexpr (TW == 2) {
      qv = *qsrc & (use ? ~0u : 0u);
    } else {
      qv = u4{0, 0, 0, 0};
      if (use) qv = *qsrc;
    }
    r.q = __builtin_bit_cast(Op, qv);
    const unsigned short* src = xb + (s & (NHS - 1)) * 16 * HROW + (rr + n / 4) * HROW + 4 * (n % 4);
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int P = TW * w + j;
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * P));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(src + 16 * P + 4 * HROW));
      r.s[j] = __builtin_bit_cast(Op, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      if constexpr (SPLIT) {
        const unsigned short* srl = xl + (s & (NHS - 1)) * 16 * HROW + (rr + n / 4) * HROW + 4 * (n % 4);
        const s4 llo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(srl + 16 * P));
        const s4 lhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(srl + 16 * P + 4 * HROW));
        r.sl[j] = __builtin_bit_cast(Op, s8{llo[0], llo[1], llo[2], llo[3], lhi[0], lhi[1], lhi[2], lhi[3]});
      }
    }
    return r;
  };
  auto readout_mma = [&](const ReadoutOps& r) {
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      Dr[j] = mfma(r.s[j], r.q, Dr[j]);
      if constexpr (SPLIT) Dr[j] = mfma(r.sl[j], r.q, Dr[j]);
    }
  };
  // this wave's columns of y for the steps t0 .. t0 + nsteps - 1, added into y.
  // A chunk's sums are added at step 1 of the next chunk, after that step's
  // staging: the staging waits for all of the wave's outstanding global
  // operations, and by then the adds are 15 steps old instead of one.
  f4 Dp[TW];
  int pend_t0 = 0, pend_n = 0;
  float* ys = reinterpret_cast<float*>(lds + L::YS_OFF) + w * 16 * L::YS_ROW;
  auto add_y = [&]() {
    if (a.y != nullptr && pend_n > 0) {
      // through the wave's own LDS tile, so that each add instruction covers two
      // rows of 32 consecutive floats
      // lane (g, n) holds sums of step row n: each goes onto that step's grid of
      // spacing 2^(E - 23) (every sum of such values below 2^(E + 1) is exact)
      // (the training forward adds its sums unrounded)
      // E from the step's ||q_t||_1 and the chunk's state bound, with a sixteenth
      // of headroom for the rounding of the bound itself and of the bf16 readout
      // operand: 2^E > 1.0625 ||q_t||_1 M
      const float* ybp = ybt + ((pend_t0 / kChunk) & (L::YB_SLOTS - 1)) * L::YB_PER;
      const int e = GRID ? __builtin_amdgcn_frexp_expf(ybp[n] * ybp[kChunk] * 1.0625f) : 0;
      // (local column within block ob: 16 (g % 2) + 8 j' + 4 (g / 2) + i, j' the
      // tile's half of the block)
#pragma unroll
      for (int j = 0; j < TW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = Dp[j][i] * kInvC;
          if constexpr (GRID) x = __builtin_amdgcn_ldexpf(__builtin_rintf(__builtin_amdgcn_ldexpf(x, 23 - e)), e - 23);
          ys[n * L::YS_ROW + 16 * (g % 2) + 8 * (TW == 2 ? j : hw) + 4 * (g / 2) + i] = x;
        }
      __builtin_amdgcn_wave_barrier();
      // every value first, then the adds with no branch between them: a row
      // past the sequence's end adds zero to the chunk's last valid row (x + 0
      // is x), so the adds need no predicate and the reads one wait. Each add
      // instruction covers 64 / (16 TW) rows of 16 TW floats of the wave's
      // columns (TW = 1: local columns 8 hw .. +7 and 16 + 8 hw .. +7)
      constexpr int LPR = 16 * TW, NV = 4 * TW;
      const int k = l % LPR;
      const int lc = TW == 2 ? k : 8 * hw + k + 8 * (k / 8);
      float val[NV];
#pragma unroll
      for (int r = 0; r < NV; ++r) val[r] = ys[((64 / LPR) * r + l / LPR) * L::YS_ROW + lc];
#pragma unroll
      for (int r = 0; r < NV; ++r) {
        const int row = (64 / LPR) * r + l / LPR;
        const bool live = row < pend_n;
        unsafeAtomicAdd(a.y + (unit * LD + pend_t0 + (live ? row : pend_n - 1)) * V + 32 * ob + lc,
                        live ? val[r] : 0.0f);
      }
    }
    pend_n = 0;
  };

  // training forward: the multi-step kernel's saved layout (per step, 1 KB per
  // row tile and 32-column block, lane l's 16 bytes at 16 l); this wave's block
  // is w
  [[maybe_unused]] char* const saved = static_cast<char*>(a.saved);
  [[maybe_unused]] const long long sv_off = (long long)(row0 / 16) * (V / 32) * 1024 + w * 1024 + l * 16;

  // initial operand: every wave's block of G_0 through the shared tile (slot NHS - 1)
  make_own();
  if constexpr (SAVE) *reinterpret_cast<bf16x8*>(saved + saved_state_off(unit, 0, T, a.K, V) + sv_off) = Bf[0];
  publish_own(NHS - 1);
  lds_barrier();  // staged chunks, W-region reuse, and the operand blocks are visible
  fetch_others(NHS - 1);
  f4 acc[TW];
  // a step's gate scalars (f, a, -2 a) from its 16-byte record: only the three
  // used components are loaded, so the allocator cannot reuse the fourth's
  // register while the load is in flight (which forced a wait for the load
  // before the exchange reads could go out)
  auto gate_at = [](const float* p) {
    const float2 fa = *reinterpret_cast<const float2*>(p);
    return f4{fa.x, fa.y, p[2], 0.0f};
  };
  f4 gate = gate_at(fs_all);  // step 0's gate scalars
  if (nchunks > 0) {
    rank1(0, 0, acc);
#pragma unroll
    for (int o = 0; o < KB; ++o) products(o, acc);
  }

  // Whole 16-step chunks with the step index a compile-time constant, so every
  // LDS address of a step is a fixed offset from the chunk's bases. Steps past
  // the sequence's end run with the staged padding (gate 1, k = v = q = 0): the
  // blend then returns the state unchanged bit for bit, and the readout rows
  // they produce are never added into y.
  for (int c = 0; c < nchunks; ++c) {
    const int sb = c & 1;
    const int ns = c == nchunks - 1 ? Tb - c * kChunk : kChunk;
    const float* fsb = fs_all + sb * kChunk * 4;
    const float* fsn = fs_all + (sb ^ 1) * kChunk * 4;
    static_for<kChunk>([&](auto si) {
      constexpr int s = decltype(si)::value;
      // the next step's rank-1 term goes first, into its own accumulators: it
      // needs only staged inputs, and the matrix cores and LDS are otherwise
      // idle during the epilogue
      f4 accn[TW];
      if constexpr (s + 1 < kChunk) rank1(sb, s + 1, accn); else rank1(sb ^ 1, 0, accn);
      // acc holds c (G_{t-1} W + k_t v_t^T) for this wave's tiles
      [[maybe_unused]] const int t = c * kChunk + s;
      if constexpr (SAVE) {
        if (t < Tb)
          *reinterpret_cast<u4*>(saved + saved_pre_off(unit, t, a.B, a.H, T, a.K, V) + sv_off) =
              u4{pack_bf16(acc[0][0], acc[0][1]), pack_bf16(acc[0][2], acc[0][3]),
                 pack_bf16(acc[TW - 1][0], acc[TW - 1][1]), pack_bf16(acc[TW - 1][2], acc[TW - 1][3])};
      }
#pragma unroll
      for (int j = 0; j < TW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(acc[j][i]);
          const float r = __builtin_amdgcn_rcpf(1.0f + e);
          G[j][i] = fmaf(gate[2], r, fmaf(gate[0], G[j][i], gate[1]));
        }
      make_own();
      if constexpr (SAVE) {
        if (t < Tb) *reinterpret_cast<bf16x8*>(saved + saved_state_off(unit, t + 1, T, a.K, V) + sv_off) = Bf[0];
      }
      publish_own(s & (NHS - 1));
      if constexpr (TW == 2) products(0, accn);  // the own block is whole in registers
      lds_barrier();
      gate = gate_at((s + 1 < kChunk ? fsb : fsn) + 4 * ((s + 1) % kChunk));
      ReadoutOps ro;
      if constexpr ((s & 1) != 0) ro = readout_load(sb, s - 1, 2);
      fetch_others(s & (NHS - 1));
      // tile by tile: tile 0's sum is complete while tile 1's last KB - 1
      // blocks (twice as many MFMAs when split) still run, and the next step's
      // epilogue of tile 0 issues under them
#pragma unroll
      for (int j = 0; j < TW; ++j)
#pragma unroll
        for (int o = TW == 2 ? 1 : 0; o < KB; ++o) {
          accn[j] = mfma(Wf[j][o], Bf[o], accn[j]);
          if constexpr (SPLIT) accn[j] = mfma(Wf[j][o], Bl[o], accn[j]);
        }
#pragma unroll
      for (int j = 0; j < TW; ++j) acc[j] = accn[j];
      if constexpr ((s & 1) != 0) readout_mma(ro);
      if constexpr (s == 1) {
        // chunks 0 and 1 were staged before the loop; from chunk 1 on, step 1
        // stages chunk c + 1 into chunk c - 1's buffer (its last reads were
        // before this step's barrier) and fetches chunk c + 2
        if (c >= 1 && c + 1 < nchunks) {
          st.store(lds, c + 1, row0, mbound);
          if (c + 2 < nchunks) st.load(a, unit, row0, c + 2, Tb, LD);
        }
        add_y();  // chunk c - 1's sums
      }
    });
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      Dp[j] = Dr[j];
      Dr[j] = f4{0, 0, 0, 0};
    }
    pend_t0 = c * kChunk;
    pend_n = ns;
  }
  add_y();  // the last chunk's sums
  // H_T: the state after step Tb (H0 itself for an empty sequence)
  if (a.HT) {
    float* HT = a.HT + (unit * a.K + my_row) * V;
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      f4 x = G[j] * kInvC;
      if (nchunks == 0 && a.H0) x = *reinterpret_cast<const f4*>(a.H0 + (unit * a.K + my_row) * V + 16 * (TW * w + j) + 4 * g);
      *reinterpret_cast<f4*>(HT + 16 * (TW * w + j) + 4 * g) = x;
    }
  }
}

}  // namespace

bool long_supports(const FwdArgs& a) {
  return a.bf16 && (a.V == 64 || a.V == 128) && a.K % 16 == 0 && a.K >= 16 && a.K <= 128;
}

// Output tiles per wave of the plain forward (the saving forward always takes
// two). At V = 64 one tile per wave (four waves per 16-row tile) runs a step in
// 0.77x the time of two (B=4 H=8 K=V=64 T=512: 0.139 against 0.181 ms, fp16
// operand); at V = 128 eight waves per tile are no faster than four (C4 and C5
// within +-2 % single operand, 6 % slower split), so it keeps two.
constexpr int long_tw(int V) { return V == 64 ? 1 : 2; }

Plan plan_long(int B, int H, int K, int V) {
  const long long grid = (long long)B * H * (K / 16);
  return Plan{grid > 0x7fffffffLL ? -1 : (int)grid, 64 * V / (16 * long_tw(V)), 16, K / 16, 1,
              V == 128 ? LongLayout<128, true, long_tw(128)>::TOTAL : LongLayout<64, true, long_tw(64)>::TOTAL};
}

hipError_t launch_long(const FwdArgs& a, bool split, hipStream_t stream, bool f16) {
  if (!long_supports(a) || (f16 && (split || a.saved))) return hipErrorInvalidValue;
  const long long grid = (long long)a.B * a.H * (a.K / 16);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (!a.accumulate && a.y) {  // y is a sum over the row tiles
    if (a.ld > 0 && a.ld != a.T) return hipErrorInvalidValue;
    hipError_t e = fill_zero(a.y, (long long)a.B * a.H * a.T * a.V, stream);
    if (e != hipSuccess) return e;
  }
  const bool save = a.saved != nullptr;
  // (the saving forward: two tiles per wave; the plain one: long_tw(V))
  const dim3 block(64 * a.V / (16 * (save ? 2 : long_tw(a.V)))), gr((unsigned)grid);
#define M2RNN_LONG_LAUNCH(V_, S_, SV_) \
  hipLaunchKernelGGL((mfma_fwd_long_kernel<V_, S_, SV_, false, SV_ ? 2 : long_tw(V_)>), gr, block, 0, stream, a)
  if (f16) {
    if (a.V == 128)
      hipLaunchKernelGGL((mfma_fwd_long_kernel<128, false, false, true, long_tw(128)>), gr, block, 0, stream, a);
    else
      hipLaunchKernelGGL((mfma_fwd_long_kernel<64, false, false, true, long_tw(64)>), gr, block, 0, stream, a);
  } else if (a.V == 128) {
    if (split) {
      if (save) M2RNN_LONG_LAUNCH(128, true, true); else M2RNN_LONG_LAUNCH(128, true, false);
    } else {
      if (save) M2RNN_LONG_LAUNCH(128, false, true); else M2RNN_LONG_LAUNCH(128, false, false);
    }
  } else {
    if (split) {
      if (save) M2RNN_LONG_LAUNCH(64, true, true); else M2RNN_LONG_LAUNCH(64, true, false);
    } else {
      if (save) M2RNN_LONG_LAUNCH(64, false, true); else M2RNN_LONG_LAUNCH(64, false, false);
    }
  }
#undef M2RNN_LONG_LAUNCH
  return hipGetLastError();
}

}  // namespace m2rnn
