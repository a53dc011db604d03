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
// tiles, one 32-wide contraction block):
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
//     K/16 contributions per element in an order that can vary between runs
//     (rounding-level differences); H_T does not depend on any order.
// Inputs k, v, q, f are staged per 16-step chunk into LDS (two stage buffers),
// fetched from HBM a chunk ahead.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(8))) float f8;
typedef __attribute__((ext_vector_type(2))) float f2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short s4;
typedef __attribute__((ext_vector_type(8))) short s8;
typedef __attribute__((ext_vector_type(4))) unsigned int u4;

constexpr float kC = 2.8853900817779268f;      // 2 / ln 2
constexpr float kInvC = 0.34657359027997264f;  // ln 2 / 2
constexpr int kChunk = 16;

__device__ __forceinline__ float bf16_to_f32(unsigned int b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ unsigned int pack_bf16(float x0, float x1) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f2{x0, x1}, bf16x2));
}
__device__ __forceinline__ f4 mfma(const bf16x8& a, const bf16x8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// barrier that orders LDS only (global loads and y atomics stay in flight)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order
template <typename F, int... S>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int V>
struct LongLayout {
  static constexpr int S = V / 32;        // waves per workgroup = column blocks
  static constexpr int CT = V / 16;       // 16-column tiles
  static constexpr int THREADS = 64 * S;
  static constexpr int HROW = V + 8;      // bf16 per state-tile row (padded)
  static constexpr int NVX = 2 * CT + 4;  // dwords per (step, column-in-tile) of rank-1 A records
  static constexpr int NHS = 4;           // state-tile slots (the readout lags a step)
  static constexpr int KX_BYTES = 2 * kChunk * 16 * 4;
  static constexpr int QS_BYTES = 2 * kChunk * 16 * 2;
  static constexpr int FS_BYTES = 2 * kChunk * 4 * 4;
  static constexpr int VX_BYTES = 2 * kChunk * 16 * NVX * 4;
  static constexpr int XB_BYTES = NHS * 16 * HROW * 2;
  static constexpr int XL_BYTES = 2 * 16 * HROW * 2;
  static constexpr int KX_OFF = 0;
  static constexpr int QS_OFF = KX_OFF + KX_BYTES;
  static constexpr int FS_OFF = QS_OFF + QS_BYTES;
  static constexpr int VX_OFF = FS_OFF + FS_BYTES;
  static constexpr int XB_OFF = VX_OFF + VX_BYTES;
  static constexpr int XL_OFF = XB_OFF + XB_BYTES;
  static constexpr int YS_ROW = 33;       // floats per row of a wave's y transpose tile
  static constexpr int YS_BYTES = S * 16 * YS_ROW * 4;
  static constexpr int YS_OFF = XL_OFF + XL_BYTES;
  static constexpr int Z_OFF = YS_OFF + YS_BYTES;
  static constexpr int TOTAL = Z_OFF + 16;
  static_assert(V * HROW * 2 <= VX_BYTES, "W fits in the rank-1 region during the prologue");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  // 16-byte global pieces of one chunk
  static constexpr int P_K = kChunk * 2;        // 16 rows of k per step: 2 pieces
  static constexpr int P_Q = kChunk * 2;
  static constexpr int P_V = kChunk * V / 8;
  static constexpr int PIECES = P_K + P_Q + P_V;
  static constexpr int PPT = (PIECES + THREADS - 1) / THREADS;
};

// One chunk of per-step inputs for the tile's 16 rows: loaded to registers, then
// stored into a stage buffer in the forms the MFMAs read.
template <int V>
struct LongStager {
  using L = LongLayout<V>;
  u4 reg[L::PPT];
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
    freg = 0x3f80u;  // gate 1 past the end: the padding steps keep the state
    if (tid < kChunk && t0 + tid < Tb) freg = f[unit * ld + t0 + tid];
  }

  __device__ __forceinline__ void store(char* lds, int buf) const {
    const int tid = threadIdx.x;
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
        *reinterpret_cast<u4*>(qs + s * 16 + 8 * part) = r;
      } else if (slot < L::PIECES) {
        const int s2 = slot - L::P_K - L::P_Q;
        const int s = s2 / (V / 8), part = s2 % (V / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int col = 8 * part + i;
          const unsigned int raw = (r[i / 2] >> (16 * (i % 2))) & 0xffffu;
          const int tile = col / 16;
          vx[(s * 16 + col % 16) * L::NVX + 4 * (tile / 2) + tile % 2] = raw | (raw << 16);
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

template <int V, bool SPLIT, bool SAVE>
__global__ __launch_bounds__(LongLayout<V>::THREADS, 1) void mfma_fwd_long_kernel(FwdArgs a) {
  using L = LongLayout<V>;
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

  unsigned short* xb = reinterpret_cast<unsigned short*>(lds + L::XB_OFF);
  unsigned short* xl = reinterpret_cast<unsigned short*>(lds + L::XL_OFF);
  const unsigned int* kx_all = reinterpret_cast<const unsigned int*>(lds + L::KX_OFF);
  const unsigned short* qs_all = reinterpret_cast<const unsigned short*>(lds + L::QS_OFF);
  const float* fs_all = reinterpret_cast<const float*>(lds + L::FS_OFF);
  const unsigned int* vx_all = reinterpret_cast<const unsigned int*>(lds + L::VX_OFF);
  const unsigned int* zero_lds = reinterpret_cast<const unsigned int*>(lds + L::Z_OFF);

  // ---- prologue: chunk 0/1 inputs, W, H0 requested before the first wait
  LongStager<V> st, st1;
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
  f4 G[2];  // own output tiles 2w, 2w + 1: lane (g, n) holds G[n][16 c + 4 g + i]
  {
    const float* H0 = a.H0 ? a.H0 + (unit * a.K + my_row) * V : nullptr;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      G[j] = H0 ? *reinterpret_cast<const f4*>(H0 + 16 * (2 * w + j) + 4 * g) * kC : f4{0, 0, 0, 0};
  }
  // zeroed state-tile slots: the readout of an odd final step multiplies a slot
  // that step never wrote (by zero q), which must not hold NaN patterns
  for (int i = tid; i < (L::XB_BYTES + L::XL_BYTES) / 4; i += L::THREADS)
    reinterpret_cast<unsigned int*>(lds + L::XB_OFF)[i] = 0u;
  // W^T fragments of this wave's two output tiles, every contraction block, via
  // LDS. Register arrays over the blocks are indexed o = 0 .. KB - 1 for block
  // (w + o) mod KB (o = 0: the wave's own block), so that every register index
  // is a compile-time constant; only LDS addresses depend on the wave.
  bf16x8 Wf[2][KB];
  {
    unsigned short* wst = reinterpret_cast<unsigned short*>(lds + L::VX_OFF);
#pragma unroll
    for (int p = 0; p < WLOADS; ++p) {
      const int i = tid + p * L::THREADS;
      *reinterpret_cast<u4*>(wst + (i / (V / 8)) * HROW + 8 * (i % (V / 8))) = wreg[p];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int o = 0; o < KB; ++o) {
        const int c = 2 * w + j, b = (w + o) % KB;
        const unsigned short* src = wst + (32 * b + 4 * g + n / 4) * HROW + 16 * c + 4 * (n % 4);
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)src);
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * HROW));
        s8 wa = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        asm volatile("" : "=a"(wa) : "0"(wa));
        Wf[j][o] = __builtin_bit_cast(bf16x8, wa);
      }
    lds_barrier();  // the region is the rank-1 stage buffers from here on
  }
  // LDS init: the zero dwords of the rank-1 records, the zero word; chunks 0, 1
  for (int i = tid; i < 2 * kChunk * 16; i += L::THREADS)
#pragma unroll
    for (int k = 0; k < L::CT / 2; ++k)
      *reinterpret_cast<uint2*>(reinterpret_cast<unsigned int*>(lds + L::VX_OFF) + i * L::NVX + 4 * k + 2) =
          uint2{0u, 0u};
  if (tid < 4) reinterpret_cast<unsigned int*>(lds + L::Z_OFF)[tid] = 0u;
  if (nchunks > 0) st.store(lds, 0);
  if (nchunks > 1) st1.store(lds, 1);
  if (nchunks > 2) st.load(a, unit, row0, 2, Tb, LD);

  // operand blocks: Bf[o] lane (g, n) = bf16 G[n][32 b + 16 (j / 4) + 4 g + j % 4],
  // b = (w + o) mod KB
  bf16x8 Bf[KB], Bl[KB];
  auto make_own = [&]() {
    f8 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = G[0][i]; x[4 + i] = G[1][i]; }
    Bf[0] = __builtin_convertvector(x, bf16x8);
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
  auto publish_own = [&](int slot, int lslot) {
    *reinterpret_cast<bf16x8*>(xb + slot * 16 * HROW + n * HROW + 32 * w + 8 * g) = Bf[0];
    if constexpr (SPLIT) *reinterpret_cast<bf16x8*>(xl + lslot * 16 * HROW + n * HROW + 32 * w + 8 * g) = Bl[0];
  };
  auto fetch_others = [&](int slot, int lslot) {
#pragma unroll
    for (int o = 1; o < KB; ++o) {
      const int b = (w + o) % KB;
      Bf[o] = *reinterpret_cast<const bf16x8*>(xb + slot * 16 * HROW + n * HROW + 32 * b + 8 * g);
      if constexpr (SPLIT) Bl[o] = *reinterpret_cast<const bf16x8*>(xl + lslot * 16 * HROW + n * HROW + 32 * b + 8 * g);
    }
  };
  // rank-1 term of step s of the chunk in stage buffer sb: acc[j] = (v, tile 2w + j) x (hi, lo of c k)
  auto rank1 = [&](int sb, int s, f4 (&acc)[2]) {
    const unsigned int* kx = kx_all + sb * kChunk * 16;
    const unsigned int* vx = vx_all + sb * kChunk * 16 * L::NVX;
    const unsigned int kp = *((g == 0) ? kx + s * 16 + n : zero_lds);
    const u4 win = *reinterpret_cast<const u4*>(vx + (s * 16 + n) * L::NVX + 4 * w);
    acc[0] = mfma(__builtin_bit_cast(bf16x8, win), __builtin_bit_cast(bf16x8, u4{kp, 0u, 0u, 0u}), f4{0, 0, 0, 0});
    acc[1] = mfma(__builtin_bit_cast(bf16x8, win), __builtin_bit_cast(bf16x8, u4{0u, kp, 0u, 0u}), f4{0, 0, 0, 0});
  };
  auto products = [&](int o, f4 (&acc)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[j] = mfma(Wf[j][o], Bf[o], acc[j]);
      if constexpr (SPLIT) acc[j] = mfma(Wf[j][o], Bl[o], acc[j]);
    }
  };

  // readout partials: Dr[j] lane (g, n) accumulates y_{t0 + n}[position 16 (2w + j) + 4 g + i]
  // over the tile's 16 rows (positions are the permuted order of the state tiles)
  f4 Dr[2] = {f4{0, 0, 0, 0}, f4{0, 0, 0, 0}};
  // in two parts, so that the LDS reads go out with the exchange's and the
  // MFMAs follow the step's products
  struct ReadoutOps {
    bf16x8 q, s[2];
  };
  auto readout_load = [&](int sb, int s0, int nvalid) {
    ReadoutOps r;
    const int p = g / 2, rr = 8 * (g % 2), s = s0 + p;
    s8 qv = *reinterpret_cast<const s8*>(qs_all + sb * kChunk * 16 + s * 16 + rr);
    if (n != s || p >= nvalid) qv = s8{0, 0, 0, 0, 0, 0, 0, 0};
    r.q = __builtin_bit_cast(bf16x8, qv);
    const unsigned short* src = xb + (s & (NHS - 1)) * 16 * HROW + (rr + n / 4) * HROW + 4 * (n % 4);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int P = 2 * w + j;
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * P));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(src + 16 * P + 4 * HROW));
      r.s[j] = __builtin_bit_cast(bf16x8, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
    return r;
  };
  auto readout_mma = [&](const ReadoutOps& r) {
#pragma unroll
    for (int j = 0; j < 2; ++j) Dr[j] = mfma(r.s[j], r.q, Dr[j]);
  };
  // this wave's columns of y for the steps t0 .. t0 + nsteps - 1, added into y.
  // A chunk's sums are added at step 1 of the next chunk, after that step's
  // staging: the staging waits for all of the wave's outstanding global
  // operations, and by then the adds are 15 steps old instead of one.
  f4 Dp[2];
  int pend_t0 = 0, pend_n = 0;
  float* ys = reinterpret_cast<float*>(lds + L::YS_OFF) + w * 16 * L::YS_ROW;
  auto add_y = [&]() {
    if (a.y != nullptr && pend_n > 0) {
      // through the wave's own LDS tile, so that each add instruction covers two
      // rows of 32 consecutive floats
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) ys[n * L::YS_ROW + 16 * (g % 2) + 8 * j + 4 * (g / 2) + i] = Dp[j][i] * kInvC;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int row = 2 * r + l / 32;
        const float val = ys[row * L::YS_ROW + l % 32];
        if (row < pend_n) unsafeAtomicAdd(a.y + (unit * LD + pend_t0 + row) * V + 32 * w + l % 32, val);
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
  publish_own(NHS - 1, 1);
  lds_barrier();  // staged chunks, W-region reuse, and the operand blocks are visible
  fetch_others(NHS - 1, 1);
  f4 acc[2];
  f4 gate = *reinterpret_cast<const f4*>(fs_all);  // step 0's gate scalars
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
      f4 accn[2];
      if constexpr (s + 1 < kChunk) rank1(sb, s + 1, accn); else rank1(sb ^ 1, 0, accn);
      // acc holds c (G_{t-1} W + k_t v_t^T) for this wave's two tiles
      [[maybe_unused]] const int t = c * kChunk + s;
      if constexpr (SAVE) {
        if (t < Tb)
          *reinterpret_cast<u4*>(saved + saved_pre_off(unit, t, a.B, a.H, T, a.K, V) + sv_off) =
              u4{pack_bf16(acc[0][0], acc[0][1]), pack_bf16(acc[0][2], acc[0][3]), pack_bf16(acc[1][0], acc[1][1]),
                 pack_bf16(acc[1][2], acc[1][3])};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j)
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
      publish_own(s & (NHS - 1), s & 1);
      products(0, accn);
      lds_barrier();
      gate = *reinterpret_cast<const f4*>((s + 1 < kChunk ? fsb : fsn) + 4 * ((s + 1) % kChunk));
      ReadoutOps ro;
      if constexpr ((s & 1) != 0) ro = readout_load(sb, s - 1, 2);
      fetch_others(s & (NHS - 1), s & 1);
      // tile by tile: tile 0's sum is complete while tile 1's last KB - 1
      // blocks (twice as many MFMAs when split) still run, and the next step's
      // epilogue of tile 0 issues under them
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int o = 1; o < KB; ++o) {
          accn[j] = mfma(Wf[j][o], Bf[o], accn[j]);
          if constexpr (SPLIT) accn[j] = mfma(Wf[j][o], Bl[o], accn[j]);
        }
      acc[0] = accn[0];
      acc[1] = accn[1];
      if constexpr ((s & 1) != 0) readout_mma(ro);
      if constexpr (s == 1) {
        // chunks 0 and 1 were staged before the loop; from chunk 1 on, step 1
        // stages chunk c + 1 into chunk c - 1's buffer (its last reads were
        // before this step's barrier) and fetches chunk c + 2
        if (c >= 1 && c + 1 < nchunks) {
          st.store(lds, (c + 1) & 1);
          if (c + 2 < nchunks) st.load(a, unit, row0, c + 2, Tb, LD);
        }
        add_y();  // chunk c - 1's sums
      }
    });
    Dp[0] = Dr[0];
    Dp[1] = Dr[1];
    pend_t0 = c * kChunk;
    pend_n = ns;
    Dr[0] = f4{0, 0, 0, 0};
    Dr[1] = f4{0, 0, 0, 0};
  }
  add_y();  // the last chunk's sums
  // H_T: the state after step Tb (H0 itself for an empty sequence)
  if (a.HT) {
    float* HT = a.HT + (unit * a.K + my_row) * V;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f4 x = G[j] * kInvC;
      if (nchunks == 0 && a.H0) x = *reinterpret_cast<const f4*>(a.H0 + (unit * a.K + my_row) * V + 16 * (2 * w + j) + 4 * g);
      *reinterpret_cast<f4*>(HT + 16 * (2 * w + j) + 4 * g) = x;
    }
  }
}

}  // namespace

bool long_supports(const FwdArgs& a) {
  return a.bf16 && (a.V == 64 || a.V == 128) && a.K % 16 == 0 && a.K >= 16 && a.K <= 128;
}

Plan plan_long(int B, int H, int K, int V) {
  const long long grid = (long long)B * H * (K / 16);
  return Plan{grid > 0x7fffffffLL ? -1 : (int)grid, 64 * (V / 32), 16, K / 16, 1,
              V == 128 ? LongLayout<128>::TOTAL : LongLayout<64>::TOTAL};
}

hipError_t launch_long(const FwdArgs& a, bool split, hipStream_t stream) {
  if (!long_supports(a)) return hipErrorInvalidValue;
  const long long grid = (long long)a.B * a.H * (a.K / 16);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (!a.accumulate && a.y) {  // y is a sum over the row tiles
    if (a.ld > 0 && a.ld != a.T) return hipErrorInvalidValue;
    hipError_t e = fill_zero(a.y, (long long)a.B * a.H * a.T * a.V, stream);
    if (e != hipSuccess) return e;
  }
  const dim3 block(64 * (a.V / 32)), gr((unsigned)grid);
  const bool save = a.saved != nullptr;
#define M2RNN_LONG_LAUNCH(V_, S_, SV_) hipLaunchKernelGGL((mfma_fwd_long_kernel<V_, S_, SV_>), gr, block, 0, stream, a)
  if (a.V == 128) {
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
