// M²RNN backward pass, latency-oriented variant for workloads with few 16-row
// tiles (small batch x heads, long sequences), on gfx950 matrix cores.
//
// The same recurrences as the multi-step reverse kernel (gist.science M²RNN
// technical summary, zh §2.1 update equations, §2.2 backward pass from the
// states the training forward kept):
//   G   = f_{t+1} G + dA_{t+1} W^T,   G += q_t dy_t^T,   dq_t = H_t dy_t
//   dA  = (1 - f_t) G (1 - Z_t^2),    df_t = sum (H_{t-1} - Z_t) G
//   dk_t = dA v_t,  dv_t = dA^T k_t,  dH0 = f_0 G + dA_0 W^T
// with 1 - Z^2 = 4 r (1 - r), r = 1 / (1 + exp2(u)), u = c A the saved
// pre-activation (c = 2 / ln 2). dW comes from the same kernels as before.
//
// The multi-step reverse kernel gives a 16-row tile to one wave (~6000 cycles
// per step at V = 128); with fewer tiles than SIMDs most of the chip idles. Here
// a tile is a workgroup of V/32 waves, each owning 32 columns: its two output
// tiles of dA W^T (W fragments of those rows only), and one 32-column block of
// dA, which it publishes into a shared LDS tile every step; after one LDS
// barrier each wave reads the other blocks back for its products. The
// per-element arithmetic, the saved layout and the operand rounding are the
// multi-step kernel's.
//   * Row sums (dq, dk) are partial per wave; the V/32 partials of each (step,
//     row) meet in LDS and are added once per chunk in a fixed order.
//   * Sums over a unit's rows (dv, df) get one partial per row tile, written to
//     a workspace; a second kernel adds a unit's K/16 partials in tile order:
//     every gradient is deterministic.
//   * The saved state and pre-activation of each step (16 bytes per lane of this
//     wave's block) are loaded four steps ahead into a ring of registers.
//   * Time runs backwards in whole 16-step chunks aligned to the sequence end,
//     with the step index a compile-time constant; steps before t = 0 are inert
//     (gate 1, zero inputs) and turn G into dH0, as in the multi-step kernel.
#include <hip/hip_runtime.h>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

using namespace dev;

constexpr int kChunk = 16;
constexpr int kAhead = 4;  // saved data loaded this many steps ahead
constexpr int kRing = 8;   // ring slots (divides kChunk; > kAhead + 1)

template <int V>
struct BwdLongLayout {
  static constexpr int S = V / 32;       // waves = column blocks
  static constexpr int THREADS = 64 * S;
  static constexpr int HROW = V + 8;     // bf16 per row of the shared dA tile
  static constexpr int NHS = 4;          // dA tile slots (the dv readout lags a step)
  static constexpr int DV_BYTES = 2 * kChunk * V * 8;   // (dy, v) per step and column, 2 buffers
  static constexpr int QK_BYTES = 2 * kChunk * 16 * 8;  // (q, k) per step and row
  static constexpr int KS_BYTES = 2 * kChunk * 16 * 2;  // k as bf16 (readout B operand)
  static constexpr int FS_BYTES = 2 * kChunk * 8;       // (f, 4 (1 - f)) per step
  static constexpr int HB_BYTES = NHS * 16 * HROW * 2;
  static constexpr int RS_BYTES = 2 * S * kChunk * 64 * 4;  // dq, dk partials per (wave, step, lane)
  static constexpr int DF_BYTES = S * kChunk * 64 * 4;      // df partials per (wave, step, lane)
  static constexpr int DV_OFF = 0;
  static constexpr int QK_OFF = DV_OFF + DV_BYTES;
  static constexpr int KS_OFF = QK_OFF + QK_BYTES;
  static constexpr int FS_OFF = KS_OFF + KS_BYTES;
  static constexpr int HB_OFF = FS_OFF + FS_BYTES;
  static constexpr int RS_OFF = HB_OFF + HB_BYTES;
  static constexpr int DF_OFF = RS_OFF + RS_BYTES;
  static constexpr int TOTAL = DF_OFF + DF_BYTES;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  // 16-byte global pieces of one chunk
  static constexpr int SLOT_DY = kChunk * V / 4;  // fp32
  static constexpr int SLOT_V = kChunk * V / 8;   // bf16
  static constexpr int SLOT_Q = kChunk * 16 / 8;
  static constexpr int SLOT_K = kChunk * 16 / 8;
  static constexpr int SLOTS = SLOT_DY + SLOT_V + SLOT_Q + SLOT_K;
  static constexpr int SPT = (SLOTS + THREADS - 1) / THREADS;
};

struct BwdLongArgs {
  const unsigned short *k, *v, *q, *f, *W;
  const char* saved;
  const float *dy, *dHT;
  float *dk, *dq, *dH0;
  char* dA_out;    // per-step bf16 dA in the saved layout (read by the dW kernel)
  float* dv_part;  // [K/16][B H][T][V]: each row tile's dv_t
  float* df_part;  // [K/16][B H][T]: each row tile's df_t
  char* dA_sink;   // one saved-layout slot that takes the inert steps' dA stores
  int B, H, T, K;
  long long ld;    // row stride (in steps) of the per-step inputs and of dk, dq
};

// One chunk of per-step inputs for the tile's 16 rows, reversed: step s of chunk
// c is t = T - 1 - 16 c - s.
template <int V>
struct BwdLongStager {
  using L = BwdLongLayout<V>;
  u4 reg[L::SPT];
  unsigned short freg;

  __device__ __forceinline__ void load(const BwdLongArgs& a, long long unit, int row0, int c) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < L::SPT; ++p) {
      int slot = tid + p * L::THREADS;
      reg[p] = u4{0, 0, 0, 0};
      if (slot < L::SLOT_DY) {
        const int s = slot / (V / 4), part = slot % (V / 4), t = a.T - 1 - kChunk * c - s;
        if (t >= 0) reg[p] = *reinterpret_cast<const u4*>(a.dy + (unit * a.ld + t) * V + 4 * part);
      } else if ((slot -= L::SLOT_DY) < L::SLOT_V) {
        const int s = slot / (V / 8), part = slot % (V / 8), t = a.T - 1 - kChunk * c - s;
        if (t >= 0) reg[p] = *reinterpret_cast<const u4*>(a.v + (unit * a.ld + t) * V + 8 * part);
      } else if ((slot -= L::SLOT_V) < L::SLOT_Q + L::SLOT_K) {
        const bool isk = slot >= L::SLOT_Q;
        const int s2 = isk ? slot - L::SLOT_Q : slot;
        const int s = s2 / 2, part = s2 % 2, t = a.T - 1 - kChunk * c - s;
        if (t >= 0) reg[p] = *reinterpret_cast<const u4*>((isk ? a.k : a.q) + (unit * a.ld + t) * a.K + row0 + 8 * part);
      }
    }
    freg = 0x3f80u;  // steps before t = 0 are inert: gate 1
    const int t = a.T - 1 - kChunk * c - tid;
    if (tid < kChunk && t >= 0) freg = a.f[unit * a.ld + t];
  }

  __device__ __forceinline__ void store(char* lds, int buf) const {
    const int tid = threadIdx.x;
    float2* dv = reinterpret_cast<float2*>(lds + L::DV_OFF) + buf * kChunk * V;
    float2* qk = reinterpret_cast<float2*>(lds + L::QK_OFF) + buf * kChunk * 16;
    unsigned short* ks = reinterpret_cast<unsigned short*>(lds + L::KS_OFF) + buf * kChunk * 16;
    float2* fs = reinterpret_cast<float2*>(lds + L::FS_OFF) + buf * kChunk;
#pragma unroll
    for (int p = 0; p < L::SPT; ++p) {
      int slot = tid + p * L::THREADS;
      const u4 r = reg[p];
      if (slot < L::SLOT_DY) {
        const int s = slot / (V / 4), part = slot % (V / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) dv[s * V + 4 * part + i].x = __uint_as_float(r[i]);
      } else if ((slot -= L::SLOT_DY) < L::SLOT_V) {
        const int s = slot / (V / 8), part = slot % (V / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) dv[s * V + 8 * part + i].y = (i & 1) ? hi_bf16(r[i / 2]) : lo_bf16(r[i / 2]);
      } else if ((slot -= L::SLOT_V) < L::SLOT_Q + L::SLOT_K) {
        const bool isk = slot >= L::SLOT_Q;
        const int s2 = isk ? slot - L::SLOT_Q : slot;
        const int s = s2 / 2, part = s2 % 2;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = (i & 1) ? hi_bf16(r[i / 2]) : lo_bf16(r[i / 2]);
          if (isk) qk[s * 16 + 8 * part + i].y = x; else qk[s * 16 + 8 * part + i].x = x;
        }
        if (isk) *reinterpret_cast<u4*>(ks + s * 16 + 8 * part) = r;
      }
    }
    if (tid < kChunk) {
      const float fg = lo_bf16(freg);
      fs[tid] = float2{fg, 4.0f * (1.0f - fg)};
    }
  }
};

template <int V>
__global__ __launch_bounds__(BwdLongLayout<V>::THREADS, 1) void mfma_bwd_long_kernel(BwdLongArgs a) {
  using L = BwdLongLayout<V>;
  constexpr int KB = V / 32, HROW = L::HROW, NHS = L::NHS, S = L::S;
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];

  const int tid = threadIdx.x;
  const int w = tid / 64, l = tid % 64, g = l / 16, n = l % 16;
  const int K = a.K, T = a.T;
  const int tiles = K / 16;
  const long long unit = blockIdx.x / tiles;
  const int rt = blockIdx.x % tiles, row0 = 16 * rt;
  const int h = static_cast<int>(unit % a.H);
  const int my_row = row0 + n;
  const long long BH = (long long)a.B * a.H;
  // this lane's 16 bytes of this wave's block in a saved-layout slot
  const long long lane_off = (long long)rt * (V / 32) * 1024 + w * 1024 + l * 16;
  const int nchunks = (T + kChunk - 1) / kChunk;

  unsigned short* hb = reinterpret_cast<unsigned short*>(lds + L::HB_OFF);
  float* rs = reinterpret_cast<float*>(lds + L::RS_OFF);  // [2][S][kChunk][64 lanes]
  float* dfs = reinterpret_cast<float*>(lds + L::DF_OFF);  // [S][kChunk][64 lanes]

  // W fragments of this wave's output tiles cc = 2w + j against every block
  // b = (w + o) mod KB (rotated so that register indices are compile-time):
  // lane (g, n) = W[16 cc + n][32 b + 16 (jj / 4) + 4 g + jj % 4], jj < 8
  bf16x8 Wp[2][KB];
  {
    const unsigned short* Wh = a.W + (long long)h * V * V;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int o = 0; o < KB; ++o) {
        const int cc = 2 * w + j, b = (w + o) % KB;
        const unsigned short* rowp = Wh + (16 * cc + n) * V + 32 * b + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(rowp);
        const uint2 hi = *reinterpret_cast<const uint2*>(rowp + 16);
        u4 wa = u4{lo.x, lo.y, hi.x, hi.y};
        asm volatile("" : "=a"(wa) : "0"(wa));  // only ever an MFMA operand
        Wp[j][o] = __builtin_bit_cast(bf16x8, wa);
      }
  }

  // G = dL/dH_T on this wave's tiles: lane (g, n) holds G[n][16 (2w + j) + 4 g + i]
  f4 G[2], cur[2];  // cur: dA_{t+1} W^T, not yet added into G
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    G[j] = a.dHT ? *reinterpret_cast<const f4*>(a.dHT + (unit * K + my_row) * V + 16 * (2 * w + j) + 4 * g)
                 : f4{0, 0, 0, 0};
    cur[j] = f4{0, 0, 0, 0};
  }
  float fnext = 1.0f;  // gate of step t + 1

  BwdLongStager<V> st;
  st.load(a, unit, row0, 0);
  st.store(lds, 0);
  if (nchunks > 1) st.load(a, unit, row0, 1);

  // saved data of step index i (t = T - 1 - i): the state operand c H_t (slot
  // t + 1, H0 for t = -1) and the pre-activation c A_t, this lane's 16 bytes.
  // Inert steps (t < 0) read a clamped step: any finite data does, since their
  // gate 1 zeroes dA and their dy, v, q are zero. The loads carry no branch, so
  // the waits for them count exactly the operations issued after them. Each
  // saved piece is read once: non-temporal loads.
  auto load_state = [&](long long i) {
    const long long t = (long long)T - 1 - i;
    const int slot = static_cast<int>(t + 1 < 0 ? 0 : t + 1);
    return __builtin_nontemporal_load(reinterpret_cast<const u4*>(a.saved + saved_state_off(unit, slot, T, K, V) + lane_off));
  };
  auto load_pre = [&](long long i) {
    const long long t = (long long)T - 1 - i;
    const int tc = static_cast<int>(t < 0 ? 0 : t);
    return __builtin_nontemporal_load(
        reinterpret_cast<const u4*>(a.saved + saved_pre_off(unit, tc, a.B, a.H, T, K, V) + lane_off));
  };
  // rings indexed by step index mod kRing: state i is read at steps i and i - 1,
  // the pre-activation at step i
  u4 sring[kRing], pring[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) {
    sring[i] = u4{0, 0, 0, 0};
    pring[i] = u4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i <= kAhead; ++i) sring[i] = load_state(i);
#pragma unroll
  for (int i = 0; i < kAhead; ++i) pring[i] = load_pre(i);
  lds_barrier();  // chunk 0 staged

  // dv readout partials: Dr[j] lane (g, n) sums over the tile's rows for step n of
  // the chunk, positions 16 (2w + j) + 4 g + i (the permuted column order)
  f4 Dr[2] = {f4{0, 0, 0, 0}, f4{0, 0, 0, 0}};

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const float2* dvs = reinterpret_cast<const float2*>(lds + L::DV_OFF) + buf * kChunk * V;
    const float2* qks = reinterpret_cast<const float2*>(lds + L::QK_OFF) + buf * kChunk * 16;
    const unsigned short* kss = reinterpret_cast<const unsigned short*>(lds + L::KS_OFF) + buf * kChunk * 16;
    const float2* fss = reinterpret_cast<const float2*>(lds + L::FS_OFF) + buf * kChunk;
    const int t_first = T - 1 - kChunk * c;

    // Per step: the parts that need the incoming dA_{t+1} W^T (the critical
    // path to the next exchange) come first; everything that depends only on
    // staged inputs and saved data (r, r (1 - r), q_t dy_t, the dq partial) is
    // formed one step early, while the previous step waits for its products; the
    // dk and df partials and the dA store follow the products' issue.
    struct Pre {
      float r[8], rr[8], qdy[8];
      float dqp;
    };
    auto precompute = [&](int sj) {  // step sj of this chunk
      Pre x;
      const u4 sc = sring[sj % kRing], uu = pring[sj % kRing];
      const float qn = qks[sj * 16 + n].x;
      float dqp = 0.0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int cc = 2 * w + j;
        const float4 d01 = *reinterpret_cast<const float4*>(dvs + sj * V + 16 * cc + 4 * g);
        const float4 d23 = *reinterpret_cast<const float4*>(dvs + sj * V + 16 * cc + 4 * g + 2);
        const float dyv[4] = {d01.x, d01.z, d23.x, d23.z};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 4 * j + e;
          const float hcur = (jj & 1) ? hi_bf16(sc[jj / 2]) : lo_bf16(sc[jj / 2]);  // c H_t
          const float u = (jj & 1) ? hi_bf16(uu[jj / 2]) : lo_bf16(uu[jj / 2]);     // c A_t
          const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u));
          x.r[jj] = r;
          x.rr[jj] = fmaf(-r, r, r);
          x.qdy[jj] = qn * dyv[e];
          dqp = fmaf(hcur, dyv[e], dqp);
        }
      }
      x.dqp = dqp;
      return x;
    };
    Pre pre;
    static_for<kChunk>([&](auto si) {
      constexpr int s = decltype(si)::value;
      const long long i = (long long)kChunk * c + s;  // step index
      const int t = t_first - s;
      // saved data kAhead steps on
      sring[(s + kAhead + 1) % kRing] = load_state(i + kAhead + 1);
      pring[(s + kAhead) % kRing] = load_pre(i + kAhead);
      if constexpr (s == 0) pre = precompute(0);  // the chunk was staged only now
      const float2 fa = fss[s];
      const float fg = fa.x, a4 = fa.y;
      // critical: G and dA of this wave's 8 elements, then the exchange
      f4 gvv[2], dA[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = 4 * j + e;
          const float gv = fmaf(fnext, G[j][e], cur[j][e]) + pre.qdy[jj];
          G[j][e] = gv;
          gvv[j][e] = gv;
          dA[j][e] = (a4 * gv) * pre.rr[jj];
        }
      const u4 pk = u4{pack_bf16(dA[0][0], dA[0][1]), pack_bf16(dA[0][2], dA[0][3]),
                       pack_bf16(dA[1][0], dA[1][1]), pack_bf16(dA[1][2], dA[1][3])};
      const bf16x8 Bown = __builtin_bit_cast(bf16x8, pk);
      // this wave's dA block into the shared tile (row n, columns 32 w + 8 g ..)
      *reinterpret_cast<u4*>(hb + (s & (NHS - 1)) * 16 * HROW + n * HROW + 32 * w + 8 * g) = pk;
      // dA_t W^T on this wave's two output tiles: own block first
      f4 acc[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[j] = mfma(Wp[j][0], Bown, f4{0, 0, 0, 0});
      lds_barrier();
      bf16x8 Bo[KB];
#pragma unroll
      for (int o = 1; o < KB; ++o) {
        const int b = (w + o) % KB;
        Bo[o] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u4*>(hb + (s & (NHS - 1)) * 16 * HROW + n * HROW + 32 * b + 8 * g));
      }
#pragma unroll
      for (int o = 1; o < KB; ++o)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j] = mfma(Wp[j][o], Bo[o], acc[j]);
      // off the critical path: dk, df and dq partials, the dA store
      {
        const u4 sp = sring[(s + 1) % kRing];
        float dkp = 0.0f, dfp = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int cc = 2 * w + j;
          const float4 d01 = *reinterpret_cast<const float4*>(dvs + s * V + 16 * cc + 4 * g);
          const float4 d23 = *reinterpret_cast<const float4*>(dvs + s * V + 16 * cc + 4 * g + 2);
          const float vv[4] = {d01.y, d01.w, d23.y, d23.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jj = 4 * j + e;
            const float hprv = (jj & 1) ? hi_bf16(sp[jj / 2]) : lo_bf16(sp[jj / 2]);  // c H_{t-1}
            dfp = fmaf(fmaf(2.0f, pre.r[jj], fmaf(hprv, kInvC, -1.0f)), gvv[j][e], dfp);
            dkp = fmaf(dA[j][e], vv[e], dkp);
          }
        }
        // each lane's partials to its own word (no branch, no two lanes on one
        // address); df first summed over the 16 lanes of each row
        rs[(w * kChunk + s) * 64 + l] = pre.dqp;
        rs[((S + w) * kChunk + s) * 64 + l] = dkp;
        dfs[(w * kChunk + s) * 64 + l] = row_sum16(dfp);
        char* dst = t >= 0 ? a.dA_out + (unit * T + t) * saved_slot_bytes(K, V) : a.dA_sink;
        __builtin_nontemporal_store(pk, reinterpret_cast<u4*>(dst + lane_off));  // read once, by the dW kernel
      }
      if constexpr (s + 1 < kChunk) pre = precompute(s + 1);
      // dv: read out the step pair (s - 1, s) on this wave's columns
      if constexpr ((s & 1) != 0) {
        const int p = g / 2, rr = 8 * (g % 2), sq = s - 1 + p;
        s8 kv = *reinterpret_cast<const s8*>(kss + sq * 16 + rr);
        if (n != sq) kv = s8{0, 0, 0, 0, 0, 0, 0, 0};
        const bf16x8 Bk = __builtin_bit_cast(bf16x8, kv);
        const unsigned short* src = hb + (sq & (NHS - 1)) * 16 * HROW + (rr + n / 4) * HROW + 4 * (n % 4);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int P = 2 * w + j;
          const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * P));
          const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s4*)(src + 16 * P + 4 * HROW));
          Dr[j] = mfma(__builtin_bit_cast(bf16x8, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}), Bk, Dr[j]);
        }
      }
      cur[0] = acc[0];
      cur[1] = acc[1];
      fnext = fg;
    });

    // ---- chunk sums. dv: this wave's columns of the tile's sum, step n of the chunk
    {
      const int t = t_first - n;
      if (t >= 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int P = 2 * w + j;
          const int col = 32 * (P / 2) + 16 * (g % 2) + 8 * (P % 2) + 4 * (g / 2);
          *reinterpret_cast<f4*>(a.dv_part + ((rt * BH + unit) * T + t) * V + col) = Dr[j];
        }
      }
      Dr[0] = f4{0, 0, 0, 0};
      Dr[1] = f4{0, 0, 0, 0};
    }
    // the last step wrote its partials after its barrier
    lds_barrier();
    // dq, dk: the partials of each (step, row) over the waves and the four lane
    // groups, in a fixed order
    for (int idx = tid; idx < kChunk * 16; idx += L::THREADS) {
      const int s = idx / 16, row = idx % 16, t = t_first - s;
      if (t < 0) continue;
      float q = 0.0f, kk = 0.0f;
#pragma unroll
      for (int ww = 0; ww < S; ++ww)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          q += rs[(ww * kChunk + s) * 64 + 16 * gg + row];
          kk += rs[((S + ww) * kChunk + s) * 64 + 16 * gg + row];
        }
      a.dq[(unit * a.ld + t) * K + row0 + row] = q * kInvC;
      a.dk[(unit * a.ld + t) * K + row0 + row] = kk;
    }
    if (tid < kChunk && t_first - tid >= 0) {  // df: the row totals of every wave
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < S; ++ww)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) sum += dfs[(ww * kChunk + tid) * 64 + 16 * gg];
      a.df_part[(rt * BH + unit) * T + (t_first - tid)] = sum;
    }
    // next chunk's inputs; the barrier also orders these reads before the next
    // chunk's partial writes
    if (c + 1 < nchunks) {
      st.store(lds, (c + 1) & 1);
      if (c + 2 < nchunks) st.load(a, unit, row0, c + 2);
    }
    lds_barrier();
  }

  // dH0 = f_0 G + dA_0 W^T (already applied when the last chunk had inert steps)
  if (a.dH0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = fmaf(fnext, G[j][e], cur[j][e]);
      *reinterpret_cast<f4*>(a.dH0 + (unit * K + my_row) * V + 16 * (2 * w + j) + 4 * g) = x;
    }
  }
}

// dv and df: a unit's K/16 row-tile partials added in tile order.
__global__ void bwd_long_sums_kernel(const float* dv_part, const float* df_part, float* dv, float* df, long long BH,
                                     int T, int V, int tiles, long long ld) {
  const long long n4 = BH * T * (V / 4);
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) {
    const long long ut = i / (V / 4);  // unit * T + t
    const int c4 = static_cast<int>(i % (V / 4));
    const long long unit = ut / T;
    const int t = static_cast<int>(ut % T);
    f4 s = *reinterpret_cast<const f4*>(dv_part + ut * V + 4 * c4);
    for (int r = 1; r < tiles; ++r) s += *reinterpret_cast<const f4*>(dv_part + (r * BH * T + ut) * V + 4 * c4);
    *reinterpret_cast<f4*>(dv + (unit * ld + t) * V + 4 * c4) = s;
  }
  if (i < BH * T) {
    const long long unit = i / T;
    const int t = static_cast<int>(i % T);
    float s = df_part[i];
    for (int r = 1; r < tiles; ++r) s += df_part[r * BH * T + i];
    df[unit * ld + t] = s;
  }
}

}  // namespace

long long bwd_long_partial_bytes(int B, int H, int T, int K, int V) {
  return (long long)(K / 16) * B * H * T * (V + 1) * 4 + 16 + saved_slot_bytes(K, V);
}

hipError_t launch_bwd_long(const BwdLaunch& p, char* dA_out, float* partials, hipStream_t stream) {
  if (!(p.V == 64 || p.V == 128) || p.K % 16 != 0 || p.K < 16 || p.K > 128) return hipErrorInvalidValue;
  const long long BH = (long long)p.B * p.H;
  const long long grid = BH * (p.K / 16);
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  BwdLongArgs a{static_cast<const unsigned short*>(p.k), static_cast<const unsigned short*>(p.v),
                static_cast<const unsigned short*>(p.q), static_cast<const unsigned short*>(p.f),
                static_cast<const unsigned short*>(p.W), static_cast<const char*>(p.saved), p.dy, p.dHT,
                p.dk, p.dq, p.dH0, dA_out, partials, partials + (long long)(p.K / 16) * BH * p.T * p.V,
                nullptr, p.B, p.H, p.T, p.K, p.ld > 0 ? (long long)p.ld : (long long)p.T};
  // the sink slot after the df partials, 16-byte aligned
  const long long sink_off = ((long long)(p.K / 16) * BH * p.T * (p.V + 1) * 4 + 15) / 16 * 16;
  a.dA_sink = reinterpret_cast<char*>(partials) + sink_off;
  if (p.V == 128)
    hipLaunchKernelGGL((mfma_bwd_long_kernel<128>), dim3((unsigned)grid), dim3(BwdLongLayout<128>::THREADS), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((mfma_bwd_long_kernel<64>), dim3((unsigned)grid), dim3(BwdLongLayout<64>::THREADS), 0,
                       stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = BH * p.T * (p.V / 4);
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_long_sums_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.dv_part, a.df_part, p.dv,
                     p.df, BH, p.T, p.V, p.K / 16, a.ld);
  return hipGetLastError();
}

}  // namespace m2rnn
