// M²RNN backward pass on gfx950 matrix cores (bf16 inputs, fp32 gradients).
//
// The forward update (gist.science M²RNN technical summary, zh §2.1):
//   A_t = H_{t-1} W + k_t v_t^T,  Z_t = tanh(A_t),  H_t = f_t H_{t-1} + (1 - f_t) Z_t,
//   y_t = H_t^T q_t.
// Going back in time with G = dL/dH_t (zh §2.2: the backward pass works from
// forward states, here the ones the training forward saved):
//   G   = f_{t+1} G + dA_{t+1} W^T      (the gradient that reaches H_t)
//   G  += q_t dy_t^T,                    dq_t = H_t dy_t
//   dA  = (1 - f_t) G (1 - Z_t^2),       df_t = sum (H_{t-1} - Z_t) G
//   dk_t = dA v_t,  dv_t = dA^T k_t,     dW += H_{t-1}^T dA (a separate kernel)
// and dH0 = f_0 G + dA_0 W^T at the end.
//
// Work split as in the forward kernel: one wave per 16-row tile of a unit's
// K x V matrices, NW waves per workgroup, K / (16 NW) workgroups per unit. G
// lives in registers in the output layout of v_mfma_f32_16x16x32_bf16 in the
// orientation D = W dA^T, so that, as in the forward pass, a lane's two output
// tiles 2b, 2b+1 are its B fragment b for the next product: dA W^T runs on the
// matrix cores with W in accumulation registers (A operand A[l][kappa] =
// W[l][perm kappa]) and dA rounded to bf16.
//
//   1 - Z_t^2 = 4 r (1 - r) with r = 1 / (1 + exp2(u_t)), u_t = c A_t the saved
//   pre-activation (c = 2 / ln 2), and Z_t = 1 - 2 r.
//
// Per-row sums (dq, dk) reduce over the four lane groups; dv = dA^T k reduces
// over rows and uses the readout scheme of the forward kernel (state tiles
// through LDS, transposed back, one MFMA per 16 columns and step pair); df
// reduces over the whole tile. Sums over the workgroups of a unit (at most 2)
// are atomic adds onto zeroed outputs, which keeps them order-free.
//
// Time runs backwards in chunks of 16 steps aligned to the end of the
// sequence; the last chunk is padded below t = 0 with inert steps (zero inputs,
// gate 1), which also apply the final update that turns G into dH0.
#include <hip/hip_runtime.h>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

using namespace dev;

constexpr int kChunk = 16;

template <int V, int NW>
struct BwdLayout {
  static constexpr int R = 16 * NW;
  static constexpr int CT = V / 16;
  static constexpr int KB = V / 32;
  static constexpr int HROW = V + 8;
  static constexpr int NHS = 4;
  static constexpr int THREADS = 64 * NW;
  static constexpr int DV_BYTES = 2 * kChunk * V * 8;   // (dy, v) per step and column, 2 buffers
  static constexpr int QK_BYTES = 2 * kChunk * R * 8;   // (q, k) per step and row
  static constexpr int KS_BYTES = 2 * kChunk * R * 2;   // k as bf16 (readout B operand)
  static constexpr int FS_BYTES = 2 * kChunk * 8;       // (f, 4 (1 - f)) per step
  static constexpr int HB_BYTES = NW * NHS * 16 * HROW * 2;
  static constexpr int YP_BYTES = NW * kChunk * V * 4;
  static constexpr int DF_BYTES = NW * kChunk * 4;
  static constexpr int DV_OFF = 0;
  static constexpr int QK_OFF = DV_OFF + DV_BYTES;
  static constexpr int KS_OFF = QK_OFF + QK_BYTES;
  static constexpr int FS_OFF = KS_OFF + KS_BYTES;
  static constexpr int HB_OFF = FS_OFF + FS_BYTES;
  static constexpr int YP_OFF = HB_OFF + HB_BYTES;
  static constexpr int DF_OFF = YP_OFF + YP_BYTES;
  static constexpr int TOTAL = DF_OFF + DF_BYTES;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  // 16-byte global pieces of one chunk
  static constexpr int SLOT_DY = kChunk * V / 4;  // fp32
  static constexpr int SLOT_V = kChunk * V / 8;   // bf16
  static constexpr int SLOT_Q = kChunk * R / 8;
  static constexpr int SLOT_K = kChunk * R / 8;
  static constexpr int SLOTS = SLOT_DY + SLOT_V + SLOT_Q + SLOT_K;
  static constexpr int SPT = (SLOTS + THREADS - 1) / THREADS;
};

struct BwdArgs {
  const unsigned short *k, *v, *q, *f, *W;
  const char* saved;
  const float *dy, *dHT;
  float *dk, *dv, *dq, *df, *dH0;
  char* dA_out;  // per-step bf16 dA, one saved-layout slot per (unit, t) (read by the dW kernel)
  // stores that must not land (a padding step's dA, the dq and dk of lanes that
  // do not own a row) go here, so that no store sits behind a branch: a global
  // memory wait could then count them only conservatively, and would drain the
  // stores issued since the saved-data prefetch at every step
  char* sink;
  int B, H, T, K;
  long long ld;  // row stride (in steps) of the per-step inputs and gradients
};

// One chunk of per-step inputs, reversed: step s of chunk c is t = T - 1 - 16 c - s.
template <int V, int NW>
struct BwdStager {
  using L = BwdLayout<V, NW>;
  u4 reg[L::SPT];
  unsigned short freg;

  __device__ __forceinline__ void load(const BwdArgs& a, long long unit, int row0, int c) {
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
        const int s = s2 / (L::R / 8), part = s2 % (L::R / 8), t = a.T - 1 - kChunk * c - s;
        if (t >= 0) reg[p] = *reinterpret_cast<const u4*>((isk ? a.k : a.q) + (unit * a.ld + t) * a.K + row0 + 8 * part);
      }
    }
    // steps before t = 0 are inert: gate 1, zero inputs
    freg = 0x3f80u;
    const int t = a.T - 1 - kChunk * c - tid;
    if (tid < kChunk && t >= 0) freg = a.f[unit * a.ld + t];
  }

  __device__ __forceinline__ void store(char* lds, int buf) const {
    const int tid = threadIdx.x;
    float2* dv = reinterpret_cast<float2*>(lds + L::DV_OFF) + buf * kChunk * V;
    float2* qk = reinterpret_cast<float2*>(lds + L::QK_OFF) + buf * kChunk * L::R;
    unsigned short* ks = reinterpret_cast<unsigned short*>(lds + L::KS_OFF) + buf * kChunk * L::R;
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
        const int s = s2 / (L::R / 8), part = s2 % (L::R / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = (i & 1) ? hi_bf16(r[i / 2]) : lo_bf16(r[i / 2]);
          if (isk) qk[s * L::R + 8 * part + i].y = x; else qk[s * L::R + 8 * part + i].x = x;
        }
        if (isk) *reinterpret_cast<u4*>(ks + s * L::R + 8 * part) = r;
      }
    }
    if (tid < kChunk) {
      const float fg = lo_bf16(freg);
      fs[tid] = float2{fg, 4.0f * (1.0f - fg)};
    }
  }
};

template <int V, int NW>
__global__ __launch_bounds__(64 * NW, 1) void mfma_bwd_kernel(BwdArgs a) {
  using L = BwdLayout<V, NW>;
  constexpr int R = L::R, CT = L::CT, KB = L::KB, HROW = L::HROW, NHS = L::NHS;
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];

  const int tid = threadIdx.x;
  const int w = tid / 64, l = tid % 64, g = l / 16, n = l % 16;
  const int K = a.K, T = a.T;
  const int splits = K / R;
  const long long unit = blockIdx.x / splits;
  const int row0 = (blockIdx.x % splits) * R;
  const int h = static_cast<int>(unit % a.H);
  const int rt = row0 / 16 + w;       // this wave's row tile
  const int my_row = 16 * rt + n;     // state row of this lane
  const long long lane_off = (long long)rt * (V / 32) * 1024 + l * 16;  // its piece of a saved slot
  const int nchunks = (T + kChunk - 1) / kChunk;

  unsigned short* hb_w = reinterpret_cast<unsigned short*>(lds + L::HB_OFF) + w * NHS * 16 * HROW;
  float* yp_all = reinterpret_cast<float*>(lds + L::YP_OFF);
  float* dfp_all = reinterpret_cast<float*>(lds + L::DF_OFF);

  // ---- W fragments for dA W^T: Wp[c][b] lane (g, n) = W[16c + n][32b + 16(j/4) + 4g + j%4]
  bf16x8 Wp[CT][KB];
  {
    const unsigned short* Wh = a.W + (long long)h * V * V;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        const unsigned short* rowp = Wh + (16 * c + n) * V + 32 * b + 4 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(rowp);
        const uint2 hi = *reinterpret_cast<const uint2*>(rowp + 16);
        u4 wa = u4{lo.x, lo.y, hi.x, hi.y};
        asm volatile("" : "=a"(wa) : "0"(wa));  // only ever an MFMA operand
        Wp[c][b] = __builtin_bit_cast(bf16x8, wa);
      }
  }

  // ---- G = dL/dH_T, output layout: lane (g, n) holds G[n][16c + 4g + i]
  f4 G[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
    G[c] = a.dHT ? *reinterpret_cast<const f4*>(a.dHT + (unit * K + my_row) * V + 16 * c + 4 * g) : f4{0, 0, 0, 0};
  f4 cur[CT];  // dA_{t+1} W^T, not yet added into G
#pragma unroll
  for (int c = 0; c < CT; ++c) cur[c] = f4{0, 0, 0, 0};
  float fnext = 1.0f;  // gate of step t + 1

  for (int i = tid; i < L::HB_BYTES / 4; i += L::THREADS) reinterpret_cast<unsigned int*>(lds + L::HB_OFF)[i] = 0u;

  BwdStager<V, NW> st;
  st.load(a, unit, row0, 0);
  st.store(lds, 0);
  if (nchunks > 1) st.load(a, unit, row0, 1);
  lds_barrier();

  // saved data of a step: this lane's blocks of a slot (read once: non-temporal)
  struct Saved {
    u4 x[KB];
  };
  auto load_slot = [&](long long off) {
    Saved r;
#pragma unroll
    for (int b = 0; b < KB; ++b)
      r.x[b] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(a.saved + off + lane_off + b * 1024));
    return r;
  };
  // state operand c H_t of step t (slot t + 1; t = -1 is H0), pre-activation c A_t.
  // Padding steps (t < 0) read the nearest real slot instead, without a branch:
  // their gate is 1 and their dy 0, so their dA is exactly 0 for any finite data.
  auto state_of = [&](int t) { return load_slot(saved_state_off(unit, max(t, -1) + 1, T, K, V)); };
  auto pre_of = [&](int t) { return load_slot(saved_pre_off(unit, max(t, 0), a.B, a.H, T, K, V)); };

  Saved s_cur = state_of(T - 1), s_prev = state_of(T - 2), u_cur = pre_of(T - 1);

  // readout accumulators for dv: Dr[P] lane (g, n) sums over this wave's rows for
  // step n of the chunk, positions 16 P + 4 g + i (as in the forward readout)
  f4 Dr[CT];
#pragma unroll
  for (int P = 0; P < CT; ++P) Dr[P] = f4{0, 0, 0, 0};

  auto readout = [&](const unsigned short* ks, int s0, int nvalid) {
    const int p = g / 2, rr = 8 * (g % 2), s = s0 + p;
    s8 kv = *reinterpret_cast<const s8*>(ks + s * R + 16 * w + rr);
    if (n != s || p >= nvalid) kv = s8{0, 0, 0, 0, 0, 0, 0, 0};
    const bf16x8 Bk = __builtin_bit_cast(bf16x8, kv);
    const unsigned short* src = hb_w + (s & (NHS - 1)) * 16 * HROW + (rr + n / 4) * HROW + 4 * (n % 4);
#pragma unroll
    for (int P = 0; P < CT; ++P) {
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * P));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(src + 16 * P + 4 * HROW));
      const s8 av = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      Dr[P] = mfma(__builtin_bit_cast(bf16x8, av), Bk, Dr[P]);
    }
  };

  const bool atomic = splits > 1;
  // dv and df of a chunk's steps (t = t_first - s for s < nsteps, t >= 0)
  auto chunk_sums = [&](int t_first, int nsteps) {
    float* ypw = yp_all + w * kChunk * V;
#pragma unroll
    for (int P = 0; P < CT; ++P) *reinterpret_cast<f4*>(ypw + n * V + 16 * P + 4 * g) = Dr[P];
#pragma unroll
    for (int P = 0; P < CT; ++P) Dr[P] = f4{0, 0, 0, 0};
    lds_barrier();
    for (int grp = tid; grp < nsteps * (V / 4); grp += L::THREADS) {
      const int sn = grp / (V / 4), pos = 4 * (grp % (V / 4));
      const int t = t_first - sn;
      if (t < 0) continue;
      f4 sum = *reinterpret_cast<const f4*>(yp_all + sn * V + pos);
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) sum += *reinterpret_cast<const f4*>(yp_all + (ww * kChunk + sn) * V + pos);
      const int P = pos / 16, gg = (pos % 16) / 4;
      const int col = 32 * (P / 2) + 16 * (gg % 2) + 8 * (P % 2) + 4 * (gg / 2);
      float* dst = a.dv + (unit * a.ld + t) * V + col;
      if (atomic) {
#pragma unroll
        for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dst + i, sum[i]);
      } else {
        *reinterpret_cast<f4*>(dst) = sum;
      }
    }
    if (tid < nsteps && t_first - tid >= 0) {
      float sum = dfp_all[tid];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) sum += dfp_all[ww * kChunk + tid];
      float* dst = a.df + unit * a.ld + (t_first - tid);
      if (atomic) unsafeAtomicAdd(dst, sum); else *dst = sum;
    }
    lds_barrier();
  };

  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const float2* dvs = reinterpret_cast<const float2*>(lds + L::DV_OFF) + buf * kChunk * V;
    const float2* qks = reinterpret_cast<const float2*>(lds + L::QK_OFF) + buf * kChunk * R;
    const unsigned short* kss = reinterpret_cast<const unsigned short*>(lds + L::KS_OFF) + buf * kChunk * R;
    const float2* fss = reinterpret_cast<const float2*>(lds + L::FS_OFF) + buf * kChunk;
    const int t_first = T - 1 - kChunk * c;

    for (int s = 0; s < kChunk; ++s) {
      const int t = t_first - s;
      // prefetch the next step's saved data (the state slot two steps back, the pre-activation one back)
      const Saved s_prev2 = state_of(t - 2);
      const Saved u_next = pre_of(t - 1);
      const float2 fa = fss[s];
      const float fg = fa.x, a4 = fa.y;
      const float2 qk = qks[s * R + 16 * w + n];
      unsigned short* hdst = hb_w + (s & (NHS - 1)) * 16 * HROW + n * HROW + 8 * g;
      float dqp = 0.0f, dkp = 0.0f, dfp = 0.0f;
      f4 acc[CT];
#pragma unroll
      for (int cc = 0; cc < CT; ++cc) acc[cc] = f4{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        f4 dA[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int cc = 2 * b + half;
          const float4 d01 = *reinterpret_cast<const float4*>(dvs + s * V + 16 * cc + 4 * g);
          const float4 d23 = *reinterpret_cast<const float4*>(dvs + s * V + 16 * cc + 4 * g + 2);
          const float dyv[4] = {d01.x, d01.z, d23.x, d23.z};
          const float vv[4] = {d01.y, d01.w, d23.y, d23.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jj = 4 * half + i;  // element of block b
            const unsigned int sc = s_cur.x[b][jj / 2], sp = s_prev.x[b][jj / 2], uu = u_cur.x[b][jj / 2];
            const float hcur = (jj & 1) ? hi_bf16(sc) : lo_bf16(sc);   // c H_t
            const float hprv = (jj & 1) ? hi_bf16(sp) : lo_bf16(sp);   // c H_{t-1}
            const float u = (jj & 1) ? hi_bf16(uu) : lo_bf16(uu);      // c A_t
            float gv = fmaf(fnext, G[cc][i], cur[cc][i]);
            gv = fmaf(qk.x, dyv[i], gv);
            dqp = fmaf(hcur, dyv[i], dqp);
            const float r = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u));
            const float d = (a4 * gv) * fmaf(-r, r, r);
            dfp = fmaf(fmaf(2.0f, r, fmaf(hprv, kInvC, -1.0f)), gv, dfp);
            dkp = fmaf(d, vv[i], dkp);
            G[cc][i] = gv;
            dA[half][i] = d;
          }
        }
        const u4 pk = u4{pack_bf16(dA[0][0], dA[0][1]), pack_bf16(dA[0][2], dA[0][3]),
                         pack_bf16(dA[1][0], dA[1][1]), pack_bf16(dA[1][2], dA[1][3])};
        const bf16x8 Bd = __builtin_bit_cast(bf16x8, pk);
        *reinterpret_cast<bf16x8*>(hdst + 32 * b) = Bd;
        {
          // streamed out once and read once by the dW kernel: non-temporal
          char* dst = t >= 0 ? a.dA_out + (unit * T + t) * saved_slot_bytes(K, V) : a.sink;
          __builtin_nontemporal_store(pk, reinterpret_cast<u4*>(dst + lane_off + b * 1024));
        }
#pragma unroll
        for (int cc = 0; cc < CT; ++cc) acc[cc] = mfma(Wp[cc][b], Bd, acc[cc]);
      }
      // per-row sums over the four lane groups
      dqp += __shfl_xor(dqp, 16);
      dqp += __shfl_xor(dqp, 32);
      dkp += __shfl_xor(dkp, 16);
      dkp += __shfl_xor(dkp, 32);
      {
        const bool own = g == 0 && t >= 0;
        float* sinkf = reinterpret_cast<float*>(a.sink + saved_slot_bytes(K, V));
        *(own ? a.dq + (unit * a.ld + t) * K + my_row : sinkf + l) = dqp * kInvC;
        *(own ? a.dk + (unit * a.ld + t) * K + my_row : sinkf + 64 + l) = dkp;
      }
      // df over the tile
#pragma unroll
      for (int m = 1; m < 64; m *= 2) dfp += __shfl_xor(dfp, m);
      if (l == 0) dfp_all[w * kChunk + s] = dfp;
      // dv: read out the step pair (s - 1, s) once its second step has written its tile
      if (s & 1) readout(kss, s - 1, 2);
#pragma unroll
      for (int cc = 0; cc < CT; ++cc) cur[cc] = acc[cc];
      fnext = fg;
      s_cur = s_prev;
      s_prev = s_prev2;
      u_cur = u_next;
    }
    chunk_sums(t_first, kChunk);
    // next chunk's inputs
    if (c + 1 < nchunks) {
      st.store(lds, (c + 1) & 1);
      if (c + 2 < nchunks) st.load(a, unit, row0, c + 2);
      lds_barrier();
    }
  }

  // dH0 = f_0 G + dA_0 W^T (already applied when the last chunk had inert steps)
  if (a.dH0) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      f4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = fmaf(fnext, G[c][i], cur[c][i]);
      *reinterpret_cast<f4*>(a.dH0 + (unit * K + my_row) * V + 16 * c + 4 * g) = x;
    }
  }
}

// ---- dW = sum over the batch rows, steps and state rows of H_{t-1}^T dA_t.
// One workgroup (4 waves) per (head, contraction split); a split covers a range
// of 32-row blocks (two row tiles of one unit and step). Each block of the saved
// operand c H_{t-1} and of dA_t goes to LDS row-major and comes back through
// transposing reads as the A (c H_{t-1}^T) and B (dA) operands; wave w owns the
// output rows [V/4 w, V/4 (w + 1)). Partial sums go to the workspace, and a
// second kernel adds the splits in a fixed order.
template <int V>
__global__ __launch_bounds__(256, 1) void dw_partial_kernel(const char* saved, const char* dA, float* partial, int B,
                                                             int H, int T, int K, int nsplit) {
  constexpr int CT = V / 16, HROW = V + 8, LT = CT / 4;  // row tiles of the output per wave
  __shared__ __attribute__((aligned(16))) unsigned short tile[2][32 * HROW];
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64, g = l / 16, n = l % 16;
  const int h = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
  const int rtiles = K / 16;
  const long long nblocks = (long long)B * T * (rtiles / 2);  // 32-row blocks of this head
  const long long b0 = nblocks * split / nsplit, b1 = nblocks * (split + 1) / nsplit;
  const long long slot = saved_slot_bytes(K, V);
  f4 acc[LT][CT];
#pragma unroll
  for (int i = 0; i < LT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = f4{0, 0, 0, 0};

  // 2 matrices x 2 row tiles x V/32 blocks x 64 lanes of 16 bytes per block
  constexpr int PIECES = 2 * 2 * (V / 32) * 64, PPT = PIECES / 256;
  static_assert(PIECES % 256 == 0, "whole pieces per thread");
  // global reads of one block into registers (each piece is read once: non-temporal)
  auto fetch = [&](long long blk, u4 (&x)[PPT]) {
    const int pair = static_cast<int>(blk % (rtiles / 2));  // block -> (batch row, step, row-tile pair)
    const long long bt = blk / (rtiles / 2);
    const int t = static_cast<int>(bt % T);
    const int bb = static_cast<int>(bt / T);
    const long long unit = (long long)bb * H + h;
    const char* srcs[2] = {saved + saved_state_off(unit, t, T, K, V), dA + (unit * T + t) * slot};
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int p = tid + 256 * r;
      const int m = p / (2 * (V / 32) * 64), q = p % (2 * (V / 32) * 64);
      x[r] = __builtin_nontemporal_load(
          reinterpret_cast<const u4*>(srcs[m] + (long long)(2 * pair) * (V / 32) * 1024 + q * 16));
    }
  };
  // the same pieces, row-major into LDS
  auto put = [&](const u4 (&x)[PPT]) {
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int p = tid + 256 * r;
      const int m = p / (2 * (V / 32) * 64), q = p % (2 * (V / 32) * 64);
      const int rtl = q / ((V / 32) * 64), q2 = q % ((V / 32) * 64);
      const int bl = q2 / 64, lane = q2 % 64, lg = lane / 16, ln = lane % 16;
      unsigned short* row = tile[m] + (16 * rtl + ln) * HROW + 32 * bl + 4 * lg;
      *reinterpret_cast<uint2*>(row) = uint2{x[r][0], x[r][1]};
      *reinterpret_cast<uint2*>(row + 16) = uint2{x[r][2], x[r][3]};
    }
  };

  u4 xr[PPT];
  if (b0 < b1) fetch(b0, xr);
  for (long long blk = b0; blk < b1; ++blk) {
    put(xr);
    __syncthreads();
    if (blk + 1 < b1) fetch(blk + 1, xr);  // in flight during this block's products
    // operands: rows 8g .. 8g+7 of the 32 at column base + n, two transposing reads each
    auto tr = [&](int m, int colbase) {
      const unsigned short* src = tile[m] + (8 * g + n / 4) * HROW + colbase + 4 * (n % 4);
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)src);
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 4 * HROW));
      return __builtin_bit_cast(bf16x8, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    bf16x8 Aop[LT];
#pragma unroll
    for (int i = 0; i < LT; ++i) Aop[i] = tr(0, 16 * (LT * w + i));
#pragma unroll
    for (int j = 0; j < CT; ++j) {
      const bf16x8 Bop = tr(1, 16 * j);
#pragma unroll
      for (int i = 0; i < LT; ++i) acc[i][j] = mfma(Aop[i], Bop, acc[i][j]);
    }
    __syncthreads();
  }
  // D[l][j] for output row tile (LT w + i), column tile j: lane (g, n) holds rows 4g + e, column n
  float* out = partial + ((long long)h * nsplit + split) * V * V;
#pragma unroll
  for (int i = 0; i < LT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[(16 * (LT * w + i) + 4 * g + e) * V + 16 * j + n] = acc[i][j][e];
}

__global__ void dw_reduce_kernel(const float* partial, float* dW, int H, int VV, int nsplit, int accumulate) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)H * VV) return;
  const int h = static_cast<int>(i / VV), e = static_cast<int>(i % VV);
  const float* p = partial + (long long)h * nsplit * VV + e;
  float s = 0.0f;
  for (int k = 0; k < nsplit; ++k) s += p[(long long)k * VV];
  s *= kInvC;  // the saved operand is c H
  dW[i] = accumulate ? dW[i] + s : s;
}

int dw_splits(int B, int T, int K) {
  const long long blocks = (long long)B * T * (K / 32);
  long long s = (blocks + 127) / 128;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return static_cast<int>(s);
}

// dW from the saved states and the reverse kernel's dA slots
template <int V>
hipError_t launch_dw(const BwdArgs& a, float* partial, float* dW, bool dW_acc, hipStream_t stream) {
  hipError_t e;
  const int ns = dw_splits(a.B, a.T, a.K);
  hipLaunchKernelGGL((dw_partial_kernel<V>), dim3((unsigned)(a.H * ns)), dim3(256), 0, stream, a.saved, a.dA_out,
                     partial, a.B, a.H, a.T, a.K, ns);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long nel = (long long)a.H * V * V;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((unsigned)((nel + 255) / 256)), dim3(256), 0, stream, partial, dW, a.H,
                     V * V, ns, dW_acc ? 1 : 0);
  return hipGetLastError();
}

template <int V, int NW>
hipError_t launch_bwd_t(const BwdArgs& a, float* partial, float* dW, bool zeroed, bool dW_acc,
                        hipStream_t stream) {
  constexpr int R = 16 * NW;
  const int splits = a.K / R;
  const long long grid = (long long)a.B * a.H * splits;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipError_t e;
  if (splits > 1 && !zeroed) {  // dv and df take two workgroups' sums
    if (a.ld != a.T) return hipErrorInvalidValue;  // a window: the caller clears dv and df
    if ((e = fill_zero(a.dv, (long long)a.B * a.H * a.T * V, stream)) != hipSuccess) return e;
    if ((e = fill_zero(a.df, (long long)a.B * a.H * a.T, stream)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((mfma_bwd_kernel<V, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_dw<V>(a, partial, dW, dW_acc, stream);
}

}  // namespace

// the multi-step reverse kernel's sink: one dA slot, then 128 floats for dq and dk
static long long bwd_sink_bytes(int K, int V) { return saved_slot_bytes(K, V) + 512; }

// workspace: the dA slots, the dW partials, the long reverse kernel's partials,
// then the sink
long long bwd_workspace_bytes(int B, int H, int T, int K, int V) {
  return (long long)B * H * T * saved_slot_bytes(K, V) + (long long)H * dw_splits(B, T, K) * V * V * 4 +
         ((V == 64 || V == 128) ? bwd_long_partial_bytes(B, H, T, K, V) : 0) + bwd_sink_bytes(K, V);
}

hipError_t launch_bwd(const BwdLaunch& p, hipStream_t stream) {
  BwdArgs a{static_cast<const unsigned short*>(p.k), static_cast<const unsigned short*>(p.v),
            static_cast<const unsigned short*>(p.q), static_cast<const unsigned short*>(p.f),
            static_cast<const unsigned short*>(p.W), static_cast<const char*>(p.saved), p.dy, p.dHT,
            p.dk, p.dv, p.dq, p.df, p.dH0, static_cast<char*>(p.workspace),
            static_cast<char*>(p.workspace) + bwd_workspace_bytes(p.B, p.H, p.T, p.K, p.V) - bwd_sink_bytes(p.K, p.V),
            p.B, p.H, p.T, p.K,
            p.ld > 0 ? (long long)p.ld : (long long)p.T};
  const bool z = p.dvdf_zeroed != 0, acc = p.dW_accumulate != 0;
  float* partial = reinterpret_cast<float*>(static_cast<char*>(p.workspace) +
                                            (long long)p.B * p.H * p.T * saved_slot_bytes(p.K, p.V));
  if (p.long_kernel) {
    float* lp = partial + (long long)p.H * dw_splits(p.B, p.T, p.K) * p.V * p.V;
    hipError_t e = launch_bwd_long(p, static_cast<char*>(p.workspace), lp, stream);
    if (e != hipSuccess) return e;
    return p.V == 128 ? launch_dw<128>(a, partial, p.dW, acc, stream) : launch_dw<64>(a, partial, p.dW, acc, stream);
  }
  const int nw = p.K % 64 == 0 && p.K / 64 <= 2 ? 4 : (p.K % 32 == 0 && p.K / 32 <= 2 ? 2 : 0);
  if (p.V == 128)
    return nw == 4 ? launch_bwd_t<128, 4>(a, partial, p.dW, z, acc, stream)
                   : launch_bwd_t<128, 2>(a, partial, p.dW, z, acc, stream);
  return nw == 4 ? launch_bwd_t<64, 4>(a, partial, p.dW, z, acc, stream)
                 : launch_bwd_t<64, 2>(a, partial, p.dW, z, acc, stream);
}

}  // namespace m2rnn
