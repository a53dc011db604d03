// M²RNN forward recurrence on gfx950 matrix cores (bf16 inputs, fp32 state).
//
// Per (batch, head) unit and step (gist.science M²RNN technical summary, zh
// §2.1 update equations; ja §2.1):
//   Z_t = tanh(H_{t-1} W + k_t v_t^T),  H_t = f_t H_{t-1} + (1 - f_t) Z_t,
//   y_t = H_t^T q_t  (readout reading, post-update state).
// The pages' own kernel runs one matrix-unit GEMM per step with dimensions
// (K, V, V) that do not involve the batch, one state per streaming
// multiprocessor (zh §2.2); this is a gfx950 design for the same computation.
//
// Work split. Rows of H evolve independently (row i of H_{t-1} W only needs row
// i of H_{t-1}), so a unit's K rows are cut into 16-row tiles, one tile per
// wave (one wave per SIMD), and a workgroup of NW waves owns R = 16*NW rows.
// K/R workgroups share a unit; they never communicate except through the
// readout sum, which is added into y atomically (at most two contributions per
// element onto a zeroed y, so the result does not depend on their order).
//
// Registers (lane l, g = l / 16, n = l % 16):
//   * the fp32 master state, carried scaled as G = c H with c = 2 log2(e) so
//     that exp2 of the pre-activation gives e^{2x} directly; lane (g, n) holds
//     G[n][16 c + 4 g + i] for every 16-column tile c and i < 4 — the output
//     layout of v_mfma_f32_16x16x32_bf16 in the orientation D = W^T G^T;
//   * W, resident for the whole sequence, as A fragments of that MFMA with the
//     contraction index permuted so that a lane's two consecutive output tiles
//     are, after rounding to bf16, exactly its B fragment for the next step:
//     B fragment b, lane (g, n), element j  =  G[n][32 b + 16 (j/4) + 4 g + j%4].
//     Hence the state never leaves the registers between steps.
// Per step per wave: V/16 * V/32 MFMAs for H_{t-1} W, then per element
//   u = acc + (c k_n) v_j; e = exp2(u); r = 1 / (1 + e)
//   G <- f G + a - 2 a r,  a = (1 - f) c        (tanh(x) = 1 - 2 / (1 + e^{2x}))
// and the bf16 rounding (round-to-nearest-even) of G for the next product.
// With SPLIT, the state operand is the pair hi = bf16(G), lo = bf16(G - hi)
// (the residual G - hi is exact in fp32), and the
// product takes two MFMA passes, W hi + W lo: the operand then carries ~16
// significant bits instead of 8, for trajectories that amplify per-step
// rounding (the transition matrix is a bf16 input, so W itself is exact).
//
// Readout. The rounded state tile is written to LDS (one 16-byte store per
// lane per 32 columns) and read back transposed with ds_read_b64_tr_b16, which
// turns the row-per-lane layout into the column-per-lane A operand of a second
// MFMA that contracts over rows against q. The readout of step t runs during
// step t+1 (double-buffered, one barrier per step). Its B operand carries q_t
// only in column t % 16, so one accumulator collects 16 consecutive steps and is
// stored as a 16-step x 16-column block.
//
// Inputs k, v, q, f are staged chunk by chunk (kChunk steps) into LDS by the
// whole workgroup, loaded from HBM one chunk ahead of use.
#include <hip/hip_runtime.h>

#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(8))) float f8;
typedef __attribute__((ext_vector_type(4))) short s4;
typedef __attribute__((ext_vector_type(8))) short s8;
typedef __attribute__((ext_vector_type(4))) unsigned int u4;

constexpr float kC = 2.8853900817779268f;      // 2 / ln 2
constexpr float kInvC = 0.34657359027997264f;  // ln 2 / 2
constexpr int kChunk = 16;                     // steps staged per LDS chunk

__device__ __forceinline__ float bf16_to_f32(unsigned short b) {
  return __uint_as_float(static_cast<unsigned int>(b) << 16);
}

template <int V, int NW>
struct Layout {
  static constexpr int R = 16 * NW;          // rows per workgroup
  static constexpr int CT = V / 16;          // 16-column tiles
  static constexpr int KB = V / 32;          // 32-wide contraction blocks
  static constexpr int HROW = V + 8;         // bf16 elements per LDS state row (padded)
  // LDS regions (bytes)
  static constexpr int H_BYTES = 2 * R * HROW * 2;            // two readout buffers
  static constexpr int K_BYTES = 2 * kChunk * R * 4;          // c*k, fp32
  static constexpr int V_BYTES = 2 * kChunk * V * 4;          // v, fp32
  static constexpr int Q_BYTES = 2 * kChunk * R * 2;          // q, bf16
  static constexpr int F_BYTES = 2 * kChunk * 4 * 4;          // f, a, -2a, pad
  static constexpr int H_OFF = 0;
  static constexpr int K_OFF = H_OFF + H_BYTES;
  static constexpr int V_OFF = K_OFF + K_BYTES;
  static constexpr int Q_OFF = V_OFF + V_BYTES;
  static constexpr int F_OFF = Q_OFF + Q_BYTES;
  static constexpr int TOTAL = F_OFF + F_BYTES;
  // 16-byte global load slots per chunk
  static constexpr int SLOT_K = kChunk * R / 8;
  static constexpr int SLOT_Q = kChunk * R / 8;
  static constexpr int SLOT_V = kChunk * V / 8;
  static constexpr int SLOTS = SLOT_K + SLOT_Q + SLOT_V;
  static constexpr int THREADS = 64 * NW;
  static constexpr int SLOTS_PER_THREAD = (SLOTS + THREADS - 1) / THREADS;
};

// Chunk staging: each thread owns up to SLOTS_PER_THREAD 16-byte slots.
template <int V, int NW>
struct Stager {
  using L = Layout<V, NW>;
  u4 reg[L::SLOTS_PER_THREAD];
  unsigned short freg;  // one gate value (threads < kChunk)

  __device__ __forceinline__ void load(const FwdArgs& a, long long unit, int row0, int chunk) {
    const int tid = threadIdx.x;
    const int t0 = chunk * kChunk;
    const unsigned short* k = static_cast<const unsigned short*>(a.k);
    const unsigned short* q = static_cast<const unsigned short*>(a.q);
    const unsigned short* v = static_cast<const unsigned short*>(a.v);
    const unsigned short* f = static_cast<const unsigned short*>(a.f);
#pragma unroll
    for (int p = 0; p < L::SLOTS_PER_THREAD; ++p) {
      const int slot = tid + p * L::THREADS;
      reg[p] = u4{0, 0, 0, 0};
      if (slot < L::SLOT_K + L::SLOT_Q) {
        const bool isq = slot >= L::SLOT_K;
        const int s2 = isq ? slot - L::SLOT_K : slot;
        const int s = s2 / (L::R / 8), part = s2 % (L::R / 8);
        const int t = t0 + s;
        if (t < a.T) {
          const unsigned short* src = (isq ? q : k) + (unit * a.T + t) * a.K + row0 + 8 * part;
          reg[p] = *reinterpret_cast<const u4*>(src);
        }
      } else if (slot < L::SLOTS) {
        const int s2 = slot - L::SLOT_K - L::SLOT_Q;
        const int s = s2 / (V / 8), part = s2 % (V / 8);
        const int t = t0 + s;
        if (t < a.T) {
          const unsigned short* src = v + (unit * a.T + t) * V + 8 * part;
          reg[p] = *reinterpret_cast<const u4*>(src);
        }
      }
    }
    freg = 0;
    if (tid < kChunk && t0 + tid < a.T) freg = f[unit * a.T + t0 + tid];
  }

  __device__ __forceinline__ void store(char* lds, int buf) const {
    const int tid = threadIdx.x;
    float* ks = reinterpret_cast<float*>(lds + L::K_OFF) + buf * kChunk * L::R;
    float* vs = reinterpret_cast<float*>(lds + L::V_OFF) + buf * kChunk * V;
    unsigned short* qs = reinterpret_cast<unsigned short*>(lds + L::Q_OFF) + buf * kChunk * L::R;
    float* fs = reinterpret_cast<float*>(lds + L::F_OFF) + buf * kChunk * 4;
#pragma unroll
    for (int p = 0; p < L::SLOTS_PER_THREAD; ++p) {
      const int slot = tid + p * L::THREADS;
      const u4 r = reg[p];
      if (slot < L::SLOT_K) {
        const int s = slot / (L::R / 8), part = slot % (L::R / 8);
        float* dst = ks + s * L::R + 8 * part;
        f4 lo, hi;
        lo[0] = __uint_as_float(r[0] << 16) * kC;
        lo[1] = __uint_as_float(r[0] & 0xffff0000u) * kC;
        lo[2] = __uint_as_float(r[1] << 16) * kC;
        lo[3] = __uint_as_float(r[1] & 0xffff0000u) * kC;
        hi[0] = __uint_as_float(r[2] << 16) * kC;
        hi[1] = __uint_as_float(r[2] & 0xffff0000u) * kC;
        hi[2] = __uint_as_float(r[3] << 16) * kC;
        hi[3] = __uint_as_float(r[3] & 0xffff0000u) * kC;
        *reinterpret_cast<f4*>(dst) = lo;
        *reinterpret_cast<f4*>(dst + 4) = hi;
      } else if (slot < L::SLOT_K + L::SLOT_Q) {
        const int s2 = slot - L::SLOT_K;
        const int s = s2 / (L::R / 8), part = s2 % (L::R / 8);
        *reinterpret_cast<u4*>(qs + s * L::R + 8 * part) = r;
      } else if (slot < L::SLOTS) {
        const int s2 = slot - L::SLOT_K - L::SLOT_Q;
        const int s = s2 / (V / 8), part = s2 % (V / 8);
        float* dst = vs + s * V + 8 * part;
        f4 lo, hi;
        lo[0] = __uint_as_float(r[0] << 16);
        lo[1] = __uint_as_float(r[0] & 0xffff0000u);
        lo[2] = __uint_as_float(r[1] << 16);
        lo[3] = __uint_as_float(r[1] & 0xffff0000u);
        hi[0] = __uint_as_float(r[2] << 16);
        hi[1] = __uint_as_float(r[2] & 0xffff0000u);
        hi[2] = __uint_as_float(r[3] << 16);
        hi[3] = __uint_as_float(r[3] & 0xffff0000u);
        *reinterpret_cast<f4*>(dst) = lo;
        *reinterpret_cast<f4*>(dst + 4) = hi;
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

// State operand(s) for the next product from the fp32 state tiles 2b, 2b+1.
template <bool SPLIT>
__device__ __forceinline__ void make_operand(const f4& g0, const f4& g1, bf16x8& hi, bf16x8& lo) {
  f8 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[i] = g0[i]; x[4 + i] = g1[i]; }
  hi = __builtin_convertvector(x, bf16x8);
  if constexpr (SPLIT) {
    // exact residual x - hi: hi widened back to fp32 from its bit pattern
    const u4 hb = __builtin_bit_cast(u4, hi);
    f8 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      r[2 * p] = x[2 * p] - __uint_as_float(hb[p] << 16);
      r[2 * p + 1] = x[2 * p + 1] - __uint_as_float(hb[p] & 0xffff0000u);
    }
    lo = __builtin_convertvector(r, bf16x8);
  }
}

template <int V, int NW, bool SPLIT>
__global__ __launch_bounds__(64 * NW, 1) void mfma_fwd_kernel(FwdArgs a) {
  using L = Layout<V, NW>;
  constexpr int R = L::R, CT = L::CT, KB = L::KB, HROW = L::HROW;
  constexpr int RT_PER_WAVE = CT / NW;  // readout position tiles per wave
  static_assert(CT % NW == 0, "readout tiles must divide among waves");
  static_assert(R % 32 == 0, "readout contracts 32 rows per MFMA");
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];

  const int tid = threadIdx.x;
  const int w = tid / 64, l = tid % 64, g = l / 16, n = l % 16;
  const int splits = a.K / R;
  const long long unit = blockIdx.x / splits;
  const int row0 = (blockIdx.x % splits) * R;
  const int h = static_cast<int>(unit % a.H);
  const int T = a.T;
  const int my_row = row0 + 16 * w + n;  // state row this lane carries (within the unit)

  // ---- W as permuted A fragments: Wf[c][b] lane (g,n) = W[32b + 16(j/4) + 4g + j%4][16c + n]
  bf16x8 Wf[CT][KB];
  {
    const unsigned short* Wp = static_cast<const unsigned short*>(a.W) + (long long)h * V * V;
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        s8 t;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = 32 * b + 16 * (j / 4) + 4 * g + (j % 4);
          t[j] = static_cast<short>(Wp[row * V + 16 * c + n]);
        }
        // pin the fragment to the accumulation registers: it is only ever a
        // matrix operand, and this leaves the arch VGPRs to the epilogue
        u4 wa = __builtin_bit_cast(u4, t);
        asm volatile("" : "=a"(wa) : "0"(wa));
        Wf[c][b] = __builtin_bit_cast(bf16x8, wa);
      }
  }

  // ---- scaled fp32 state G = c H, output layout
  f4 G[CT];
  {
    const float* H0 = a.H0 ? a.H0 + (unit * a.K + my_row) * V : nullptr;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      if (H0) {
        f4 x = *reinterpret_cast<const f4*>(H0 + 16 * c + 4 * g);
        G[c] = x * kC;
      } else {
        G[c] = f4{0, 0, 0, 0};
      }
    }
  }
  bf16x8 Bf[KB], Bl[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b) make_operand<SPLIT>(G[2 * b], G[2 * b + 1], Bf[b], Bl[b]);

  // ---- input staging: chunk 0 now, chunk 1 in flight
  Stager<V, NW> st;
  st.load(a, unit, row0, 0);
  st.store(lds, 0);
  const int nchunks = (T + kChunk - 1) / kChunk;
  if (nchunks > 1) st.load(a, unit, row0, 1);

  f4 Dr[RT_PER_WAVE];
#pragma unroll
  for (int p = 0; p < RT_PER_WAVE; ++p) Dr[p] = f4{0, 0, 0, 0};

  unsigned short* Hs = reinterpret_cast<unsigned short*>(lds + L::H_OFF);
  const float* ks_all = reinterpret_cast<const float*>(lds + L::K_OFF);
  const float* vs_all = reinterpret_cast<const float*>(lds + L::V_OFF);
  const unsigned short* qs_all = reinterpret_cast<const unsigned short*>(lds + L::Q_OFF);
  const float* fs_all = reinterpret_cast<const float*>(lds + L::F_OFF);
  float* y = a.y;
  const bool atomic_y = splits > 1 || a.accumulate;

  // readout of step tt (state in Hs buffer tt & 1, q in stage buffer (tt / kChunk) & 1)
  auto readout = [&](int tt) {
    const int nsel = tt % kChunk;
    const int qbuf = (tt / kChunk) & 1;
    const unsigned short* qrow = qs_all + (qbuf * kChunk + nsel) * R;
    const unsigned short* hb = Hs + (tt & 1) * R * HROW;
#pragma unroll
    for (int rb = 0; rb < R / 32; ++rb) {
      s8 qv = *reinterpret_cast<const s8*>(qrow + 32 * rb + 8 * g);
      if (n != nsel) qv = s8{0, 0, 0, 0, 0, 0, 0, 0};
      const bf16x8 Bq = __builtin_bit_cast(bf16x8, qv);
#pragma unroll
      for (int p = 0; p < RT_PER_WAVE; ++p) {
        const int P = w + NW * p;  // position tile
        // source lane (g, r = n): row 32rb + 8g + n/4 (+4), positions 16P + 4 (n%4)
        const unsigned short* src0 = hb + (32 * rb + 8 * g + n / 4) * HROW + 16 * P + 4 * (n % 4);
        const unsigned short* src1 = src0 + 4 * HROW;
        s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src0));
        s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src1));
        s8 av = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        Dr[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), Bq, Dr[p], 0, 0, 0);
      }
    }
    if (nsel == kChunk - 1 || tt == T - 1) {
      // lane (g, n) holds y_{tt - nsel + n}[col(16P + 4g) + i]
      const int tfirst = tt - nsel;
      if (n <= nsel) {
        float* yrow = y + (unit * T + tfirst + n) * V;
#pragma unroll
        for (int p = 0; p < RT_PER_WAVE; ++p) {
          const int P = w + NW * p;
          const int col = 32 * (P / 2) + 16 * (g % 2) + 8 * (P % 2) + 4 * (g / 2);
          const f4 val = Dr[p] * kInvC;
          if (atomic_y) {
#pragma unroll
            for (int i = 0; i < 4; ++i) unsafeAtomicAdd(yrow + col + i, val[i]);
          } else {
            *reinterpret_cast<f4*>(yrow + col) = val;
          }
        }
      }
#pragma unroll
      for (int p = 0; p < RT_PER_WAVE; ++p) Dr[p] = f4{0, 0, 0, 0};
    }
  };

  // One step, software-pipelined across steps: `cur` holds the finished
  // H_{t-1} W of step t; as soon as the epilogue has produced state tiles 2b and
  // 2b+1 (the next operand block b), the MFMAs of step t+1 for block b are issued
  // into `nxt`, so the matrix cores work on step t+1 while the VALU finishes step t.
  auto step = [&](int t, f4 (&cur)[CT], f4 (&nxt)[CT]) {
    const int s = t % kChunk;
    const int sb = (t / kChunk) & 1;
    const float* fs = fs_all + (sb * kChunk + s) * 4;
    const float fg = fs[0], av = fs[1], m2a = fs[2];
    const float ck = ks_all[(sb * kChunk + s) * R + 16 * w + n];
    const float* vrow = vs_all + (sb * kChunk + s) * V;
    unsigned short* hdst = Hs + (t & 1) * R * HROW + (16 * w + n) * HROW + 8 * g;
#pragma unroll
    for (int b = 0; b < KB; ++b) {
#pragma unroll
      for (int c = 2 * b; c < 2 * b + 2; ++c) {
        const f4 vv = *reinterpret_cast<const f4*>(vrow + 16 * c + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // rank-1 write, tanh via exp2/rcp, gate blend
          const float u = fmaf(ck, vv[i], cur[c][i]);
          const float e = __builtin_amdgcn_exp2f(u);
          const float r = __builtin_amdgcn_rcpf(1.0f + e);
          G[c][i] = fmaf(m2a, r, fmaf(fg, G[c][i], av));
        }
      }
      make_operand<SPLIT>(G[2 * b], G[2 * b + 1], Bf[b], Bl[b]);
      // rounded state block -> LDS for the readout (row 16w + n, positions 32b + 8g)
      *reinterpret_cast<bf16x8*>(hdst + 32 * b) = Bf[b];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const f4 c_in = (b == 0) ? f4{0, 0, 0, 0} : nxt[c];
        nxt[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Wf[c][b], Bf[b], c_in, 0, 0, 0);
        if constexpr (SPLIT) nxt[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Wf[c][b], Bl[b], nxt[c], 0, 0, 0);
      }
      if (b == 0 && t > 0) readout(t - 1);
    }
    // chunk boundary: publish the prefetched chunk, start the next load
    if (s == kChunk - 1) {
      const int next = t / kChunk + 1;
      if (next < nchunks) {
        st.store(lds, next & 1);
        if (next + 1 < nchunks) st.load(a, unit, row0, next + 1);
      }
    }
    __syncthreads();
  };

  // prologue: H_0 W for step 0
  f4 accA[CT], accB[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    accA[c] = f4{0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      accA[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Wf[c][b], Bf[b], accA[c], 0, 0, 0);
      if constexpr (SPLIT) accA[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Wf[c][b], Bl[b], accA[c], 0, 0, 0);
    }
  }
  __syncthreads();

  int t = 0;
  for (; t + 1 < T; t += 2) {
    step(t, accA, accB);
    step(t + 1, accB, accA);
  }
  if (t < T) step(t, accA, accB);
  readout(T - 1);

  if (a.HT) {
    float* HT = a.HT + (unit * a.K + my_row) * V;
#pragma unroll
    for (int c = 0; c < CT; ++c) *reinterpret_cast<f4*>(HT + 16 * c + 4 * g) = G[c] * kInvC;
  }
}

__global__ void zero_fill_kernel(float* p, long long n) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0.0f;
}

template <int V, int NW, bool SPLIT>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int R = 16 * NW;
  const int splits = a.K / R;
  const long long grid = (long long)a.B * a.H * splits;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (splits > 1 && !a.accumulate) {
    const long long ny = (long long)a.B * a.H * a.T * a.V;
    long long blocks = (ny + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.y, ny);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((mfma_fwd_kernel<V, NW, SPLIT>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

// waves per workgroup: R = 16 * NW rows must divide K, readout needs R >= 32,
// at most two workgroups per unit (so atomic readout sums stay order-free).
int pick_nw(int K) {
  if (K % 64 == 0 && K / 64 <= 2) return 4;
  if (K % 32 == 0 && K / 32 <= 2) return 2;
  return 0;
}

}  // namespace

bool mfma_supports(int K, int V, int bf16) {
  if (!bf16) return false;
  if (V != 64 && V != 128) return false;
  return pick_nw(K) != 0;
}

Plan plan_mfma(int B, int H, int K, int V, bool split) {
  const int nw = pick_nw(K);
  if (!nw || (V != 64 && V != 128)) return Plan{-1, 0, 0, 0, 0, 0};
  const int R = 16 * nw, splits = K / R;
  const long long grid = (long long)B * H * splits;
  int lds = 0;
  if (V == 128) lds = nw == 4 ? Layout<128, 4>::TOTAL : Layout<128, 2>::TOTAL;
  else lds = nw == 4 ? Layout<64, 4>::TOTAL : Layout<64, 2>::TOTAL;
  (void)split;
  return Plan{grid > 0x7fffffffLL ? -1 : (int)grid, 64 * nw, R, splits, splits > 1 ? 1 : 0, lds};
}

hipError_t launch_mfma(const FwdArgs& a, bool split, hipStream_t stream) {
  if (!mfma_supports(a.K, a.V, a.bf16)) return hipErrorInvalidValue;
  const int nw = pick_nw(a.K);
  if (split) {
    if (a.V == 128) return nw == 4 ? launch_t<128, 4, true>(a, stream) : launch_t<128, 2, true>(a, stream);
    return nw == 4 ? launch_t<64, 4, true>(a, stream) : launch_t<64, 2, true>(a, stream);
  }
  if (a.V == 128) return nw == 4 ? launch_t<128, 4, false>(a, stream) : launch_t<128, 2, false>(a, stream);
  return nw == 4 ? launch_t<64, 4, false>(a, stream) : launch_t<64, 2, false>(a, stream);
}

}  // namespace m2rnn
