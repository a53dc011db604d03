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
// i of H_{t-1}), so a unit's K rows are cut into 16-row tiles and each wave (one
// per SIMD) carries one tile through all T steps without talking to any other
// wave. A workgroup of NW waves (R = 16 NW rows) shares the staging of the
// per-step inputs and sums its waves' readouts every kChunk steps; K/R
// workgroups share a unit and add their readout sums into y atomically (at most
// two contributions per element onto a cleared y, so the order cannot change
// the result).
//
// Registers (lane l, g = l / 16, n = l % 16):
//   * the fp32 state, carried scaled as G = c H with c = 2 log2(e) so that exp2
//     of the pre-activation gives e^{2x}; lane (g, n) holds G[n][16 c + 4 g + i]
//     for every 16-column tile c and i < 4 — the output layout of
//     v_mfma_f32_16x16x32_bf16 in the orientation D = W^T G^T;
//   * W (AGPRs, for the whole sequence) as A fragments of that MFMA with the
//     contraction index permuted so that a lane's two consecutive output tiles
//     are, rounded to bf16, exactly its B fragment for the next product:
//     B fragment b, lane (g, n), element j = G[n][32 b + 16 (j/4) + 4 g + j%4].
//     The state never leaves the registers between steps.
// Per step per wave:
//   * products: V/16 x V/32 MFMAs for G_{t-1} W, issued block by block as soon
//     as the previous step's epilogue has produced the operand block
//     (software-pipelined across steps, loop unrolled by two);
//   * rank-1 write: one more MFMA per 16-column tile adds c k_t v_t^T: its A
//     operand carries (v_j, v_j) in one contraction pair, its B operand the
//     bf16 hi/lo split of c k_n in the same pair, zero elsewhere (error about
//     2^-17 relative); v and the k pairs are staged in LDS already packed;
//   * epilogue per element: e = exp2(u), r = 1 / (1 + e), then
//     G <- f G + a - 2 a r with a = (1 - f) c   (tanh(x) = 1 - 2 / (1 + e^{2x}));
//   * the bf16 (round-to-nearest-even) operand of the next product.
// With SPLIT the operand is the pair hi = bf16(G), lo = bf16(G - hi) (the
// residual is exact in fp32) and every product takes two passes, W hi + W lo:
// ~16 significant bits instead of 8 for trajectories that amplify per-step
// rounding (W is a bf16 input, so it is exact either way).
//
// Readout. Each wave writes its rounded state tile to its own LDS slot and,
// every second step, reads the two tiles back transposed with
// ds_read_b64_tr_b16: the column-per-lane A operand of one MFMA per 16 columns
// whose 32-long contraction covers 16 rows x 2 steps against q. Its B operand
// carries q_t only in column t % kChunk, so one accumulator per 16 columns
// collects a whole chunk of steps; at the chunk end the waves' partial sums are
// added in LDS in a fixed order and stored. No barrier is needed between
// chunk ends.
//
// Inputs k, v, q, f are staged chunk by chunk into LDS by the whole workgroup,
// loaded from HBM one chunk ahead of use.
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

__device__ __forceinline__ float bf16_to_f32(unsigned int b) { return __uint_as_float(b << 16); }

typedef __attribute__((ext_vector_type(2))) float f2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32: round to nearest even)
__device__ __forceinline__ unsigned int pack_bf16(float x0, float x1) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f2{x0, x1}, bf16x2));
}

template <int V, int NW>
struct Layout {
  static constexpr int R = 16 * NW;   // rows per workgroup
  static constexpr int CT = V / 16;   // 16-column tiles
  static constexpr int KB = V / 32;   // 32-wide contraction blocks
  // dwords per row and step of the rank-1 A operands: per tile pair k, dwords
  // 4k .. 4k+3 = (v pair of tile 2k, v pair of tile 2k+1, 0, 0), so one aligned
  // 16-byte read is the operand; the 4 padding dwords make those reads
  // conflict-free across a row group
  static constexpr int NVX = 2 * CT + 4;
  static constexpr int HROW = V + 8;  // bf16 per LDS state row (padded)
  // stage buffers: chunk c+1 goes into chunk c-1's buffer early in chunk c, once
  // the readout of chunk c-1's last steps (step 0 of chunk c) is behind a barrier
  static constexpr int NSB = 2;
  static constexpr int NHS = 4;       // state-tile slots per wave (readout lags one step pair)
  static constexpr int THREADS = 64 * NW;
  // LDS regions (bytes)
  static constexpr int KX_BYTES = NSB * kChunk * R * 4;          // (hi, lo) of c k, bf16 pair
  static constexpr int VX_BYTES = NSB * kChunk * 16 * NVX * 4;   // rank-1 A operands, [s][m][.]
  static constexpr int QS_BYTES = NSB * kChunk * R * 2;          // q, bf16
  static constexpr int FS_BYTES = NSB * kChunk * 4 * 4;          // f, a, -2a, pad
  static constexpr int HB_BYTES = NW * NHS * 16 * HROW * 2;      // per-wave state tiles
  static constexpr int YP_BYTES = NW * kChunk * V * 4;           // per-wave partial readouts
  static constexpr int Z_BYTES = 16;                             // zeros
  static constexpr int KX_OFF = 0;
  static constexpr int VX_OFF = KX_OFF + KX_BYTES;
  static constexpr int QS_OFF = VX_OFF + VX_BYTES;
  static constexpr int FS_OFF = QS_OFF + QS_BYTES;
  static constexpr int HB_OFF = FS_OFF + FS_BYTES;
  static constexpr int YP_OFF = HB_OFF + HB_BYTES;
  static constexpr int Z_OFF = YP_OFF + YP_BYTES;
  static constexpr int TOTAL = Z_OFF + Z_BYTES;
  // 16-byte global load slots per chunk
  static constexpr int SLOT_K = kChunk * R / 8;
  static constexpr int SLOT_Q = kChunk * R / 8;
  static constexpr int SLOT_V = kChunk * V / 8;
  static constexpr int SLOTS = SLOT_K + SLOT_Q + SLOT_V;
  static constexpr int SLOTS_PER_THREAD = (SLOTS + THREADS - 1) / THREADS;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Chunk staging: each thread owns up to SLOTS_PER_THREAD 16-byte global slots.
template <int V, int NW>
struct Stager {
  using L = Layout<V, NW>;
  u4 reg[L::SLOTS_PER_THREAD];
  unsigned short freg;  // one gate value (threads < kChunk)

  // chunk `chunk` of a sequence with Tb steps (the row stride is ld)
  __device__ __forceinline__ void load(const FwdArgs& a, long long unit, int row0, int chunk, int Tb) {
    const int tid = threadIdx.x;
    const long long ld = a.ld > 0 ? a.ld : a.T;
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
        if (t < Tb) reg[p] = *reinterpret_cast<const u4*>((isq ? q : k) + (unit * ld + t) * a.K + row0 + 8 * part);
      } else if (slot < L::SLOTS) {
        const int s2 = slot - L::SLOT_K - L::SLOT_Q;
        const int s = s2 / (V / 8), part = s2 % (V / 8);
        const int t = t0 + s;
        if (t < Tb) reg[p] = *reinterpret_cast<const u4*>(v + (unit * ld + t) * V + 8 * part);
      }
    }
    // steps past the sequence's end get gate 1: they leave the state exactly
    // unchanged, and their readouts are never stored
    freg = 0x3f80u;
    if (tid < kChunk && t0 + tid < Tb) freg = f[unit * ld + t0 + tid];
  }

  // Publish into stage buffer `buf`: c k as a bf16 (hi, lo) pair per row, v as
  // (v, v) pairs in [m][c] order, q raw, and the gate scalars.
  __device__ __forceinline__ void store(char* lds, int buf) const {
    const int tid = threadIdx.x;
    unsigned int* kx = reinterpret_cast<unsigned int*>(lds + L::KX_OFF) + buf * kChunk * L::R;
    unsigned int* vx = reinterpret_cast<unsigned int*>(lds + L::VX_OFF) + buf * kChunk * 16 * L::NVX;
    unsigned short* qs = reinterpret_cast<unsigned short*>(lds + L::QS_OFF) + buf * kChunk * L::R;
    float* fs = reinterpret_cast<float*>(lds + L::FS_OFF) + buf * kChunk * 4;
#pragma unroll
    for (int p = 0; p < L::SLOTS_PER_THREAD; ++p) {
      const int slot = tid + p * L::THREADS;
      const u4 r = reg[p];
      if (slot < L::SLOT_K) {
        const int s = slot / (L::R / 8), part = slot % (L::R / 8);
        u4 lo4, hi4;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // elements 2d, 2d+1: c k rounded to bf16 (hi) and the exact residual rounded (lo)
          const float ck0 = __uint_as_float(r[d] << 16) * kC;
          const float ck1 = __uint_as_float(r[d] & 0xffff0000u) * kC;
          const unsigned int hp = pack_bf16(ck0, ck1);
          const unsigned int lp = pack_bf16(ck0 - __uint_as_float(hp << 16), ck1 - __uint_as_float(hp & 0xffff0000u));
          const unsigned int p0 = (hp & 0xffffu) | (lp << 16);
          const unsigned int p1 = (hp >> 16) | (lp & 0xffff0000u);
          if (d < 2) { lo4[2 * d] = p0; lo4[2 * d + 1] = p1; } else { hi4[2 * d - 4] = p0; hi4[2 * d - 3] = p1; }
        }
        *reinterpret_cast<u4*>(kx + s * L::R + 8 * part) = lo4;
        *reinterpret_cast<u4*>(kx + s * L::R + 8 * part + 4) = hi4;
      } else if (slot < L::SLOT_K + L::SLOT_Q) {
        const int s2 = slot - L::SLOT_K;
        const int s = s2 / (L::R / 8), part = s2 % (L::R / 8);
        *reinterpret_cast<u4*>(qs + s * L::R + 8 * part) = r;
      } else if (slot < L::SLOTS) {
        const int s2 = slot - L::SLOT_K - L::SLOT_Q;
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

// Workgroup barrier that orders LDS only. Global loads (the chunk prefetch) and
// the atomic y updates stay in flight across it; a full __syncthreads would
// wait for them, i.e. for a whole HBM round trip at every chunk end.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Issue order for one pipeline phase: each matrix instruction followed by NV
// vector-ALU instructions, so the matrix core works while the wave issues the
// epilogue (a wave issues in order: back-to-back MFMAs leave the VALU idle).
template <int NM, int NV>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);  // NV VALU
  }
}
// VALU instructions after each MFMA (measured on C3: phase 0 has 14 MFMAs, the
// readout phase 16, the others 8, against ~44 VALU of epilogue each)
constexpr int kNvPhase0 = 3, kNvReadout = 2, kNvPhase = 5;
// the same for the two-pass variant (twice the product MFMAs)
constexpr int kNvPhase0Split = 1, kNvReadoutSplit = 1, kNvPhaseSplit = 3;

__device__ __forceinline__ f4 mfma(const bf16x8& a, const bf16x8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int V, int NW, bool SPLIT, bool SAVE>
__global__ __launch_bounds__(64 * NW, 1) void mfma_fwd_kernel(FwdArgs a) {
  using L = Layout<V, NW>;
  constexpr int R = L::R, CT = L::CT, KB = L::KB, HROW = L::HROW, NVX = L::NVX, NSB = L::NSB, NHS = L::NHS;
  static_assert(KB >= 2 && CT == 2 * KB, "V must be a multiple of 32, at least 64");
  __shared__ __attribute__((aligned(16))) char lds[L::TOTAL];

  const int tid = threadIdx.x;
  const int w = tid / 64, l = tid % 64, g = l / 16, n = l % 16;
  const int splits = a.K / R;
  const long long unit = blockIdx.x / splits;
  const int row0 = (blockIdx.x % splits) * R;
  const int h = static_cast<int>(unit % a.H);
  const int T = a.T;                                  // steps of this call
  const long long LD = a.ld > 0 ? a.ld : a.T;          // row stride of the per-step inputs and of y
  // this sequence's length (all of T unless lengths are given)
  const int Tb = a.lens ? min(max(a.lens[unit / a.H], 0), T) : T;
  const int my_row = row0 + 16 * w + n;  // state row this lane carries (within the unit)

  const unsigned int* kx_all = reinterpret_cast<const unsigned int*>(lds + L::KX_OFF);
  unsigned int* vx_all = reinterpret_cast<unsigned int*>(lds + L::VX_OFF);
  const unsigned short* qs_all = reinterpret_cast<const unsigned short*>(lds + L::QS_OFF);
  const float* fs_all = reinterpret_cast<const float*>(lds + L::FS_OFF);
  unsigned short* hb_w = reinterpret_cast<unsigned short*>(lds + L::HB_OFF) + w * NHS * 16 * HROW;
  float* yp_all = reinterpret_cast<float*>(lds + L::YP_OFF);
  const unsigned int* zero_lds = reinterpret_cast<const unsigned int*>(lds + L::Z_OFF);

  // ---- prologue. Every global read of the prologue (W, H0, chunks 0 and 1) is
  // issued before the first wait, so their latencies overlap.
  Stager<V, NW> st, st1;
  const int nchunks = (Tb + kChunk - 1) / kChunk;
  st.load(a, unit, row0, 0, Tb);
  if (nchunks > 1) st1.load(a, unit, row0, 1, Tb);
  constexpr int WLOADS = V * V / 8 / L::THREADS;  // 16-byte pieces of W per thread
  static_assert(WLOADS * 8 * L::THREADS == V * V, "W splits evenly over the workgroup");
  u4 wreg[WLOADS];
  {
    const u4* Wg = reinterpret_cast<const u4*>(static_cast<const unsigned short*>(a.W) + (long long)h * V * V);
#pragma unroll
    for (int p = 0; p < WLOADS; ++p) wreg[p] = Wg[tid + p * L::THREADS];
  }
  f4 h0v[CT];
  {
    const float* H0 = a.H0 ? a.H0 + (unit * a.K + my_row) * V : nullptr;
#pragma unroll
    for (int c = 0; c < CT; ++c) h0v[c] = H0 ? *reinterpret_cast<const f4*>(H0 + 16 * c + 4 * g) : f4{0, 0, 0, 0};
  }

  // ---- W as permuted A fragments: Wf[c][b] lane (g,n) = W[32b + 16(j/4) + 4g + j%4][16c + n].
  // The head's W goes through LDS (the state-tile region, not yet in use), and
  // each fragment comes back as two transposing reads.
  bf16x8 Wf[CT][KB];
  {
    constexpr int WROW = HROW;  // padded row, as the state tiles
    static_assert(V * WROW * 2 <= L::HB_BYTES, "W fits in the state-tile region");
    unsigned short* wst = reinterpret_cast<unsigned short*>(lds + L::HB_OFF);
#pragma unroll
    for (int p = 0; p < WLOADS; ++p) {
      const int i = tid + p * L::THREADS;
      *reinterpret_cast<u4*>(wst + (i / (V / 8)) * WROW + 8 * (i % (V / 8))) = wreg[p];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        // lane (g, n) points at row 32b + 4g + n/4, columns 16c + 4(n%4) ..+3; the
        // transpose hands it column 16c + n of rows 32b + 4g .. +3 (and +16 .. +19)
        const unsigned short* src = wst + (32 * b + 4 * g + n / 4) * WROW + 16 * c + 4 * (n % 4);
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)src);
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * WROW));
        s8 wa = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        // pin the fragment to the accumulation registers: it is only ever a
        // matrix operand, and this leaves the arch VGPRs to the epilogue
        asm volatile("" : "=a"(wa) : "0"(wa));
        Wf[c][b] = __builtin_bit_cast(bf16x8, wa);
      }
    lds_barrier();  // every wave has its fragments before the region is cleared
  }

  // ---- one-time LDS init: the zero dwords of the rank-1 operands, the state tiles,
  // the zero word; then chunks 0 and 1 into the stage buffers (other addresses)
  for (int i = tid; i < NSB * kChunk * 16; i += L::THREADS)
#pragma unroll
    for (int k = 0; k < CT / 2; ++k) *reinterpret_cast<uint2*>(vx_all + i * NVX + 4 * k + 2) = uint2{0u, 0u};
  for (int i = tid; i < L::HB_BYTES / 4; i += L::THREADS)
    reinterpret_cast<unsigned int*>(lds + L::HB_OFF)[i] = 0u;
  if (tid < 4) reinterpret_cast<unsigned int*>(lds + L::Z_OFF)[tid] = 0u;
  st.store(lds, 0);
  if (nchunks > 1) st1.store(lds, 1);
  if (nchunks > 2) st.load(a, unit, row0, 2, Tb);  // staged early in chunk 1

  // ---- scaled fp32 state G = c H, output layout
  f4 G[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) G[c] = h0v[c] * kC;
  bf16x8 Bf[KB], Bl[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b) make_operand<SPLIT>(G[2 * b], G[2 * b + 1], Bf[b], Bl[b]);
  // training forward: this row tile's 16-byte piece of a saved slot, per block b
  [[maybe_unused]] char* const saved = static_cast<char*>(a.saved);
  [[maybe_unused]] const long long rt_off = (long long)(row0 / 16 + w) * (V / 32) * 1024 + l * 16;
  if constexpr (SAVE) {
#pragma unroll
    for (int b = 0; b < KB; ++b)
      *reinterpret_cast<bf16x8*>(saved + saved_state_off(unit, 0, T, a.K, V) + rt_off + b * 1024) = Bf[b];
  }
  lds_barrier();  // staged chunks and zeroed tiles visible; the chunk-2 loads stay in flight

  // one stage buffer's views
  struct Buf {
    const unsigned int* kx;
    const unsigned int* vx;
    const unsigned short* qs;
    const float* fs;
  };
  auto buf = [&](int sb) {
    return Buf{kx_all + sb * kChunk * R, vx_all + sb * kChunk * 16 * NVX, qs_all + sb * kChunk * R,
               fs_all + sb * kChunk * 4};
  };

  // rank-1 write of a step as the initial accumulator: acc[c] = (v, tile c) x (hi, lo of c k).
  struct R1 {
    unsigned int kpair;
    u4 win[CT / 2];  // tile pair k: (v pair of tile 2k, of tile 2k+1, 0, 0)
  };
  auto rank1_load = [&](const Buf& B, int s) {
    R1 r;
    const unsigned int* kp = (g == 0) ? B.kx + s * R + 16 * w + n : zero_lds;
    r.kpair = *kp;
    const unsigned int* vp = B.vx + (s * 16 + n) * NVX;
#pragma unroll
    for (int k = 0; k < CT / 2; ++k) r.win[k] = *reinterpret_cast<const u4*>(vp + 4 * k);
    return r;
  };
  auto rank1_init = [&](const R1& r, f4 (&acc)[CT]) {
    const u4 bx0 = u4{r.kpair, 0u, 0u, 0u};
    const u4 bx1 = u4{0u, r.kpair, 0u, 0u};
#pragma unroll
    for (int c = 0; c < CT; ++c)
      acc[c] = mfma(__builtin_bit_cast(bf16x8, r.win[c / 2]), __builtin_bit_cast(bf16x8, (c & 1) ? bx1 : bx0),
                    f4{0, 0, 0, 0});
  };

  // readout partials: Dr[P] lane (g, n) accumulates y_{t0 + n}[position 16 P + 4 g + i]
  // over this wave's 16 rows, t0 the chunk start.
  f4 Dr[CT];
#pragma unroll
  for (int p = 0; p < CT; ++p) Dr[p] = f4{0, 0, 0, 0};

  // readout of the steps s0, s0 + 1 (s0 even) of the chunk in B, state tiles in
  // slots s0 & 3 and (s0 + 1) & 3; step s0 + p contributes only if p < nvalid
  auto readout = [&](const Buf& B, int s0, int nvalid) {
    const int p = g / 2;                 // which step of the pair this lane group carries
    const int rr = 8 * (g % 2);          // first of its 8 rows
    const int s = s0 + p;
    s8 qv = *reinterpret_cast<const s8*>(B.qs + s * R + 16 * w + rr);
    if (n != s || p >= nvalid) qv = s8{0, 0, 0, 0, 0, 0, 0, 0};
    const bf16x8 Bq = __builtin_bit_cast(bf16x8, qv);
    // source lane (g, n): row rr + n/4 (+4) of the step's slot, positions 16 P + 4 (n % 4)
    const unsigned short* src = hb_w + (s & (NHS - 1)) * 16 * HROW + (rr + n / 4) * HROW + 4 * (n % 4);
#pragma unroll
    for (int P = 0; P < CT; ++P) {
      const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * P));
      const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s4*)(src + 16 * P + 4 * HROW));
      const s8 av = s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      Dr[P] = mfma(__builtin_bit_cast(bf16x8, av), Bq, Dr[P]);
    }
  };

  float* y = a.y;
  const bool atomic_y = splits > 1 || a.accumulate;

  // y for the steps t0 .. t0 + nsteps - 1 of one chunk from the summed partials
  auto ysum_group = [&](int t0, int grp) {
    const int sn = grp / (V / 4), pos = 4 * (grp % (V / 4));
    f4 sum = *reinterpret_cast<const f4*>(yp_all + sn * V + pos);
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += *reinterpret_cast<const f4*>(yp_all + (ww * kChunk + sn) * V + pos);
    sum *= kInvC;
    // position 16 P + 4 gg  ->  column 32 (P/2) + 16 (gg%2) + 8 (P%2) + 4 (gg/2)
    const int P = pos / 16, gg = (pos % 16) / 4;
    const int col = 32 * (P / 2) + 16 * (gg % 2) + 8 * (P % 2) + 4 * (gg / 2);
    if (y == nullptr) return;  // states recomputed for the backward pass: no readout wanted
    float* dst = y + (unit * LD + t0 + sn) * V + col;
    if (atomic_y) {
#pragma unroll
      for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dst + i, sum[i]);
    } else {
      *reinterpret_cast<f4*>(dst) = sum;
    }
  };

  // Chunk end, spread over the first steps of the next chunk so that its LDS
  // round trips overlap with their compute:
  //   step 0 (end): publish the waves' partial readouts of the finished chunk
  //                 (Dr, which that step's readout has just completed); LDS barrier
  //   step 1:       stage the next chunk from the registers loaded a chunk ago,
  //                 then fetch the one after it
  //   steps 2..:    sum the partials into y, one group per step and thread
  //   step kSync:   LDS barrier: the staged chunk is visible before the step
  //                 that first prefetches from it (step 14), and every wave has
  //                 summed before the next chunk end overwrites the partials
  constexpr int kGroups = kChunk * (V / 4) / L::THREADS;  // y-sum groups per thread
  static_assert(kGroups * L::THREADS == kChunk * (V / 4), "whole groups per thread");
  constexpr int kSync = 8;
  static_assert(2 + kGroups <= kSync && kSync < kChunk - 2, "chunk-end schedule");
  auto publish = [&]() {
    float* ypw = yp_all + w * kChunk * V;
#pragma unroll
    for (int P = 0; P < CT; ++P) *reinterpret_cast<f4*>(ypw + n * V + 16 * P + 4 * g) = Dr[P];
#pragma unroll
    for (int P = 0; P < CT; ++P) Dr[P] = f4{0, 0, 0, 0};
    lds_barrier();
  };
  auto stage_next = [&](int c1) {
    if (c1 < nchunks) {
      st.store(lds, c1 % NSB);
      if (c1 + 1 < nchunks) st.load(a, unit, row0, c1 + 1, Tb);
    }
  };
  auto chunk_end_work = [&](int s, int c) {
    if (s == 0) publish();
    if (s == 1) stage_next(c + 1);
    if (s >= 2 && s < 2 + kGroups) ysum_group((c - 1) * kChunk, tid + (s - 2) * L::THREADS);
    if (s == kSync) lds_barrier();
  };

  // epilogue of state tiles 2b, 2b+1: tanh via exp2/rcp, gate blend, next operand
  // block, rounded tile to the readout slot
  auto epilogue = [&](int b, const f4 (&cur)[CT], float fg, float av, float m2a, unsigned short* hdst, int t) {
    if constexpr (SAVE) {
      // the pre-activation c A_t of tiles 2b, 2b+1, as bf16
      if (t < T) {
        const f4 u0 = cur[2 * b], u1 = cur[2 * b + 1];
        const u4 pk = u4{pack_bf16(u0[0], u0[1]), pack_bf16(u0[2], u0[3]), pack_bf16(u1[0], u1[1]),
                         pack_bf16(u1[2], u1[3])};
        *reinterpret_cast<u4*>(saved + saved_pre_off(unit, t, a.B, a.H, T, a.K, V) + rt_off + b * 1024) = pk;
      }
    }
#pragma unroll
    for (int c = 2 * b; c < 2 * b + 2; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(cur[c][i]);
        const float r = __builtin_amdgcn_rcpf(1.0f + e);
        G[c][i] = fmaf(m2a, r, fmaf(fg, G[c][i], av));
      }
    }
    make_operand<SPLIT>(G[2 * b], G[2 * b + 1], Bf[b], Bl[b]);
    *reinterpret_cast<bf16x8*>(hdst + 32 * b) = Bf[b];
    if constexpr (SAVE) {
      if (t < T) *reinterpret_cast<bf16x8*>(saved + saved_state_off(unit, t + 1, T, a.K, V) + rt_off + b * 1024) = Bf[b];
    }
  };

  auto products = [&](int b, int c_lo, int c_hi, f4 (&acc)[CT]) {
#pragma unroll
    for (int c = c_lo; c < c_hi; ++c) {
      acc[c] = mfma(Wf[c][b], Bf[b], acc[c]);
      if constexpr (SPLIT) acc[c] = mfma(Wf[c][b], Bl[b], acc[c]);
    }
  };

  // per-step operands fetched ahead: the gate scalars of the next step and the
  // rank-1 operands of the step after it
  struct Pre {
    f4 fs;
    R1 r1;
  };

  // Step s of chunk c (C, Cn, Cp: the stage buffers of chunks c, c + 1, c - 1).
  // On entry `cur` holds c (G_{t-1} W + k_t v_t^T) except the last operand
  // block's share for tiles 2.., which phase 0 adds. The next step's
  // accumulators `nxt` start from its rank-1 write and take operand block b
  // right after the epilogue has produced it; block KB-1 is finished for tiles
  // 0, 1 here and for the other tiles in the next step's phase 0.
  auto step = [&](const int s, f4 (&cur)[CT], f4 (&nxt)[CT], Pre& pre, const Buf& C, const Buf& Cn,
                  const Buf& Cp, const int c) {
    const float fg = pre.fs[0], av = pre.fs[1], m2a = pre.fs[2];
    unsigned short* hdst = hb_w + (s & (NHS - 1)) * 16 * HROW + n * HROW + 8 * g;
    // phase 0
    products(KB - 1, 2, CT, cur);
    if constexpr (SPLIT)  // no registers to spare for the early fetch
      rank1_init(s + 1 < kChunk ? rank1_load(C, s + 1) : rank1_load(Cn, s + 1 - kChunk), nxt);
    else
      rank1_init(pre.r1, nxt);
    pre.fs = *reinterpret_cast<const f4*>(s + 1 < kChunk ? C.fs + (s + 1) * 4 : Cn.fs + (s + 1 - kChunk) * 4);
    if constexpr (!SPLIT) pre.r1 = s + 2 < kChunk ? rank1_load(C, s + 2) : rank1_load(Cn, s + 2 - kChunk);
    epilogue(0, cur, fg, av, m2a, hdst, c * kChunk + s);
    interleave_mfma<(SPLIT ? 2 : 1) * (CT - 2) + CT, SPLIT ? kNvPhase0Split : kNvPhase0>();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 1; b < KB; ++b) {
      products(b - 1, 0, CT, nxt);
      if (b == 1 && s % 2 == 0) {
        // the previous two steps; at a chunk start they close the previous chunk
        if (s >= 2) readout(C, s - 2, 2);
        else readout(Cp, kChunk - 2, c > 0 ? 2 : 0);
      }
      epilogue(b, cur, fg, av, m2a, hdst, c * kChunk + s);
      if (b == 1 && s % 2 == 0)
        interleave_mfma<(SPLIT ? 2 : 1) * CT + CT, SPLIT ? kNvReadoutSplit : kNvReadout>();
      else
        interleave_mfma<(SPLIT ? 2 : 1) * CT, SPLIT ? kNvPhaseSplit : kNvPhase>();
      __builtin_amdgcn_sched_barrier(0);
    }
    products(KB - 1, 0, 2, nxt);
    if (c > 0) chunk_end_work(s, c);
  };

  // prologue: c (H_0 W + k_0 v_0^T) for step 0, last operand block for tiles 0, 1 only
  f4 accA[CT], accB[CT];
  rank1_init(rank1_load(buf(0), 0), accA);
#pragma unroll
  for (int b = 0; b < KB - 1; ++b) products(b, 0, CT, accA);
  products(KB - 1, 0, 2, accA);
  Pre pre;
  pre.fs = *reinterpret_cast<const f4*>(buf(0).fs);
  if constexpr (!SPLIT) pre.r1 = rank1_load(buf(0), 1);

  // Chunks of 16 steps in pairs; the last chunk stops after the pair that holds
  // the sequence's last step (the pair's second step may be an identity step).
  for (int c = 0; c < nchunks; ++c) {
    const Buf C = buf(c % NSB), Cn = buf((c + 1) % NSB), Cp = buf((c + NSB - 1) % NSB);
    const int ns = c == nchunks - 1 ? Tb - c * kChunk : kChunk;  // real steps in this chunk
#pragma unroll
    for (int s = 0; s < kChunk; s += 2) {
      step(s, accA, accB, pre, C, Cn, Cp, c);
      step(s + 1, accB, accA, pre, C, Cn, Cp, c);
      if (s + 2 >= ns) break;
    }
  }
  // the last chunk's pending steps and its y
  if (nchunks > 0) {
    const int c = nchunks - 1;
    const int ns = Tb - c * kChunk;
    if (c > 0) {
      // the previous chunk's y groups a short last chunk did not reach, before
      // the partials are overwritten
      const int done = min(max(((ns + 1) & ~1) - 2, 0), kGroups);
      for (int i = done; i < kGroups; ++i) ysum_group((c - 1) * kChunk, tid + i * L::THREADS);
      lds_barrier();
    }
    const int te = (ns - 1) & ~1;
    readout(buf(c % NSB), te, min(ns - te, 2));
    publish();
    const int t0 = c * kChunk;
    for (int grp = tid; grp < ns * (V / 4); grp += L::THREADS) ysum_group(t0, grp);
  }

  if (a.HT) {
    float* HT = a.HT + (unit * a.K + my_row) * V;
    const float* H0 = a.H0 ? a.H0 + (unit * a.K + my_row) * V : nullptr;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      f4 x = G[c] * kInvC;
      if (nchunks == 0)  // an empty sequence hands H0 back unchanged
        x = H0 ? *reinterpret_cast<const f4*>(H0 + 16 * c + 4 * g) : f4{0, 0, 0, 0};
      *reinterpret_cast<f4*>(HT + 16 * c + 4 * g) = x;
    }
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
  // y starts at zero when two workgroups add into it, or when sequences end
  // early (their remaining rows read as zero)
  if ((splits > 1 || a.lens) && !a.accumulate && a.y) {
    if (a.ld > 0 && a.ld != a.T) return hipErrorInvalidValue;  // a window of y: the caller clears it
    hipError_t e = fill_zero(a.y, (long long)a.B * a.H * a.T * a.V, stream);
    if (e != hipSuccess) return e;
  }
  if (a.saved)
    hipLaunchKernelGGL((mfma_fwd_kernel<V, NW, SPLIT, true>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, a);
  else
    hipLaunchKernelGGL((mfma_fwd_kernel<V, NW, SPLIT, false>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

// waves per workgroup: R = 16 NW rows must divide K, at most two workgroups per
// unit (so atomic readout sums stay order-free).
int pick_nw(int K) {
  if (K % 64 == 0 && K / 64 <= 2) return 4;
  if (K % 32 == 0 && K / 32 <= 2) return 2;
  return 0;
}

template <int V>
int lds_bytes(int nw) {
  return nw == 4 ? Layout<V, 4>::TOTAL : Layout<V, 2>::TOTAL;
}

}  // namespace

hipError_t fill_zero(float* p, long long n, hipStream_t stream) {
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

bool mfma_supports(int K, int V, int bf16) {
  if (!bf16) return false;
  if (V != 64 && V != 128) return false;
  return pick_nw(K) != 0;
}

Plan plan_mfma(int B, int H, int K, int V, bool split) {
  (void)split;
  const int nw = pick_nw(K);
  if (!nw || (V != 64 && V != 128)) return Plan{-1, 0, 0, 0, 0, 0};
  const int R = 16 * nw, splits = K / R;
  const long long grid = (long long)B * H * splits;
  const int lds = V == 128 ? lds_bytes<128>(nw) : lds_bytes<64>(nw);
  return Plan{grid > 0x7fffffffLL ? -1 : (int)grid, 64 * nw, R, splits, splits > 1 ? 1 : 0, lds};
}

Plan plan_decode(int B, int H, int K, int V) {
  const long long grid = (long long)H * decode_splits(B, H);
  const int lds = (V * (V + 8)) * 2 + 2 * 8 * V * 4;
  return Plan{grid > 0x7fffffffLL ? -1 : (int)grid, 256, 16, K / 16, 0, lds};
}

hipError_t launch_mfma(const FwdArgs& a, bool split, hipStream_t stream) {
  if (!mfma_supports(a.K, a.V, a.bf16)) return hipErrorInvalidValue;
  if (decode_supports(a)) return launch_decode(a, stream);  // one step: the decoding kernel
  const int nw = pick_nw(a.K);
  if (split) {
    if (a.V == 128) return nw == 4 ? launch_t<128, 4, true>(a, stream) : launch_t<128, 2, true>(a, stream);
    return nw == 4 ? launch_t<64, 4, true>(a, stream) : launch_t<64, 2, true>(a, stream);
  }
  if (a.V == 128) return nw == 4 ? launch_t<128, 4, false>(a, stream) : launch_t<128, 2, false>(a, stream);
  return nw == 4 ? launch_t<64, 4, false>(a, stream) : launch_t<64, 2, false>(a, stream);
}

}  // namespace m2rnn
