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
// rounding (W is a bf16 input, so it is exact either way). With F16 the single
// operand is fp16 instead (11 significant bits, the same MFMA rate and layout on
// v_mfma_f32_16x16x32_f16; W and q converted once, exactly inside fp16's range,
// and a value beyond that range turned into NaN).
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

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

using namespace dev;

constexpr int kChunk = 16;                     // steps staged per LDS chunk

template <int V, int NW, bool SPLIT>
struct Layout {
  static constexpr int R = 16 * NW;   // rows per workgroup
  static constexpr int CT = V / 16;   // 16-column tiles
  static constexpr int KB = V / 32;   // 32-wide contraction blocks
  // dwords per row and step of the rank-1 A operands: per tile pair k, dwords
  // 2k, 2k+1 = (v pair of tile 2k, v pair of tile 2k+1), one aligned 8-byte read;
  // the 2 padding dwords put the 16 rows a 16-lane group reads on distinct banks
  static constexpr int NVX = CT + 2;
  static constexpr int HROW = V + 8;  // bf16 per LDS state row (padded)
  // floats per row of the partial readouts: the 4-float pad puts the 16 rows a
  // publishing 16-lane group writes on distinct banks (unpadded, all 16 hit the same)
  static constexpr int YROW = V + 4;
  // One LDS barrier per chunk where three stage buffers and two partial-readout
  // buffers fit (the single operand): chunk c+2 is staged early in chunk c into
  // chunk c-1's buffer and becomes visible at the next chunk's barrier, and the
  // partials alternate between buffers. Otherwise (the split operand, whose
  // state tiles take twice the room) two buffers of each and a second barrier
  // per chunk: chunk c+1 is staged early in chunk c and made visible mid-chunk,
  // and the partials are summed before that barrier.
  static constexpr bool ONEBAR = !SPLIT;
  static constexpr int NSB = ONEBAR ? 3 : 2;
  static constexpr int NYP = ONEBAR ? 2 : 1;
  // state-tile slots per wave: a step pair's readout operands are read at the
  // start of the next pair, before its first step overwrites the older slot
  static constexpr int NHS = 2;
  static constexpr int NPL = SPLIT ? 2 : 1;  // planes per slot: bf16 hi (and lo with SPLIT)
  static constexpr int THREADS = 64 * NW;
  // LDS regions (bytes)
  static constexpr int KX_BYTES = NSB * kChunk * R * 4;          // (hi, lo) of c k, bf16 pair
  static constexpr int VX_BYTES = NSB * kChunk * 16 * NVX * 4;   // rank-1 A operands, [s][m][.]
  static constexpr int QS_BYTES = NSB * kChunk * R * 2;          // q, bf16
  static constexpr int FS_BYTES = NSB * kChunk * 4 * 4;          // f, a, -2a, pad
  static constexpr int HB_BYTES = NW * NHS * NPL * 16 * HROW * 2;  // per-wave state tiles
  static constexpr int YP_BYTES = NYP * NW * kChunk * YROW * 4;  // per-wave partial readouts
  static constexpr int Z_BYTES = 16;                             // zeros
  static constexpr int KX_OFF = 0;
  static constexpr int VX_OFF = KX_OFF + KX_BYTES;
  static constexpr int QS_OFF = VX_OFF + VX_BYTES;
  static constexpr int FS_OFF = QS_OFF + QS_BYTES;
  static constexpr int HB_OFF = FS_OFF + FS_BYTES;
  static constexpr int YP_OFF = HB_OFF + HB_BYTES;
  static constexpr int Z_OFF = YP_OFF + YP_BYTES;
  // before the loop the head's W (V padded rows) is staged from HB_OFF on, over
  // the state tiles and, if they are smaller, the partial readouts
  static constexpr int W_STAGE_BYTES = V * HROW * 2;
  static constexpr int TOTAL = (Z_OFF + Z_BYTES > HB_OFF + W_STAGE_BYTES) ? Z_OFF + Z_BYTES : HB_OFF + W_STAGE_BYTES;
  // 16-byte global load slots per chunk
  static constexpr int SLOT_K = kChunk * R / 8;
  static constexpr int SLOT_Q = kChunk * R / 8;
  static constexpr int SLOT_V = kChunk * V / 8;
  static constexpr int SLOTS = SLOT_K + SLOT_Q + SLOT_V;
  static constexpr int SLOTS_PER_THREAD = (SLOTS + THREADS - 1) / THREADS;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// Chunk staging: each thread owns up to SLOTS_PER_THREAD 16-byte global slots.
// F16: q is staged as fp16 (the readout's operand type).
template <int V, int NW, bool SPLIT, bool F16 = false>
struct Stager {
  using L = Layout<V, NW, SPLIT>;
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
  // (v, v) pairs in [m][c] order, q (raw, or fp16 with F16), and the gate scalars.
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
        if constexpr (F16)
          *reinterpret_cast<f16x8*>(qs + s * L::R + 8 * part) = bf16x8_to_f16(__builtin_bit_cast(s8, r));
        else
          *reinterpret_cast<u4*>(qs + s * L::R + 8 * part) = r;
      } else if (slot < L::SLOTS) {
        const int s2 = slot - L::SLOT_K - L::SLOT_Q;
        const int s = s2 / (V / 8), part = s2 % (V / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int col = 8 * part + i;
          const unsigned int raw = (r[i / 2] >> (16 * (i % 2))) & 0xffffu;
          const int tile = col / 16;
          vx[(s * 16 + col % 16) * L::NVX + 2 * (tile / 2) + tile % 2] = raw | (raw << 16);
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
template <bool SPLIT, typename Op>
__device__ __forceinline__ void make_operand(const f4& g0, const f4& g1, Op& hi, Op& lo) {
  f8 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[i] = g0[i]; x[4 + i] = g1[i]; }
  hi = __builtin_convertvector(x, Op);
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

template <int V, int NW, bool SPLIT, bool SAVE, bool F16>
__global__ __launch_bounds__(64 * NW, 1) void mfma_fwd_kernel(FwdArgs a) {
  using L = Layout<V, NW, SPLIT>;
  // the state operand's type: bf16, or fp16 (F16: one operand, no saved data)
  static_assert(!F16 || (!SPLIT && !SAVE), "the fp16 operand is a single-operand forward");
  using Op = std::conditional_t<F16, f16x8, bf16x8>;
  constexpr int R = L::R, CT = L::CT, KB = L::KB, HROW = L::HROW, NVX = L::NVX, NSB = L::NSB, NHS = L::NHS;
  constexpr int NPL = L::NPL;
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
  unsigned short* hb_w = reinterpret_cast<unsigned short*>(lds + L::HB_OFF) + w * NHS * NPL * 16 * HROW;
  float* yp_all = reinterpret_cast<float*>(lds + L::YP_OFF);
  const unsigned int* zero_lds = reinterpret_cast<const unsigned int*>(lds + L::Z_OFF);

  // ---- prologue. Every global read of the prologue (W, H0, chunks 0 and 1) is
  // issued before the first wait, so their latencies overlap.
  Stager<V, NW, SPLIT, F16> st, st1;
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
  Op Wf[CT][KB];
  {
    constexpr int WROW = HROW;  // padded row, as the state tiles
    static_assert(L::HB_OFF + V * WROW * 2 <= L::TOTAL, "W fits in the staging region");
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
        if constexpr (F16) wa = __builtin_bit_cast(s8, bf16x8_to_f16(wa));
        // pin the fragment to the accumulation registers: it is only ever a
        // matrix operand, and this leaves the arch VGPRs to the epilogue
        asm volatile("" : "=a"(wa) : "0"(wa));
        Wf[c][b] = __builtin_bit_cast(Op, wa);
      }
    lds_barrier();  // every wave has its fragments before the region is cleared
  }

  // ---- one-time LDS init: the state tiles, the zero word; then chunks 0 and 1
  // into the stage buffers (other addresses)
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
  if constexpr (F16) {
    // an initial state beyond the fp16 operand's range is NaN from the start;
    // with gates in [0, 1] the state never grows past max(1, max |H0|) after it
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) G[c][i] = f16_range_or_nan(G[c][i]);
  }
  Op Bf[KB], Bl[KB];
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
    uint2 win[CT / 2];  // tile pair k: (v pair of tile 2k, v pair of tile 2k+1)
  };
  auto rank1_load = [&](const Buf& B, int s) {
    R1 r;
    const unsigned int* kp = (g == 0) ? B.kx + s * R + 16 * w + n : zero_lds;
    r.kpair = *kp;
    const unsigned int* vp = B.vx + (s * 16 + n) * NVX;
#pragma unroll
    for (int k = 0; k < CT / 2; ++k) r.win[k] = *reinterpret_cast<const uint2*>(vp + 2 * k);
    return r;
  };

  // readout partials: Dr[P] lane (g, n) accumulates y_{t0 + n}[position 16 P + 4 g + i]
  // over this wave's 16 rows, t0 the chunk start.
  f4 Dr[CT];
#pragma unroll
  for (int p = 0; p < CT; ++p) Dr[p] = f4{0, 0, 0, 0};

  // Readout of a step pair (s0, s0 + 1), s0 even, on step s0 + 2: the transposed
  // state tiles of both steps (slots s0 & 1 and (s0 + 1) & 1; with SPLIT the low
  // halves too) and q, read half the tiles at a time a phase before their MFMAs.
  // The step writes its own state tiles at its end, after these reads.
  constexpr int HT = CT / 2;  // tiles per readout half
  struct RO {
    Op a[NPL][HT];  // A operand per plane (hi, lo) and 16-column tile of the half
  };
  auto readout_q = [&](const Buf& B, int s0, int nvalid) {
    const int p = g / 2;                 // which step of the pair this lane group carries
    const int rr = 8 * (g % 2);          // first of its 8 rows
    const int s = s0 + p;
    // q_{s0 + p} in column s0 + p (p < nvalid), zero elsewhere. With the split
    // operand every lane loads and the lanes of other columns mask their q to
    // zero (1.2 % faster on C3 than the load under a lane condition, which
    // compiles into exec-mask changes); with one operand the conditional load
    // measured 0.4-0.8 % faster.
    if constexpr (SPLIT) {
      const u4 qv = *reinterpret_cast<const u4*>(B.qs + s * R + 16 * w + rr) & ((n != s || p >= nvalid) ? 0u : ~0u);
      return __builtin_bit_cast(Op, qv);
    } else {
      s8 qv = *reinterpret_cast<const s8*>(B.qs + s * R + 16 * w + rr);
      if (n != s || p >= nvalid) qv = s8{0, 0, 0, 0, 0, 0, 0, 0};
      return __builtin_bit_cast(Op, qv);
    }
  };
  auto readout_load = [&](int s0, int half) {
    RO ro;
    const int p = g / 2, rr = 8 * (g % 2), s = s0 + p;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl) {
      // source lane (g, n): row rr + n/4 (+4) of the step's slot, positions 16 P + 4 (n % 4)
      const unsigned short* src =
          hb_w + ((s & (NHS - 1)) * NPL + pl) * 16 * HROW + (rr + n / 4) * HROW + 4 * (n % 4);
#pragma unroll
      for (int i = 0; i < HT; ++i) {
        const int P = half * HT + i;
        const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(src + 16 * P));
        const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4*)(src + 16 * P + 4 * HROW));
        ro.a[pl][i] = __builtin_bit_cast(Op, s8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
    }
    return ro;
  };
  // readout MFMA j (< NPL HT) of a half
  auto readout_mma = [&](const RO& ro, const Op& bq, int half, int j) {
    const int pl = j / HT, i = j % HT;
    Dr[half * HT + i] = mfma(ro.a[pl][i], bq, Dr[half * HT + i]);
  };
  constexpr int NRH = NPL * HT;  // readout MFMAs per half

  float* y = a.y;
  const bool atomic_y = splits > 1 || a.accumulate;

  // y of one group (a step and 4 columns) of the chunk starting at t0, from the
  // waves' partials in partial buffer yb, added in wave order. The partials sit
  // in the permuted order of the readout: position 16 P + 4 gg + i holds column
  // 32 (P/2) + 16 (gg%2) + 8 (P%2) + 4 (gg/2) + i.
  auto ysum_group = [&](int t0, int grp, int yb) {
    const float* ypb = yp_all + yb * NW * kChunk * L::YROW;
    const int sn = grp / (V / 4), j = grp % (V / 4);
    if (y == nullptr) return;  // states recomputed for the backward pass: no readout wanted
    // (the split-operand and saving forwards keep one 16-byte group per lane for
    // their atomic adds too: the column-spread adds below cost those kernels
    // more LDS reads and registers than the write traffic they save; measured
    // 1.3% slower with the split operand)
    if (!atomic_y || SAVE || SPLIT) {
      // four consecutive columns, one 16-byte store
      const int pos = 4 * j;
      f4 sum = *reinterpret_cast<const f4*>(ypb + sn * L::YROW + pos);
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) sum += *reinterpret_cast<const f4*>(ypb + (ww * kChunk + sn) * L::YROW + pos);
      sum *= kInvC;
      const int P = pos / 16, gg = (pos % 16) / 4;
      const int col = 32 * (P / 2) + 16 * (gg % 2) + 8 * (P % 2) + 4 * (gg / 2);
      float* dst = y + (unit * LD + t0 + sn) * V + col;
      if (atomic_y) {
#pragma unroll
        for (int i = 0; i < 4; ++i) unsafeAtomicAdd(dst + i, sum[i]);
      } else {
        *reinterpret_cast<f4*>(dst) = sum;
      }
      return;
    }
    // atomic adds: columns j, j + V/4, j + V/2, j + 3V/4, so that consecutive
    // threads add into consecutive floats and each add instruction covers whole
    // 128-byte rows of y (with four consecutive floats per lane each 4-byte add
    // rewrote a 16-byte piece of memory: 3.9x the HBM writes at C3)
    // (every partial is read before the first add, so the reads share one wait
    // instead of one LDS round trip per column)
    float* dst = y + (unit * LD + t0 + sn) * V;
    float part[4][NW];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = j + (V / 4) * i, r = col % 32;
      const int pos = 16 * (2 * (col / 32) + (r % 16) / 8) + 4 * (2 * ((r % 8) / 4) + r / 16) + r % 4;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) part[i][ww] = ypb[(ww * kChunk + sn) * L::YROW + pos];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sum = part[i][0];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) sum += part[i][ww];
      unsafeAtomicAdd(dst + j + (V / 4) * i, sum * kInvC);
    }
  };

  // Chunk end of chunk c - 1, spread over the first steps of chunk c so that its
  // LDS round trips overlap with their compute:
  //   step 1 (end): publish the waves' partial readouts of chunk c - 1 (Dr,
  //                 which the readout MFMAs of steps 0 and 1 have just completed
  //                 with its last pair); LDS barrier
  //   step 2:       stage a chunk from the registers loaded a chunk ago (c + 2
  //                 with one barrier per chunk, which this step runs in chunk 0
  //                 too; else c + 1), then fetch the one after it
  //   steps 3..:    sum the partials into y, one group per step and thread
  //   step kSync:   (two barriers per chunk only) LDS barrier: the staged chunk
  //                 is visible before the step that first prefetches from it
  //                 (step 14), and every wave has summed before the next chunk
  //                 end overwrites the partials
  constexpr bool ONEBAR = L::ONEBAR;
  constexpr int kGroups = kChunk * (V / 4) / L::THREADS;  // y-sum groups per thread
  static_assert(kGroups * L::THREADS == kChunk * (V / 4), "whole groups per thread");
  constexpr int kSum0 = 3, kSync = 8;
  static_assert(kSum0 + kGroups <= kSync && kSync < kChunk - 2, "chunk-end schedule");
  auto ybuf = [](int c) { return ONEBAR ? (c & 1) : 0; };  // partial buffer of chunk c
  auto publish = [&](int yb) {
    float* ypw = yp_all + (yb * NW + w) * kChunk * L::YROW;
#pragma unroll
    for (int P = 0; P < CT; ++P) *reinterpret_cast<f4*>(ypw + n * L::YROW + 16 * P + 4 * g) = Dr[P];
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
    if (c > 0 && s == 1) publish(ybuf(c - 1));
    if (s == 2 && (ONEBAR || c > 0)) stage_next(ONEBAR ? c + 2 : c + 1);
    if (c > 0 && s >= kSum0 && s < kSum0 + kGroups)
      ysum_group((c - 1) * kChunk, tid + (s - kSum0) * L::THREADS, ybuf(c - 1));
    if (!ONEBAR && c > 0 && s == kSync) lds_barrier();
  };

  // one state element, tile c, register i, in two parts so that consecutive
  // groups overlap: r = 1 / (1 + exp2(u)) (tanh(x) = 1 - 2 r), then the gate
  // blend G <- f G + a - 2 a r; the blend of an element runs in the group after
  // its reciprocal, so no blend waits on a transcendental result
  auto elem_r = [&](const f4 (&cur)[CT], int c, int i) {
    const float e = __builtin_amdgcn_exp2f(cur[c][i]);
    return __builtin_amdgcn_rcpf(1.0f + e);
  };
  auto elem_g = [&](int c, int i, float r, float fg, float av, float m2a) {
    G[c][i] = fmaf(m2a, r, fmaf(fg, G[c][i], av));
  };
  // the operand block b for the next product from the new tiles 2b, 2b + 1, and
  // the block's rounded state into step s's readout slot(s). A slot is read for
  // the readout two steps later, half A at that step's start and half B (blocks
  // KB/2 .. KB-1) at its phase 1, before the same step writes those blocks.
  auto block_out = [&](int b, int t, int s) {
    make_operand<SPLIT>(G[2 * b], G[2 * b + 1], Bf[b], Bl[b]);
    if constexpr (SAVE) {
      if (t < T) *reinterpret_cast<bf16x8*>(saved + saved_state_off(unit, t + 1, T, a.K, V) + rt_off + b * 1024) = Bf[b];
    }
    unsigned short* hdst = hb_w + (s & (NHS - 1)) * NPL * 16 * HROW + n * HROW + 8 * g;
    *reinterpret_cast<Op*>(hdst + 32 * b) = Bf[b];
    if constexpr (SPLIT) *reinterpret_cast<Op*>(hdst + 16 * HROW + 32 * b) = Bl[b];
  };
  // training forward: the pre-activation c A_t of tiles 2b, 2b+1, as bf16
  auto save_pre = [&](int b, const f4 (&cur)[CT], int t) {
    if constexpr (SAVE) {
      if (t < T) {
        const f4 u0 = cur[2 * b], u1 = cur[2 * b + 1];
        const u4 pk = u4{pack_bf16(u0[0], u0[1]), pack_bf16(u0[2], u0[3]), pack_bf16(u1[0], u1[1]),
                         pack_bf16(u1[2], u1[3])};
        *reinterpret_cast<u4*>(saved + saved_pre_off(unit, t, a.B, a.H, T, a.K, V) + rt_off + b * 1024) = pk;
      }
    }
  };

  // product of operand block b into tile c (two passes with SPLIT)
  auto prod = [&](int b, int c, f4 (&acc)[CT]) {
    acc[c] = mfma(Wf[c][b], Bf[b], acc[c]);
    if constexpr (SPLIT) acc[c] = mfma(Wf[c][b], Bl[b], acc[c]);
  };
  // rank-1 write c k v^T of a step into tile c as the accumulator's start: the
  // pair (v, v) of the tile against (hi, lo) of c k.
  //
  // In the step loop this is a 16x16x16 product (fewer issue cycles than the
  // 16x16x32 form). On gfx950 a 16x16x32 product that takes a 16x16x16 result as
  // its accumulator only four instructions later, with no wait between them (as
  // the compiler scheduled it), read the accumulator before the result was in
  // it. In the loop the fenced phase schedule puts a whole phase (tens of
  // instructions) between a step's rank-1 write and the first product into that
  // accumulator; a build test checks that distance on the disassembly. The
  // prologue, where the products follow at once, takes the 16x16x32 form (the
  // pair in its first k slots, the others zero), whose accumulation into the
  // next 16x16x32 product the compiler orders.
  auto rank1_tile = [&](const R1& r, int c, f4 (&acc)[CT]) {
    const s4 av4 = __builtin_bit_cast(s4, r.win[c / 2]);
    const s4 bk4 = __builtin_bit_cast(s4, (c & 1) ? uint2{0u, r.kpair} : uint2{r.kpair, 0u});
    acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av4, bk4, f4{0, 0, 0, 0}, 0, 0, 0);
  };
  auto rank1_tile_prologue = [&](const R1& r, int c, f4 (&acc)[CT]) {
    const uint2 wv = r.win[c / 2];
    const bf16x8 av = __builtin_bit_cast(bf16x8, u4{wv.x, wv.y, 0u, 0u});
    const bf16x8 bk = __builtin_bit_cast(bf16x8, (c & 1) ? u4{0u, r.kpair, 0u, 0u} : u4{r.kpair, 0u, 0u, 0u});
    acc[c] = mfma(av, bk, f4{0, 0, 0, 0});
  };

  // per-step operands fetched ahead: the gate scalars of the next step and the
  // rank-1 operands of the step after it
  struct Pre {
    float2 fs;  // f and a = (1 - f) c (every loaded component is used: no load's register is reused early)
    R1 r1;
  };

  // Matrix-core work of phase p of a step (p < KB; phase p runs the epilogue of
  // tiles 2p, 2p + 1), in issue order; a product is two MFMAs with SPLIT:
  //   the last block's products for tiles 2p + 2, 2p + 3 of this step (cur),
  //   phase 0: the next step's rank-1 writes (nxt); phase p > 0: operand block
  //   p - 1 into every tile of the next step (nxt),
  //   on even steps the previous pair's readout: half of it in phase 1, the other
  //   half in phase 3 (both in phase 1 when V = 64);
  // and at the step's end the last block's products for tiles 0, 1 (nxt). Each
  // tile's epilogue comes a phase after its last product.
  constexpr int NPU = SPLIT ? 2 : 1;  // MFMAs per product
  auto n_last = [](int p) { return 2 * p + 2 < CT ? 2 : 0; };  // last-block products into cur in phase p
  // readout halves whose MFMAs run in phase p (even steps)
  auto ro_halves = [](int p) { return KB == 2 ? (p == 1 ? 2 : 0) : (p == 1 || p == 3 ? 1 : 0); };
  auto n_mfma = [&](int p, bool even) {
    return n_last(p) * NPU + (p == 0 ? CT : CT * NPU) + (even ? ro_halves(p) * NRH : 0);
  };
  auto mfma_unit = [&](int p, int j, f4 (&cur)[CT], f4 (&nxt)[CT], const R1& r1, const RO& roA, const RO& roB,
                       const Op& bq) {
    if (j < n_last(p) * NPU) {
      const int c = 2 * p + 2 + j / NPU;
      if (j % NPU == 0) cur[c] = mfma(Wf[c][KB - 1], Bf[KB - 1], cur[c]);
      else if constexpr (SPLIT) cur[c] = mfma(Wf[c][KB - 1], Bl[KB - 1], cur[c]);
      return;
    }
    j -= n_last(p) * NPU;
    if (p == 0) {
      if (j < CT) {
        rank1_tile(r1, j, nxt);
        return;
      }
      j -= CT;
    } else {
      if (j < CT * NPU) {
        const int c = j / NPU, b = p - 1;
        if (j % NPU == 0) nxt[c] = mfma(Wf[c][b], Bf[b], nxt[c]);
        else if constexpr (SPLIT) nxt[c] = mfma(Wf[c][b], Bl[b], nxt[c]);
        return;
      }
      j -= CT * NPU;
    }
    // readout: half A (tiles 0 .. CT/2 - 1) first, then half B
    const int half = (KB == 2) ? j / NRH : (p == 3 ? 1 : 0);
    readout_mma(half == 0 ? roA : roB, bq, half, j % NRH);
  };

  // Step s of chunk c (C, Cn, Cp: the stage buffers of chunks c, c + 1, c - 1).
  // On entry `cur` holds c (G_{t-1} W + k_t v_t^T) except the last operand
  // block's share for tiles 2.., which the phases add ahead of their epilogue.
  // The next step's accumulators `nxt` start from its rank-1 write and take
  // operand block b in phase b + 1; block KB-1 is finished for tiles 0, 1 at the
  // step's end and for the other tiles in the next step. Each matrix instruction
  // is followed by one state element of the epilogue, and every such group is
  // fenced so the compiler keeps the order: a wave issues in order, and an MFMA
  // takes the SIMD's issue port for about half of its 16 cycles, so back-to-back
  // MFMAs leave the vector ALU idle while spread ones hide under the epilogue.
  auto step = [&](const int s, f4 (&cur)[CT], f4 (&nxt)[CT], Pre& pre, const Buf& C, const Buf& Cn,
                  const Buf& Cp, const int c) {
    const float fg = pre.fs.x, av = pre.fs.y, m2a = -2.0f * av;
    const int t = c * kChunk + s;
    const bool even = s % 2 == 0;
    const R1 r1 = pre.r1;
    // the previous pair's readout operands (even steps): q and the first half
    const Buf& RB = s >= 2 ? C : Cp;
    const int rs0 = s >= 2 ? s - 2 : kChunk - 2, rnv = (s >= 2 || c > 0) ? 2 : 0;
    Op bq{};
    RO roA{}, roB{};
    if (even) {
      bq = readout_q(RB, rs0, rnv);
      roA = readout_load(rs0, 0);
      if (KB == 2) roB = readout_load(rs0, 1);
    }
    pre.fs = *reinterpret_cast<const float2*>(s + 1 < kChunk ? C.fs + (s + 1) * 4 : Cn.fs + (s + 1 - kChunk) * 4);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      save_pre(p, cur, t);
      if (p == 1) {  // the rank-1 operands of the step after next, once phase 0 has used this step's
        pre.r1 = s + 2 < kChunk ? rank1_load(C, s + 2) : rank1_load(Cn, s + 2 - kChunk);
        if (even && KB > 2) roB = readout_load(rs0, 1);
      }
      const int nm = n_mfma(p, even);
      // nine VALU groups over the eight elements of tiles 2p, 2p + 1 (group q:
      // element q's reciprocal, element q - 1's blend) and the operand block
      float rq = 0.0f;
#pragma unroll
      for (int q = 0; q < 9; ++q) {
#pragma unroll
        for (int j = (q * nm + 8) / 9; j < ((q + 1) * nm + 8) / 9; ++j) mfma_unit(p, j, cur, nxt, r1, roA, roB, bq);
        const float rn = q < 8 ? elem_r(cur, 2 * p + q / 4, q % 4) : 0.0f;
        if (q > 0) elem_g(2 * p + (q - 1) / 4, (q - 1) % 4, rq, fg, av, m2a);
        if (q == 8) block_out(p, t, s);
        rq = rn;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // tail: the last block into tiles 0, 1 of the next step
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) prod(KB - 1, cc, nxt);
    __builtin_amdgcn_sched_barrier(0);
    chunk_end_work(s, c);
  };

  // prologue: c (H_0 W + k_0 v_0^T) for step 0, last operand block for tiles 0, 1 only
  f4 accA[CT], accB[CT];
  {
    const R1 r0 = rank1_load(buf(0), 0);
#pragma unroll
    for (int cc = 0; cc < CT; ++cc) rank1_tile_prologue(r0, cc, accA);
  }
#pragma unroll
  for (int b = 0; b < KB - 1; ++b)
#pragma unroll
    for (int cc = 0; cc < CT; ++cc) prod(b, cc, accA);
  prod(KB - 1, 0, accA);
  prod(KB - 1, 1, accA);
  Pre pre;
  pre.fs = *reinterpret_cast<const float2*>(buf(0).fs);
  pre.r1 = rank1_load(buf(0), 1);

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
    const int ran = (ns + 1) & ~1;  // steps the loop ran in the last chunk
    if (c > 0) {
      // the previous chunk's y groups a short last chunk did not reach, before
      // the partials are overwritten
      const int done = min(max(ran - kSum0, 0), kGroups);
      for (int i = done; i < kGroups; ++i) ysum_group((c - 1) * kChunk, tid + i * L::THREADS, ybuf(c - 1));
      lds_barrier();
    }
    const int te = ran - 2;  // the last pair: steps te, te + 1
    const Op bq = readout_q(buf(c % NSB), te, min(ns - te, 2));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const RO rl = readout_load(te, half);
#pragma unroll
      for (int j = 0; j < NRH; ++j) readout_mma(rl, bq, half, j);
    }
    publish(ybuf(c));
    const int t0 = c * kChunk;
    for (int grp = tid; grp < ns * (V / 4); grp += L::THREADS) ysum_group(t0, grp, ybuf(c));
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

template <int V, int NW, bool SPLIT, bool F16 = false>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  if (F16 && a.saved) return hipErrorInvalidValue;  // the training forward saves bf16 operands
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
  if constexpr (F16)
    hipLaunchKernelGGL((mfma_fwd_kernel<V, NW, false, false, true>), dim3((unsigned)grid), dim3(64 * NW), 0, stream, a);
  else if (a.saved)
    hipLaunchKernelGGL((mfma_fwd_kernel<V, NW, SPLIT, true, false>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                       a);
  else
    hipLaunchKernelGGL((mfma_fwd_kernel<V, NW, SPLIT, false, false>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                       a);
  return hipGetLastError();
}

// waves per workgroup: R = 16 NW rows must divide K, at most two workgroups per
// unit (so atomic readout sums stay order-free).
int pick_nw(int K) {
  if (K % 64 == 0 && K / 64 <= 2) return 4;
  if (K % 32 == 0 && K / 32 <= 2) return 2;
  return 0;
}

template <int V, bool SPLIT>
int lds_bytes(int nw) {
  return nw == 4 ? Layout<V, 4, SPLIT>::TOTAL : Layout<V, 2, SPLIT>::TOTAL;
}

}  // namespace

hipError_t fill_zero(float* p, long long n, hipStream_t stream) {
  long long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

int mfma_groups(int K) {
  const int nw = pick_nw(K);
  return nw ? K / (16 * nw) : 0;
}

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
  const int lds = V == 128 ? (split ? lds_bytes<128, true>(nw) : lds_bytes<128, false>(nw))
                           : (split ? lds_bytes<64, true>(nw) : lds_bytes<64, false>(nw));
  return Plan{grid > 0x7fffffffLL ? -1 : (int)grid, 64 * nw, R, splits, splits > 1 ? 1 : 0, lds};
}

hipError_t launch_mfma(const FwdArgs& a, bool split, hipStream_t stream, bool f16) {
  if (!mfma_supports(a.K, a.V, a.bf16) || (split && f16)) return hipErrorInvalidValue;
  if (decode_supports(a)) return launch_decode(a, stream);  // one step: the decoding kernel
  const int nw = pick_nw(a.K);
  if (f16) {
    if (a.V == 128) return nw == 4 ? launch_t<128, 4, false, true>(a, stream) : launch_t<128, 2, false, true>(a, stream);
    return nw == 4 ? launch_t<64, 4, false, true>(a, stream) : launch_t<64, 2, false, true>(a, stream);
  }
  if (split) {
    if (a.V == 128) return nw == 4 ? launch_t<128, 4, true>(a, stream) : launch_t<128, 2, true>(a, stream);
    return nw == 4 ? launch_t<64, 4, true>(a, stream) : launch_t<64, 2, true>(a, stream);
  }
  if (a.V == 128) return nw == 4 ? launch_t<128, 4, false>(a, stream) : launch_t<128, 2, false>(a, stream);
  return nw == 4 ? launch_t<64, 4, false>(a, stream) : launch_t<64, 2, false>(a, stream);
}

}  // namespace m2rnn
