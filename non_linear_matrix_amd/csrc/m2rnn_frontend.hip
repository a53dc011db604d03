// Layer front-end of M²RNN: the per-head projections of the layer input x_t
// that the recurrence consumes, k_t, v_t, q_t, and the forget gate
// f_t = psi(x_t) (gist.science technical summary (zh) §2.1: the gate depends on
// x_t only and is kept in [0, 1] by a parameterised function, with per-head
// decay rates). psi is read as the logistic sigmoid of a linear projection plus
// a per-head bias.
//
// All of it is one matrix product over the model width D followed by a
// per-column epilogue:
//   P[m][n] = sum_d x[m][d] Wx[n][d],   m = b T + t,  n = h R + r,  R = 2K + V + 1
// row r of head h feeds k (r < K), v (K <= r < K + V), q (K + V <= r < 2K + V) or
// the gate logit (r = 2K + V), which gets the head's bias and the sigmoid. The
// epilogue writes bf16 straight into the [B][H][T][*] layouts the recurrence
// reads, so nothing else touches the projections.
//
// Kernel: 128 x 128 output tiles per workgroup of 4 waves (2 x 2 waves of
// 64 x 64, each 4 x 4 tiles of v_mfma_f32_16x16x32_bf16). Both operands are
// contiguous along D, so a lane's MFMA fragment (8 consecutive d of one row) is
// one 16-byte LDS read. The k-loop stages 32-wide slices of x and Wx through
// double-buffered LDS (40 KB, 124 VGPRs: four workgroups per CU, whose waves
// hide each other's barrier and load latencies); the global reads of the next
// slice are in flight while the current one is multiplied. Tiles are dealt so that each XCD gets a contiguous
// range, walked in groups of 8 tile rows, which keeps the x rows and the Wx
// tiles in flight within one XCD's L2.
#include <hip/hip_runtime.h>

#include "m2rnn_device.h"
#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

using namespace dev;

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LROW = BK + 8;                   // bf16 per LDS row: 16 bytes of padding
constexpr int THREADS = 256;
constexpr int PPT = BM * BK / 8 / THREADS;     // 16-byte pieces per thread and operand
constexpr int GROUP_M = 8;                     // tile rows walked together
static_assert(BM == BN && PPT * THREADS * 8 == BM * BK, "tile shape");

struct FrontArgs {
  const unsigned short* x;   // [M][D]
  const unsigned short* Wx;  // [N][D]
  const float* bias;         // [H]
  unsigned short *k, *v, *q, *f;
  long long M;
  int N, D, T, H, K, V, R;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ unsigned short to_bf16(float x) {
  const unsigned int p = __builtin_bit_cast(unsigned int, __builtin_convertvector(f2{x, 0.0f}, bf16x2));
  return static_cast<unsigned short>(p & 0xffffu);
}

__global__ __launch_bounds__(THREADS, 4) void frontend_kernel(FrontArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned short As[2][BM * LROW];
  __shared__ __attribute__((aligned(16))) unsigned short Bs[2][BN * LROW];
  const int tid = threadIdx.x, w = tid / 64, l = tid % 64, g = l / 16, n = l % 16;
  const int wm = w / 2, wn = w % 2;

  // workgroup -> tile. Workgroups are dealt round-robin over the 8 XCDs; give
  // XCD x the contiguous range of tiles [start(x), start(x) + count(x)).
  const int nwg = gridDim.x, bid = blockIdx.x;
  const int per = nwg / 8, rem = nwg % 8, xcd = bid % 8;
  const int tile = xcd * per + min(xcd, rem) + bid / 8;
  // then groups of GROUP_M tile rows, column by column
  const int in_group = GROUP_M * a.tiles_n;
  const int first_m = (tile / in_group) * GROUP_M;
  const int gsize = min(a.tiles_m - first_m, GROUP_M);
  const int tm = first_m + (tile % in_group) % gsize;
  const int tn = (tile % in_group) / gsize;
  const long long m0 = (long long)tm * BM;
  const int n0 = tn * BN;

  // global reads of the next slice, staged in registers
  u4 ra0[PPT], rb0[PPT];
  // piece r of a slice is row tid / 8 + 32 r, columns 8 (tid % 8) .. + 7 of the slice
  constexpr int RSTEP = THREADS / (BK / 8);
  const int prow = tid / (BK / 8), pcol = 8 * (tid % (BK / 8));
  const unsigned short* xp = a.x + (m0 + prow) * a.D + pcol;
  const unsigned short* wp = a.Wx + (long long)(n0 + prow) * a.D + pcol;
  unsigned int xok = 0, wok = 0;  // bit r: piece r's row exists
#pragma unroll
  for (int r = 0; r < PPT; ++r) {
    xok |= (m0 + prow + RSTEP * r < a.M) ? 1u << r : 0u;
    wok |= (n0 + prow + RSTEP * r < a.N) ? 1u << r : 0u;
  }
  const long long xstep = (long long)RSTEP * a.D;
  auto fetch = [&](int k0, u4 (&xa)[PPT], u4 (&xb)[PPT]) {
    const bool kin = k0 + pcol < a.D;
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      xa[r] = u4{0, 0, 0, 0};
      xb[r] = u4{0, 0, 0, 0};
      if (kin && ((xok >> r) & 1u)) xa[r] = *reinterpret_cast<const u4*>(xp + r * xstep + k0);
      if (kin && ((wok >> r) & 1u)) xb[r] = *reinterpret_cast<const u4*>(wp + r * xstep + k0);
    }
  };
  auto put = [&](int buf, const u4 (&xa)[PPT], const u4 (&xb)[PPT]) {
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int off = (prow + RSTEP * r) * LROW + pcol;
      *reinterpret_cast<u4*>(&As[buf][off]) = xa[r];
      *reinterpret_cast<u4*>(&Bs[buf][off]) = xb[r];
    }
  };

  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f4{0, 0, 0, 0};
  auto products = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 A[4], Bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        A[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(wm * 64 + 16 * i + n) * LROW + kk + 8 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        Bf[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(wn * 64 + 16 * j + n) * LROW + kk + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma(A[i], Bf[j], acc[i][j]);
    }
  };

  // slice j sits in LDS buffer j % 2; a buffer is rewritten only after the
  // barrier that follows its last products
  const int nk = (a.D + BK - 1) / BK;
  fetch(0, ra0, rb0);
  put(0, ra0, rb0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch((kt + 1) * BK, ra0, rb0);
    products(buf);
    if (kt + 1 < nk) put(buf ^ 1, ra0, rb0);
    __syncthreads();
  }

  // epilogue: lane (g, n) of tile (i, j) holds P[m0 + 64 wm + 16 i + 4 g + e][n0 + 64 wn + 16 j + n].
  // Per column: its head, output array and row length; per row: its (b, t),
  // from one division per lane and then at most one wrap (T >= 64) per row.
  unsigned short* dst[4];
  int ldc[4], hj[4];
  float bj[4];
  bool gate[4], col_ok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int nn = n0 + wn * 64 + 16 * j + n;
    col_ok[j] = nn < a.N;
    const int h = col_ok[j] ? nn / a.R : 0, r = nn - h * a.R;
    hj[j] = h;
    bj[j] = a.bias[h];
    gate[j] = r == 2 * a.K + a.V;
    if (r < a.K) {
      dst[j] = a.k + r; ldc[j] = a.K;
    } else if (r < a.K + a.V) {
      dst[j] = a.v + (r - a.K); ldc[j] = a.V;
    } else if (r < 2 * a.K + a.V) {
      dst[j] = a.q + (r - a.K - a.V); ldc[j] = a.K;
    } else {
      dst[j] = a.f; ldc[j] = 1;
    }
  }
  const long long mbase = m0 + wm * 64 + 4 * g;  // rows mbase + 16 i + e
  const long long b0 = mbase / a.T;
  const int t0 = static_cast<int>(mbase - b0 * a.T);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int o = 16 * i + e;
      if (mbase + o >= a.M) continue;
      long long b = b0;
      int t = t0 + o;
      if (t >= a.T) {
        if (a.T >= 64) {
          t -= a.T;
          ++b;
        } else {
          b += t / a.T;
          t %= a.T;
        }
      }
      const long long bh = b * a.H;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!col_ok[j]) continue;
        const long long row = (bh + hj[j]) * a.T + t;  // (unit, step)
        const float val = acc[i][j][e];
        dst[j][row * ldc[j]] = to_bf16(gate[j] ? 1.0f / (1.0f + __expf(-(val + bj[j]))) : val);
      }
    }
}

}  // namespace

hipError_t launch_frontend(const FrontLaunch& p, hipStream_t stream) {
  FrontArgs a{};
  a.x = static_cast<const unsigned short*>(p.x);
  a.Wx = static_cast<const unsigned short*>(p.Wx);
  a.bias = p.bias;
  a.k = static_cast<unsigned short*>(p.k);
  a.v = static_cast<unsigned short*>(p.v);
  a.q = static_cast<unsigned short*>(p.q);
  a.f = static_cast<unsigned short*>(p.f);
  a.M = (long long)p.B * p.T;
  a.R = 2 * p.K + p.V + 1;
  a.N = p.H * a.R;
  a.D = p.D;
  a.T = p.T;
  a.H = p.H;
  a.K = p.K;
  a.V = p.V;
  const long long tm = (a.M + BM - 1) / BM, tn = (a.N + BN - 1) / BN;
  if (tm * tn > 0x7fffffffLL || GROUP_M * tn > 0x7fffffffLL) return hipErrorInvalidValue;
  a.tiles_m = static_cast<int>(tm);
  a.tiles_n = static_cast<int>(tn);
  hipLaunchKernelGGL(frontend_kernel, dim3(static_cast<unsigned>(tm * tn)), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace m2rnn
