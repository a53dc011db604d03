// Training with recomputation: the backward pass rebuilds the forward states it
// needs instead of keeping every H_t from the forward pass (gist.science technical
// summary (zh) §2.2, the parallelism paragraph: the states are recomputed in the
// backward pass and cached in HBM).
//
// The sequence is cut into segments of S steps. The training forward runs one
// window launch per segment and keeps the state at each segment start (a
// checkpoint, fp32, B H K V floats per segment after the first). The backward
// pass visits the segments last to first: it recomputes the segment's states and
// pre-activations from its checkpoint with the saving forward kernel into a
// workspace that holds one segment, runs the reverse-time kernel and the dW
// kernels over that segment, and hands the state gradient at the segment start
// to the next segment. Peak memory is one segment's saved data plus the
// checkpoints, instead of the whole sequence's.
//
// Host code only: it strings together the launchers of the recurrence kernels.
#include <cstdint>

#include "m2rnn_internal.h"

namespace m2rnn {

namespace {

long long round256(long long n) { return (n + 255) / 256 * 256; }

int nsegments(int T, int S) { return (T + S - 1) / S; }

}  // namespace

long long ckpt_bytes(int B, int H, int T, int K, int V, int S) {
  return (long long)(nsegments(T, S) - 1) * B * H * K * V * 4;
}

long long bwd_recompute_workspace_bytes(int B, int H, int T, int K, int V, int S) {
  const int Sw = S < T ? S : T;
  return round256(saved_total_bytes(B, H, Sw, K, V)) + round256(bwd_workspace_bytes(B, H, Sw, K, V)) +
         2 * round256((long long)B * H * K * V * 4);
}

hipError_t launch_fwd_ckpt(const FwdArgs& a, float* ckpt, int S, bool split, bool lng, hipStream_t stream) {
  const int nseg = nsegments(a.T, S);
  bool add = true;  // the latency-oriented kernel's row tiles add their readouts into y
  if (!lng) {
    const Plan pl = plan_mfma(a.B, a.H, a.K, a.V, split);
    if (pl.grid < 0) return hipErrorInvalidValue;
    add = pl.groups_per_unit > 1;  // two workgroups add their readouts into y
  }
  hipError_t e;
  if (add && (e = fill_zero(a.y, (long long)a.B * a.H * a.T * a.V, stream)) != hipSuccess) return e;
  const long long unitKV = (long long)a.B * a.H * a.K * a.V;
  for (int j = 0; j < nseg; ++j) {
    const long long t0 = (long long)j * S;
    FwdArgs w = a;
    w.k = static_cast<const unsigned short*>(a.k) + t0 * a.K;
    w.q = static_cast<const unsigned short*>(a.q) + t0 * a.K;
    w.v = static_cast<const unsigned short*>(a.v) + t0 * a.V;
    w.f = static_cast<const unsigned short*>(a.f) + t0;
    w.y = a.y + t0 * a.V;
    w.T = static_cast<int>(j == nseg - 1 ? a.T - t0 : S);
    w.ld = a.T;
    w.accumulate = add ? 1 : 0;
    w.H0 = j == 0 ? a.H0 : ckpt + (j - 1) * unitKV;
    w.HT = j == nseg - 1 ? a.HT : ckpt + j * unitKV;
    w.lens = nullptr;
    w.saved = nullptr;
    if ((e = lng ? launch_long(w, split, stream) : launch_mfma(w, split, stream)) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_recompute(const BwdLaunch& p, const float* H0, const float* ckpt, int S, bool split,
                                bool lng, hipStream_t stream) {
  const int nseg = nsegments(p.T, S);
  const int Sw = S < p.T ? S : p.T;
  char* ws = static_cast<char*>(p.workspace);
  char* saved = ws;
  char* bws = saved + round256(saved_total_bytes(p.B, p.H, Sw, p.K, p.V));
  float* carry[2];
  carry[0] = reinterpret_cast<float*>(bws + round256(bwd_workspace_bytes(p.B, p.H, Sw, p.K, p.V)));
  carry[1] = reinterpret_cast<float*>(reinterpret_cast<char*>(carry[0]) +
                                      round256((long long)p.B * p.H * p.K * p.V * 4));
  hipError_t e;
  // dv and df take sums from two workgroups per unit: cleared once, for all segments
  if ((e = fill_zero(p.dv, (long long)p.B * p.H * p.T * p.V, stream)) != hipSuccess) return e;
  if ((e = fill_zero(p.df, (long long)p.B * p.H * p.T, stream)) != hipSuccess) return e;
  const long long unitKV = (long long)p.B * p.H * p.K * p.V;
  const float* dH_in = p.dHT;
  for (int j = nseg - 1; j >= 0; --j) {
    const long long t0 = (long long)j * S;
    const int Tj = static_cast<int>(j == nseg - 1 ? p.T - t0 : S);
    const unsigned short* k = static_cast<const unsigned short*>(p.k) + t0 * p.K;
    const unsigned short* q = static_cast<const unsigned short*>(p.q) + t0 * p.K;
    const unsigned short* v = static_cast<const unsigned short*>(p.v) + t0 * p.V;
    const unsigned short* f = static_cast<const unsigned short*>(p.f) + t0;
    // 1. the segment's states and pre-activations, from its checkpoint
    FwdArgs fa{k, v, q, f, p.W, j == 0 ? H0 : ckpt + (j - 1) * unitKV, nullptr, nullptr,
               p.B, p.H, Tj, p.K, p.V, 1, 0, nullptr, saved, p.T};
    if ((e = lng ? launch_long(fa, split, stream) : launch_mfma(fa, split, stream)) != hipSuccess) return e;
    // 2. reverse time over the segment, then its share of dW
    float* dH_out = j == 0 ? p.dH0 : carry[j & 1];
    BwdLaunch b{k, v, q, f, p.W, saved, p.dy + t0 * p.V, dH_in,
                p.dk + t0 * p.K, p.dv + t0 * p.V, p.dq + t0 * p.K, p.df + t0, p.dW, dH_out, bws,
                p.B, p.H, Tj, p.K, p.V, p.T, 1, j == nseg - 1 ? 0 : 1, lng ? 1 : 0};
    if ((e = launch_bwd(b, stream)) != hipSuccess) return e;
    dH_in = dH_out;
  }
  return hipSuccess;
}

}  // namespace m2rnn
