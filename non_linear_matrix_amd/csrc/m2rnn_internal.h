// Internal declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace m2rnn {

struct FwdArgs {
  const void* k;
  const void* v;
  const void* q;
  const void* f;
  const void* W;
  const float* H0;
  float* y;
  float* HT;
  int B, H, T, K, V;
  int bf16;        // 1: inputs are bfloat16 bit patterns, 0: fp32
  int accumulate;  // 1: y += readout (y is never cleared by the library)
  const int* lens; // device [B] sequence lengths, clamped to [0, T]; null: all T
  void* saved;     // training forward: per-step data for the backward pass; null: none
  int ld;          // steps between consecutive units' rows of k, v, q, f and y (0: T), so
                   // that a call can cover a window of a longer sequence; with ld != T
                   // the library never clears y (accumulate, or y null)
};
// y may be null when `saved` is set: the states are recomputed for the backward
// pass and the readout is not needed.

// Layout of the training forward's saved data (private to the library). A slot
// holds one K x V matrix as bf16 in the MFMA register layout: K/16 row tiles x
// V/32 blocks x 64 lanes x 16 bytes. Per unit there are T + 1 state slots (slot 0:
// c H0, slot t + 1: c H_t, c = 2/ln 2, the operand of the next step's product),
// and after all units' state slots, T pre-activation slots per unit (c A_t, as
// the MFMA accumulators of tiles 2b, 2b + 1 packed per block b).
__host__ __device__ inline long long saved_slot_bytes(int K, int V) { return (long long)K * V * 2; }
__host__ __device__ inline long long saved_state_off(long long unit, int slot, int T, int K, int V) {
  return (unit * (T + 1) + slot) * saved_slot_bytes(K, V);
}
__host__ __device__ inline long long saved_pre_off(long long unit, int t, int B, int H, int T, int K, int V) {
  return ((long long)B * H * (T + 1) + unit * T + t) * saved_slot_bytes(K, V);
}
__host__ __device__ inline long long saved_total_bytes(int B, int H, int T, int K, int V) {
  return (long long)B * H * (2LL * T + 1) * saved_slot_bytes(K, V);
}

// Launchers return the hipError_t of the launch (hipSuccess when enqueued).
hipError_t launch_simple(const FwdArgs& a, hipStream_t stream);
// Returns hipErrorInvalidValue when the MFMA kernel does not cover the shape
// (callers check mfma_supports first).
// split: state operand as bf16 hi + lo (two MFMA passes) instead of one bf16;
// f16: one fp16 state operand (W and q converted to fp16; no saved data).
hipError_t launch_mfma(const FwdArgs& a, bool split, hipStream_t stream, bool f16 = false);
bool mfma_supports(int K, int V, int bf16);
// fp32 matrix-core kernel (m2rnn_f32.hip): fp32 inputs, no saved data; writes y
// itself in a fixed summation order (clears it only for ragged lengths).
bool mfma_f32_supports(int K, int V);
hipError_t launch_mfma_f32(const FwdArgs& a, hipStream_t stream);
// workgroups the multi-step kernel gives one (b, h) unit (0: K not covered)
int mfma_groups(int K);
// One-step kernel (m2rnn_decode.hip): T == 1, no saved data, bf16, MFMA shapes.
// launch_mfma routes such calls to it; it writes y itself (no clearing needed).
bool decode_supports(const FwdArgs& a);
int decode_splits(int B, int H);
hipError_t launch_decode(const FwdArgs& a, hipStream_t stream);
// Fill n floats at p with zeros on `stream` (a kernel, so it can be captured).
hipError_t fill_zero(float* p, long long n, hipStream_t stream);

// Backward pass (bf16 inputs, MFMA shapes): the recurrence kernel, then dW.
struct BwdLaunch {
  const void *k, *v, *q, *f, *W;
  const void* saved;
  const float *dy, *dHT;
  float *dk, *dv, *dq, *df, *dW, *dH0;
  void* workspace;
  int B, H, T, K, V;
  int ld;             // steps between consecutive units' rows of k, v, q, f, dy, dk, dv, dq, df (0: T)
  int dvdf_zeroed;    // 1: dv and df already hold zeros (the launcher does not clear them)
  int dW_accumulate;  // 1: dW += this call's sum (else dW =)
  int long_kernel;    // 1: the latency-oriented reverse kernel (V in {64, 128})
};
hipError_t launch_bwd(const BwdLaunch& p, hipStream_t stream);
// dA slots, dW partials, then the latency-oriented kernel's dv / df partials
long long bwd_workspace_bytes(int B, int H, int T, int K, int V);
long long bwd_long_partial_bytes(int B, int H, int T, int K, int V);
// the latency-oriented reverse kernel and the sums of its dv / df partials (the
// dW kernels are launch_bwd's)
hipError_t launch_bwd_long(const BwdLaunch& p, char* dA_out, float* partials, hipStream_t stream);

// The library-owned backward workspace of m2rnn_bwd_noalloc (m2rnn_noalloc.hip):
// its size, and its device address on the current device (resolved on the first
// call per device; no allocation).
long long noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);

// Training with recomputation over segments of S steps (m2rnn_ckpt.cpp).
long long ckpt_bytes(int B, int H, int T, int K, int V, int S);
long long bwd_recompute_workspace_bytes(int B, int H, int T, int K, int V, int S);
// a.saved, a.lens and a.ld are ignored; ckpt receives the states at steps S, 2S, ...
// lng / split pick the forward kernel (latency-oriented or multi-step, split operand)
hipError_t launch_fwd_ckpt(const FwdArgs& a, float* ckpt, int S, bool split, bool lng, hipStream_t stream);
// p.saved, p.ld and the flags are ignored; p.workspace holds
// bwd_recompute_workspace_bytes; lng / split pick the forward that recomputes the states
hipError_t launch_bwd_recompute(const BwdLaunch& p, const float* H0, const float* ckpt, int S, bool split,
                                bool lng, hipStream_t stream);

// Layer front-end (m2rnn_frontend.hip): k, v, q and f from x (bf16).
struct FrontLaunch {
  const void* x;      // [B][T][D]
  const void* Wx;     // [H][2K + V + 1][D]
  const float* bias;  // [H]
  void *k, *v, *q, *f;
  int B, T, D, H, K, V;
};
hipError_t launch_frontend(const FrontLaunch& p, hipStream_t stream);

struct Plan {
  int grid, block, rows_per_group, groups_per_unit, clears_y, lds_bytes;
};
Plan plan_simple(int B, int H, int K, int V);
Plan plan_mfma(int B, int H, int K, int V, bool split);
Plan plan_decode(int B, int H, int K, int V);
Plan plan_mfma_f32(int B, int H, int K, int V);
// Latency-oriented forward (m2rnn_long.hip): one workgroup of V/32 waves per
// 16-row tile; y summed over the tiles with atomic adds.
bool long_supports(const FwdArgs& a);
Plan plan_long(int B, int H, int K, int V);
hipError_t launch_long(const FwdArgs& a, bool split, hipStream_t stream, bool f16 = false);

}  // namespace m2rnn
