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
};

// Launchers return the hipError_t of the launch (hipSuccess when enqueued).
hipError_t launch_simple(const FwdArgs& a, hipStream_t stream);
// Returns hipErrorInvalidValue when the MFMA kernel does not cover the shape
// (callers check mfma_supports first).
// split: state operand as bf16 hi + lo (two MFMA passes) instead of one bf16.
hipError_t launch_mfma(const FwdArgs& a, bool split, hipStream_t stream);
bool mfma_supports(int K, int V, int bf16);
// Fill n floats at p with zeros on `stream` (a kernel, so it can be captured).
hipError_t fill_zero(float* p, long long n, hipStream_t stream);

struct Plan {
  int grid, block, rows_per_group, groups_per_unit, clears_y, lds_bytes;
};
Plan plan_simple(int B, int H, int K, int V);
Plan plan_mfma(int B, int H, int K, int V, bool split);

}  // namespace m2rnn
