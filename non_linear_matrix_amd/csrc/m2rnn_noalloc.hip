// Library-owned scratch for the backward pass of callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).
//
// The backward pass's workspace (the dA slots, the dW partial sums, the long
// reverse kernel's dv / df partials and its sink) lives here in a fixed device
// array instead of a caller's buffer. Every part of it is written before it is
// read, so nothing is cleared between calls. Each GPU holds its own copy of the
// array, at its own address, until the process ends; all calls on one GPU share
// it, so calls that overlap on one GPU (two streams, two host threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "m2rnn_internal.h"

namespace m2rnn {
namespace {

constexpr long long kScratchBytes = 64LL << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

// the array's device address per device, resolved once with that device current
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

long long noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    // the host-side name `scratch` is only a stand-in: the kernels get this address
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace m2rnn
