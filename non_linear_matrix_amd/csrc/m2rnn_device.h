// Device helpers shared by the kernel files: vector types, bf16 <-> fp32
// conversions, the 16x16x32 bf16 and fp16 matrix products, the LDS-only workgroup barrier,
// a 16-lane DPP row sum and a compile-time loop. Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

namespace m2rnn {
namespace dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) float f2;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(8))) float f8;
typedef __attribute__((ext_vector_type(4))) short s4;
typedef __attribute__((ext_vector_type(8))) short s8;
typedef __attribute__((ext_vector_type(2))) unsigned int u2;
typedef __attribute__((ext_vector_type(4))) unsigned int u4;

// The matrix-core kernels carry the state scaled by c = 2 / ln 2, so that the
// exponential in tanh x = 1 - 2 / (1 + e^(2x)) is the hardware's exp2 of the
// scaled pre-activation: 2^(c x) = e^(2x).
constexpr float kC = 2.8853900817779268f;      // 2 / ln 2
constexpr float kInvC = 0.34657359027997264f;  // ln 2 / 2

// bf16 bit patterns to fp32 (exact): one value in the low 16 bits, or the low /
// high half of a packed pair
__device__ __forceinline__ float bf16_to_f32(unsigned int b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float lo_bf16(unsigned int x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf16(unsigned int x) { return __uint_as_float(x & 0xffff0000u); }
// two fp32 values to a packed bf16 pair (x0 low), round to nearest even
__device__ __forceinline__ unsigned int pack_bf16(float x0, float x1) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f2{x0, x1}, bf16x2));
}

// D = A B + C on a 16x16 fp32 tile, A and B bf16 with 32-deep contraction
__device__ __forceinline__ f4 mfma(const bf16x8& a, const bf16x8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// the same product with fp16 operands (11 significant bits instead of 8)
__device__ __forceinline__ f4 mfma(const f16x8& a, const f16x8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// Largest magnitude an fp16 operand takes: beyond it the kernels put NaN in the
// operand (rather than the infinity the conversion would give, which tanh could
// turn into a finite, wrong state), so a value outside fp16's range shows as NaN
// in the outputs.
constexpr float kF16Max = 65504.0f;
__device__ __forceinline__ float f16_range_or_nan(float x) {
  return fabsf(x) <= kF16Max ? x : __builtin_nanf("");
}
// eight bf16 bit patterns to fp16, round to nearest even: exact for magnitudes
// from 2^-17 to 65504 (a bf16 significand has 8 bits, fp16 keeps 11 and its
// subnormals reach 2^-24); larger magnitudes give NaN
__device__ __forceinline__ f16x8 bf16x8_to_f16(const s8& b) {
  f8 x;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = f16_range_or_nan(bf16_to_f32(static_cast<unsigned short>(b[i])));
  return __builtin_convertvector(x, f16x8);
}

// Workgroup barrier that orders LDS only: global loads and atomics stay in
// flight across it (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum over the 16 lanes of a DPP row; every lane of the row ends with the total.
// Each stage adds a lane and its partner (x + y and y + x are the same float).
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));   // lane ^ 1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));   // lane ^ 2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));  // half mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));  // mirror
  return x;
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order
template <typename F, int... S>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace dev
}  // namespace m2rnn
