// C ABI of the M²RNN forward recurrence: host-side validation and dispatch.
// Validation touches no HIP API, so every error path runs without a GPU.
#include "m2rnn.h"

#include <cstdint>

#include "m2rnn_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<std::uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int d) { return d >= 16 && d <= 128 && (d % 16) == 0; }

// element counts must stay far below 2^62 so 64-bit index arithmetic cannot wrap
bool counts_fit(int B, int H, int T, int K, int V) {
  const long double lim = 4.0e18L;
  long double bh = (long double)B * H;
  long double n1 = bh * T * (K > V ? K : V);
  long double n2 = bh * K * V;
  long double n3 = (long double)H * V * V;
  return n1 < lim && n2 < lim && n3 < lim;
}

m2rnn_status check(const void* k, const void* v, const void* q, const void* f, const void* W,
                   const float* H0, const float* y, const float* HT, int B, int H, int T, int K,
                   int V, m2rnn_dtype dt, m2rnn_algo algo) {
  if (!k || !v || !q || !f || !W || !y) return M2RNN_ERROR_INVALID_VALUE;
  if (B < 1 || H < 1 || T < 1 || K < 1 || V < 1) return M2RNN_ERROR_INVALID_VALUE;
  if (!aligned16(k) || !aligned16(v) || !aligned16(q) || !aligned16(f) || !aligned16(W) ||
      !aligned16(y) || (H0 && !aligned16(H0)) || (HT && !aligned16(HT)))
    return M2RNN_ERROR_INVALID_VALUE;
  if (!counts_fit(B, H, T, K, V)) return M2RNN_ERROR_INVALID_VALUE;
  if (dt != M2RNN_DTYPE_F32 && dt != M2RNN_DTYPE_BF16) return M2RNN_ERROR_NOT_SUPPORTED;
  if (!supported_dim(K) || !supported_dim(V)) return M2RNN_ERROR_NOT_SUPPORTED;
  switch (algo) {
    case M2RNN_ALGO_AUTO:
    case M2RNN_ALGO_SIMPLE:
      return M2RNN_SUCCESS;
    case M2RNN_ALGO_MFMA:
    case M2RNN_ALGO_MFMA_SPLIT:
    case M2RNN_ALGO_MFMA_F16:
      return m2rnn::mfma_supports(K, V, dt == M2RNN_DTYPE_BF16) ? M2RNN_SUCCESS
                                                                 : M2RNN_ERROR_NOT_SUPPORTED;
    case M2RNN_ALGO_MFMA_LONG:
    case M2RNN_ALGO_MFMA_LONG_SPLIT:
    case M2RNN_ALGO_MFMA_LONG_F16:
      return (dt == M2RNN_DTYPE_BF16 && (V == 64 || V == 128)) ? M2RNN_SUCCESS : M2RNN_ERROR_NOT_SUPPORTED;
    case M2RNN_ALGO_MFMA_F32:
      return (dt == M2RNN_DTYPE_F32 && m2rnn::mfma_f32_supports(K, V)) ? M2RNN_SUCCESS : M2RNN_ERROR_NOT_SUPPORTED;
    default:
      return M2RNN_ERROR_NOT_SUPPORTED;
  }
}

}  // namespace

extern "C" m2rnn_algo m2rnn_pick_algo(int B, int H, int T, int K, int V, m2rnn_dtype in_dtype);

namespace {

// The training entry points' forward kernel: AUTO takes the split operand (the
// backward pass reads bf16 operands), on the latency-oriented kernel where
// m2rnn_pick_algo would; explicit families are the four bf16 matrix-core ones,
// on the shapes the backward pass covers.
m2rnn_status training_algo(m2rnn_algo& algo, int B, int H, int T, int K, int V, m2rnn_dtype dt) {
  if (algo == M2RNN_ALGO_AUTO) {
    algo = m2rnn_pick_algo(B, H, T, K, V, dt);
    algo = algo == M2RNN_ALGO_MFMA_LONG_F16 ? M2RNN_ALGO_MFMA_LONG_SPLIT : M2RNN_ALGO_MFMA_SPLIT;
  }
  switch (algo) {
    case M2RNN_ALGO_MFMA:
    case M2RNN_ALGO_MFMA_SPLIT:
      return M2RNN_SUCCESS;
    case M2RNN_ALGO_MFMA_LONG:
    case M2RNN_ALGO_MFMA_LONG_SPLIT:
      return m2rnn::mfma_supports(K, V, dt == M2RNN_DTYPE_BF16) ? M2RNN_SUCCESS : M2RNN_ERROR_NOT_SUPPORTED;
    default:
      return M2RNN_ERROR_NOT_SUPPORTED;
  }
}

bool is_long(m2rnn_algo algo) {
  return algo == M2RNN_ALGO_MFMA_LONG || algo == M2RNN_ALGO_MFMA_LONG_SPLIT || algo == M2RNN_ALGO_MFMA_LONG_F16;
}
bool is_split(m2rnn_algo algo) { return algo == M2RNN_ALGO_MFMA_SPLIT || algo == M2RNN_ALGO_MFMA_LONG_SPLIT; }
bool is_f16(m2rnn_algo algo) { return algo == M2RNN_ALGO_MFMA_F16 || algo == M2RNN_ALGO_MFMA_LONG_F16; }
// the multi-step kernel family with a latency-oriented family's state operand
m2rnn_algo multistep_of(m2rnn_algo algo) {
  return algo == M2RNN_ALGO_MFMA_LONG ? M2RNN_ALGO_MFMA
         : algo == M2RNN_ALGO_MFMA_LONG_F16 ? M2RNN_ALGO_MFMA_F16
                                            : M2RNN_ALGO_MFMA_SPLIT;
}

// Whether a forward call's y is bitwise repeatable (the order of its atomic adds
// cannot change it). Kernels whose workgroups share a unit add their readouts
// into y atomically: the multi-step kernels' K/(16 NW) workgroups and the long
// kernels' K/16 row tiles. One contribution per element, or two onto a cleared y
// (0 + a + b = 0 + b + a exactly), cannot depend on the order. The long kernels
// round every contribution to a grid on which all the sums are exact, so any
// number of them onto a cleared y is repeatable. Adds onto a y that already holds
// values (M2RNN_FLAG_ACCUMULATE_Y) from two workgroups or more are not. One step
// on the matrix-core shapes runs the decoding kernel, which sums in LDS in a
// fixed order.
bool atomic_free(m2rnn_algo algo, int T, int K, int V, bool bf16, bool accumulate) {
  int adds = 1;
  const bool decode = T == 1 && m2rnn::mfma_supports(K, V, bf16);
  if (algo == M2RNN_ALGO_MFMA || algo == M2RNN_ALGO_MFMA_SPLIT || algo == M2RNN_ALGO_MFMA_F16)
    adds = decode ? 1 : m2rnn::mfma_groups(K);
  if (is_long(algo)) adds = decode ? 1 : K / 16;
  return adds <= 1 || (!accumulate && (adds == 2 || is_long(algo)));
}

// The kernel family a forward call runs: AUTO resolved, and the rules of the
// flags applied (unknown flag bits and a deterministic call on a family that
// sums y atomically are NOT_SUPPORTED). Host only.
m2rnn_status resolve_algo(m2rnn_algo& algo, int B, int H, int T, int K, int V, m2rnn_dtype dt, unsigned flags) {
  if ((flags & ~static_cast<unsigned>(M2RNN_FLAG_ACCUMULATE_Y | M2RNN_FLAG_DETERMINISTIC)) != 0u)
    return M2RNN_ERROR_NOT_SUPPORTED;
  const bool det = (flags & M2RNN_FLAG_DETERMINISTIC) != 0u;
  const bool acc = (flags & M2RNN_FLAG_ACCUMULATE_Y) != 0u;
  const bool bf = dt == M2RNN_DTYPE_BF16;
  if (algo == M2RNN_ALGO_AUTO) {
    algo = m2rnn_pick_algo(B, H, T, K, V, dt);
    if (det && !atomic_free(algo, T, K, V, bf, acc) && is_long(algo))
      algo = !m2rnn::mfma_supports(K, V, bf) ? M2RNN_ALGO_SIMPLE : multistep_of(algo);
    if (det && !atomic_free(algo, T, K, V, bf, acc)) algo = M2RNN_ALGO_SIMPLE;
  }
  if (det && !atomic_free(algo, T, K, V, bf, acc)) return M2RNN_ERROR_NOT_SUPPORTED;
  return M2RNN_SUCCESS;
}

}  // namespace

extern "C" {

m2rnn_status m2rnn_check_args(const void* k, const void* v, const void* q, const void* f,
                              const void* W, const float* H0, const float* y, const float* H_T,
                              int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                              m2rnn_algo algo) {
  return check(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype, algo);
}

m2rnn_algo m2rnn_pick_algo(int B, int H, int T, int K, int V, m2rnn_dtype in_dtype) {
  // The latency-oriented kernel gives each 16-row tile a workgroup of V/32 waves,
  // two of which fit on a CU of a 256-CU gfx950 (LDS): up to 512 tiles run at
  // once, and up to 768 a second partial pass still finishes before the
  // multi-step kernel (one wave per tile, 1024 at once); beyond that the latter
  // wins (measured at K = V = 128).
  constexpr long double kLongMaxTiles = 768;
  // bf16 inputs: the fp16 state operand, which meets the bf16 bar on every
  // workload measured at the single operand's cost (the split operand costs a
  // third more time; it stays the choice of the training entry points)
  if (in_dtype == M2RNN_DTYPE_F32 && m2rnn::mfma_f32_supports(K, V)) return M2RNN_ALGO_MFMA_F32;
  if (in_dtype == M2RNN_DTYPE_BF16 && T > 1 && (V == 64 || V == 128) && supported_dim(K) &&
      (long double)B * H * (K / 16) <= kLongMaxTiles)
    return M2RNN_ALGO_MFMA_LONG_F16;
  if (m2rnn::mfma_supports(K, V, in_dtype == M2RNN_DTYPE_BF16)) return M2RNN_ALGO_MFMA_F16;
  return M2RNN_ALGO_SIMPLE;
}

m2rnn_status m2rnn_fwd_varlen(const void* k, const void* v, const void* q, const void* f,
                              const void* W, const float* H0, float* y, float* H_T,
                              const int* seq_len, int B, int H, int T, int K, int V,
                              m2rnn_dtype in_dtype, m2rnn_algo algo, unsigned flags, void* stream) {
  m2rnn_status st = check(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype, algo);
  if (st != M2RNN_SUCCESS) return st;
  if (seq_len && (reinterpret_cast<std::uintptr_t>(seq_len) & 3u) != 0) return M2RNN_ERROR_INVALID_VALUE;
  if ((st = resolve_algo(algo, B, H, T, K, V, in_dtype, flags)) != M2RNN_SUCCESS) return st;
  m2rnn::FwdArgs a{k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype == M2RNN_DTYPE_BF16 ? 1 : 0,
                   (flags & M2RNN_FLAG_ACCUMULATE_Y) ? 1 : 0, seq_len, nullptr};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (algo == M2RNN_ALGO_MFMA || algo == M2RNN_ALGO_MFMA_SPLIT || algo == M2RNN_ALGO_MFMA_F16)
    e = m2rnn::launch_mfma(a, algo == M2RNN_ALGO_MFMA_SPLIT, s, is_f16(algo));
  else if (is_long(algo))
    e = m2rnn::decode_supports(a) ? m2rnn::launch_decode(a, s)  // one step: the decoding kernel
                                  : m2rnn::launch_long(a, algo == M2RNN_ALGO_MFMA_LONG_SPLIT, s, is_f16(algo));
  else if (algo == M2RNN_ALGO_MFMA_F32)
    e = m2rnn::launch_mfma_f32(a, s);
  else
    e = m2rnn::launch_simple(a, s);
  return e == hipSuccess ? M2RNN_SUCCESS : M2RNN_ERROR_LAUNCH;
}

m2rnn_status m2rnn_fwd_ex(const void* k, const void* v, const void* q, const void* f,
                          const void* W, const float* H0, float* y, float* H_T, int B, int H,
                          int T, int K, int V, m2rnn_dtype in_dtype, m2rnn_algo algo,
                          unsigned flags, void* stream) {
  return m2rnn_fwd_varlen(k, v, q, f, W, H0, y, H_T, nullptr, B, H, T, K, V, in_dtype, algo, flags,
                          stream);
}

m2rnn_status m2rnn_fwd_algo(const void* k, const void* v, const void* q, const void* f,
                            const void* W, const float* H0, float* y, float* H_T, int B, int H,
                            int T, int K, int V, m2rnn_dtype in_dtype, m2rnn_algo algo,
                            void* stream) {
  return m2rnn_fwd_ex(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype, algo, 0u, stream);
}

m2rnn_status m2rnn_fwd(const void* k, const void* v, const void* q, const void* f, const void* W,
                       const float* H0, float* y, float* H_T, int B, int H, int T, int K, int V,
                       m2rnn_dtype in_dtype, void* stream) {
  return m2rnn_fwd_algo(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype, M2RNN_ALGO_AUTO,
                        stream);
}

unsigned long long m2rnn_saved_bytes(int B, int H, int T, int K, int V) {
  if (B < 1 || H < 1 || T < 1 || !counts_fit(B, H, T, K, V) || !m2rnn::mfma_supports(K, V, 1)) return 0;
  return static_cast<unsigned long long>(m2rnn::saved_total_bytes(B, H, T, K, V));
}

m2rnn_status m2rnn_fwd_save(const void* k, const void* v, const void* q, const void* f,
                            const void* W, const float* H0, float* y, float* H_T, void* saved,
                            int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, void* stream) {
  m2rnn_status st = check(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype, algo);
  if (st != M2RNN_SUCCESS) return st;
  if ((st = training_algo(algo, B, H, T, K, V, in_dtype)) != M2RNN_SUCCESS) return st;
  if ((st = check(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype, algo)) != M2RNN_SUCCESS) return st;
  if (!saved || !aligned16(saved)) return M2RNN_ERROR_INVALID_VALUE;
  m2rnn::FwdArgs a{k, v, q, f, W, H0, y, H_T, B, H, T, K, V, 1, 0, nullptr, saved};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = is_long(algo) ? m2rnn::launch_long(a, is_split(algo), s) : m2rnn::launch_mfma(a, is_split(algo), s);
  return e == hipSuccess ? M2RNN_SUCCESS : M2RNN_ERROR_LAUNCH;
}

unsigned long long m2rnn_bwd_workspace_bytes(int B, int H, int T, int K, int V) {
  if (B < 1 || H < 1 || T < 1 || !counts_fit(B, H, T, K, V) || !m2rnn::mfma_supports(K, V, 1)) return 0;
  return static_cast<unsigned long long>(m2rnn::bwd_workspace_bytes(B, H, T, K, V));
}

}  // extern "C"

namespace {

// Validation of a backward call (everything but the workspace), then the launch
// with the given workspace.
m2rnn_status bwd_check(const void* k, const void* v, const void* q, const void* f, const void* W,
                       const float* H0, const void* saved, const float* dy, const float* dH_T, float* dk,
                       float* dv, float* dq, float* df, float* dW, float* dH0, int B, int H, int T, int K, int V,
                       m2rnn_dtype in_dtype, m2rnn_algo& algo) {
  // the forward's argument rules, with dy standing in for y
  m2rnn_status st = check(k, v, q, f, W, H0, dy, dH_T, B, H, T, K, V, in_dtype, M2RNN_ALGO_MFMA);
  if (st != M2RNN_SUCCESS) return st;
  if ((st = training_algo(algo, B, H, T, K, V, in_dtype)) != M2RNN_SUCCESS) return st;
  if (!saved || !dk || !dv || !dq || !df || !dW) return M2RNN_ERROR_INVALID_VALUE;
  if (!aligned16(saved) || !aligned16(dk) || !aligned16(dv) || !aligned16(dq) || !aligned16(df) ||
      !aligned16(dW) || (dH0 && !aligned16(dH0)))
    return M2RNN_ERROR_INVALID_VALUE;
  return M2RNN_SUCCESS;
}

m2rnn_status bwd_launch(const void* k, const void* v, const void* q, const void* f, const void* W,
                        const void* saved, const float* dy, const float* dH_T, float* dk, float* dv, float* dq,
                        float* df, float* dW, float* dH0, void* workspace, int B, int H, int T, int K, int V,
                        m2rnn_algo algo, void* stream) {
  m2rnn::BwdLaunch p{k, v, q, f, W, saved, dy, dH_T, dk, dv, dq, df, dW, dH0, workspace, B, H, T, K, V,
                     0, 0, 0, is_long(algo) ? 1 : 0};
  hipError_t e = m2rnn::launch_bwd(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? M2RNN_SUCCESS : M2RNN_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

m2rnn_status m2rnn_bwd_algo(const void* k, const void* v, const void* q, const void* f, const void* W,
                            const float* H0, const void* saved, const float* dy, const float* dH_T,
                            float* dk, float* dv, float* dq, float* df, float* dW, float* dH0,
                            void* workspace, int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, void* stream) {
  m2rnn_status st = bwd_check(k, v, q, f, W, H0, saved, dy, dH_T, dk, dv, dq, df, dW, dH0, B, H, T, K, V,
                              in_dtype, algo);
  if (st != M2RNN_SUCCESS) return st;
  if (!workspace || !aligned16(workspace)) return M2RNN_ERROR_INVALID_VALUE;
  return bwd_launch(k, v, q, f, W, saved, dy, dH_T, dk, dv, dq, df, dW, dH0, workspace, B, H, T, K, V, algo,
                    stream);
}

m2rnn_status m2rnn_bwd_noalloc(const void* k, const void* v, const void* q, const void* f, const void* W,
                               const float* H0, const void* saved, const float* dy, const float* dH_T,
                               float* dk, float* dv, float* dq, float* df, float* dW, float* dH0,
                               int B, int H, int T, int K, int V, m2rnn_dtype in_dtype, m2rnn_algo algo,
                               void* stream) {
  m2rnn_status st = bwd_check(k, v, q, f, W, H0, saved, dy, dH_T, dk, dv, dq, df, dW, dH0, B, H, T, K, V,
                              in_dtype, algo);
  if (st != M2RNN_SUCCESS) return st;
  // refused before any HIP call when the library's array cannot hold the workspace
  if (m2rnn::bwd_workspace_bytes(B, H, T, K, V) > m2rnn::noalloc_scratch_bytes())
    return M2RNN_ERROR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if (m2rnn::noalloc_scratch(&ws) != hipSuccess) return M2RNN_ERROR_LAUNCH;
  return bwd_launch(k, v, q, f, W, saved, dy, dH_T, dk, dv, dq, df, dW, dH0, ws, B, H, T, K, V, algo, stream);
}

m2rnn_status m2rnn_bwd(const void* k, const void* v, const void* q, const void* f, const void* W,
                       const float* H0, const void* saved, const float* dy, const float* dH_T,
                       float* dk, float* dv, float* dq, float* df, float* dW, float* dH0,
                       void* workspace, int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                       void* stream) {
  return m2rnn_bwd_algo(k, v, q, f, W, H0, saved, dy, dH_T, dk, dv, dq, df, dW, dH0, workspace, B, H, T, K, V,
                        in_dtype, M2RNN_ALGO_AUTO, stream);
}

unsigned long long m2rnn_ckpt_bytes(int B, int H, int T, int K, int V, int segment) {
  if (B < 1 || H < 1 || T < 1 || segment < 1 || !counts_fit(B, H, T, K, V)) return 0;
  return static_cast<unsigned long long>(m2rnn::ckpt_bytes(B, H, T, K, V, segment));
}

m2rnn_status m2rnn_fwd_ckpt(const void* k, const void* v, const void* q, const void* f,
                            const void* W, const float* H0, float* y, float* H_T, float* ckpt,
                            int B, int H, int T, int K, int V, int segment, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, void* stream) {
  m2rnn_status st = check(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype, algo);
  if (st != M2RNN_SUCCESS) return st;
  if ((st = training_algo(algo, B, H, T, K, V, in_dtype)) != M2RNN_SUCCESS) return st;
  if ((st = check(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, in_dtype, algo)) != M2RNN_SUCCESS) return st;
  if (segment < 1) return M2RNN_ERROR_INVALID_VALUE;
  if (m2rnn::ckpt_bytes(B, H, T, K, V, segment) > 0 && (!ckpt || !aligned16(ckpt)))
    return M2RNN_ERROR_INVALID_VALUE;
  m2rnn::FwdArgs a{k, v, q, f, W, H0, y, H_T, B, H, T, K, V, 1, 0, nullptr, nullptr, 0};
  hipError_t e = m2rnn::launch_fwd_ckpt(a, ckpt, segment, is_split(algo), is_long(algo),
                                        reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? M2RNN_SUCCESS : M2RNN_ERROR_LAUNCH;
}

unsigned long long m2rnn_bwd_recompute_workspace_bytes(int B, int H, int T, int K, int V, int segment) {
  if (B < 1 || H < 1 || T < 1 || segment < 1 || !counts_fit(B, H, T, K, V) || !m2rnn::mfma_supports(K, V, 1))
    return 0;
  return static_cast<unsigned long long>(m2rnn::bwd_recompute_workspace_bytes(B, H, T, K, V, segment));
}

m2rnn_status m2rnn_bwd_recompute(const void* k, const void* v, const void* q, const void* f,
                                 const void* W, const float* H0, const float* ckpt, const float* dy,
                                 const float* dH_T, float* dk, float* dv, float* dq, float* df,
                                 float* dW, float* dH0, void* workspace, int B, int H, int T, int K,
                                 int V, int segment, m2rnn_dtype in_dtype, m2rnn_algo algo,
                                 void* stream) {
  m2rnn_status st = check(k, v, q, f, W, H0, dy, dH_T, B, H, T, K, V, in_dtype, algo);
  if (st != M2RNN_SUCCESS) return st;
  if ((st = training_algo(algo, B, H, T, K, V, in_dtype)) != M2RNN_SUCCESS) return st;
  if ((st = check(k, v, q, f, W, H0, dy, dH_T, B, H, T, K, V, in_dtype, algo)) != M2RNN_SUCCESS) return st;
  if (segment < 1 || !dk || !dv || !dq || !df || !dW || !workspace) return M2RNN_ERROR_INVALID_VALUE;
  if (m2rnn::ckpt_bytes(B, H, T, K, V, segment) > 0 && (!ckpt || !aligned16(ckpt)))
    return M2RNN_ERROR_INVALID_VALUE;
  if (!aligned16(dk) || !aligned16(dv) || !aligned16(dq) || !aligned16(df) || !aligned16(dW) ||
      !aligned16(workspace) || (dH0 && !aligned16(dH0)))
    return M2RNN_ERROR_INVALID_VALUE;
  m2rnn::BwdLaunch p{k, v, q, f, W, nullptr, dy, dH_T, dk, dv, dq, df, dW, dH0, workspace, B, H, T, K, V,
                     0, 0, 0};
  hipError_t e = m2rnn::launch_bwd_recompute(p, H0, ckpt, segment, is_split(algo), is_long(algo),
                                             reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? M2RNN_SUCCESS : M2RNN_ERROR_LAUNCH;
}

m2rnn_status m2rnn_frontend(const void* x, const void* Wx, const float* bias, void* k, void* v,
                            void* q, void* f, int B, int T, int D, int H, int K, int V,
                            m2rnn_dtype in_dtype, void* stream) {
  if (!x || !Wx || !bias || !k || !v || !q || !f) return M2RNN_ERROR_INVALID_VALUE;
  if (B < 1 || T < 1 || D < 1 || H < 1 || K < 1 || V < 1) return M2RNN_ERROR_INVALID_VALUE;
  if (!aligned16(x) || !aligned16(Wx) || !aligned16(k) || !aligned16(v) || !aligned16(q) ||
      !aligned16(f) || (reinterpret_cast<std::uintptr_t>(bias) & 3u))
    return M2RNN_ERROR_INVALID_VALUE;
  if (in_dtype != M2RNN_DTYPE_BF16) return M2RNN_ERROR_NOT_SUPPORTED;
  if (!supported_dim(K) || !supported_dim(V) || D % 8 != 0) return M2RNN_ERROR_NOT_SUPPORTED;
  // element counts: x (B T D), Wx (H R D), the outputs (B H T max(K, V))
  const long double lim = 4.0e18L;
  const long double R = 2.0L * K + V + 1;
  if ((long double)B * T * D >= lim || (long double)H * R * D >= lim || (long double)H * R >= 2.0e9L ||
      !counts_fit(B, H, T, K, V) || ((long double)B * T / 128 + 1) * ((long double)H * R / 128 + 1) >= 2.0e9L)
    return M2RNN_ERROR_INVALID_VALUE;
  m2rnn::FrontLaunch p{x, Wx, bias, k, v, q, f, B, T, D, H, K, V};
  hipError_t e = m2rnn::launch_frontend(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? M2RNN_SUCCESS : M2RNN_ERROR_LAUNCH;
}

m2rnn_status m2rnn_get_plan_ex(int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                               m2rnn_algo algo, unsigned flags, m2rnn_plan* plan) {
  if (!plan) return M2RNN_ERROR_INVALID_VALUE;
  const void* p = reinterpret_cast<const void*>(static_cast<std::uintptr_t>(0x10000));
  const float* pf = static_cast<const float*>(p);
  m2rnn_status st = check(p, p, p, p, p, nullptr, pf, nullptr, B, H, T, K, V, in_dtype, algo);
  if (st != M2RNN_SUCCESS) return st;
  if ((st = resolve_algo(algo, B, H, T, K, V, in_dtype, flags)) != M2RNN_SUCCESS) return st;
  const bool mf = algo == M2RNN_ALGO_MFMA || algo == M2RNN_ALGO_MFMA_SPLIT || algo == M2RNN_ALGO_MFMA_F16;
  const bool lg = is_long(algo);
  m2rnn::Plan pl = algo == M2RNN_ALGO_MFMA_F32 ? m2rnn::plan_mfma_f32(B, H, K, V)
                   : !(mf || lg)                 ? m2rnn::plan_simple(B, H, K, V)
                   : T == 1 && m2rnn::mfma_supports(K, V, 1) ? m2rnn::plan_decode(B, H, K, V)
                   : lg ? m2rnn::plan_long(B, H, K, V)
                        : m2rnn::plan_mfma(B, H, K, V, algo == M2RNN_ALGO_MFMA_SPLIT);
  if (pl.grid < 0) return M2RNN_ERROR_INVALID_VALUE;
  plan->algo = algo;
  plan->grid = pl.grid;
  plan->block = pl.block;
  plan->rows_per_group = pl.rows_per_group;
  plan->groups_per_unit = pl.groups_per_unit;
  plan->clears_y = pl.clears_y;
  plan->lds_bytes = pl.lds_bytes;
  return M2RNN_SUCCESS;
}

m2rnn_status m2rnn_get_plan(int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, m2rnn_plan* plan) {
  return m2rnn_get_plan_ex(B, H, T, K, V, in_dtype, algo, 0u, plan);
}

const char* m2rnn_status_string(m2rnn_status status) {
  switch (status) {
    case M2RNN_SUCCESS:
      return "success";
    case M2RNN_ERROR_INVALID_VALUE:
      return "invalid value (null pointer, size < 1, misaligned pointer or size overflow)";
    case M2RNN_ERROR_NOT_SUPPORTED:
      return "not supported (K or V not in {16, 32, ..., 128}, unknown dtype or algorithm, "
             "or an algorithm that does not cover the shape)";
    case M2RNN_ERROR_LAUNCH:
      return "kernel launch failed";
    case M2RNN_ERROR_SCRATCH_TOO_SMALL:
      return "the workspace this shape needs exceeds the library-owned scratch array "
             "(m2rnn_bwd_noalloc: 64 MiB per GPU)";
    default:
      return "unknown status";
  }
}

int m2rnn_version(void) { return 1000; }

}  // extern "C"
