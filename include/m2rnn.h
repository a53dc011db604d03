/*
 * m2rnn.h — C ABI of the M²RNN forward recurrence for AMD Instinct MI355X (gfx950).
 *
 * The operation (state update as in the gist.science technical summary of
 * "M²RNN: Non-Linear RNNs with Matrix-Valued States for Scalable Language
 * Modeling", §2.1 core architecture design, update equations; the same pair in
 * the Japanese summary §2.1): for every (batch b, head h) independently, with
 * a K x V state H and t = 1..T,
 *
 *     Z_t = tanh(H_{t-1} W_h + k_t v_t^T)
 *     H_t = f_t H_{t-1} + (1 - f_t) Z_t
 *     y_t = H_t^T q_t            (readout: not given on the pages; the reading
 *                                 taken here uses the post-update state)
 *
 * W_h is the head's V x V transition matrix, multiplied from the right so that
 * it mixes the value axis; f_t is one scalar gate per (b, h, t) in [0, 1],
 * consumed as given (its parameterisation from the input is outside this call).
 *
 * Layouts (all contiguous, row-major, no strides):
 *   k, q  [B][H][T][K]        in_dtype
 *   v     [B][H][T][V]        in_dtype
 *   f     [B][H][T]           in_dtype
 *   W     [H][V][V]           in_dtype, (H W)[i][j] = sum_l H[i][l] * W[h][l][j]
 *   H0    [B][H][K][V]        fp32, may be NULL (zero initial state)
 *   y     [B][H][T][V]        fp32 output
 *   H_T   [B][H][K][V]        fp32 output, may be NULL; may equal H0 (in-place
 *                             continuation); no other overlap is allowed.
 * in_dtype M2RNN_DTYPE_BF16 means every input element is a bfloat16 bit
 * pattern (uint16); M2RNN_DTYPE_F32 means IEEE fp32.
 *
 * Pointers are device pointers (hipMalloc'd or equivalent), each 16-byte
 * aligned. The caller owns every buffer and the stream. The library allocates
 * nothing; calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream) and results are valid once the caller synchronises that stream.
 * Before the recurrence kernel, a call may clear y with a fill kernel enqueued
 * on the same stream. The library keeps no global mutable state and is safe to
 * call from several host threads.
 *
 * Errors: arguments are validated on the host before any HIP call; a failed
 * validation enqueues nothing. INVALID_VALUE: a required pointer (k, v, q, f,
 * W, y) is NULL, a size is < 1, a pointer is not 16-byte aligned, or the
 * element counts overflow 2^62. NOT_SUPPORTED: K or V is not one of 16, 32,
 * ..., 128 (multiples of 16, the matrix-unit granularity the pages state in
 * the zh summary §2.2), an unknown dtype or algorithm, or an algorithm that
 * does not cover the requested shape/dtype. LAUNCH: the HIP launch reported
 * an error. NaN/Inf inputs are not checked; they propagate.
 */
#ifndef M2RNN_H_
#define M2RNN_H_

#ifdef __cplusplus
extern "C" {
#endif

typedef enum m2rnn_status {
  M2RNN_SUCCESS = 0,
  M2RNN_ERROR_INVALID_VALUE = 1,
  M2RNN_ERROR_NOT_SUPPORTED = 2,
  M2RNN_ERROR_LAUNCH = 3,
  /* m2rnn_bwd_noalloc only: the shape needs more workspace than the
   * library-owned scratch array holds (64 MiB per GPU) */
  M2RNN_ERROR_SCRATCH_TOO_SMALL = 4
} m2rnn_status;

typedef enum m2rnn_dtype {
  M2RNN_DTYPE_F32 = 0,
  M2RNN_DTYPE_BF16 = 1
} m2rnn_dtype;

/* Kernel family.
 * SIMPLE:     one workgroup per (b, h), fp32 arithmetic from LDS; covers every
 *             supported shape and both dtypes.
 * MFMA_F32:   fp32 inputs, every supported K and V: the fp32 path on the matrix
 *             cores. One workgroup of K/16 waves per (b, h); the state, W, the
 *             rank-1 term and the readout stay fp32 (H_{t-1} W on
 *             v_mfma_f32_16x16x4_f32, no operand rounding beyond fp32). y is
 *             summed over the waves in a fixed order and written once, so every
 *             output is bitwise repeatable.
 * MFMA:       bf16 inputs, K in {32, 64, 128}, V in {64, 128}; the fp32 state
 *             stays in registers across all steps, H_{t-1} W runs on
 *             v_mfma_f32_16x16x32_bf16 with the state rounded to bf16
 *             (round-to-nearest-even) as the matrix operand and fp32
 *             accumulation; rank-1 write, tanh, gate blend and readout are
 *             fused in the same kernel. Fastest; per-step operand rounding of
 *             2^-9 relative, which a sensitive trajectory can amplify: on the
 *             workloads with gates near 1 and inputs scaled by 1/sqrt(K)
 *             (B=4 H=8 K=V=64 T=512, and B=2 H=16 K=64 V=128 T=32768) it misses
 *             the 2e-2 normwise bar (measured on all units: H_T 2.2e-2 on the
 *             first, y 2.4e-2 on the second); on the others it is ~2e-3.
 * MFMA_SPLIT: as MFMA with the state operand split into bf16 hi + bf16 lo and
 *             two MFMA passes (~2^-17 relative operand error); the readout
 *             takes both halves too (y and H_T within ~1e-5 to 3e-4 of the
 *             fp64 definition on every workload measured).
 * AUTO:       fp32: MFMA_F32. bf16 with V in {64, 128}, T > 1 and at most
 *             768 16-row tiles (B H K / 16 <= 768; two workgroups fit per CU of
 *             a 256-CU gfx950): MFMA_LONG_F16; else MFMA_F16 where it covers
 *             the shape, else SIMPLE. The fp16 operand meets the 2e-2 bar on
 *             every unit of every workload measured, at the single operand's
 *             cost; inputs outside its domain (see MFMA_F16) need MFMA_SPLIT or
 *             MFMA_LONG_SPLIT, named explicitly. Every choice gives a bitwise
 *             repeatable y onto a y the call clears; with
 *             M2RNN_FLAG_DETERMINISTIC and M2RNN_FLAG_ACCUMULATE_Y together it
 *             avoids the families that add two or more partial readouts into y.
 *             The training entry points resolve AUTO to MFMA_SPLIT or
 *             MFMA_LONG_SPLIT (the backward pass reads bf16 operands).
 * MFMA_LONG, MFMA_LONG_SPLIT: the same arithmetic as MFMA / MFMA_SPLIT, for
 *             workloads with few 16-row tiles (B H K / 16 well below the GPU's
 *             1024 SIMDs: small batches, long sequences). Each tile's V columns
 *             are spread over V/32 waves (V/16 at V = 64, except in the training
 *             forwards) that exchange the state operand through LDS every step,
 *             which cuts the per-step latency; each tile is its
 *             own workgroup, so y is summed over a unit's K/16 tiles with atomic
 *             adds. Each tile's contribution to y_t is first rounded to a grid of
 *             spacing 2^(E-23), where 2^E > 1.0625 ||q_t||_1 M_t bounds |y_t|
 *             (M_t: the bound on |H_t| from the gated convex update, M_0 =
 *             max(1, max |H0|)); sums of such values are exact in fp32, so y does
 *             not depend on the order of the adds (onto the y the call clears)
 *             and is bitwise repeatable. The grid adds at most
 *             2^-23 ||q_t||_1 M_t per tile to an element's error. The saving
 *             forward of the training entry points adds unrounded sums (its y's
 *             last bits can vary between runs; H_T and `saved` cannot).
 *             bf16, K in {16, ..., 128}, V in {64, 128}; the
 *             training forwards take them for K in {32, 64, 128} (the shapes
 *             the backward pass covers) and write the same `saved` layout.
 *             MFMA_LONG has MFMA's precision (misses the bar on the same two
 *             workloads: H_T 2.6e-2, y 2.6e-2); MFMA_LONG_SPLIT has MFMA_SPLIT's
 *             (both halves in the products and the readout).
 * MFMA_F16, MFMA_LONG_F16: MFMA / MFMA_LONG with the state operand rounded to
 *             fp16 (round-to-nearest-even, 11 significant bits: 2^-12 relative
 *             per step instead of 2^-9) on v_mfma_f32_16x16x32_f16, at the single
 *             operand's cost; W and q are converted from bf16 to fp16 inside the
 *             kernel (exact for magnitudes in [2^-17, 65504]). Their domain is
 *             fp16's range: |W| and |q| at most 65504, max |H0| at most 22 700
 *             (the operand is 2/ln 2 H, and |H_t| <= max(1, max |H0|) for gates
 *             in [0, 1]); a W, q or H0 value beyond it makes the outputs it
 *             reaches NaN (never a finite wrong value), and gates outside [0, 1]
 *             are outside the method. Magnitudes below fp16's normal range
 *             (6.1e-5) keep fewer bits (absolute rounding 2^-25), which matters
 *             only for workloads whose states and inputs are all that small.
 *             Forward only (no training entry point takes them); one step
 *             (T = 1) runs the decoding kernel as for every matrix-core family;
 *             their y is as repeatable as MFMA's / MFMA_LONG's. Measured on
 *             every unit of the five workloads: see the parity tests. */
typedef enum m2rnn_algo {
  M2RNN_ALGO_AUTO = 0,
  M2RNN_ALGO_SIMPLE = 1,
  M2RNN_ALGO_MFMA = 2,
  M2RNN_ALGO_MFMA_SPLIT = 3,
  M2RNN_ALGO_MFMA_LONG = 4,
  M2RNN_ALGO_MFMA_LONG_SPLIT = 5,
  M2RNN_ALGO_MFMA_F32 = 6,
  M2RNN_ALGO_MFMA_F16 = 7,
  M2RNN_ALGO_MFMA_LONG_F16 = 8
} m2rnn_algo;

/* The forward recurrence with the automatically chosen kernel. */
m2rnn_status m2rnn_fwd(const void* k, const void* v, const void* q, const void* f, const void* W,
                       const float* H0, float* y, float* H_T,
                       int B, int H, int T, int K, int V, m2rnn_dtype in_dtype, void* stream);

/* The same with an explicit kernel family (for tests and measurements). */
m2rnn_status m2rnn_fwd_algo(const void* k, const void* v, const void* q, const void* f, const void* W,
                            const float* H0, float* y, float* H_T,
                            int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, void* stream);

/* Flags for m2rnn_fwd_ex. */
enum {
  /* Add the readout into y instead of overwriting it: y[b][h][t][:] += H_t^T q_t.
   * The library then never clears y itself, so a caller that zeroes y first
   * gets the plain result with the recurrence as the only kernel on the stream. */
  M2RNN_FLAG_ACCUMULATE_Y = 1u,
  /* Every output bitwise repeatable from run to run. H_T always is; y is
   * whenever each element receives at most one atomic contribution, two onto a
   * y the call cleared itself, or the long families' grid-rounded contributions
   * onto a y the call cleared itself. The families that add partial readouts into
   * y atomically are MFMA and MFMA_SPLIT at K = 128 (two workgroups per unit) and
   * MFMA_LONG* with T > 1 (K/16 row tiles per unit; T = 1 on the matrix-core
   * shapes runs the decoding kernel, which has no atomics). So only together
   * with M2RNN_FLAG_ACCUMULATE_Y does this flag change anything: AUTO then keeps
   * to a repeatable combination (MFMA_SPLIT in place of MFMA_LONG_SPLIT where it
   * has one workgroup per unit, SIMPLE where nothing else is), and an explicit
   * family that adds two or more contributions into the caller's y is
   * NOT_SUPPORTED. */
  M2RNN_FLAG_DETERMINISTIC = 2u
};

/* m2rnn_fwd_algo with flags (a bitwise OR of M2RNN_FLAG_*; unknown bits are
 * NOT_SUPPORTED). */
m2rnn_status m2rnn_fwd_ex(const void* k, const void* v, const void* q, const void* f, const void* W,
                          const float* H0, float* y, float* H_T,
                          int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                          m2rnn_algo algo, unsigned flags, void* stream);

/* Variable-length batch in the padded layout above (continuous decoding and
 * ragged batches). Sequence b uses its first seq_len[b] steps: T is the longest
 * length and the rows t >= seq_len[b] of k, v, q, f are not read. H_T[b] is the
 * state after seq_len[b] steps (H0[b] unchanged for seq_len[b] = 0), and the y
 * rows t >= seq_len[b] are set to zero (left untouched with
 * M2RNN_FLAG_ACCUMULATE_Y). For serving with a state cache, call with T = 1 and
 * H_T == H0 and give idle sequences length 0. The per-step arithmetic is that of
 * m2rnn_fwd; the pages define only the recurrence, so this entry point is an
 * interface of this library.
 *   seq_len: device array of B int32, 4-byte aligned; NULL means every length
 *            is T. The host cannot read device memory without synchronising, so
 *            the kernels clamp each length into [0, T] instead of rejecting it.
 * Errors as m2rnn_fwd_ex, plus INVALID_VALUE for a misaligned seq_len. */
m2rnn_status m2rnn_fwd_varlen(const void* k, const void* v, const void* q, const void* f, const void* W,
                              const float* H0, float* y, float* H_T, const int* seq_len,
                              int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                              m2rnn_algo algo, unsigned flags, void* stream);

/* ---- Training: the forward pass that keeps what the backward pass reads, and
 * the backward pass (gradients of a loss L given dL/dy and dL/dH_T). The
 * gradients are the chain rule of the update equations above; the pages state
 * that the backward pass works from recomputed forward states cached in HBM
 * (zh summary §2.2, parallelism paragraph). Here the forward pass writes, per
 * step, the bf16 state operand of the matrix product and the bf16
 * pre-activation into `saved`, and the backward pass reads them in reverse.
 * Both cover bf16 inputs on the MFMA kernel family only (K in {32, 64, 128},
 * V in {64, 128}); other shapes and dtypes are NOT_SUPPORTED. */

/* Bytes of the `saved` buffer for one forward pass of this shape
 * ((2T + 1) * B * H * K * V * 2; 0 when the shape is not covered). */
unsigned long long m2rnn_saved_bytes(int B, int H, int T, int K, int V);

/* Training forward: m2rnn_fwd_algo that also fills `saved` (device, 16-byte
 * aligned, m2rnn_saved_bytes large, caller-owned; its layout is private to the
 * library and only m2rnn_bwd reads it). algo: MFMA, MFMA_SPLIT, MFMA_LONG,
 * MFMA_LONG_SPLIT (the same layout), or AUTO = the split operand: MFMA_LONG_SPLIT
 * where m2rnn_pick_algo takes the latency-oriented kernel (MFMA_LONG_F16), else
 * MFMA_SPLIT. The fp16-operand families are NOT_SUPPORTED here. */
m2rnn_status m2rnn_fwd_save(const void* k, const void* v, const void* q, const void* f, const void* W,
                            const float* H0, float* y, float* H_T, void* saved,
                            int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, void* stream);

/* Bytes of the backward pass's scratch buffer for this shape (0 when not covered). */
unsigned long long m2rnn_bwd_workspace_bytes(int B, int H, int T, int K, int V);

/* Backward pass. Inputs as m2rnn_fwd_save, plus `saved` from that call with the
 * same inputs, dy [B][H][T][V] fp32 (dL/dy) and dH_T [B][H][K][V] fp32 (dL/dH_T;
 * NULL means 0). Outputs, fp32 and caller-owned: dk, dq [B][H][T][K],
 * dv [B][H][T][V], df [B][H][T], dW [H][V][V] (summed over the batch),
 * dH0 [B][H][K][V] (may be NULL). `workspace`: device, 16-byte aligned,
 * m2rnn_bwd_workspace_bytes large. The matrix products take the bf16 state and
 * gradient operands, like the forward's MFMA kernel. Asynchronous on `stream`;
 * the outputs are complete when the stream is. Errors as m2rnn_fwd_ex. */
m2rnn_status m2rnn_bwd(const void* k, const void* v, const void* q, const void* f, const void* W,
                       const float* H0, const void* saved, const float* dy, const float* dH_T,
                       float* dk, float* dv, float* dq, float* df, float* dW, float* dH0,
                       void* workspace, int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                       void* stream);

/* m2rnn_bwd with an explicit reverse-time kernel (m2rnn_bwd is AUTO). MFMA,
 * MFMA_SPLIT: one wave per 16-row tile; MFMA_LONG, MFMA_LONG_SPLIT: a workgroup
 * of V/32 waves per tile exchanging dA through LDS every step (few tiles, long
 * sequences), its dv and df sums over a unit's tiles added in tile order by a
 * second kernel; AUTO: MFMA_LONG_SPLIT where m2rnn_pick_algo takes the
 * latency-oriented kernel (MFMA_LONG_F16), else MFMA_SPLIT.
 * Either kernel reads the `saved` of either forward family, and every output is
 * deterministic. NOT_SUPPORTED for other families. */
m2rnn_status m2rnn_bwd_algo(const void* k, const void* v, const void* q, const void* f, const void* W,
                            const float* H0, const void* saved, const float* dy, const float* dH_T,
                            float* dk, float* dv, float* dq, float* df, float* dW, float* dH0,
                            void* workspace, int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, void* stream);

/* m2rnn_bwd_algo for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * arguments are m2rnn_bwd_algo's without `workspace`: the workspace lives in a
 * device array inside the library, 64 MiB per GPU, which each GPU holds from its
 * first use until the process ends. The call allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine); the caller still passes every
 * input and output. Its first call on a device resolves the array's address on
 * that device (do it once before capturing a graph). Results are bitwise those
 * of m2rnn_bwd_algo with the same arguments.
 * All calls on one GPU share its array: calls that overlap on one GPU (other
 * streams, other host threads) race and give undefined results; calls ordered
 * on one stream are safe (each call writes every part of the array it reads).
 * Errors as m2rnn_bwd_algo, plus M2RNN_ERROR_SCRATCH_TOO_SMALL, returned before
 * any HIP call, when m2rnn_bwd_workspace_bytes(B, H, T, K, V) exceeds 64 MiB
 * (for example B H T K V above about 29 million elements at K = V = 128). */
m2rnn_status m2rnn_bwd_noalloc(const void* k, const void* v, const void* q, const void* f, const void* W,
                               const float* H0, const void* saved, const float* dy, const float* dH_T,
                               float* dk, float* dv, float* dq, float* df, float* dW, float* dH0,
                               int B, int H, int T, int K, int V, m2rnn_dtype in_dtype, m2rnn_algo algo,
                               void* stream);

/* ---- Training with recomputation (zh summary §2.2, parallelism paragraph: the
 * backward pass recomputes the forward states rather than keeping them all).
 * The sequence is cut into segments of `segment` steps (the last one may be
 * shorter). The training forward keeps only the state at each segment start
 * after the first; the backward pass visits the segments last to first,
 * recomputes each segment's states from its checkpoint into its workspace and
 * runs the reverse-time pass over it. Memory: checkpoints of (ceil(T/segment) - 1)
 * B H K V floats, plus a workspace that holds one segment. With segment >= T there
 * is no checkpoint at all: the plain forward pass (m2rnn_fwd) is the training
 * forward, and the backward pass recomputes the whole sequence from H0. Same
 * shapes and dtypes as m2rnn_fwd_save; same outputs and errors as m2rnn_bwd. */

/* Bytes of the checkpoint buffer: (ceil(T/segment) - 1) * B * H * K * V * 4
 * (0: none needed, or invalid sizes). */
unsigned long long m2rnn_ckpt_bytes(int B, int H, int T, int K, int V, int segment);

/* m2rnn_fwd_algo (algo as m2rnn_fwd_save) that also writes
 * ckpt[j - 1] = H_{j * segment} for j = 1 .. ceil(T/segment) - 1, fp32
 * [B][H][K][V] each (device, 16-byte aligned, caller-owned; may be NULL when
 * m2rnn_ckpt_bytes is 0). It runs as one launch per segment.
 * INVALID_VALUE also for segment < 1. */
m2rnn_status m2rnn_fwd_ckpt(const void* k, const void* v, const void* q, const void* f, const void* W,
                            const float* H0, float* y, float* H_T, float* ckpt,
                            int B, int H, int T, int K, int V, int segment, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, void* stream);

/* Bytes of m2rnn_bwd_recompute's workspace (0 when the shape is not covered). */
unsigned long long m2rnn_bwd_recompute_workspace_bytes(int B, int H, int T, int K, int V, int segment);

/* Backward pass from checkpoints: arguments as m2rnn_bwd, with `ckpt` from
 * m2rnn_fwd_ckpt (same inputs, same segment) in place of `saved`, and H0 the
 * initial state of the forward call (NULL: zero). `algo` (as m2rnn_fwd_save)
 * picks the forward that recomputes the states and the reverse kernel (as
 * m2rnn_bwd_algo); it should be the one the forward pass ran, so that the
 * recomputed states are the ones that produced y (another family rebuilds them
 * to fp32 rounding). `workspace`: m2rnn_bwd_recompute_workspace_bytes large.
 * Issues five to seven launches per segment on `stream`. */
m2rnn_status m2rnn_bwd_recompute(const void* k, const void* v, const void* q, const void* f,
                                 const void* W, const float* H0, const float* ckpt, const float* dy,
                                 const float* dH_T, float* dk, float* dv, float* dq, float* df,
                                 float* dW, float* dH0, void* workspace, int B, int H, int T, int K,
                                 int V, int segment, m2rnn_dtype in_dtype, m2rnn_algo algo,
                                 void* stream);

/* ---- Layer front-end: the inputs of the recurrence from the layer input.
 * The pages derive k_t, v_t (and q_t) from x_t and make the forget gate a
 * parameterised function psi(x_t) of the input alone that keeps f_t in [0, 1],
 * with different decay rates per head (zh summary §2.1). Read here as per-head
 * linear projections and a logistic sigmoid with a per-head bias:
 *   k_t = Wk_h x_t,  v_t = Wv_h x_t,  q_t = Wq_h x_t,
 *   f_t = 1 / (1 + exp(-(w_h . x_t + bias_h))).
 * One matrix product over the model width D with the sigmoid and the layout
 * change fused into its epilogue.
 *   x    [B][T][D] bf16, the layer input (row b T + t);
 *   Wx   [H][2K + V + 1][D] bf16: per head K rows for k, V rows for v, K rows
 *        for q, then the gate row;
 *   bias [H] fp32 (4-byte aligned);
 *   k, q [B][H][T][K], v [B][H][T][V], f [B][H][T]: bf16 outputs (round to
 *        nearest even), exactly the inputs m2rnn_fwd and the training entry
 *        points read.
 * Accumulation is fp32. All pointers are device memory owned by the caller;
 * x, Wx and the outputs 16-byte aligned. Asynchronous on `stream`.
 * INVALID_VALUE: a NULL or misaligned pointer, a size < 1, sizes that overflow.
 * NOT_SUPPORTED: in_dtype not BF16, K or V not in {16, 32, ..., 128}, D not a
 * multiple of 8. */
m2rnn_status m2rnn_frontend(const void* x, const void* Wx, const float* bias, void* k, void* v,
                            void* q, void* f, int B, int T, int D, int H, int K, int V,
                            m2rnn_dtype in_dtype, void* stream);

/* Host-only argument check: returns exactly what m2rnn_fwd_algo would return
 * before launching, without touching the GPU. */
m2rnn_status m2rnn_check_args(const void* k, const void* v, const void* q, const void* f, const void* W,
                              const float* H0, const float* y, const float* H_T,
                              int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                              m2rnn_algo algo);

/* The kernel family AUTO resolves to for a shape without flags (never AUTO;
 * host only). */
m2rnn_algo m2rnn_pick_algo(int B, int H, int T, int K, int V, m2rnn_dtype in_dtype);

/* Launch plan of one call (host only, no GPU access). */
typedef struct m2rnn_plan {
  int algo;             /* resolved m2rnn_algo (never AUTO) */
  int grid;             /* workgroups of the recurrence kernel */
  int block;            /* threads per workgroup */
  int rows_per_group;   /* state rows (of K) one workgroup carries */
  int groups_per_unit;  /* workgroups sharing one (b, h); their readouts are summed into y */
  int clears_y;         /* 1 if a call without M2RNN_FLAG_ACCUMULATE_Y enqueues a fill of y first */
  int lds_bytes;        /* LDS per workgroup */
} m2rnn_plan;

/* Fill *plan for a call with these arguments. INVALID_VALUE for a NULL plan or
 * sizes < 1; NOT_SUPPORTED as m2rnn_check_args. */
m2rnn_status m2rnn_get_plan(int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                            m2rnn_algo algo, m2rnn_plan* plan);

/* m2rnn_get_plan for a call of m2rnn_fwd_ex / m2rnn_fwd_varlen with `flags`:
 * plan->algo is the family that call runs (AUTO resolved under the flags'
 * rules), and the status is the one that call would return before launching
 * (NOT_SUPPORTED for unknown flag bits or a deterministic call on a family that
 * sums y atomically). Host only. */
m2rnn_status m2rnn_get_plan_ex(int B, int H, int T, int K, int V, m2rnn_dtype in_dtype,
                               m2rnn_algo algo, unsigned flags, m2rnn_plan* plan);

/* Static text for a status code ("unknown status" for other values). */
const char* m2rnn_status_string(m2rnn_status status);

/* Library ABI version: major * 10000 + minor * 100 + patch (0.2.0 added
 * m2rnn_fwd_varlen and the training entry points, 0.3.0 the recomputing ones and the front-end, 0.4.0 MFMA_LONG, 0.5.0 AUTO's
 * choice of MFMA_LONG_SPLIT and M2RNN_FLAG_DETERMINISTIC, 0.6.0 MFMA_LONG* in
 * the training forwards and m2rnn_bwd_algo, 0.7.0 m2rnn_get_plan_ex and
 * m2rnn_bwd_noalloc, 0.8.0 MFMA_F32, 0.9.0 the grid-rounded, order-independent y of
 * MFMA_LONG*, 0.10.0 MFMA_F16 and MFMA_LONG_F16). */
int m2rnn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* M2RNN_H_ */
