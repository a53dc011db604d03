"""fp64 CPU oracle for the M²RNN forward recurrence.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the test suite, the smoke check and the CPU-baseline leg of
the benchmark use it. It shares no code with the HIP library; it reads the same
stored input bits and widens them itself.

What it computes (the definition, written out step by step):

  state update — gist.science technical summary (zh) §2.1 "core architecture
  design", the two update equations (restated in the ja summary §2.1 and, with
  garbled TeX, in the wispaper blog §"1. The Core Recurrence"):
      Z_t = tanh(H_{t-1} W + k_t v_t^T)
      H_t = f_t H_{t-1} + (1 - f_t) Z_t
  with H_t a K x V matrix, k_t in R^K, v_t in R^V, W the V x V transition
  matrix (the shape forced by the product H_{t-1} W being K x V; one matrix per
  head), and f_t a scalar gate in [0, 1] that depends on the input only
  (zh §2.1, forget-gate bullet list).

  readout — not given on the pages (they name queries only in the tensor-
  parallel paragraph of zh §2.2). The reading taken here: y_t = H_t^T q_t with
  q_t in R^K and the post-update state H_t, no scale, norm or gate.

Everything is evaluated in IEEE fp64 from the exactly widened stored inputs.
Units (batch, head) are independent and are evaluated side by side as a batch
of separate matrices; each unit's arithmetic is the per-step sequence above.
The products H_{t-1} W and H_t^T q_t use numpy's matmul as a library step.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

__all__ = ["widen", "m2rnn_fwd_ref", "round_to_bf16", "round_to_f16"]


def widen(x: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Exact fp64 value of stored inputs: fp32 arrays, or uint16 bfloat16 bits."""
    if x is None:
        return None
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":  # exact fp64 inputs (finite-difference checks of the oracle)
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Diagnostic only: value of x (fp64) rounded to fp32, then to bfloat16 (RNE)."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_to_f16(x: np.ndarray) -> np.ndarray:
    """Diagnostic only: value of x (fp64) rounded to fp32, then to IEEE binary16
    (RNE, subnormals kept, overflow to infinity)."""
    with np.errstate(over="ignore"):
        return x.astype(np.float32).astype(np.float16).astype(np.float64)


def m2rnn_fwd_ref(
    k: np.ndarray,
    v: np.ndarray,
    q: np.ndarray,
    f: np.ndarray,
    W: np.ndarray,
    H0: Optional[np.ndarray] = None,
    *,
    dtype: str,
    return_states: bool = False,
    state_rounding: Optional[str] = None,
) -> Tuple[np.ndarray, ...]:
    """Forward recurrence in fp64.

    Arguments are the stored inputs: k, q [B,H,T,K]; v [B,H,T,V]; f [B,H,T];
    W [H,V,V]; all in ``dtype`` storage ("f32" arrays or "bf16" uint16 bits).
    H0 [B,H,K,V] fp32 (or fp64, to continue an earlier oracle run exactly), or
    None for the zero state.

    Returns (y [B,H,T,V], H_T [B,H,K,V]) in fp64, plus all states
    [B,H,T,K,V] when ``return_states``.

    ``state_rounding="bf16"`` (or ``"f16"``) is a diagnostic variant (not the
    definition): the state is rounded to bfloat16 (IEEE binary16) before each
    product with W, to estimate how much a matrix product on such an operand
    perturbs the trajectory.
    """
    kk, vv, qq, ff, WW = (widen(a, dtype) for a in (k, v, q, f, W))
    B, H, T, K = kk.shape
    V = vv.shape[-1]
    if vv.shape != (B, H, T, V) or qq.shape != (B, H, T, K) or ff.shape != (B, H, T):
        raise ValueError("inconsistent input shapes")
    if WW.shape != (H, V, V):
        raise ValueError("W must be [H, V, V]")
    if T < 1:
        raise ValueError("T must be >= 1")
    if H0 is None:
        S = np.zeros((B, H, K, V), dtype=np.float64)
    else:
        H0 = np.asarray(H0)
        # fp32 at the boundary; an fp64 state (a continued oracle run) is taken as is
        S = H0.astype(np.float64) if H0.dtype == np.float64 else H0.astype(np.float32).astype(np.float64)
        if S.shape != (B, H, K, V):
            raise ValueError("H0 must be [B, H, K, V]")
    y = np.empty((B, H, T, V), dtype=np.float64)
    states = np.empty((B, H, T, K, V), dtype=np.float64) if return_states else None
    Wb = WW[None, :, :, :]  # the per-head matrix, shared by every batch row
    for t in range(T):
        S_in = round_to_bf16(S) if state_rounding == "bf16" else round_to_f16(S) if state_rounding == "f16" else S
        A = np.matmul(S_in, Wb)                                       # H_{t-1} W
        outer = kk[:, :, t, :, None] * vv[:, :, t, None, :]           # k_t v_t^T
        Z = np.tanh(A + outer)
        ft = ff[:, :, t, None, None]
        S = ft * S + (1.0 - ft) * Z                                   # gate blend
        y[:, :, t, :] = np.matmul(qq[:, :, t, None, :], S)[:, :, 0, :]  # H_t^T q_t
        if states is not None:
            states[:, :, t] = S
    if return_states:
        return y, S, states
    return y, S
