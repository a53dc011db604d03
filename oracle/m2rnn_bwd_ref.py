"""fp64 CPU oracle for the gradients of the M²RNN forward recurrence.

TEST INFRASTRUCTURE ONLY (like m2rnn_ref): nothing on the product path imports,
calls or runs this module, and it shares no code with the HIP library.

What it computes. The pages give the forward update only (gist.science
technical summary (zh) §2.1, the two update equations) and say that the
backward pass recomputes the forward states (zh §2.2, parallelism paragraph).
The gradients are therefore the plain definition: the chain rule applied to the
forward function as the oracle defines it,

    A_t = H_{t-1} W + k_t v_t^T,   Z_t = tanh(A_t),
    H_t = f_t H_{t-1} + (1 - f_t) Z_t,   y_t = H_t^T q_t,

for a loss L whose gradients with respect to the outputs are given: dy_t = dL/dy_t
(V entries per step) and dH_T = dL/dH_T (K x V). Going backwards in time with
G = dL/dH_t (the total gradient reaching the state after step t):

    G      += q_t dy_t^T                      (y_t reads H_t)
    dq_t    = H_t dy_t
    dZ      = (1 - f_t) G
    df_t    = sum_ij (H_{t-1} - Z_t)_ij G_ij
    dA      = dZ * (1 - Z_t^2)
    dk_t    = dA v_t,   dv_t = dA^T k_t
    dW     += H_{t-1}^T dA                    (summed over the batch rows too)
    G       = f_t G + dA W^T                  (the gradient reaching H_{t-1})

and dH0 = G after step 0. Everything runs in IEEE fp64 from the exactly widened
stored inputs; the products use numpy's matmul as a library step.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .m2rnn_ref import widen

__all__ = ["m2rnn_bwd_ref"]


def m2rnn_bwd_ref(
    k: np.ndarray,
    v: np.ndarray,
    q: np.ndarray,
    f: np.ndarray,
    W: np.ndarray,
    H0: Optional[np.ndarray],
    dy: np.ndarray,
    dH_T: Optional[np.ndarray] = None,
    *,
    dtype: str,
) -> Dict[str, np.ndarray]:
    """Gradients of L with respect to every input, in fp64.

    Inputs as m2rnn_fwd_ref (stored k, v, q, f, W in ``dtype``; H0 fp32 or None);
    dy [B,H,T,V] and dH_T [B,H,K,V] (None: no gradient on the final state) are
    taken as given (widened to fp64). Returns a dict with dk, dq [B,H,T,K],
    dv [B,H,T,V], df [B,H,T], dW [H,V,V], dH0 [B,H,K,V], plus y and H_T of the
    forward pass.
    """
    kk, vv, qq, ff, WW = (widen(a, dtype) for a in (k, v, q, f, W))
    B, H, T, K = kk.shape
    V = vv.shape[-1]
    if vv.shape != (B, H, T, V) or qq.shape != (B, H, T, K) or ff.shape != (B, H, T):
        raise ValueError("inconsistent input shapes")
    if WW.shape != (H, V, V):
        raise ValueError("W must be [H, V, V]")
    dyy = np.asarray(dy, dtype=np.float64)
    if dyy.shape != (B, H, T, V):
        raise ValueError("dy must be [B, H, T, V]")
    if H0 is None:
        S0 = np.zeros((B, H, K, V))
    else:
        # fp32 at the boundary; an fp64 state is taken as is (as in m2rnn_fwd_ref)
        H0 = np.asarray(H0)
        S0 = H0.astype(np.float64) if H0.dtype == np.float64 else H0.astype(np.float32).astype(np.float64)

    # forward pass, keeping every state and every tanh output
    Wb = WW[None]
    S = np.empty((T + 1, B, H, K, V))
    Zs = np.empty((T, B, H, K, V))
    S[0] = S0
    y = np.empty((B, H, T, V))
    for t in range(T):
        A = np.matmul(S[t], Wb) + kk[:, :, t, :, None] * vv[:, :, t, None, :]
        Zs[t] = np.tanh(A)
        ft = ff[:, :, t, None, None]
        S[t + 1] = ft * S[t] + (1.0 - ft) * Zs[t]
        y[:, :, t] = np.matmul(qq[:, :, t, None, :], S[t + 1])[:, :, 0, :]

    # backward pass
    G = np.zeros((B, H, K, V)) if dH_T is None else np.asarray(dH_T, dtype=np.float64).copy()
    dk = np.empty((B, H, T, K))
    dq = np.empty((B, H, T, K))
    dv = np.empty((B, H, T, V))
    df = np.empty((B, H, T))
    dW = np.zeros((H, V, V))
    WT = np.swapaxes(WW, -1, -2)[None]
    for t in range(T - 1, -1, -1):
        G = G + qq[:, :, t, :, None] * dyy[:, :, t, None, :]
        dq[:, :, t] = np.matmul(S[t + 1], dyy[:, :, t, :, None])[..., 0]
        ft = ff[:, :, t, None, None]
        dZ = (1.0 - ft) * G
        df[:, :, t] = np.sum((S[t] - Zs[t]) * G, axis=(-2, -1))
        dA = dZ * (1.0 - Zs[t] ** 2)
        dk[:, :, t] = np.matmul(dA, vv[:, :, t, :, None])[..., 0]
        dv[:, :, t] = np.matmul(np.swapaxes(dA, -1, -2), kk[:, :, t, :, None])[..., 0]
        dW += np.sum(np.matmul(np.swapaxes(S[t], -1, -2), dA), axis=0)
        G = ft * G + np.matmul(dA, WT)
    return {"dk": dk, "dv": dv, "dq": dq, "df": df, "dW": dW, "dH0": G, "y": y, "H_T": S[T]}
