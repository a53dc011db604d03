"""fp64 CPU oracle for the layer front-end that feeds the M²RNN recurrence.

TEST INFRASTRUCTURE ONLY (like m2rnn_ref): nothing on the product path imports,
calls or runs this module, and it shares no code with the HIP library.

What it computes. The pages describe the layer around the recurrence in words
(gist.science technical summary (zh) §2.1): k_t, v_t (and q_t) come from the
input x_t, and the scalar forget gate is f_t = psi(x_t), a parameterised function
of the input alone that keeps f_t in [0, 1], with the heads initialised to
different decay rates. The reading taken here is the plainest one the rest
supports: per head h, linear projections of x_t, and psi = the logistic sigmoid
of a linear projection plus a per-head bias,

    k_t = Wk_h x_t,   v_t = Wv_h x_t,   q_t = Wq_h x_t,
    f_t = 1 / (1 + exp(-(w_h . x_t + b_h))),

with the per-head weights stored as the rows of one matrix Wx_h of
2K + V + 1 rows: K rows for k, V for v, K for q, then the gate row. Everything
is fp64 from the exactly widened stored inputs; the contraction over the model
width is numpy's matmul, used as a library step.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .m2rnn_ref import widen

__all__ = ["m2rnn_frontend_ref", "sigmoid_ref"]


def sigmoid_ref(z: np.ndarray) -> np.ndarray:
    """The logistic function 1 / (1 + e^-z), in fp64, written so that neither
    branch overflows: for z < 0 it is e^z / (1 + e^z)."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def m2rnn_frontend_ref(x: np.ndarray, Wx: np.ndarray, bias: np.ndarray, *, K: int, V: int,
                       dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """x [B,T,D] and Wx [H, 2K+V+1, D] in ``dtype`` storage, bias [H] (fp32).

    Returns fp64 k, q [B,H,T,K], v [B,H,T,V], the gate logit z and f [B,H,T] —
    the values before the boundary stores them as bf16."""
    xx = widen(x, dtype)
    WW = widen(Wx, dtype)
    bb = np.asarray(bias, dtype=np.float32).astype(np.float64)
    B, T, D = xx.shape
    H, R, D2 = WW.shape
    if D2 != D or R != 2 * K + V + 1 or bb.shape != (H,):
        raise ValueError("inconsistent shapes")
    # proj[b, h, t, r] = sum_d Wx[h, r, d] x[b, t, d]
    proj = np.matmul(xx[:, None, :, :], np.swapaxes(WW, -1, -2)[None])   # [B, H, T, R]
    z = proj[..., 2 * K + V] + bb[None, :, None]
    return {
        "k": proj[..., :K],
        "v": proj[..., K:K + V],
        "q": proj[..., K + V:2 * K + V],
        "z": z,
        "f": sigmoid_ref(z),
    }
