"""Sensitivity preflight for the five workloads (diagnostic; CPU only).

For a few sampled (batch, head) units of each workload, at the full sequence
length, it reports:
  (i)  how a 1e-9 perturbation of the initial state grows along the sequence
       (a chaotic trajectory would make any rounding difference explode);
  (ii) the normwise error of the diagnostic run that rounds the state to
       bfloat16 before every product with W — an estimate of the error a
       bf16-operand matrix product adds on its own.
Usage: python -m oracle.preflight [C2 C3 ...]
"""
from __future__ import annotations

import sys
import time

import numpy as np

from non_linear_matrix_amd.inputs import CONFIGS, generate
from .m2rnn_ref import m2rnn_fwd_ref


def _err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def sample_units(x, units):
    """Restrict an input dict to the listed (b, h) units (as a batch of 1 x n heads)."""
    out = {}
    for key in ("k", "v", "q", "f"):
        out[key] = np.stack([x[key][b, h] for b, h in units])[None]
    out["W"] = np.stack([x["W"][h] for _, h in units])
    out["H0"] = None if x["H0"] is None else np.stack([x["H0"][b, h] for b, h in units])[None]
    return out


def run(name, units=((0, 0), (1, 1)), seed=0):
    cfg = CONFIGS[name]
    x = sample_units(generate(cfg, seed), [(b % cfg.B, h % cfg.H) for b, h in units])
    t0 = time.time()
    y, HT = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=cfg.dtype)
    rng = np.random.default_rng(1234)
    base = np.zeros_like(HT) if x["H0"] is None else x["H0"].astype(np.float64)
    H0p = base + 1e-9 * rng.standard_normal(HT.shape)
    yp, HTp = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], H0p, dtype=cfg.dtype)
    yr, HTr = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=cfg.dtype,
                            state_rounding="bf16" if cfg.dtype == "bf16" else None)
    growth_y = np.max(np.abs(yp - y)) / 1e-9
    growth_h = np.max(np.abs(HTp - HT)) / 1e-9
    print(f"{name}: T={cfg.T} units={len(units)} | perturbation growth y {growth_y:.3g} H_T {growth_h:.3g} | "
          f"bf16-state diag err y {_err(yr, y):.3e} H_T {_err(HTr, HT):.3e} | "
          f"max|y| {np.max(np.abs(y)):.3g} max|H_T| {np.max(np.abs(HT)):.3g} | {time.time() - t0:.1f}s",
          flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or ["C1", "C2", "C3", "C4", "C5"]):
        run(n)
