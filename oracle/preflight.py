"""Sensitivity preflight for the five workloads (diagnostic; CPU only).

TEST INFRASTRUCTURE ONLY (it runs the oracle); nothing on the product path uses it.

For every (batch, head) unit of a workload (or the first `--units` of them), at
the full sequence length, it reports:
  (i)  how a 1e-9 perturbation of the initial state grows along the sequence:
       growth = max|H_T(H0 + d) - H_T(H0)| / 1e-9 per unit (a chaotic trajectory
       would make any rounding difference explode; a contracting one forgets it);
  (ii) the normwise error of the diagnostic runs that round the state to
       bfloat16, and to fp16, before every product with W (the oracle's
       `state_rounding` modes), against the exact run: an estimate of the error
       a single bf16- or fp16-operand matrix product adds on its own, per output
       tensor and for the worst unit.
Usage: python -m oracle.preflight [--units N] [C1 C2 ...]
"""
from __future__ import annotations

import argparse
import time

import numpy as np

from non_linear_matrix_amd.inputs import CONFIGS, generate
from .m2rnn_ref import m2rnn_fwd_ref


def _err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _unit_err(a, b):
    B, H = b.shape[:2]
    d = np.abs(a - b).reshape(B, H, -1).max(axis=2)
    return d / np.maximum(np.abs(b).reshape(B, H, -1).max(axis=2), 1e-300)


def sample_units(x, units):
    """Restrict an input dict to the listed (b, h) units (as a batch of 1 x n heads)."""
    out = {}
    for key in ("k", "v", "q", "f"):
        out[key] = np.stack([x[key][b, h] for b, h in units])[None]
    out["W"] = np.stack([x["W"][h] for _, h in units])
    out["H0"] = None if x["H0"] is None else np.stack([x["H0"][b, h] for b, h in units])[None]
    return out


def run(name, max_units=None, seed=0):
    cfg = CONFIGS[name]
    units = [(b, h) for b in range(cfg.B) for h in range(cfg.H)][:max_units]
    x = sample_units(generate(cfg, seed), units)
    t0 = time.time()
    y, HT = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=cfg.dtype)
    rng = np.random.default_rng(1234)
    base = np.zeros_like(HT) if x["H0"] is None else x["H0"].astype(np.float64)
    H0p = base + 1e-9 * rng.standard_normal(HT.shape)
    _, HTp = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], H0p, dtype=cfg.dtype)
    growth = np.abs(HTp - HT).reshape(len(units), -1).max(axis=1) / 1e-9
    line = (f"{name}: T={cfg.T} units={len(units)} | perturbation growth of H_T: max {growth.max():.3g} "
            f"median {np.median(growth):.3g}")
    if cfg.dtype == "bf16":
        for mode in ("bf16", "f16"):
            yr, HTr = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=cfg.dtype,
                                    state_rounding=mode)
            uy, uh = _unit_err(yr, y)[0], _unit_err(HTr, HT)[0]
            wy, wh = int(np.argmax(uy)), int(np.argmax(uh))
            line += (f" | {mode}-state diagnostic: y {_err(yr, y):.3e} H_T {_err(HTr, HT):.3e}; worst unit y "
                     f"{units[wy]} {uy[wy]:.3e}, H_T {units[wh]} {uh[wh]:.3e}")
    line += f" | max|y| {np.max(np.abs(y)):.3g} max|H_T| {np.max(np.abs(HT)):.3g} | {time.time() - t0:.1f}s"
    print(line, flush=True)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--units", type=int, default=None, help="first N units only (default: all)")
    ap.add_argument("names", nargs="*", default=["C1", "C2", "C3", "C4", "C5"])
    args = ap.parse_args()
    for n in args.names:
        run(n, args.units)
