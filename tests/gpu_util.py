"""Helpers shared by the GPU tests: device upload, oracle runs (sampled units, or
every unit of a full-size workload, cached per session), error metrics."""
from __future__ import annotations

import os
import sys
import time
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from oracle import m2rnn_fwd_ref


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def nerr(got: np.ndarray, ref: np.ndarray) -> float:
    """Normwise error max|got - ref| / max|ref| (the parity metric)."""
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got.astype(np.float64) - ref))) / max(den, 1e-300)


def to_device(x: Dict[str, Optional[np.ndarray]], device: str = "cuda"):
    import torch

    out = {}
    for key, a in x.items():
        if a is None:
            out[key] = None
        elif a.dtype == np.uint16:
            out[key] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        else:
            out[key] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out


def gpu_run(x, algo: str = "auto", **kw) -> Tuple[np.ndarray, np.ndarray]:
    import torch
    from non_linear_matrix_amd import m2rnn

    d = to_device(x)
    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), HT.cpu().numpy()


def sample_units(x, units: Sequence[Tuple[int, int]]):
    """Inputs of the listed (b, h) units, as one batch row of len(units) heads."""
    out = {}
    for key in ("k", "v", "q", "f"):
        out[key] = np.stack([x[key][b, h] for b, h in units])[None]
    out["W"] = np.stack([x["W"][h] for _, h in units])
    out["H0"] = None if x["H0"] is None else np.stack([x["H0"][b, h] for b, h in units])[None]
    return out


def oracle_units(x, dtype: str, units: Optional[List[Tuple[int, int]]] = None):
    """Oracle y, H_T for all units ([B,H,...]) or for the listed units ([1,n,...])."""
    if units is not None:
        x = sample_units(x, units)
    return m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=dtype)


def unit_errors(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-(b, h) normwise error max|got - ref| / max|ref| over each unit: [B, H]."""
    B, H = ref.shape[:2]
    d = np.abs(got.astype(np.float64) - ref).reshape(B, H, -1).max(axis=2)
    den = np.abs(ref).reshape(B, H, -1).max(axis=2)
    return d / np.maximum(den, 1e-300)


def worst_unit(got: np.ndarray, ref: np.ndarray) -> Tuple[Tuple[int, int], float]:
    e = unit_errors(got, ref)
    b, h = np.unravel_index(int(np.argmax(e)), e.shape)
    return (int(b), int(h)), float(e[b, h])


def oracle_all_units(x, dtype: str, max_threads: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    """The oracle on every unit of x ([B,H,...] results), the units split over
    host threads (numpy releases the GIL inside its products and large
    elementwise loops; BLAS threads are capped so the total stays within
    max_threads). Each unit is an independent computation, so the split changes
    nothing but the wall time."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    B, H = x["k"].shape[:2]
    units = [(b, h) for b in range(B) for h in range(H)]
    cpus = max(1, min(os.cpu_count() or 1, max_threads))
    n = max(1, min(cpus, len(units) // 8))
    if n == 1:
        return oracle_units(x, dtype)
    parts = [units[i::n] for i in range(n)]
    subs = [sample_units(x, p) for p in parts]
    run = lambda s: m2rnn_fwd_ref(s["k"], s["v"], s["q"], s["f"], s["W"], s["H0"], dtype=dtype)
    with threadpool_limits(limits=max(1, cpus // n), user_api="blas"):
        with ThreadPoolExecutor(max_workers=n) as pool:
            outs = list(pool.map(run, subs))
    y = np.empty((B, H) + outs[0][0].shape[2:], dtype=np.float64)
    HT = np.empty((B, H) + outs[0][1].shape[2:], dtype=np.float64)
    for p, (yp, HTp) in zip(parts, outs):
        for i, (b, h) in enumerate(p):
            y[b, h], HT[b, h] = yp[0, i], HTp[0, i]
    return y, HT


def bwd_oracle_all_units(x, dy, dtype: str, max_threads: int = 16, mem_budget: float = 48e9):
    """The gradient oracle on every (b, h) unit of x, the units split over host
    threads (as oracle_all_units; the thread count is also capped so the oracle's
    per-step state histories fit in mem_budget bytes). dW of a head is the sum of
    its batch rows' dW, added in batch order. Returns the oracle's dict with
    every tensor at full shape."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import m2rnn_bwd_ref

    B, H, T, K = x["k"].shape
    V = x["v"].shape[-1]
    units = [(b, h) for b in range(B) for h in range(H)]
    per_unit = 2.0 * (T + 1) * K * V * 8  # the states and tanh outputs the oracle keeps
    cpus = max(1, min(os.cpu_count() or 1, max_threads))
    n = max(1, min(cpus, len(units), int(mem_budget // per_unit)))

    done = [0]

    def one(u):
        b, h = u
        sub = {key: (None if a is None else (a[h:h + 1] if key == "W" else a[b:b + 1, h:h + 1]))
               for key, a in x.items()}
        out = m2rnn_bwd_ref(sub["k"], sub["v"], sub["q"], sub["f"], sub["W"], sub["H0"],
                            dy[b:b + 1, h:h + 1], dtype=dtype)
        done[0] += 1
        if done[0] % max(1, len(units) // 8) == 0:
            announce(f"gradient oracle: {done[0]} of {len(units)} units")
        return out

    with threadpool_limits(limits=max(1, cpus // n), user_api="blas"):
        with ThreadPoolExecutor(max_workers=n) as pool:
            outs = list(pool.map(one, units))
    ref = {}
    for key, a in outs[0].items():
        if key == "dW":
            ref[key] = np.zeros((H,) + a.shape[1:])
        else:
            ref[key] = np.empty((B, H) + a.shape[2:])
    for (b, h), o in zip(units, outs):  # batch rows of a head in order b = 0, 1, ...
        for key, a in o.items():
            if key == "dW":
                ref[key][h] += a[0]
            else:
                ref[key][b, h] = a[0, 0]
    return ref


_FULL: Dict[Tuple[str, int], tuple] = {}


def oracle_full(name: str, seed: int = 0):
    """(inputs, y_ref, H_T_ref) of a full-size named workload, every unit,
    computed once per test session."""
    from non_linear_matrix_amd.inputs import CONFIGS, generate

    key = (name, seed)
    if key not in _FULL:
        cfg = CONFIGS[name]
        t0 = time.time()
        x = generate(cfg, seed)
        yr, HTr = oracle_all_units(x, cfg.dtype)
        announce(f"oracle {name} seed {seed}: all {cfg.B * cfg.H} units in {time.time() - t0:.1f}s")
        _FULL[key] = (x, yr, HTr)
    return _FULL[key]


def full_parity(name: str, algo: str, tol: float) -> Tuple[float, float]:
    """Run `algo` on the full-size workload and compare every unit with the oracle:
    prints the normwise errors of y and H_T and the worst unit of each, and
    returns the two normwise errors."""
    x, yr, HTr = oracle_full(name)
    announce(f"{name} full size, algo={algo}, every unit")
    y, HT = gpu_run(x, algo=algo)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(HT)), (name, algo)
    ey, eh = nerr(y, yr), nerr(HT, HTr)
    uy, ey_u = worst_unit(y, yr)
    uh, eh_u = worst_unit(HT, HTr)
    print(f"{name} {algo}: err y {ey:.3e} H_T {eh:.3e} (bar {tol:g}) | worst unit y {uy} {ey_u:.3e}, "
          f"H_T {uh} {eh_u:.3e}", flush=True)
    return ey, eh
