"""Helpers shared by the GPU tests: device upload, sampled-unit oracle runs, error metric."""
from __future__ import annotations

import sys
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


def pick(arr: np.ndarray, units) -> np.ndarray:
    return np.stack([arr[b, h] for b, h in units])[None]
