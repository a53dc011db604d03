"""Seeded synthetic inputs for the M²RNN forward recurrence.

This module only draws random numbers and encodes them in the storage formats
the library consumes (IEEE fp32, or bfloat16 bit patterns held in uint16). It
holds none of the recurrence's arithmetic, so both the fp64 oracle and the HIP
path can be fed from it.

Workloads (shapes and distributions) are the five named configurations of the
forward recurrence; their shapes follow the matrix-valued state of the method
(state ``H_t`` is K x V, ``W`` is V x V, ``k_t`` has K entries, ``v_t`` has V
entries, the gate ``f_t`` is one scalar in [0, 1] per (batch, head, step)) as
described in the gist.science technical summary of "M²RNN: Non-Linear RNNs with
Matrix-Valued States for Scalable Language Modeling", §2.1.

Draw order and rounding (fixed here so that a seed names one exact input set):
  * ``numpy.random.default_rng(seed)``; every draw is fp64;
  * order: W, k, v, q, gate logit, H0;
  * fp64 -> fp32 by IEEE round-to-nearest-even (numpy ``astype``), then for
    bf16 workloads fp32 -> bf16 by round-to-nearest-even on the bit pattern;
  * H0 is always stored as fp32 (the state is fp32 at the boundary).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Config",
    "CONFIGS",
    "SERVING",
    "ragged_lengths",
    "fp32_to_bf16_bits",
    "bf16_bits_to_fp32",
    "generate",
    "scaled",
    "frontend_width",
    "frontend_rows",
    "generate_frontend",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload of the forward recurrence."""

    name: str
    dtype: str            # "f32" or "bf16": storage type of k, v, q, f, W
    B: int
    H: int
    K: int
    V: int
    T: int
    qkv_scale: str        # "1" -> k, v, q ~ N(0, 1); "rsqrtK" -> N(0, 1) / sqrt(K)
    gate_mu: float        # f = sigmoid(N(gate_mu, 1))
    h0: str               # "zero" or "uniform" (U(-0.5, 0.5))
    w_std: str = "rsqrtV"  # W ~ N(0, 1/V), one V x V matrix per head

    @property
    def units(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads. C3/C4 take "the same distributions as config 1", read
# 1-based: k, v, q ~ N(0, 1) unscaled and f = sigmoid(N(0, 1) + 2), with a
# per-head W and H0 ~ U(-0.5, 0.5).
CONFIGS: Dict[str, Config] = {
    "C1": Config("C1", "f32", 1, 1, 16, 16, 64, "1", 2.0, "zero"),
    "C2": Config("C2", "bf16", 4, 8, 64, 64, 512, "rsqrtK", 2.0, "zero"),
    "C3": Config("C3", "bf16", 8, 16, 128, 128, 2048, "1", 2.0, "uniform"),
    "C4": Config("C4", "bf16", 1, 32, 128, 128, 8192, "1", 2.0, "uniform"),
    "C5": Config("C5", "bf16", 2, 16, 64, 128, 32768, "rsqrtK", 3.0, "zero"),
}


# Serving-side workloads of the same recurrence, measured but not among the five
# parity configurations: D1 is one decoding step (T = 1) for 512 sequences of 16
# heads with the state carried in place; R1 is C3's shape as a ragged batch whose
# lengths come from ``ragged_lengths``.
SERVING: Dict[str, Config] = {
    "D1": Config("D1", "bf16", 512, 16, 128, 128, 1, "1", 2.0, "uniform"),
    "R1": Config("R1", "bf16", 8, 16, 128, 128, 2048, "1", 2.0, "uniform"),
}


def ragged_lengths(B: int, T: int, seed: int = 0) -> np.ndarray:
    """Per-sequence lengths, uniform in [T/4, T], int32 (own generator stream)."""
    rng = np.random.default_rng(seed + 1_000_003)
    return rng.integers(max(T // 4, 1), T + 1, size=B).astype(np.int32)


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return fp32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def scaled(cfg: Config, **shape) -> Config:
    """Same distributions as ``cfg`` with some of B, H, K, V, T replaced."""
    return cfg.with_(**shape)


def generate(cfg: Config, seed: int = 0, *, qkv_scale: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Draw one input set for ``cfg``.

    Returns a dict with ``k`` [B,H,T,K], ``v`` [B,H,T,V], ``q`` [B,H,T,K],
    ``f`` [B,H,T], ``W`` [H,V,V] in the config's storage type (fp32 arrays, or
    uint16 bfloat16 bit patterns) and ``H0`` [B,H,K,V] fp32 (or ``None`` when
    the config starts from the zero state).
    """
    B, H, K, V, T = cfg.B, cfg.H, cfg.K, cfg.V, cfg.T
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((H, V, V)) * (1.0 / math.sqrt(V))
    scale = 1.0
    mode = qkv_scale if qkv_scale is not None else cfg.qkv_scale
    if mode == "rsqrtK":
        scale = 1.0 / math.sqrt(K)
    elif mode != "1":
        raise ValueError(f"unknown qkv_scale {mode!r}")
    out: Dict[str, np.ndarray] = {}
    out["W"] = _store(W, cfg.dtype)
    del W
    for name, last in (("k", K), ("v", V), ("q", K)):
        a = rng.standard_normal((B, H, T, last))
        if scale != 1.0:
            a *= scale
        out[name] = _store(a, cfg.dtype)
        del a
    logit = rng.standard_normal((B, H, T)) + cfg.gate_mu
    out["f"] = _store(1.0 / (1.0 + np.exp(-logit)), cfg.dtype)
    if cfg.h0 == "uniform":
        out["H0"] = rng.uniform(-0.5, 0.5, size=(B, H, K, V)).astype(np.float32)
    elif cfg.h0 == "zero":
        out["H0"] = None
    else:
        raise ValueError(f"unknown h0 {cfg.h0!r}")
    return out


# ---- inputs of the layer front-end (the projections of x_t that produce k, v,
# q and the gate logit). The pages give no model width or weight scale; the
# width is taken as D = H V (the layer's value width) and the weights are drawn
# so that the projections have the same distributions as the configuration's
# k, v, q and gate logit: x ~ N(0, 1); the k, v, q rows ~ N(0, s^2 / D) with s
# the configuration's k/v/q scale; the gate row ~ N(0, 1 / D); one gate bias per
# head, spread evenly over [gate_mu - 1, gate_mu + 1] so that the heads start
# with different decay rates.

def frontend_width(cfg: Config) -> int:
    return cfg.H * cfg.V


def frontend_rows(cfg: Config) -> int:
    """Weight rows per head: K (k), V (v), K (q) and 1 (gate logit), in that order."""
    return 2 * cfg.K + cfg.V + 1


def generate_frontend(cfg: Config, seed: int = 0, D: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw x [B,T,D] and Wx [H, 2K+V+1, D] (bfloat16 bit patterns, uint16) and
    the gate bias [H] (fp32), from their own generator stream (seed + 2_000_003)."""
    B, H, K, V, T = cfg.B, cfg.H, cfg.K, cfg.V, cfg.T
    D = frontend_width(cfg) if D is None else D
    rng = np.random.default_rng(seed + 2_000_003)
    s = 1.0 / math.sqrt(K) if cfg.qkv_scale == "rsqrtK" else 1.0
    Wx = rng.standard_normal((H, frontend_rows(cfg), D)) * (1.0 / math.sqrt(D))
    Wx[:, :2 * K + V] *= s
    out = {"Wx": fp32_to_bf16_bits(Wx.astype(np.float32))}
    del Wx
    out["bias"] = (cfg.gate_mu + (np.linspace(-1.0, 1.0, H) if H > 1 else np.zeros(1))).astype(np.float32)
    x = np.empty((B, T, D), dtype=np.uint16)
    for b in range(B):  # row by row, so that full-size draws stay small in fp64
        x[b] = fp32_to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    out["x"] = x
    return out
