"""The oracle's pins are strong enough: each planted mistake fails at least one.

The mistakes are planted in a copy of the oracle's step loop written here (CPU
only); the real oracle is untouched. A mutant that every pin accepted would mean
the pins could not tell that mistake from the definition.
"""
import inspect

import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import widen


def make_mutant(kind):
    def fwd(k, v, q, f, W, H0=None, *, dtype, return_states=False, state_rounding=None):
        kk, vv, qq, ff, WW = (widen(a, dtype) for a in (k, v, q, f, W))
        B, H, T, K = kk.shape
        V = vv.shape[-1]
        S = np.zeros((B, H, K, V)) if H0 is None else np.asarray(H0).astype(np.float64)
        y = np.empty((B, H, T, V))
        states = np.empty((B, H, T, K, V))
        Wb = WW[None]
        for t in range(T):
            Wt = np.swapaxes(Wb, -1, -2) if kind == "W transposed" else Wb
            A = np.matmul(S, Wt)
            if kind == "no transition":
                A = 0 * A
            tv = max(t - 1, 0) if kind == "v one step late" else t
            outer = kk[:, :, t, :, None] * vv[:, :, tv, None, :]
            if kind == "no rank-1 write":
                outer = 0 * outer
            if kind == "rank-1 outside tanh":
                Z = np.tanh(A) + outer
            elif kind == "no tanh":
                Z = A + outer
            else:
                Z = np.tanh(A + outer)
            tf = max(t - 1, 0) if kind == "gate one step late" else t
            ft = ff[:, :, tf, None, None]
            S_prev = S
            if kind == "gate swapped":
                S = (1 - ft) * S + ft * Z
            elif kind == "no carry":
                S = (1 - ft) * Z
            else:
                S = ft * S + (1 - ft) * Z
            src = S_prev if kind == "readout of previous state" else S
            if kind == "readout scaled by gate":
                src = ft * src
            y[:, :, t, :] = np.matmul(qq[:, :, t, None, :], src)[:, :, 0, :]
            states[:, :, t] = S
        if kind == "H_T off by one step" and T > 1:
            S = states[:, :, T - 2]
        return (y, S, states) if return_states else (y, S)
    return fwd


KINDS = ["W transposed", "no transition", "no rank-1 write", "rank-1 outside tanh", "no tanh",
         "gate swapped", "no carry", "gate one step late", "v one step late",
         "readout of previous state", "readout scaled by gate", "H_T off by one step"]


def _pin_calls():
    calls = []
    for name, fn in sorted(vars(pins).items()):
        if not name.startswith("test_") or not callable(fn) or "diagnostic" in name:
            continue
        params = [p for p in inspect.signature(fn).parameters if p != "fwd"]
        marks = getattr(fn, "pytestmark", [])
        grid = [{}]
        for m in marks:
            if m.name == "parametrize":
                argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
                grid = [dict(g, **dict(zip(argnames, vals if len(argnames) > 1 else (vals,)))) for g in grid for vals in m.args[1]]
        for g in grid:
            if set(g) == set(params):
                calls.append((name, fn, g))
    return calls


def test_real_oracle_reproduces_itself_through_the_mutant_harness():
    """Sanity: the harness with no mutation passes every pin."""
    ok = make_mutant("none")
    for name, fn, g in _pin_calls():
        fn(**g, fwd=ok)


@pytest.mark.parametrize("kind", KINDS)
def test_every_planted_mistake_is_caught(kind):
    mutant = make_mutant(kind)
    caught = []
    for name, fn, g in _pin_calls():
        try:
            fn(**g, fwd=mutant)
        except AssertionError:
            caught.append(name)
    assert caught, f"no pin catches the mistake {kind!r}"
