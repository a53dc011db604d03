"""High-precision brute-force evaluation of the M²RNN forward recurrence.

A pin for the fp64 oracle on tiny shapes: every operation is done in Python's
``decimal`` at 60 significant digits, with tanh built from an exp series (not
libm), and plain index loops (no numpy). The update is the state-update pair of
the gist.science technical summary (zh) §2.1; the readout is the y_t = H_t^T q_t
reading documented with the oracle.
"""
from __future__ import annotations

from decimal import Decimal, getcontext, localcontext
from typing import List, Optional, Sequence, Tuple

PREC = 60


def _exp(x: Decimal) -> Decimal:
    """e**x by argument halving + Taylor series."""
    with localcontext() as ctx:
        ctx.prec = PREC + 20
        n = 0
        y = x
        while abs(y) > Decimal("0.01"):
            y /= 2
            n += 1
        term = Decimal(1)
        s = Decimal(1)
        i = 1
        while True:
            term = term * y / i
            if abs(term) < Decimal(10) ** (-(PREC + 15)):
                break
            s += term
            i += 1
        for _ in range(n):
            s = s * s
        return +s


def tanh_dec(x: Decimal) -> Decimal:
    with localcontext() as ctx:
        ctx.prec = PREC + 10
        if x < 0:
            return -tanh_dec(-x)
        if x > 60:
            return Decimal(1)
        e = _exp(2 * x)
        return (e - 1) / (e + 1)


def fwd_decimal(
    k: Sequence, v: Sequence, q: Sequence, f: Sequence, W: Sequence, H0: Optional[Sequence] = None
) -> Tuple[List[List[Decimal]], List[List[Decimal]]]:
    """One unit. k, q: [T][K]; v: [T][V]; f: [T]; W: [V][V]; H0: [K][V] or None.

    Inputs are Python floats (converted exactly). Returns (y [T][V], H_T [K][V]).
    """
    getcontext().prec = PREC
    T = len(f)
    K = len(k[0])
    V = len(v[0])
    D = Decimal
    S = [[D(H0[i][j]) if H0 is not None else D(0) for j in range(V)] for i in range(K)]
    Wd = [[D(W[l][j]) for j in range(V)] for l in range(V)]
    ys = []
    for t in range(T):
        ft = D(f[t])
        new = [[D(0)] * V for _ in range(K)]
        for i in range(K):
            for j in range(V):
                acc = D(0)
                for l in range(V):
                    acc += S[i][l] * Wd[l][j]
                z = tanh_dec(acc + D(k[t][i]) * D(v[t][j]))
                new[i][j] = ft * S[i][j] + (1 - ft) * z
        S = new
        ys.append([sum((S[i][j] * D(q[t][i]) for i in range(K)), D(0)) for j in range(V)])
    return ys, S
