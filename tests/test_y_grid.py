"""The arithmetic behind the latency-oriented kernels' order-independent y sum,
checked in IEEE fp32 on the host (numpy float32 has the device's round-to-nearest
-even addition).

Each of a unit's row tiles adds its partial readout p_r = sum over its rows of
H_t[i][j] q_t[i] into y. Every partial is first rounded to the grid of spacing
2^(E - 23), where 2^E > 1.0625 ||q_t||_1 M_t and M_t bounds |H_t| (the gated
update is a convex combination of the previous state and a tanh, so |H_t| <=
max(1, max |H0|) and decays toward 1 with the gates). Every partial sum over a
subset of tiles is bounded by the same quantity, so it is a multiple of the
spacing below 2^(E + 1): representable exactly, and the result cannot depend on
the order of the adds.
"""
import itertools

import numpy as np


def _grid(p: np.ndarray, bound: np.float32) -> np.ndarray:
    e = int(np.frexp(np.float32(bound * np.float32(1.0625)))[1])
    return np.ldexp(np.rint(np.ldexp(p, 23 - e)), e - 23).astype(np.float32), e


def _sum32(vals) -> np.float32:
    acc = np.float32(0.0)
    for v in vals:
        acc = np.float32(acc + np.float32(v))
    return acc


def test_grid_sums_do_not_depend_on_the_order():
    rng = np.random.default_rng(0)
    for trial in range(300):
        n = int(rng.integers(2, 9))                       # row tiles of a unit (K/16)
        rows = 16
        q = rng.standard_normal((n, rows)).astype(np.float32) * np.float32(rng.choice([1.0, 1 / 8, 1e-3]))
        m = np.float32(max(1.0, abs(rng.standard_normal()) * rng.choice([1.0, 30.0])))
        # a state within the bound, the partials as the tiles would form them
        H = (rng.uniform(-1, 1, (n, rows)) * m).astype(np.float32)
        p = np.array([_sum32(H[r] * q[r]) for r in range(n)], dtype=np.float32)
        qn = _sum32(np.abs(q).ravel())
        g, e = _grid(p, np.float32(qn * m))
        sums = {float(_sum32(g[list(perm)])) for perm in itertools.permutations(range(n))} if n <= 6 else \
            {float(_sum32(g[rng.permutation(n)])) for _ in range(200)}
        assert len(sums) == 1, (trial, sums)
        exact = float(np.sum(p.astype(np.float64)))
        assert abs(next(iter(sums)) - exact) <= n * 2.0 ** (e - 24) + 1e-30, trial


def test_plain_fp32_sums_can_depend_on_the_order():
    """Without the grid the same partials give order-dependent sums (the reason
    for it): a case where the fp32 result of three adds changes with the order."""
    a, b, c = np.float32(1.0), np.float32(2.0 ** -24), np.float32(2.0 ** -24)
    assert _sum32([a, b, c]) != _sum32([b, c, a])
    g, _ = _grid(np.array([a, b, c], dtype=np.float32), np.float32(1.5))
    assert _sum32(g) == _sum32(g[::-1])


def test_state_bound_covers_the_update():
    """M_t = f_t M_{t-1} + 1 - f_t bounds |H_t| for H_t = f H_{t-1} + (1 - f) tanh(.);
    it never grows (M >= 1), so the bound at a 16-step chunk's start covers the
    chunk, and after the chunk it is 1 + (f_0 ... f_15)(M - 1), the per-chunk
    update the kernel makes (in fp32, the product in its DPP-row order)."""
    rng = np.random.default_rng(1)
    for _ in range(50):
        H = rng.uniform(-3, 3, 32)
        M = np.float32(max(1.0, float(np.max(np.abs(H)))))
        for _c in range(20):
            f = (1 / (1 + np.exp(-rng.normal(2, 1, 16)))).astype(np.float32)
            for t in range(16):
                H = f[t] * H + (1 - f[t]) * np.tanh(rng.normal(0, 3, 32))
                assert np.max(np.abs(H)) <= M * 1.0625
            x = f.copy()  # the butterfly order of the DPP row product
            for perm in ([1, 0, 3, 2], [2, 3, 0, 1]):
                x = (x * x.reshape(-1, 4)[:, perm].reshape(-1)).astype(np.float32)
            x = (x * x.reshape(2, 8)[:, ::-1].reshape(-1)).astype(np.float32)
            x = (x * x[::-1]).astype(np.float32)
            assert np.all(x == x[0])
            M = np.float32(np.float32(x[0]) * np.float32(M - np.float32(1.0)) + np.float32(1.0))
            assert np.max(np.abs(H)) <= M * 1.0625
