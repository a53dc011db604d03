"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a 60-digit
brute force, a closed form, a special case that reduces to a library routine,
an invariant, or an exact relation between two oracle runs. Together they are
chosen so that a dropped term, a swapped gate, a transposed W or a readout over
the wrong axis fails at least one of them.

Definition pinned: the state-update pair of the gist.science technical summary
of M²RNN (zh) §2.1 (same equations in the ja summary §2.1),
    Z_t = tanh(H_{t-1} W + k_t v_t^T),  H_t = f_t H_{t-1} + (1 - f_t) Z_t,
and the readout reading y_t = H_t^T q_t.
"""
import math

import numpy as np
import pytest

from decimal_ref import fwd_decimal
from oracle import m2rnn_fwd_ref, round_to_bf16, round_to_f16
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled


def _rand_inputs(rng, B, H, T, K, V, f_lo=0.0, f_hi=1.0, h0_scale=0.5, w_scale=None):
    """fp32 inputs (so the oracle's exact widening is the identity on them)."""
    w_scale = (1.0 / math.sqrt(V)) if w_scale is None else w_scale
    k = rng.standard_normal((B, H, T, K)).astype(np.float32)
    v = rng.standard_normal((B, H, T, V)).astype(np.float32)
    q = rng.standard_normal((B, H, T, K)).astype(np.float32)
    f = rng.uniform(f_lo, f_hi, (B, H, T)).astype(np.float32)
    W = (rng.standard_normal((H, V, V)) * w_scale).astype(np.float32)
    H0 = rng.uniform(-h0_scale, h0_scale, (B, H, K, V)).astype(np.float32)
    return k, v, q, f, W, H0


FWD = m2rnn_fwd_ref


def _nrm(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("K,V,T", [(1, 1, 6), (2, 3, 5), (3, 2, 4), (3, 3, 3), (1, 3, 6), (2, 2, 6)])
def test_decimal_brute_force(K, V, T, fwd=FWD):
    """P1: fp64 oracle vs a 60-digit brute force with its own series tanh."""
    rng = np.random.default_rng(100 + 10 * K + V)
    k, v, q, f, W, H0 = _rand_inputs(rng, 1, 1, T, K, V, w_scale=0.9)
    y, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    yd, Sd = fwd_decimal(k[0, 0].tolist(), v[0, 0].tolist(), q[0, 0].tolist(), f[0, 0].tolist(),
                         W[0].tolist(), H0[0, 0].tolist())
    yd = np.array([[float(x) for x in row] for row in yd])
    Sd = np.array([[float(x) for x in row] for row in Sd])
    assert _nrm(y[0, 0], yd) <= 1e-13
    assert _nrm(HT[0, 0], Sd) <= 1e-13


def test_gate_one_freezes_state(fwd=FWD):
    """P2: f = 1 keeps H_t = H_0 exactly; with q = e_i the readout is row i of H_0."""
    rng = np.random.default_rng(1)
    B, H, T, K, V = 2, 3, 7, 5, 6
    k, v, q, f, W, H0 = _rand_inputs(rng, B, H, T, K, V)
    f[:] = 1.0
    i = 3
    q[:] = 0.0
    q[..., i] = 1.0
    y, HT, states = fwd(k, v, q, f, W, H0, dtype="f32", return_states=True)
    h0 = H0.astype(np.float64)
    assert np.array_equal(HT, h0)
    assert np.array_equal(states, np.broadcast_to(h0[:, :, None], states.shape))
    assert np.array_equal(y, np.broadcast_to(h0[:, :, None, i, :], y.shape))


def test_gate_zero_without_transition_is_tanh_of_outer_product(fwd=FWD):
    """P3: f = 0 and W = 0 give H_t = tanh(k_t v_t^T) at every step."""
    rng = np.random.default_rng(2)
    B, H, T, K, V = 2, 2, 5, 4, 7
    k, v, q, f, W, H0 = _rand_inputs(rng, B, H, T, K, V)
    f[:] = 0.0
    W[:] = 0.0
    _, _, states = fwd(k, v, q, f, W, H0, dtype="f32", return_states=True)
    kk, vv = k.astype(np.float64), v.astype(np.float64)
    expect = np.tanh(kk[..., :, None] * vv[..., None, :])
    assert np.allclose(states, expect, rtol=0, atol=1e-15)


def test_zero_transition_closed_form(fwd=FWD):
    """P4: W = 0 turns the update into a gated average of tanh(k_s v_s^T):
    H_T = (prod_s f_s) H_0 + sum_s (1 - f_s) (prod_{r>s} f_r) tanh(k_s v_s^T)."""
    rng = np.random.default_rng(3)
    B, H, T, K, V = 2, 2, 9, 3, 4
    k, v, q, f, W, H0 = _rand_inputs(rng, B, H, T, K, V)
    W[:] = 0.0
    _, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    ff = f.astype(np.float64)
    kk, vv = k.astype(np.float64), v.astype(np.float64)
    expect = np.prod(ff, axis=2)[..., None, None] * H0.astype(np.float64)
    for s in range(T):
        tail = np.prod(ff[:, :, s + 1:], axis=2) if s + 1 < T else np.ones((B, H))
        expect = expect + ((1 - ff[:, :, s]) * tail)[..., None, None] * np.tanh(
            kk[:, :, s, :, None] * vv[:, :, s, None, :])
    assert _nrm(HT, expect) <= 1e-12


def test_scalar_case_is_leaky_tanh_rnn(fwd=FWD):
    """P5: K = V = 1 is the scalar leaky tanh RNN h <- f h + (1-f) tanh(w h + k v)."""
    rng = np.random.default_rng(4)
    T = 40
    k, v, q, f, W, H0 = _rand_inputs(rng, 1, 1, T, 1, 1, w_scale=1.3)
    y, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    h = float(H0[0, 0, 0, 0])
    w = float(W[0, 0, 0])
    for t in range(T):
        ft = float(f[0, 0, t])
        h = ft * h + (1 - ft) * math.tanh(w * h + float(k[0, 0, t, 0]) * float(v[0, 0, t, 0]))
        assert abs(y[0, 0, t, 0] - h * float(q[0, 0, t, 0])) <= 1e-15 * max(1.0, abs(h))
    assert abs(HT[0, 0, 0, 0] - h) <= 1e-15


def test_transition_acts_on_the_value_axis_from_the_right(fwd=FWD):
    """Orientation pin: W with one non-zero entry W[a, b] = w, f = 0, H_0 = 0.
    (H W)[i, j] = H[i, a] w if j == b else 0, so after two steps
    H_2[i, b] = tanh(w tanh(k1_i v1_a) + k2_i v2_b), other columns tanh(k2_i v2_j)."""
    rng = np.random.default_rng(5)
    K, V, a, b, w = 4, 5, 1, 3, 1.7
    k, v, q, f, W, H0 = _rand_inputs(rng, 1, 1, 2, K, V)
    W[:] = 0.0
    W[0, a, b] = w
    f[:] = 0.0
    _, HT = fwd(k, v, q, f, W, None, dtype="f32")
    w32 = float(np.float32(w))
    for i in range(K):
        for j in range(V):
            k1, k2 = float(k[0, 0, 0, i]), float(k[0, 0, 1, i])
            pre = k2 * float(v[0, 0, 1, j])
            if j == b:
                pre += w32 * math.tanh(k1 * float(v[0, 0, 0, a]))
            assert abs(HT[0, 0, i, j] - math.tanh(pre)) <= 1e-15


def test_readout_reduces_over_the_key_axis(fwd=FWD):
    """Readout pin: with q_t = e_i the readout y_t is row i of the post-update H_t."""
    rng = np.random.default_rng(6)
    B, H, T, K, V = 1, 2, 6, 5, 3
    k, v, q, f, W, H0 = _rand_inputs(rng, B, H, T, K, V)
    q[:] = 0.0
    rows = rng.integers(0, K, size=T)
    for t in range(T):
        q[:, :, t, rows[t]] = 1.0
    y, _, states = fwd(k, v, q, f, W, H0, dtype="f32", return_states=True)
    for t in range(T):
        assert np.array_equal(y[:, :, t], states[:, :, t, rows[t], :])


def test_row_separability(fwd=FWD):
    """Rows of H evolve independently (the update mixes the value axis only), so a
    K-row run equals K one-row runs; a K = 1 run is a vector tanh RNN."""
    rng = np.random.default_rng(7)
    B, H, T, K, V = 1, 2, 12, 6, 5
    k, v, q, f, W, H0 = _rand_inputs(rng, B, H, T, K, V)
    _, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    for i in range(K):
        _, HTi = fwd(k[..., i:i + 1], v, q[..., i:i + 1], f, W, H0[:, :, i:i + 1, :], dtype="f32")
        assert np.allclose(HTi[:, :, 0, :], HT[:, :, i, :], rtol=0, atol=1e-14)


@pytest.mark.parametrize("h0_scale", [0.5, 3.0])
def test_convexity_bound(h0_scale, fwd=FWD):
    """P7: f in [0, 1] and |tanh| <= 1 make H_t a convex mix, so
    max|H_t| <= max(max|H_0|, 1), and |y_t[j]| <= ||q_t||_1 max(max|H_0|, 1)."""
    rng = np.random.default_rng(8)
    B, H, T, K, V = 2, 2, 30, 6, 7
    k, v, q, f, W, H0 = _rand_inputs(rng, B, H, T, K, V, h0_scale=h0_scale, w_scale=2.0)
    y, _, states = fwd(k, v, q, f, W, H0, dtype="f32", return_states=True)
    bound = np.maximum(np.max(np.abs(H0.astype(np.float64)), axis=(2, 3)), 1.0)
    assert np.all(np.max(np.abs(states), axis=(3, 4)) <= bound[:, :, None] * (1 + 1e-15))
    q1 = np.sum(np.abs(q.astype(np.float64)), axis=3)
    assert np.all(np.max(np.abs(y), axis=3) <= q1 * bound[:, :, None] * (1 + 1e-14))


def test_odd_symmetry(fwd=FWD):
    """P8: tanh is odd, so (H_0, k) -> (-H_0, -k) maps (H_t, y_t) -> (-H_t, -y_t)."""
    rng = np.random.default_rng(9)
    k, v, q, f, W, H0 = _rand_inputs(rng, 2, 2, 10, 4, 6)
    y, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    yn, HTn = fwd(-k, v, q, f, W, -H0, dtype="f32")
    assert np.allclose(yn, -y, rtol=0, atol=1e-15)
    assert np.allclose(HTn, -HT, rtol=0, atol=1e-15)


def test_key_axis_permutation_equivariance(fwd=FWD):
    """P8: permuting the key axis (rows of H_0, entries of k and q) permutes the rows of
    H_T and leaves y unchanged."""
    rng = np.random.default_rng(10)
    k, v, q, f, W, H0 = _rand_inputs(rng, 1, 2, 10, 6, 5)
    perm = rng.permutation(6)
    y, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    yp, HTp = fwd(k[..., perm], v, q[..., perm], f, W, H0[:, :, perm, :], dtype="f32")
    assert np.allclose(HTp, HT[:, :, perm, :], rtol=0, atol=1e-14)
    assert np.allclose(yp, y, rtol=0, atol=1e-13)


def test_value_axis_permutation_equivariance(fwd=FWD):
    """P8: permuting the value axis (columns of H_0, entries of v, and W -> P^T W P)
    permutes the columns of H_T and of y."""
    rng = np.random.default_rng(11)
    k, v, q, f, W, H0 = _rand_inputs(rng, 1, 2, 10, 4, 6)
    perm = rng.permutation(6)
    y, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    Wp = W[:, perm][:, :, perm]
    yp, HTp = fwd(k, v[..., perm], q, f, Wp, H0[..., perm], dtype="f32")
    assert np.allclose(HTp, HT[..., perm], rtol=0, atol=1e-14)
    assert np.allclose(yp, y[..., perm], rtol=0, atol=1e-13)


def test_readout_is_linear_in_q_and_state_ignores_q(fwd=FWD):
    rng = np.random.default_rng(12)
    k, v, q, f, W, H0 = _rand_inputs(rng, 2, 2, 8, 5, 4)
    # quarter-integers: q + 2 q2 is exact in fp32 storage
    q = (rng.integers(-8, 9, q.shape) / 4).astype(np.float32)
    q2 = (rng.integers(-8, 9, q.shape) / 4).astype(np.float32)
    y1, HT1 = fwd(k, v, q, f, W, H0, dtype="f32")
    y2, HT2 = fwd(k, v, q2, f, W, H0, dtype="f32")
    q3 = (q + 2 * q2).astype(np.float32)
    y3, HT3 = fwd(k, v, q3, f, W, H0, dtype="f32")
    assert np.array_equal(HT1, HT2) and np.array_equal(HT1, HT3)
    assert np.allclose(y3, y1 + 2 * y2, rtol=0, atol=1e-13)


def test_units_are_independent_and_w_is_per_head(fwd=FWD):
    """Batch/head units share nothing but their head's W (parallel over batch x head:
    gist.science zh §2.2, forward-pass bullet)."""
    rng = np.random.default_rng(13)
    k, v, q, f, W, H0 = _rand_inputs(rng, 2, 3, 6, 4, 5)
    y, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    k2 = k.copy(); k2[1, 2] += 1.0
    y2, HT2 = fwd(k2, v, q, f, W, H0, dtype="f32")
    mask = np.ones((2, 3), bool); mask[1, 2] = False
    assert np.array_equal(y2[mask], y[mask]) and np.array_equal(HT2[mask], HT[mask])
    assert not np.array_equal(HT2[1, 2], HT[1, 2])
    W2 = W.copy(); W2[1] *= 0.5
    y3, HT3 = fwd(k, v, q, f, W2, H0, dtype="f32")
    assert np.array_equal(HT3[:, [0, 2]], HT[:, [0, 2]])
    assert not np.array_equal(HT3[:, 1], HT[:, 1])
    # batch rows of the same head with identical inputs give identical outputs
    kb, vb, qb, fb, H0b = (a.copy() for a in (k, v, q, f, H0))
    for a in (kb, vb, qb, fb, H0b):
        a[1] = a[0]
    y4, HT4 = fwd(kb, vb, qb, fb, W, H0b, dtype="f32")
    assert np.array_equal(HT4[0], HT4[1]) and np.array_equal(y4[0], y4[1])


def test_chunked_continuation_is_exact(fwd=FWD):
    """Resuming from the returned state continues the same trajectory bit for bit."""
    rng = np.random.default_rng(14)
    k, v, q, f, W, H0 = _rand_inputs(rng, 2, 2, 13, 4, 6)
    y, HT = fwd(k, v, q, f, W, H0, dtype="f32")
    ya, HTa = fwd(k[:, :, :5], v[:, :, :5], q[:, :, :5], f[:, :, :5], W, H0, dtype="f32")
    yb, HTb = fwd(k[:, :, 5:], v[:, :, 5:], q[:, :, 5:], f[:, :, 5:], W, HTa, dtype="f32")
    assert np.array_equal(np.concatenate([ya, yb], axis=2), y)
    assert np.array_equal(HTb, HT)


def test_bf16_inputs_are_widened_exactly(fwd=FWD):
    """bf16 storage: the oracle's value is the exact bf16 value (here: small integers
    and powers of two, exact in bf16, give the same result as fp32 storage)."""
    rng = np.random.default_rng(15)
    B, H, T, K, V = 1, 1, 4, 3, 4
    k = rng.integers(-3, 4, (B, H, T, K)).astype(np.float32)
    v = rng.integers(-3, 4, (B, H, T, V)).astype(np.float32) * 0.25
    q = rng.integers(-3, 4, (B, H, T, K)).astype(np.float32)
    f = np.full((B, H, T), 0.75, np.float32)
    W = rng.integers(-2, 3, (H, V, V)).astype(np.float32) * 0.125
    from non_linear_matrix_amd.inputs import fp32_to_bf16_bits
    a = fwd(k, v, q, f, W, None, dtype="f32")
    b = fwd(*(fp32_to_bf16_bits(x) for x in (k, v, q, f, W)), None, dtype="bf16")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bf16_state_rounding_diagnostic_stays_close(fwd=FWD):
    """The diagnostic bf16-state variant is a perturbation of the definition, not a
    different method: on a small bf16 workload it stays within the bf16 tolerance."""
    cfg = scaled(CONFIGS["C2"], B=1, H=2, T=64)
    x = generate(cfg, seed=0)
    y, HT = fwd(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype="bf16")
    yr, HTr = fwd(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype="bf16",
                            state_rounding="bf16")
    assert 0 < _nrm(yr, y) < 2e-2 and 0 < _nrm(HTr, HT) < 2e-2
    r = round_to_bf16(np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5]))
    assert list(r) == [1.0, 1.0 + 2.0 ** -6, -2.5]


def test_f16_state_rounding_diagnostic(fwd=FWD):
    """The fp16-state variant: closer to the definition than the bf16 one (2^-12
    against 2^-9 relative rounding per step), and its rounding is IEEE binary16's
    round to nearest even: ties to the even neighbour, subnormals down to 2^-24,
    overflow past 65504 + 16 to infinity."""
    cfg = scaled(CONFIGS["C2"], B=1, H=2, T=64)
    x = generate(cfg, seed=0)
    y, HT = fwd(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype="bf16")
    yb, HTb = fwd(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype="bf16", state_rounding="bf16")
    yh, HTh = fwd(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype="bf16", state_rounding="f16")
    assert 0 < _nrm(yh, y) < _nrm(yb, y) and 0 < _nrm(HTh, HT) < _nrm(HTb, HT)
    r = round_to_f16(np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -2.5, 65519.0, 65520.0,
                               2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14 * (1 + 2.0 ** -10)]))
    assert list(r[:4]) == [1.0, 1.0 + 2.0 ** -9, -2.5, 65504.0]
    assert np.isinf(r[4]) and r[5] == 0.0 and r[6] == 2.0 ** -24 and r[7] == 2.0 ** -14 * (1 + 2.0 ** -10)
