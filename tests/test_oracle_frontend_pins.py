"""Pins of the front-end oracle (oracle.m2rnn_frontend_ref) to things other than itself.

* one-hot inputs: with x_t = e_d the projections are column d of the weights, so
  every output is a stored weight, exactly; this fixes which rows feed k, v, q
  and the gate, and that the product runs over the model width;
* the logistic function: its closed-form values (sigma(0) = 1/2,
  sigma(ln 3) = 3/4), the symmetry sigma(z) + sigma(-z) = 1, scipy's expit (an
  independent implementation) and the extremes (no overflow);
* brute force on tiny inputs: exact sums (math.fsum) and math.exp per element;
* exact scaling: x -> 2x doubles k, v, q exactly;
* the planted-mistake check: plausible errors in a copy of the oracle are each
  caught by one of the pins above.
"""
import math

import numpy as np
import pytest

from non_linear_matrix_amd.inputs import CONFIGS, fp32_to_bf16_bits, generate_frontend, scaled
from oracle import m2rnn_frontend_ref, sigmoid_ref, widen

K, V, H, D = 3, 4, 2, 5
R = 2 * K + V + 1


def _small(seed=0, B=2, T=3):
    rng = np.random.default_rng(seed)
    x = fp32_to_bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32))
    Wx = fp32_to_bf16_bits(rng.standard_normal((H, R, D)).astype(np.float32))
    bias = rng.standard_normal(H).astype(np.float32)
    return x, Wx, bias


def _one_hot_check(fn):
    x, Wx, bias = _small(1, B=1, T=D)
    onehot = np.zeros((1, D, D), dtype=np.float32)
    for t in range(D):
        onehot[0, t, (3 * t + 1) % D] = 1.0
    xo = fp32_to_bf16_bits(onehot)
    out = fn(xo, Wx, bias, K=K, V=V)
    W = widen(Wx, "bf16")
    for t in range(D):
        d = (3 * t + 1) % D
        for h in range(H):
            assert np.array_equal(out["k"][0, h, t], W[h, :K, d])
            assert np.array_equal(out["v"][0, h, t], W[h, K:K + V, d])
            assert np.array_equal(out["q"][0, h, t], W[h, K + V:2 * K + V, d])
            assert out["z"][0, h, t] == W[h, 2 * K + V, d] + np.float64(bias[h])


def _brute_check(fn):
    x, Wx, bias = _small(2)
    out = fn(x, Wx, bias, K=K, V=V)
    xw, Ww = widen(x, "bf16"), widen(Wx, "bf16")
    B, T, _ = xw.shape
    for b in range(B):
        for h in range(H):
            for t in range(T):
                dots = [math.fsum(float(Ww[h, r, d]) * float(xw[b, t, d]) for d in range(D)) for r in range(R)]
                np.testing.assert_allclose(out["k"][b, h, t], dots[:K], rtol=1e-14, atol=1e-14)
                np.testing.assert_allclose(out["v"][b, h, t], dots[K:K + V], rtol=1e-14, atol=1e-14)
                np.testing.assert_allclose(out["q"][b, h, t], dots[K + V:2 * K + V], rtol=1e-14, atol=1e-14)
                z = dots[2 * K + V] + float(bias[h])
                assert abs(out["f"][b, h, t] - 1.0 / (1.0 + math.exp(-z))) <= 1e-15


def test_one_hot_inputs_select_weight_columns():
    _one_hot_check(m2rnn_frontend_ref)


def test_brute_force_tiny():
    _brute_check(m2rnn_frontend_ref)


def test_sigmoid_closed_forms_and_symmetry():
    assert sigmoid_ref(np.array([0.0]))[0] == 0.5
    assert abs(sigmoid_ref(np.array([math.log(3.0)]))[0] - 0.75) <= 1e-16
    assert abs(sigmoid_ref(np.array([-math.log(3.0)]))[0] - 0.25) <= 1e-16
    z = np.random.default_rng(3).standard_normal(1000) * 10
    np.testing.assert_allclose(sigmoid_ref(z) + sigmoid_ref(-z), 1.0, rtol=0, atol=5e-16)  # two roundings


def test_sigmoid_matches_scipy_and_has_no_overflow():
    special = pytest.importorskip("scipy.special")
    z = np.concatenate([np.linspace(-40, 40, 801), [-800.0, 800.0]])
    with np.errstate(over="raise", invalid="raise"):
        s = sigmoid_ref(z)
    np.testing.assert_allclose(s, special.expit(z), rtol=1e-15, atol=0)
    assert s[-1] == 1.0 and 0.0 <= s[-2] < 1e-300


def test_doubling_x_doubles_the_projections_exactly():
    x, Wx, bias = _small(4)
    x2 = fp32_to_bf16_bits(2.0 * widen(x, "bf16").astype(np.float32))
    a = m2rnn_frontend_ref(x, Wx, bias, K=K, V=V)
    b = m2rnn_frontend_ref(x2, Wx, bias, K=K, V=V)
    for key in ("k", "v", "q"):
        assert np.array_equal(b[key], 2.0 * a[key])


def test_generated_projections_have_the_configured_spread():
    cfg = scaled(CONFIGS["C3"], B=2, H=4, T=64)
    g = generate_frontend(cfg, 0)
    out = m2rnn_frontend_ref(g["x"], g["Wx"], g["bias"], K=cfg.K, V=cfg.V)
    for key in ("k", "v", "q"):
        assert 0.9 < float(np.std(out[key])) < 1.1, key
    assert np.allclose(g["bias"], [1.0, 5.0 / 3.0, 7.0 / 3.0, 3.0])
    assert np.all((out["f"] > 0) & (out["f"] < 1))


# ---- planted mistakes: each must fail one of the pins above

def _mutant(kind):
    def fn(x, Wx, bias, *, K, V, dtype="bf16"):
        xx, WW = widen(x, dtype), widen(Wx, dtype)
        bb = np.asarray(bias, dtype=np.float32).astype(np.float64)
        if kind == "bias reversed over heads":
            bb = bb[::-1]
        proj = np.matmul(xx[:, None], np.swapaxes(WW, -1, -2)[None])
        k, v, q = proj[..., :K], proj[..., K:K + V], proj[..., K + V:2 * K + V]
        if kind == "k and q swapped":
            k, q = q, k
        if kind == "v slice off by one":
            v = proj[..., K + 1:K + V + 1]
        z = proj[..., 2 * K + V] + (0.0 if kind == "bias dropped" else bb[None, :, None])
        if kind == "gate from the last v row":
            z = proj[..., K + V - 1] + bb[None, :, None]
        f = 1.0 / (1.0 + np.exp(z if kind == "sigmoid sign" else -z))
        if kind == "x rows mixed over time":
            k = np.roll(k, 1, axis=2)
        return {"k": k, "v": v, "q": q, "z": z, "f": f}
    return fn


MUTANTS = ["bias reversed over heads", "k and q swapped", "v slice off by one", "bias dropped",
           "gate from the last v row", "sigmoid sign", "x rows mixed over time"]


def test_the_mutant_harness_reproduces_the_oracle():
    _one_hot_check(_mutant("none"))
    _brute_check(_mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_every_planted_mistake_is_caught(kind):
    caught = 0
    for check in (_one_hot_check, _brute_check):
        try:
            check(_mutant(kind))
        except AssertionError:
            caught += 1
    assert caught > 0, kind
