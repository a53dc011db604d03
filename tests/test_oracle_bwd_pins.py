"""Pins of the gradient oracle (oracle.m2rnn_bwd_ref) to things other than itself.

* central finite differences of the forward oracle on every input element
  (tiny shapes, exact fp64 inputs): the definition of a derivative;
* torch autograd of a separate torch fp64 forward: an independent derivation of
  the same chain rule;
* the gate f = 1 closed form (the state never moves);
* the planted-mistake check: plausible errors in a copy of the backward pass
  (a transposed W, a lost tanh derivative, the wrong state in dq, ...) are each
  caught by the finite-difference pin.
"""
import numpy as np
import pytest

from oracle import m2rnn_bwd_ref, m2rnn_fwd_ref

RNG_SHAPES = [(1, 1, 1, 1, 3), (1, 2, 2, 3, 3), (2, 1, 3, 2, 4), (1, 1, 2, 2, 1)]


def _inputs(rng, B, H, K, V, T, f_lo=0.05, f_hi=0.95):
    k = rng.standard_normal((B, H, T, K))
    v = rng.standard_normal((B, H, T, V))
    q = rng.standard_normal((B, H, T, K))
    f = rng.uniform(f_lo, f_hi, (B, H, T))
    W = rng.standard_normal((H, V, V)) * 0.7
    H0 = rng.uniform(-0.5, 0.5, (B, H, K, V))
    dy = rng.standard_normal((B, H, T, V))
    dHT = rng.standard_normal((B, H, K, V))
    return dict(k=k, v=v, q=q, f=f, W=W, H0=H0), dy, dHT


def _loss(x, dy, dHT):
    y, HT = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype="f64")
    return float(np.sum(y * dy) + np.sum(HT * dHT))


def _fd_grads(x, dy, dHT, h=1e-6):
    out = {}
    for name, arr in x.items():
        g = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            g[idx] = (_loss(xp, dy, dHT) - _loss(xm, dy, dHT)) / (2 * h)
        out[name] = g
    return out


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


GRAD_OF = {"k": "dk", "v": "dv", "q": "dq", "f": "df", "W": "dW", "H0": "dH0"}


@pytest.mark.parametrize("B,H,K,V,T", RNG_SHAPES)
def test_every_gradient_matches_finite_differences(B, H, K, V, T, bwd=m2rnn_bwd_ref):
    rng = np.random.default_rng(7 + B + 3 * H + 5 * K + 7 * V + 11 * T)
    x, dy, dHT = _inputs(rng, B, H, K, V, T)
    g = bwd(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dHT, dtype="f64")
    fd = _fd_grads(x, dy, dHT)
    for name, key in GRAD_OF.items():
        assert _rel(g[key], fd[name]) <= 1e-7, f"{key}: {_rel(g[key], fd[name]):.3e}"


def test_outputs_match_the_forward_oracle():
    rng = np.random.default_rng(3)
    x, dy, dHT = _inputs(rng, 2, 2, 4, 5, 6)
    g = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dHT, dtype="f64")
    y, HT = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype="f64")
    assert np.array_equal(g["y"], y) and np.array_equal(g["H_T"], HT)


def test_autograd_of_an_independent_torch_forward():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    B, H, K, V, T = 2, 2, 5, 7, 6
    x, dy, dHT = _inputs(rng, B, H, K, V, T)
    tx = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True) for n, a in x.items()}
    S = tx["H0"]
    ys = []
    for t in range(T):
        A = S @ tx["W"][None] + tx["k"][:, :, t, :, None] * tx["v"][:, :, t, None, :]
        ft = tx["f"][:, :, t, None, None]
        S = ft * S + (1 - ft) * torch.tanh(A)
        ys.append((tx["q"][:, :, t, :, None] * S).sum(-2))
    loss = (torch.stack(ys, 2) * torch.tensor(dy)).sum() + (S * torch.tensor(dHT)).sum()
    loss.backward()
    g = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dHT, dtype="f64")
    for name, key in GRAD_OF.items():
        assert _rel(g[key], tx[name].grad.numpy()) <= 1e-12, key


def test_gate_one_closed_form():
    """f = 1: H_t = H0 for all t, so dH0 = dH_T + sum_t q_t dy_t^T, dW = dk = dv = 0,
    dq_t = H0 dy_t, and df_t = sum (H0 - Z_t) G_t with G_t = dH_T + sum_{s >= t} q_s dy_s^T."""
    rng = np.random.default_rng(9)
    B, H, K, V, T = 1, 2, 3, 4, 5
    x, dy, dHT = _inputs(rng, B, H, K, V, T)
    x["f"] = np.ones((B, H, T))
    g = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dHT, dtype="f64")
    outer = x["q"][..., :, None] * dy[..., None, :]          # [B,H,T,K,V]
    assert np.allclose(g["dH0"], dHT + outer.sum(2), rtol=0, atol=1e-12)
    assert not np.any(g["dW"]) and not np.any(g["dk"]) and not np.any(g["dv"])
    assert np.allclose(g["dq"], np.einsum("bhkv,bhtv->bhtk", x["H0"], dy), rtol=0, atol=1e-12)
    for t in range(T):
        Z = np.tanh(x["H0"] @ x["W"][None] + x["k"][:, :, t, :, None] * x["v"][:, :, t, None, :])
        Gt = dHT + outer[:, :, t:].sum(2)
        assert np.allclose(g["df"][:, :, t], ((x["H0"] - Z) * Gt).sum((-2, -1)), rtol=0, atol=1e-11)


def test_bf16_storage_is_widened_exactly():
    from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled

    cfg = scaled(CONFIGS["C3"], B=1, H=2, K=4, V=6, T=5)
    x = generate(cfg, 4)
    rng = np.random.default_rng(4)
    dy = rng.standard_normal((1, 2, 5, 6))
    g16 = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dtype="bf16")
    from oracle import widen
    w = {n: widen(x[n], "bf16") for n in ("k", "v", "q", "f", "W")}
    g64 = m2rnn_bwd_ref(w["k"], w["v"], w["q"], w["f"], w["W"], x["H0"].astype(np.float64), dy, dtype="f64")
    for key in ("dk", "dv", "dq", "df", "dW", "dH0"):
        assert np.array_equal(g16[key], g64[key]), key


# ---- planted mistakes: each must be caught by the finite-difference pin

def _mutant(kind):
    def bwd(k, v, q, f, W, H0, dy, dH_T, *, dtype):
        B, H, T, K = k.shape
        V = v.shape[-1]
        S = np.empty((T + 1, B, H, K, V))
        Zs = np.empty((T, B, H, K, V))
        S[0] = H0
        for t in range(T):
            A = np.matmul(S[t], W[None]) + k[:, :, t, :, None] * v[:, :, t, None, :]
            Zs[t] = np.tanh(A)
            ft = f[:, :, t, None, None]
            S[t + 1] = ft * S[t] + (1 - ft) * Zs[t]
        G = dH_T.copy()
        out = {"dk": np.empty((B, H, T, K)), "dq": np.empty((B, H, T, K)), "dv": np.empty((B, H, T, V)),
               "df": np.empty((B, H, T)), "dW": np.zeros((H, V, V))}
        Wm = W if kind == "W not transposed" else np.swapaxes(W, -1, -2)
        for t in range(T - 1, -1, -1):
            if kind != "readout gradient dropped":
                G = G + q[:, :, t, :, None] * dy[:, :, t, None, :]
            Sq = S[t] if kind == "dq from the previous state" else S[t + 1]
            out["dq"][:, :, t] = np.matmul(Sq, dy[:, :, t, :, None])[..., 0]
            ft = f[:, :, t, None, None]
            dZ = (ft if kind == "gate swapped" else 1 - ft) * G
            out["df"][:, :, t] = np.sum(((Zs[t] - S[t]) if kind == "df sign" else (S[t] - Zs[t])) * G, axis=(-2, -1))
            dA = dZ if kind == "no tanh derivative" else dZ * (1 - Zs[t] ** 2)
            out["dk"][:, :, t] = np.matmul(dA, v[:, :, t, :, None])[..., 0]
            dAv = dA if kind == "dv not transposed" else np.swapaxes(dA, -1, -2)
            out["dv"][:, :, t] = np.matmul(dAv, k[:, :, t, :, None])[..., 0]
            Sw = S[t + 1] if kind == "dW from the new state" else S[t]
            out["dW"] += np.sum(np.matmul(np.swapaxes(Sw, -1, -2), dA), axis=0)
            G = (G if kind == "no carry" else ft * G) + np.matmul(dA, Wm[None])
        out["dH0"] = G
        return out
    return bwd


MUTANTS = ["W not transposed", "readout gradient dropped", "dq from the previous state", "gate swapped",
           "df sign", "no tanh derivative", "dv not transposed", "dW from the new state", "no carry"]


def test_the_mutant_harness_reproduces_the_oracle():
    rng = np.random.default_rng(21)
    x, dy, dHT = _inputs(rng, 1, 2, 3, 3, 4)
    good = _mutant("none")(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dHT, dtype="f64")
    ref = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dHT, dtype="f64")
    for key in ("dk", "dv", "dq", "df", "dW", "dH0"):
        assert np.allclose(good[key], ref[key], rtol=0, atol=1e-12), key


@pytest.mark.parametrize("kind", MUTANTS)
def test_every_planted_mistake_is_caught(kind):
    # square states, so that a transposition mistake still has valid shapes
    with pytest.raises(AssertionError):
        for shape in [(1, 2, 2, 2, 3), (2, 1, 3, 3, 4)]:
            test_every_gradient_matches_finite_differences(*shape, bwd=_mutant(kind))
