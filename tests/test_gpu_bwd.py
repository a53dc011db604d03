"""GPU parity of the training path (m2rnn_fwd_save + m2rnn_bwd) against the fp64
gradient oracle on the same seeded inputs and output gradients.

Metric as the forward tests: per gradient, max|g - g_ref| / max|g_ref|. The
backward matrix products take bf16 operands (the saved state, dA), like the
forward's MFMA kernel, so the bar is the bf16 one, 2e-2.
"""
import time

import numpy as np
import pytest

from gpu_util import announce, nerr, to_device
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled
from oracle import m2rnn_bwd_ref

pytestmark = pytest.mark.gpu

TOL = 2e-2
GRADS = ("dk", "dv", "dq", "df", "dW", "dH0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


def _grads(cfg, seed, algo="auto", with_dHT=True):
    import torch
    from non_linear_matrix_amd import m2rnn

    x = generate(cfg, seed)
    rng = np.random.default_rng(seed + 77)
    dy = rng.standard_normal((cfg.B, cfg.H, cfg.T, cfg.V)).astype(np.float32)
    dHT = rng.standard_normal((cfg.B, cfg.H, cfg.K, cfg.V)).astype(np.float32) if with_dHT else None
    d = to_device(x)
    y, HT, saved = m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
    g = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, torch.from_numpy(dy).cuda(),
                  None if dHT is None else torch.from_numpy(dHT).cuda(), algo=algo)
    torch.cuda.synchronize()
    got = {key: g[key].cpu().numpy() for key in GRADS}
    got["y"], got["H_T"] = y.cpu().numpy(), HT.cpu().numpy()
    ref = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dHT, dtype=cfg.dtype)
    return got, ref


SHAPES = [
    ("C2", dict(B=2, H=2, T=20)),                    # K = V = 64, one workgroup per unit
    ("C3", dict(B=1, H=2, T=37)),                    # K = V = 128, two workgroups, ragged T
    ("C5", dict(B=2, H=1, T=16, K=32)),              # K = 32, V = 128, two-wave workgroups
    ("C3", dict(B=2, H=2, T=48, K=64, V=128)),
    ("C3", dict(B=2, H=1, T=17, K=128, V=64)),       # K = 128, V = 64
    ("C2", dict(B=1, H=3, T=33, K=32, V=64)),        # K = 32, V = 64
    ("C3", dict(B=3, H=2, T=1)),                     # a single step
    ("C5", dict(B=2, H=2, T=19)),                    # H0 = 0 (C5 starts from the zero state)
]


# "auto" takes the latency-oriented forward and reverse kernels on these few-tile
# shapes (T > 1); "mfma_split" the one-wave-per-tile ones
@pytest.mark.parametrize("algo", ["auto", "mfma_split"])
@pytest.mark.parametrize("name,shape", SHAPES)
def test_gradients_match_the_oracle(name, shape, algo):
    cfg = scaled(CONFIGS[name], **shape)
    announce(f"bwd {name} {shape} forward {algo}")
    got, ref = _grads(cfg, 31, algo=algo)
    errs = {key: nerr(got[key], ref[key]) for key in GRADS}
    errs["y"], errs["H_T"] = nerr(got["y"], ref["y"]), nerr(got["H_T"], ref["H_T"])
    print(" ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, f"{key}: {e:.3e}"


def test_without_final_state_gradient():
    cfg = scaled(CONFIGS["C2"], B=1, H=2, T=16)
    announce("bwd without dH_T")
    got, ref = _grads(cfg, 32, with_dHT=False)
    for key in GRADS:
        assert nerr(got[key], ref[key]) <= TOL, key


def test_without_initial_state_gradient():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=1, H=2, T=21)
    announce("bwd without dH0")
    x = generate(cfg, 35)
    d = to_device(x)
    dy = torch.randn((cfg.B, cfg.H, cfg.T, cfg.V), generator=torch.Generator().manual_seed(7)).cuda()
    _, _, saved = m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"])
    g0 = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy, want_dH0=False)
    g1 = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy)
    torch.cuda.synchronize()
    assert g0["dH0"] is None
    for key in ("dk", "dv", "dq", "df", "dW"):
        assert torch.equal(g0[key], g1[key]), key


def test_single_operand_forward_feeds_the_same_backward():
    cfg = scaled(CONFIGS["C3"], B=1, H=2, T=24)
    announce("bwd after the single-operand forward")
    got, ref = _grads(cfg, 33, algo="mfma")
    for key in GRADS:
        assert nerr(got[key], ref[key]) <= TOL, key


def test_the_two_reverse_kernels_agree():
    """Both reverse-time kernels on one saved buffer: the same per-element
    arithmetic, sums in other orders (dq and dk over column blocks, dv and df
    over row tiles, dA W^T over blocks), so the gradients agree to fp32
    summation order, amplified along the sequence."""
    import torch
    from non_linear_matrix_amd import m2rnn

    for cfg in (scaled(CONFIGS["C3"], B=2, H=2, T=40), scaled(CONFIGS["C2"], B=2, H=3, T=33, K=32)):
        announce(f"reverse kernels agree K={cfg.K} V={cfg.V} T={cfg.T}")
        x = generate(cfg, 36)
        d = to_device(x)
        dy = torch.randn((cfg.B, cfg.H, cfg.T, cfg.V), generator=torch.Generator().manual_seed(9)).cuda()
        dHT = torch.randn((cfg.B, cfg.H, cfg.K, cfg.V), generator=torch.Generator().manual_seed(10)).cuda()
        _, _, saved = m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo="mfma_split")
        g1 = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy, dHT, algo="mfma_split")
        g2 = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy, dHT, algo="mfma_long_split")
        torch.cuda.synchronize()
        for key in GRADS:
            a, b = g1[key].cpu().numpy(), g2[key].cpu().numpy()
            assert np.all(np.isfinite(b)), key
            assert nerr(b, a.astype(np.float64)) <= 1e-3, (key, nerr(b, a.astype(np.float64)))


def test_backward_is_deterministic():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=32)
    announce("bwd determinism")
    x = generate(cfg, 34)
    d = to_device(x)
    dy = torch.randn((cfg.B, cfg.H, cfg.T, cfg.V), generator=torch.Generator().manual_seed(5)).cuda()
    _, _, saved = m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"])
    g1 = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy)
    g2 = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy)
    torch.cuda.synchronize()
    for key in GRADS:
        assert torch.equal(g1[key], g2[key]), key


# (workload, heads compared: None = every head). C5's gradient oracle over all 32
# units takes several minutes of host time; four of its heads (8 units, among
# them the units the forward tests find most sensitive) stand in for it.
FULL = [("C2", None), ("C3", None), ("C4", None), ("C5", (0, 7, 12, 15))]


@pytest.mark.parametrize("name,heads", FULL, ids=[n for n, _ in FULL])
def test_full_size_every_unit(name, heads):
    """Full-size workloads in the launch configuration the training benchmark
    uses (AUTO: the split-operand forward and the reverse kernel it pairs with),
    every gradient of every (b, h) unit of the listed heads against the oracle;
    dW of a head sums over its batch rows."""
    import torch
    from gpu_util import bwd_oracle_all_units, unit_errors
    from non_linear_matrix_amd import m2rnn

    cfg = CONFIGS[name]
    hs = list(range(cfg.H)) if heads is None else list(heads)
    announce(f"bwd {name} full size, heads {'all' if heads is None else hs}")
    x = generate(cfg, 0)
    rng = np.random.default_rng(99)
    dy = rng.standard_normal((cfg.B, cfg.H, cfg.T, cfg.V), dtype=np.float32)
    d = to_device(x)
    y, HT, saved = m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"])
    g = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, torch.from_numpy(dy).cuda())
    torch.cuda.synchronize()
    got = {key: (g[key][hs] if key == "dW" else g[key][:, hs]).cpu().numpy() for key in GRADS}
    del saved, g
    xs = {key: (None if a is None else (a[hs] if key == "W" else a[:, hs])) for key, a in x.items()}
    t0 = time.time()
    ref = bwd_oracle_all_units(xs, dy[:, hs], cfg.dtype)
    announce(f"bwd oracle {name}: {cfg.B * len(hs)} units in {time.time() - t0:.1f}s")
    errs, worst = {}, {}
    for key, a in got.items():
        assert np.all(np.isfinite(a)), key
        errs[key] = nerr(a, ref[key])
        if key != "dW":
            e = unit_errors(a, ref[key])
            b, j = np.unravel_index(int(np.argmax(e)), e.shape)
            worst[key] = ((int(b), hs[j]), float(e[b, j]))
    print(f"{name} bwd every unit: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()) + " | worst unit "
          + " ".join(f"{k} {u} {e:.2e}" for k, (u, e) in worst.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, f"{key}: {e:.3e}"
