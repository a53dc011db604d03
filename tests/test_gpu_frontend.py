"""GPU parity of the layer front-end (m2rnn_frontend) against the fp64 oracle.

Each output element is one fp32 dot product over the model width, rounded once
to bf16, so the bound is elementwise and derived from that arithmetic:

    |got - ref| <= 2^-8 |ref| + 2^-20 * sum_d |x_d w_d|

(half an ulp of bf16 is 2^-9 relative; the second term covers fp32 accumulation
over D <= 4096 terms with room to spare). The gate is a sigmoid of such a dot
product (slope <= 1/4) rounded to bf16: |got - ref| <= 2^-8 ref + 2^-20 * sum.
"""
import numpy as np
import pytest

from gpu_util import announce, nerr
from non_linear_matrix_amd.inputs import CONFIGS, fp32_to_bf16_bits, generate, generate_frontend, scaled
from oracle import m2rnn_frontend_ref, m2rnn_fwd_ref, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host_bf16(t):
    import torch
    return widen(t.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")


def _run(g, K, V):
    import torch
    from non_linear_matrix_amd import m2rnn

    out = m2rnn.frontend(_dev(g["x"]), _dev(g["Wx"]), _dev(g["bias"]), K=K, V=V)
    torch.cuda.synchronize()
    return {key: _host_bf16(out[key]) for key in ("k", "v", "q", "f")}, out


def _bound_check(got, ref, x, Wx, K, V):
    # sum_d |x_d w_d| per (b, h, t, r), the scale of the accumulation error
    absum = np.matmul(np.abs(widen(x, "bf16"))[:, None], np.abs(np.swapaxes(widen(Wx, "bf16"), -1, -2))[None])
    parts = {"k": absum[..., :K], "v": absum[..., K:K + V], "q": absum[..., K + V:2 * K + V],
             "f": absum[..., 2 * K + V]}
    for key in ("k", "v", "q", "f"):
        err = np.abs(got[key] - ref[key])
        lim = 2.0 ** -8 * np.abs(ref[key]) + 2.0 ** -20 * parts[key]
        worst = float(np.max(err - lim))
        assert worst <= 0.0, f"{key}: bound exceeded by {worst:.3e}"


SHAPES = [
    # (B, T, H, K, V, D): ragged in every tile dimension where it can be
    (2, 70, 3, 16, 32, 200),     # M = 140 (two row tiles), N = 3 x 65, D = 3 slices + 8
    (1, 5, 2, 128, 128, 256),    # K = V = 128, N = 2 x 385, M < one tile
    (3, 50, 2, 64, 64, 136),
    (2, 33, 4, 64, 128, 64),     # one k-slice exactly
    (1, 300, 1, 16, 16, 8),      # D = 8: one partial slice
]


@pytest.mark.parametrize("B,T,H,K,V,D", SHAPES)
def test_projections_and_gate_match_the_oracle(B, T, H, K, V, D):
    cfg = scaled(CONFIGS["C3"], B=B, T=T, H=H, K=K, V=V)
    announce(f"frontend B{B} T{T} H{H} K{K} V{V} D{D}")
    g = generate_frontend(cfg, 5, D=D)
    got, _ = _run(g, K, V)
    ref = m2rnn_frontend_ref(g["x"], g["Wx"], g["bias"], K=K, V=V)
    _bound_check(got, ref, g["x"], g["Wx"], K, V)
    print(" ".join(f"{key} {nerr(got[key], ref[key]):.2e}" for key in ("k", "v", "q", "f")), flush=True)


def test_full_size_sampled_tokens():
    """C3's full front-end (B=8, T=2048, D=2048, 16 heads): every output of a
    sample of tokens (b, t) against the oracle."""
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = CONFIGS["C3"]
    announce("frontend C3 full size, sampled tokens")
    g = generate_frontend(cfg, 0)
    out = m2rnn.frontend(_dev(g["x"]), _dev(g["Wx"]), _dev(g["bias"]), K=cfg.K, V=cfg.V)
    torch.cuda.synchronize()
    toks = [(0, 0), (0, 2047), (3, 1000), (7, 129), (5, 1), (7, 2047)]
    xs = np.stack([g["x"][b, t] for b, t in toks])[None]             # [1, n, D]
    ref = m2rnn_frontend_ref(xs, g["Wx"], g["bias"], K=cfg.K, V=cfg.V)
    got = {}
    for key in ("k", "v", "q", "f"):
        host = out[key]
        got[key] = np.stack([_host_bf16(host[b, :, t]) for b, t in toks], axis=1)[None]
    _bound_check(got, ref, xs, g["Wx"], cfg.K, cfg.V)


def test_feeds_the_recurrence():
    """Front-end then the recurrence on the GPU, against the oracle front-end
    (stored as bf16, the boundary's format) then the oracle recurrence."""
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=40)
    announce("frontend -> recurrence")
    g = generate_frontend(cfg, 6)
    rec = generate(cfg, 6)
    got, dev = _run(g, cfg.K, cfg.V)
    W, H0 = _dev(rec["W"]), _dev(rec["H0"])
    y, HT = m2rnn.fwd(dev["k"], dev["v"], dev["q"], dev["f"], W, H0)
    torch.cuda.synchronize()
    ref = m2rnn_frontend_ref(g["x"], g["Wx"], g["bias"], K=cfg.K, V=cfg.V)
    stored = {key: fp32_to_bf16_bits(ref[key].astype(np.float32)) for key in ("k", "v", "q", "f")}
    yr, HTr = m2rnn_fwd_ref(stored["k"], stored["v"], stored["q"], stored["f"], rec["W"], rec["H0"], dtype="bf16")
    assert nerr(y.cpu().numpy(), yr) <= 2e-2 and nerr(HT.cpu().numpy(), HTr) <= 2e-2


def test_frontend_is_deterministic():
    import torch

    cfg = scaled(CONFIGS["C3"], B=2, T=100, H=2)
    announce("frontend determinism")
    g = generate_frontend(cfg, 7, D=512)
    _, a = _run(g, cfg.K, cfg.V)
    _, b = _run(g, cfg.K, cfg.V)
    for key in ("k", "v", "q", "f"):
        assert torch.equal(a[key], b[key]), key
