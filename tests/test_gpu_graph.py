"""HIP graph capture of the library's calls (through torch.cuda.CUDAGraph, which
captures the calls' launches on its capture stream): the path allocates nothing
and clears its buffers with kernels, so a captured forward, decoding step,
front-end or training step replays to the eager result. Each graph is replayed
several times with eager work and synchronisations in between, and every replay
is checked against the eager result, bit for bit.
"""
import numpy as np
import pytest

from gpu_util import announce, to_device
from non_linear_matrix_amd.inputs import CONFIGS, SERVING, generate, generate_frontend, scaled

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


def _replay_check(fn, outs, eager, close=()):
    """Capture fn (writing into outs), replay it, compare each replay with eager
    (bit for bit; to rounding for the outputs listed in close, sums of atomic
    adds)."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):       # warm-up outside the capture
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            if i in close:
                assert (o - e).abs().max().item() <= 1e-6 * e.abs().max().item(), f"replay {r}, output {i}"
            else:
                assert torch.equal(o, e), f"replay {r}, output {i}"


@pytest.mark.parametrize("algo", ["mfma", "mfma_split", "mfma_f16"])
def test_forward_replays(algo):
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=40)   # two workgroups per unit: y is cleared by a kernel
    announce(f"graph forward {algo}")
    d = to_device(generate(cfg, 51))
    y_e, HT_e = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
    torch.cuda.synchronize()
    y = torch.empty_like(y_e)
    HT = torch.empty_like(HT_e)
    _replay_check(lambda: m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y, H_T=HT, algo=algo),
                  [y, HT], [y_e, HT_e])


def test_decoding_step_replays():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(SERVING["D1"], B=64, H=4)
    announce("graph decoding step")
    d = to_device(generate(cfg, 52))
    y_e, HT_e = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"])
    torch.cuda.synchronize()
    y = torch.empty_like(y_e)
    HT = torch.empty_like(HT_e)
    _replay_check(lambda: m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y, H_T=HT),
                  [y, HT], [y_e, HT_e])


def test_frontend_replays():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=50)
    announce("graph front-end")
    g = generate_frontend(cfg, 53, D=256)
    dev = {}
    for key, a in g.items():
        if a.dtype == np.uint16:
            dev[key] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        else:
            dev[key] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    e = m2rnn.frontend(dev["x"], dev["Wx"], dev["bias"], K=cfg.K, V=cfg.V)
    torch.cuda.synchronize()
    out = {key: torch.empty_like(t) for key, t in e.items()}
    keys = ("k", "v", "q", "f")

    def fn():
        m2rnn.frontend(dev["x"], dev["Wx"], dev["bias"], K=cfg.K, V=cfg.V, out=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    for r in range(REPLAYS):
        for key in keys:
            out[key].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key in keys:
            assert torch.equal(out[key], e[key]), (key, r)


@pytest.mark.parametrize("algo", ["mfma_split", "mfma_long_split"])
def test_training_step_replays(algo):
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=48)
    announce(f"graph training step (recompute mode), forward {algo}")
    d = to_device(generate(cfg, 54))
    dy = torch.randn((cfg.B, cfg.H, cfg.T, cfg.V), generator=torch.Generator().manual_seed(8)).cuda()
    y_e, HT_e, ck_e = m2rnn.fwd_ckpt(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], segment=16, algo=algo)
    g_e = m2rnn.bwd_recompute(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], ck_e, dy, segment=16, algo=algo)
    torch.cuda.synchronize()
    keys = ("dk", "dv", "dq", "df", "dW", "dH0")
    y, HT, ck = torch.empty_like(y_e), torch.empty_like(HT_e), torch.empty_like(ck_e)
    out = {key: torch.empty_like(g_e[key]) for key in keys}
    ws = torch.empty_like(g_e["workspace"])

    def fn():
        m2rnn.fwd_ckpt(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], segment=16, ckpt=ck, y=y, H_T=HT, algo=algo)
        m2rnn.bwd_recompute(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], ck, dy, segment=16, out=out,
                            workspace=ws, algo=algo)

    _replay_check(fn, [y, HT, ck] + [out[key] for key in keys], [y_e, HT_e, ck_e] + [g_e[key] for key in keys],
                  close=(0,) if algo == "mfma_long_split" else ())
