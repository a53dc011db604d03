"""The backward pass with the library's own workspace (m2rnn_bwd_noalloc, for
callers that cannot allocate) against m2rnn_bwd_algo with a caller workspace:
the same kernels on the same inputs, so every gradient must agree bit for bit.
Two calls in a row, the second on a smaller shape (the array keeps the first
call's contents), for both reverse-kernel families."""
import numpy as np
import pytest

from gpu_util import announce, nerr, to_device
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled

pytestmark = pytest.mark.gpu

KEYS = ("dk", "dv", "dq", "df", "dW", "dH0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


@pytest.mark.parametrize("algo", ["mfma_split", "mfma_long_split"])
def test_noalloc_backward_matches_the_workspace_backward(algo):
    import torch
    from non_linear_matrix_amd import m2rnn
    from oracle import m2rnn_bwd_ref

    shapes = [dict(B=2, H=3, T=70, K=64, V=128), dict(B=1, H=2, T=33, K=32, V=64)]
    for i, shp in enumerate(shapes):
        cfg = scaled(CONFIGS["C3"], **shp)
        announce(f"no-alloc backward, call {i + 1}, {shp}, algo={algo}")
        assert m2rnn.bwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.K, cfg.V) <= 64 << 20
        x = generate(cfg, 90 + i)
        d = to_device(x)
        dy = torch.randn((cfg.B, cfg.H, cfg.T, cfg.V), generator=torch.Generator().manual_seed(7 + i)).cuda()
        dHT = torch.randn((cfg.B, cfg.H, cfg.K, cfg.V), generator=torch.Generator().manual_seed(17 + i)).cuda()
        _, _, saved = m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
        ref = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy, dHT, algo=algo)
        torch.cuda.synchronize()
        ref = {k: ref[k].clone() for k in KEYS}
        got = m2rnn.bwd_noalloc(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy, dHT, algo=algo)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], ref[key]), (i, key)
        # and both within the bf16 bar of the fp64 gradient oracle
        oref = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy.cpu().numpy(),
                             dHT.cpu().numpy(), dtype=cfg.dtype)
        for key in KEYS:
            assert nerr(got[key].cpu().numpy(), oref[key]) <= 2e-2, (i, key)

