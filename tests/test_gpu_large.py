"""Index range: calls whose y, state or inputs hold more than 2^31 elements, so
that every offset computation past the 32-bit range is exercised.

A small seeded workload is generated once and tiled over a large batch and head
count on the device (every (b, h) unit is an independent computation, so a tiled
unit must equal its small original). Units near the end of the arrays, where the
offsets exceed 2^31 elements, are compared with the oracle run on the small
workload. Device memory: ~24 GB for the forward case, ~17 GB for the decoding
step.
"""
import numpy as np
import pytest

from gpu_util import announce, nerr, to_device
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled
from oracle import m2rnn_fwd_ref

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


def _tile(d, rb, rh):
    """The small workload's device tensors repeated rb times over the batch and rh
    times over the heads."""
    out = {}
    for key, t in d.items():
        if t is None:
            out[key] = None
        elif key == "W":
            out[key] = t.repeat(rh, 1, 1)
        else:
            out[key] = t.repeat(rb, rh, *([1] * (t.dim() - 2)))
    return out


@pytest.mark.parametrize("algo", ["auto", "mfma_long_split"])
def test_forward_past_2_31_elements(algo):
    import torch
    from non_linear_matrix_amd import m2rnn

    small = scaled(CONFIGS["C3"], B=4, H=4, K=32, V=128, T=65)
    x = generate(small, 71)
    rb, rh = 512, 32                      # B = 2048, H = 128
    B, H = small.B * rb, small.H * rh
    assert B * H * small.T * small.V > 2 ** 31
    announce(f"forward past 2^31 elements, algo={algo}, B={B} H={H} T={small.T} K={small.K} V={small.V}")
    d = _tile(to_device(x), rb, rh)
    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
    torch.cuda.synchronize()
    yr, HTr = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=small.dtype)
    for b, h in [(B - 1, H - 1), (B - 2, H - 3), (B // 2 + 5, H // 2 + 2), (0, 1)]:
        bs, hs = b % small.B, h % small.H
        ey = nerr(y[b, h].cpu().numpy(), yr[bs, hs])
        eh = nerr(HT[b, h].cpu().numpy(), HTr[bs, hs])
        print(f"unit ({b}, {h}) = small ({bs}, {hs}): y {ey:.2e} H_T {eh:.2e}", flush=True)
        assert ey <= TOL_BF16 and eh <= TOL_BF16, (b, h, ey, eh)
    del d, y, HT
    torch.cuda.empty_cache()


def test_decoding_step_past_2_31_state_elements():
    """T = 1, state updated in place, B H K V > 2^31."""
    import torch
    from non_linear_matrix_amd import m2rnn

    small = scaled(CONFIGS["C3"], B=1, H=4, K=32, V=128, T=1)
    x = generate(small, 72)
    rb, rh = 4097, 32                     # B = 4097, H = 128
    B, H = small.B * rb, small.H * rh
    assert B * H * small.K * small.V > 2 ** 31
    announce(f"decoding step past 2^31 state elements, B={B} H={H} K={small.K} V={small.V}")
    d = _tile(to_device(x), rb, rh)
    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], H_T=d["H0"])
    torch.cuda.synchronize()
    assert HT.data_ptr() == d["H0"].data_ptr()
    yr, HTr = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=small.dtype)
    for b, h in [(B - 1, H - 1), (B - 1, H - 2), (B // 2, H // 2 + 1), (0, 0)]:
        hs = h % small.H
        ey = nerr(y[b, h].cpu().numpy(), yr[0, hs])
        eh = nerr(HT[b, h].cpu().numpy(), HTr[0, hs])
        print(f"unit ({b}, {h}) = small (0, {hs}): y {ey:.2e} H_T {eh:.2e}", flush=True)
        assert ey <= 2e-3 and eh <= 2e-3, (b, h, ey, eh)
    del d, y, HT
    torch.cuda.empty_cache()
