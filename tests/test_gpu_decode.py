"""GPU parity of the one-step (decoding) kernel, which every call with T = 1 on
the matrix-core path takes, against the fp64 oracle.

Covers: the decoding workload's shape at reduced batch, every K/V the kernel
takes, the state updated in place, empty sequences, the accumulate flag, a
null H0, and a decoding loop of many single-step calls chained through the
state (the split operand keeps it within the bar where a single bf16 operand
would drift). Bar as the other bf16 tests: 2e-2 normwise; over one step the
kernel is far inside it (the printed errors).
"""
import numpy as np
import pytest

from gpu_util import announce, nerr, to_device
from non_linear_matrix_amd.inputs import CONFIGS, SERVING, generate, scaled
from oracle import m2rnn_fwd_ref

pytestmark = pytest.mark.gpu

TOL = 2e-2
ONE_STEP_TOL = 2e-3   # a single step: one bf16-split product, fp32 elsewhere


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


def _step(d, algo="auto", **kw):
    import torch
    from non_linear_matrix_amd import m2rnn

    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo, **kw)
    torch.cuda.synchronize()
    return y, HT


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (32, 128), (64, 64), (32, 64), (128, 64)])
@pytest.mark.parametrize("algo", ["auto", "mfma", "mfma_split"])
def test_one_step_matches_the_oracle(K, V, algo):
    cfg = scaled(SERVING["D1"], B=37, H=3, K=K, V=V)
    announce(f"decode K={K} V={V} algo={algo}")
    x = generate(cfg, 21)
    y, HT = _step(to_device(x), algo)
    yr, HTr = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=cfg.dtype)
    ey, eh = nerr(y.cpu().numpy(), yr), nerr(HT.cpu().numpy(), HTr)
    print(f"y {ey:.2e} H_T {eh:.2e}", flush=True)
    assert ey <= ONE_STEP_TOL and eh <= ONE_STEP_TOL


def test_decoding_workload_sampled_in_place():
    """D1's full shape (512 sequences x 16 heads), state updated in place."""
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = SERVING["D1"]
    announce("decode D1 full size, in place")
    x = generate(cfg, 0)
    d = to_device(x)
    H0_before = d["H0"].clone()
    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], H_T=d["H0"])
    torch.cuda.synchronize()
    assert HT.data_ptr() == d["H0"].data_ptr()
    assert not torch.equal(HT, H0_before)
    rows = [0, 1, 255, 300, 511]
    sub = {key: x[key][rows] for key in ("k", "v", "q", "f", "H0")}
    yr, HTr = m2rnn_fwd_ref(sub["k"], sub["v"], sub["q"], sub["f"], x["W"], sub["H0"], dtype=cfg.dtype)
    assert nerr(y[rows].cpu().numpy(), yr) <= ONE_STEP_TOL
    assert nerr(HT[rows].cpu().numpy(), HTr) <= ONE_STEP_TOL


def test_empty_sequences_and_accumulate():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(SERVING["D1"], B=6, H=2)
    announce("decode: lengths 0/1, accumulate")
    x = generate(cfg, 22)
    d = to_device(x)
    lens = torch.tensor([1, 0, 1, 1, 0, 1], dtype=torch.int32, device="cuda")
    base = torch.full((cfg.B, cfg.H, 1, cfg.V), 0.5, device="cuda")
    y = base.clone()
    _, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y, seq_len=lens, accumulate_y=True)
    torch.cuda.synchronize()
    yr, HTr = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=cfg.dtype)
    for b in range(cfg.B):
        if lens[b] == 0:
            assert torch.equal(HT[b].cpu(), torch.from_numpy(x["H0"][b])), b
            assert torch.equal(y[b], base[b]), b
        else:
            assert nerr(HT[b].cpu().numpy(), HTr[b]) <= ONE_STEP_TOL, b
            assert nerr((y[b] - base[b]).cpu().numpy(), yr[b]) <= ONE_STEP_TOL, b


def test_zero_initial_state_and_no_final_state():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(SERVING["D1"], B=5, H=2, K=64, V=64, h0="zero")
    announce("decode: H0 = NULL, H_T = NULL")
    x = generate(cfg, 23)
    d = to_device(x)
    y = torch.empty((cfg.B, cfg.H, 1, cfg.V), device="cuda")
    lib = m2rnn.load()
    st = lib.m2rnn_fwd(d["k"].data_ptr(), d["v"].data_ptr(), d["q"].data_ptr(), d["f"].data_ptr(),
                       d["W"].data_ptr(), None, y.data_ptr(), None, cfg.B, cfg.H, 1, cfg.K, cfg.V,
                       m2rnn.DTYPES["bf16"], torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    yr, _ = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], None, dtype=cfg.dtype)
    assert nerr(y.cpu().numpy(), yr) <= ONE_STEP_TOL


@pytest.mark.parametrize("name", ["C3", "C5"])
def test_decoding_loop_tracks_the_full_sequence(name):
    """T single-step calls, the state carried in place, against the oracle over
    the whole sequence (the per-step inputs sliced from one draw)."""
    import torch
    from non_linear_matrix_amd import m2rnn

    T = 96
    cfg = scaled(CONFIGS[name], B=3, H=2, T=T)
    announce(f"decode loop {name} T={T}")
    x = generate(cfg, 24)
    d = to_device(x)
    state = d["H0"].clone() if d["H0"] is not None else torch.zeros((cfg.B, cfg.H, cfg.K, cfg.V), device="cuda")
    ys = []
    for t in range(T):
        sl = {key: d[key][:, :, t:t + 1].contiguous() for key in ("k", "v", "q", "f")}
        y, _ = m2rnn.fwd(sl["k"], sl["v"], sl["q"], sl["f"], d["W"], state, H_T=state)
        ys.append(y)
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=2).cpu().numpy()
    yr, HTr = m2rnn_fwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dtype=cfg.dtype)
    ey, eh = nerr(y, yr), nerr(state.cpu().numpy(), HTr)
    print(f"{name}: y {ey:.2e} H_T {eh:.2e}", flush=True)
    assert ey <= TOL and eh <= TOL


def test_plan_reports_the_decoding_kernel():
    from non_linear_matrix_amd import m2rnn

    p = m2rnn.get_plan(512, 16, 1, 128, 128, "bf16", "auto")
    assert p["clears_y"] == 0 and p["block"] == 256 and p["grid"] == 16 * 32
    q = m2rnn.get_plan(512, 16, 2, 128, 128, "bf16", "auto")
    assert q["grid"] == 512 * 16 * 2
