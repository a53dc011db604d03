"""GPU parity of the latency-oriented forward (algos "mfma_long",
"mfma_long_split") against the fp64 oracle.

Bars as the other bf16 tests (2e-2 normwise). The kernel does the same per-step
arithmetic as the multi-step kernel, so beyond the oracle: its H_T matches the
multi-step kernel's closely, is bit-identical between runs, and y (summed over
the row tiles with atomic adds) matches the multi-step kernel's to rounding.
"""
import numpy as np
import pytest

from gpu_util import announce, full_parity, gpu_run, nerr, oracle_units, to_device
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


SHAPES = [(K, V) for K in (16, 32, 48, 64, 128) for V in (64, 128)]


@pytest.mark.parametrize("T", [15, 16, 17, 37])
@pytest.mark.parametrize("K,V", SHAPES)
def test_shapes_and_ragged_lengths(K, V, T):
    cfg = scaled(CONFIGS["C3"], B=2, H=2, K=K, V=V, T=T)
    announce(f"long K={K} V={V} T={T}")
    x = generate(cfg, 61)
    yr, HTr = oracle_units(x, cfg.dtype)
    for algo in ("mfma_long_split", "mfma_long"):
        y, HT = gpu_run(x, algo=algo)
        ey, eh = nerr(y, yr), nerr(HT, HTr)
        assert ey <= TOL and eh <= TOL, (algo, ey, eh)


FULL = [("C2", "mfma_long_split"), ("C4", "mfma_long"), ("C4", "mfma_long_split"), ("C5", "mfma_long_split")]


@pytest.mark.parametrize("name,algo", FULL)
def test_full_size_configs(name, algo):
    """The small-batch workloads this kernel is for (AUTO's choice there), at full
    size, every unit against the oracle."""
    ey, eh = full_parity(name, algo, TOL)
    assert ey <= TOL and eh <= TOL
    if algo.endswith("split"):
        # ~16 significant bits in the operand (measured at most 1.1e-4, C2 H_T):
        # a lost low half would show long before the 2e-2 bar
        assert ey <= 1e-3 and eh <= 1e-3


@pytest.mark.parametrize("split", [False, True])
def test_agrees_with_the_multi_step_kernel(split):
    cfg = scaled(CONFIGS["C3"], B=2, H=3, T=70)
    announce(f"long vs multi-step, split={split}")
    x = generate(cfg, 62)
    y0, HT0 = gpu_run(x, algo="mfma_split" if split else "mfma")
    y1, HT1 = gpu_run(x, algo="mfma_long_split" if split else "mfma_long")
    # The same arithmetic per step, but the operand blocks are added in another
    # order, so the fp32 accumulators differ in their last bits; with a single bf16
    # operand that can flip the rounding of a state element (2^-9 relative) and the
    # trajectories part at that level, while the split operand keeps ~2^-17. Both
    # readouts take the state rounded to bf16, so y can differ by such a flip in
    # either variant (bar 2^-8).
    assert nerr(HT1, HT0) <= (1e-4 if split else 4e-3)
    assert nerr(y1, y0) <= 2.0 ** -8


def test_final_state_is_bitwise_repeatable():
    import torch

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=40)
    announce("long repeatability")
    x = generate(cfg, 63)
    y0, HT0 = gpu_run(x, algo="mfma_long_split")
    y1, HT1 = gpu_run(x, algo="mfma_long_split")
    assert np.array_equal(HT0, HT1)
    assert np.array_equal(y0, y1)  # grid-rounded row-tile sums: order-independent


@pytest.mark.parametrize("algo", ["mfma_long_split", "mfma_long_f16"])
def test_ragged_lengths_and_accumulate(algo):
    import torch
    from non_linear_matrix_amd import m2rnn
    from oracle import m2rnn_fwd_ref

    T = 37
    lens = [37, 0, 1, 16, 17, 30]
    cfg = scaled(CONFIGS["C3"], B=len(lens), H=2, T=T, K=64)
    announce(f"long varlen lens={lens} {algo}")
    x = generate(cfg, 64)
    d = to_device(x)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    base = torch.full((cfg.B, cfg.H, T, cfg.V), 0.25, device="cuda")
    y = base.clone()
    _, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y, seq_len=sl, algo=algo,
                      accumulate_y=True)
    torch.cuda.synchronize()
    yd = (y - base).cpu().numpy()
    HT = HT.cpu().numpy()
    for b, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(HT[b], x["H0"][b]) and not np.any(yd[b])
            continue
        sub = {key: x[key][b:b + 1, :, :n] for key in ("k", "v", "q", "f")}
        yr, HTr = m2rnn_fwd_ref(sub["k"], sub["v"], sub["q"], sub["f"], x["W"], x["H0"][b:b + 1], dtype=cfg.dtype)
        assert nerr(yd[b:b + 1, :, :n], yr) <= TOL and nerr(HT[b:b + 1], HTr) <= TOL, b
        assert not np.any(yd[b, :, n:]), b


def test_auto_takes_the_long_kernel_and_is_repeatable():
    """AUTO on a small-batch shape is the long kernel with the fp16 operand, with
    or without the deterministic flag: its row tiles' readouts go onto a common
    grid, so y is bit for bit the same from run to run. With the flag and
    accumulation the call leaves the long kernel (several row tiles would add
    into the caller's y)."""
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C5"], B=1, H=2, T=100)
    announce("AUTO / deterministic flag")
    x = generate(cfg, 65)
    yA, HA = gpu_run(x, algo="auto")
    yL, HL = gpu_run(x, algo="mfma_long_f16")
    assert np.array_equal(HA, HL) and np.array_equal(yA, yL)
    yD1, HD1 = gpu_run(x, algo="auto", deterministic=True)
    yD2, HD2 = gpu_run(x, algo="auto", deterministic=True)
    assert np.array_equal(yD1, yA) and np.array_equal(HD1, HA)
    assert np.array_equal(yD1, yD2) and np.array_equal(HD1, HD2)
    # accumulating under the flag: the multi-step kernel (one workgroup at K = 64)
    d = to_device(x)
    y0 = torch.zeros((1, 2, cfg.T, cfg.V), dtype=torch.float32, device="cuda")
    m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y0, accumulate_y=True, deterministic=True)
    torch.cuda.synchronize()
    yS, HS = gpu_run(x, algo="mfma_f16")
    assert np.array_equal(y0.cpu().numpy(), yS)
    # a single step under the flag: the decoding kernel, which has no atomics
    one = scaled(cfg, T=1)
    x1 = generate(one, 66)
    y1, H1 = gpu_run(x1, algo="mfma_long_split", deterministic=True)
    y2, H2 = gpu_run(x1, algo="mfma_long_split", deterministic=True)
    assert np.array_equal(y1, y2) and np.array_equal(H1, H2)


@pytest.mark.parametrize("K", [16, 48, 128])
def test_repeatable_with_a_large_initial_state(K):
    """The y grid's state bound starts at max |H0| when that exceeds 1 and decays
    with the gates: with H0 ~ U(-40, 40) y is still the same bit for bit from run
    to run and within the bar of the oracle (K = 16: one row tile, K = 48: three)."""
    cfg = scaled(CONFIGS["C5"], B=1, H=3, K=K, T=90)
    announce(f"large H0, K={K}")
    x = generate(cfg, 68)
    x["H0"] = (np.random.default_rng(69).uniform(-40, 40, (1, 3, K, cfg.V))).astype(np.float32)
    y1, H1 = gpu_run(x, algo="mfma_long_split")
    y2, H2 = gpu_run(x, algo="mfma_long_split")
    assert np.array_equal(y1, y2) and np.array_equal(H1, H2)
    yr, HTr = oracle_units(x, "bf16")
    assert nerr(y1, yr) <= TOL and nerr(H1, HTr) <= TOL


@pytest.mark.parametrize("name", ["C2", "C4", "C5"])
def test_default_forward_is_bitwise_repeatable(name):
    """The library's default forward (AUTO: the long kernel with the fp16 operand
    on these workloads) at full size gives the same y and H_T bit for bit on
    every run, although a unit's K/16 row tiles add into y in whatever order they
    finish."""
    from non_linear_matrix_amd import m2rnn
    cfg = CONFIGS[name]
    assert m2rnn.pick_algo(cfg.B, cfg.H, cfg.T, cfg.K, cfg.V, cfg.dtype) == "mfma_long_f16"
    announce(f"{name} full size, default forward, repeatability")
    x = generate(cfg, 0)
    y1, H1 = gpu_run(x)
    for _ in range(3):
        y2, H2 = gpu_run(x)
        assert np.array_equal(y1, y2) and np.array_equal(H1, H2)


@pytest.mark.parametrize("algo", ["mfma_long_split", "mfma_long_f16"])
def test_graph_replays(algo):
    """Captured in a HIP graph (y cleared by a fill kernel): every replay gives
    the eager H_T bit for bit and y to rounding."""
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=1, H=2, K=64, T=40)
    announce(f"long kernel graph replay, {algo}")
    d = to_device(generate(cfg, 67))
    y_e, HT_e = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
    torch.cuda.synchronize()
    y, HT = torch.empty_like(y_e), torch.empty_like(HT_e)
    fn = lambda: m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y, H_T=HT, algo=algo)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for r in range(3):
        y.fill_(float("nan"))
        HT.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(HT, HT_e), r
        assert (y - y_e).abs().max().item() <= 1e-6 * y_e.abs().max().item(), r


@pytest.mark.parametrize("split", [True, False])
def test_training_forward_feeds_the_backward(split):
    """The saving forward on the latency-oriented kernel writes the multi-step
    kernel's saved layout: the backward takes either, the gradients agree to the
    fp32 summation order of the states (and both match the oracle)."""
    import torch
    from non_linear_matrix_amd import m2rnn
    from oracle import m2rnn_bwd_ref

    cfg = scaled(CONFIGS["C3"], B=2, H=2, K=64, T=45)
    announce(f"long saving forward, split={split}")
    x = generate(cfg, 68)
    d = to_device(x)
    dy = torch.randn((cfg.B, cfg.H, cfg.T, cfg.V), generator=torch.Generator().manual_seed(8)).cuda()
    grads, outs = [], []
    for algo in (("mfma_long_split", "mfma_split") if split else ("mfma_long", "mfma")):
        y, HT, saved = m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
        grads.append(m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dy))
        outs.append((y, HT))
    torch.cuda.synchronize()
    assert nerr(outs[0][1].cpu().numpy(), outs[1][1].cpu().numpy().astype(np.float64)) <= (1e-4 if split else 4e-3)
    assert nerr(outs[0][0].cpu().numpy(), outs[1][0].cpu().numpy().astype(np.float64)) <= 2.0 ** -8
    ref = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy.cpu().numpy(), dtype=cfg.dtype)
    for key in ("dk", "dv", "dq", "df", "dW", "dH0"):
        a, b = grads[0][key].cpu().numpy(), grads[1][key].cpu().numpy()
        assert nerr(a, b.astype(np.float64)) <= (1e-3 if split else 1e-2), key
        assert nerr(a, ref[key]) <= TOL, key


def test_recompute_mode_on_the_long_kernel():
    """Checkpointing forward and recomputing backward with the latency-oriented
    forward, several segments, against the oracle."""
    import torch
    from non_linear_matrix_amd import m2rnn
    from oracle import m2rnn_bwd_ref

    cfg = scaled(CONFIGS["C5"], B=2, H=2, T=70)
    announce("long kernel recompute mode, segments of 16")
    x = generate(cfg, 69)
    d = to_device(x)
    dy = torch.randn((cfg.B, cfg.H, cfg.T, cfg.V), generator=torch.Generator().manual_seed(9)).cuda()
    y, HT, ck = m2rnn.fwd_ckpt(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], segment=16, algo="mfma_long_split")
    g = m2rnn.bwd_recompute(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], ck, dy, segment=16,
                            algo="mfma_long_split")
    torch.cuda.synchronize()
    ref = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy.cpu().numpy(), dtype=cfg.dtype)
    assert nerr(y.cpu().numpy(), ref["y"]) <= TOL and nerr(HT.cpu().numpy(), ref["H_T"]) <= TOL
    for key in ("dk", "dv", "dq", "df", "dW", "dH0"):
        assert nerr(g[key].cpu().numpy(), ref[key]) <= TOL, key


@pytest.mark.parametrize("algo", ["mfma_long_f16", "mfma_long_split", "mfma_long"])
def test_more_row_tiles_than_cus(algo):
    """More 16-row tiles than the GPU has CUs (3 x 16 x 128 rows: 384 tiles, two
    workgroups on some CUs), every unit against the oracle."""
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C3"], B=3, H=16, K=128, T=37)
    p = m2rnn.get_plan(cfg.B, cfg.H, cfg.T, cfg.K, cfg.V, cfg.dtype, algo)
    assert p["rows_per_group"] == 16 and p["grid"] == 384
    announce(f"long kernel, 16-row tiles, {algo}")
    x = generate(cfg, 70)
    yr, HTr = oracle_units(x, cfg.dtype)
    y, HT = gpu_run(x, algo=algo)
    ey, eh = nerr(y, yr), nerr(HT, HTr)
    print(f"{algo} 384 tiles: y {ey:.2e} H_T {eh:.2e}", flush=True)
    assert ey <= TOL and eh <= TOL
