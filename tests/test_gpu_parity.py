"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Metric: per output tensor, max|X_gpu - X_ref| / max|X_ref|. Bars: 1e-4 for the
fp32 path (and for the simple kernel, which computes in fp32 throughout), 2e-2
for the bf16-operand matrix-core path.
"""
import numpy as np
import pytest

from gpu_util import announce, full_parity, gpu_run, nerr, oracle_units, to_device
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
SPLIT_GUARD = 1e-3


def _tol(cfg, algo):
    if cfg.dtype == "f32" or algo == "simple":
        return TOL_F32
    return TOL_BF16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


def test_c1_fp32_full():
    cfg = CONFIGS["C1"]
    announce("C1 fp32 full, auto")
    x = generate(cfg, 0)
    y, HT = gpu_run(x)
    yr, HTr = oracle_units(x, cfg.dtype)
    assert nerr(y, yr) <= TOL_F32 and nerr(HT, HTr) <= TOL_F32


# (workload, kernel family) pairs compared with the oracle on every (b, h) unit at
# full size: every family AUTO or the benchmark runs there, and the fp32 simple
# kernel. The latency-oriented families are in test_gpu_long.py.
FULL = [("C2", "mfma_split"), ("C2", "simple"),
        ("C3", "mfma"), ("C3", "mfma_split"), ("C3", "simple"),
        ("C4", "mfma"), ("C4", "mfma_split"), ("C4", "simple"),
        ("C5", "mfma_split"), ("C5", "simple")]


@pytest.mark.parametrize("name,algo", FULL)
def test_full_size_configs(name, algo):
    """Full-size workloads in the launch configuration the benchmark times,
    every unit against the oracle."""
    tol = _tol(CONFIGS[name], algo)
    ey, eh = full_parity(name, algo, tol)
    assert ey <= tol and eh <= tol
    if algo.endswith("split"):
        # the split operand carries ~16 significant bits: measured at most 1.1e-4
        # (C2, H_T) on these workloads, so 1e-3 catches a lost low half long
        # before the 2e-2 bar would
        assert ey <= SPLIT_GUARD and eh <= SPLIT_GUARD


# The single bf16 operand (MFMA, MFMA_LONG) meets the bar on C3 and C4, but on C2
# and C5 (gates near 1 and inputs scaled by 1/sqrt(K), where the trajectory
# amplifies per-step rounding) it goes past 2e-2; the split operand of the
# default families is for those. The measured errors are recorded here so the
# gap stays visible; the bound only says the result is still the same
# trajectory to within a few percent.
RECORDED_GAP = [("C2", "mfma"), ("C5", "mfma"), ("C2", "mfma_long"), ("C5", "mfma_long")]


@pytest.mark.parametrize("name,algo", RECORDED_GAP)
def test_single_operand_error_on_sensitive_workloads(name, algo):
    ey, eh = full_parity(name, algo, TOL_BF16)
    assert ey <= 0.1 and eh <= 0.1


SHAPES = [(K, V) for K in (16, 32, 64, 128) for V in (16, 64, 128)] + [(48, 112), (96, 32)]


@pytest.mark.parametrize("T", [1, 37])
@pytest.mark.parametrize("K,V", SHAPES)
def test_shapes_and_ragged_lengths(K, V, T):
    """Several tiles and a ragged tail (T not a multiple of the 16-step staging
    chunk), random H0, every kernel that covers the shape."""
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C3"], B=2, H=3, K=K, V=V, T=T)
    x = generate(cfg, seed=K + V + T)
    yr, HTr = oracle_units(x, "bf16")
    covered = m2rnn.check_args(1 << 16, 1 << 16, 1 << 16, 1 << 16, 1 << 16, None, 1 << 16,
                               None, 2, 3, T, K, V, "bf16", "mfma") == 0
    algos = ["simple"] + (["mfma", "mfma_split"] if covered else [])
    for algo in algos:
        announce(f"shape K={K} V={V} T={T} algo={algo}")
        y, HT = gpu_run(x, algo=algo)
        assert nerr(y, yr) <= _tol(cfg, algo), (algo, nerr(y, yr))
        assert nerr(HT, HTr) <= _tol(cfg, algo), (algo, nerr(HT, HTr))


@pytest.mark.parametrize("algo", ["simple", "mfma", "mfma_split"])
def test_qkv_scale_alternative_reading(algo):
    """C3 distributions under the other reading of 'same distributions' (k, v, q
    scaled by 1/sqrt(K)), reduced length."""
    cfg = scaled(CONFIGS["C3"], B=2, H=4, T=300)
    x = generate(cfg, 3, qkv_scale="rsqrtK")
    announce(f"C3 rsqrtK reading, algo={algo}")
    y, HT = gpu_run(x, algo=algo)
    yr, HTr = oracle_units(x, "bf16")
    assert nerr(y, yr) <= _tol(cfg, algo) and nerr(HT, HTr) <= _tol(cfg, algo)


@pytest.mark.parametrize("algo", ["simple", "mfma", "mfma_split", "mfma_long", "mfma_long_split"])
def test_h0_null_equals_zero_state_and_state_optional(algo):
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C2"], B=2, H=2, T=40)
    x = generate(cfg, 5)
    announce(f"H0 NULL vs zeros, algo={algo}")
    d = to_device(x)
    y1, HT1 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], None, algo=algo)
    z = torch.zeros((2, 2, cfg.K, cfg.V), dtype=torch.float32, device="cuda")
    y2, HT2 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], z, algo=algo)
    y3, HT3 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], None, algo=algo, want_state=False)
    torch.cuda.synchronize()
    assert HT3 is None
    assert torch.equal(HT1, HT2)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)


@pytest.mark.parametrize("algo", ["simple", "mfma", "mfma_split", "mfma_long", "mfma_long_split"])
def test_gate_one_keeps_state(algo):
    """f = 1: H_T = H_0 (bitwise for the fp32 kernel; within 2 ulp for the matrix-core
    kernel, which carries the state scaled by 2/ln 2) and y_t = H_0^T q_t."""
    cfg = scaled(CONFIGS["C3"], B=2, H=2, K=64, V=128, T=33)
    x = generate(cfg, 6)
    x["f"][:] = 0x3F80  # bf16 1.0
    announce(f"gate one, algo={algo}")
    y, HT = gpu_run(x, algo=algo)
    H0 = x["H0"]
    if algo == "simple":
        assert np.array_equal(HT, H0)
    else:
        assert np.max(np.abs(HT - H0) / np.maximum(np.abs(H0), 1e-30)) <= 2.5e-7
    yr, _ = oracle_units(x, "bf16")
    assert nerr(y, yr) <= _tol(cfg, algo)


@pytest.mark.parametrize("algo", ["simple", "mfma", "mfma_split", "mfma_long", "mfma_long_split", "mfma_f16",
                                  "mfma_long_f16"])
def test_deterministic(algo):
    cfg = scaled(CONFIGS["C3"], B=2, H=4, T=64)
    x = generate(cfg, 7)
    announce(f"determinism, algo={algo}")
    y1, HT1 = gpu_run(x, algo=algo)
    y2, HT2 = gpu_run(x, algo=algo)
    assert np.array_equal(y1, y2) and np.array_equal(HT1, HT2)


@pytest.mark.parametrize("algo", ["simple", "mfma", "mfma_split", "mfma_long", "mfma_long_split", "mfma_f16",
                                  "mfma_long_f16"])
def test_chunked_continuation(algo):
    """fwd(T1) then fwd(T2, H0 = H_T) continues fwd(T1 + T2): bitwise for the fp32
    kernel. The matrix-core kernels carry c H (c = 2 / ln 2) and hand back
    H_T = (c H) / c in fp32, so the continued call can start one rounding away
    from the single call's state: with the split operand that stays at the fp32
    level (bound 5e-5; measured ~2e-6 to 4e-6), with one bf16 operand a one-ulp
    change can move one element's operand rounding (2^-9) and carry it forward
    (bound 2^-8; measured 4e-8 to 3e-4)."""
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=50)
    x = generate(cfg, 8)
    d = to_device(x)
    announce(f"chunked continuation, algo={algo}")
    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
    T1 = 21
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    ya, HTa = m2rnn.fwd(sl(d["k"], 0, T1), sl(d["v"], 0, T1), sl(d["q"], 0, T1), sl(d["f"], 0, T1), d["W"], d["H0"], algo=algo)
    yb, HTb = m2rnn.fwd(sl(d["k"], T1, 50), sl(d["v"], T1, 50), sl(d["q"], T1, 50), sl(d["f"], T1, 50), d["W"], HTa,
                        H_T=HTa, algo=algo)  # in-place continuation
    torch.cuda.synchronize()
    yc = torch.cat([ya, yb], dim=2)
    if algo == "simple":
        assert torch.equal(yc, y) and torch.equal(HTb, HT)
    else:
        ey = nerr(yc.cpu().numpy(), y.cpu().numpy().astype(np.float64))
        eh = nerr(HTb.cpu().numpy(), HT.cpu().numpy().astype(np.float64))
        print(f"{algo}: continuation against one call: y {ey:.2e} H_T {eh:.2e}", flush=True)
        tol = 5e-5 if algo.endswith("split") else 2.0 ** -8
        assert ey <= tol and eh <= tol


@pytest.mark.parametrize("algo", ["mfma", "mfma_split", "mfma_long", "mfma_long_split"])
def test_readout_self_consistency(algo):
    """y_T against H_T^T q_T recomputed in fp64 from the kernel's own H_T. The
    single-operand families read out from the state rounded to bf16 (2^-9
    relative per element; bound 8e-3, measured 2.2e-3); the split families from
    both bf16 halves, ~16 significant bits (bound 1e-4, measured 2e-6 to 4e-6)."""
    from non_linear_matrix_amd.inputs import bf16_bits_to_fp32
    cfg = scaled(CONFIGS["C3"], B=2, H=4, T=20)
    x = generate(cfg, 9)
    announce(f"readout self-consistency, {algo}")
    y, HT = gpu_run(x, algo=algo)
    q = bf16_bits_to_fp32(x["q"]).astype(np.float64)
    yT = np.einsum("bhkv,bhk->bhv", HT.astype(np.float64), q[:, :, -1])
    e = nerr(y[:, :, -1], yT)
    print(f"{algo}: y_T against H_T^T q_T {e:.2e}", flush=True)
    assert e <= (1e-4 if algo.endswith("split") else 8e-3)


def test_nondefault_stream_ordering():
    """The kernel runs on the caller's stream, ordered after earlier work on it."""
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=24)
    x = generate(cfg, 10)
    d = to_device(x)
    announce("non-default stream")
    # bitwise comparison: the kernels with a fixed summation order
    ref_y, ref_HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], deterministic=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = torch.empty_like(ref_y)
    HT = torch.empty_like(ref_HT)
    with torch.cuda.stream(s):
        y.fill_(float("nan"))
        HT.fill_(float("nan"))
        m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y, H_T=HT, stream=s, deterministic=True)
    s.synchronize()
    assert torch.equal(y, ref_y) and torch.equal(HT, ref_HT)


def test_launch_error_is_reported_not_raised_on_bad_args():
    import torch
    from non_linear_matrix_amd import m2rnn
    x = torch.zeros((1, 1, 4, 20), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m2rnn.M2RNNError) as ei:
        m2rnn.fwd(x, x, x, torch.zeros((1, 1, 4), dtype=torch.bfloat16, device="cuda"),
                  torch.zeros((1, 20, 20), dtype=torch.bfloat16, device="cuda"))
    assert ei.value.status == 2


@pytest.mark.parametrize("algo", ["simple", "mfma", "mfma_split"])
def test_accumulate_flag_adds_into_y(algo):
    """M2RNN_FLAG_ACCUMULATE_Y: y += readout, with nothing cleared by the library."""
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=30)
    x = generate(cfg, 11)
    d = to_device(x)
    announce(f"accumulate flag, algo={algo}")
    y0, _ = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
    base = torch.full_like(y0, 0.25)
    y1 = base.clone()
    m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y1, algo=algo, accumulate_y=True)
    torch.cuda.synchronize()
    assert torch.allclose(y1, y0 + 0.25, rtol=0, atol=1e-6)
