"""GPU parity of the fp16-operand forwards ("mfma_f16", the multi-step kernel,
and "mfma_long_f16", the latency-oriented one) against the fp64 oracle.

Same state arithmetic as "mfma" / "mfma_long" (fp32 state, one rounded operand
per step), but the operand of H_{t-1} W and of the readout is fp16 (11
significant bits, 2^-12 relative rounding) instead of bf16 (8 bits, 2^-9); W and
q are bf16 inputs, converted exactly. Bar: 2e-2 normwise, the bf16-input bar,
on every unit of every full-size workload, including the two where one bf16
operand misses it.
"""
import numpy as np
import pytest

from gpu_util import announce, full_parity, gpu_run, nerr, oracle_units, to_device
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled

pytestmark = pytest.mark.gpu

TOL = 2e-2
# The fp16 operand's rounding is 1/8 of the bf16 operand's: on the workloads
# where one bf16 operand reaches 2.2e-2 to 2.6e-2 this keeps 1e-2 (measured
# values are printed); losing the extra bits would show here first.
F16_GUARD = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


FULL = [("C2", "mfma_f16"), ("C3", "mfma_f16"), ("C4", "mfma_f16"), ("C5", "mfma_f16"),
        ("C2", "mfma_long_f16"), ("C4", "mfma_long_f16"), ("C5", "mfma_long_f16")]


@pytest.mark.parametrize("name,algo", FULL)
def test_full_size_configs(name, algo):
    """Every unit of the full-size workloads against the oracle."""
    ey, eh = full_parity(name, algo, TOL)
    assert ey <= TOL and eh <= TOL
    assert ey <= F16_GUARD and eh <= F16_GUARD


SHAPES = [(K, V) for K in (16, 32, 48, 64, 128) for V in (64, 128)]


@pytest.mark.parametrize("T", [1, 17, 37])
@pytest.mark.parametrize("K,V", SHAPES)
def test_shapes_and_ragged_lengths(K, V, T):
    """Several tiles, a ragged tail and one step, random H0, both families where
    they cover the shape (the multi-step kernel needs K in {32, 64, 128})."""
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C3"], B=2, H=3, K=K, V=V, T=T)
    x = generate(cfg, seed=3 * K + V + T)
    yr, HTr = oracle_units(x, "bf16")
    algos = ["mfma_long_f16"]
    if m2rnn.check_args(1 << 16, 1 << 16, 1 << 16, 1 << 16, 1 << 16, None, 1 << 16, None, 2, 3, T, K, V,
                        "bf16", "mfma_f16") == 0:
        algos.append("mfma_f16")
    for algo in algos:
        announce(f"f16 shape K={K} V={V} T={T} algo={algo}")
        y, HT = gpu_run(x, algo=algo)
        ey, eh = nerr(y, yr), nerr(HT, HTr)
        assert ey <= TOL and eh <= TOL, (algo, ey, eh)


@pytest.mark.parametrize("algo", ["mfma_f16", "mfma_long_f16"])
def test_gate_one_keeps_state(algo):
    """f = 1: the blend returns the state (to the 2/ln 2 scaling's rounding) and
    y_t = H_0^T q_t."""
    cfg = scaled(CONFIGS["C3"], B=2, H=2, K=64, V=128, T=33)
    x = generate(cfg, 6)
    x["f"][:] = 0x3F80  # bf16 1.0
    announce(f"gate one, algo={algo}")
    y, HT = gpu_run(x, algo=algo)
    H0 = x["H0"]
    assert np.max(np.abs(HT - H0) / np.maximum(np.abs(H0), 1e-30)) <= 2.5e-7
    yr, _ = oracle_units(x, "bf16")
    assert nerr(y, yr) <= TOL


@pytest.mark.parametrize("algo", ["mfma_f16", "mfma_long_f16"])
def test_h0_null_equals_zero_state(algo):
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C2"], B=2, H=2, T=40)
    x = generate(cfg, 5)
    announce(f"H0 NULL vs zeros, algo={algo}")
    d = to_device(x)
    y1, HT1 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], None, algo=algo)
    z = torch.zeros((2, 2, cfg.K, cfg.V), dtype=torch.float32, device="cuda")
    y2, HT2 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], z, algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(HT1, HT2) and torch.equal(y1, y2)


@pytest.mark.parametrize("algo", ["mfma_f16", "mfma_long_f16"])
def test_repeatable(algo):
    """Same inputs, same bits: the multi-step kernel's two workgroups per unit add
    onto a cleared y (0 + a + b = 0 + b + a), the long kernel's row tiles onto
    its y grid."""
    cfg = scaled(CONFIGS["C3"], B=2, H=4, T=64)
    x = generate(cfg, 7)
    announce(f"repeatability, algo={algo}")
    y1, HT1 = gpu_run(x, algo=algo)
    y2, HT2 = gpu_run(x, algo=algo)
    assert np.array_equal(y1, y2) and np.array_equal(HT1, HT2)


def test_long_agrees_with_the_multi_step_kernel():
    """The two kernels add the operand blocks in different orders, so their fp32
    accumulators differ in the last bits; an fp16 rounding flip (2^-12) of one
    state element then parts the trajectories at about that level."""
    cfg = scaled(CONFIGS["C3"], B=2, H=3, T=70)
    announce("f16 long vs multi-step")
    x = generate(cfg, 62)
    y0, HT0 = gpu_run(x, algo="mfma_f16")
    y1, HT1 = gpu_run(x, algo="mfma_long_f16")
    eh, ey = nerr(HT1, HT0), nerr(y1, y0)
    print(f"f16 long vs multi-step: y {ey:.2e} H_T {eh:.2e}", flush=True)
    assert eh <= 1e-3 and ey <= 2.0 ** -10


@pytest.mark.parametrize("algo", ["mfma_f16", "mfma_long_f16"])
def test_readout_self_consistency(algo):
    """y_T against H_T^T q_T recomputed in fp64 from the kernel's own H_T: the
    readout takes the state rounded to fp16 (2^-12 relative per element)."""
    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=24)
    x = generate(cfg, 9)
    announce(f"readout self-consistency, algo={algo}")
    y, HT = gpu_run(x, algo=algo)
    from non_linear_matrix_amd.inputs import bf16_bits_to_fp32
    q = bf16_bits_to_fp32(x["q"]).astype(np.float64)[:, :, -1, :]
    yT = np.einsum("bhk,bhkv->bhv", q, HT.astype(np.float64))
    e = nerr(y[:, :, -1, :], yT)
    print(f"{algo}: readout self-consistency {e:.2e}", flush=True)
    assert e <= 1e-3


def test_training_entry_points_refuse_the_f16_families():
    """The backward pass reads bf16 operands saved by the forward: the training
    forwards take only the bf16 families (NOT_SUPPORTED before any launch)."""
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = scaled(CONFIGS["C3"], B=1, H=2, K=64, T=16)
    d = to_device(generate(cfg, 11))
    for algo in ("mfma_f16", "mfma_long_f16"):
        with pytest.raises(RuntimeError):
            m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo=algo)
    torch.cuda.synchronize()


@pytest.mark.parametrize("algo", ["mfma_f16", "mfma_long_f16"])
def test_values_beyond_the_fp16_range_give_nan(algo):
    """One W, q or H0 value beyond the fp16 operand's range makes the outputs it
    reaches NaN, never a finite wrong value; in range (65504 itself) all is finite.
    The split operand (full bf16 range) keeps every output finite."""
    from non_linear_matrix_amd.inputs import fp32_to_bf16_bits
    cfg = scaled(CONFIGS["C3"], B=1, H=2, K=64, V=128, T=20)
    base = generate(cfg, 12)
    big = fp32_to_bf16_bits(np.array([1.0e5], np.float32))[0]
    edge = fp32_to_bf16_bits(np.array([65280.0], np.float32))[0]   # the largest bf16 below 65504

    def case(what):
        x = {k: (None if a is None else a.copy()) for k, a in base.items()}
        if what == "W":
            x["W"][1, 3, 5] = big
        elif what == "q":
            x["q"][0, 1, 7, 2] = big
        elif what == "H0":
            x["H0"][0, 1, 4, 9] = 3.0e4
        elif what == "W_edge":
            x["W"][1, 3, 5] = edge
        return x

    announce(f"fp16 range, algo={algo}")
    for what in ("W", "H0"):
        y, HT = gpu_run(case(what), algo=algo)
        assert np.all(np.isfinite(y[:, 0])) and np.all(np.isfinite(HT[:, 0])), what   # head 0 untouched
        assert np.any(np.isnan(HT[:, 1])) and np.any(np.isnan(y[:, 1])), what
        ys, HTs = gpu_run(case(what), algo="mfma_split")
        assert np.all(np.isfinite(ys)) and np.all(np.isfinite(HTs)), what
    y, HT = gpu_run(case("q"), algo=algo)
    assert np.all(np.isnan(y[0, 1, 7])) and np.all(np.isfinite(HT)), "q"
    assert np.all(np.isfinite(np.delete(y[0, 1], 7, axis=0)))
    y, HT = gpu_run(case("W_edge"), algo=algo)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(HT)), "W at 65280"
