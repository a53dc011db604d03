"""GPU parity of the fp32 matrix-core family (MFMA_F32) against the fp64 oracle,
beside the fp32 simple kernel, plus its contract: fixed summation order, empty
and ragged sequences, continuation, accumulation.

Bar: the fp32 path's 1e-4 on max|X_gpu - X_ref| / max|X_ref| per output tensor.
"""
import numpy as np
import pytest

from gpu_util import announce, gpu_run, nerr, oracle_units, to_device, worst_unit
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled
from oracle import m2rnn_fwd_ref

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


def _f32(name, **shape):
    """A workload's distributions with fp32 storage."""
    return scaled(CONFIGS[name], **shape).with_(dtype="f32")


@pytest.mark.parametrize("algo", ["auto", "mfma_f32", "simple"])
def test_c1(algo):
    from non_linear_matrix_amd import m2rnn
    cfg = CONFIGS["C1"]
    assert m2rnn.pick_algo(cfg.B, cfg.H, cfg.T, cfg.K, cfg.V, "f32") == "mfma_f32"
    announce(f"C1 fp32, algo={algo}")
    x = generate(cfg, 0)
    y, HT = gpu_run(x, algo=algo)
    yr, HTr = oracle_units(x, "f32")
    print(f"C1 {algo}: err y {nerr(y, yr):.3e} H_T {nerr(HT, HTr):.3e}", flush=True)
    assert nerr(y, yr) <= TOL and nerr(HT, HTr) <= TOL


SHAPES = ([(K, V) for K in (16, 32, 64, 128) for V in (16, 48, 64, 80, 128)]
          + [(48, 112), (96, 32), (112, 96)])


@pytest.mark.parametrize("T", [1, 37])
@pytest.mark.parametrize("K,V", SHAPES)
def test_shapes_and_ragged_lengths(K, V, T):
    """Every tile count of both dimensions (W in registers up to V = 64, from
    LDS above), one step and a ragged 16-step chunk, random H0."""
    cfg = _f32("C1", B=2, H=3, K=K, V=V, T=T).with_(h0="uniform")
    x = generate(cfg, seed=K + V + T)
    yr, HTr = oracle_units(x, "f32")
    for algo in ("mfma_f32", "simple"):
        announce(f"fp32 shape K={K} V={V} T={T} algo={algo}")
        y, HT = gpu_run(x, algo=algo)
        assert nerr(y, yr) <= TOL, (algo, nerr(y, yr))
        assert nerr(HT, HTr) <= TOL, (algo, nerr(HT, HTr))


# the larger workloads' distributions in fp32 (several chunks, many units):
# C2 at full size on every unit, C3 and C5 shortened
LARGER = [("C2", {}), ("C3", dict(B=2, H=4, T=300)), ("C5", dict(B=1, H=4, T=700))]


@pytest.mark.parametrize("algo", ["mfma_f32", "simple"])
@pytest.mark.parametrize("name,shape", LARGER, ids=[n for n, _ in LARGER])
def test_larger_workloads_every_unit(name, shape, algo):
    cfg = _f32(name, **shape)
    x = generate(cfg, 0)
    announce(f"fp32 {name} {shape}, {algo}")
    y, HT = gpu_run(x, algo=algo)
    yr, HTr = oracle_units(x, "f32")
    (uy, ey), (uh, eh) = worst_unit(y, yr), worst_unit(HT, HTr)
    print(f"fp32 {name} {algo}: err y {nerr(y, yr):.3e} H_T {nerr(HT, HTr):.3e} | worst unit y {uy} {ey:.3e}, "
          f"H_T {uh} {eh:.3e}", flush=True)
    assert nerr(y, yr) <= TOL and nerr(HT, HTr) <= TOL


def test_gate_one_keeps_state():
    """f = 1: H_T = H_0 bit for bit (H + 0 * Z), y_t = H_0^T q_t."""
    cfg = _f32("C3", B=2, H=2, K=64, V=128, T=33)
    x = generate(cfg, 6)
    x["f"][:] = 1.0
    announce("fp32 gate one")
    y, HT = gpu_run(x, algo="mfma_f32")
    H0 = x["H0"]
    assert np.array_equal(HT, H0)
    yr, _ = oracle_units(x, "f32")
    assert nerr(y, yr) <= TOL


def test_h0_null_equals_zero_state_and_state_optional():
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = _f32("C2", B=2, H=2, T=40)
    x = generate(cfg, 5)
    announce("fp32 H0 NULL vs zeros")
    d = to_device(x)
    y1, HT1 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], None, algo="mfma_f32")
    z = torch.zeros((2, 2, cfg.K, cfg.V), dtype=torch.float32, device="cuda")
    y2, HT2 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], z, algo="mfma_f32")
    y3, HT3 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], None, algo="mfma_f32", want_state=False)
    torch.cuda.synchronize()
    assert HT3 is None
    assert torch.equal(HT1, HT2) and torch.equal(y1, y2) and torch.equal(y1, y3)


def test_bitwise_repeatable_and_deterministic_flag():
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = _f32("C3", B=2, H=4, T=64)
    x = generate(cfg, 7)
    announce("fp32 determinism")
    y1, HT1 = gpu_run(x, algo="mfma_f32")
    y2, HT2 = gpu_run(x, algo="mfma_f32")
    assert np.array_equal(y1, y2) and np.array_equal(HT1, HT2)
    d = to_device(x)
    y3, HT3 = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], deterministic=True)
    torch.cuda.synchronize()
    assert np.array_equal(y3.cpu().numpy(), y1) and np.array_equal(HT3.cpu().numpy(), HT1)


def test_accumulate_flag_adds_into_y():
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = _f32("C3", B=2, H=2, T=30)
    x = generate(cfg, 11)
    d = to_device(x)
    announce("fp32 accumulate flag")
    y0, _ = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo="mfma_f32")
    y1 = torch.full_like(y0, 0.25)
    m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y1, algo="mfma_f32", accumulate_y=True,
              deterministic=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, 0.25 + y0)  # one add per element: 0.25 + s exactly as torch rounds it


def test_chunked_continuation():
    """fwd(T1) then fwd(T2, H0 = H_T, in place) continues fwd(T1 + T2) bit for
    bit: the state crosses the boundary as the kernel holds it."""
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = _f32("C3", B=2, H=2, T=50)
    x = generate(cfg, 8)
    d = to_device(x)
    announce("fp32 chunked continuation")
    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo="mfma_f32")
    T1 = 21
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    ya, HTa = m2rnn.fwd(sl(d["k"], 0, T1), sl(d["v"], 0, T1), sl(d["q"], 0, T1), sl(d["f"], 0, T1), d["W"],
                        d["H0"], algo="mfma_f32")
    yb, HTb = m2rnn.fwd(sl(d["k"], T1, 50), sl(d["v"], T1, 50), sl(d["q"], T1, 50), sl(d["f"], T1, 50), d["W"],
                        HTa, H_T=HTa, algo="mfma_f32")
    torch.cuda.synchronize()
    yc = torch.cat([ya, yb], dim=2)
    assert torch.equal(yc, y) and torch.equal(HTb, HT)


@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (16, 16)])
def test_varlen_matches_per_sequence_oracle(K, V):
    import torch
    from non_linear_matrix_amd import m2rnn
    lens = [40, 17, 1, 0, 33]
    cfg = _f32("C3", B=len(lens), H=2, K=K, V=V, T=40)
    x = generate(cfg, seed=11)
    announce(f"fp32 varlen K={K} V={V} lens={lens}")
    d = to_device(x)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], seq_len=sl, algo="mfma_f32")
    torch.cuda.synchronize()
    y, HT = y.cpu().numpy(), HT.cpu().numpy()
    for b, n in enumerate(lens):
        assert not np.any(y[b, :, n:]), f"seq {b}: rows past the length not zero"
        if n == 0:
            assert np.array_equal(HT[b], x["H0"][b]), f"seq {b}: H_T != H0"
            continue
        sub = {key: x[key][b:b + 1, :, :n] for key in ("k", "v", "q", "f")}
        yr, HTr = m2rnn_fwd_ref(sub["k"], sub["v"], sub["q"], sub["f"], x["W"], x["H0"][b:b + 1], dtype="f32")
        assert nerr(y[b:b + 1, :, :n], yr) <= TOL and nerr(HT[b:b + 1], HTr) <= TOL, b


def test_nondefault_stream_ordering():
    import torch
    from non_linear_matrix_amd import m2rnn
    cfg = _f32("C3", B=2, H=2, T=24)
    x = generate(cfg, 10)
    d = to_device(x)
    announce("fp32 non-default stream")
    ref_y, ref_HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], algo="mfma_f32")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = torch.empty_like(ref_y)
    HT = torch.empty_like(ref_HT)
    with torch.cuda.stream(s):
        y.fill_(float("nan"))
        HT.fill_(float("nan"))
        m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=y, H_T=HT, stream=s, algo="mfma_f32")
    s.synchronize()
    assert torch.equal(y, ref_y) and torch.equal(HT, ref_HT)
