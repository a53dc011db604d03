"""GPU parity of training with recomputation (m2rnn_fwd_ckpt + m2rnn_bwd_recompute)
against the fp64 oracles on the same seeded inputs and output gradients.

Bars as the other bf16 tests (normwise, 2e-2). Beyond parity: the checkpoints
are the oracle's states at the segment starts, and with one segment the
recomputing backward pass is bit-identical to the one that reads the saving
forward's buffer (same kernels, same operands).
"""
import numpy as np
import pytest

from gpu_util import announce, nerr, to_device
from non_linear_matrix_amd.inputs import CONFIGS, bf16_bits_to_fp32, generate, scaled
from oracle import m2rnn_bwd_ref, m2rnn_fwd_ref

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


def _dy(cfg, seed, with_dHT=True):
    rng = np.random.default_rng(seed + 77)
    dy = rng.standard_normal((cfg.B, cfg.H, cfg.T, cfg.V)).astype(np.float32)
    dHT = rng.standard_normal((cfg.B, cfg.H, cfg.K, cfg.V)).astype(np.float32) if with_dHT else None
    return dy, dHT


def _train(cfg, seed, segment, with_dHT=True, zero_h0=False):
    import torch
    from non_linear_matrix_amd import m2rnn

    x = generate(cfg, seed)
    if zero_h0:
        x["H0"] = None
    dy, dHT = _dy(cfg, seed, with_dHT)
    d = to_device(x)
    y, HT, ckpt = m2rnn.fwd_ckpt(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], segment=segment)
    g = m2rnn.bwd_recompute(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], ckpt, torch.from_numpy(dy).cuda(),
                            None if dHT is None else torch.from_numpy(dHT).cuda(), segment=segment)
    torch.cuda.synchronize()
    got = {key: g[key].cpu().numpy() for key in GRADS}
    got["y"], got["H_T"] = y.cpu().numpy(), HT.cpu().numpy()
    got["ckpt"] = None if ckpt is None else ckpt.cpu().numpy()
    return x, dy, dHT, got


CASES = [
    ("C2", dict(B=2, H=2, T=20), 8),             # three segments, the last one 4 steps
    ("C2", dict(B=1, H=2, T=33), 16),            # 16 + 16 + 1
    ("C3", dict(B=1, H=2, T=37), 16),            # K = V = 128, two workgroups per unit
    ("C3", dict(B=2, H=1, T=40), 7),             # a segment that is not a multiple of the chunk
    ("C5", dict(B=2, H=1, T=16, K=32), 5),       # two-wave workgroups
    ("C3", dict(B=2, H=2, T=48, K=64, V=128), 48),   # one segment: recompute everything from H0
    ("C3", dict(B=1, H=2, T=24), 1),             # one step per segment
]


@pytest.mark.parametrize("name,shape,segment", CASES)
def test_gradients_match_the_oracle(name, shape, segment):
    cfg = scaled(CONFIGS[name], **shape)
    announce(f"recompute {name} {shape} segment {segment}")
    x, dy, dHT, got = _train(cfg, 41, segment)
    ref = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], x["H0"], dy, dHT, dtype=cfg.dtype)
    errs = {key: nerr(got[key], ref[key]) for key in GRADS + ("y", "H_T")}
    print(" ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, f"{key}: {e:.3e}"


def test_checkpoints_are_the_states_at_segment_starts():
    cfg = scaled(CONFIGS["C3"], B=1, H=2, T=50)
    segment = 16
    announce("recompute: checkpoint contents")
    x, _, _, got = _train(cfg, 42, segment)
    ck = got["ckpt"]
    assert ck.shape == (3, 1, 2, cfg.K, cfg.V)
    for j in range(1, 4):
        part = {key: (a[:, :, :j * segment] if key in ("k", "v", "q", "f") else a) for key, a in x.items()}
        _, Hj = m2rnn_fwd_ref(part["k"], part["v"], part["q"], part["f"], part["W"], part["H0"], dtype=cfg.dtype)
        assert nerr(ck[j - 1], Hj) <= TOL, j


def test_zero_initial_state_and_no_final_gradient():
    cfg = scaled(CONFIGS["C2"], B=2, H=1, T=30)
    announce("recompute: H0 = 0, dH_T = 0")
    x, dy, dHT, got = _train(cfg, 43, 12, with_dHT=False, zero_h0=True)
    ref = m2rnn_bwd_ref(x["k"], x["v"], x["q"], x["f"], x["W"], None, dy, None, dtype=cfg.dtype)
    for key in GRADS:
        assert nerr(got[key], ref[key]) <= TOL, key


def test_one_segment_equals_the_saved_state_backward_bit_for_bit():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=40)
    announce("recompute: one segment vs saved states")
    x = generate(cfg, 44)
    dy, dHT = _dy(cfg, 44)
    d = to_device(x)
    dyt, dHTt = torch.from_numpy(dy).cuda(), torch.from_numpy(dHT).cuda()
    y1, H1, saved = m2rnn.fwd_save(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"])
    g1 = m2rnn.bwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], saved, dyt, dHTt)
    y2, H2, ck = m2rnn.fwd_ckpt(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], segment=cfg.T)
    g2 = m2rnn.bwd_recompute(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], ck, dyt, dHTt, segment=cfg.T)
    torch.cuda.synchronize()
    assert ck is None
    assert torch.equal(H1, H2)
    # y: the latency-oriented forward (AUTO here) sums it over its K/16 row tiles;
    # the plain forward first rounds each tile's sum onto a grid of spacing
    # 2^(E - 23) with 2^E < 2.125 ||q_t||_1 (here max|H0| < 1), the saving forward
    # does not: they differ by at most K/16 half-spacings per element
    K = cfg.K
    qn = bf16_bits_to_fp32(x["q"]).astype(np.float64)
    bound = (K // 16) * 2.0 ** -24 * 2.125 * float(np.max(np.sum(np.abs(qn), axis=-1)))
    assert (y1 - y2).abs().max().item() <= bound
    for key in GRADS:
        assert torch.equal(g1[key], g2[key]), key


def test_recompute_is_deterministic():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=45)
    announce("recompute: determinism")
    x = generate(cfg, 45)
    d = to_device(x)
    dy = torch.randn((cfg.B, cfg.H, cfg.T, cfg.V), generator=torch.Generator().manual_seed(6)).cuda()
    _, _, ck = m2rnn.fwd_ckpt(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], segment=16)
    g1 = m2rnn.bwd_recompute(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], ck, dy, segment=16)
    g2 = m2rnn.bwd_recompute(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], ck, dy, segment=16)
    torch.cuda.synchronize()
    for key in GRADS:
        assert torch.equal(g1[key], g2[key]), key


FULL = [("C3", 7, 256), ("C5", 15, 4096)]


@pytest.mark.parametrize("name,head,segment", FULL)
def test_full_size_sampled_head(name, head, segment):
    """Full-size workloads with the segment length the training benchmark uses;
    the oracle runs on every batch row of one head."""
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = CONFIGS[name]
    announce(f"recompute {name} full size, head {head}, segment {segment}")
    x = generate(cfg, 0)
    dy = np.random.default_rng(98).standard_normal((cfg.B, cfg.H, cfg.T, cfg.V), dtype=np.float32)
    d = to_device(x)
    y, HT, ck = m2rnn.fwd_ckpt(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], segment=segment)
    g = m2rnn.bwd_recompute(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], ck, torch.from_numpy(dy).cuda(),
                            segment=segment)
    torch.cuda.synchronize()
    got = {key: g[key][head].cpu().numpy() if key == "dW" else g[key][:, head].cpu().numpy() for key in GRADS}
    got["y"] = y[:, head].cpu().numpy()
    del g, ck
    sl = {key: (None if a is None else (a[head:head + 1] if key == "W" else a[:, head:head + 1]))
          for key, a in x.items()}
    ref = m2rnn_bwd_ref(sl["k"], sl["v"], sl["q"], sl["f"], sl["W"], sl["H0"], dy[:, head:head + 1],
                        dtype=cfg.dtype)
    errs = {}
    for key in GRADS + ("y",):
        r = ref[key][0] if key == "dW" else ref[key][:, 0]
        assert np.all(np.isfinite(got[key])), key
        errs[key] = nerr(got[key], r)
    print(f"{name} head {head}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= TOL, f"{key}: {e:.3e}"
