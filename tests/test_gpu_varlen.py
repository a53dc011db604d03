"""GPU parity of the variable-length entry point (m2rnn_fwd_varlen) against the
fp64 oracle run on each sequence's own steps, plus its edge cases: empty
sequences, full lengths, step-by-step decoding with the state kept in place.
"""
import numpy as np
import pytest

from gpu_util import announce, nerr, to_device
from non_linear_matrix_amd.inputs import CONFIGS, generate, scaled
from oracle import m2rnn_fwd_ref

pytestmark = pytest.mark.gpu

TOL = {"mfma": 2e-2, "mfma_split": 2e-2, "mfma_f16": 2e-2, "simple": 1e-4}
ALGOS = ("mfma", "mfma_split", "mfma_f16", "simple")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from non_linear_matrix_amd import m2rnn
    m2rnn.load()


def _run(x, lens, algo, **kw):
    import torch
    from non_linear_matrix_amd import m2rnn

    d = to_device(x)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    y, HT = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], seq_len=sl, algo=algo, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy(), HT.cpu().numpy()


def _oracle_seq(x, b, n, dtype):
    """Oracle over the first n steps of batch row b (all heads)."""
    sub = {key: x[key][b:b + 1, :, :n] for key in ("k", "v", "q", "f")}
    H0 = None if x["H0"] is None else x["H0"][b:b + 1]
    return m2rnn_fwd_ref(sub["k"], sub["v"], sub["q"], sub["f"], x["W"], H0, dtype=dtype)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("K,V", [(128, 128), (64, 128), (64, 64)])
def test_varlen_matches_per_sequence_oracle(algo, K, V):
    T = 40
    lens = [40, 17, 1, 0, 33]
    cfg = scaled(CONFIGS["C3"], B=len(lens), H=2, K=K, V=V, T=T)
    announce(f"varlen {algo} K={K} V={V} T={T} lens={lens}")
    x = generate(cfg, seed=11)
    y, HT = _run(x, lens, algo)
    for b, n in enumerate(lens):
        if n == 0:
            # an empty sequence hands H0 back bit for bit and leaves y at zero
            assert np.array_equal(HT[b], x["H0"][b]), f"seq {b}: H_T != H0"
            assert not np.any(y[b]), f"seq {b}: y not zero"
            continue
        yr, HTr = _oracle_seq(x, b, n, cfg.dtype)
        ey, eh = nerr(y[b:b + 1, :, :n], yr), nerr(HT[b:b + 1], HTr)
        print(f"seq {b} len {n}: err y {ey:.3e} H_T {eh:.3e}", flush=True)
        assert ey <= TOL[algo] and eh <= TOL[algo]
        assert not np.any(y[b, :, n:]), f"seq {b}: rows past the length not zero"


@pytest.mark.parametrize("algo", ALGOS)
def test_full_lengths_equal_the_plain_call(algo):
    cfg = scaled(CONFIGS["C3"], B=3, H=2, T=37)
    announce(f"varlen full lengths {algo}")
    x = generate(cfg, seed=12)
    y0, H0 = _run(x, None, algo)
    y1, H1 = _run(x, [cfg.T] * cfg.B, algo)
    assert np.array_equal(y0, y1) and np.array_equal(H0, H1)


def test_lengths_are_clamped():
    cfg = scaled(CONFIGS["C3"], B=2, H=1, T=20)
    announce("varlen clamping")
    x = generate(cfg, seed=13)
    y, HT = _run(x, [-5, 1000], "mfma_split")
    assert np.array_equal(HT[0], x["H0"][0]) and not np.any(y[0])
    yr, HTr = _oracle_seq(x, 1, cfg.T, cfg.dtype)
    assert nerr(HT[1:2], HTr) <= 2e-2 and nerr(y[1:2], yr) <= 2e-2


@pytest.mark.parametrize("algo", ALGOS)
def test_decode_steps_in_place_match_one_call(algo):
    """T = 1 calls with H_T aliasing H0, sequence 1 idle (length 0) every other step."""
    import torch
    from non_linear_matrix_amd import m2rnn

    steps = 6
    cfg = scaled(CONFIGS["C3"], B=2, H=4, T=steps)
    announce(f"decode in place {algo}")
    x = generate(cfg, seed=14)
    d = to_device(x)
    state = d["H0"].clone()
    ys = []
    took = [0, 0]
    for t in range(steps):
        lens = [1, t % 2]
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        sel = {}
        for key in ("k", "v", "q", "f"):
            # sequence 1 consumes its own next step when it is active
            rows = [d[key][0, :, t:t + 1], d[key][1, :, took[1]:took[1] + 1]]
            sel[key] = torch.stack(rows).contiguous()
        y, _ = m2rnn.fwd(sel["k"], sel["v"], sel["q"], sel["f"], d["W"], state, H_T=state, seq_len=sl, algo=algo)
        ys.append(y.cpu().numpy())
        took = [took[0] + 1, took[1] + lens[1]]
    torch.cuda.synchronize()
    HT = state.cpu().numpy()
    yr0, HTr0 = _oracle_seq(x, 0, steps, cfg.dtype)
    yr1, HTr1 = _oracle_seq(x, 1, took[1], cfg.dtype)
    y0 = np.concatenate([yy[0:1] for yy in ys], axis=2)
    tol = TOL[algo]
    assert nerr(HT[0:1], HTr0) <= tol and nerr(y0, yr0) <= tol
    assert nerr(HT[1:2], HTr1) <= tol
    # the idle steps of sequence 1 gave zero rows
    assert all(not np.any(ys[t][1]) for t in range(steps) if t % 2 == 0)


def test_accumulate_leaves_rows_past_the_length():
    import torch
    from non_linear_matrix_amd import m2rnn

    cfg = scaled(CONFIGS["C3"], B=2, H=2, T=24)
    announce("varlen accumulate")
    x = generate(cfg, seed=15)
    d = to_device(x)
    base = torch.full((cfg.B, cfg.H, cfg.T, cfg.V), 0.5, dtype=torch.float32, device="cuda")
    sl = torch.tensor([24, 9], dtype=torch.int32, device="cuda")
    y, _ = m2rnn.fwd(d["k"], d["v"], d["q"], d["f"], d["W"], d["H0"], y=base, seq_len=sl,
                     algo="mfma_split", accumulate_y=True)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.all(y[1, :, 9:] == 0.5)
    yr, _ = _oracle_seq(x, 1, 9, cfg.dtype)
    assert nerr(y[1:2, :, :9] - 0.5, yr) <= 2e-2
