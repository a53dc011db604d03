"""The C-ABI library on the host (no GPU): it loads, exports every declared
symbol, and its argument validation returns the documented codes without
touching the GPU."""
import ctypes
import os

import pytest

from non_linear_matrix_amd import m2rnn

OK, INVALID, UNSUPPORTED = 0, 1, 2
A = 0x10000  # a 16-byte aligned fake device address; validation never dereferences it


def _args(**over):
    base = dict(k=A, v=A + 0x100, q=A + 0x200, f=A + 0x300, W=A + 0x400, H0=None, y=A + 0x500,
                H_T=A + 0x600, B=2, H=3, T=5, K=64, V=128, dtype="bf16", algo="auto")
    base.update(over)
    return base


def _check(**over):
    a = _args(**over)
    return m2rnn.check_args(a["k"], a["v"], a["q"], a["f"], a["W"], a["H0"], a["y"], a["H_T"],
                            a["B"], a["H"], a["T"], a["K"], a["V"], a["dtype"], a["algo"])


def test_library_exists_and_loads():
    assert os.path.exists(m2rnn.LIB_PATH), "build the library first (python -m non_linear_matrix_amd.build)"
    lib = m2rnn.load()
    assert m2rnn.version() == 600


def test_every_declared_symbol_is_exported():
    names = m2rnn.declared_functions()
    assert set(names) >= {"m2rnn_fwd", "m2rnn_fwd_algo", "m2rnn_fwd_ex", "m2rnn_fwd_varlen",
                          "m2rnn_check_args", "m2rnn_pick_algo", "m2rnn_status_string", "m2rnn_version",
                          "m2rnn_saved_bytes", "m2rnn_fwd_save", "m2rnn_bwd_workspace_bytes", "m2rnn_bwd",
                          "m2rnn_ckpt_bytes", "m2rnn_fwd_ckpt", "m2rnn_bwd_recompute_workspace_bytes",
                          "m2rnn_bwd_recompute", "m2rnn_frontend"}
    raw = ctypes.CDLL(m2rnn.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), f"{name} declared in include/m2rnn.h but not exported"


def test_status_strings_cover_every_code():
    seen = set()
    for code in (0, 1, 2, 3):
        s = m2rnn.status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 4
    assert m2rnn.status_string(99) == "unknown status"


def test_valid_arguments_pass():
    assert _check() == OK
    assert _check(H0=A + 0x700, H_T=None) == OK
    assert _check(dtype="f32", K=16, V=16, algo="simple") == OK
    assert _check(K=128, V=128, algo="mfma") == OK


@pytest.mark.parametrize("name", ["k", "v", "q", "f", "W", "y"])
def test_null_required_pointer(name):
    assert _check(**{name: None}) == INVALID


@pytest.mark.parametrize("name", ["k", "v", "q", "f", "W", "y", "H0", "H_T"])
def test_misaligned_pointer(name):
    assert _check(**{name: A + 0x800 + 4}) == INVALID


@pytest.mark.parametrize("name", ["B", "H", "T", "K", "V"])
@pytest.mark.parametrize("value", [0, -1])
def test_bad_sizes(name, value):
    assert _check(**{name: value}) == INVALID


@pytest.mark.parametrize("K,V", [(8, 64), (64, 8), (20, 64), (64, 20), (144, 64), (64, 144), (1, 1)])
def test_unsupported_dims(K, V):
    assert _check(K=K, V=V) == UNSUPPORTED


def test_size_overflow_is_rejected():
    assert _check(B=2 ** 30, H=2 ** 30, T=2 ** 30) == INVALID


def test_unknown_dtype_and_algo():
    assert _check(dtype=7) == UNSUPPORTED
    assert _check(algo=9) == UNSUPPORTED


@pytest.mark.parametrize("algo", ["mfma", "mfma_split"])
def test_mfma_coverage(algo):
    assert _check(dtype="f32", algo=algo) == UNSUPPORTED          # fp32 inputs: simple kernel only
    assert _check(K=16, V=128, algo=algo) == UNSUPPORTED          # fewer than 32 rows
    assert _check(K=96, V=128, algo=algo) == UNSUPPORTED          # more than two row groups
    assert _check(K=128, V=96, algo=algo) == UNSUPPORTED
    for K in (32, 64, 128):
        for V in (64, 128):
            assert _check(K=K, V=V, algo=algo) == OK


def test_launch_plans():
    p = m2rnn.get_plan(8, 16, 2048, 128, 128, "bf16", "auto")
    assert p["algo"] == "mfma_split" and p["grid"] == 256 and p["block"] == 256
    assert p["rows_per_group"] == 64 and p["groups_per_unit"] == 2 and p["clears_y"] == 1
    assert p["lds_bytes"] <= 160 * 1024
    p = m2rnn.get_plan(2, 16, 32768, 64, 128, "bf16", "mfma")
    assert p["grid"] == 32 and p["groups_per_unit"] == 1 and p["clears_y"] == 0
    p = m2rnn.get_plan(1, 1, 64, 16, 16, "f32", "auto")
    assert p["algo"] == "simple" and p["grid"] == 1
    with pytest.raises(m2rnn.M2RNNError):
        m2rnn.get_plan(1, 1, 64, 20, 16, "f32", "auto")


def test_unknown_flag_bits_are_rejected():
    lib = m2rnn.load()
    for bad in (4, 0x80000000, 4 | m2rnn.FLAG_ACCUMULATE_Y):
        st = lib.m2rnn_fwd_ex(A, A, A, A, A, None, A, None, 1, 1, 4, 64, 64, 1, 0, bad, None)
        assert st == UNSUPPORTED, bad
    st = lib.m2rnn_fwd_ex(None, A, A, A, A, None, A, None, 1, 1, 4, 64, 64, 1, 0, 1, None)
    assert st == INVALID


def test_auto_picks_a_kernel_that_covers_the_shape():
    assert m2rnn.pick_algo(8, 16, 2048, 128, 128, "bf16") == "mfma_split"     # 1024 row tiles
    assert m2rnn.pick_algo(1, 1, 64, 16, 16, "f32") == "simple"
    assert m2rnn.pick_algo(1, 1, 64, 16, 96, "bf16") == "simple"
    # up to 768 16-row tiles: the latency-oriented kernel
    assert m2rnn.pick_algo(1, 1, 64, 16, 128, "bf16") == "mfma_long_split"
    assert m2rnn.pick_algo(1, 32, 8192, 128, 128, "bf16") == "mfma_long_split"
    assert m2rnn.pick_algo(2, 16, 32768, 64, 128, "bf16") == "mfma_long_split"
    assert m2rnn.pick_algo(4, 8, 512, 64, 64, "bf16") == "mfma_long_split"
    assert m2rnn.pick_algo(6, 16, 100, 128, 128, "bf16") == "mfma_long_split"  # 768 tiles
    assert m2rnn.pick_algo(7, 16, 100, 128, 128, "bf16") == "mfma_split"       # 896 tiles
    assert m2rnn.pick_algo(1, 32, 1, 128, 128, "bf16") == "mfma_split"         # one step: decoding kernel
    assert m2rnn.pick_algo(1, 4, 64, 32, 64, "f32") == "simple"
    p = m2rnn.get_plan(1, 32, 8192, 128, 128, "bf16", "auto")
    assert p["algo"] == "mfma_long_split" and p["grid"] == 256 and p["block"] == 256 and p["clears_y"] == 1


def test_deterministic_flag_refuses_the_atomic_kernels():
    """M2RNN_FLAG_DETERMINISTIC: explicit MFMA_LONG* with T > 1 is refused before
    any launch (their y adds over row tiles are atomic)."""
    lib = m2rnn.load()
    det = m2rnn.FLAG_DETERMINISTIC
    for algo in ("mfma_long", "mfma_long_split"):
        st = lib.m2rnn_fwd_ex(A, A, A, A, A, None, A, None, 1, 2, 16, 64, 128, 1, m2rnn.ALGOS[algo], det, None)
        assert st == UNSUPPORTED, algo
        st = lib.m2rnn_fwd_ex(A, A, A, A, A, None, A, None, 1, 2, 16, 64, 128, 1, m2rnn.ALGOS[algo],
                              det | m2rnn.FLAG_ACCUMULATE_Y, None)
        assert st == UNSUPPORTED, algo


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 1, 2, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        m2rnn.fwd(x, x, x, torch.zeros((1, 1, 2), dtype=torch.bfloat16),
                  torch.zeros((1, 16, 16), dtype=torch.bfloat16))


def test_varlen_rejects_a_misaligned_length_array():
    lib = m2rnn.load()
    p = 0x10000
    st = lib.m2rnn_fwd_varlen(p, p, p, p, p, None, p, None, p + 2, 2, 2, 16, 64, 64,
                              m2rnn.DTYPES["bf16"], m2rnn.ALGOS["mfma"], 0, None)
    assert st == 1  # M2RNN_ERROR_INVALID_VALUE, before any HIP call
    st = lib.m2rnn_fwd_varlen(None, p, p, p, p, None, p, None, p, 2, 2, 16, 64, 64,
                              m2rnn.DTYPES["bf16"], m2rnn.ALGOS["mfma"], 0, None)
    assert st == 1


def test_checkpoint_and_workspace_sizes():
    B, H, T, K, V = 8, 16, 2048, 128, 128
    kv = B * H * K * V * 4
    assert m2rnn.ckpt_bytes(B, H, T, K, V, 256) == 7 * kv
    assert m2rnn.ckpt_bytes(B, H, T, K, V, 300) == 6 * kv      # ceil(2048 / 300) = 7 segments
    assert m2rnn.ckpt_bytes(B, H, T, K, V, T) == 0
    assert m2rnn.ckpt_bytes(B, H, T, K, V, 10 * T) == 0
    assert m2rnn.ckpt_bytes(B, H, T, K, V, 0) == 0
    # one segment's saved data is what the workspace grows with
    w256 = m2rnn.bwd_recompute_workspace_bytes(B, H, T, K, V, 256)
    wall = m2rnn.bwd_recompute_workspace_bytes(B, H, T, K, V, T)
    assert w256 >= m2rnn.saved_bytes(B, H, 256, K, V) + m2rnn.bwd_workspace_bytes(B, H, 256, K, V)
    assert wall >= m2rnn.saved_bytes(B, H, T, K, V) + m2rnn.bwd_workspace_bytes(B, H, T, K, V)
    assert w256 < wall / 6
    assert m2rnn.bwd_recompute_workspace_bytes(B, H, T, K, V, 10 * T) == wall
    assert m2rnn.bwd_recompute_workspace_bytes(B, H, T, 48, 112, 256) == 0   # not an MFMA shape


def test_recompute_entry_points_validate_before_launching():
    lib = m2rnn.load()
    p = 0x10000
    bf16, auto, simple = m2rnn.DTYPES["bf16"], m2rnn.ALGOS["auto"], m2rnn.ALGOS["simple"]
    fwd = lambda ckpt, seg, algo=auto, dt=bf16: lib.m2rnn_fwd_ckpt(p, p, p, p, p, None, p, None, ckpt,
                                                                   2, 2, 64, 64, 64, seg, dt, algo, None)
    assert fwd(p, 0) == INVALID                 # segment < 1
    assert fwd(None, 16) == INVALID             # four segments need checkpoints
    assert fwd(p + 4, 16) == INVALID            # misaligned checkpoints
    assert fwd(p, 16, algo=simple) == UNSUPPORTED
    assert fwd(p, 16, dt=m2rnn.DTYPES["f32"]) == UNSUPPORTED

    def bwd(ckpt, seg, ws=p, dk=p, algo=auto):
        return lib.m2rnn_bwd_recompute(p, p, p, p, p, None, ckpt, p, None, dk, p, p, p, p, None, ws,
                                       2, 2, 64, 64, 64, seg, bf16, algo, None)
    assert bwd(p, 0) == INVALID
    assert bwd(None, 16) == INVALID
    assert bwd(p, 16, ws=None) == INVALID
    assert bwd(p, 16, dk=None) == INVALID
    assert bwd(p, 16, algo=simple) == UNSUPPORTED


def test_training_forwards_take_the_long_kernel_only_where_the_backward_covers_the_shape():
    """The saving forwards accept MFMA_LONG* (same saved layout), but not for a
    shape the backward pass does not cover (K = 16, V = 96) nor in fp32; all
    refused before any launch."""
    lib = m2rnn.load()
    p = 0x10000
    bf16, f32 = m2rnn.DTYPES["bf16"], m2rnn.DTYPES["f32"]
    for algo in ("mfma_long", "mfma_long_split"):
        a = m2rnn.ALGOS[algo]
        save = lambda K, V, dt=bf16: lib.m2rnn_fwd_save(p, p, p, p, p, None, p, None, p, 2, 2, 16, K, V, dt, a, None)
        assert save(16, 64) == UNSUPPORTED, algo
        assert save(64, 96) == UNSUPPORTED, algo
        assert save(64, 64, f32) == UNSUPPORTED, algo
        ck = lambda K: lib.m2rnn_fwd_ckpt(p, p, p, p, p, None, p, None, p, 2, 2, 64, K, 64, 16, bf16, a, None)
        assert ck(16) == UNSUPPORTED, algo
        rc = lambda K: lib.m2rnn_bwd_recompute(p, p, p, p, p, None, p, p, None, p, p, p, p, p, None, p,
                                               2, 2, 64, K, 64, 16, bf16, a, None)
        assert rc(16) == UNSUPPORTED, algo
        assert lib.m2rnn_fwd_save(None, p, p, p, p, None, p, None, p, 2, 2, 16, 64, 64, bf16, a, None) == INVALID
        bw = lambda K, V, alg=a, dk=p: lib.m2rnn_bwd_algo(p, p, p, p, p, None, p, p, None, dk, p, p, p, p, None, p,
                                                          2, 2, 16, K, V, bf16, alg, None)
        assert bw(16, 64) == UNSUPPORTED, algo
        assert bw(64, 64, dk=None) == INVALID, algo
    for other in ("simple", 6, 99):
        alg = m2rnn.ALGOS[other] if isinstance(other, str) else other
        assert lib.m2rnn_bwd_algo(p, p, p, p, p, None, p, p, None, p, p, p, p, p, None, p, 2, 2, 16, 64, 64, bf16,
                                  alg, None) == UNSUPPORTED, other


def test_frontend_validates_before_launching():
    lib = m2rnn.load()
    p = 0x10000
    bf16 = m2rnn.DTYPES["bf16"]

    def call(x=p, Wx=p, bias=p, k=p, B=2, T=3, D=64, H=2, K=64, V=64, dt=bf16):
        return lib.m2rnn_frontend(x, Wx, bias, k, p, p, p, B, T, D, H, K, V, dt, None)
    assert call(x=None) == INVALID
    assert call(bias=None) == INVALID
    assert call(x=p + 8) == INVALID          # misaligned
    assert call(bias=p + 2) == INVALID
    assert call(B=0) == INVALID
    assert call(D=0) == INVALID
    assert call(D=60) == UNSUPPORTED         # rows of x must be whole 16-byte pieces
    assert call(K=40) == UNSUPPORTED
    assert call(dt=m2rnn.DTYPES["f32"]) == UNSUPPORTED
