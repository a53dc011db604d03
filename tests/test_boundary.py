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
    assert m2rnn.version() == 1000


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
    for code in (0, 1, 2, 3, 4):
        s = m2rnn.status_string(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 5
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
    assert _check(dtype="f32", algo=algo) == UNSUPPORTED          # fp32 inputs: the fp32 kernels
    assert _check(K=16, V=128, algo=algo) == UNSUPPORTED          # fewer than 32 rows
    assert _check(K=96, V=128, algo=algo) == UNSUPPORTED          # more than two row groups
    assert _check(K=128, V=96, algo=algo) == UNSUPPORTED
    for K in (32, 64, 128):
        for V in (64, 128):
            assert _check(K=K, V=V, algo=algo) == OK


def test_mfma_f32_coverage():
    """The fp32 matrix-core family takes fp32 inputs of every supported shape and
    nothing else; it has one fixed y summation order, so AUTO keeps it under
    M2RNN_FLAG_DETERMINISTIC, with or without accumulation."""
    for K in range(16, 129, 16):
        for V in range(16, 129, 16):
            assert _check(dtype="f32", K=K, V=V, algo="mfma_f32") == OK, (K, V)
    assert _check(K=64, V=64, algo="mfma_f32") == UNSUPPORTED     # bf16 inputs
    assert _check(dtype="f32", K=20, V=64, algo="mfma_f32") == UNSUPPORTED
    det, acc = m2rnn.FLAG_DETERMINISTIC, m2rnn.FLAG_ACCUMULATE_Y
    for flags in (det, det | acc):
        assert m2rnn.get_plan(8, 16, 64, 128, 128, "f32", "auto", flags)["algo"] == "mfma_f32"
    assert m2rnn.get_plan(8, 16, 64, 128, 128, "f32", "mfma_f32", det | acc)["algo"] == "mfma_f32"


def test_launch_plans():
    p = m2rnn.get_plan(8, 16, 2048, 128, 128, "bf16", "auto")
    assert p["algo"] == "mfma_f16" and p["grid"] == 256 and p["block"] == 256
    assert p["rows_per_group"] == 64 and p["groups_per_unit"] == 2 and p["clears_y"] == 1
    assert p["lds_bytes"] <= 160 * 1024
    p = m2rnn.get_plan(2, 16, 32768, 64, 128, "bf16", "mfma")
    assert p["grid"] == 32 and p["groups_per_unit"] == 1 and p["clears_y"] == 0
    p = m2rnn.get_plan(1, 1, 64, 16, 16, "f32", "auto")
    assert p["algo"] == "mfma_f32" and p["grid"] == 1 and p["block"] == 64 and p["clears_y"] == 0
    # fp32 on the matrix cores: one workgroup of K/16 waves per unit, LDS within a CU's 160 KiB
    for K in range(16, 129, 16):
        for V in range(16, 129, 16):
            p = m2rnn.get_plan(3, 5, 100, K, V, "f32", "mfma_f32")
            assert p["grid"] == 15 and p["block"] == 4 * K and p["groups_per_unit"] == 1, (K, V)
            assert 0 < p["lds_bytes"] <= 160 * 1024, (K, V)
    assert m2rnn.get_plan(1, 1, 64, 16, 16, "f32", "simple")["algo"] == "simple"
    # the latency-oriented kernel: one workgroup of V/32 waves per 16-row tile
    p = m2rnn.get_plan(1, 32, 8192, 128, 128, "bf16", "mfma_long")
    assert p["grid"] == 32 * 8 and p["block"] == 256 and p["clears_y"] == 1
    assert m2rnn.get_plan(2, 16, 32768, 64, 128, "bf16", "mfma_long_split")["grid"] == 32 * 4
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
    assert m2rnn.pick_algo(8, 16, 2048, 128, 128, "bf16") == "mfma_f16"     # 1024 row tiles
    assert m2rnn.pick_algo(1, 1, 64, 16, 16, "f32") == "mfma_f32"
    assert m2rnn.pick_algo(1, 1, 64, 16, 96, "bf16") == "simple"
    # up to 768 16-row tiles: the latency-oriented kernel
    assert m2rnn.pick_algo(1, 1, 64, 16, 128, "bf16") == "mfma_long_f16"
    assert m2rnn.pick_algo(1, 32, 8192, 128, 128, "bf16") == "mfma_long_f16"
    assert m2rnn.pick_algo(2, 16, 32768, 64, 128, "bf16") == "mfma_long_f16"
    assert m2rnn.pick_algo(4, 8, 512, 64, 64, "bf16") == "mfma_long_f16"
    assert m2rnn.pick_algo(6, 16, 100, 128, 128, "bf16") == "mfma_long_f16"  # 768 tiles
    assert m2rnn.pick_algo(7, 16, 100, 128, 128, "bf16") == "mfma_f16"       # 896 tiles
    assert m2rnn.pick_algo(1, 32, 1, 128, 128, "bf16") == "mfma_f16"         # one step: decoding kernel
    assert m2rnn.pick_algo(1, 4, 64, 32, 64, "f32") == "mfma_f32"
    assert m2rnn.pick_algo(8, 16, 2048, 128, 128, "f32") == "mfma_f32"
    p = m2rnn.get_plan(1, 32, 8192, 128, 128, "bf16", "auto")
    assert p["algo"] == "mfma_long_f16" and p["grid"] == 256 and p["block"] == 256 and p["clears_y"] == 1


def test_decoding_plan():
    """Every T = 1 call on the matrix-core shapes plans the one-step kernel: 256
    threads, two workgroups per CU by LDS (at most 80 KiB each), about 512
    workgroups spread over the heads with at least one batch row each. Host only."""
    p = m2rnn.get_plan(512, 16, 1, 128, 128, "bf16", "auto")
    assert p["block"] == 256 and p["grid"] == 16 * 32 and p["clears_y"] == 0
    assert 0 < p["lds_bytes"] <= 80 * 1024
    for K, V in [(32, 64), (64, 64), (128, 64), (32, 128), (64, 128)]:
        q = m2rnn.get_plan(3, 5, 1, K, V, "bf16", "mfma_split")
        assert q["grid"] == 5 * 3 and q["block"] == 256, (K, V)   # min(B, ceil(512 / H)) rows per head
        assert 0 < q["lds_bytes"] <= 80 * 1024, (K, V)
    assert m2rnn.get_plan(1000, 1, 1, 128, 128, "bf16", "auto")["grid"] == 512


def test_deterministic_flag_and_the_long_kernels():
    """M2RNN_FLAG_DETERMINISTIC: the long kernels round each row tile's readout
    onto a common grid, so their y is repeatable onto the y the call clears (any
    number of row tiles) and they are accepted; adding into the caller's y from
    two or more row tiles is refused before any launch."""
    lib = m2rnn.load()
    det, acc = m2rnn.FLAG_DETERMINISTIC, m2rnn.FLAG_ACCUMULATE_Y
    for algo in ("mfma_long", "mfma_long_split"):
        for K in (16, 64, 128):
            st = lib.m2rnn_check_args(A, A, A, A, A, None, A, None, 1, 2, 16, K, 128, 1, m2rnn.ALGOS[algo])
            assert st == OK
            assert m2rnn.get_plan(1, 2, 16, K, 128, "bf16", algo, det)["algo"] == algo, (algo, K)
        st = lib.m2rnn_fwd_ex(A, A, A, A, A, None, A, None, 1, 2, 16, 64, 128, 1, m2rnn.ALGOS[algo], det | acc, None)
        assert st == UNSUPPORTED, algo
        # one row tile: a single add per element, accumulation included
        assert m2rnn.get_plan(1, 2, 16, 16, 128, "bf16", algo, det | acc)["algo"] == algo


def test_deterministic_auto_resolves_to_a_covering_repeatable_kernel():
    """AUTO under M2RNN_FLAG_DETERMINISTIC keeps its choice unless the call also
    accumulates into y from two or more workgroups: then it takes the multi-step
    kernel with the same operand where that has one workgroup per unit, else the
    simple kernel.
    Host only: the plan query launches nothing."""
    det, acc = m2rnn.FLAG_DETERMINISTIC, m2rnn.FLAG_ACCUMULATE_Y
    # the long kernel stays under the flag alone, for every K
    for K in (16, 32, 48, 64, 80, 96, 112, 128):
        assert m2rnn.get_plan(2, 3, 37, K, 128, "bf16", "auto", det)["algo"] == "mfma_long_f16", K
    assert m2rnn.get_plan(1, 32, 8192, 128, 128, "bf16", "auto", det)["algo"] == "mfma_long_f16"
    # accumulating: the multi-step kernel where it runs one workgroup per unit
    assert m2rnn.get_plan(2, 3, 37, 32, 128, "bf16", "auto", det | acc)["algo"] == "mfma_f16"
    assert m2rnn.get_plan(2, 3, 37, 64, 128, "bf16", "auto", det | acc)["algo"] == "mfma_f16"
    # ... and the simple kernel where it does not cover the shape (K = 48, ...) or
    # runs two workgroups (K = 128); one row tile stays on the long kernel
    for K in (48, 80, 96, 112, 128):
        assert m2rnn.get_plan(2, 3, 37, K, 128, "bf16", "auto", det | acc)["algo"] == "simple", K
    assert m2rnn.get_plan(2, 3, 37, 16, 128, "bf16", "auto", det | acc)["algo"] == "mfma_long_f16"
    # K = 128 on the multi-step kernel: two workgroups add into a cleared y
    assert m2rnn.get_plan(8, 16, 64, 128, 128, "bf16", "auto", det)["algo"] == "mfma_f16"
    assert m2rnn.get_plan(8, 16, 64, 128, 128, "bf16", "auto", det | acc)["algo"] == "simple"
    # without the flag nothing changes
    assert m2rnn.get_plan(2, 3, 37, 48, 128, "bf16", "auto")["algo"] == "mfma_long_f16"
    assert m2rnn.get_plan(8, 16, 64, 128, 128, "bf16", "auto", acc)["algo"] == "mfma_f16"


def test_deterministic_accumulate_refuses_two_atomic_groups():
    """DETERMINISTIC | ACCUMULATE_Y on the multi-step kernels at K = 128 (two
    workgroups add into a y that already holds values, and (y + a) + b need not
    equal (y + b) + a) is refused before any launch; at K = 64 (one workgroup) and
    for one step (the decoding kernel) it is accepted."""
    lib = m2rnn.load()
    det, acc = m2rnn.FLAG_DETERMINISTIC, m2rnn.FLAG_ACCUMULATE_Y
    for algo in ("mfma", "mfma_split"):
        st = lib.m2rnn_fwd_ex(A, A, A, A, A, None, A, None, 2, 2, 40, 128, 128, 1, m2rnn.ALGOS[algo], det | acc,
                              None)
        assert st == UNSUPPORTED, algo
        with pytest.raises(m2rnn.M2RNNError):
            m2rnn.get_plan(2, 2, 40, 128, 128, "bf16", algo, det | acc)
        assert m2rnn.get_plan(2, 2, 40, 64, 128, "bf16", algo, det | acc)["algo"] == algo
        assert m2rnn.get_plan(2, 2, 1, 128, 128, "bf16", algo, det | acc)["algo"] == algo
        assert m2rnn.get_plan(2, 2, 40, 128, 128, "bf16", algo, det)["algo"] == algo
    for algo in ("mfma_long", "mfma_long_split"):
        assert m2rnn.get_plan(2, 2, 40, 48, 128, "bf16", algo, det)["algo"] == algo
        assert m2rnn.get_plan(2, 2, 40, 32, 128, "bf16", algo, det)["algo"] == algo
        with pytest.raises(m2rnn.M2RNNError):
            m2rnn.get_plan(2, 2, 40, 32, 128, "bf16", algo, det | acc)
    # unknown flag bits are refused by the plan query too
    with pytest.raises(m2rnn.M2RNNError):
        m2rnn.get_plan(2, 2, 40, 64, 128, "bf16", "auto", 4)


def test_noalloc_backward_refuses_a_shape_beyond_its_array():
    """m2rnn_bwd_noalloc: a workspace above the library's 64 MiB array is refused
    with its own status before any HIP call; invalid arguments keep the usual
    codes."""
    lib = m2rnn.load()
    bf, auto = m2rnn.DTYPES["bf16"], m2rnn.ALGOS["auto"]
    B, H, T, K, V = 8, 16, 2048, 128, 128
    assert m2rnn.bwd_workspace_bytes(B, H, T, K, V) > 64 << 20
    st = lib.m2rnn_bwd_noalloc(A, A, A, A, A, None, A, A, None, A, A, A, A, A, None, B, H, T, K, V, bf, auto, None)
    assert st == 4 and "scratch" in m2rnn.status_string(st)
    st = lib.m2rnn_bwd_noalloc(A, A, A, A, A, None, None, A, None, A, A, A, A, A, None, 1, 2, 40, 64, 128, bf,
                               auto, None)
    assert st == INVALID  # no saved buffer
    st = lib.m2rnn_bwd_noalloc(A, A, A, A, A, None, A, A, None, A, A, A, A, A, None, 1, 2, 40, 48, 128, bf,
                               m2rnn.ALGOS["mfma"], None)
    assert st == UNSUPPORTED  # K = 48 has no backward kernel


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
    for other in ("simple", "mfma_f32", 99):
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


def test_f16_operand_families():
    """MFMA_F16 covers the multi-step kernel's shapes and MFMA_LONG_F16 the long
    kernel's (bf16 inputs only); with the deterministic flag and accumulation AUTO
    never resolves to them, a deterministic call keeps them where their y adds are
    order-free and refuses them where two or more row groups would add into the
    caller's y; no training entry point takes them. All host-side, before any
    launch."""
    lib = m2rnn.load()
    p = 0x10000
    bf16, f32 = m2rnn.DTYPES["bf16"], m2rnn.DTYPES["f32"]
    det, acc = m2rnn.FLAG_DETERMINISTIC, m2rnn.FLAG_ACCUMULATE_Y
    for K in (32, 64, 128):
        for V in (64, 128):
            assert _check(K=K, V=V, algo="mfma_f16") == OK
    assert _check(K=16, V=128, algo="mfma_f16") == UNSUPPORTED
    assert _check(dtype="f32", algo="mfma_f16") == UNSUPPORTED
    for K in (16, 48, 128):
        assert _check(K=K, V=128, algo="mfma_long_f16") == OK
    assert _check(K=64, V=96, algo="mfma_long_f16") == UNSUPPORTED
    assert _check(dtype="f32", algo="mfma_long_f16") == UNSUPPORTED
    # plans: the kernels of the bf16 single-operand families
    for algo, ref in (("mfma_f16", "mfma"), ("mfma_long_f16", "mfma_long")):
        a, b = m2rnn.get_plan(8, 16, 2048, 128, 128, "bf16", algo), m2rnn.get_plan(8, 16, 2048, 128, 128, "bf16", ref)
        assert a["algo"] == algo and {k: v for k, v in a.items() if k != "algo"} == \
            {k: v for k, v in b.items() if k != "algo"}
        assert m2rnn.get_plan(8, 16, 64, 128, 128, "bf16", algo, det)["algo"] == algo
    # deterministic + accumulate: two workgroups (K = 128) or several row tiles refused
    with pytest.raises(m2rnn.M2RNNError):
        m2rnn.get_plan(2, 2, 40, 128, 128, "bf16", "mfma_f16", det | acc)
    with pytest.raises(m2rnn.M2RNNError):
        m2rnn.get_plan(2, 2, 40, 32, 128, "bf16", "mfma_long_f16", det | acc)
    assert m2rnn.get_plan(2, 2, 40, 64, 128, "bf16", "mfma_f16", det | acc)["algo"] == "mfma_f16"
    # the training forwards and the backward pass refuse them
    for algo in ("mfma_f16", "mfma_long_f16"):
        a = m2rnn.ALGOS[algo]
        assert lib.m2rnn_fwd_save(p, p, p, p, p, None, p, None, p, 2, 2, 16, 64, 64, bf16, a, None) == UNSUPPORTED
        assert lib.m2rnn_fwd_ckpt(p, p, p, p, p, None, p, None, p, 2, 2, 64, 64, 64, 16, bf16, a, None) == UNSUPPORTED
        assert lib.m2rnn_bwd_recompute(p, p, p, p, p, None, p, p, None, p, p, p, p, p, None, p,
                                       2, 2, 64, 64, 64, 16, bf16, a, None) == UNSUPPORTED
        assert lib.m2rnn_bwd_algo(p, p, p, p, p, None, p, p, None, p, p, p, p, p, None, p, 2, 2, 16, 64, 64, bf16,
                                  a, None) == UNSUPPORTED
        assert lib.m2rnn_fwd_save(p, p, p, p, p, None, p, None, p, 2, 2, 16, 64, 64, f32, a, None) == UNSUPPORTED
