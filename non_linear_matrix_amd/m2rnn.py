"""Python binding of libm2rnn.so (ctypes). Argument marshalling only.

Every step of the recurrence runs in the library's HIP kernels; PyTorch is used
here for device buffers and the current stream. If the library is not built,
every call raises — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "LIB_PATH", "M2RNNError", "load", "fwd", "check_args", "pick_algo", "status_string", "version",
    "fwd_save", "bwd", "bwd_noalloc", "saved_bytes", "bwd_workspace_bytes",
    "STATUS", "ALGOS", "DTYPES", "declared_functions", "get_plan", "Plan", "FLAG_ACCUMULATE_Y",
    "FLAG_DETERMINISTIC",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libm2rnn.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "m2rnn.h")

STATUS = {0: "M2RNN_SUCCESS", 1: "M2RNN_ERROR_INVALID_VALUE", 2: "M2RNN_ERROR_NOT_SUPPORTED", 3: "M2RNN_ERROR_LAUNCH",
          4: "M2RNN_ERROR_SCRATCH_TOO_SMALL"}
ALGOS = {"auto": 0, "simple": 1, "mfma": 2, "mfma_split": 3, "mfma_long": 4, "mfma_long_split": 5,
         "mfma_f32": 6, "mfma_f16": 7, "mfma_long_f16": 8}
DTYPES = {"f32": 0, "bf16": 1}
FLAG_ACCUMULATE_Y = 1
FLAG_DETERMINISTIC = 2

_lib = None


class Plan(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int), ("grid", ctypes.c_int), ("block", ctypes.c_int),
                ("rows_per_group", ctypes.c_int), ("groups_per_unit", ctypes.c_int),
                ("clears_y", ctypes.c_int), ("lds_bytes", ctypes.c_int)]


def get_plan(B: int, H: int, T: int, K: int, V: int, dtype: str, algo: str = "auto", flags: int = 0) -> dict:
    """The launch plan the library would use (host only); `flags` as m2rnn_fwd_ex's."""
    p = Plan()
    st = load().m2rnn_get_plan_ex(B, H, T, K, V, DTYPES[dtype], ALGOS[algo], flags, ctypes.byref(p))
    if st != 0:
        raise M2RNNError(st, "m2rnn_get_plan_ex")
    d = {name: getattr(p, name) for name, _ in Plan._fields_}
    d["algo"] = {v: k for k, v in ALGOS.items()}[d["algo"]]
    return d


class M2RNNError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


def load() -> ctypes.CDLL:
    """Load libm2rnn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m non_linear_matrix_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, fp, i = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int
    lib.m2rnn_fwd.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, vp]
    lib.m2rnn_fwd.restype = i
    lib.m2rnn_fwd_algo.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, i, vp]
    lib.m2rnn_fwd_algo.restype = i
    lib.m2rnn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, i, ctypes.c_uint, vp]
    lib.m2rnn_fwd_ex.restype = i
    lib.m2rnn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, vp, i, i, i, i, i, i, i, ctypes.c_uint, vp]
    lib.m2rnn_fwd_varlen.restype = i
    lib.m2rnn_check_args.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, i]
    lib.m2rnn_check_args.restype = i
    lib.m2rnn_pick_algo.argtypes = [i, i, i, i, i, i]
    lib.m2rnn_pick_algo.restype = i
    lib.m2rnn_status_string.argtypes = [i]
    lib.m2rnn_status_string.restype = ctypes.c_char_p
    lib.m2rnn_get_plan.argtypes = [i, i, i, i, i, i, i, ctypes.POINTER(Plan)]
    lib.m2rnn_get_plan.restype = i
    lib.m2rnn_get_plan_ex.argtypes = [i, i, i, i, i, i, i, ctypes.c_uint, ctypes.POINTER(Plan)]
    lib.m2rnn_get_plan_ex.restype = i
    u64 = ctypes.c_ulonglong
    lib.m2rnn_saved_bytes.argtypes = [i, i, i, i, i]
    lib.m2rnn_saved_bytes.restype = u64
    lib.m2rnn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.m2rnn_bwd_workspace_bytes.restype = u64
    lib.m2rnn_fwd_save.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, vp, i, i, i, i, i, i, i, vp]
    lib.m2rnn_fwd_save.restype = i
    lib.m2rnn_bwd.argtypes = [vp, vp, vp, vp, vp, fp, vp, fp, fp, fp, fp, fp, fp, fp, fp, vp,
                              i, i, i, i, i, i, vp]
    lib.m2rnn_bwd.restype = i
    lib.m2rnn_bwd_algo.argtypes = lib.m2rnn_bwd.argtypes[:-1] + [i, vp]
    lib.m2rnn_bwd_algo.restype = i
    lib.m2rnn_bwd_noalloc.argtypes = lib.m2rnn_bwd.argtypes[:15] + [i, i, i, i, i, i, i, vp]
    lib.m2rnn_bwd_noalloc.restype = i
    lib.m2rnn_frontend.argtypes = [vp, vp, fp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.m2rnn_frontend.restype = i
    lib.m2rnn_ckpt_bytes.argtypes = [i, i, i, i, i, i]
    lib.m2rnn_ckpt_bytes.restype = u64
    lib.m2rnn_fwd_ckpt.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, fp, i, i, i, i, i, i, i, i, vp]
    lib.m2rnn_fwd_ckpt.restype = i
    lib.m2rnn_bwd_recompute_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.m2rnn_bwd_recompute_workspace_bytes.restype = u64
    lib.m2rnn_bwd_recompute.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp, vp,
                                        i, i, i, i, i, i, i, i, vp]
    lib.m2rnn_bwd_recompute.restype = i
    lib.m2rnn_version.argtypes = []
    lib.m2rnn_version.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().m2rnn_status_string(int(status)).decode()


def version() -> int:
    return int(load().m2rnn_version())


def pick_algo(B: int, H: int, T: int, K: int, V: int, dtype: str) -> str:
    code = load().m2rnn_pick_algo(B, H, T, K, V, DTYPES[dtype])
    return {v: k for k, v in ALGOS.items()}[code]


def check_args(k, v, q, f, W, H0, y, H_T, B, H, T, K, V, dtype, algo="auto") -> int:
    """Host-only validation on raw addresses (ints or None); returns the status code."""
    return int(load().m2rnn_check_args(k, v, q, f, W, H0, y, H_T, B, H, T, K, V,
                                       DTYPES.get(dtype, dtype) if isinstance(dtype, str) else dtype,
                                       ALGOS.get(algo, algo) if isinstance(algo, str) else algo))


def declared_functions() -> list:
    """Names of the functions include/m2rnn.h declares."""
    import re
    with open(HEADER_PATH) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(m2rnn_\w+)\s*\(", text)))


def fwd(k, v, q, f, W, H0=None, *, y=None, H_T=None, seq_len=None, algo: str = "auto", stream=None,
        want_state: bool = True, accumulate_y: bool = False,
        deterministic: bool = False) -> Tuple["object", Optional["object"]]:
    """Run the forward recurrence on torch device tensors.

    k, q [B,H,T,K]; v [B,H,T,V]; f [B,H,T]; W [H,V,V] — all torch.bfloat16 or all
    torch.float32; H0 [B,H,K,V] float32 or None. y / H_T may be given (float32,
    contiguous) to write into; otherwise they are allocated with torch.
    seq_len: optional int32 device tensor [B] of per-sequence lengths
    (m2rnn_fwd_varlen); H_T may then be H0 itself for in-place continuation.
    Returns (y, H_T) (H_T is None when want_state is False and none was given).
    accumulate_y adds the readout into the given y (M2RNN_FLAG_ACCUMULATE_Y);
    deterministic asks for bitwise repeatable outputs (M2RNN_FLAG_DETERMINISTIC).
    """
    import torch

    lib = load()
    if k.dtype == torch.bfloat16:
        dt = DTYPES["bf16"]
    elif k.dtype == torch.float32:
        dt = DTYPES["f32"]
    else:
        raise TypeError(f"unsupported input dtype {k.dtype}")
    for name, t in (("v", v), ("q", q), ("f", f), ("W", W)):
        if t.dtype != k.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {k.dtype}")
    tensors = [k, v, q, f, W] + [t for t in (H0, y, H_T, seq_len) if t is not None]
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    if k.dim() != 4 or v.dim() != 4 or q.shape != k.shape or f.dim() != 3 or W.dim() != 3:
        raise ValueError("expected k,q [B,H,T,K], v [B,H,T,V], f [B,H,T], W [H,V,V]")
    B, H, T, K = k.shape
    V = v.shape[-1]
    if tuple(v.shape) != (B, H, T, V) or tuple(f.shape) != (B, H, T) or tuple(W.shape) != (H, V, V):
        raise ValueError("inconsistent shapes")
    if H0 is not None and (H0.dtype != torch.float32 or tuple(H0.shape) != (B, H, K, V)):
        raise ValueError("H0 must be float32 [B,H,K,V]")
    if seq_len is not None and (seq_len.dtype != torch.int32 or tuple(seq_len.shape) != (B,)):
        raise ValueError("seq_len must be int32 [B]")
    if accumulate_y and y is None:
        raise ValueError("accumulate_y needs y")
    if y is None:
        y = torch.empty((B, H, T, V), dtype=torch.float32, device=k.device)
    elif y.dtype != torch.float32 or tuple(y.shape) != (B, H, T, V):
        raise ValueError("y must be float32 [B,H,T,V]")
    if H_T is None and want_state:
        H_T = torch.empty((B, H, K, V), dtype=torch.float32, device=k.device)
    elif H_T is not None and (H_T.dtype != torch.float32 or tuple(H_T.shape) != (B, H, K, V)):
        raise ValueError("H_T must be float32 [B,H,K,V]")
    if stream is None:
        stream = torch.cuda.current_stream(k.device)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.m2rnn_fwd_varlen(ptr(k), ptr(v), ptr(q), ptr(f), ptr(W), ptr(H0), ptr(y), ptr(H_T),
                              ptr(seq_len), B, H, T, K, V, dt, ALGOS[algo],
                              (FLAG_ACCUMULATE_Y if accumulate_y else 0)
                              | (FLAG_DETERMINISTIC if deterministic else 0), stream.cuda_stream)
    if st != 0:
        raise M2RNNError(st, "m2rnn_fwd")
    return y, H_T


def saved_bytes(B: int, H: int, T: int, K: int, V: int) -> int:
    """Size of the training forward's saved buffer (0: shape not covered)."""
    return int(load().m2rnn_saved_bytes(B, H, T, K, V))


def bwd_workspace_bytes(B: int, H: int, T: int, K: int, V: int) -> int:
    return int(load().m2rnn_bwd_workspace_bytes(B, H, T, K, V))


def fwd_save(k, v, q, f, W, H0=None, *, saved=None, y=None, H_T=None, algo: str = "auto", stream=None):
    """Training forward (m2rnn_fwd_save) on bf16 device tensors: returns
    (y, H_T, saved), saved being the uint8 device buffer m2rnn_bwd reads (pass
    saved / y / H_T to reuse buffers)."""
    import torch

    lib = load()
    B, H, T, K = k.shape
    V = v.shape[-1]
    for t in [k, v, q, f, W] + ([H0] if H0 is not None else []):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    if k.dtype != torch.bfloat16:
        raise TypeError("the training path takes bf16 inputs")
    nbytes = saved_bytes(B, H, T, K, V)
    if nbytes == 0:
        raise M2RNNError(2, "m2rnn_saved_bytes")
    if saved is None:
        saved = torch.empty(nbytes, dtype=torch.uint8, device=k.device)
    elif saved.numel() < nbytes or not saved.is_cuda:
        raise ValueError(f"saved must be a device buffer of at least {nbytes} bytes")
    y = torch.empty((B, H, T, V), dtype=torch.float32, device=k.device) if y is None else y
    HT = torch.empty((B, H, K, V), dtype=torch.float32, device=k.device) if H_T is None else H_T
    if stream is None:
        stream = torch.cuda.current_stream(k.device)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.m2rnn_fwd_save(ptr(k), ptr(v), ptr(q), ptr(f), ptr(W), ptr(H0), ptr(y), ptr(HT), ptr(saved),
                            B, H, T, K, V, DTYPES["bf16"], ALGOS[algo], stream.cuda_stream)
    if st != 0:
        raise M2RNNError(st, "m2rnn_fwd_save")
    return y, HT, saved


def _grad_buffers(B, H, T, K, V, dev, want_dH0):
    import torch

    return {
        "dk": torch.empty((B, H, T, K), dtype=torch.float32, device=dev),
        "dq": torch.empty((B, H, T, K), dtype=torch.float32, device=dev),
        "dv": torch.empty((B, H, T, V), dtype=torch.float32, device=dev),
        "df": torch.empty((B, H, T), dtype=torch.float32, device=dev),
        "dW": torch.empty((H, V, V), dtype=torch.float32, device=dev),
        "dH0": torch.empty((B, H, K, V), dtype=torch.float32, device=dev) if want_dH0 else None,
    }


def _check_dy(dy, dH_T, B, H, T, K, V):
    import torch

    if dy.dtype != torch.float32 or tuple(dy.shape) != (B, H, T, V) or not dy.is_contiguous():
        raise ValueError("dy must be contiguous float32 [B,H,T,V]")
    if dH_T is not None and (dH_T.dtype != torch.float32 or tuple(dH_T.shape) != (B, H, K, V)
                             or not dH_T.is_contiguous()):
        raise ValueError("dH_T must be contiguous float32 [B,H,K,V]")


def bwd(k, v, q, f, W, H0, saved, dy, dH_T=None, *, want_dH0: bool = True, out=None, workspace=None,
        stream=None, algo: str = "auto") -> dict:
    """Backward pass (m2rnn_bwd_algo): gradients dk, dv, dq, df, dW, dH0 (fp32).
    `out` (a dict as returned) and `workspace` may be passed to reuse buffers;
    algo picks the reverse kernel family (any forward's `saved` is accepted)."""
    import torch

    lib = load()
    B, H, T, K = k.shape
    V = v.shape[-1]
    dev = k.device
    _check_dy(dy, dH_T, B, H, T, K, V)
    if out is None:
        out = _grad_buffers(B, H, T, K, V, dev, want_dH0)
    need = max(bwd_workspace_bytes(B, H, T, K, V), 16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if workspace is None else workspace
    if ws.numel() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.m2rnn_bwd_algo(ptr(k), ptr(v), ptr(q), ptr(f), ptr(W), ptr(H0), ptr(saved), ptr(dy), ptr(dH_T),
                            ptr(out["dk"]), ptr(out["dv"]), ptr(out["dq"]), ptr(out["df"]), ptr(out["dW"]),
                            ptr(out["dH0"]), ptr(ws), B, H, T, K, V, DTYPES["bf16"], ALGOS[algo],
                            stream.cuda_stream)
    if st != 0:
        raise M2RNNError(st, "m2rnn_bwd_algo")
    out["workspace"] = ws  # keep alive until the stream has run
    return out


def bwd_noalloc(k, v, q, f, W, H0, saved, dy, dH_T=None, *, want_dH0: bool = True, out=None, stream=None,
                algo: str = "auto") -> dict:
    """Backward pass with the library's own workspace (m2rnn_bwd_noalloc): as
    bwd(), for shapes whose workspace fits the library's 64 MiB array."""
    import torch

    lib = load()
    B, H, T, K = k.shape
    V = v.shape[-1]
    _check_dy(dy, dH_T, B, H, T, K, V)
    if out is None:
        out = _grad_buffers(B, H, T, K, V, k.device, want_dH0)
    if stream is None:
        stream = torch.cuda.current_stream(k.device)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.m2rnn_bwd_noalloc(ptr(k), ptr(v), ptr(q), ptr(f), ptr(W), ptr(H0), ptr(saved), ptr(dy), ptr(dH_T),
                               ptr(out["dk"]), ptr(out["dv"]), ptr(out["dq"]), ptr(out["df"]), ptr(out["dW"]),
                               ptr(out["dH0"]), B, H, T, K, V, DTYPES["bf16"], ALGOS[algo], stream.cuda_stream)
    if st != 0:
        raise M2RNNError(st, "m2rnn_bwd_noalloc")
    return out


def ckpt_bytes(B: int, H: int, T: int, K: int, V: int, segment: int) -> int:
    """Size of the checkpoint buffer of m2rnn_fwd_ckpt (0: none needed)."""
    return int(load().m2rnn_ckpt_bytes(B, H, T, K, V, segment))


def bwd_recompute_workspace_bytes(B: int, H: int, T: int, K: int, V: int, segment: int) -> int:
    return int(load().m2rnn_bwd_recompute_workspace_bytes(B, H, T, K, V, segment))


def fwd_ckpt(k, v, q, f, W, H0=None, *, segment: int, ckpt=None, y=None, H_T=None, algo: str = "auto",
             stream=None):
    """Training forward with checkpoints every `segment` steps (m2rnn_fwd_ckpt) on
    bf16 device tensors: returns (y, H_T, ckpt), ckpt a float32 device tensor
    [nseg - 1, B, H, K, V] (None when there is a single segment)."""
    import torch

    lib = load()
    B, H, T, K = k.shape
    V = v.shape[-1]
    for t in [k, v, q, f, W] + ([H0] if H0 is not None else []):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    if k.dtype != torch.bfloat16:
        raise TypeError("the training path takes bf16 inputs")
    nbytes = ckpt_bytes(B, H, T, K, V, segment)
    if ckpt is None and nbytes > 0:
        ckpt = torch.empty((nbytes // (4 * B * H * K * V), B, H, K, V), dtype=torch.float32, device=k.device)
    if ckpt is not None and ckpt.numel() * 4 < nbytes:
        raise ValueError(f"ckpt must hold {nbytes} bytes")
    y = torch.empty((B, H, T, V), dtype=torch.float32, device=k.device) if y is None else y
    HT = torch.empty((B, H, K, V), dtype=torch.float32, device=k.device) if H_T is None else H_T
    if stream is None:
        stream = torch.cuda.current_stream(k.device)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.m2rnn_fwd_ckpt(ptr(k), ptr(v), ptr(q), ptr(f), ptr(W), ptr(H0), ptr(y), ptr(HT), ptr(ckpt),
                            B, H, T, K, V, segment, DTYPES["bf16"], ALGOS[algo], stream.cuda_stream)
    if st != 0:
        raise M2RNNError(st, "m2rnn_fwd_ckpt")
    return y, HT, ckpt


def bwd_recompute(k, v, q, f, W, H0, ckpt, dy, dH_T=None, *, segment: int, algo: str = "auto",
                  want_dH0: bool = True, out=None, workspace=None, stream=None) -> dict:
    """Backward pass from checkpoints (m2rnn_bwd_recompute): recomputes each
    segment's states, then its gradients. Returns the dict of bwd()."""
    import torch

    lib = load()
    B, H, T, K = k.shape
    V = v.shape[-1]
    dev = k.device
    _check_dy(dy, dH_T, B, H, T, K, V)
    if ckpt_bytes(B, H, T, K, V, segment) > 0 and (ckpt is None or not ckpt.is_cuda):
        raise ValueError("ckpt from fwd_ckpt is required for more than one segment")
    if out is None:
        out = _grad_buffers(B, H, T, K, V, dev, want_dH0)
    need = bwd_recompute_workspace_bytes(B, H, T, K, V, segment)
    if need == 0:
        raise M2RNNError(2, "m2rnn_bwd_recompute_workspace_bytes")
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if workspace is None else workspace
    if ws.numel() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ptr = lambda t: None if t is None else t.data_ptr()
    st = lib.m2rnn_bwd_recompute(ptr(k), ptr(v), ptr(q), ptr(f), ptr(W), ptr(H0), ptr(ckpt), ptr(dy), ptr(dH_T),
                                 ptr(out["dk"]), ptr(out["dv"]), ptr(out["dq"]), ptr(out["df"]), ptr(out["dW"]),
                                 ptr(out["dH0"]), ptr(ws), B, H, T, K, V, segment, DTYPES["bf16"], ALGOS[algo],
                                 stream.cuda_stream)
    if st != 0:
        raise M2RNNError(st, "m2rnn_bwd_recompute")
    out["workspace"] = ws
    return out


def frontend(x, Wx, bias, *, K: int, V: int, out=None, stream=None) -> dict:
    """Layer front-end (m2rnn_frontend): x [B,T,D] bf16, Wx [H, 2K+V+1, D] bf16,
    bias [H] float32, all on the device. Returns dict(k, v, q, f) of bf16 device
    tensors in the recurrence's layouts (pass `out`, a dict of the same, to reuse)."""
    import torch

    lib = load()
    B, T, D = x.shape
    H, R, D2 = Wx.shape
    if D2 != D or R != 2 * K + V + 1 or tuple(bias.shape) != (H,):
        raise ValueError("inconsistent shapes")
    for t in (x, Wx, bias):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("x, Wx and bias must be contiguous device tensors")
    if x.dtype != torch.bfloat16 or Wx.dtype != torch.bfloat16 or bias.dtype != torch.float32:
        raise TypeError("x and Wx take bf16, bias float32")
    dev = x.device
    if out is None:
        out = {
            "k": torch.empty((B, H, T, K), dtype=torch.bfloat16, device=dev),
            "v": torch.empty((B, H, T, V), dtype=torch.bfloat16, device=dev),
            "q": torch.empty((B, H, T, K), dtype=torch.bfloat16, device=dev),
            "f": torch.empty((B, H, T), dtype=torch.bfloat16, device=dev),
        }
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    st = lib.m2rnn_frontend(x.data_ptr(), Wx.data_ptr(), bias.data_ptr(), out["k"].data_ptr(), out["v"].data_ptr(),
                            out["q"].data_ptr(), out["f"].data_ptr(), B, T, D, H, K, V, DTYPES["bf16"],
                            stream.cuda_stream)
    if st != 0:
        raise M2RNNError(st, "m2rnn_frontend")
    return out
