"""Build the HIP library libm2rnn.so in-tree for gfx950 (hipcc, no GPU needed).

    python -m non_linear_matrix_amd.build

Each source compiles to its own object in `_build/` (in parallel), then one
link makes the shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libm2rnn.so")
OBJDIR = os.path.join(ROOT, "_build")
SOURCES = ["m2rnn_api.cpp", "m2rnn_simple.hip", "m2rnn_mfma.hip", "m2rnn_bwd.hip", "m2rnn_ckpt.cpp",
           "m2rnn_frontend.hip", "m2rnn_decode.hip", "m2rnn_long.hip", "m2rnn_bwd_long.hip", "m2rnn_noalloc.hip",
           "m2rnn_f32.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17",
            # packed fp32 VALU forms are kept out of the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results land in arch VGPRs, where the fused epilogue reads them
            "-mllvm", "-amdgpu-mfma-vgpr-form"]


def run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)


def compile_command(src: str, obj: str) -> list:
    return [hipcc()] + flags() + ["-fPIC", "-c", "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", obj]


def command(out: str) -> list:
    """One-step build of the whole library (the same flags as the per-object build)."""
    return ([hipcc()] + flags() + ["-fPIC", "-shared", "-I", INCLUDE, "-I", CSRC]
            + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out])


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(lambda so: run(compile_command(*so), verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
