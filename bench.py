"""Benchmark of the M²RNN forward recurrence on one MI355X.

One step = one full forward call over the whole workload batch (every
(batch, head) unit, every time step), inputs already resident in HBM. Default
workload: B=8, H=16, K=V=128, T=2048, bf16 inputs with an fp32 state (the
K=V=128 configuration the headline metric is quoted on).

Prints ONE JSON line (rank 0). Usage:
    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload C3] [--algo mfma_f16]

Every workload runs the library's automatic choice of kernel family (on this
one "mfma_f16": the fp32 state enters the matrix product as one fp16 operand
per step, within the 2e-2 bound on every unit of every workload, which the GPU
parity tests check); any family can be timed with --algo. The GPU's clock ramps over the first tens of
milliseconds of work, hence an untimed settling phase of at least 100 ms (its
call count is in the JSON line) before the W warmup and K timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # MI355X dense matrix-core peaks
HBM_PEAK_GBS = 8000.0                            # MI355X HBM3E
METRIC = "M2RNN fwd tokens·heads/sec + MFMA util % at K=V=128, 1×MI355X"

# HBM bytes per launch of the recurrence kernel: rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads for a
# plain 1 GiB device copy (bench.py --copy-calibration 1024: FETCH_SIZE reads
# half the copied bytes, WRITE_SIZE all of them). A reading holds only for the
# kernel source it was taken on; for any other source the traffic is unknown.
COUNTER_SCALE = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
TRAFFIC_KIB = {
    # (workload, algo): (FETCH_SIZE KiB, WRITE_SIZE KiB, kernel source, its sha256)
    ("C3", "mfma_f16"): (136562.8, 270336.0, "m2rnn_mfma.hip",
                         "c0221ee00f30a9a0fcd443891b9b410f7f841bd197bebde88055a087d4980c0c"),
    ("D1", "decode"): (267349.0, 528389.4, "m2rnn_decode.hip",
                       "d6f09bfc7c21aa0dc4fc5e513ca60a152b47059c85446459709af8e502678a47"),
    ("C4", "mfma_long_f16"): (669879.5, 1050624.0, "m2rnn_long.hip",
                              "044752d9671f142c0c248f310f8d9d597aba91fc478870a0af20264645e9a3f1"),
    ("C5", "mfma_long_f16"): (1053879.0, 2098176.0, "m2rnn_long.hip",
                              "044752d9671f142c0c248f310f8d9d597aba91fc478870a0af20264645e9a3f1"),
}
CSRC = os.path.join(ROOT, "non_linear_matrix_amd", "csrc")
# the save-mode backward call on C3 (reverse kernel + dW partials + dW reduce), the
# same counters summed over its kernels, and the source they were taken on
TRAIN_TRAFFIC_KIB = (8661945.0 + 8388671.6 + 32785.5, 9709579.4 + 65544.6 + 1024.0, "m2rnn_bwd.hip",
                     "af64cdf526e2745dd3c68adcecdd0c404bfbd190a5fcb7efdc093b1afaa2e255")


def measured_traffic(workload, algo):
    import hashlib

    rec = TRAIN_TRAFFIC_KIB if (workload, algo) == ("C3", "train") else TRAFFIC_KIB.get((workload, algo))
    if rec is None:
        return None
    src = os.path.join(CSRC, rec[2])
    if not os.path.exists(src):
        return None
    with open(src, "rb") as fh:
        if hashlib.sha256(fh.read()).hexdigest() != rec[3]:
            return None
    return 1024.0 * (rec[0] * COUNTER_SCALE["FETCH_SIZE"] + rec[1] * COUNTER_SCALE["WRITE_SIZE"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C3",
                    help="C1..C5 (the parity configurations), D1 (one decoding step, state in place) "
                         "or R1 (C3's shape with ragged lengths)")
    ap.add_argument("--algo", default=None,
                    help="kernel family; default: the library's automatic choice (mfma_f16 on C3)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time for the oracle baseline sample (0 disables)")
    ap.add_argument("--train", action="store_true",
                    help="time the training step instead: m2rnn_fwd_save then m2rnn_bwd (bf16 workloads)")
    ap.add_argument("--frontend", action="store_true",
                    help="time the layer front-end (projections of x and the gate) and the front-end + "
                         "recurrence forward instead")
    ap.add_argument("--segment", type=int, default=256,
                    help="--train: steps per segment of the recomputing training mode")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (a few times) and exit: "
                         "the reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return ap.parse_args()


SETTLE_MS = 100.0  # untimed work before the warmup steps: the GPU clock ramps over ~tens of ms


def settle(fn, min_ms=SETTLE_MS, max_calls=20000):
    """Run fn (one untimed step) until min_ms of wall time has passed, so that the
    timed steps run at the settled clock whatever the step length; returns the
    number of calls. Short steps need it (a 0.25 ms decoding step measured 10%
    slower after 10 warmup steps than after 400); long ones are past it after a
    few steps."""
    import torch

    n, t0 = 0, time.perf_counter()
    while n < max_calls:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= min_ms:
                break
    torch.cuda.synchronize()
    return n


def copy_calibration(mib, reps=3):
    """A plain copy of known size: under rocprofv3 --pmc its FETCH_SIZE and
    WRITE_SIZE per dispatch, divided by mib * 1024 KiB, give the counter's scale."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst[-4:], src[-4:])
    print(json.dumps({"copy_calibration_bytes": n * 4, "dispatches": reps}), flush=True)


def cpu_baseline(cfg, x, budget_s):
    """The fp64 oracle as it stands, on all units of the workload for a bounded
    number of leading steps; throughput in tokens*heads/s (linear in T)."""
    import numpy as np
    from oracle import m2rnn_fwd_ref

    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=None)
    except Exception:
        pass

    def run(ts):
        sub = {k: (None if v is None else (v[:, :, :ts] if k in ("k", "v", "q", "f") else v)) for k, v in x.items()}
        t0 = time.perf_counter()
        m2rnn_fwd_ref(sub["k"], sub["v"], sub["q"], sub["f"], sub["W"], sub["H0"], dtype=cfg.dtype)
        return time.perf_counter() - t0

    probe = min(8, cfg.T)
    dt = run(probe)
    ts = int(min(cfg.T, max(probe, probe * budget_s / max(dt, 1e-6))))
    dt = run(ts)
    out = {
        "value": cfg.B * cfg.H * ts / dt,
        "unit": "tok·heads/s",
        "cores": threads if threads else os.cpu_count(),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle, all {cfg.B * cfg.H} (b,h) units of {cfg.name}, first {ts} of {cfg.T} steps "
                  f"({dt:.1f}s); matmul on OpenBLAS threads, elementwise single-threaded",
        "cpu_model": cpu_model(),
    }
    # the same oracle held to one thread, on a quarter of the budget
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            d1 = run(probe)
            t1 = int(min(cfg.T, max(probe, probe * budget_s / 4 / max(d1, 1e-6))))
            d1 = run(t1)
        out["single_thread_value"] = cfg.B * cfg.H * t1 / d1
        out["single_thread_sample"] = f"first {t1} of {cfg.T} steps ({d1:.1f}s), one thread"
    except Exception:
        pass
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


TRAIN_METRIC = "M2RNN training step (fwd_save + bwd) tokens·heads/sec at K=V=128, 1×MI355X"


def cpu_baseline_train(cfg, x, dy, budget_s):
    """The fp64 gradient oracle (forward included) on all units for a bounded
    number of leading steps; tokens*heads/s of whole training steps."""
    from oracle import m2rnn_bwd_ref

    def run(ts):
        sub = {k: (None if v is None else (v[:, :, :ts] if k in ("k", "v", "q", "f") else v)) for k, v in x.items()}
        t0 = time.perf_counter()
        m2rnn_bwd_ref(sub["k"], sub["v"], sub["q"], sub["f"], sub["W"], sub["H0"], dy[:, :, :ts], dtype=cfg.dtype)
        return time.perf_counter() - t0

    probe = min(4, cfg.T)
    dt = run(probe)
    # the oracle keeps every state and tanh output in fp64: at most 256 steps
    ts = int(min(cfg.T, 256, max(probe, probe * budget_s / max(dt, 1e-6))))
    dt = run(ts)
    return {
        "value": cfg.B * cfg.H * ts / dt,
        "unit": "tok·heads/s",
        "cores": os.cpu_count(),
        "kind": "oracle",
        "sample": f"fp64 numpy gradient oracle (forward + backward), all {cfg.B * cfg.H} (b,h) units of "
                  f"{cfg.name}, first {ts} of {cfg.T} steps ({dt:.1f}s)",
    }


def train_bench(args, cfg, dev, x):
    """Times whole training steps, in the two ways the library offers, with
    output gradients dy (no gradient on the final state):
      save:      m2rnn_fwd_save (every step's state and pre-activation kept),
                 then m2rnn_bwd;
      recompute: m2rnn_fwd_ckpt (a checkpoint every --segment steps), then
                 m2rnn_bwd_recompute (each segment's states rebuilt first).
    HIP events bracket the forward and the backward call on the launch stream."""
    import numpy as np
    import torch

    from non_linear_matrix_amd import m2rnn

    if cfg.dtype != "bf16":
        print("the training path takes bf16 workloads", file=sys.stderr)
        sys.exit(2)
    B, H, T, K, V = cfg.B, cfg.H, cfg.T, cfg.K, cfg.V
    S = args.segment
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(args.seed + 1)
    dy = torch.randn((B, H, T, V), dtype=torch.float32, device="cuda", generator=g)
    y = torch.empty((B, H, T, V), dtype=torch.float32, device="cuda")
    HT = torch.empty((B, H, K, V), dtype=torch.float32, device="cuda")
    # default: the library's choice for training (the split operand; on the
    # latency-oriented kernel for few row tiles)
    if args.algo in (None, "auto"):
        picked = m2rnn.pick_algo(B, H, T, K, V, cfg.dtype)
        algo = "mfma_long_split" if picked == "mfma_long_f16" else "mfma_split"
    else:
        algo = args.algo
    k, v, q, f, W, H0 = (dev[n] for n in ("k", "v", "q", "f", "W", "H0"))

    def timed(fwd, bwd):
        settle(lambda: (fwd(), bwd()))
        for _ in range(args.warmup):
            fwd()
            bwd()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        t_start.record(stream)
        for e in evs:
            e[0].record(stream)
            fwd()
            e[1].record(stream)
            bwd()
            e[2].record(stream)
        t_end.record(stream)
        torch.cuda.synchronize()
        return {
            "ms_per_step": t_start.elapsed_time(t_end) / args.steps,
            "fwd_ms": sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps,
            "bwd_ms": sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps,
            "wall_s": time.perf_counter() - w0,
        }

    modes = {}
    # save mode
    saved = torch.empty(m2rnn.saved_bytes(B, H, T, K, V), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(m2rnn.bwd_workspace_bytes(B, H, T, K, V), 16), dtype=torch.uint8, device="cuda")
    out = m2rnn._grad_buffers(B, H, T, K, V, "cuda", True)
    modes["save"] = timed(
        lambda: m2rnn.fwd_save(k, v, q, f, W, H0, saved=saved, y=y, H_T=HT, algo=algo, stream=stream),
        lambda: m2rnn.bwd(k, v, q, f, W, H0, saved, dy, out=out, workspace=ws, stream=stream))
    modes["save"]["memory_GB"] = (saved.numel() + ws.numel()) / 1e9
    g_save = {key: out[key].clone() for key in ("dW", "dk")}
    del saved, ws
    torch.cuda.empty_cache()
    # recompute mode
    nck = m2rnn.ckpt_bytes(B, H, T, K, V, S)
    ckpt = torch.empty((max(nck // (4 * B * H * K * V), 1), B, H, K, V), dtype=torch.float32, device="cuda")
    ws = torch.empty(m2rnn.bwd_recompute_workspace_bytes(B, H, T, K, V, S), dtype=torch.uint8, device="cuda")
    modes["recompute"] = timed(
        lambda: m2rnn.fwd_ckpt(k, v, q, f, W, H0, segment=S, ckpt=ckpt, y=y, H_T=HT, algo=algo, stream=stream),
        lambda: m2rnn.bwd_recompute(k, v, q, f, W, H0, ckpt, dy, segment=S, algo=algo, out=out, workspace=ws,
                                    stream=stream))
    modes["recompute"]["memory_GB"] = (nck + ws.numel()) / 1e9
    modes["recompute"]["segment"] = S
    torch.cuda.synchronize()
    # the two modes compute the same gradients up to rounding
    agree = max(float((out[key] - g_save[key]).abs().max() / g_save[key].abs().max().clamp_min(1e-30))
                for key in g_save)

    tokens = B * H * T
    # algorithmic flops of the backward call: dA W^T (the state gradient) and
    # H_{t-1}^T dA (the W gradient), 2 K V^2 each per (b, h, t)
    bwd_flops = 4.0 * K * V * V * tokens
    peak = PEAK_TFLOPS["bf16"]
    best = min(modes, key=lambda m: modes[m]["ms_per_step"])
    bwd_ms = modes[best]["bwd_ms"]
    achieved = bwd_flops / (bwd_ms * 1e-3) / 1e12
    res = {
        "metric": TRAIN_METRIC,
        "value": tokens / (modes[best]["ms_per_step"] * 1e-3),
        "unit": "tok·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": modes[best]["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={B} H={H} K={K} V={V} T={T}, {cfg.dtype} inputs, fp32 state, seed "
                        f"{args.seed}; training step = forward ({algo}) + backward, dy ~ N(0,1); mode {best}",
            "B": B, "H": H, "K": K, "V": V, "T": T,
            "parallelism": "one GPU; (b,h) units x row groups across CUs",
        },
        "modes": modes,
        "modes_max_rel_diff": agree,
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": measured_traffic(cfg.name, "train") if best == "save" else None,
            "traffic_GBps": (measured_traffic(cfg.name, "train") / (bwd_ms * 1e-3) / 1e9
                             if best == "save" and measured_traffic(cfg.name, "train") else None),
            "kernel": f"backward call of mode {best}",
            "kernel_avg_ms": bwd_ms,
            "flops_per_launch": bwd_flops,
        },
    }
    if args.cpu_seconds > 0:
        dy_np = dy.cpu().numpy().astype(np.float64)
        res["cpu_baseline"] = cpu_baseline_train(cfg, x, dy_np, args.cpu_seconds)
    print(json.dumps(res), flush=True)


FRONT_METRIC = "M2RNN layer front-end (x -> k, v, q, f) tokens·heads/sec at K=V=128, 1×MI355X"


def cpu_baseline_frontend(cfg, g, budget_s):
    """The fp64 front-end oracle on the first tokens of every batch row."""
    from oracle import m2rnn_frontend_ref

    def run(ts):
        t0 = time.perf_counter()
        m2rnn_frontend_ref(g["x"][:, :ts], g["Wx"], g["bias"], K=cfg.K, V=cfg.V)
        return time.perf_counter() - t0

    probe = min(4, cfg.T)
    dt = run(probe)
    ts = int(min(cfg.T, max(probe, probe * budget_s / max(dt, 1e-6))))
    dt = run(ts)
    return {
        "value": cfg.B * cfg.H * ts / dt,
        "unit": "tok·heads/s",
        "cores": os.cpu_count(),
        "kind": "oracle",
        "sample": f"fp64 numpy front-end oracle, all {cfg.B} batch rows x {cfg.H} heads of {cfg.name}, "
                  f"first {ts} of {cfg.T} steps ({dt:.1f}s)",
    }


def frontend_bench(args, cfg):
    """Times the front-end alone (the dominant kernel here) and the layer's
    forward: front-end, then the recurrence on its outputs."""
    import numpy as np
    import torch

    from non_linear_matrix_amd import m2rnn
    from non_linear_matrix_amd.inputs import frontend_rows, frontend_width, generate, generate_frontend

    B, H, T, K, V = cfg.B, cfg.H, cfg.T, cfg.K, cfg.V
    D, R = frontend_width(cfg), frontend_rows(cfg)
    g = generate_frontend(cfg, args.seed)
    rec = generate(cfg.with_(T=1), args.seed)   # a W and an H0 of the right shapes (T = 1 keeps the draw small)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    x, Wx, bias, W = dev(g["x"]), dev(g["Wx"]), dev(g["bias"]), dev(rec["W"])
    H0 = None if rec["H0"] is None else dev(rec["H0"])
    stream = torch.cuda.current_stream()
    out = m2rnn.frontend(x, Wx, bias, K=K, V=V, stream=stream)
    y = torch.empty((B, H, T, V), dtype=torch.float32, device="cuda")
    HT = torch.empty((B, H, K, V), dtype=torch.float32, device="cuda")

    def front():
        m2rnn.frontend(x, Wx, bias, K=K, V=V, out=out, stream=stream)

    def layer():
        front()
        m2rnn.fwd(out["k"], out["v"], out["q"], out["f"], W, H0, y=y, H_T=HT, algo=args.algo or "mfma", stream=stream)

    def timed(fn, steps):
        settle(fn)
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    front_ms = timed(front, args.steps)
    layer_ms = timed(layer, args.steps)
    tokens = B * H * T
    M, N = B * T, H * R
    flops = 2.0 * M * N * D
    # bytes the product must move once: x and Wx (bf16), bias, outputs (bf16)
    algo_bytes = 2.0 * (M * D + N * D) + 4 * H + 2.0 * M * N
    peak = PEAK_TFLOPS["bf16"]
    achieved = flops / (front_ms * 1e-3) / 1e12
    res = {
        "metric": FRONT_METRIC,
        "value": tokens / (front_ms * 1e-3),
        "unit": "tok·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": front_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name} front-end: x [B={B}, T={T}, D={D}] bf16, Wx [H={H}, 2K+V+1={R}, D] bf16, "
                        f"K={K} V={V}, seed {args.seed}",
            "B": B, "H": H, "K": K, "V": V, "T": T, "D": D,
            "parallelism": "one GPU; 128x128 output tiles across CUs",
        },
        "layer_fwd_ms": layer_ms,
        "layer_fwd_tok_heads_per_s": tokens / (layer_ms * 1e-3),
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": None,
            "kernel": "frontend_kernel",
            "kernel_avg_ms": front_ms,
            "flops_per_launch": flops,
            "algorithmic_bytes_per_launch": algo_bytes,
        },
    }
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_frontend(cfg, g, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); units shard across GPUs "
              "with no communication, so N GPUs run N independent copies of this measurement.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from non_linear_matrix_amd import m2rnn
    from non_linear_matrix_amd.inputs import CONFIGS, SERVING, generate, ragged_lengths

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    m2rnn.load()
    cfg = {**CONFIGS, **SERVING}[args.workload]
    if args.frontend:
        frontend_bench(args, cfg)
        return
    if args.algo is None and not args.train:
        args.algo = m2rnn.pick_algo(cfg.B, cfg.H, cfg.T, cfg.K, cfg.V, cfg.dtype)
    plan = m2rnn.get_plan(cfg.B, cfg.H, cfg.T, cfg.K, cfg.V, cfg.dtype, args.algo or "auto")
    print(f"[bench] workload {cfg} plan {plan}", file=sys.stderr, flush=True)
    x = generate(cfg, args.seed)
    dev = {}
    for key, a in x.items():
        if a is None:
            dev[key] = None
        elif a.dtype == np.uint16:
            dev[key] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        else:
            dev[key] = torch.from_numpy(a).cuda()
    if args.train:
        train_bench(args, cfg, dev, x)
        return
    y = torch.zeros((cfg.B, cfg.H, cfg.T, cfg.V), dtype=torch.float32, device="cuda")
    # D1 carries the state in place (H_T is H0), as a decoding loop does
    HT = dev["H0"] if cfg.name == "D1" else torch.empty((cfg.B, cfg.H, cfg.K, cfg.V), dtype=torch.float32,
                                                        device="cuda")
    lens = ragged_lengths(cfg.B, cfg.T, args.seed) if cfg.name == "R1" else None
    seq_len = None if lens is None else torch.from_numpy(lens).cuda()
    stream = torch.cuda.current_stream()
    # When the library would clear y first (several workgroups add into it, or
    # sequences end early), the step clears y itself (part of the timed work) and
    # asks the library to accumulate, so the events below bracket the recurrence
    # kernel alone.
    clear_here = bool(plan["clears_y"]) or lens is not None

    def step(ev0=None, ev1=None):
        if clear_here:
            y.zero_()
        if ev0 is not None:
            ev0.record(stream)
        m2rnn.fwd(dev["k"], dev["v"], dev["q"], dev["f"], dev["W"], dev["H0"], y=y, H_T=HT,
                  seq_len=seq_len, algo=args.algo, stream=stream, accumulate_y=clear_here)
        if ev1 is not None:
            ev1.record(stream)

    settle_calls = settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(*evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t_start.elapsed_time(t_end)
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    kern_avg = sum(kern_ms) / len(kern_ms)
    kern_median = sorted(kern_ms)[len(kern_ms) // 2]
    ms_per_step = total_ms / args.steps
    tokens = cfg.H * (int(lens.sum()) if lens is not None else cfg.B * cfg.T)
    value = tokens / (ms_per_step * 1e-3)
    flops = 2.0 * cfg.K * cfg.V * cfg.V * tokens          # H_{t-1} W per (b, h, t)
    esize = 2 if cfg.dtype == "bf16" else 4
    # bytes the operation must move once: k, q, v, f per token; W per head; H0 and
    # H_T per unit; y per token (fp32)
    algo_bytes = (tokens * ((2 * cfg.K + cfg.V + 1) * esize + 4 * cfg.V) + cfg.H * cfg.V * cfg.V * esize
                  + 2 * cfg.B * cfg.H * cfg.K * cfg.V * 4)
    # the matrix products' operand type: fp16 for the fp16-operand families (bf16
    # inputs converted exactly), else the input type
    mma_dtype = "f16" if (args.algo or "").endswith("f16") and cfg.T > 1 else cfg.dtype
    peak = PEAK_TFLOPS[mma_dtype]
    # the bound is whichever of the matrix cores and HBM needs longer at its peak
    hbm_bound = algo_bytes / (HBM_PEAK_GBS * 1e9) > flops / (peak * 1e12)
    achieved = flops / (kern_avg * 1e-3) / 1e12
    hbm_gbs = algo_bytes / (kern_avg * 1e-3) / 1e9
    # the other matrix-core variant on the same workload, for reference (not `value`)
    alt = None
    # the other operand variants of the same kernel family on the same workload,
    # timed for reference (never `value`)
    others = {"mfma": ["mfma_split"], "mfma_split": ["mfma"], "mfma_long": ["mfma_long_split"],
              "mfma_long_split": ["mfma_long"], "mfma_f16": ["mfma_split", "mfma"],
              "mfma_long_f16": ["mfma_long_split", "mfma_long"]}
    alts = []
    for other in (others.get(args.algo, []) if cfg.T > 1 else []):
        def alt_step():
            if clear_here:
                y.zero_()
            m2rnn.fwd(dev["k"], dev["v"], dev["q"], dev["f"], dev["W"], dev["H0"], y=y, H_T=HT,
                      seq_len=seq_len, algo=other, stream=stream, accumulate_y=clear_here)
        for _ in range(3):
            alt_step()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_alt = max(5, args.steps // 2)
        a0.record(stream)
        for _ in range(n_alt):
            alt_step()
        a1.record(stream)
        torch.cuda.synchronize()
        alt_ms = a0.elapsed_time(a1) / n_alt
        alts.append({"algo": other, "ms_per_step": alt_ms, "tok_heads_per_s": tokens / (alt_ms * 1e-3),
                     "note": "another operand variant of the same kernel family; not the headline value"})
    alt = alts[0] if alts else None
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tok·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": mma_dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} H={cfg.H} K={cfg.K} V={cfg.V} T={cfg.T}, "
                        f"{cfg.dtype} inputs, fp32 state"
                        + (", fp16 matrix operands" if mma_dtype == "f16" else "") + f", seed {args.seed}"
                        + (f", lengths U[{cfg.T // 4}, {cfg.T}] ({tokens // cfg.H} tokens)" if lens is not None else "")
                        + (", state updated in place" if cfg.name == "D1" else ""),
            "B": cfg.B, "H": cfg.H, "K": cfg.K, "V": cfg.V, "T": cfg.T,
            "algo": plan["algo"], "grid": plan["grid"], "block": plan["block"],
            "parallelism": "one GPU; (b,h) units x row groups across CUs",
        },
        "mfma_util_pct": 100.0 * achieved / peak,
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "achieved": hbm_gbs if hbm_bound else achieved,
            "peak": HBM_PEAK_GBS if hbm_bound else peak,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": hbm_gbs / HBM_PEAK_GBS if hbm_bound else achieved / peak,
            "traffic": measured_traffic(args.workload, "decode" if cfg.T == 1 else plan["algo"]),
            "kernel": ("decode_kernel" if cfg.T == 1 else
                       "mfma_f32_fwd_kernel" if plan["algo"] == "mfma_f32" else
                       "mfma_fwd_long_kernel" if plan["algo"].startswith("mfma_long") else "mfma_fwd_kernel")
                      if plan["algo"].startswith("mfma") else "simple_fwd_kernel",
            "kernel_avg_ms": kern_avg,
            "kernel_median_ms": kern_median,
            "flops_per_launch": flops,
            "algorithmic_bytes_per_launch": algo_bytes,
        },
        "hbm_GBps_algorithmic": hbm_gbs,
        "other_variant": alt,
        "other_variants": alts,
        "settle": {"calls": settle_calls, "min_ms": SETTLE_MS,
                   "note": "untimed steps before the warmup, until the clock has settled"},
        "wall_s": wall,
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
