"""Benchmark: one step = the whole Forgetting Attention hot path on one synthetic batch.

Workload (the one the headline metric is quoted on): B=1, H=12, L=16384, D=128, bf16 q/k/v/dO,
fp32 log forget gates drawn per head as log sigmoid(z), z ~ N(mu_h, 1), mu_h ~ U[1, 6].
A step runs, on one HIP stream:
    fox_logf_cumsum -> fox_attn_fwd (fp32 O + LSE) -> fox_attn_bwd_delta -> fox_attn_bwd_dq
    -> fox_attn_bwd_dkv -> fox_dlogf_from_dc
(the four backward calls are fox_attn_bwd's steps). Inputs are resident in HBM before timing.

Prints ONE JSON line. value = causal fwd+bwd TFLOP/s with the FlashAttention convention:
fwd = 4*B*H*D*L^2/2 FLOPs (two causal contractions), bwd = 2.5 x fwd (five contractions).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Forgetting-attn fwd(+bwd) causal TFLOP/s @L=16384,D=128; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, 2.4 GHz
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def contraction_flops(B, H, L, D):
    """One causal L x L x D contraction (half of the square): 2*D*L^2/2 per (b, h)."""
    return B * H * D * L * L


def cpu_baseline(case, seconds_hint=True):
    """Time the fp64 oracle on one head of the workload (fwd + bwd) on this host's cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: report the affinity set numpy's BLAS sees
        threads = len(os.sched_getaffinity(0))
    sl = (slice(0, 1), slice(0, 1))
    s = 1.0 / math.sqrt(case.D)
    t0 = time.perf_counter()
    oracle.attn_bwd(case.q[sl], case.k[sl], case.v[sl], case.log_f[sl], case.do[sl], scale=s,
                    block=1024)
    dt = time.perf_counter() - t0
    flops = 7 * contraction_flops(1, 1, case.L, case.D)  # fwd (2) + bwd (5), as for the GPU
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"one head (b=0, h=0) of the workload, fwd+bwd in fp64 NumPy: {dt:.2f} s",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import fox_inputs as fi
    import gated_softmax_attention_fox_amd as fox

    fox.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    case = fi.config_case(5)
    B, H, L, D = case.B, case.H, case.L, case.D
    log(f"workload B={B} H={H} L={L} D={D} steps={args.steps} warmup={args.warmup}")

    def up(a, dt):
        if dt == "bf16":
            return torch.from_numpy(fi.bf16_bits(a)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    q, k, v, do = (up(getattr(case, n), "bf16") for n in ("q", "k", "v", "do"))
    log_f = up(case.log_f, "f32")
    torch.cuda.synchronize()

    names = ["scan", "fwd", "delta", "dq", "dkv", "dlogf"]
    ev = {n: [] for n in names}
    stream = torch.cuda.current_stream(dev)

    def step(record):
        def timed(n, fn):
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                r = fn()
                e1.record(stream)
                ev[n].append((e0, e1))
                return r
            return fn()
        c = timed("scan", lambda: fox.fox_logf_cumsum(log_f))
        o, lse = timed("fwd", lambda: fox.fox_attn_fwd(q, k, v, c, o_dtype=torch.float32))
        delta = timed("delta", lambda: fox.fox_attn_bwd_delta(do, o))
        dq, dcq, delta = timed("dq", lambda: fox.fox_attn_bwd_dq(q, k, v, c, lse, do, delta,
                                                                  delta_out=delta))
        dk, dv, dck = timed("dkv", lambda: fox.fox_attn_bwd_dkv(q, k, v, c, lse, do, delta))
        dlf = timed("dlogf", lambda: fox.fox_dlogf_from_dc(dcq, dck))
        return dq, dk, dv, dlf

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # timed region 1: the plain step loop (this is `value`)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step(False)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # timed region 2: the same steps with an event pair around every launch, per-kernel times
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    kern_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names}

    unit = contraction_flops(B, H, L, D)
    fwd_flops, bwd_flops = 2 * unit, 5 * unit
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12
    # algorithmic work of each MFMA kernel per launch (causal contractions it must perform)
    kernel_flops = {"fwd": 2 * unit, "dkv": 4 * unit, "dq": 3 * unit}
    dom = max(kernel_flops, key=lambda n: kern_ms[n])
    ach = kernel_flops[dom] / (kern_ms[dom] * 1e-3) / 1e12
    fwd_tf = kernel_flops["fwd"] / (kern_ms["fwd"] * 1e-3) / 1e12
    fwd_path_tf = fwd_flops / ((kern_ms["fwd"] + kern_ms["scan"]) * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fox_attn_fwd_bwd B=1 H=12 L=16384 D=128 (bf16 q/k/v/dO, "
                               "per-head gates mu_h~U[1,6], z~N(mu_h,1))",
                   "B": B, "H": H, "L": L, "D": D, "causal": True, "o_dtype": "fp32",
                   "grad_dtype": "fp32"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None},
        "fwd": {"kernel_ms": round(kern_ms["fwd"], 4), "tflops": round(fwd_tf, 2),
                "frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                "scan_plus_fwd_tflops": round(fwd_path_tf, 2)},
        "kernel_ms": {n: round(kern_ms[n], 4) for n in names},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on one head (CPU) ...")
        cb = cpu_baseline(case)
        cb.pop("seconds")
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
