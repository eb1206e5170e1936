"""Benchmark: one step = the whole Forgetting Attention hot path on one synthetic batch.

Workload (the one the headline metric is quoted on): B=1, H=12, L=16384, D=128, bf16 q/k/v/dO,
fp32 log forget gates drawn per head as log sigmoid(z), z ~ N(mu_h, 1), mu_h ~ U[1, 6].
A step runs, on one HIP stream:
    fox_logf_cumsum -> fox_attn_fwd (fp32 O + LSE) -> fox_attn_bwd_dq (row term formed from O
    inside) -> fox_attn_bwd_dkv -> fox_dlogf_from_dc
(the backward calls are fox_attn_bwd's launches). Inputs are resident in HBM before timing.

Prints ONE JSON line. value = causal fwd+bwd TFLOP/s with the FlashAttention convention:
fwd = 4*B*H*D*L^2/2 FLOPs (two causal contractions), bwd = 2.5 x fwd (five contractions).
Every launch in the timed loop is bracketed by events on the stream it runs on, so the
per-kernel averages and the step time come from the same K steps.

The roofline object covers the kernel with the longest average duration. Its "traffic" (HBM bytes
per launch) is read from profiles/hbm_traffic.txt, which holds FETCH_SIZE / WRITE_SIZE counter
readings scaled by a copy kernel of known size; it is null when the kernel's source has changed
since the counters were taken (the file records a hash of the sources). "clock_ghz" is the
shader clock each attention kernel ran at in the committed counter passes
(profiles/counters_L16384_D128.txt), under the same rule.
"""
from __future__ import annotations

import argparse
import hashlib
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
CSRC = os.path.join(ROOT, "gated_softmax_attention_fox_amd", "csrc")
# sources that define each timed kernel (a change to any of them invalidates its counter data)
KERNEL_SOURCES = {
    "fwd": ["attn_fwd.hip", "fox_device.h"],
    "dq": ["attn_bwd.hip", "fox_device.h"],
    "dkv": ["attn_bwd.hip", "fox_device.h"],
    "scan": ["scan.hip"],
    "dlogf": ["scan.hip"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def contraction_flops(B, H, L, D):
    """One causal L x L x D contraction (half of the square): 2*D*L^2/2 per (b, h)."""
    return B * H * D * L * L


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


COUNTER_FILE = os.path.join(ROOT, "profiles", "counters_L16384_D128.txt")


def read_profile_value(path: str, kernel: str, key: str):
    """`key` of section [kernel] in a committed counter summary, or None if the file is absent
    or was taken from other kernel sources (its source_sha256 differs from the current one)."""
    if not os.path.exists(path):
        return None
    sec, vals = None, {}
    for line in open(path):
        line = line.strip()
        if line.startswith("[") and line.endswith("]"):
            sec = line[1:-1]
        elif "=" in line and not line.startswith("#") and sec == kernel:
            k, v = (s.strip() for s in line.split("=", 1))
            vals[k] = v
    if not vals or vals.get("source_sha256") != source_hash(kernel) or key not in vals:
        return None
    return float(vals[key])


def counter_clock():
    """Shader clock (GHz) of each attention kernel from the committed counter passes
    (GRBM_GUI_ACTIVE per XCD over the dispatch's duration), null where stale."""
    return {"fwd": read_profile_value(COUNTER_FILE, "fwd", "clock_ghz"),
            "dq": read_profile_value(COUNTER_FILE, "dq", "clock_ghz"),
            "dkv": read_profile_value(COUNTER_FILE, "dkv", "clock_ghz"),
            "source": "profiles/counters_L16384_D128.txt"}


def read_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the counter file, or None if absent or stale."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sec, vals = None, {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if line.startswith("[") and line.endswith("]"):
            sec = line[1:-1]
        elif "=" in line and not line.startswith("#") and sec == kernel:
            k, v = (s.strip() for s in line.split("=", 1))
            vals[k] = v
    if not vals or vals.get("source_sha256") != source_hash(kernel):
        return None
    return float(vals["traffic_bytes_per_launch"])


def cpu_baseline(case, heads: int):
    """Time the fp64 oracle (fwd + bwd) on the first `heads` heads of the workload, with the BLAS
    threads pinned to the cores this process may run on."""
    import contextlib

    import oracle
    threads = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=threads, user_api="blas")
    except Exception:  # threadpoolctl missing: BLAS keeps its own default
        limit = contextlib.nullcontext()
    sl = (slice(0, 1), slice(0, heads))
    s = 1.0 / math.sqrt(case.D)
    with limit:
        t0 = time.perf_counter()
        oracle.attn_bwd(case.q[sl], case.k[sl], case.v[sl], case.log_f[sl], case.do[sl], scale=s,
                        block=1024)
        dt = time.perf_counter() - t0
    flops = 7 * contraction_flops(1, heads, case.L, case.D)  # fwd (2) + bwd (5), as for the GPU
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of the workload's {case.H} heads (b=0, h=0..{heads - 1}), fwd+bwd in "
                      f"fp64 NumPy: {dt:.2f} s"}


def step_medians(events, names):
    """Median per-kernel duration and median step duration (first launch to last) over the steps."""
    per = {n: [a.elapsed_time(b) for m, a, b in events if m == n] for n in names}
    starts = [a for m, a, b in events if m == names[0]]
    ends = [b for m, a, b in events if m == names[-1]]
    steps = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    return ({n: round(float(np.median(v)), 4) for n, v in per.items() if v},
            round(float(np.median(steps)), 4))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="heads of the workload the oracle is timed on (about 1.5 s each)")
    ap.add_argument("--paper-shape", action="store_true",
                    help="the FoX paper's own head shape instead: B=1, H=24, L=16384, D=64 "
                         "(same input recipe); a second measurement, not the headline line")
    ap.add_argument("--pro", action="store_true",
                    help="the Pro block's whole attention step instead (x [1, 16384, 1536], 12 heads of D=128, plus dO): gate, "
                         "scan, QK-norm, attention forward and backward, QK-norm and gate backward")
    ap.add_argument("--decode", action="store_true",
                    help="single-token decode against a full KV cache instead: B=8 sequences of "
                         "12 heads, 16384 cached positions, D=128 (a separate, HBM-bound line)")
    ap.add_argument("--lengths", action="store_true",
                    help="forward and backward at other batch and sequence shapes instead (one "
                         "JSON line per shape; a separate measurement, not the headline line)")
    ap.add_argument("--no-skip", action="store_true",
                    help="leave out the second measurement with exact tile skipping")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run 3 device copies of this many MiB (a known-size kernel "
                         "that scales HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import fox_inputs as fi
    import gated_softmax_attention_fox_amd as fox

    fox.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.pro:
        return pro_step(args, torch, fi, fox, dev)
    if args.decode:
        return decode_step(args, torch, fi, fox, dev)
    if args.lengths:
        return length_sweep(args, torch, fi, fox, dev)
    if args.paper_shape:
        case = fi.make_case(1, 24, 16384, 64, "bf16", seed=6, gate="per_head", with_do=True,
                            name="paper_shape")
        workload = ("fox_attn_fwd_bwd B=1 H=24 L=16384 D=64 (the paper's head shape; bf16 "
                    "q/k/v/dO, per-head gates mu_h~U[1,6], z~N(mu_h,1))")
    else:
        case = fi.config_case(5)
        workload = ("fox_attn_fwd_bwd B=1 H=12 L=16384 D=128 (bf16 q/k/v/dO, "
                    "per-head gates mu_h~U[1,6], z~N(mu_h,1))")
    B, H, L, D = case.B, case.H, case.L, case.D
    # counters were taken on the headline workload only
    traffic = read_traffic if not args.paper_shape else (lambda kernel: None)
    log(f"workload B={B} H={H} L={L} D={D} steps={args.steps} warmup={args.warmup}")

    def up(a, dt):
        if dt == "bf16":
            return torch.from_numpy(fi.bf16_bits(a)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    q, k, v, do = (up(getattr(case, n), "bf16") for n in ("q", "k", "v", "do"))
    log_f = up(case.log_f, "f32")
    torch.cuda.synchronize()

    names = ["scan", "fwd", "dq", "dkv", "dlogf"]
    stream = torch.cuda.current_stream(dev)  # the library launches on this stream

    def step(events, skip=False):
        def run(n, fn):
            if events is None:
                return fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            r = fn()
            e1.record(stream)
            events.append((n, e0, e1))
            return r
        c = run("scan", lambda: fox.fox_logf_cumsum(log_f))
        plan = run("plan", lambda: fox.fox_attn_skip_plan(q, k, c)) if skip else None
        o, lse = run("fwd", lambda: fox.fox_attn_fwd(q, k, v, c, o_dtype=torch.float32,
                                                     skip_plan=plan))
        dq, dcq, delta, lse2 = run("dq", lambda: fox.fox_attn_bwd_dq(q, k, v, c, lse, do, None,
                                                                      o=o, skip_plan=plan))
        dk, dv, dck = run("dkv", lambda: fox.fox_attn_bwd_dkv(q, k, v, c, lse2, do, delta,
                                                              skip_plan=plan))
        dlf = run("dlogf", lambda: fox.fox_dlogf_from_dc(dcq, dck))
        return dq, dk, dv, dlf, plan

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    # the timed region: exactly K steps, every launch bracketed by events on its stream
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_per_step = events[0][1].elapsed_time(events[-1][2]) / args.steps
    kern_ms = {n: float(np.mean([a.elapsed_time(b) for m, a, b in events if m == n]))
               for n in names}
    kern_med, step_med = step_medians(events, names)

    unit = contraction_flops(B, H, L, D)
    fwd_flops, bwd_flops = 2 * unit, 5 * unit
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12
    # algorithmic work of each MFMA kernel per launch (the causal contractions it performs)
    kernel_flops = {"fwd": 2 * unit, "dkv": 4 * unit, "dq": 3 * unit}
    dom = max(kernel_flops, key=lambda n: kern_ms[n])
    ach = kernel_flops[dom] / (kern_ms[dom] * 1e-3) / 1e12
    fwd_tf = kernel_flops["fwd"] / (kern_ms["fwd"] * 1e-3) / 1e12
    fwd_path_tf = fwd_flops / ((kern_ms["fwd"] + kern_ms["scan"]) * 1e-3) / 1e12
    bwd_ms = sum(kern_ms[n] for n in ("dq", "dkv", "dlogf"))

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
        "config": {"workload": workload,
                   "B": B, "H": H, "L": L, "D": D, "causal": True, "o_dtype": "fp32",
                   "grad_dtype": "fp32"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic(dom)},
        "fwd": {"kernel_ms": round(kern_ms["fwd"], 4), "tflops": round(fwd_tf, 2),
                "frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                "scan_plus_fwd_tflops": round(fwd_path_tf, 2),
                "traffic": traffic("fwd")},
        "bwd": {"ms": round(bwd_ms, 4),
                "tflops_credited": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2)},
        "kernel_ms": {n: round(kern_ms[n], 4) for n in names},
        "kernel_ms_median": kern_med,
        "ms_per_step_median": step_med,
        "fwd_frac_of_peak_median": round(kernel_flops["fwd"] / (kern_med["fwd"] * 1e-3) / 1e12
                                         / PEAK_BF16_TFLOPS, 4),
        "clock_ghz": counter_clock() if not args.paper_shape else None,
        "host_wall_ms_per_step": round(wall_ms, 4),
    }
    if not args.no_skip:
        out["skip_decayed"] = skip_measurement(args, torch, fox, step, names, ms_per_step,
                                               fwd_flops + bwd_flops, (B, H, L))
        out["fused_scan"] = fused_scan_measurement(args, torch, fox, (q, k, v, do, log_f),
                                                   stream, kern_ms)
    copy_calibration(args, torch, dev, out)
    if not args.no_cpu_baseline:
        log(f"timing the oracle on {args.cpu_heads} heads (CPU) ...")
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_heads)
    print(json.dumps(out), flush=True)


def skip_measurement(args, torch, fox, step, names, dense_ms, dense_flops, bhl):
    """The same step with exact tile skipping (a skip plan made inside every step from q, k, c):
    a separate measurement, credited with the dense FLOPs ("effective"), never the headline."""
    B, H, L = bhl
    ref = step(None)
    got = step(None, skip=True)
    torch.cuda.synchronize()
    identical = all(torch.equal(a, b) for a, b in zip(ref[:4], got[:4]))
    q_skip, kv_tiles = (a.cpu().numpy().astype(np.int64)
                        for a in fox.skip_plan_arrays(got[4], B, H, L)[:2])
    n_qt, n_kb = q_skip.shape[1], kv_tiles.shape[1]
    q_dense = np.minimum(np.arange(n_qt) * 256 + 255, L - 1) // 64 + 1
    kv_dense = -(-(L - 128 * np.arange(n_kb)) // 64)
    for _ in range(args.warmup):
        step(None, skip=True)
    events = []
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step(events, skip=True)
    torch.cuda.synchronize()
    ms = events[0][1].elapsed_time(events[-1][2]) / args.steps
    kern = {n: float(np.mean([a.elapsed_time(b) for m, a, b in events if m == n]))
            for n in ["plan"] + names}
    return {
        "ms_per_step": round(ms, 4),
        "effective_tflops": round(dense_flops / (ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense": round(dense_ms / ms, 3),
        "bit_identical_to_dense": bool(identical),
        "fwd_dq_key_tiles_walked_frac": round(
            float((q_dense - q_skip).sum() / (B * H * q_dense.sum())), 4),
        "dkv_query_tiles_walked_frac": round(float(kv_tiles.sum() / (B * H * kv_dense.sum())), 4),
        "kernel_ms": {n: round(kern[n], 4) for n in kern},
    }


def fused_scan_measurement(args, torch, fox, inputs, stream, dense_kern):
    """The same step with the prefix sum fused into the forward (fox_attn_fwd_logf takes log f and
    writes c for the backward) in place of the scan kernel and the forward. A separate
    measurement of the option, never the headline."""
    q, k, v, do, log_f = inputs

    def fstep(events):
        def run(n, fn):
            if events is None:
                return fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            r = fn()
            e1.record(stream)
            events.append((n, e0, e1))
            return r
        o, lse, c = run("fwd_logf", lambda: fox.fox_attn_fwd_logf(q, k, v, log_f,
                                                                  o_dtype=torch.float32))
        dq, dcq, delta, lse2 = run("dq", lambda: fox.fox_attn_bwd_dq(q, k, v, c, lse, do, None,
                                                                      o=o))
        dk, dv, dck = run("dkv", lambda: fox.fox_attn_bwd_dkv(q, k, v, c, lse2, do, delta))
        run("dlogf", lambda: fox.fox_dlogf_from_dc(dcq, dck))
        return o, c

    o_f, c_f = fstep(None)
    c_s = fox.fox_logf_cumsum(log_f)
    o_s, _ = fox.fox_attn_fwd(q, k, v, c_s, o_dtype=torch.float32)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        fstep(None)
    events = []
    torch.cuda.synchronize()
    for _ in range(args.steps):
        fstep(events)
    torch.cuda.synchronize()
    ms = events[0][1].elapsed_time(events[-1][2]) / args.steps
    names = ["fwd_logf", "dq", "dkv", "dlogf"]
    kern = {n: float(np.mean([a.elapsed_time(b) for m, a, b in events if m == n])) for n in names}
    return {
        "ms_per_step": round(ms, 4),
        "fused_fwd_ms": round(kern["fwd_logf"], 4),
        "separate_scan_plus_fwd_ms": round(dense_kern["scan"] + dense_kern["fwd"], 4),
        "c_equal_to_scan_kernel_frac": round(float((c_f == c_s).float().mean()), 6),
        "o_max_abs_diff_vs_separate": float((o_f - o_s).abs().max()),
        "kernel_ms": {n: round(kern[n], 4) for n in names},
    }


def copy_calibration(args, torch, dev, out):
    """After timing: 3 elementwise kernels that read and write --copy-mib MiB each (a kernel of
    known traffic that scales the HBM byte counters)."""
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n


# (B, H, L, D): the bench workload, shorter sequences at the same or larger batch, and the
# paper's head shape
LENGTH_SHAPES = [(1, 12, 16384, 128), (2, 12, 8192, 128), (1, 12, 4096, 128), (4, 12, 2048, 128),
                 (1, 48, 2048, 128), (8, 12, 1024, 128), (1, 24, 16384, 64)]


def length_sweep(args, torch, fi, fox, dev):
    """fox_attn_fwd (fp32 O) and fox_attn_bwd at each of LENGTH_SHAPES, timed separately over
    args.steps calls each with HIP events on the library's stream, inputs resident in HBM. One
    JSON line per shape; the forward's fraction of the bf16 peak uses its causal FLOPs."""
    stream = torch.cuda.current_stream()
    for B, H, L, D in LENGTH_SHAPES:
        case = fi.make_case(B, H, L, D, "bf16", seed=1, gate="per_head", with_do=True)
        up = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
        q, k, v, do = (up(getattr(case, n), torch.bfloat16) for n in ("q", "k", "v", "do"))
        c = fox.fox_logf_cumsum(up(case.log_f, torch.float32))
        ws = torch.empty(fox.fox_attn_bwd_workspace_bytes(B, H, L, D), dtype=torch.uint8,
                         device=dev)
        o, lse = fox.fox_attn_fwd(q, k, v, c, o_dtype=torch.float32)
        for _ in range(args.warmup):
            fox.fox_attn_fwd(q, k, v, c, o_dtype=torch.float32)
            fox.fox_attn_bwd(q, k, v, c, o, lse, do, workspace=ws)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        for _ in range(args.steps):
            fox.fox_attn_fwd(q, k, v, c, o_dtype=torch.float32)
        ev[1].record(stream)
        for _ in range(args.steps):
            fox.fox_attn_bwd(q, k, v, c, o, lse, do, workspace=ws)
        ev[2].record(stream)
        torch.cuda.synchronize()
        t_f = ev[0].elapsed_time(ev[1]) / args.steps
        t_b = ev[1].elapsed_time(ev[2]) / args.steps
        one = contraction_flops(B, H, L, D)
        print(json.dumps({
            "shape": {"B": B, "H": H, "L": L, "D": D},
            "fwd_ms": round(t_f, 4),
            "fwd_tflops": round(2 * one / (t_f * 1e-3) / 1e12, 1),
            "fwd_frac_of_peak": round(2 * one / (t_f * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bwd_ms": round(t_b, 4),
            "bwd_tflops_credited": round(5 * one / (t_b * 1e-3) / 1e12, 1),
            "steps": args.steps, "warmup": args.warmup, "dtype": "bf16", "data": "synthetic",
        }), flush=True)
        del q, k, v, do, c, ws, o, lse
        torch.cuda.empty_cache()


def decode_step(args, torch, fi, fox, dev):
    """Single-token decode: one new query per sequence against a full cache of the bench's
    sequence length (every cached K and V row read once; bound by HBM)."""
    B, H, T, D = 8, 12, 16384, 128
    case = fi.make_case(B, H, T, D, "bf16", seed=8, gate="per_head", name="decode")
    rng = np.random.default_rng(88)
    qn = fi.bf16_round(rng.standard_normal((B, H, D), dtype=np.float32))
    up = lambda a: torch.from_numpy(fi.bf16_bits(a)).view(torch.bfloat16).to(dev)
    q, k, v = up(qn), up(case.k), up(case.v)
    c = fox.fox_logf_cumsum(torch.from_numpy(case.log_f).to(dev))
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    ws = torch.empty(fox.fox_attn_decode_workspace_bytes(B, H, T, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(max(args.warmup, 3)):
        fox.fox_attn_decode(q, k, v, c, lens, workspace=ws)
    torch.cuda.synchronize()
    steps = args.steps * 10  # a decode step is about 0.2 ms
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        fox.fox_attn_decode(q, k, v, c, lens, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = B * H * T * (2 * D * 2 + 4)  # K and V rows (bf16) and c (fp32), each read once
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "Forgetting-attn single-token decode, KV-cache read bandwidth",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": max(args.warmup, 3), "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"fox_attn_decode B={B} H={H} T={T} D={D} (full caches, bf16 "
                               "K/V, per-head gates mu_h~U[1,6], z~N(mu_h,1))",
                   "B": B, "H": H, "T": T, "D": D},
        "roofline": {"kernel": "decode", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None},
    }
    if not args.no_skip:  # the same decode with the cache's key norms (exact chunk skipping)
        kn = fox.fox_attn_decode_key_norms(k, lens)
        o0, l0 = fox.fox_attn_decode(q, k, v, c, lens, workspace=ws)
        o1, l1 = fox.fox_attn_decode(q, k, v, c, lens, workspace=ws, k_norms=kn)
        torch.cuda.synchronize()
        identical = torch.equal(o0, o1) and torch.equal(l0, l1)
        for _ in range(3):
            fox.fox_attn_decode(q, k, v, c, lens, workspace=ws, k_norms=kn)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fox.fox_attn_decode(q, k, v, c, lens, workspace=ws, k_norms=kn)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_s = e0.elapsed_time(e1) / steps
        out["skip_decayed"] = {"ms_per_step": round(ms_s, 4),
                               "effective_GB_per_s": round(nbytes / (ms_s * 1e-3) / 1e9, 1),
                               "speedup_vs_dense": round(ms / ms_s, 3),
                               "bit_identical_to_dense": bool(identical)}
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        cc = oracle.cumsum_logf(case.log_f[:1])
        n = 0
        for h in range(H):
            qf = np.zeros((T, D), np.float32)
            qf[T - 1] = qn[0, h]
            oracle.attn_fwd_rows(qf, case.k[0, h], case.v[0, h], cc[0, h], np.array([T - 1]),
                                 scale=1.0 / math.sqrt(D))
            n += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n * T * (2 * D * 2 + 4) / dt / 1e9, 3),
                               "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
                               "kind": "oracle",
                               "sample": f"sequence 0, all {H} heads, one decode row each in fp64 "
                                         f"NumPy: {dt:.2f} s"}
    copy_calibration(args, torch, dev, out)
    print(json.dumps(out), flush=True)


def pro_fused_forward(args, torch, fox, q, k, v, x, w_f, b_f, stream):
    """The Pro forward from the raw key and value candidates, three ways, all with the same
    shift gates, c and output-gate input, and O still written for the backward:
    - separate: key shift + RMSNorm and value shift passes, q-norm pass, forward, output norm +
      gate pass;
    - fused: the two shift passes, then fox_attn_fwd_ex normalising q as it is loaded and
      applying the output norm + gate in its epilogue;
    - fused_prologue: fox_attn_fwd_ex alone, shifting and normalising the key and value tiles as
      they are loaded as well (no shifted keys or values are written)."""
    B, H, L, D = q.shape
    dm = x.shape[-1]
    rng = torch.Generator(device=q.device).manual_seed(47)
    g = torch.randn(B, H, L, D, device=q.device, generator=rng).to(torch.bfloat16)
    ak = fox.fox_shift_gate(x, 0.02 * torch.randn(H, dm, device=q.device, generator=rng))
    av = fox.fox_shift_gate(x, 0.02 * torch.randn(H, dm, device=q.device, generator=rng))
    c = fox.fox_logf_cumsum(fox.fox_gate_logf(x, w_f, b_f))

    def separate():
        kn = fox.fox_kv_shift(k, ak, normalize=True, eps=1e-6)
        vs = fox.fox_kv_shift(v, av)
        qn = fox.fox_qk_rmsnorm(q, eps=1e-6)
        o, lse = fox.fox_attn_fwd(qn, kn, vs, c, o_dtype=torch.float32)
        return o, lse, fox.fox_out_norm_gate(o, g, eps=1e-6)

    def fused():
        kn = fox.fox_kv_shift(k, ak, normalize=True, eps=1e-6)
        vs = fox.fox_kv_shift(v, av)
        return fox.fox_attn_fwd_ex(q, kn, vs, c, o_dtype=torch.float32, q_norm_eps=1e-6, gate=g,
                                   out_norm_eps=1e-6)

    def fused_prologue():
        return fox.fox_attn_fwd_ex(q, k, v, c, o_dtype=torch.float32, q_norm_eps=1e-6, gate=g,
                                   out_norm_eps=1e-6, k_shift_alpha=ak, v_shift_alpha=av,
                                   k_norm_eps=1e-6)

    res = {}
    for name, fn in (("separate", separate), ("fused", fused), ("fused_prologue", fused_prologue)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[name + "_ms"] = round(e0.elapsed_time(e1) / args.steps, 4)
    so, sl, sy = separate()
    fo, fl, fy = fused()
    po, pl, py = fused_prologue()
    torch.cuda.synchronize()
    res["o_max_abs_diff"] = float((so - fo).abs().max())
    res["y_max_abs_diff"] = float((sy.float() - fy.float()).abs().max())
    res["prologue_bit_identical_to_fused"] = bool(torch.equal(po, fo) and torch.equal(pl, fl)
                                                  and torch.equal(py, fy))
    res["saved_ms"] = round(res["separate_ms"] - res["fused_ms"], 4)
    res["prologue_saved_ms"] = round(res["fused_ms"] - res["fused_prologue_ms"], 4)
    return res


def pro_extra_kernels(torch, fox, x, k, v, stream):
    """The Pro block's shift gates, token shift (keys with RMSNorm, values without) and output
    norm + gate, forward and backward, at the workload's shape: each timed alone, 20 calls,
    with its algorithmic HBM bytes (every input read once, every output written once)."""
    B, L, dm = x.shape
    H, D = k.shape[1], k.shape[3]
    rng = torch.Generator(device=x.device).manual_seed(46)
    w_k = 0.02 * torch.randn(H, dm, device=x.device, generator=rng)
    alpha = fox.fox_shift_gate(x, w_k)
    g = torch.randn(B, H, L, D, device=x.device, generator=rng).to(torch.bfloat16)
    dy = torch.randn(B, H, L, D, device=x.device, generator=rng)
    dal = torch.randn(B, H, L, device=x.device, generator=rng)
    o_prev = torch.randn(B, H, L, D, device=x.device, generator=rng)  # an fp32 attention output
    n_row, n_tok = B * H * L * D, B * L
    cases = {
        "shift_gate": (lambda: fox.fox_shift_gate(x, w_k), n_tok * dm * 2 + B * H * L * 4),
        "shift_gate_bwd": (lambda: fox.fox_shift_gate_bwd(x, w_k, dal),
                           n_tok * dm * (2 + 4) + B * H * L * 4),
        "k_shift_norm": (lambda: fox.fox_kv_shift(k, alpha, normalize=True),
                         n_row * (2 + 2) + B * H * L * 4),
        "v_shift": (lambda: fox.fox_kv_shift(v, alpha), n_row * (2 + 2) + B * H * L * 4),
        "k_shift_norm_bwd": (lambda: fox.fox_kv_shift_bwd(k, alpha, dy, normalize=True),
                             n_row * (2 + 4 + 4) + B * H * L * 8),
        "out_norm_gate": (lambda: fox.fox_out_norm_gate(o_prev, g), n_row * (4 + 2 + 2)),
        "out_norm_gate_bwd": (lambda: fox.fox_out_norm_gate_bwd(o_prev, g, dy),
                              n_row * (4 + 2 + 4 + 4 + 4)),
    }
    res = {}
    for name, (fn, nbytes) in cases.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(20):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        res[name] = {"ms": round(ms, 4), "bytes": int(nbytes),
                     "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_of_8TBps": round(nbytes / (ms * 1e-3) / 8e12, 4)}
    return res


def pro_step(args, torch, fi, fox, dev):
    """One training step of the Pro block's attention path (x [1, 16384, 1536], q, k, v
    [1, 12, 16384, 128], plus a seeded dO)."""
    case = fi.config_case(4)
    B, H, L, D, dm = case.B, case.H, case.L, case.D, case.x.shape[-1]
    up = lambda a, dt: (torch.from_numpy(fi.bf16_bits(a)).view(torch.bfloat16) if dt == "bf16"
                        else torch.from_numpy(np.ascontiguousarray(a, np.float32))).to(dev)
    x, q, k, v = up(case.x, "bf16"), up(case.q, "bf16"), up(case.k, "bf16"), up(case.v, "bf16")
    w_f, b_f = up(case.w_f, "f32"), up(case.b_f, "f32")
    do = up(fi.bf16_round(np.random.default_rng(45).standard_normal((B, H, L, D),
                                                                    dtype=np.float32)), "bf16")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    names = ["gate", "scan", "qnorm", "knorm", "fwd", "dq", "dkv", "dlogf", "qnorm_bwd",
             "knorm_bwd", "gate_bwd"]

    def step(events, skip=False):
        def run(n, fn):
            if events is None:
                return fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            r = fn()
            e1.record(stream)
            events.append((n, e0, e1))
            return r
        lf = run("gate", lambda: fox.fox_gate_logf(x, w_f, b_f))
        c = run("scan", lambda: fox.fox_logf_cumsum(lf))
        qn = run("qnorm", lambda: fox.fox_qk_rmsnorm(q, eps=1e-6))
        kn = run("knorm", lambda: fox.fox_qk_rmsnorm(k, eps=1e-6))
        plan = run("plan", lambda: fox.fox_attn_skip_plan(qn, kn, c)) if skip else None
        o, lse = run("fwd", lambda: fox.fox_attn_fwd(qn, kn, v, c, o_dtype=torch.float32,
                                                     skip_plan=plan))
        dqn, dcq, delta, lse2 = run("dq", lambda: fox.fox_attn_bwd_dq(qn, kn, v, c, lse, do, None,
                                                                       o=o, skip_plan=plan))
        dkn, dv, dck = run("dkv", lambda: fox.fox_attn_bwd_dkv(qn, kn, v, c, lse2, do, delta,
                                                               skip_plan=plan))
        dlf = run("dlogf", lambda: fox.fox_dlogf_from_dc(dcq, dck))
        dq, _ = run("qnorm_bwd", lambda: fox.fox_qk_rmsnorm_bwd(q, dqn, eps=1e-6))
        dk, _ = run("knorm_bwd", lambda: fox.fox_qk_rmsnorm_bwd(k, dkn, eps=1e-6))
        dx, dw, db = run("gate_bwd", lambda: fox.fox_gate_logf_bwd(x, w_f, b_f, dlf, log_f=lf))
        return dq, dk, dv, dx, dw, db

    for _ in range(args.warmup):
        step(None)
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_per_step = events[0][1].elapsed_time(events[-1][2]) / args.steps
    kern_ms = {n: float(np.mean([a.elapsed_time(b) for m, a, b in events if m == n])) for n in names}
    unit = contraction_flops(B, H, L, D)
    value = 7 * unit / (ms_per_step * 1e-3) / 1e12
    n_tok, n_qk = B * L, B * H * L * D
    # algorithmic bytes: every input read once, every output written once
    hbm_bytes = {
        "gate": n_tok * dm * 2 + B * H * L * 4,
        "qnorm": n_qk * 2 * 2, "knorm": n_qk * 2 * 2,
        "qnorm_bwd": n_qk * (2 + 4 + 4), "knorm_bwd": n_qk * (2 + 4 + 4),
        "gate_bwd": n_tok * dm * (2 + 4) + B * H * L * 8,  # x, dx; dlog_f and log f
    }
    hbm = {n: {"ms": round(kern_ms[n], 4), "bytes": int(b),
               "GB_per_s": round(b / (kern_ms[n] * 1e-3) / 1e9, 1),
               "frac_of_8TBps": round(b / (kern_ms[n] * 1e-3) / 8e12, 4)} for n, b in hbm_bytes.items()}
    fwd_tf = 2 * unit / (kern_ms["fwd"] * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "pro_block_attention_step B=1 H=12 L=16384 D=128 d_model=1536 "
                               "(gate, scan, QK-norm, attention fwd+bwd, QK-norm and gate "
                               "backward; bf16 x/q/k/v/dO; 7 contractions credited)",
                   "B": B, "H": H, "L": L, "D": D, "d_model": dm, "causal": True},
        "fwd": {"kernel_ms": round(kern_ms["fwd"], 4), "tflops": round(fwd_tf, 2),
                "frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4)},
        "hbm_kernels": hbm,
        "kernel_ms": {n: round(kern_ms[n], 4) for n in names},
        "host_wall_ms_per_step": round(wall_ms, 4),
    }
    out["pro_shift_output_kernels"] = pro_extra_kernels(torch, fox, x, k, v, stream)
    out["fused_forward"] = pro_fused_forward(args, torch, fox, q, k, v, x, w_f, b_f, stream)
    if not args.no_skip:  # the same step with exact tile skipping, a separate measurement
        ref = step(None)
        got = step(None, skip=True)
        torch.cuda.synchronize()
        identical = all(torch.equal(a, b) for a, b in zip(ref, got))
        for _ in range(args.warmup):
            step(None, skip=True)
        ev = []
        torch.cuda.synchronize()
        for _ in range(args.steps):
            step(ev, skip=True)
        torch.cuda.synchronize()
        ms = ev[0][1].elapsed_time(ev[-1][2]) / args.steps
        out["skip_decayed"] = {
            "ms_per_step": round(ms, 4),
            "effective_tflops": round(7 * unit / (ms * 1e-3) / 1e12, 2),
            "speedup_vs_dense": round(ms_per_step / ms, 3),
            "bit_identical_to_dense": bool(identical),
            "kernel_ms": {n: round(float(np.mean([a.elapsed_time(b) for m, a, b in ev if m == n])), 4)
                          for n in ["plan"] + names},
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
