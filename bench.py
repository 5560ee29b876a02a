#!/usr/bin/env python3
"""Throughput of the affine-recurrence look-back scan (and, as secondary lines
of the same record, the S6 selective scan) on one MI355X.

A step is one pass of the linear recurrence h[t] = a[t] h[t-1] + b[t] over a
single fp32 sequence of n = 2^27 elements (a ~ U(0.5, 1), b ~ N(0, 1), h0 = 0),
inputs resident in HBM. `value` is elements per second over the timed steps.
The S6 workloads (forward fp32 16x1024x256, forward bf16 1x65536x1024,
bidirectional bf16 4x8192x1536, N = 16) are timed the same way and reported
under "s6". Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
CUS, CLOCK_GHZ, LANES = 256, 2.4, 64
VALU_PEAK_T = CUS * LANES * CLOCK_GHZ / 1e3   # 39.32 T lane-instructions/s (fp32, unpacked)
LINEAR_WORKLOAD = "linear-n134217728"
LINEAR_BYTES_PER_ELEM = 12     # read a, b; write h (fp32)
PROFILES = ROOT / "profiles"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        h.update((ROOT / "mamba_s6_selective_amd" / "csrc" / n).read_bytes())
    return h.hexdigest()[:16]


def load_traffic(kind, *kernel_srcs):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or
    None if absent or taken on a different kernel source."""
    f = PROFILES / f"{kind}_traffic.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text())
    if d.get("kernel_source_sha") != source_hash(*kernel_srcs):
        return None
    return d.get("bytes_per_launch")


# Untimed work before each timed section lasts at least SETTLE["s"] seconds
# (--settle-seconds). After an idle spell the GPU's clocks ramp for about a second under load: the
# long S6 workload measured 336-380 us per call over its first 40 calls and
# 315 us once settled, the 2^27 linear scan 358 us on its first call and
# 272-285 us before settling at ~273 us.
SETTLE = {"s": 1.0}


def load_s6_traffic(name):
    """HBM bytes of one S6 call (chunk + carry + fix passes) on workload `name`
    from committed rocprofv3 counter summaries, or None if absent or taken on
    a different kernel source."""
    f = PROFILES / "s6_traffic.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text()).get(name)
    if not d or d.get("kernel_source_sha") != source_hash("s6_scan.hip", "s6_internal.h"):
        return None
    return d.get("bytes_per_launch")


def load_s6_valu(name):
    """rocprofv3 VALUBusy (per cent of GPU time the VALUs issue) and VALU
    instructions per (b, t, d, n) of each S6 pass on workload `name`, from a
    committed counter summary, or None if absent or taken on a different
    kernel source."""
    f = PROFILES / "s6_valu.json"
    if not f.exists():
        return None
    d = json.loads(f.read_text()).get(name)
    if not d or d.get("kernel_source_sha") != source_hash("s6_scan.hip", "s6_internal.h"):
        return None
    return d.get("kernels")


def time_steps(fn, steps, warmup):
    """Runs fn() warmup times (and on, untimed, until SETTLE["s"] seconds have
    passed, so that the clocks have settled), then `steps` timed times
    back to back. Returns the wall time per step and the GPU time per step
    from one HIP event pair around the timed steps on torch's current stream
    (where the library launches): an event pair around every step would put
    two timestamp packets between consecutive launches, which measured about
    7 us per step of added wall time on the 2^27 linear scan."""
    import torch
    t_settle = time.perf_counter() + SETTLE["s"]
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while time.perf_counter() < t_settle:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, start.elapsed_time(end) / steps


def sentinel_ok(dev):
    import torch
    import mamba_s6_selective_amd as ssm
    x = torch.arange(1 << 22, dtype=torch.float32, device=dev) * 0.5 - 7.0
    y = torch.empty_like(x)
    ssm.copy_f32(x, y)
    torch.cuda.synchronize()
    return bool(torch.equal(x, y))


def bench_linear(dev, steps, warmup):
    import torch
    import mamba_s6_selective_amd as ssm
    from mamba_s6_selective_amd.workloads import LINEAR_WORKLOADS, linear_workload_inputs
    n = LINEAR_WORKLOADS[LINEAR_WORKLOAD]["n"]
    a, b = linear_workload_inputs(LINEAR_WORKLOAD)
    a, b = a.to(dev), b.to(dev)
    h = torch.empty_like(a)
    ms_step, ms_kernel = time_steps(lambda: ssm.linear_scan(a, b, 0.0, out=h), steps, warmup)
    return n, ms_step, ms_kernel


def bench_linear_small(dev, steps, warmup):
    """The n = 65,536 workload (a ~ U(0.9, 1)): its 786 KB stay in L2, so one
    call is bound by launch and look-back latency, not by HBM. Reported as the
    latency of one call (host clock around a call and a synchronisation,
    median of 200) and as elements/s of calls issued back to back."""
    import torch
    import mamba_s6_selective_amd as ssm
    from mamba_s6_selective_amd.workloads import LINEAR_WORKLOADS, linear_workload_inputs
    name = "linear-n65536"
    n = LINEAR_WORKLOADS[name]["n"]
    a, b = linear_workload_inputs(name)
    a, b = a.to(dev), b.to(dev)
    h = torch.empty_like(a)
    _, ms_kernel = time_steps(lambda: ssm.linear_scan(a, b, 0.0, out=h), steps * 10, warmup)
    lat = []
    for _ in range(200):
        t0 = time.perf_counter()
        ssm.linear_scan(a, b, 0.0, out=h)
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - t0)
    return {"workload": name, "n": n, "latency_us": round(statistics.median(lat) * 1e6, 2),
            "ms_per_launch_back_to_back": round(ms_kernel, 5),
            "elements_per_s": n / (ms_kernel * 1e-3)}


def bench_linear_3pass(dev, steps, warmup, ms_single):
    """The three-pass design on the same workload, for the pages' traffic model:
    28 B/element (read a, b; write and re-read the in-tile compositions A, B;
    write h) against the single pass's 12, so a predicted ratio of 28/12."""
    import torch
    import mamba_s6_selective_amd as ssm
    from mamba_s6_selective_amd.workloads import LINEAR_WORKLOADS, linear_workload_inputs
    n = LINEAR_WORKLOADS[LINEAR_WORKLOAD]["n"]
    a, b = linear_workload_inputs(LINEAR_WORKLOAD)
    a, b = a.to(dev), b.to(dev)
    h = torch.empty_like(a)
    _, ms_kernel = time_steps(lambda: ssm.linear_scan_3pass(a, b, 0.0, out=h), steps, warmup)
    # the same three passes with a register-resident Hillis-Steele local pass
    _, ms_hs = time_steps(lambda: ssm.linear_scan_hs(a, b, 0.0, out=h), steps, warmup)
    return {
        "workload": LINEAR_WORKLOAD, "ms_per_launch": round(ms_kernel, 4),
        "hillis_steele_ms_per_launch": round(ms_hs, 4),
        "hillis_steele_ratio": round(ms_hs / ms_kernel, 3),
        "bytes_per_elem": 28, "single_pass_bytes_per_elem": LINEAR_BYTES_PER_ELEM,
        "achieved_GBs": round(28 * n / (ms_kernel * 1e-3) / 1e9, 1),
        "predicted_ratio": round(28 / LINEAR_BYTES_PER_ELEM, 3),
        "measured_ratio": round(ms_kernel / ms_single, 3),
    }


def bench_linear_batched(dev, steps, warmup, nseq=4096, length=32768):
    """The batched form (independent sequences with their own h0 and h_last)
    on the same 2^27 elements and distributions, as nseq x length."""
    import torch
    import mamba_s6_selective_amd as ssm
    from mamba_s6_selective_amd.workloads import LINEAR_WORKLOADS, linear_workload_inputs
    a, b = linear_workload_inputs(LINEAR_WORKLOAD)
    assert a.numel() == nseq * length
    a, b = a.to(dev).view(nseq, length), b.to(dev).view(nseq, length)
    h0 = torch.zeros(nseq, device=dev)
    h = torch.empty_like(a)
    last = torch.empty(nseq, device=dev)
    _, ms_kernel = time_steps(lambda: ssm.linear_scan_batched(a, b, h0, out=h, h_last=last),
                                 steps, warmup)
    nbytes = 12 * a.numel() + 8 * nseq
    return {"workload": f"{LINEAR_WORKLOAD} as {nseq} x {length}",
            "ms_per_launch": round(ms_kernel, 4),
            "elements_per_s": a.numel() / (ms_kernel * 1e-3),
            "achieved_GBs": round(nbytes / (ms_kernel * 1e-3) / 1e9, 1)}


def bench_copy(dev, steps, warmup):
    import torch
    import mamba_s6_selective_amd as ssm
    n = 1 << 28
    x = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
    y = torch.empty_like(x)
    _, ms_kernel = time_steps(lambda: ssm.copy_f32(x, y), steps, warmup)
    return 8.0 * n / (ms_kernel * 1e-3) / 1e9


def bench_stream(dev, steps, warmup, n):
    """The library's stream kernel, h = a * b over n floats: the linear
    scan's 12 bytes per element with no recurrence, in the launch shape that
    measured fastest for that traffic -- the rate the scan can approach."""
    import torch
    import mamba_s6_selective_amd as ssm
    a = torch.empty(n, dtype=torch.float32, device=dev).uniform_(0.5, 1.0)
    b = torch.empty(n, dtype=torch.float32, device=dev).normal_()
    h = torch.empty_like(a)
    _, ms_kernel = time_steps(lambda: ssm.stream_mul_f32(a, b, out=h), steps, warmup)
    return LINEAR_BYTES_PER_ELEM * n / (ms_kernel * 1e-3) / 1e9, ms_kernel


S6_BENCH = ["s6-fwd-b16-L1024-d256-N16-f32", "s6-fwd-b1-L65536-d1024-N16-bf16",
            "s6-bidir-b4-L8192-d1536-N16-bf16"]


def s6_algorithmic(w):
    """Algorithmic HBM bytes and VALU lane-instructions per step.

    Bytes: u and delta read once, y written once (fp32), B and C read once,
    A and D read once. VALU per (b, t, d, n): delta*A, the exponential, dBu,
    the state FMA and the output FMA (one exponential, four other
    instructions); the bidirectional pass adds one state FMA and one output
    FMA for the second direction (shared discretization).
    """
    es = 2 if w["dtype"] == "bf16" else 4
    E = w["batch"] * w["L"] * w["d_inner"]
    nbytes = E * (2 * es + 4) + 2 * w["batch"] * w["L"] * w["N"] * es + \
        w["d_inner"] * (w["N"] + 1) * 4
    other = 6 if w["direction"] == "bidir" else 4
    return E, nbytes, E * w["N"], other


def bench_s6(dev, name, steps, warmup, exp_cost, extras=True):
    import torch
    import mamba_s6_selective_amd as ssm
    from mamba_s6_selective_amd.workloads import S6_WORKLOADS, s6_workload_inputs
    w = S6_WORKLOADS[name]
    inp = s6_workload_inputs(name)
    E, nbytes, tdn, other = s6_algorithmic(w)
    # Rotate input sets so the working set (over 512 MB) exceeds the 256 MB
    # Infinity Cache.
    sets = max(2, min(16, math.ceil(6.0e8 / max(nbytes, 1))))
    bufs = []
    for _ in range(sets):
        bufs.append([x.to(dev).clone() for x in (inp.u, inp.delta, inp.A, inp.B, inp.C, inp.D)]
                    + [torch.empty(inp.u.shape, dtype=torch.float32, device=dev)])
    k = [0]

    def step():
        t = bufs[k[0] % sets]
        k[0] += 1
        ssm.selective_scan_fwd(*t[:6], direction=w["direction"], out=t[6])

    ms_step, ms_kernel = time_steps(step, steps, warmup)
    extra = {}
    fused = None
    if extras and w["direction"] == "fwd" and w["dtype"] == "bf16":
        # the same scan with delta given before its activation and softplus fused in
        pre = [inp.delta_pre.to(dev).clone() for _ in range(sets)]
        dl = [torch.empty_like(p) for p in pre]

        def step_fused():
            t = bufs[k[0] % sets]
            ssm.selective_scan_fwd(t[0], pre[k[0] % sets], *t[2:6], direction=w["direction"],
                                   out=t[6], delta_softplus=True)
            k[0] += 1

        def step_softplus():  # the separate elementwise pass the fusion saves
            j = k[0] % sets
            torch.nn.functional.softplus(pre[j], out=dl[j])
            k[0] += 1

        def step_separate():  # that pass, then the scan on its output
            j = k[0] % sets
            t = bufs[j]
            torch.nn.functional.softplus(pre[j], out=dl[j])
            ssm.selective_scan_fwd(t[0], dl[j], *t[2:6], direction=w["direction"], out=t[6])
            k[0] += 1

        _, ms_fused = time_steps(step_fused, steps, warmup)
        _, ms_sp = time_steps(step_softplus, steps, warmup)
        _, ms_sep = time_steps(step_separate, steps, warmup)
        fused = {"ms_kernel_avg": round(ms_fused, 4),
                 "ratio_to_unfused": round(ms_fused / ms_kernel, 3),
                 "separate_pass_bytes": 2 * E * (2 if w["dtype"] == "bf16" else 4),
                 "separate_softplus_ms": round(ms_sp, 4),
                 "separate_softplus_then_scan_ms": round(ms_sep, 4),
                 "ratio_to_separate": round(ms_fused / ms_sep, 3)}
        # The fix pass leaves out carry terms once they are proven below 2^-24,
        # so its cost depends on how fast the states decay: with every term
        # evaluated, and with A 64 times closer to 0.
        os.environ["SSMSCAN_S6_FULL_FIX"] = "1"
        try:
            _, ms_full = time_steps(step, steps, warmup)
        finally:
            del os.environ["SSMSCAN_S6_FULL_FIX"]
        for t in bufs:
            t[2].div_(64.0)  # A[d, n] = -(n + 1) / 64
        try:
            _, ms_slow = time_steps(step, steps, warmup)
        finally:
            for t in bufs:
                t[2].mul_(64.0)
        extra["general_A"] = {
            "full_fix_ms": round(ms_full, 4), "ratio_full_fix": round(ms_full / ms_kernel, 3),
            "slow_decay_A": "-(n+1)/64", "slow_decay_ms": round(ms_slow, 4),
            "ratio_slow_decay": round(ms_slow / ms_kernel, 3)}
    if extras and w["direction"] == "bidir":
        # the fused call against one forward and one reverse call on the same inputs
        def step_separate_dirs():
            t = bufs[k[0] % sets]
            ssm.selective_scan_fwd(*t[:6], direction="fwd", out=t[6])
            ssm.selective_scan_fwd(*t[:6], direction="rev", out=t[6])
            k[0] += 1

        _, ms_two = time_steps(step_separate_dirs, steps, warmup)
        extra["fusion"] = {"separate_fwd_plus_rev_ms": round(ms_two, 4),
                           "fusion_ratio": round(ms_two / ms_kernel, 3)}
    lane_cycles = tdn * (other + exp_cost)
    alu_frac = lane_cycles / (ms_kernel * 1e-3) / (VALU_PEAK_T * 1e12)
    gbs = nbytes / (ms_kernel * 1e-3) / 1e9
    return {
        "workload": name, "ms_per_step": round(ms_step, 4), "ms_kernel_avg": round(ms_kernel, 4),
        "elements_per_s": E / (ms_step * 1e-3), "rotating_sets": sets,
        "roofline": {"bound": "alu", "achieved": round(lane_cycles / (ms_kernel * 1e-3) / 1e12, 3),
                     "peak": round(VALU_PEAK_T, 2), "unit": "T lane-cycles/s",
                     "frac": round(alu_frac, 4), "exp_cost_lane_cycles": exp_cost,
                     "traffic": load_s6_traffic(name)},
        "hbm": {"achieved_GBs": round(gbs, 1), "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4),
                "algorithmic_bytes": nbytes},
        "valu_rocprof": load_s6_valu(name),
        "fused_softplus": fused,
        **extra,
    }


def cpu_baseline(budget_s):
    """The float64 C oracle on the same workload, single thread (the recurrence
    is sequential), repeated for about `budget_s` seconds."""
    import numpy as np
    from mamba_s6_selective_amd.workloads import LINEAR_WORKLOADS, linear_workload_inputs
    from oracle import native
    n = LINEAR_WORKLOADS[LINEAR_WORKLOAD]["n"]
    a, b = linear_workload_inputs(LINEAR_WORKLOAD)
    a = a.numpy().astype(np.float64)
    b = b.numpy().astype(np.float64)
    native.load()
    times = []
    t_end = time.perf_counter() + budget_s
    while not times or (time.perf_counter() < t_end and len(times) < 50):
        t0 = time.perf_counter()
        native.linear_scan(a, b, 0.0)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"value": n / med, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"whole n=2^27 sequence, float64 C loop, {len(times)} passes "
                      f"(median {med:.3f} s)"}


def cpu_baseline_small():
    """The float64 C oracle on the whole n = 65,536 workload, single thread."""
    import numpy as np
    from mamba_s6_selective_amd.workloads import linear_workload_inputs
    from oracle import native
    a, b = linear_workload_inputs("linear-n65536")
    a = a.numpy().astype(np.float64)
    b = b.numpy().astype(np.float64)
    native.load()
    times = []
    for _ in range(50):
        t0 = time.perf_counter()
        native.linear_scan(a, b, 0.0)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"value": a.size / med, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"whole n=65536 sequence, float64 C loop, 50 passes (median {med * 1e6:.0f} us)"}


def cpu_baseline_batched(budget_s, nseq=4096, length=32768):
    """The float64 C oracle on the batched form of the same 2^27 elements:
    one sequential loop per sequence (h0 = 0), over as many sequences as
    about budget_s allows."""
    import numpy as np
    from mamba_s6_selective_amd.workloads import linear_workload_inputs
    from oracle import native
    a, b = linear_workload_inputs(LINEAR_WORKLOAD)
    a = a.numpy().astype(np.float64).reshape(nseq, length)
    b = b.numpy().astype(np.float64).reshape(nseq, length)
    native.load()
    done = 0
    t0 = time.perf_counter()
    while done < nseq and (done == 0 or time.perf_counter() - t0 < budget_s):
        native.linear_scan(a[done], b[done], 0.0)
        done += 1
    dt = time.perf_counter() - t0
    return {"value": done * length / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"sequences [0, {done}) of {nseq} x {length}, float64 C loop, "
                      f"{dt:.2f} s"}


def cpu_baseline_s6(name, budget_s):
    """The float64 C oracle on a bounded sample of an S6 workload: the first
    k (batch, channel) sequences over all L steps, k doubled until one pass
    takes about budget_s / 4, then repeated for about budget_s seconds."""
    import numpy as np
    from mamba_s6_selective_amd.workloads import S6_WORKLOADS, s6_workload_inputs
    from oracle import native
    w = S6_WORKLOADS[name]
    u, dl, A, B, C, D = s6_workload_inputs(name).as_f64()
    channels = w["batch"] * w["d_inner"]
    out = np.empty(u.shape, dtype=np.float64)
    native.load()

    def one(k):
        t0 = time.perf_counter()
        _, used = native.selective_scan(u, dl, A, B, C, D, w["direction"], 0, k, 0, out)
        return time.perf_counter() - t0, used

    k = 8
    dt, used = one(k)
    while dt < budget_s / 4 and k < channels:
        k = min(channels, 2 * k)
        dt, used = one(k)
    times = [dt]
    t_end = time.perf_counter() + budget_s
    while time.perf_counter() < t_end and len(times) < 20:
        times.append(one(k)[0])
    med = statistics.median(times)
    return {"value": k * w["L"] / med, "unit": "elements/s", "cores": used, "kind": "oracle",
            "sample": f"(batch, channel) sequences [0, {k}) of {channels}, all {w['L']} steps "
                      f"({w['direction']}), float64 C loop over OpenMP threads, {len(times)} passes "
                      f"(median {med:.3f} s)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-s6", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="S6: time only the workload itself (no fused-softplus, full-fix, "
                         "slow-decay or separate fwd + rev variants), so that a counter run "
                         "sees only its launches")
    ap.add_argument("--s6-only", choices=S6_BENCH,
                    help="time only this S6 workload (for per-workload profiles) and print its record")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--exp-cost", type=float, default=2.0,
                    help="lane-cycles one v_exp_f32 occupies relative to an FMA")
    ap.add_argument("--settle-seconds", type=float, default=SETTLE["s"],
                    help="least untimed run time before each timed section (clock ramp)")
    args = ap.parse_args()
    SETTLE["s"] = args.settle_seconds
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the scan runs on a single device and this "
              "build has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import mamba_s6_selective_amd as ssm
    ssm.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")
    if not sentinel_ok(dev):
        raise SystemExit("sentinel copy kernel did not reproduce its input; sweep discarded")

    if args.s6_only:
        print(json.dumps(bench_s6(dev, args.s6_only, args.steps, args.warmup, args.exp_cost,
                                  extras=not args.no_extras)),
              flush=True)
        return
    copy_gbs = bench_copy(dev, 10, 3)
    log(f"copy kernel: {copy_gbs:.0f} GB/s")
    n, ms_step, ms_kernel = bench_linear(dev, args.steps, args.warmup)
    alg_bytes = LINEAR_BYTES_PER_ELEM * n
    achieved = alg_bytes / (ms_kernel * 1e-3) / 1e9
    log(f"linear scan: {ms_kernel * 1e3:.1f} us/launch, {achieved:.0f} GB/s algorithmic")
    stream_gbs, stream_ms = bench_stream(dev, args.steps, args.warmup, n)
    log(f"stream reference: {stream_ms * 1e3:.1f} us/launch, {stream_gbs:.0f} GB/s; "
        f"scan at {achieved / stream_gbs:.3f} of it")
    traffic = load_traffic("linear_scan", "linear_scan.hip", "scan_common.h")
    record = {
        "metric": "scan elements/s + achieved HBM GB/s (% of MI355X peak), linear & S6 fwd",
        "value": n / (ms_step * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "settle_s": args.settle_seconds,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded; pages' distributions)",
        "config": {"workload": LINEAR_WORKLOAD, "n": n, "h0": 0.0,
                   "a": "U(0.5,1)", "b": "N(0,1)", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "copy_kernel_GBs": round(copy_gbs, 1),
        "stream_reference": {"kernel": "stream_mul_kernel: h = a * b, 12 B/element, "
                                       "one 16-byte vector per lane, 256 lanes per workgroup",
                             "n": n, "ms_per_launch": round(stream_ms, 5),
                             "achieved_GBs": round(stream_gbs, 1),
                             "frac_of_8TBs": round(stream_gbs / HBM_PEAK_GBS, 4),
                             "scan_frac_of_stream": round(achieved / stream_gbs, 4)},
    }
    record["linear_n65536"] = bench_linear_small(dev, args.steps, args.warmup)
    log(f"linear n=65536: {record['linear_n65536']['latency_us']} us per synchronised call")
    record["three_pass"] = bench_linear_3pass(dev, max(5, args.steps // 2), 2, ms_kernel)
    log(f"three-pass: {record['three_pass']['ms_per_launch'] * 1e3:.1f} us, ratio "
        f"{record['three_pass']['measured_ratio']} (model {record['three_pass']['predicted_ratio']})")
    record["batched"] = bench_linear_batched(dev, max(5, args.steps // 2), 2)
    log(f"batched: {record['batched']['ms_per_launch'] * 1e3:.1f} us, "
        f"{record['batched']['achieved_GBs']} GB/s")
    if not args.no_s6:
        record["s6"] = [bench_s6(dev, name, max(5, args.steps // 2), 2, args.exp_cost)
                        for name in S6_BENCH]
        for r in record["s6"]:
            log(f"{r['workload']}: {r['ms_kernel_avg'] * 1e3:.1f} us, "
                f"alu frac {r['roofline']['frac']:.3f}, hbm frac {r['hbm']['frac_of_8TBs']:.3f}")
    if not args.no_cpu_baseline:
        record["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        # the three-pass scan computes the same workload: the same oracle run
        record["three_pass"]["cpu_baseline"] = record["cpu_baseline"]
        record["linear_n65536"]["cpu_baseline"] = cpu_baseline_small()
        record["batched"]["cpu_baseline"] = cpu_baseline_batched(args.cpu_seconds / 4)
        for r in record.get("s6", []):
            r["cpu_baseline"] = cpu_baseline_s6(r["workload"], args.cpu_seconds / 4)
            log(f"{r['workload']}: oracle {r['cpu_baseline']['value']:.3g} elements/s on "
                f"{r['cpu_baseline']['cores']} threads")
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
