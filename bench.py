#!/usr/bin/env python3
"""Benchmark of the SSD forward scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one ssd_scan_fwd call over the Mamba-2 2.7B layer-shape
workload (b=4, L=4096, H=80, P=64, G=1, N=128, chunk 256, bf16 inputs,
fp32 initial and final state), inputs resident in HBM.  W untimed steps
(default 200: back-to-back calls reach the sustained clock after about 150
to 200 calls), then exactly K timed steps (default 100) between two device
synchronisations; value =
b*L*K / elapsed.  Two HIP events on the stream the library launches on
bracket the K steps, giving the call's average duration for the roofline
figure (every launch of the call: the operand records and the walk under
the automatic plan); no event sits between two timed steps (one would add
about 4 us of GPU time per step).  The per-step spread (p10/p90) comes from
a second run of K steps with an event between every two.  Rank 0 prints
one JSON line.

Cold-cache protocol (roofline.cold and extra.configs): 30 repetitions,
each after a 512 MiB device write on the same stream (outside the events)
that evicts L2 and the 256 MB MALL; median with p10/p90.  The warm figure
is the mean of back-to-back calls, each leg after about 30 ms of untimed
back-to-back calls of its own (the clock ramps up under sustained load).

Also reported (context, not the metric): every scan workload under the
automatic plan, the other algorithms, the gated scan, the backward, the
selective scan, the recurrent-step workload (b=256, H=80, P=64, N=128, 64
steps) and the fp64 oracle timed on the host cores (cpu_baseline, all
threads and one thread).

Counter runs (rocprofv3 --pmc) use the same entry with a short leg mix,
e.g. --steps 3 --warmup 1 --no-cpu-baseline --no-configs --copy-probe;
--copy-probe adds a 1 GiB device copy whose FETCH_SIZE / WRITE_SIZE
calibrate the byte counters.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD fwd scan tokens/s and % of roofline, 2.7B layer shape L=4096, 1 GPU"
WORKLOAD = "mamba2_2p7b_b4_L4096_H80_P64_N128"
DECODE = "decode_step_b256_H80_P64_N128_T64"
SSCAN = "mamba1_2p8b_b4_L2048_D5120_N16"
# Vector ALU of MI355X without packed fp32: 256 CUs x 4 SIMDs x 16 lanes at
# 2.4 GHz = 39.3e12 full-rate lane operations per second; a transcendental
# (exp2) occupies four full-rate slots.
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16 MFMA, 256 CU x 4096 FLOP/clk x 2.4 GHz
ELEM = {"bf16": 2, "f32": 4}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "mamba_ssd_scan_05_amd", "csrc")


def scan_bytes(b, L, H, P, G, N, dtype, init, final):
    """Algorithmic bytes: every input read once, every output written once."""
    e = ELEM[dtype]
    n = 2 * b * L * H * P * e            # x in, y out
    n += 2 * b * L * G * N * e           # B, C
    n += b * L * H * 4 + 3 * H * 4       # dt; dt_bias, A, D
    n += (int(init) + int(final)) * b * H * P * N * 4
    return n


def scan_flops(b, L, H, P, G, N, Q):
    """Counted FLOPs of the chunked method: C B^T once per group and chunk,
    causal half of the masked product, chunk states and the state term."""
    nc = (L + Q - 1) // Q
    return b * G * nc * Q * (Q + 1) * N + b * H * nc * (Q * (Q + 1) * P + 4 * Q * N * P)


def step_bytes(b, H, P, G, N, dtype):
    e = ELEM[dtype]
    return 2 * b * H * P * N * 4 + 2 * b * H * P * e + 2 * b * G * N * e + b * H * 4 + 2 * H * 4


# Sources each plan's kernels are built from (the launch plan itself is
# fixed by the shape): counter-derived traffic is used only while these
# files are unchanged since the counters were taken.
PLAN_SOURCES = {
    "rows": ["ssd_rwalk.hip", "ssd_prep.hip", "ssd_device.h", "ssd_internal.h"],
    "chunked": ["ssd_kernels.hip", "ssd_device.h", "ssd_internal.h"],
    "fused": ["ssd_kernels.hip", "ssd_device.h", "ssd_internal.h"],
    "step": ["ssd_kernels.hip", "ssd_device.h", "ssd_internal.h"],
    "bwd": ["ssd_bwd.hip", "ssd_device.h", "ssd_internal.h"],
    "sscan": ["ssd_sscan.hip", "ssd_device.h", "ssd_internal.h"],
}


def kernel_sha(files):
    """Hash of the named kernel sources (sha256, first 16 hex digits)."""
    h = hashlib.sha256()
    for name in sorted(files):
        h.update(name.encode())
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(plan, workload):
    """HBM bytes per call of a plan from committed counter runs (the sum
    over the call's launches), if its kernel sources are unchanged since
    they were taken; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = t.get(plan, {}).get(workload)
    base = plan.split("_seg")[0]
    if not rec or base not in PLAN_SOURCES or rec.get("kernel_source_sha") != kernel_sha(PLAN_SOURCES[base]):
        return None
    return rec.get("hbm_bytes_per_call")


def cpu_baseline(si, reps):
    """The fp64 oracle on the host cores over the whole workload."""
    import oracle
    f = si.f64()
    b, L = si.x.shape[0], si.x.shape[1]
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.scan(**f)
        times.append(time.perf_counter() - t0)
    best = min(times)
    return {"value": b * L / best, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu": cpu_info(),
            "sample": "whole workload (b=4, L=4096, H=80, P=64, N=128, fp64), best of %d runs, "
                      "%.2f s each" % (reps, best)}


def sscan_ops(b, L, Dc, N):
    """Full-rate lane-operation equivalents of one selective scan, counted
    for a single pass of the recurrence: per (token, channel) and state
    index one Delta*A product, one exp2 (4 slots), Delta*x*B, the state
    fma and the readout fma; softplus (two exp2/log2 and five more
    operations) and D*x once per (token, channel)."""
    per = N * (1 + 4 + 1 + 1 + 1) + (2 * 4 + 5) + 1
    return b * L * Dc * per


def bench_sscan(ssd, staging, inputs, torch, dev):
    si = inputs.make_sscan_workload(SSCAN)
    t = staging.sscan_tensors(si, dev)
    out = torch.empty_like(t["x"])
    b, L, Dc = si.x.shape
    N = si.B.shape[3]
    fin = torch.empty((b, Dc, N), dtype=torch.float32, device=dev)
    for _ in range(100):  # ~30 ms of back-to-back calls first
        ssd.ssd_selective_scan_fwd(**t, out=out, final_state=fin)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 50
    e0.record()
    for _ in range(reps):
        ssd.ssd_selective_scan_fwd(**t, out=out, final_state=fin)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    ops = sscan_ops(b, L, Dc, N)
    nbytes = b * L * Dc * (2 * ELEM[si.dtype] + 4) + 2 * b * L * N * ELEM[si.dtype] + Dc * N * 4 \
        + 2 * b * Dc * N * 4 + 2 * Dc * 4
    return {"workload": SSCAN, "ms_per_step": ms, "tokens_per_s": b * L / (ms * 1e-3),
            "roofline": {"bound": "alu", "achieved": ops / (ms * 1e-3) / 1e9,
                         "peak": VALU_LANE_OPS / 1e9, "unit": "G lane-op/s",
                         "frac": ops / (ms * 1e-3) / VALU_LANE_OPS, "ops_per_launch": ops},
            "hbm_GBs": nbytes / (ms * 1e-3) / 1e9, "bytes_per_launch": nbytes}


EVICT_BYTES = 512 << 20   # written between cold reps: more than the 256 MB MALL plus L2
COLD_REPS = 30


def percentiles(ms):
    return {"median_ms": float(np.median(ms)), "p10_ms": float(np.percentile(ms, 10)),
            "p90_ms": float(np.percentile(ms, 90)), "mean_ms": float(np.mean(ms)), "reps": len(ms)}


def time_cold(fn, torch, evict, reps=COLD_REPS):
    """Each rep: a 512 MiB device write on the same stream (outside the events)
    evicts L2 and the MALL, then HIP events bracket one call."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for k in range(reps):
        evict.fill_(k & 0x7f)
        ev[k][0].record()
        fn()
        ev[k][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def time_warm(fn, torch, reps=COLD_REPS):
    """Back-to-back calls, HIP events between consecutive calls."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for k in range(reps):
        fn()
        ev[k + 1].record()
    torch.cuda.synchronize()
    return [ev[k].elapsed_time(ev[k + 1]) for k in range(reps)]


def state_bytes(b, L, H, P, N, Q):
    """One write and one read of the fp32 inter-chunk states of the chunked
    method (chunk Q): the traffic the secondary roofline fraction counts."""
    nc = (L + Q - 1) // Q
    return 2 * b * H * nc * P * N * 4


def bench_scan_config(name, ssd, staging, inputs, torch, dev, evict):
    """One named scan workload under the automatic plan: cold-cache median
    (p10/p90) of 30 reps and warm back-to-back mean, tokens/s and roofline
    fractions (strict: algorithmic bytes and FLOPs; secondary: plus the
    inter-chunk states of the chunked method)."""
    si = inputs.make_workload(name)
    shp = si.shape
    b, L, H, P, G, N = (shp[k] for k in ("b", "L", "H", "P", "G", "N"))
    Q = si.chunk
    t = staging.scan_tensors(si, dev)
    out = torch.empty_like(t["x"])
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)

    def fn():
        ssd.ssd_scan_fwd(**t, out=out, final_state=fin, chunk=Q)
    for _ in range(100):  # to the sustained clock
        fn()
    torch.cuda.synchronize()
    cold = percentiles(time_cold(fn, torch, evict))
    warm = percentiles(time_warm(fn, torch))
    nbytes = scan_bytes(b, L, H, P, G, N, si.dtype, si.init is not None, True)
    flops = scan_flops(b, L, H, P, G, N, Q)
    peak_flops = (MFMA_BF16_PEAK_TFLOPS * 1e12) if si.dtype == inputs.BF16 else MFMA_F32
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / peak_flops
    t_roof = max(t_hbm, t_mfma)
    sec = nbytes + state_bytes(b, L, H, P, N, Q)
    a, seg = ssd.ssd_scan_plan(b, L, H, P, G, N, t["x"].dtype,
                               torch.cuda.get_device_properties(0).multi_processor_count)
    med = cold["median_ms"] * 1e-3
    res = {"workload": name, "dtype": si.dtype, "plan": {"algo": a, "segment": seg},
           "cold": cold, "warm": warm, "tokens_per_s": b * L / med,
           "algorithmic_bytes": nbytes, "counted_flops": flops,
           "bound": "hbm" if t_hbm >= t_mfma else "mfma",
           "roofline_us": t_roof * 1e6, "roofline_tokens_per_s": b * L / t_roof,
           "frac": t_roof / med, "frac_warm": t_roof / (warm["mean_ms"] * 1e-3),
           "achieved_GBs": nbytes / med / 1e9,
           "secondary_bytes": sec, "secondary_frac": (sec / (HBM_PEAK_GBS * 1e9)) / med}
    del t, out, fin
    return res


def cpu_info():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count()}


def cpu_single_thread(names, inputs):
    """The fp64 oracle on one host thread over each named workload (once)."""
    import oracle
    n0 = oracle.num_threads()
    res = {}
    try:
        oracle.set_num_threads(1)
        for name in names:
            si = inputs.make_workload(name)
            f = si.f64()
            b, L = si.x.shape[0], si.x.shape[1]
            t0 = time.perf_counter()
            oracle.scan(**f)
            dt = time.perf_counter() - t0
            res[name] = {"seconds": dt, "tokens_per_s": b * L / dt, "threads": 1}
    finally:
        oracle.set_num_threads(n0)
    return res


MFMA_F32 = 157.3e12   # MI355X dense fp32 matrix peak, FLOP/s
MFMA_BF16 = 2.5e15    # MI355X dense bf16 matrix peak, FLOP/s


def bwd_flops(b, L, H, P, G, N, Q=64):
    """Matrix-product FLOPs of the chunked backward as built: per (batch, head,
    64-token chunk) dY X^T and M^T dY (Q*Q*P each), dY H, B G^T, X G and the
    chunk's own adjoint state (Q*P*N each), (DX o E) B and (DX o E)^T C
    (Q*Q*N each); per (batch, group, chunk) S = C B^T (Q*Q*N); the forward
    chunk-state walk that recomputes the states (Q*P*N per (batch, head,
    chunk)); 2 FLOPs per multiply-add."""
    nc = -(-L // Q)
    per_head = 2 * Q * Q * P + 5 * Q * P * N + 2 * Q * Q * N
    return 2 * (b * H * nc * per_head + b * G * nc * Q * Q * N)


def bench_bwd(ssd, staging, inputs, torch, dev):
    si = inputs.make_workload(WORKLOAD)
    t = staging.scan_tensors(si, dev)
    b, L, H, P = si.x.shape
    G, N = si.B.shape[2], si.B.shape[3]
    g = torch.Generator(device="cpu").manual_seed(1)
    dy = torch.randn((b, L, H, P), generator=g).to(t["x"].dtype).to(dev)
    df = torch.randn((b, H, P, N), generator=g).to(dev)
    out = ssd.ssd_scan_bwd(**t, dout=dy, dfinal_state=df)
    # ~30 ms of back-to-back calls first: the clock settles under sustained load
    for _ in range(20):
        ssd.ssd_scan_bwd(**t, dout=dy, dfinal_state=df, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        ssd.ssd_scan_bwd(**t, dout=dy, dfinal_state=df, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    fl = bwd_flops(b, L, H, P, G, N)
    el = ELEM[si.dtype]
    nbytes = b * L * H * P * (2 * el + 4) + b * L * H * 8 + 2 * b * L * G * N * (el + 4) + 3 * b * H * P * N * 4
    # the contraction runs in bf16 for bf16 inputs (fp32 operands carried as
    # two bf16 parts), in fp32 for fp32 inputs: the peak of that dtype
    peak = MFMA_BF16 if si.dtype == inputs.BF16 else MFMA_F32
    return {"workload": WORKLOAD, "ms_per_step": ms, "tokens_per_s": b * L / (ms * 1e-3),
            "roofline": {"bound": "mfma", "achieved": fl / (ms * 1e-3) / 1e12, "peak": peak / 1e12,
                         "unit": "TFLOP/s", "frac": fl / (ms * 1e-3) / peak, "flops_per_launch": fl,
                         "dtype": "bf16" if si.dtype == inputs.BF16 else "f32",
                         "of_fp32_peak": fl / (ms * 1e-3) / MFMA_F32},
            "hbm_GBs": nbytes / (ms * 1e-3) / 1e9, "bytes_per_launch": nbytes}


def bench_decode(ssd, staging, inputs, torch, dev):
    sp = inputs.make_workload(DECODE)
    t = staging.step_tensors(sp, dev)
    T = sp.x.shape[0]
    for k in range(4):  # warm-up on a copy of the state
        st = t["state"].clone()
        ssd.ssd_step(st, t["x"][k], t["dt"][k], t["A"], t["B"][k], t["C"][k], t["D"])
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(T + 1)]
    ev[0].record()
    for k in range(T):
        ssd.ssd_step(t["state"], t["x"][k], t["dt"][k], t["A"], t["B"][k], t["C"][k], t["D"])
        ev[k + 1].record()
    torch.cuda.synchronize()
    per = [ev[k].elapsed_time(ev[k + 1]) for k in range(T)]
    avg_ms = float(np.mean(per))
    stats = percentiles(per)
    b, H, P, N = sp.state.shape
    G = sp.B.shape[2]
    nbytes = step_bytes(b, H, P, G, N, sp.dtype)
    return {"workload": DECODE, "tokens_per_s": b / (avg_ms * 1e-3), "ms_per_step": avg_ms,
            "achieved_GBs": nbytes / (avg_ms * 1e-3) / 1e9, "peak_GBs": HBM_PEAK_GBS,
            "frac": nbytes / (avg_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "bytes_per_step": nbytes,
            "per_step": stats,
            "frac_median": nbytes / (stats["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # back-to-back calls settle only after ~150-200 calls (the clock ramps
    # up under sustained load): 200 untimed steps, about 35 ms
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--algo", choices=["auto", "fused", "chunked", "rows"], default="auto")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward (gradients) leg")
    ap.add_argument("--no-sscan", action="store_true",
                    help="skip the timing of the selective scan (diagonal A per channel)")
    ap.add_argument("--no-gated", action="store_true",
                    help="skip the timing of the gated scan (out = y * silu(z))")
    ap.add_argument("--no-alt", action="store_true", help="skip timing the other algorithm")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload table (all scan workloads, cold-cache protocol)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the SSD scan here runs on a single MI355X "
              "(no collectives); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch
    from mamba_ssd_scan_05_amd import inputs, ssd, staging

    # Python's cyclic garbage collector stays off while the legs run (a
    # collection inside a timed loop stalled the host ~38 ms, long enough
    # for the queued GPU work to drain); each leg starts after a collection.
    gc.collect()
    gc.disable()

    dev = "cuda:0"
    torch.cuda.set_device(0)
    names = {ssd.SSD_ALGO_FUSED: "fused", ssd.SSD_ALGO_CHUNKED: "chunked", ssd.SSD_ALGO_ROWS: "rows"}
    algo = {"auto": ssd.SSD_ALGO_AUTO, "fused": ssd.SSD_ALGO_FUSED,
            "chunked": ssd.SSD_ALGO_CHUNKED, "rows": ssd.SSD_ALGO_ROWS}[args.algo]
    si = inputs.make_workload(args.workload)
    shp = si.shape
    b, L, H, P, G, N = (shp[k] for k in ("b", "L", "H", "P", "G", "N"))
    Q = si.chunk
    t = staging.scan_tensors(si, dev)
    out = torch.empty_like(t["x"])
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)

    def one(a=algo):
        ssd.ssd_scan_fwd(**t, out=out, final_state=fin, chunk=Q, algo=a)

    print("bench: workload %s algo %s warmup %d steps %d" % (args.workload, args.algo,
                                                              args.warmup, args.steps),
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    # The timed steps run back to back with HIP events only around the whole
    # run (an event recorded between two calls adds ~4 us of GPU time per
    # step); the kernel average is the event span over the steps.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for k in range(args.steps):
        one()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = e0.elapsed_time(e1) / args.steps
    # per-step spread from a separate run with an event between every two steps
    per_ms = time_warm(one, torch, reps=args.steps)
    ms_per_step = elapsed * 1e3 / args.steps
    tokens = b * L
    value = tokens * args.steps / elapsed

    nbytes = scan_bytes(b, L, H, P, G, N, si.dtype, si.init is not None, True)
    flops = scan_flops(b, L, H, P, G, N, Q)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    used_algo, seg_len = args.algo, Q
    if args.algo == "auto":
        a, seg_len = ssd.ssd_scan_plan(b, L, H, P, G, N, t["x"].dtype,
                                       torch.cuda.get_device_properties(0).multi_processor_count)
        used_algo = names[a]
    if used_algo == "fused":
        dominant = "walk_kernel (fused walk, one launch)"
        seg_len = L
    elif used_algo == "rows":
        dominant = ("rwalk_kernel (row-sliced walk) with its prep_kernel operand records: "
                    "the timed duration is the whole call, both launches")
        seg_len = L
    else:
        dominant = ("ssd_scan_fwd chunked path, segment %d: cumsum + chunk-state walk + "
                    "state pass + chunk-output walk (4 launches)" % seg_len)
    plan_key = "%s_seg%d" % (used_algo, seg_len)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS,
                "traffic": load_traffic(plan_key, args.workload),
                "kernel": dominant, "kernel_avg_ms": kern_ms,
                "algorithmic_bytes_per_launch": nbytes, "bytes_per_token": nbytes / tokens,
                "counted_flops": flops, "t_hbm_us": t_hbm * 1e6, "t_mfma_us": t_mfma * 1e6,
                "roofline_tokens_per_s": tokens / max(t_hbm, t_mfma),
                "mfma_frac": flops / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS}

    extra = {"p10_ms": float(np.percentile(per_ms, 10)), "p90_ms": float(np.percentile(per_ms, 90)),
             "median_ms": float(np.median(per_ms)),
             "per_step_spread": "p10/p90/median from a second run of the same steps with an event "
                                "between every two (those events add ~4 us per step)"}
    # cold-cache protocol: 30 reps, each after a 512 MiB eviction write on the
    # same stream outside the events; median with p10/p90
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    cold = percentiles(time_cold(one, torch, evict))
    roofline["cold"] = cold
    roofline["frac_cold_median"] = nbytes / (cold["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
    roofline["secondary_frac_cold_median"] = (
        (nbytes + state_bytes(b, L, H, P, N, Q)) / (cold["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS)
    if not args.no_configs:
        # every scan workload under the automatic plan, the same protocol
        extra["configs"] = {}
        for name in inputs.WORKLOAD_ORDER:
            if inputs.WORKLOADS[name]["kind"] != "scan":
                continue
            print("bench: config %s" % name, file=sys.stderr, flush=True)
            gc.collect()
            extra["configs"][name] = bench_scan_config(name, ssd, staging, inputs, torch, dev, evict)
    if not args.no_alt:
        gc.collect()
        alts = {}
        for name_a, a, q in (("rows", ssd.SSD_ALGO_ROWS, Q), ("fused", ssd.SSD_ALGO_FUSED, Q),
                             ("chunked_256", ssd.SSD_ALGO_CHUNKED, 256),
                             ("chunked_1024", ssd.SSD_ALGO_CHUNKED, 1024),
                             ("chunked_2048", ssd.SSD_ALGO_CHUNKED, 2048)):
            def run_alt():
                ssd.ssd_scan_fwd(**t, out=out, final_state=fin, chunk=q, algo=a)
            try:
                run_alt()
            except ssd.SsdError:  # plan not available for this shape or dtype
                alts[name_a] = None
                continue
            for _ in range(100):  # ~20-30 ms of back-to-back calls first
                run_alt()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                run_alt()
            e1.record()
            torch.cuda.synchronize()
            alts[name_a] = e0.elapsed_time(e1) / 20
        extra["algorithms_ms"] = alts
    if not args.no_gated:
        gc.collect()
        # the scan with the output gate fused (out = y * silu(z)): the same
        # automatic plan, z read once more (the bytes of x)
        z = staging.tensor(inputs.make_gate(si), si.dtype, dev)

        def run_gated():
            ssd.ssd_scan_fwd_gated(**t, z=z, out=out, final_state=fin, chunk=Q)
        for _ in range(150):  # ~35 ms of back-to-back calls first
            run_gated()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            run_gated()
        e1.record()
        torch.cuda.synchronize()
        g_ms = e0.elapsed_time(e1) / 50
        g_bytes = nbytes + b * L * H * P * ELEM[si.dtype]
        extra["gated"] = {"ms_per_step": g_ms, "tokens_per_s": tokens / (g_ms * 1e-3),
                          "algorithmic_bytes": g_bytes,
                          "achieved_GBs": g_bytes / (g_ms * 1e-3) / 1e9,
                          "frac": g_bytes / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "ungated_ms_per_step": kern_ms}
        del z
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_probe_bytes"] = 2 * (1 << 30)
    if not args.no_bwd:
        print("bench: backward", WORKLOAD, file=sys.stderr, flush=True)
        gc.collect()
        extra["backward"] = bench_bwd(ssd, staging, inputs, torch, dev)
    if not args.no_sscan:
        print("bench: selective scan %s" % SSCAN, file=sys.stderr, flush=True)
        gc.collect()
        extra["selective_scan"] = bench_sscan(ssd, staging, inputs, torch, dev)
    if not args.no_decode:
        print("bench: decode step workload", file=sys.stderr, flush=True)
        gc.collect()
        extra["decode_step"] = bench_decode(ssd, staging, inputs, torch, dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(si, reps=2)
        print("bench: cpu baseline, one thread", file=sys.stderr, flush=True)
        cpu["single_thread"] = cpu_single_thread(
            ["tiny_fp32_b1_L256_H4_P16_N16", WORKLOAD], inputs)

    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": si.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "b": b, "L": L, "H": H, "P": P, "G": G, "N": N,
                   "chunk": Q, "init_state": si.init is not None, "algo": used_algo,
                   "segment": seg_len},
        "roofline": roofline, "cpu_baseline": cpu, "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
