#!/usr/bin/env python3
"""Benchmark: exact attention forward + recompute backward on one MI355X.

One step is the whole hot path over one batch of synthetic inputs:
fa_fwd (fused forward, writes O and lse) followed by the backward's two
stages fa_bwd_dq_first (query-outer: dQ, plus the row terms D = rowsum(dO*O)
and lse*log2(e) for the next stage) and fa_bwd_main (key-outer: dK, dV) --
exactly what fa_bwd enqueues.
Workload: B=2, H=16, N=4096, d=128, bf16, causal, iid N(0,1) inputs (seed 0).

Prints one JSON line.  `value` is the whole step's throughput in TFLOP/s with
the FLOP convention 4*B*H*N^2*d for the forward (halved for causal) and 2.5x
that for the backward; inputs are resident in HBM before timing starts.
The K timed steps enqueue nothing but the step's own launches; K further
steps with HIP events recorded on the launch stream around every call give
the per-call times, and `roofline` reports the backward's key-outer kernel
(the dominant one: four of the five products) from them against the bf16
dense matrix-core peak.  `cpu_baseline` times the fp64 oracle on a
bounded sample of the same workload (a few heads).

Timing: W untimed warm-up steps, then untimed settle steps until --settle-s
seconds (default 0.3) of sustained load have passed -- the GPU's shader clock
ramps up over about a tenth of a second, so the K timed steps measure the
steady state (their count is reported as `settle_steps`) -- then exactly K
timed steps.  `call_us` gives the median, p10 and p90 of every entry point's
per-call event time.

Options: --steps K --warmup W (timed / untimed steps), --gpus N (only 1 is
supported: the implementation runs on a single GPU), --workload NAME (another
workload of workloads.WORKLOADS, forward only unless it has a backward; the
paged decode workload reports GB/s against the HBM peak),
--no-cpu-baseline, --copy-calib (run a plain device copy first, for the
profiler's traffic calibration), --settle-s S, --launch stream|graph (the
timed steps as separate launches on the stream, or replays of one captured
HIP graph of the step, checked bit for bit against the eager step first).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402
from workloads import accounting as A  # noqa: E402

METRIC = "attention fwd/bwd TFLOP/s (4·B·H·N²·d, causal halved) and % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 bf16 FLOP/clk x 2.4 GHz, dense
PEAK_FP8_TFLOPS = 5033.2   # 256 CU x 8192 fp8 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "bf16_causal_fwdbwd_b2h16n4096d128"


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def kernel_source_digest(names) -> str:
    """sha256 of the kernel sources with // comments and blank lines removed
    (a comment edit does not change the counted kernels)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_io_aware_59_amd", "csrc", n)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(workload: str, kernel_api: str):
    """HBM bytes per launch of `kernel_api` from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy's readings), or
    None when that summary is for another workload or the kernel sources have
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)["workloads"][workload]
        src = kernel_source_digest(t["sources"])
    except (OSError, KeyError, ValueError):
        return None
    if src != t.get("kernel_source_sha256"):
        return None
    return t["per_launch"].get(kernel_api)


def cpu_baseline(w, x, mask_np, heads: int) -> dict:
    """Time the fp64 oracle as it stands on a bounded sample of the workload.

    Sample: forward (and backward) of the first `heads` heads of batch 0 when
    a head's N x N matrices fit comfortably (N <= 8192); otherwise 512 seeded
    sampled rows of the forward.
    """
    import oracle
    sl = (slice(0, 1), slice(0, heads))
    window, slopes = W.workload_variant(w)
    var = {}
    if w.variant:
        var = dict(window=window, slopes=None if slopes is None else slopes[:heads].astype(np.float64))
    if w.N <= 8192:
        t0 = time.perf_counter()
        oracle.attn_fwd(x["q"].values[sl], x["k"].values[sl], x["v"].values[sl], w.scale, w.causal, mask_np,
                        **var)
        if w.backward:
            oracle.attn_bwd(x["q"].values[sl], x["k"].values[sl], x["v"].values[sl], x["do"].values[sl],
                            w.scale, w.causal, mask_np, **var)
        dt = time.perf_counter() - t0
        if window is not None:
            fl = A.fwd_flops_window(1, heads, w.N, w.d, w.causal, window)
        else:
            fl = A.fwd_flops(1, heads, w.N, w.d, w.causal, mask_np)
        if w.backward:
            fl *= 3.5
        performed = A.oracle_flops(heads, w.N, w.d, A.allowed_pairs(w.N, w.causal, mask_np, window), w.backward)
        what = (f"{'forward+backward' if w.backward else 'forward'} of heads (b=0, h=0..{heads - 1}) of "
                f"{w.B * w.H}")
    else:
        rows = W.sample_rows(w.B * w.H, w.N, 512, seed=W.SEED_ROWS)
        t0 = time.perf_counter()
        oracle.attn_fwd_rows(x["q"].values, x["k"].values, x["v"].values, w.scale, rows, w.causal, mask_np,
                             **(dict(window=window, slopes=None if slopes is None else slopes.astype(np.float64))
                                if w.variant else {}))
        dt = time.perf_counter() - t0
        if window is not None:
            fl = A.fwd_flops_window(1, 1, w.N, w.d, w.causal, window) * len(rows) / w.N
        else:
            fl = A.fwd_flops(1, 1, w.N, w.d, w.causal, mask_np) * len(rows) / w.N
        # per sampled row: dense scores over all N keys, P V over its admitted keys
        performed = len(rows) * 2.0 * w.N * w.d + fl / 2.0
        what = f"forward of 512 sampled rows of {w.B * w.H * w.N}"
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"{what} (N={w.N}, d={w.d}, {'causal' if w.causal else 'non-causal'}"
                   f"{variant_label(w)}), fp64, {dt:.2f} s; value credits the metric's FLOPs of the sample"),
        "seconds": round(dt, 3),
        "metric_flops": fl,
        # the oracle materializes the dense N x N matrices, so it does more arithmetic than the metric credits
        "oracle_flops_performed": performed,
        "oracle_gflops_performed": round(performed / dt / 1e9, 2),
        "host_cpu": host_cpu_model(),
    }


def settle_until(step, t_start: float, settle_s: float) -> int:
    """Run untimed steps until `settle_s` seconds have passed since `t_start`.

    The GPU raises its shader clock over roughly a tenth of a second of
    sustained load (measured on the MI355X: a matrix-core stream runs at
    1.63 GHz after 0.6 ms and 1.97 GHz after 6 ms of load; the causal forward
    at 1.32 GHz a few ms after a cold start and at 1.69 GHz after 0.2 s), so a
    handful of warm-up steps leaves the timed steps on the ramp.  Returns the
    number of extra steps run."""
    import torch
    n = 0
    while settle_s > 0 and time.perf_counter() - t_start < settle_s:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
        n += 8
    return n


def percentiles_us(times_ms) -> dict:
    """Median, p10 and p90 of per-call event times (ms in, us out)."""
    t = sorted(times_ms)
    return {"median": round(statistics.median(t) * 1e3, 2), "p10": round(t[len(t) // 10] * 1e3, 2),
            "p90": round(t[(9 * len(t)) // 10] * 1e3, 2)}


def variant_label(w) -> str:
    parts = []
    if w.window is not None:
        parts.append(f"window {tuple(w.window)}")
    if w.alibi:
        parts.append("ALiBi")
    return "".join(", " + p for p in parts)


DECODE_METRIC = "paged-KV decode throughput (algorithmic HBM bytes / s) and % of HBM peak"


def bench_decode(args, w) -> int:
    """One step = one fa_decode_paged call over the workload's paged cache."""
    import torch
    import exact_io_aware_59_amd as fa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    x = W.decode_inputs(w, seed=0)

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, kc, vc = (to_dev(x[n]) for n in ("q", "k_cache", "v_cache"))
    bt = torch.from_numpy(x["block_table"]).to(dev)
    sl = torch.from_numpy(x["seqlens"]).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    ws = fa.decode_workspace(q, kc, bt)
    if args.copy_calib:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step():
        fa.fa_decode_paged(q, kc, vc, bt, sl, o, lse, w.scale, w.causal, ws, stream)

    # (events created before the warm-up: creating them leaves the GPU idle long enough to cool its clock)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_warm = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settle_steps = settle_until(step, t_warm, args.settle_s)
    # timed steps: nothing but the launches between the synchronizations; then as many again with events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) for a, b in ev)
    med = statistics.median(times)
    lens = x["seqlens"]
    nbytes = A.decode_bytes(w, lens)
    flops = A.decode_flops(w, lens)
    ms_per_step = wall / args.steps * 1e3
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (med * 1e-3) / 1e9
    out = {
        "metric": DECODE_METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "H_kv": w.Hkv, "Nq": w.Nq, "d": w.d,
            "page_size": w.page_size, "max_pages": w.max_pages, "causal": w.causal,
            "seqlens_total": int(np.sum(lens)), "step": "fa_decode_paged (split keys + merge)",
            "algorithmic_bytes": nbytes, "step_flops": flops,
            "workspace_bytes": 0 if ws is None else int(ws.numel()),
        },
        "pct_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "call_us": percentiles_us(times),
        "tflops": round(flops / (med * 1e-3) / 1e12, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None if measured_traffic(w.name, "fa_decode_paged") is None
            else measured_traffic(w.name, "fa_decode_paged")["traffic_bytes"],
            "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "kernel": "decode_kernel + decode_merge_kernel (fa_decode_paged)",
            "kernel_ms": round(med, 4),
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        nb = min(4, w.B)
        t1 = time.perf_counter()
        oracle.attn_paged_fwd(x["q"].values[:nb], x["k_cache"].values, x["v_cache"].values, x["block_table"][:nb],
                              lens[:nb], w.scale, w.causal)
        dt = time.perf_counter() - t1
        sub = A.decode_bytes(w, lens[:nb])
        out["cpu_baseline"] = {
            "value": round(sub / dt / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"decode of the first {nb} of {w.B} sequences ({int(np.sum(lens[:nb]))} cached tokens), "
                      f"fp64, {dt:.2f} s",
            "seconds": round(dt, 3), "host_cpu": host_cpu_model(),
        }
    print(json.dumps(out), flush=True)
    return 0


def capture_step(torch, step, outputs):
    """Capture one step (its kernel launches only: the step allocates nothing and
    enqueues no memset) into a HIP graph and return its replay.  Replays must
    reproduce the eager step bit for bit (every kernel is deterministic): three
    replays, each after an eager step and a synchronization, are compared
    before the graph is used; a mismatch stops the benchmark."""
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(stream=side)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in outputs:
            t.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        for t in outputs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outputs, ref):
            if not torch.equal(t, r):
                raise RuntimeError("graph replay differs from the eager step")
    return g.replay


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--launch", choices=("stream", "graph"), default="stream",
                    help="timed steps launched call by call on the stream, or as one captured HIP graph "
                         "(checked bit for bit against the eager step before timing)")
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="after the warm-up steps, run further untimed steps until this many seconds of "
                         "sustained load have passed (the GPU clock ramps up over ~0.1 s); 0 disables")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the implementation runs on a single GPU; --gpus must be 1 "
              "(no multi-GPU path is implemented)", file=sys.stderr)
        return 2

    import torch
    import exact_io_aware_59_amd as fa

    w = W.WORKLOADS[args.workload]
    if getattr(w, "kind", "attn") == "decode":
        return bench_decode(args, w)
    if w.dtype != "bf16":
        print("bench.py: only bf16 workloads are benchmarked", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    x = W.workload_inputs(w, seed=0)
    mask_np = W.workload_mask(w, seed=0)

    def to_dev(t):
        return torch.from_numpy(t.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = (to_dev(x[n]) for n in "qkv")
    do = to_dev(x["do"]) if w.backward else None
    mask = torch.from_numpy(mask_np).to(dev) if mask_np is not None else None
    B, H, N, d = w.B, w.H, w.N, w.d
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if w.backward:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = fa.workspace(B, H, N, d, dev)

    if args.copy_calib:
        # a plain copy of known size, for scaling the profiler's byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    n_ev = 4 if w.backward else 2

    window, slopes_np = W.workload_variant(w)
    slopes = torch.from_numpy(slopes_np).to(dev) if slopes_np is not None else None
    var = dict(window=window, alibi_slopes=slopes)
    fp8 = w.precision == "fp8"
    if fp8:
        # inputs quantized once, outside the timed steps (the quantization is timed on its own below)
        signs = torch.from_numpy(W.fp8_signs(w.d)).to(dev)
        q8, qe = fa.quantize_fp8(q, signs, False, stream)
        k8, ke = fa.quantize_fp8(k, signs, True, stream)
        v8, ve = fa.quantize_fp8(v, None, False, stream)

    def step(evs=None, stream=stream):
        if evs is not None:
            evs[0].record(stream)
        if fp8:
            fa.fa_fwd_fp8(q8, qe, k8, ke, v8, ve, o, lse, w.scale, w.causal, stream)
        elif w.variant:
            fa.fa_fwd_ex(q, k, v, o, lse, w.scale, w.causal, mask, stream=stream, **var)
        else:
            fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal, mask, stream)
        if evs is not None:
            evs[1].record(stream)
        if w.backward:
            if w.variant:
                fa.fa_bwd_dq_first_ex(q, k, v, o, do, lse, dq, w.scale, w.causal, mask, workspace=ws,
                                      stream=stream, **var)
            else:
                fa.fa_bwd_dq_first(q, k, v, o, do, lse, dq, w.scale, w.causal, mask, ws, stream)
            if evs is not None:
                evs[2].record(stream)
            if w.variant:
                fa.fa_bwd_main_ex(q, k, v, do, dk, dv, w.scale, w.causal, mask, workspace=ws, stream=stream, **var)
            else:
                fa.fa_bwd_main(q, k, v, do, dk, dv, w.scale, w.causal, mask, ws, stream)
            if evs is not None:
                evs[3].record(stream)

    launch = step
    if args.launch == "graph":
        launch = capture_step(torch, step, [o, lse] + ([dq, dk, dv] if w.backward else []))
    # (created up front: creating them takes tens of ms, an idle gap long enough for the clock to drop)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    t_warm = time.perf_counter()
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    settle_steps = settle_until(launch, t_warm, args.settle_s)

    # the timed steps: nothing but the step's launches between the two synchronizations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        launch()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # per-call times: the same number of steps again, right after, each call bracketed by events on the
    # launch stream
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()

    t_fwd = [e[0].elapsed_time(e[1]) for e in events]
    res = {"fwd_ms": statistics.median(t_fwd)}
    per_call = {"fa_fwd_fp8" if w.precision == "fp8" else "fa_fwd": t_fwd}
    if w.backward:
        t_dq = [e[1].elapsed_time(e[2]) for e in events]
        t_main = [e[2].elapsed_time(e[3]) for e in events]
        res.update(bwd_dq_ms=statistics.median(t_dq), bwd_main_ms=statistics.median(t_main))
        per_call.update(fa_bwd_dq_first=t_dq, fa_bwd_main=t_main, fa_bwd=[a + b for a, b in zip(t_dq, t_main)])

    quant_ms = None
    if fp8:
        qa, qb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        qa.record(stream)
        for _ in range(10):
            fa.quantize_fp8(q, signs, False, stream)
            fa.quantize_fp8(k, signs, True, stream)
            fa.quantize_fp8(v, None, False, stream)
        qb.record(stream)
        torch.cuda.synchronize()
        quant_ms = qa.elapsed_time(qb) / 10
    flops = A.workload_flops(w, mask_np)
    bytes_ = A.workload_bytes(w, mask_np)
    total_flops = flops["fwd"] + flops.get("bwd", 0.0)
    ms_per_step = wall / args.steps * 1e3
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    fwd_tflops = flops["fwd"] / (res["fwd_ms"] * 1e-3) / 1e12
    extra = {
        "fwd_ms": round(res["fwd_ms"], 4),
        "fwd_tflops": round(fwd_tflops, 1),
        "fwd_pct_peak": round(100 * fwd_tflops / PEAK_BF16_TFLOPS, 2),
    }
    if w.backward:
        bwd_ms = statistics.median(per_call["fa_bwd"])
        bwd_tflops = flops["bwd"] / (bwd_ms * 1e-3) / 1e12
        extra.update({
            "bwd_ms": round(bwd_ms, 4),
            "bwd_tflops": round(bwd_tflops, 1),
            "bwd_pct_peak": round(100 * bwd_tflops / PEAK_BF16_TFLOPS, 2),
            "bwd_dq_ms": round(res["bwd_dq_ms"], 4),
            "bwd_main_ms": round(res["bwd_main_ms"], 4),
        })
        # fa_bwd_main computes four of the backward's five products (S, dP, dV, dK): 4/5 of its FLOPs
        dom_name, dom_ms, dom_flops = "bwd_bf16_kernel (fa_bwd_main)", res["bwd_main_ms"], flops["bwd"] * 4 / 5
        dom_api = "fa_bwd_main"
    elif fp8:
        dom_name, dom_ms, dom_flops = "fwd_fp8_kernel (fa_fwd_fp8)", res["fwd_ms"], flops["fwd"]
        dom_api = "fa_fwd_fp8"
        extra["fwd_pct_peak_fp8"] = round(100 * fwd_tflops / PEAK_FP8_TFLOPS, 2)
        extra["quantize_ms"] = round(quant_ms, 4)
    else:
        dom_name, dom_ms, dom_flops = "fwd_bf16_kernel (fa_fwd)", res["fwd_ms"], flops["fwd"]
        dom_api = "fa_fwd"
    tr = measured_traffic(w.name, dom_api)
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    roofline = {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": None if tr is None else tr["traffic_bytes"],
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "traffic_vs_algorithmic": None if tr is None else round(tr["traffic_bytes"] / tr["algorithmic_bytes"], 3),
        "kernel": dom_name,
        "kernel_ms": round(dom_ms, 4),
    }

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "launch": args.launch,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 (fp32 accumulate)" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": B, "H": H, "N": N, "d": d,
            "causal": w.causal,
            "window": None if w.window is None else list(w.window),
            "alibi": w.alibi,
            "block_density": None if mask_np is None else float(mask_np.mean()),
            "step": ("fa_fwd_fp8 (inputs quantized beforehand)" if fp8 else
                     ("fa_fwd + fa_bwd" if w.backward else "fa_fwd") + (" (_ex variant)" if w.variant else "")),
            "step_flops": total_flops,
            "algorithmic_bytes": sum(bytes_.values()),
        },
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        **extra,
        "call_us": {name: percentiles_us(t) for name, t in per_call.items()},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, mask_np, min(args.cpu_heads, w.H))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
