#!/usr/bin/env python3
"""Summaries of rocprofv3 runs of bench.py, written under profiles/.

Three summaries, each from the CSV files of one profiler run (or one pair):

  traffic   HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run of
            `bench.py --copy-calib`: every count is scaled by what the same
            counter reads for the 256 MiB device copy that --copy-calib runs
            first (262,144 KiB read and written).  Writes
            profiles/hbm_traffic.json (one entry per workload, tagged with a
            digest of the kernel sources so that bench.py stops reporting it
            once the kernels change) and a markdown table.
  mfma      matrix-core busy fraction per SIMD and the clock, from
            SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE.
  trace     per-kernel durations from a --kernel-trace run, beside the HIP
            event medians of the bench.py line that run printed.
  dram      read / write requests the L2 sends to the memory controllers
            (TCC_EA0_RDREQ_DRAM, TCC_EA0_WRREQ_DRAM) beside all L2 -> fabric
            requests, from one run of `bench.py --copy-calib`, scaled to bytes
            by the same counters of the 256 MiB copy.
  mix       instruction mix per kernel (VALU, SALU, LDS, transcendental and
            matrix instructions, LDS bank-conflict cycles, issue waits).

The mfma summary also reports the matrix operations each kernel executes
(SQ_INSTS_VALU_MFMA_MOPS_*, 512 FLOPs per unit) against the FLOPs the metric
credits to it.

Usage:
  python bench_counters.py traffic --workload NAME --fetch F.csv --write W.csv --command "..." [--command "..."]
  python bench_counters.py mfma --workload NAME --csv M.csv --command "..."
  python bench_counters.py trace --workload NAME --csv KT_kernel_trace.csv --bench-line B.json --command "..."
  python bench_counters.py dram --workload NAME --csv D.csv --command "..."
  python bench_counters.py mix --workload NAME --csv X.csv --command "..."
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402
from workloads import accounting as A  # noqa: E402

COPY_KIB = 262144.0
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic.json")
def kernel_sources(w) -> list:
    """The kernel sources a workload's counted launches are built from."""
    if getattr(w, "kind", "attn") == "decode":
        return ["fa_common.h", "fa_decode.hip"]
    if getattr(w, "precision", "bf16") == "fp8":
        return ["fa_common.h", "fa_fp8.hip"]
    return ["fa_common.h", "fa_fwd.h", "fa_fwd.hip", "fa_fwd_64.hip", "fa_fwd_96.hip", "fa_fwd_128.hip",
            "fa_fwd_192.hip", "fa_fwd_256.hip", "fa_bwd.hip"]

# kernel-name substring -> entry point that launches it
# (the benchmarked step launches the dQ kernel through fa_bwd_dq_first, before fa_bwd_main)
ENTRY = [("fwd_bf16_kernel", "fa_fwd"), ("rowdot_kernel", "fa_bwd_prep"),
         ("bwd_dq_kernel", "fa_bwd_dq_first"), ("bwd_bf16_kernel", "fa_bwd_main"),
         ("decode_kernel", "fa_decode_paged"), ("decode_merge_kernel", "fa_decode_paged"),
         ("fp8_quant_kernel", "fa_fp8_quantize"), ("fwd_fp8_kernel", "fa_fwd_fp8")]
ORDER = list(dict.fromkeys(e for _, e in ENTRY))


def entry_of(kernel: str):
    for key, api in ENTRY:
        if key in kernel:
            return api
    return None


def is_copy(kernel: str) -> bool:
    return "copyBuffer" in kernel


def read_counters(path: str):
    """{(kernel, counter): [value per dispatch]} from a counter_collection CSV."""
    d = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        d[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return d


def workload_title(w) -> str:
    if getattr(w, "kind", "attn") == "decode":
        return w.description
    parts = [f"B={w.B} H={w.H} N={w.N} d={w.d} {w.dtype}", "causal" if w.causal else "non-causal"]
    if w.window is not None:
        parts.append(f"window {tuple(w.window)}")
    if w.alibi:
        parts.append("ALiBi")
    if w.mask:
        parts.append(f"block mask {w.mask}")
    if getattr(w, "precision", "bf16") == "fp8":
        parts.append("FP8 E4M3")
    return ", ".join(parts) + (" (forward + backward step)" if w.backward else " (forward)")


def commands_block(cmds) -> list:
    return ["Commands (run from /tmp with TMPDIR=/tmp on the GPU host):", "", "```", *cmds, "```", ""]


def traffic(args) -> None:
    w = W.WORKLOADS[args.workload]
    f, wr = read_counters(args.fetch), read_counters(args.write)
    copy = [k for (k, c) in f if is_copy(k) and c == "FETCH_SIZE"]
    copy_w = [k for (k, c) in wr if is_copy(k) and c == "WRITE_SIZE"]
    if not copy or not copy_w:
        raise SystemExit("no calibration copy in the profile: run bench.py with --copy-calib")
    # the 256 MiB calibration copy is the largest copy dispatch (input uploads are copies too)
    f_copy = max(f[(copy[0], "FETCH_SIZE")])
    w_copy = max(wr[(copy_w[0], "WRITE_SIZE")])
    fs, ws = COPY_KIB / f_copy, COPY_KIB / w_copy
    if getattr(w, "kind", "attn") == "decode":
        alg = {"fa_decode_paged": A.decode_bytes(w, W.decode_inputs(w, seed=0)["seqlens"])}
    else:
        alg = A.launch_bytes(w, W.workload_mask(w, seed=0))
    per = {}
    rows = []
    for (k, c), vals in f.items():
        api = entry_of(k)
        if api is None or c != "FETCH_SIZE" or api not in alg:
            continue
        fk = statistics.mean(vals)
        wk = statistics.mean(wr[(k, "WRITE_SIZE")])
        rb, wb = fk * fs * 1024, wk * ws * 1024
        # an entry point that launches several kernels sums their traffic per call
        e = per.setdefault(api, {"read_bytes": 0, "write_bytes": 0, "traffic_bytes": 0, "algorithmic_bytes": alg[api]})
        e["read_bytes"] += round(rb)
        e["write_bytes"] += round(wb)
        e["traffic_bytes"] += round(rb + wb)
        rows.append((ORDER.index(api), f"| {api} | `{k[:60]}` | {len(vals)} | {fk:.1f} | {wk:.1f} | {rb / 1e6:.1f} | "
                                       f"{wb / 1e6:.1f} | {(rb + wb) / 1e6:.1f} | {alg[api] / 1e6:.1f} | "
                                       f"{(rb + wb) / alg[api]:.2f} |"))
    try:
        allw = json.load(open(TRAFFIC_JSON))
        if "workloads" not in allw:
            allw = {"workloads": {}}
    except (OSError, ValueError):
        allw = {"workloads": {}}
    allw["workloads"][w.name] = {
        "kernel_source_sha256": bench.kernel_source_digest(kernel_sources(w)), "sources": kernel_sources(w),
        "fetch_scale": fs, "write_scale": ws, "per_launch": per}
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(allw, fh, indent=1, sort_keys=True)
        fh.write("\n")
    lines = [f"# HBM traffic per launch: {workload_title(w)}", ""]
    lines += commands_block(args.command)
    lines += [f"Calibration: the 256 MiB device copy that `--copy-calib` runs first reads FETCH_SIZE = {f_copy:.1f} KiB "
              f"and WRITE_SIZE = {w_copy:.1f} KiB per dispatch for {COPY_KIB:.0f} KiB moved each way, so fetch counts "
              f"are scaled by {fs:.4f} and write counts by {ws:.4f}.", "",
              "| entry point | kernel | dispatches | FETCH_SIZE KiB (raw) | WRITE_SIZE KiB (raw) | read MB | write MB | "
              "traffic MB | algorithmic MB | ratio |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    lines += [r for _, r in sorted(rows)]
    lines += ["", "Algorithmic bytes: each tensor read or written once per launch (bf16 Q, K, V, dO, O, dQ, dK, dV; "
              "fp32 lse and D; the block mask).  Traffic above them is K/V (forward, dQ) and Q/dO (key-outer "
              "backward) tiles that the workgroups sharing them re-read past L2."]
    out = os.path.join(ROOT, "profiles", f"{args.workload}_hbm_traffic.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mfma(args) -> None:
    w = W.WORKLOADS[args.workload]
    m = read_counters(args.csv)
    dur = collections.defaultdict(list)
    for r in csv.DictReader(open(args.csv)):
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    lines = [f"# Matrix-core busy fraction and clock: {workload_title(w)}", ""]
    lines += commands_block(args.command)
    credited = metric_flops_per_launch(w)
    mops_names = [c for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                              "SQ_INSTS_VALU_MFMA_MOPS_F6F4") if any(c == n for _, n in m)]
    lines += ["GRBM_GUI_ACTIVE is summed over the 8 XCDs; busy per SIMD = SQ_VALU_MFMA_BUSY_CYCLES / "
              "(1024 SIMDs x GRBM_GUI_ACTIVE / 8); clock = (GRBM_GUI_ACTIVE / 8) / dispatch duration; medians over "
              "the dispatches.  GRBM_GUI_ACTIVE also counts ~20k cycles around each dispatch (the 12 µs rowdot "
              "stage reads 45k), so busy reads a few per cent low and the clock a few per cent high on the long "
              "kernels.  "
              "Executed matrix FLOPs = " + " + ".join(mops_names or ["(no MOPS counter)"]) + " x 512 per "
              "dispatch (the SQ counters read per dispatch: the forward's SQ_INSTS_MFMA equals its product "
              "count computed from the tiling); credited = the FLOPs the metric gives that entry point.", "",
              "| entry point | dispatches | GRBM_GUI_ACTIVE | SQ_VALU_MFMA_BUSY_CYCLES | MFMA busy per SIMD | clock GHz "
              "| SQ_INSTS_MFMA | executed GFLOP | credited GFLOP | executed / credited |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    rows = []
    for k in sorted({k for k, _ in m}):
        api = entry_of(k)
        if api is None:
            continue
        g = statistics.median(m[(k, "GRBM_GUI_ACTIVE")])
        b = statistics.median(m[(k, "SQ_VALU_MFMA_BUSY_CYCLES")])
        d = statistics.median(dur[k])
        ni = statistics.median(m[(k, "SQ_INSTS_MFMA")]) if (k, "SQ_INSTS_MFMA") in m else None
        ex = sum(statistics.median(m[(k, c)]) for c in mops_names if (k, c) in m) * 512 if mops_names else None
        cr = credited.get(api)
        rows.append((ORDER.index(api), f"| {api} | {len(dur[k])} | {g:.4g} | {b:.4g} | {b / (1024 * g / 8):.3f} | "
                                       f"{g / 8 / d / 1e9:.2f} | {'' if ni is None else f'{ni:.4g}'} | "
                                       f"{'' if ex is None else f'{ex / 1e9:.1f}'} | "
                                       f"{'' if cr is None else f'{cr / 1e9:.1f}'} | "
                                       f"{'' if (ex is None or not cr) else f'{ex / cr:.3f}'} |"))
    lines += [r for _, r in sorted(rows)]
    lines += ["", "The published peaks assume 2.4 GHz; a dispatch too short for the estimate (the rowdot stage) "
              "reads a clock dominated by that overhead."]
    out = os.path.join(ROOT, "profiles", f"{args.workload}_mfma_busy.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def metric_flops_per_launch(w) -> dict:
    """FLOPs the metric credits to each entry point of one step: the forward's
    two products, and of the backward's five, four to the key-outer kernel
    (S, dP, dV, dK) and one to the dQ kernel."""
    if getattr(w, "kind", "attn") == "decode":
        return {"fa_decode_paged": A.decode_flops(w, W.decode_inputs(w, seed=0)["seqlens"])}
    f = A.workload_flops(w, W.workload_mask(w, seed=0))
    out = {"fa_fwd_fp8" if getattr(w, "precision", "bf16") == "fp8" else "fa_fwd": f["fwd"]}
    if "bwd" in f:
        out.update({"fa_bwd_prep": 0.0, "fa_bwd_main": f["bwd"] * 4 / 5, "fa_bwd_dq_first": f["bwd"] / 5})
    return out


def dram(args) -> None:
    w = W.WORKLOADS[args.workload]
    m = read_counters(args.csv)
    copy = [k for (k, c) in m if is_copy(k) and c == "TCC_EA0_RDREQ_DRAM_sum"]
    if not copy:
        raise SystemExit("no calibration copy in the profile: run bench.py with --copy-calib")
    rd_copy = max(m[(copy[0], "TCC_EA0_RDREQ_DRAM_sum")])
    wr_copy = max(m[(copy[0], "TCC_EA0_WRREQ_DRAM_sum")])
    rb_req, wb_req = COPY_KIB * 1024 / rd_copy, COPY_KIB * 1024 / wr_copy
    if getattr(w, "kind", "attn") == "decode":
        alg = {"fa_decode_paged": A.decode_bytes(w, W.decode_inputs(w, seed=0)["seqlens"])}
    else:
        alg = A.launch_bytes(w, W.workload_mask(w, seed=0))
    lines = [f"# Memory-controller traffic per launch: {workload_title(w)}", ""]
    lines += commands_block(args.command)
    lines += [f"Calibration: the 256 MiB device copy reads TCC_EA0_RDREQ_DRAM_sum = {rd_copy:.4g} and "
              f"TCC_EA0_WRREQ_DRAM_sum = {wr_copy:.4g} requests per dispatch, i.e. {rb_req:.1f} and "
              f"{wb_req:.1f} bytes per request; the kernels' counts are scaled by the same factors.  "
              "All-request columns (TCC_EA0_RDREQ_sum / TCC_EA0_WRREQ_sum) count every L2 -> fabric request.", "",
              "| entry point | kernel | dispatches | RDREQ (all) | RDREQ_DRAM | WRREQ (all) | WRREQ_DRAM | "
              "DRAM read MB | DRAM write MB | algorithmic MB | DRAM / algorithmic |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    rows, per = [], collections.defaultdict(lambda: [0.0, 0.0, 0.0, 0.0])
    for (k, c), vals in m.items():
        api = entry_of(k)
        if api is None or c != "TCC_EA0_RDREQ_DRAM_sum" or api not in alg:
            continue
        ra = statistics.mean(m[(k, "TCC_EA0_RDREQ_sum")])
        rd = statistics.mean(vals)
        wa = statistics.mean(m[(k, "TCC_EA0_WRREQ_sum")])
        wd = statistics.mean(m[(k, "TCC_EA0_WRREQ_DRAM_sum")])
        rbytes, wbytes = rd * rb_req, wd * wb_req
        rows.append((ORDER.index(api), f"| {api} | `{k[:60]}` | {len(vals)} | {ra:.4g} | {rd:.4g} | {wa:.4g} | "
                                       f"{wd:.4g} | {rbytes / 1e6:.1f} | {wbytes / 1e6:.1f} | {alg[api] / 1e6:.1f} | "
                                       f"{(rbytes + wbytes) / alg[api]:.2f} |"))
    lines += [r for _, r in sorted(rows)]
    out = os.path.join(ROOT, "profiles", f"{args.workload}_dram_traffic.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


MIX = ["SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA",
       "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"]


def mix(args) -> None:
    w = W.WORKLOADS[args.workload]
    m = read_counters(args.csv)
    lines = [f"# Instruction mix per kernel: {workload_title(w)}", ""]
    lines += commands_block(args.command)
    lines += ["Per dispatch (means).  Per-MFMA columns divide by SQ_INSTS_MFMA; SQ_INSTS_VALU includes the "
              "matrix and transcendental instructions, so 'other VALU' = VALU - MFMA - TRANS.  Bank conflicts are "
              "LDS cycles lost to conflicts per LDS instruction; issue wait is SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES "
              "(wave-cycles with an instruction ready but not issued).", "",
              "| entry point | " + " | ".join(MIX) + " | other VALU / MFMA | TRANS / MFMA | SALU / MFMA | LDS / MFMA "
              "| conflict cycles / LDS | issue wait |",
              "|---|" + "---|" * (len(MIX) + 6)]
    rows = []
    for k in sorted({k for k, _ in m}):
        api = entry_of(k)
        if api is None or (k, "SQ_INSTS_MFMA") not in m:
            continue
        v = {c: statistics.mean(m[(k, c)]) if (k, c) in m else float("nan") for c in MIX}
        nm = v["SQ_INSTS_MFMA"] or float("nan")
        other = v["SQ_INSTS_VALU"] - v["SQ_INSTS_MFMA"] - v["SQ_INSTS_VALU_TRANS_F32"]
        lds = v["SQ_INSTS_LDS"] or float("nan")
        rows.append((ORDER.index(api), f"| {api} | " + " | ".join(f"{v[c]:.4g}" for c in MIX) +
                     f" | {other / nm:.2f} | {v['SQ_INSTS_VALU_TRANS_F32'] / nm:.2f} | {v['SQ_INSTS_SALU'] / nm:.2f} "
                     f"| {v['SQ_INSTS_LDS'] / nm:.2f} | {v['SQ_LDS_BANK_CONFLICT'] / lds:.2f} | "
                     f"{v['SQ_WAIT_INST_ANY'] / v['SQ_WAVE_CYCLES']:.2f} |"))
    lines += [r for _, r in sorted(rows)]
    out = os.path.join(ROOT, "profiles", f"{args.workload}_instruction_mix.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace(args) -> None:
    w = W.WORKLOADS[args.workload]
    line = [json.loads(x) for x in open(args.bench_line) if x.startswith('{"metric"')][-1]
    steps, warm = line["steps"], line["warmup"]
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(args.csv)):
        api = entry_of(r["Kernel_Name"])
        if api is None:
            continue
        per[(api, r["Kernel_Name"])].append(
            (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3))
    ev = {"fa_fwd": line.get("fwd_ms"), "fa_bwd_prep": None,
          "fa_bwd_main": line.get("bwd_main_ms"), "fa_bwd_dq_first": line.get("bwd_dq_ms"),
          "fa_fwd_fp8": line.get("fwd_ms") if "fwd_pct_peak_fp8" in line else None,
          "fa_decode_paged": None}
    if "fwd_pct_peak_fp8" in line:
        ev["fa_fwd"] = None
    calls = line.get("call_us", {})
    if "median" in calls:  # one entry point per step (paged decode)
        ev["fa_decode_paged"] = calls["median"] / 1e3
    for api, c in calls.items():
        if isinstance(c, dict) and "median" in c:
            ev[api] = c["median"] / 1e3
    lines = [f"# Kernel trace: {workload_title(w) if getattr(w, 'kind', 'attn') == 'attn' else w.description}", ""]
    lines += commands_block(args.command)
    lines += [f"{warm} warm-up steps, then {steps} timed steps.  The last column is the median of the HIP-event "
              f"times bench.py measured on the launch stream for the same timed steps (per entry point: the "
              f"sum of its kernels).", "",
              "| entry point | kernel | calls | avg µs (all) | avg µs (timed) | min µs | max µs | bench.py event median µs |",
              "|---|---|---|---|---|---|---|---|"]
    shown = set()
    for (api, name) in sorted(per, key=lambda x: (ORDER.index(x[0]), x[1])):
        d = [x for _, x in sorted(per[(api, name)])]
        timed = d[-steps:]
        e = ev.get(api) if api not in shown else None
        shown.add(api)
        lines.append(f"| {api} | `{name[:60]}` | {len(d)} | {statistics.mean(d):.1f} | "
                     f"{statistics.mean(timed):.1f} | {min(d):.1f} | {max(d):.1f} | "
                     f"{'' if e is None else f'{e * 1e3:.1f}'} |")
    keep = {k: line[k] for k in ("metric", "value", "unit", "ms_per_step", "fwd_ms", "bwd_ms", "bwd_prep_ms",
                                 "bwd_main_ms", "bwd_dq_ms", "call_us") if k in line}
    lines += ["", "bench.py line printed by the profiled run (abridged):", "", "```", json.dumps(keep), "```"]
    out = os.path.join(ROOT, "profiles", f"{args.workload}_kernel_trace.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--csv", required=True)
    k = sub.add_parser("trace")
    k.add_argument("--csv", required=True)
    k.add_argument("--bench-line", required=True)
    dr = sub.add_parser("dram")
    dr.add_argument("--csv", required=True)
    mx = sub.add_parser("mix")
    mx.add_argument("--csv", required=True)
    for p in (t, m, k, dr, mx):
        p.add_argument("--workload", default=bench.DEFAULT_WORKLOAD, choices=sorted(W.WORKLOADS))
        p.add_argument("--command", action="append", default=[])
    args = ap.parse_args()
    {"traffic": traffic, "mfma": mfma, "trace": trace, "dram": dram, "mix": mix}[args.what](args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
