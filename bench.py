#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_bf16]

A step is one pass of the whole layer (route, regroup, W13 + SiLU*mul,
W2 + gate scale, combine: one moe_forward call) over every batch of the
workload, back to back; for the default workload (decode bf16, Mixtral-like
shapes d=4096, E=8, top-2, I=14336) that is T = 1, 8, 32 and 64 tokens.
Inputs are seeded synthetic tensors already resident in HBM.  Two copies of
the weights alternate between consecutive forwards, so no forward finds the
previous one's weights in the 256 MB Infinity Cache.

Prints one JSON line on stdout: tokens/s over the K timed steps, the
dominant kernel's achieved HBM bandwidth against the 8 TB/s peak (its
average duration measured with HIP events recorded on its own stream inside
the timed region), and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused-MoE tokens/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0
# dense MFMA peaks by what the expert products compute in: W8A16 widens its
# e4m3fn weights to bf16; the W8A8 mode multiplies e4m3fn by e4m3fn
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "e4m3fn": 2500.0, "f32": 157.3, "mx_e4m3": 5000.0}
WORKLOAD_BATCHES = {
    "decode_bf16": (1, 8, 32, 64),
    "prefill_bf16": (4096,),
    "prefill_w8a8": (4096,),
    "fp8": (64, 2048),
    "skew": (512,),
    "tiny_fp32": (16,),
}
# Oracle sample per workload: (batch T, number of its tokens run on the CPU)
CPU_SAMPLE = {"decode_bf16": (64, 64), "prefill_bf16": (4096, 16), "prefill_w8a8": (4096, 16),
              "fp8": (2048, 4),
              "skew": (512, 64), "tiny_fp32": (16, 16)}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_bf16", choices=sorted(WORKLOAD_BATCHES))
    ap.add_argument("--batches", default=None, help="comma-separated T values (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-breakdown", action="store_true", help="skip the per-kernel breakdown pass")
    ap.add_argument("--block-m", type=int, default=0, help="regrouping block size (0 = library default)")
    ap.add_argument("--schedule", default="auto", choices=["auto", "static", "queue"],
                    help="tile schedule of the 128-token-block expert kernels")
    ap.add_argument("--act-quant", default=None, choices=["mx_e4m3", "none"],
                    help="override the workload's activation mode: mx_e4m3 (W8A8, e4m3fn weights "
                         "only) or none (activations as given)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the layer, run a plain device copy of this many bytes "
                         "(reference reading for HBM traffic counters)")
    ap.add_argument("--summarize-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="no GPU: write profiles/ffn13_<workload>_traffic.json from the output "
                         "directories of four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE over "
                         "this bench, then over --copy-bytes %d)" % (1 << 30))
    ap.add_argument("--summarize-stats", nargs="+", metavar="DIR",
                    help="no GPU: write profiles/<workload>_kernel_stats.md from a rocprofv3 "
                         "--kernel-trace --stats output directory (and the run's stdout file)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="no GPU: write profiles/<workload>_mfma_counters.md from rocprofv3 --pmc "
                         "output directories (matrix-core counters) and a --kernel-trace --stats "
                         "directory given last")
    ap.add_argument("--summarize-mempath", nargs="+", metavar="DIR",
                    help="no GPU: write profiles/<workload>_memory_path_counters.md from rocprofv3 "
                         "--pmc output directories (texture unit, L1 and L2 counters)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode workload: skip the prefill sub-record (T = 4096 on the same weights)")
    ap.add_argument("--cpu-reps", type=int, default=3, help="CPU oracle repetitions (median reported)")
    ap.add_argument("--command", default="", help="profiling command recorded in the summary")
    return ap.parse_args()


# sources that routing and regrouping alone use: they do not change the
# expert kernels, so their edits leave recorded ffn13 traffic valid
ROUTING_ONLY_SOURCES = ("router.hip", "align.hip")


def kernel_source_sha(exclude=()) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_moe_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name in exclude:
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def copy_calibration(nbytes: int, reps: int = 5) -> None:
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def alg_work(inp, ids, k) -> dict:
    """Algorithmic bytes and flops of one forward, from the realised routing.
    Bytes: weights (and fp8 scales) of the touched experts, W_gate, x, out.
    ffn13 bytes: touched experts' W13 (+ scales), x, h written for real slots
    (in the W8A8 mode x and h are e4m3fn codes plus one exponent byte per 32)."""
    import torch
    T, d, E, I = inp.T, inp.d, inp.E, inp.I
    wb = {"f32": 4, "bf16": 2, "e4m3fn": 1}[inp.w]
    ab = 4 if inp.act == "f32" else 2
    touched = int(torch.unique(ids).numel()) if T else 0
    A = T * k
    sc13 = 2 * I * 4 if inp.w == "e4m3fn" else 0
    sc2 = d * 4 if inp.w == "e4m3fn" else 0
    w13 = touched * (2 * I * d * wb + sc13)
    w2 = touched * (d * I * wb + sc2)
    return {
        "T": T, "touched_experts": touched,
        "bytes": w13 + w2 + E * d * 4 + T * d * 2 * ab,
        "flops": A * 6 * d * I + 2 * T * d * E,
        "ffn13_bytes": w13 + (T * d * 33 // 32 + A * I * 33 // 32 if inp.act_quant
                              else T * d * ab + A * I * ab),
        "ffn13_flops": A * 4 * d * I,
        # W2: touched experts' W2 (+ scales), h of the real slots, and one fp32
        # output row per slot handed to the combine
        "ffn2_bytes": w2 + (A * I * 33 // 32 if inp.act_quant else A * I * ab) + A * d * 4,
        "ffn2_flops": A * 2 * d * I,
    }


def cpu_baseline(inp_T, k_sample: int, workload: str, reps: int = 3) -> dict:
    """The oracle as it stands, on `k_sample` tokens of the batch, timed on
    this host's cores: the median of `reps` forwards."""
    import numpy as np
    import threadpoolctl

    import oracle
    from mixture_experts_moe_amd import synth
    from dataclasses import replace
    import torch

    tokens = torch.linspace(0, inp_T.T - 1, k_sample).round().long().to(inp_T.x.device)
    sub = replace(inp_T, x=inp_T.x.index_select(0, tokens).contiguous())
    kw = synth.to_oracle(sub)
    # fetch the experts the sample touches before timing (host copies are not oracle work)
    lg = oracle.router_logits(oracle.decode_bf16(kw["x"]) if kw["act_fmt"] == "bf16"
                              else kw["x"].astype(np.float64), kw["w_gate"])
    for e in np.unique(oracle.select_topk(lg, sub.top_k)):
        kw["w13"][e]
        kw["w2"][e]
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    times = []
    for _ in range(max(reps, 1)):
        t0 = time.perf_counter()
        oracle.moe_forward(**kw, block_m=16)
        times.append(time.perf_counter() - t0)
    times.sort()
    dt = times[len(times) // 2]
    return {"value": round(k_sample / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{workload}: {k_sample} of the T={inp_T.T} batch's tokens through the "
                      f"fp64 NumPy per-expert-loop oracle, median of {len(times)} forwards "
                      f"({', '.join(f'{t:.2f}' for t in times)} s; "
                      f"{len(os.sched_getaffinity(0))} host cores visible, BLAS threads {threads})"}


COPY_CAL_BYTES = 1 << 30


def _counter_rows(directory: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    return rows


def _short_kernel(name: str) -> str:
    name = name.replace("void ", "", 1)
    depth, out = 0, []
    for ch in name:  # drop the parameter list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).replace("moe::", "")


EXPERT_KINDS = (("ffn13", "ffn13 (grouped W13 + SiLU*mul)"), ("ffn2", "ffn2 (grouped W2 + gate scale)"))


def summarize_traffic(workload: str, dirs, command: str) -> str:
    """HBM bytes per ffn13 and per ffn2 launch: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) scaled by what the same counters read for a plain
    device copy of COPY_CAL_BYTES bytes."""
    fetch, write, cfetch, cwrite = (_counter_rows(d) for d in dirs)

    def factor(rows, counter):
        vals = sorted(float(r["Counter_Value"]) for r in rows
                      if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"])
        if not vals:
            raise SystemExit(f"no copy kernel with {counter} in the calibration run")
        return COPY_CAL_BYTES / (vals[len(vals) // 2] * 1024.0)

    ff, fw = factor(cfetch, "FETCH_SIZE"), factor(cwrite, "WRITE_SIZE")

    def launches(rows, counter, kind):
        got = [(int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"]))
               for r in rows if r["Counter_Name"] == counter and kind + "_" in r["Kernel_Name"]]
        return sorted(got)

    out = {
        "workload": workload,
        # expert-kernel sources (all but the routing-only files)
        "kernel_source_sha": kernel_source_sha(exclude=ROUTING_ONLY_SOURCES),
        "command": command,
        "calibration": {
            "copy_bytes": COPY_CAL_BYTES,
            "FETCH_SIZE_bytes_per_counted_byte": round(ff, 4),
            "WRITE_SIZE_bytes_per_counted_byte": round(fw, 4),
            "note": "counter values are KiB per dispatch; each is scaled by the bytes a plain "
                    "device copy of copy_bytes moves per counted byte",
        },
    }
    for kind, label in EXPERT_KINDS:
        lf, lw = launches(fetch, "FETCH_SIZE", kind), launches(write, "WRITE_SIZE", kind)
        if len(lf) != len(lw) or not lf:
            raise SystemExit(f"{kind} launches differ between the runs: {len(lf)} vs {len(lw)}")
        rows = []
        for (_, kf, gf, vf), (_, kw, gw, vw) in zip(lf, lw):
            if kf != kw or gf != gw:
                raise SystemExit(f"the two runs launched different {kind} kernels in order")
            rows.append({"kernel": _short_kernel(kf), "grid_threads": gf,
                         "fetch_bytes": int(vf * 1024 * ff), "write_bytes": int(vw * 1024 * fw)})
        per_launch = sum(r["fetch_bytes"] + r["write_bytes"] for r in rows) / len(rows)
        out[kind] = {"kernel": label, "launches": rows, "traffic_bytes_per_launch": int(per_launch)}
    path = os.path.join(ROOT, "profiles", f"{workload}_expert_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return path


def summarize_stats(workload: str, paths, command: str) -> str:
    """Markdown table of the layer's kernels from rocprofv3 --stats."""
    import csv
    import glob
    files = glob.glob(os.path.join(paths[0], "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {paths[0]}")
    with open(files[0]) as fh:
        stats = [r for r in csv.DictReader(fh) if "moe::" in r["Name"]]
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# Kernel stats: {workload} workload (batches {', '.join(map(str, WORKLOAD_BATCHES[workload]))})",
             "", "Command (from the repository root, one MI355X):", "", f"    {command}", "",
             f"Kernel sources sha (bench.py kernel_source_sha): `{kernel_source_sha()}`", "",
             "| kernel | calls | avg us | min us | max us | total us |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{_short_kernel(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e3:.0f} |")
    lines.append("")
    for kind, _ in EXPERT_KINDS:
        ks = [r for r in stats if kind + "_" in r["Name"]]
        if ks:
            calls = sum(int(r["Calls"]) for r in ks)
            total = sum(float(r["TotalDurationNs"]) for r in ks)
            lines.append(f"{kind} over all its instantiations: {calls} calls, average "
                         f"{total / calls / 1e3:.1f} us per launch.")
    if len(paths) > 1 and os.path.exists(paths[1]):
        with open(paths[1]) as fh:
            for line in fh:
                if line.startswith("{") and '"roofline"' in line:
                    j = json.loads(line)
                    r = j["roofline"]
                    msg = (f"bench.py in the same run measured {r['avg_launch_us']} us per ffn13 "
                           f"launch")
                    if r.get("ffn2"):
                        msg += f" and {r['ffn2']['avg_launch_us']} us per ffn2 launch"
                    lines.append(msg + " with HIP events inside its timed region (those "
                                 "launches run under the profiler too).")
    lines += ["Other kernels in the trace (torch RNG, casts, copies) are input generation, "
              "outside the timed region.", ""]
    path = os.path.join(ROOT, "profiles", f"{workload}_kernel_stats.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA",
                 "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
N_CU, N_XCD = 256, 8


def summarize_pmc(workload: str, paths, command: str) -> str:
    """Matrix-core counters of the expert kernels, per dispatch: MFMA work
    counted by the hardware (512 flops per MOPS unit) and MFMA busy cycles
    against the cycles the GPU was active, with the expressions
    rocprof-compute uses for gfx950 (GRBM_GUI_ACTIVE is summed over the 8
    XCDs, so one XCD's active cycles are a eighth of it; each CU has 4 SIMDs
    with one matrix core each).  The last path is a --kernel-trace --stats
    directory of the same command, whose average durations turn counted
    flops into a rate (counter runs serialise kernels, so their own
    timestamps are not used)."""
    import csv
    import glob
    *pmc_dirs, stats_dir = paths
    rows = []
    for d in pmc_dirs:
        rows += _counter_rows(d)
    files = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {stats_dir}")
    with open(files[0]) as fh:
        stats = [r for r in csv.DictReader(fh) if "moe::" in r["Name"]]
    peak = MFMA_PEAK_TFLOPS["mx_e4m3" if workload == "prefill_w8a8" else "bf16"]
    lines = [f"# Matrix-core counters: {workload} workload (batches "
             f"{', '.join(map(str, WORKLOAD_BATCHES[workload]))})", "",
             "Commands (from the repository root, one MI355X), one counter pass each:", ""]
    lines += [f"    {c}" for c in command.split(" ;; ")]
    lines += ["", f"Kernel sources sha (bench.py kernel_source_sha): `{kernel_source_sha()}`", "",
              "Per dispatch, averaged over the dispatches of each kind. flops = 512 x "
              "(MOPS_BF16 + MOPS_F8 + MOPS_F6F4); util = 100 x MFMA_BUSY_CYCLES / "
              f"(4 x {N_CU} CUs x GRBM_GUI_ACTIVE / {N_XCD}); rate = flops / the kernel's average "
              f"duration in the stats run; frac = rate / {peak:.0f} TFLOP/s.", "",
              "| kernel kind | dispatches | " + " | ".join(MFMA_COUNTERS) +
              " | counted TFLOP | avg us (stats) | TFLOP/s | frac | MFMA busy % | GHz |",
              "|---|---|" + "---|" * len(MFMA_COUNTERS) + "---|---|---|---|---|---|"]
    for kind, _ in EXPERT_KINDS:
        per = {}
        clocks = []
        for r in rows:
            if kind + "_" not in r["Kernel_Name"] or r["Counter_Name"] not in MFMA_COUNTERS:
                continue
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            ns = float(r.get("End_Timestamp") or 0) - float(r.get("Start_Timestamp") or 0)
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE" and ns > 0:
                clocks.append(float(r["Counter_Value"]) / N_XCD / ns)
        if not per:
            continue
        n = max(len(v) for v in per.values())
        mean = {c: (sum(per[c]) / len(per[c]) if c in per else None) for c in MFMA_COUNTERS}
        mops = sum(mean[c] or 0.0 for c in MFMA_COUNTERS[:3])
        flops = 512.0 * mops
        ks = [r for r in stats if kind + "_" in r["Name"]]
        us = (sum(float(r["TotalDurationNs"]) for r in ks) / sum(int(r["Calls"]) for r in ks) / 1e3
              if ks else None)
        rate = flops / (us * 1e-6) / 1e12 if us else None
        util = (100.0 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * N_CU * mean["GRBM_GUI_ACTIVE"] / N_XCD)
                if mean.get("SQ_VALU_MFMA_BUSY_CYCLES") and mean.get("GRBM_GUI_ACTIVE") else None)
        ghz = f"{sum(clocks) / len(clocks):.2f}" if clocks else "-"
        cells = [f"{mean[c]:.4g}" if mean[c] is not None else "-" for c in MFMA_COUNTERS]
        lines.append(f"| {kind} | {n} | " + " | ".join(cells) +
                     f" | {flops / 1e12:.4f} | {us:.1f} | {rate:.1f} | {rate / peak:.3f} | "
                     f"{util:.1f} | {ghz} |" if us and util is not None else
                     f"| {kind} | {n} | " + " | ".join(cells) + f" | - | - | - | - | - | {ghz} |")
    lines += ["", "GHz: one XCD's active cycles over the dispatch's duration in the counter run "
              "(the clock the kernel ran at there). MFMA busy % counts against that clock, frac "
              "against the published peak.", ""]
    path = os.path.join(ROOT, "profiles", f"{workload}_mfma_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


MEMPATH_COUNTERS = ["TA_TA_BUSY_sum", "TD_TD_BUSY_sum", "TD_TC_STALL_sum",
                    "TCP_PENDING_STALL_CYCLES_sum", "TCC_HIT_sum", "TCC_MISS_sum", "GRBM_GUI_ACTIVE"]


def summarize_mempath(workload: str, dirs, command: str) -> str:
    """Vector-memory path counters of the expert kernels, per dispatch
    averaged per kernel kind: the texture address (TA) and data (TD) units'
    busy cycles, the data unit's cycles stalled on the cache (TD_TC_STALL),
    the L1's cycles at its pending-request limit (TCP_PENDING_STALL_CYCLES),
    each summed over the CUs and divided by the CUs and by one XCD's active
    cycles (GRBM_GUI_ACTIVE is summed over the XCDs), and the L2 hit rate.
    `dirs`: output directories of rocprofv3 --pmc runs of one command."""
    lines = [f"# Vector-memory path counters: {workload} workload", "",
             "Commands (from the repository root, one MI355X), one counter pass each:", ""]
    lines += [f"    {c}" for c in command.split(" ;; ")]
    lines += ["", f"Kernel sources sha (bench.py kernel_source_sha): `{kernel_source_sha()}`", "",
              f"Per dispatch, averaged over the dispatches of each kind. Unit fractions = "
              f"counter / {N_CU} CUs / (GRBM_GUI_ACTIVE / {N_XCD}); L2 hit = TCC_HIT / "
              "(TCC_HIT + TCC_MISS).", "",
              "| kernel kind | dispatches | TA busy | TD busy | TD stalled on cache | "
              "L1 at pending limit | L2 hit |",
              "|---|---|---|---|---|---|---|"]
    for kind, _ in EXPERT_KINDS:
        # each pass has its own GRBM_GUI_ACTIVE: pair every counter with its pass's
        per = {}
        for d in dirs:
            drows = [r for r in _counter_rows(d) if kind + "_" in r["Kernel_Name"]]
            by_disp = {}
            for r in drows:
                by_disp.setdefault(r["Dispatch_Id"], {})[r["Counter_Name"]] = float(r["Counter_Value"])
            for cs in by_disp.values():
                g = cs.get("GRBM_GUI_ACTIVE")
                for c, v in cs.items():
                    if c in ("TCC_HIT_sum", "TCC_MISS_sum"):
                        per.setdefault(c, []).append(v)
                    elif c != "GRBM_GUI_ACTIVE" and g:
                        per.setdefault(c, []).append(v / N_CU / (g / N_XCD))
        if not per:
            continue
        n = max(len(v) for v in per.values())
        mean = {c: sum(v) / len(v) for c, v in per.items()}

        def cell(c):
            return f"{mean[c]:.3f}" if c in mean else "-"
        hit = (f"{mean['TCC_HIT_sum'] / (mean['TCC_HIT_sum'] + mean['TCC_MISS_sum']):.3f}"
               if "TCC_HIT_sum" in mean and "TCC_MISS_sum" in mean else "-")
        lines.append(f"| {kind} | {n} | {cell('TA_TA_BUSY_sum')} | {cell('TD_TD_BUSY_sum')} | "
                     f"{cell('TD_TC_STALL_sum')} | {cell('TCP_PENDING_STALL_CYCLES_sum')} | {hit} |")
    lines.append("")
    path = os.path.join(ROOT, "profiles", f"{workload}_memory_path_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def main() -> int:
    args = parse()
    if args.summarize_traffic:
        print(summarize_traffic(args.workload, args.summarize_traffic, args.command))
        return 0
    if args.summarize_stats:
        print(summarize_stats(args.workload, args.summarize_stats, args.command))
        return 0
    if args.summarize_pmc:
        print(summarize_pmc(args.workload, args.summarize_pmc, args.command))
        return 0
    if args.summarize_mempath:
        print(summarize_mempath(args.workload, args.summarize_mempath, args.command))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the layer runs "
              "on a single GPU (how it would shard is a design, not code).", file=sys.stderr)
        return 2
    import torch

    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return 0

    from mixture_experts_moe_amd import binding as B
    from mixture_experts_moe_amd import synth
    from dataclasses import replace

    if not os.path.exists(B._LIB_PATH):
        log("libmoe.so missing: building")
        from mixture_experts_moe_amd import build
        build.build()
    B.lib()

    wl = args.workload
    batches = tuple(int(t) for t in args.batches.split(",")) if args.batches else WORKLOAD_BATCHES[wl]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating {wl} inputs, batches {batches}")
    base = synth.make_inputs(wl, T=batches[0], device=dev)
    if args.act_quant:
        base = replace(base, act_quant=None if args.act_quant == "none" else args.act_quant)
    cfg = synth.WORKLOADS[wl]
    inputs = [replace(base, x=synth.make_x(T, base.d, base.act, cfg["x_std"], 0, dev, skew=cfg["skew"]))
              for T in batches]
    weight_bytes = base.w13.numel() * base.w13.element_size() + base.w2.numel() * base.w2.element_size()
    copies = [(base.w13, base.w2)]
    if weight_bytes > (64 << 20):
        copies.append((base.w13.clone(), base.w2.clone()))
    sc = (base.s13, base.s2) if base.w == "e4m3fn" else None
    outs = [torch.empty_like(i.x) for i in inputs]
    wss = []
    for i in inputs:
        desc = B.make_desc(i.T, i.d, i.E, i.I, B._act_code(i.x), B._w_code(i.w13),
                           act_quant=i.act_quant, schedule=args.schedule)
        desc.block_m = args.block_m
        wss.append(torch.empty(max(B.moe_workspace_bytes(desc, i.top_k, True), 1), dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()
    log(f"weights {weight_bytes / 1e9:.2f} GB x {len(copies)} copies")

    counter = [0]

    def step():
        for bi, i in enumerate(inputs):
            w13, w2 = copies[counter[0] % len(copies)]
            counter[0] += 1
            B.moe_forward(i.x, i.w_gate, w13, w2, i.top_k, sc, outs[bi], block_m=args.block_m,
                          workspace=wss[bi], act_quant=i.act_quant,
                          schedule=args.schedule)

    # realised routing -> algorithmic work per forward
    work = []
    for i in inputs:
        _, ids, _ = B.moe_route(i.x, i.w_gate, i.top_k)
        work.append(alg_work(i, ids, i.top_k))
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; timing {args.steps} steps")

    # timed region 1 (value): K steps; one torch event between steps on the
    # launch stream marks each step's end (no synchronisation between steps)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for si in range(args.steps):
        step()
        marks[si + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens = sum(batches)
    value = tokens / (ms_per_step / 1e3)

    # timed region 2 (roofline): the next K steps with the library's HIP
    # events around the two expert kernels (ffn13 and ffn2) on the stream
    # they run on.  Those events put gaps between launches (about 4% of a
    # decode step), so the step time is taken from region 1.
    B.moe_timing_collect(reset=True)
    B.moe_timing_enable(["ffn13", "ffn2", "ffn_fused"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_with_events = (time.perf_counter() - t0) * 1e3 / args.steps
    B.moe_timing_enable(False)
    tim = B.moe_timing_collect(reset=True)
    ffn13_ms, ffn13_n = tim["ffn13"]
    log(f"{ms_per_step:.3f} ms/step, {value:,.0f} tokens/s; with kernel events {ms_with_events:.3f} "
        f"ms/step, ffn13 {ffn13_ms / max(ffn13_n, 1) * 1e3:.1f} us avg")

    bytes_step = sum(w["bytes"] for w in work)
    flops_step = sum(w["flops"] for w in work)
    mfma_bound = wl in ("prefill_bf16", "prefill_w8a8")
    compute = base.act_quant or base.w

    def kernel_roof(kind, ms_total, launches, kind_bytes, kind_flops):
        """Achieved rate of one kernel kind over the timed steps."""
        ms_step = ms_total / args.steps
        if not launches or ms_step <= 0:
            return None
        if mfma_bound:
            peak = MFMA_PEAK_TFLOPS[compute]
            achieved = kind_flops / (ms_step / 1e3) / 1e12
            r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s"}
        else:
            peak = HBM_PEAK_GBS
            achieved = kind_bytes / (ms_step / 1e3) / 1e9
            r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s"}
        r["frac"] = round(achieved / peak, 4)
        r["avg_launch_us"] = round(ms_total / launches * 1e3, 2)
        r["launches"] = launches
        return r

    roof = kernel_roof("ffn13", ffn13_ms, ffn13_n, sum(w["ffn13_bytes"] for w in work),
                       sum(w["ffn13_flops"] for w in work))
    label = "ffn13 (grouped W13 + SiLU*mul)"
    if roof is None:  # the persistent decode launch runs W13, W2 and the combine
        roof = kernel_roof("ffn_fused", *tim.get("ffn_fused", (0.0, 0)),
                           sum(w["ffn13_bytes"] + w["ffn2_bytes"] for w in work),
                           sum(w["ffn13_flops"] + w["ffn2_flops"] for w in work))
        label = "ffn_fused (W13 + SiLU*mul, W2 + gate, combine in one launch)"
    achieved = roof["achieved"]
    # the chip's attainable rate for the same bound, measured here
    # (include/moe_bench.h): a streaming read in the weight-streaming pattern
    # over 1 GiB (past the 256 MB last-level cache), or the big tile's LDS-fed
    # MFMA loop on random bf16
    try:
        if mfma_bound and compute == "mx_e4m3":
            att = B.bench_mfma_fp8(iters=4096, reps=4, device=dev)
        elif mfma_bound:
            att = B.bench_mfma_bf16(iters=4096, reps=4, device=dev)
        else:
            probe = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            att = B.bench_hbm_read(probe, reps=5)
            del probe
        roof["attainable"] = round(att, 1)
        roof["frac_attainable"] = round(achieved / att, 4)
    except (RuntimeError, OSError) as e:
        log(f"attainable-rate probe unavailable: {e}")
        att = None
        roof["attainable"] = roof["frac_attainable"] = None
    roof["kernel"] = label
    # the whole layer over the same timed steps (all kernels, algorithmic
    # bytes or flops of the step)
    roof["layer_frac"] = round((flops_step / (ms_per_step / 1e3) / 1e12 / roof["peak"]) if mfma_bound
                               else (bytes_step / (ms_per_step / 1e3) / 1e9 / roof["peak"]), 4)
    # the stored counters belong to the workload's own mode and schedule
    stored = None if args.act_quant or args.schedule != "auto" else load_traffic(wl)
    roof["traffic"] = stored.get("ffn13") if stored else None
    # the other expert kernel, timed in the same region
    f2 = kernel_roof("ffn2", *tim.get("ffn2", (0.0, 0)), sum(w["ffn2_bytes"] for w in work),
                     sum(w["ffn2_flops"] for w in work))
    if f2 is not None:
        f2["kernel"] = "ffn2 (grouped W2 + gate scale)"
        f2["frac_attainable"] = round(f2["achieved"] / att, 4) if att else None
        f2["traffic"] = stored.get("ffn2") if stored else None
    roof["ffn2"] = f2

    # the same step as one recorded graph per forward (moe_graph_*): one
    # launch per forward, weights rotated through the same copies
    graphs = [[B.MoeGraph(i.x, i.w_gate, w13, w2, i.top_k, sc, out=outs[bi], block_m=args.block_m,
                          workspace=wss[bi], act_quant=i.act_quant,
                          schedule=args.schedule) for (w13, w2) in copies]
              for bi, i in enumerate(inputs)]
    gcount = [0]

    def gstep():
        for bi in range(len(inputs)):
            graphs[bi][gcount[0] % len(copies)].launch()
            gcount[0] += 1

    for _ in range(args.warmup):
        gstep()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        gstep()
    torch.cuda.synchronize()
    graph_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"graph replay: {graph_ms_per_step:.3f} ms/step")

    breakdown = None
    per_batch = []
    if not args.no_breakdown:
        # second pass, batch by batch, K forwards each, one at a time
        # (synchronised): the whole forward between two torch events; then K
        # more with every kernel kind timed by the library's HIP events (the
        # breakdown; those events are kept out of the forward times)
        breakdown = {}
        for bi, (i, w) in enumerate(zip(inputs, work)):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

            def one():
                w13, w2 = copies[counter[0] % len(copies)]
                counter[0] += 1
                B.moe_forward(i.x, i.w_gate, w13, w2, i.top_k, sc, outs[bi], block_m=args.block_m,
                              workspace=wss[bi], act_quant=i.act_quant,
                              schedule=args.schedule)

            fw = 0.0
            fws = []
            for _ in range(args.steps):
                ev0.record()
                one()
                ev1.record()
                torch.cuda.synchronize()
                fws.append(ev0.elapsed_time(ev1))
                fw += fws[-1]
            B.moe_timing_collect(reset=True)
            B.moe_timing_enable(True)
            for _ in range(args.steps):
                one()
                torch.cuda.synchronize()
            B.moe_timing_enable(False)
            t2 = B.moe_timing_collect(reset=True)
            # one forward at a time, as a single graph launch
            gfw = 0.0
            gfws = []
            for _ in range(args.steps):
                g = graphs[bi][counter[0] % len(copies)]
                counter[0] += 1
                ev0.record()
                g.launch()
                ev1.record()
                torch.cuda.synchronize()
                gfws.append(ev0.elapsed_time(ev1))
                gfw += gfws[-1]
            kern = {k: round(v[0] / args.steps * 1e3, 2) for k, v in t2.items()}
            for k, v in kern.items():
                breakdown[k] = round(breakdown.get(k, 0.0) + v, 2)
            ms = fw / args.steps
            f13_us = kern["ffn13"]
            per_batch.append({
                "T": w["T"], "us": round(ms * 1e3, 1), "tokens_per_s": round(w["T"] / (ms / 1e3), 1),
                "us_p10_p50_p90": _percentiles_us(fws),
                "graph_us": round(gfw / args.steps * 1e3, 1),
                "graph_us_p10_p50_p90": _percentiles_us(gfws),
                "touched_experts": w["touched_experts"],
                "layer_hbm_GBps": round(w["bytes"] / (ms / 1e3) / 1e9, 1),
                "layer_hbm_frac": round(w["bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                "layer_TFLOPs": round(w["flops"] / (ms / 1e3) / 1e12, 2),
                "ffn13_hbm_frac": round(w["ffn13_bytes"] / (f13_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4) if f13_us else None,
                "ffn13_TFLOPs": round(w["ffn13_flops"] / (f13_us / 1e6) / 1e12, 2) if f13_us else None,
                "kernel_us": kern,
            })

    prefill = None
    if wl == "decode_bf16" and not args.no_prefill and not args.batches:
        prefill = prefill_record(B, base, copies, dev, args, counter)

    cpu = None
    if not args.no_cpu_baseline and wl in CPU_SAMPLE:
        T_s, n_s = CPU_SAMPLE[wl]
        src = next((i for i in inputs if i.T == T_s), inputs[-1])
        log(f"timing the CPU oracle on {min(n_s, src.T)} tokens of T={src.T}")
        cpu = cpu_baseline(src, min(n_s, src.T), wl, args.cpu_reps)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_p10_p50_p90": [round(v / 1e3, 4) for v in _percentiles_us(step_ms)],
        "ms_per_step_with_kernel_events": round(ms_with_events, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "mx_e4m3": "e4m3fn"}.get(compute, "bf16"),
        "data": "synthetic (seeded Gaussian inputs and random-init weights; no trained model)",
        "config": {
            "workload": wl,
            "batches_T": list(batches),
            "hidden": base.d, "experts": base.E, "top_k": base.top_k, "intermediate": base.I,
            "act": base.act, "weights": base.w, "act_quant": base.act_quant,
            "schedule": args.schedule,
            "tokens_per_step": tokens,
            "alg_bytes_per_step": bytes_step,
            "alg_flops_per_step": flops_step,
            "layer_hbm_frac": round(bytes_step / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "layer_TFLOPs": round(flops_step / (ms_per_step / 1e3) / 1e12, 2),
            "weight_copies_rotated": len(copies),
            "kernel_source_sha": kernel_source_sha(),
        },
        "roofline": roof,
        "graph_replay": {"ms_per_step": round(graph_ms_per_step, 4),
                         "tokens_per_s": round(tokens / (graph_ms_per_step / 1e3), 1)},
        "cpu_baseline": cpu,
        "prefill": prefill,
        "per_batch": per_batch,
        "kernel_us_per_step": breakdown,
    }
    print(json.dumps(line), flush=True)
    return 0


PREFILL_T = 4096


def prefill_record(B, base, copies, dev, args, counter) -> dict:
    """The prefill half of the metric on the decode layer's own weights: one
    forward of T = 4096 tokens (x ~ N(0, 1), the prefill configuration; only
    x differs from decode), timed like the main loop: K forwards after W
    warm-up (torch events between forwards), then K more with the two expert
    kernels bracketed by the library's HIP events; weights rotated through
    the same copies.
    MFMA rates use the realised routing's flops (4 d I per slot for W13, 2 d I
    for W2, plus the router's 2 d E per token for the layer)."""
    import torch
    from mixture_experts_moe_amd import synth
    from dataclasses import replace
    inp = replace(base, x=synth.make_x(PREFILL_T, base.d, base.act, 1.0, 0, dev))
    out = torch.empty_like(inp.x)
    desc = B.make_desc(inp.T, inp.d, inp.E, inp.I, B._act_code(inp.x), B._w_code(inp.w13))
    ws = torch.empty(B.moe_workspace_bytes(desc, inp.top_k, True), dtype=torch.uint8, device=dev)
    _, ids, _ = B.moe_route(inp.x, inp.w_gate, inp.top_k)
    w = alg_work(inp, ids, inp.top_k)

    def fw():
        w13, w2 = copies[counter[0] % len(copies)]
        counter[0] += 1
        B.moe_forward(inp.x, inp.w_gate, w13, w2, inp.top_k, None, out, workspace=ws)

    for _ in range(args.warmup):
        fw()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    marks[0].record()
    for si in range(args.steps):
        fw()
        marks[si + 1].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    # K more with the expert kernels timed by the library's events
    B.moe_timing_collect(reset=True)
    B.moe_timing_enable(["ffn13", "ffn2"])
    for _ in range(args.steps):
        fw()
    torch.cuda.synchronize()
    B.moe_timing_enable(False)
    tim = B.moe_timing_collect(reset=True)
    peak = MFMA_PEAK_TFLOPS["bf16"]
    rec = {"T": PREFILL_T, "x_std": 1.0, "tokens_per_s": round(PREFILL_T / (ms / 1e3), 1),
           "ms_per_forward": round(ms, 4), "forward_ms_p10_p50_p90":
           [round(v / 1e3, 4) for v in _percentiles_us(fms)],
           "touched_experts": w["touched_experts"], "peak": peak, "unit": "TFLOP/s",
           "layer_TFLOPs": round(w["flops"] / (ms / 1e3) / 1e12, 1),
           "layer_frac": round(w["flops"] / (ms / 1e3) / 1e12 / peak, 4)}
    for kind in ("ffn13", "ffn2"):
        k_ms, k_n = tim.get(kind, (0.0, 0))
        if not k_n:
            rec[kind] = None
            continue
        us = k_ms / k_n * 1e3
        tf = w[kind + "_flops"] / (us * 1e-6) / 1e12
        rec[kind] = {"bound": "mfma", "achieved": round(tf, 1), "frac": round(tf / peak, 4),
                     "avg_launch_us": round(us, 1), "launches": k_n}
    try:
        att = B.bench_mfma_bf16(iters=4096, reps=4, device=dev)
        rec["attainable"] = round(att, 1)
        for kind in ("ffn13", "ffn2"):
            if rec[kind]:
                rec[kind]["frac_attainable"] = round(rec[kind]["achieved"] / att, 4)
    except (RuntimeError, OSError) as e:
        log(f"attainable-rate probe unavailable: {e}")
        rec["attainable"] = None
    log(f"prefill T={PREFILL_T}: {ms:.3f} ms/forward, ffn13 {rec['ffn13']}, ffn2 {rec['ffn2']}")
    return rec


def _percentiles_us(ms_list):
    """p10, median, p90 of per-forward times (ms in, us out)."""
    a = sorted(ms_list)
    if not a:
        return None
    def q(f):
        x = f * (len(a) - 1)
        i = int(x)
        j = min(i + 1, len(a) - 1)
        return (a[i] + (a[j] - a[i]) * (x - i)) * 1e3
    return [round(q(0.1), 1), round(q(0.5), 1), round(q(0.9), 1)]


def load_traffic(workload: str):
    """HBM bytes per ffn13 and per ffn2 launch ({"ffn13": B, "ffn2": B}) from
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if they were taken on the current
    expert-kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{workload}_expert_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha(exclude=ROUTING_ONLY_SOURCES):
        return None
    return {kind: t[kind]["traffic_bytes_per_launch"] for kind, _ in EXPERT_KINDS if kind in t}


if __name__ == "__main__":
    sys.exit(main())
