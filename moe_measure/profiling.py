"""Profiling helpers: library kernel names, rocprofv3 names, counter summaries.

The library's profiler (moe_profile_start/stop) names kernels by role
("ffn_gemm1_skinny", ...); rocprofv3 reports demangled template names.
``rocprof_name`` maps one to the other for a given weight dtype, and
``kernel_source_hash`` fingerprints the sources a kernel is built from, so a
stored counter reading is only used while the kernel is unchanged.

CLI (writes profiles/<kernel>_<workload>.md and
profiles/traffic_<kernel>_<workload>.json from rocprofv3 CSV output):

  python -m moe_measure.profiling --workload decode16 \\
      --kernel ffn_gemm1_skinny --stats RUN_kernel_stats.csv \\
      --fetch FETCH_counter_collection.csv --write WRITE_counter_collection.csv \\
      --copy-fetch COPYF.csv --copy-write COPYW.csv --copy-bytes 1073741824 \\
      --bench-log BENCH.log --command "..." [--command "..."]
"""

import argparse
import csv
import hashlib
import json
import os
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_11_amd", "csrc")

KERNEL_SOURCES = {
    "ffn_gemm1_skinny": "ffn_skinny.hip", "ffn_gemm2_skinny": "ffn_skinny.hip",
    "ffn_gemm1_shared_skinny": "ffn_skinny.hip", "ffn_gemm2_shared_skinny": "ffn_skinny.hip",
    **{f"ffn_gemm{g}_{s}tiled{t}": "ffn_tiled.hip" for g in (1, 2) for s in ("", "shared_") for t in ("", "128")},
    "ffn_plan": "ffn.hip",
    "route_gate_fused": "route.hip", "route_gate_split": "route.hip", "route_gate_tiled": "route.hip",
    "route_reduce_select": "route.hip",
    "dispatch_count": "dispatch.hip", "dispatch_scan": "dispatch.hip", "dispatch_scatter": "dispatch.hip",
    "dispatch_small": "dispatch.hip",
    "quant_fp8": "quant.hip", "combine": "combine.hip",
}

_DT = {"f32": 0, "bf16": 1, "fp8": 2}


# Files that decide a kernel's launch geometry and what shares the device
# with it, besides its own source: the expert FFN's launcher and work-list
# builder (grids, tile lists, side streams), and the stream helpers.
LAUNCH_SOURCES = {"ffn": ("ffn.hip", "plan.h", "streams.cpp"), "route": (), "dispatch": ("plan.h",),
                  "quant": (), "combine": (), "stats": ()}


def kernel_source_hash(kernel: str) -> str:
    """sha256 prefix of every source a stored counter reading depends on: the
    kernel's own file, its launcher, and all device and launch headers."""
    h = hashlib.sha256()
    src = KERNEL_SOURCES.get(kernel, "")
    launch = LAUNCH_SOURCES.get(src.split(".")[0].split("_")[0], ())
    headers = sorted(f for f in os.listdir(CSRC) if f.endswith(".h"))
    for f in [src, *launch, *headers]:
        p = os.path.join(CSRC, f)
        if f and os.path.isfile(p):
            h.update(f.encode())
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def rocprof_name(kernel: str, w_dtype: str) -> str:
    """Prefix of the demangled name rocprofv3 reports for a library kernel."""
    dt = _DT[w_dtype]
    if kernel in ("ffn_gemm1_skinny", "ffn_gemm2_skinny"):
        return f"void (anonymous namespace)::ffn_skinny_kernel<{dt}, {int(kernel[8])}>"
    if kernel.startswith("ffn_gemm") and "_tiled" in kernel:
        shared = "true" if "_shared_" in kernel else "false"
        tm = 128 if kernel.endswith("128") else 256
        return f"void (anonymous namespace)::ffn_fat_kernel<{dt}, {int(kernel[8])}, {shared}, {tm}, "   # then the fp8 scale-block and streamed-weight flags
    if kernel.startswith("ffn_gemm") and kernel.endswith("_shared_skinny"):
        return f"void (anonymous namespace)::ffn_shared_skinny_kernel<{dt}, {int(kernel[8])}, "
    fixed = {"ffn_plan": "(anonymous namespace)::ffn_plan_kernel",
             "route_reduce_select": "(anonymous namespace)::route_reduce_kernel",
             "dispatch_count": "(anonymous namespace)::dispatch_count_kernel",
             "dispatch_scan": "(anonymous namespace)::dispatch_scan_kernel",
             "dispatch_scatter": "(anonymous namespace)::dispatch_scatter_kernel",
             "route_gate_fused": "void (anonymous namespace)::gate_kernel<",
             "route_gate_split": "void (anonymous namespace)::gate_kernel<",
             "route_gate_tiled": "void (anonymous namespace)::gate_tile_kernel<",
             "combine": "void (anonymous namespace)::combine",
             "quant_fp8": "void (anonymous namespace)::quant_fp8_kernel<"}
    return fixed[kernel]


def _counter_values(path, prefix, counter):
    vals = []
    for r in csv.DictReader(open(path)):
        if r["Kernel_Name"].startswith(prefix) and r["Counter_Name"] == counter:
            vals.append(float(r["Counter_Value"]))
    return vals


def _copy_factor(path, counter, copy_bytes):
    vals = []
    for r in csv.DictReader(open(path)):
        if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no copy dispatch with {counter} in {path}")
    return copy_bytes / (statistics.median(vals) * 1024.0), vals


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--w-dtype", default=None)
    ap.add_argument("--stats", required=True, help="rocprofv3 --kernel-trace --stats kernel_stats.csv")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--counters", action="append", default=[],
                    help="counter_collection.csv of another --pmc pass (SQ_*, GRBM_* counters), repeatable")
    ap.add_argument("--bench-log", help="output of the bench run profiled with --kernel-trace")
    ap.add_argument("--command", action="append", default=[], help="command lines that produced the inputs")
    ap.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args(argv)

    import sys
    sys.path.insert(0, ROOT)
    from moe_inputs import get_config
    cfg = get_config(args.workload)
    wdt = args.w_dtype or cfg.w_dtype
    prefix = rocprof_name(args.kernel, wdt)

    stats = [r for r in csv.DictReader(open(args.stats))]
    ours = [r for r in stats if r["Name"].startswith(("void (anonymous namespace)::", "(anonymous namespace)::"))]
    dom = [r for r in ours if r["Name"].startswith(prefix)]
    if not dom:
        raise SystemExit(f"{prefix} not in {args.stats}")
    avg_us = float(dom[0]["AverageNs"]) / 1e3

    bench = None
    if args.bench_log:
        for line in open(args.bench_log):
            if line.startswith("{"):
                bench = json.loads(line)

    traffic = None
    lines = [f"# {args.kernel} on {args.workload}", "",
             f"Library kernel `{args.kernel}` = rocprofv3 `{prefix}...`.", "", "## Commands", ""]
    lines += [f"    {c}" for c in args.command]
    lines += ["", "## Kernel trace (rocprofv3 --kernel-trace --stats), library kernels", "",
              "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(ours, key=lambda r: -float(r["TotalDurationNs"])):
        nm = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "")
        nm = nm.split("(")[0] if "(" in nm else nm
        lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                     f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} |")
    lines += ["", f"Average duration of `{args.kernel}`: **{avg_us:.2f} us** (rocprofv3)."]
    if bench:
        r = bench["roofline"]
        lines += [f"Same kernel timed live by bench.py with HIP events: **{r['kernel_avg_us']} us** "
                  f"(kernel `{r['kernel']}`); algorithmic bytes per launch {r['algorithmic_per_launch']['bytes']}; "
                  f"achieved {r['achieved']} {r['unit']} = {r['frac']:.3f} of {r['peak']}."]
    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        ff, fv = _copy_factor(args.copy_fetch, "FETCH_SIZE", args.copy_bytes)
        wf, wv = _copy_factor(args.copy_write, "WRITE_SIZE", args.copy_bytes)
        fk = _counter_values(args.fetch, prefix, "FETCH_SIZE")
        wk = _counter_values(args.write, prefix, "WRITE_SIZE")
        fetch_b = statistics.median(fk) * 1024.0 * ff
        write_b = statistics.median(wk) * 1024.0 * wf
        traffic = fetch_b + write_b
        lines += ["", "## HBM traffic (rocprofv3 --pmc, one counter per run)", "",
                  f"Calibration: a plain {args.copy_bytes} B device copy reads FETCH_SIZE "
                  f"{statistics.median(fv):.1f} KiB and WRITE_SIZE {statistics.median(wv):.1f} KiB per dispatch, "
                  f"so FETCH_SIZE is scaled by {ff:.4f} and WRITE_SIZE by {wf:.4f}.", "",
                  f"`{args.kernel}`: FETCH_SIZE median {statistics.median(fk):.1f} KiB over {len(fk)} dispatches "
                  f"-> {fetch_b:.4e} B read; WRITE_SIZE median {statistics.median(wk):.1f} KiB -> {write_b:.4e} B "
                  f"written; traffic {traffic:.4e} B per launch."]
        if bench:
            alg = bench["roofline"]["algorithmic_per_launch"]["bytes"]
            lines.append(f"Algorithmic bytes per launch {alg:.4e} B: traffic / algorithmic = {traffic / alg:.4f}.")
        rec = {"kernel": args.kernel, "workload": args.workload, "source_hash": kernel_source_hash(args.kernel),
               "bytes_per_launch": traffic, "fetch_bytes": fetch_b, "write_bytes": write_b,
               "fetch_scale": ff, "write_scale": wf, "commands": args.command}
        with open(os.path.join(args.out_dir, f"traffic_{args.kernel}_{args.workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
    if args.counters:
        med = {}
        for path in args.counters:
            names = sorted({r["Counter_Name"] for r in csv.DictReader(open(path))})
            for c in names:
                v = _counter_values(path, prefix, c)
                if v:
                    med[c] = (statistics.median(v), len(v))
        lines += ["", "## Shader counters (rocprofv3 --pmc, medians over dispatches)", "",
                  "| counter | median per dispatch | dispatches |", "|---|---|---|"]
        lines += [f"| {c} | {v:.4e} | {n} |" for c, (v, n) in sorted(med.items())]
        if "GRBM_GUI_ACTIVE" in med:
            raw = med["GRBM_GUI_ACTIVE"][0] / avg_us          # cycles per us = MHz
            # the counter is summed over the 8 XCDs' graphics blocks when it reads above any clock
            per = 8 if raw > 4000 else 1
            mhz = raw / per
            lines += ["", f"Clock while the kernel runs: GRBM_GUI_ACTIVE {med['GRBM_GUI_ACTIVE'][0]:.4e} / "
                          f"{avg_us:.1f} us{' / 8 XCDs' if per == 8 else ''} = **{mhz:.0f} MHz** "
                          f"(2400 MHz is the clock of the published peaks)."]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
                simd_cycles = mhz * avg_us * 1024          # 256 CUs x 4 SIMDs
                busy = med["SQ_VALU_MFMA_BUSY_CYCLES"][0] / simd_cycles
                lines.append(f"MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x 1024 SIMDs) = **{busy:.3f}**.")
                if "SQ_INSTS_MFMA" in med:
                    lines.append(f"Busy cycles per MFMA instruction: "
                                 f"{med['SQ_VALU_MFMA_BUSY_CYCLES'][0] / med['SQ_INSTS_MFMA'][0]:.1f}.")
            if "SQ_INSTS_VALU" in med and "SQ_INSTS_MFMA" in med and med["SQ_INSTS_MFMA"][0] > 0:
                lines.append(f"Vector ALU instructions per MFMA instruction: SQ_INSTS_VALU / SQ_INSTS_MFMA = "
                             f"**{med['SQ_INSTS_VALU'][0] / med['SQ_INSTS_MFMA'][0]:.2f}**.")
            if bench and bench["roofline"]["unit"] == "TFLOP/s":
                at_clock = bench["roofline"]["peak"] * mhz / 2400.0
                lines.append(f"Peak at that clock {at_clock:.0f} TFLOP/s: the kernel runs at "
                             f"{bench['roofline']['achieved'] / at_clock:.3f} of it.")
    with open(os.path.join(args.out_dir, f"{args.kernel}_{args.workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
