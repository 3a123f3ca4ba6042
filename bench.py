"""Benchmark of the MoE-layer forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill8192_ep8]

One step = one moe_forward call (router, dispatch, expert FFNs with the
shared expert, combine) over one batch of seeded synthetic input already
resident in HBM.  The default workload is the largest single-GPU one: one
expert-parallel rank's share of an 8192-token prefill (32 local experts,
Zipf-skewed routing, bf16), where the grouped GEMM is MFMA-bound.  Prints
ONE JSON line:

* value      whole-layer tokens/s = T * K / (wall time of the K timed steps)
* roofline   for the kernel with the largest share of GPU time: algorithmic
             bytes (or FLOPs) per launch, from the step's real per-expert
             counts, divided by the kernel's mean launch time measured with
             HIP events on its own stream during the timed steps; the peak is
             MI355X's published HBM3E bandwidth (8 TB/s) when the kernel's
             FLOPs per byte lie below the ridge point, else its dense MFMA
             rate for the weight dtype.
             `traffic` is the measured HBM bytes per launch from rocprofv3
             counters (profiles/traffic_<kernel>_<workload>.json) when those
             were taken on the current kernel source, else null.
* step_spread  median / p10 / p90 of single steps, each bracketed by HIP
             events, in a pass of its own after the timed steps.
* input_gen_s  seconds spent drawing the synthetic inputs (outside every
             timed figure).
* cpu_baseline  the fp64 oracle timed on the host on a bounded sample of the
             same workload (first n tokens, single thread), as tokens/s,
             with the host's CPU model, logical CPUs and RAM.
* workloads  the other six workloads measured in the same run (fewer steps,
             no graph, no CPU baseline): tokens/s, the layer's fraction of
             its roofline and the dominant kernel's.  Where the streaming and
             tiled GEMMs share the device, the layer fraction is the figure
             that means something; the per-kernel one is shown beside it.

Only one GPU is used; --gpus above 1 exits with a message.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at 1 GPU + achieved HBM GB/s (decode) / MFMA % (prefill)"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
SKINNY_ROWS = 32          # groups with at most this many rows take the streaming (skinny) kernels
HALVES_ROWS = 16          # up to this many tokens every group, the shared expert too, runs in 8-row halves
DEFAULT_WORKLOAD = "prefill8192_ep8"
OTHER_WORKLOADS = ("decode16", "decode256", "clustered2048_fp8", "decode16_fp8", "decode256_fp8", "tiny_f32")


def shared_in_lists(cfg):
    """Whether the shared expert's tiles go into the routed tile launches: a
    tiled shared expert without fp8 quantisation between its GEMMs whose GEMM1
    has at least 256 tiles of 256 x 256."""
    tiles1 = -(-cfg.T // 256) * -(-cfg.I // 128)
    return bool(cfg.I_shared) and cfg.w_dtype != "fp8" and cfg.T > SKINNY_ROWS and tiles1 >= 256


def kernel_models(cfg, counts):
    """Algorithmic bytes and FLOPs of each kernel per launch, from the counts.

    Bytes count what the operation must move at least once: the weights of
    the groups it serves (with fp8 scales), the activation rows it reads and
    the outputs it writes.  h is bf16 for bf16 weights and fp32 otherwise (the
    fp8 layer reads h as e4m3 codes plus scales in the down projection, and
    its routed tiles write those codes and scales instead of h).
    """
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    fp8 = cfg.w_dtype == "fp8"
    wb = 1 if fp8 else (4 if cfg.w_dtype == "f32" else 2)
    ab = 4 if cfg.act_dtype == "f32" else 2
    hb_out = 2 if cfg.w_dtype == "bf16" else 4
    a1b = 1 if fp8 else ab
    a2b = 1 if fp8 else hb_out
    qb = cfg.quant_block
    br = getattr(cfg, "w_block_rows", 1)
    sc13 = (2 * I // br) * (H // qb) * 4 if fp8 else 0
    sc2 = (H // br) * (I // qb) * 4 if fp8 else 0
    groups = [int(c) for c in counts]
    # fp8 with more than 16 rows per routed expert on average (and T > 32):
    # the routed tiles quantise h in GEMM1's epilogue
    tile_quant = fp8 and T > SKINNY_ROWS and (T * k) // E > SKINNY_ROWS // 2
    regions = ("skinny", "tiled", "tiled128", "shared_skinny", "shared_tiled", "shared_tiled128")
    m = {f"ffn_gemm{g}_{r}": {"bytes": 0, "flops": 0} for g in (1, 2) for r in regions}
    # (rows, region): a group of > 32 rows takes 256-row tiles; with fp8
    # weights only its floor(m / 256) full tiles do, and its other m mod 256
    # rows take the 128-row kernel (routed groups: when they are at most 128,
    # else one more 256-row tile).  Each kernel that serves a group streams
    # that group's weights once.
    def tiled(mg, pre):
        rest = mg % 256
        if not fp8 or (not pre and rest > 128):
            return [(mg, pre + "tiled")]
        return [(mg - rest, pre + "tiled"), (rest, pre + "tiled128")]
    items = []
    for mg in [int(c) for c in counts]:
        if mg <= SKINNY_ROWS:
            items.append((mg, "skinny"))
        else:
            items += tiled(mg, "")
    if cfg.I_shared:
        # T <= 16: the shared expert runs as two 8-row halves inside the routed
        # streaming launch; up to 32 tokens it has a streaming launch of its own;
        # when its GEMM1 fills the device (bf16/fp32) its tiles join the routed lists
        if T <= HALVES_ROWS:
            items.append((T, "skinny"))
        elif T <= SKINNY_ROWS:
            items.append((T, "shared_skinny"))
        elif shared_in_lists(cfg):
            items += tiled(T, "")
        else:
            items += tiled(T, "shared_")
    for mg, reg in items:
        if mg == 0:
            continue
        g1, g2 = m[f"ffn_gemm1_{reg}"], m[f"ffn_gemm2_{reg}"]
        h_out = mg * I + mg * (I // qb) * 4 if tile_quant and reg in ("tiled", "tiled128") else mg * I * hb_out
        g1["bytes"] += 2 * I * H * wb + sc13 + mg * H * a1b + h_out + (mg * H // qb * 4 if fp8 else 0)
        g1["flops"] += 2 * mg * 2 * I * H
        g2["bytes"] += H * I * wb + sc2 + mg * I * a2b + mg * H * ab + (mg * I // qb * 4 if fp8 else 0)
        g2["flops"] += 2 * mg * H * I
    touched = sum(1 for c in counts if int(c) > 0)
    layer_bytes = (touched + (1 if cfg.I_shared else 0)) * (3 * H * I * wb + sc13 + sc2) \
        + E * H * ab + E * 4 + 2 * T * H * ab
    layer_flops = (T * k + (T if cfg.I_shared else 0)) * 6 * H * I + 2 * T * H * E
    return m, dict(bytes=layer_bytes, flops=layer_flops, touched=touched)


def kernel_line(name, prof_entry, models):
    """us per launch (with events around every kernel) and, for modelled kernels, GB/s or TFLOP/s."""
    launches, tot_ms = prof_entry
    us = tot_ms / max(launches, 1) * 1e3
    d = {"us": round(us, 2)}
    mm = models.get(name)
    if mm and us > 0 and (mm["bytes"] or mm["flops"]):
        d["GBps"] = round(mm["bytes"] / (us * 1e-6) / 1e9, 1)
        d["TFLOPs"] = round(mm["flops"] / (us * 1e-6) / 1e12, 2)
    return d


def traffic_for(kernel, workload):
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.isfile(p):
        return None
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    from moe_measure.profiling import kernel_source_hash
    if d.get("source_hash") != kernel_source_hash(kernel):
        return None
    return d.get("bytes_per_launch")


def host_info():
    """CPU model, logical CPUs and RAM of the host the oracle is timed on."""
    model, ram_gb = None, None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram_gb = round(int(line.split()[1]) / 2**20, 1)
                break
    except OSError:
        pass
    return {"cpu": model, "nproc": os.cpu_count(), "ram_gib": ram_gb}


def cpu_baseline(inp_gpu, n_tokens, min_s=10.0, max_passes=8):
    """Time the fp64 oracle, single-threaded, on the first n tokens, repeating
    the pass until at least min_s seconds of CPU work (at most max_passes).
    Returns (seconds, passes)."""
    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    from moe_inputs import MoEInputs

    host = MoEInputs(inp_gpu.cfg, *[getattr(inp_gpu, f).cpu() if getattr(inp_gpu, f) is not None else None
                                    for f in ("x", "wg", "bias", "w13", "w2", "ws13", "ws2", "w13_scale",
                                              "w2_scale", "ws13_scale", "ws2_scale")])
    toks = list(range(n_tokens))
    nthreads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with threadpool_limits(limits=1):
            passes = 0
            t0 = time.perf_counter()
            while True:
                oracle.forward_tokens(host, toks)
                passes += 1
                dt = time.perf_counter() - t0
                if dt >= min_s or passes >= max_passes:
                    break
    finally:
        torch.set_num_threads(nthreads)
    return dt, passes


def shares_device(cfg):
    """Whether the streaming and tiled GEMMs of a step run at the same time:
    the library forks the tiled launches onto a side stream when the mean
    rows per routed expert lie in 17..1023 and the layer has more than 32
    tokens; per-kernel spans then include the sharing."""
    mean_rows = cfg.T * cfg.k // cfg.E
    return cfg.T > SKINNY_ROWS and SKINNY_ROWS // 2 < mean_rows < 1024


def measure(moe, torch, cfg, steps, warmup, detail=True, graph=True, warm_s=0.0):
    """Time `steps` whole-layer steps of one workload; returns a dict.
    Warm-up is `warmup` steps, continued until at least `warm_s` seconds of
    steps have run (the GPU's clocks drop while the host works alone)."""
    from moe_inputs import make_inputs

    tg = time.perf_counter()
    inp = make_inputs(cfg, "cuda")
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - tg   # input generation, reported apart from every timed figure
    mc = moe.cfg_from(cfg)
    ws = moe.alloc_workspace(mc)
    w = moe.Weights.from_inputs(inp)
    y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32,
                    device="cuda")
    step = lambda: moe.moe_forward(mc, inp.x, inp.wg, inp.bias, w, ws=ws, y=y)   # noqa: E731

    tw = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - tw < warm_s:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # untimed pass: routing of this batch (for the byte model) and the per-kernel
    # breakdown of instrumented steps (every kernel bracketed by events)
    _, idx, _, counts = moe.moe_forward(mc, inp.x, inp.wg, inp.bias, w, ws=ws, return_routing=True)
    torch.cuda.synchronize()
    counts_h = counts.cpu().tolist()
    moe.moe_profile_start()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    breakdown = moe.moe_profile_stop()
    # The dominant kernel is the one with the longest roofline time: its
    # algorithmic bytes at the HBM peak or its FLOPs at the MFMA peak,
    # whichever is longer, which the routing alone fixes.  Event spans would
    # serve where kernels run one after another, but the streaming and tiled
    # GEMMs that share the device swap places from run to run.  Spans break
    # ties and cover unmodelled kernels.
    models, layer = kernel_models(cfg, counts_h)
    wdt = "fp8" if cfg.w_dtype == "fp8" else cfg.act_dtype
    peak = MFMA_PEAK_TFLOPS[wdt]

    def roof_s(n):
        mm = models.get(n)
        if not mm:
            return -1.0
        return max(mm["bytes"] / (HBM_PEAK_GBPS * 1e9), mm["flops"] / (peak * 1e12))

    dom = max(breakdown, key=lambda n: (roof_s(n), breakdown[n][1]))

    # timed region: K steps; the dominant kernel is bracketed by HIP events on its launch stream
    moe.moe_profile_start(dom)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    prof = moe.moe_profile_stop()
    gpu_ms = ev0.elapsed_time(ev1)

    ms_per_step = wall_ms / steps
    tokens_per_s = cfg.T * steps / (wall_ms / 1e3)

    launches, tot_ms = prof[dom]
    avg_ms = tot_ms / max(launches, 1)
    ridge = peak * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if dom in models:
        mm = models[dom]
        # the kernel's own roofline: HBM-bound below the ridge point
        # (peak FLOP/s / peak bytes/s), MFMA-bound above it
        tflops = mm["flops"] / (avg_ms * 1e-3) / 1e12
        if mm["flops"] < ridge * mm["bytes"]:
            achieved = mm["bytes"] / (avg_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "mfma_frac": round(tflops / peak, 4)}   # the MFMA rate beside it, for reference
        else:
            roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4)}
        roof["traffic"] = traffic_for(dom, cfg.name)
    else:
        roof = {"bound": "hbm", "achieved": None, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": None,
                "traffic": None}
    roof["kernel"] = dom
    roof["kernel_avg_us"] = round(avg_ms * 1e3, 2)
    roof["algorithmic_per_launch"] = models.get(dom, {})

    layer_gbps = layer["bytes"] / (ms_per_step * 1e-3) / 1e9
    layer_tflops = layer["flops"] / (ms_per_step * 1e-3) / 1e12
    layer_bound = "mfma" if layer["flops"] >= ridge * layer["bytes"] else "hbm"
    layer_frac = layer_tflops / peak if layer_bound == "mfma" else layer_gbps / HBM_PEAK_GBPS
    out = {
        "workload": cfg.name, "T": cfg.T, "dtype": wdt, "tokens_per_s": round(tokens_per_s, 1),
        "ms_per_step": round(ms_per_step, 4), "steps": steps, "warmup": n_warm,
        "roofline": roof,
        "layer": {"algorithmic_bytes": layer["bytes"], "flops": layer["flops"], "GBps": round(layer_gbps, 1),
                  "hbm_frac": round(layer_gbps / HBM_PEAK_GBPS, 4), "TFLOPs": round(layer_tflops, 2),
                  "mfma_frac": round(layer_tflops / peak, 4), "bound": layer_bound, "frac": round(layer_frac, 4),
                  "gpu_event_ms_per_step": round(gpu_ms / steps, 4)},
        "gemms_share_device": shares_device(cfg),
        "touched_experts": layer["touched"],
        "input_gen_s": round(gen_s, 2),
    }
    if detail:
        out["kernels"] = {n: kernel_line(n, v, models) for n, v in sorted(breakdown.items())}
        # per-step spread, in a pass of its own after the timed region: each step
        # bracketed by events on the caller's stream (the side stream joins it)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a0, a1 in evs:
            a0.record()
            step()
            a1.record()
        torch.cuda.synchronize()
        per_step = sorted(a0.elapsed_time(a1) for a0, a1 in evs)
        pct = lambda q: per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]   # noqa: E731
        out["step_spread"] = {"median_ms": round(pct(0.5), 4), "p10_ms": round(pct(0.1), 4),
                              "p90_ms": round(pct(0.9), 4)}
        # beside the timed steps: the same step captured once as a HIP graph
        # (moe_graph_capture) and replayed K times
        out["graph"] = None
        if graph:
            g = moe.MoEGraph(mc, inp.x, inp.wg, inp.bias, w, y, ws)
            for _ in range(warmup):
                g.launch()
            torch.cuda.synchronize()
            g0 = time.perf_counter()
            for _ in range(steps):
                g.launch()
            torch.cuda.synchronize()
            graph_ms = (time.perf_counter() - g0) * 1e3 / steps
            g.close()
            out["graph"] = {"ms_per_step": round(graph_ms, 4), "tokens_per_s": round(cfg.T / (graph_ms * 1e-3), 1),
                            "eager_minus_graph_us": round((ms_per_step - graph_ms) * 1e3, 2)}
        # beside the layer, outside the timed steps: routing statistics of this
        # batch (loads over 8 expert-parallel ranks when E allows, skews, affinity)
        n_ranks = 8 if cfg.E % 8 == 0 else 1
        moe.moe_routing_stats(mc, idx, n_ranks)
        torch.cuda.synchronize()
        moe.moe_profile_start()
        for _ in range(5):
            _, _, skew, _ = moe.moe_routing_stats(mc, idx, n_ranks)
        torch.cuda.synchronize()
        sp = moe.moe_profile_stop()
        stat_us = {n: round(v[1] / max(v[0], 1) * 1e3, 2) for n, v in sorted(sp.items())}
        skew_h = skew.cpu().tolist()
        out["routing_stats"] = {"n_ranks": n_ranks, "rho_rank": round(skew_h[0], 4),
                                "rho_expert": round(skew_h[1], 4), "us_per_call": round(sum(stat_us.values()), 2),
                                "kernels_us": stat_us}
        out["inputs"] = inp
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-tokens", type=int, default=16, help="tokens in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="measure only --workload")
    ap.add_argument("--other-steps", type=int, default=10, help="timed steps per other workload")
    ap.add_argument("--quick", action="store_true", help="--workload only, no CPU baseline (tuning sweeps)")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay measurement (profiled runs)")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr, flush=True)
        return 2

    import torch

    import mixture_experts_layer_11_amd as moe
    from moe_inputs import get_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    moe.load_library()
    cfg = get_config(args.workload)
    print(f"[bench] {cfg.name}: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    r = measure(moe, torch, cfg, args.steps, args.warmup, detail=True, graph=not args.no_graph)
    inp = r.pop("inputs")

    cpu = None
    if not (args.no_cpu_baseline or args.quick):
        n = min(args.cpu_tokens, cfg.T)
        print(f"[bench] cpu baseline: fp64 oracle on {n} tokens", file=sys.stderr, flush=True)
        dt, passes = cpu_baseline(inp, n)
        cpu = {"value": round(n * passes / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "host": host_info(),
               "sample": f"first {n} of {cfg.T} tokens of {cfg.name}, {passes} passes: fp64 numpy oracle, token "
                         f"by token (routing, fp64 upcast of each touched expert, SwiGLU, weighted sum), 1 thread, "
                         f"inputs already in host memory; {dt:.2f} s"}
    del inp
    torch.cuda.empty_cache()

    others = None
    if not (args.no_others or args.quick):
        others = {}
        for name in OTHER_WORKLOADS:
            if name == cfg.name:
                continue
            print(f"[bench] {name}: >= 3 warmup steps over >= 0.5 s + {args.other_steps} timed steps", file=sys.stderr,
                  flush=True)
            o = measure(moe, torch, get_config(name), args.other_steps, 3, detail=False, warm_s=0.5)
            rf = o["roofline"]
            others[name] = {"tokens_per_s": o["tokens_per_s"], "ms_per_step": o["ms_per_step"],
                            "steps": o["steps"], "warmup_steps": o["warmup"],
                            "layer_bound": o["layer"]["bound"], "layer_frac": o["layer"]["frac"],
                            "layer_GBps": o["layer"]["GBps"], "layer_TFLOPs": o["layer"]["TFLOPs"],
                            "gemms_share_device": o["gemms_share_device"],
                            "dominant_kernel": rf["kernel"], "kernel_bound": rf["bound"],
                            "kernel_frac": rf["frac"], "kernel_avg_us": rf["kernel_avg_us"]}
            torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k, "I": cfg.I,
                   "I_shared": cfg.I_shared, "score": cfg.score, "weights": cfg.w_dtype, "routing": cfg.routing,
                   "touched_experts": r["touched_experts"], "parallelism": "none (1 GPU)"},
        "roofline": r["roofline"],
        "layer": r["layer"],
        "kernels": r["kernels"],
        "step_spread": r["step_spread"],
        "input_gen_s": r["input_gen_s"],
        "graph": r["graph"],
        "routing_stats": r["routing_stats"],
        "cpu_baseline": cpu,
        "workloads": others,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
