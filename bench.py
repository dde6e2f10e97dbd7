#!/usr/bin/env python3
"""Benchmark of the output-centric MoE decode layer on one MI355X.

One step = one MoE decode layer (gate/up kernel + down kernel) over one batch
of synthetic input. Default workload: B=1 token, E=128 experts, top-8,
H=2048, I=768, MXFP8 weights (the single-token wide-MoE decode layer).

Weights must come from HBM, not from the 256 MB Infinity Cache: the timed run
cycles through R identical copies of the layer's weights at distinct HBM
addresses (like consecutive layers of a model), so any one copy's bytes are
touched again only after R-1 other layers' worth of traffic (R * 39 MB >> the
cache). The K steps are captured once in a HIP graph and replayed, so the
time is the GPU's, not the Python launch loop's.

Prints ONE JSON line. value = achieved GB/s over the unique routed-weight
bytes (codes + scales of every distinct routed expert) per layer.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak, AMD specification
METRIC = "µs/MoE layer + achieved HBM GB/s (routed weight bytes) vs peak, B=1..64"
DEFAULT_WORKLOAD = "wide_B1_E128_k8_H2048_I768"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(src: str) -> str:
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.strip() for line in src.splitlines() if line.strip())


# The sources the kernels of the decode-batch layer (per-slot gate/up, per-output down) are
# compiled from, with the launch table; and those of the large-batch kernels. A committed profile
# of either set stays valid while the code in these files (comments and blank lines removed) is
# unchanged.
LAYER_SOURCES = ("gate_up.hip", "gate_up_body.h", "down.hip", "down_body.h", "down_onepass.hip", "launch.h",
                 "mx_device.h", "moedecode.hip")
GROUPED_SOURCES = ("gate_up_grouped.hip", "down_grouped.hip", "grouped_common.h", "launch.h", "mx_device.h",
                   "moedecode.hip")


def source_digest(files=LAYER_SOURCES) -> str:
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "output_centric_expert_amd", "csrc", name)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_profile(prefix: str, workload: str, files=LAYER_SOURCES):
    """A committed profile summary (profiles/<prefix>_<workload>.json), if it was taken from the
    current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{prefix}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("source_digest") != source_digest(files):
        return None
    d["_file"] = os.path.relpath(p, ROOT)
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--wformat", default="mxfp8", choices=["mxfp8", "mxfp4"],
                    help="routed-weight format (the headline metric is quoted on mxfp8)")
    ap.add_argument("--copies", type=int, default=32, help="distinct HBM copies of the layer weights")
    ap.add_argument("--tune", default=None, help="launch-shape override (a moed_tuning_init spec)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--single", action="store_true",
                    help="time only --workload (no per-config list of every workload)")
    ap.add_argument("--all", action="store_true",
                    help="time every decode workload (one JSON line each); not the driver's line")
    ap.add_argument("--diagnostics", action="store_true",
                    help="labelled diagnostics, not the driver's line: adjacent vs scattered expert ids, "
                         "warm cache (one weight copy), contiguous hot experts on the skewed workload")
    ap.add_argument("--counters", action="store_true",
                    help="eager launches for rocprofv3 --pmc passes (copy kernel of known size, "
                         "then the two layer kernels); prints the launch plan, no timing")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer runs on a single MI355X and "
              "there is no multi-GPU path in this build (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from output_centric_expert_amd import moedecode as md
    from output_centric_expert_amd import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    md.load()
    if args.tune:
        md.set_default_tuning(args.tune)

    if args.all:
        all_workloads(md, synth, args)
        return
    if args.diagnostics:
        diagnostics(md, synth, args)
        return

    shape = synth.WORKLOADS[args.workload]
    t0 = time.time()
    L = synth.make_layer(shape, device="cuda", wformat=args.wformat)
    R = max(1, args.copies)
    log(f"inputs ready in {time.time() - t0:.1f} s: {shape}, {R} weight copies")
    if args.counters:
        x, ids, w = md.layer_device_inputs(L)
        copies = weight_copies(L, R)
        out = torch.empty((shape.B, shape.H), dtype=torch.bfloat16, device="cuda")
        a = torch.empty((shape.B, shape.k, shape.I), dtype=torch.float32, device="cuda")
        counters_run(md, x, ids, w, copies, out, a, args.workload, L.wformat)
        return

    K, W = args.steps, args.warmup
    log("step: the timed layer graph")
    t = measure_layer(md, L, R, K, W)
    B, E, k, H, I = shape.B, shape.E, shape.k, shape.H, shape.I
    U = L.unique_experts
    uniq = L.unique_weight_bytes
    gu_bytes, dn_bytes = kernel_bytes(L)
    ms_per_step = t["ms_per_step"]
    gbs = uniq / (ms_per_step * 1e-3) / 1e9

    log("step: read floors")
    peak = measured_read_peak(md)
    floors = read_floors(md, (dn_bytes, gu_bytes, gu_bytes + dn_bytes)) if uniq < (1 << 30) else None
    files = LAYER_SOURCES if gate_up_kernel_name(L) != "moe_gate_up_grouped_wide_kernel" else GROUPED_SOURCES
    counters = load_profile("counters_layer", args.workload, files) if L.wformat == "mxfp8" else None
    trace = load_profile("kernel_trace", args.workload, files) if L.wformat == "mxfp8" else None
    roof = roofline(L, "gate_up", gu_bytes, t, counters, trace, floors)
    roof_dn = roofline(L, "down", dn_bytes, t, counters, trace, floors)

    per_config = None
    if not args.single:
        per_config = []
        for name in synth.WORKLOAD_ORDER:
            log(f"step: per-config {name}")
            per_config.append(config_entry(md, synth, name, args.wformat,
                                           reuse=(L, t) if name == args.workload else None,
                                           cpu=not args.no_cpu, peak=peak))
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        log("step: cpu baseline")
        cpu = cpu_baseline(L, uniq, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": f"synthetic (seeded N(0,1) activations, N(0,0.02) weights encoded to {L.wformat.upper()}, "
                "softmax top-k routing)",
        "config": {"workload": args.workload, "B": B, "E": E, "k": k, "H": H, "I": I,
                   "weights": WEIGHT_DESC[L.wformat], "activations": "bf16", "out": "bf16",
                   "unique_experts": U, "unique_weight_bytes": uniq, "weight_copies": R,
                   "timing": "HIP graph of K layers, HIP events on the launch stream"},
        **timing_fields(L, t),
        "measured_read_peak_gbs": round(peak, 1),
        "frac_of_measured_read_peak": round(gbs / peak, 4),
        "read_floors": floors,
        "roofline": roof,
        "roofline_down": roof_dn,
        "per_config": per_config,
        "cpu_baseline": cpu,
        "tuning": args.tune or "built-in",
    }
    print(json.dumps(res), flush=True)


def down_kernel_name(L):
    """The down kernel(s) the built-in launch table picks inside moe_decode: the expert-major
    kernel plus its combine once B*k >= 2E; else, for float32 a when the token's k slots form one
    lane-group set and a row is at most one chunk per lane, the blocks form of the one-pass kernel
    once B*k >= E (H a multiple of 64) and the one-pass kernel below; else the staged per-output
    kernel."""
    sh = L.shape
    if sh.B * sh.k >= 2 * sh.E:
        return "moe_down_expert_kernel + moe_down_combine_kernel"
    cpr = sh.I // 32 if L.wformat == "mxfp4" else sh.I // 16
    groups = 1
    while groups < 4 and cpr <= 64 // (2 * groups) and 2 * groups <= sh.k:
        groups *= 2
    jb = sh.k // groups
    one_pass_shape = sh.k == groups * jb and jb & (jb - 1) == 0 and jb <= 8 and cpr <= 64 // groups and \
        sh.k * sh.I * 4 <= 65536
    if one_pass_shape and sh.B * sh.k >= sh.E and sh.H % 64 == 0 and not (L.wformat == "mxfp4" and jb == 8):
        return "moe_down_blocks_kernel"
    if one_pass_shape and sh.B * sh.k < sh.E:
        return "moe_down_onepass_kernel"
    return "moe_down_staged_kernel"


def roofline(L, step, alg_bytes, t, counters, trace, floors):
    """Roofline entry of one layer step: algorithmic bytes per launch over the kernel's average
    launch duration, against MI355X's 8 TB/s. The duration is measured live: HIP events on the
    launch stream around a graph of K launches of the step alone (weights rotating through the
    copies), divided by K. The entry also carries the mean duration the committed rocprofv3
    kernel trace gives for the same launches (the one-step graph; tracing lengthens each
    dispatch a little), when the trace was taken from the current sources, HBM traffic from the
    committed counter runs, and the best same-size pure read."""
    us = t["ms_" + step] * 1e3
    achieved = alg_bytes / (us * 1e-6) / 1e9
    e = {"bound": "hbm", "kernel": gate_up_kernel_name(L) if step == "gate_up" else down_kernel_name(L),
         "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
         "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_us": round(us, 3),
         "avg_launch_us_source": "HIP events around a graph of K launches of this step, / K"}
    if counters and step in counters:
        e["traffic"] = counters[step]["hbm_bytes_per_launch"]
        e["traffic_over_algorithmic"] = round(counters[step]["traffic_over_algorithmic"], 4)
        e["traffic_source"] = counters["_file"]
    ctx = f"{step} after {step}"
    if trace and ctx in trace.get("contexts", {}):
        tr = trace["contexts"][ctx]
        e["avg_launch_us_rocprof"] = round(tr["mean_ns"] * 1e-3, 3)
        e["frac_rocprof"] = round(alg_bytes / (tr["mean_ns"] * 1e-9) / 1e9 / PEAK_HBM_GBS, 4)
        e["rocprof_source"] = f"{trace['_file']} (context '{ctx}', {tr['dispatches']} dispatches)"
    if floors and str(alg_bytes) in floors["single"]:
        e["same_size_read_us"] = floors["single"][str(alg_bytes)]["us"]
        e["frac_of_same_size_read"] = round(floors["single"][str(alg_bytes)]["us"] / us, 4)
    return e


# Launch shapes the read-floor probe tries: one-pass grids and persistent grids of 1-8
# workgroups per CU (256 CUs), 1-16 chunks of 1 KiB per wavefront in flight.
FLOOR_SHAPES = ([(u, wpg, 0) for u in (1, 2, 4, 8) for wpg in (4, 8)] +
                [(u, wpg, 256 * m) for u in (2, 4, 8, 16) for wpg in (4, 8, 16) for m in (1, 2, 4, 8)
                 if wpg * m <= 32])


def read_floors(md, sizes, K=300, min_total=1 << 30):
    """The fastest a pure streaming read of each byte count takes in one launch, over the launch
    shapes in FLOOR_SHAPES (graph of K back-to-back launches over rotating buffers, so the 256 MB
    cache cannot serve them), and the fastest two dependent launches of sizes[1] then sizes[0]
    bytes (the layer's two steps), each with its own best shape. Microseconds per launch."""
    import numpy as np
    import torch

    big = max(sizes)
    R = max(2, -(-min_total // big))
    bufs = [torch.empty(big + 256, dtype=torch.uint8, device="cuda") for _ in range(R)]
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")

    def timed(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(K):
                fn(r)
        g.replay()
        torch.cuda.synchronize()
        res = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) * 1e3 / K)
        del g
        return float(np.median(res))

    single = {}
    for nb in sizes:
        best = None
        for (u, wpg, groups) in FLOOR_SHAPES:
            us = timed(lambda r: md.moed_bench_read_cfg(bufs[r % R], sink, nb, u, wpg, groups))
            if best is None or us < best["us"]:
                best = {"us": round(us, 3), "unroll": u, "waves_per_group": wpg, "groups": groups,
                        "gbs": round(nb / (us * 1e-6) / 1e9, 1)}
        best["frac_of_8TBps"] = round(best["gbs"] / PEAK_HBM_GBS, 4)
        single[str(nb)] = best
    a, b = single[str(sizes[1])], single[str(sizes[0])]
    pair = timed(lambda r: (md.moed_bench_read_cfg(bufs[r % R], sink, sizes[1], a["unroll"], a["waves_per_group"],
                                                   a["groups"]),
                            md.moed_bench_read_cfg(bufs[(r + 1) % R], sink, sizes[0], b["unroll"],
                                                   b["waves_per_group"], b["groups"])))
    del bufs
    torch.cuda.empty_cache()
    return {"single": single, "pair_us": round(pair, 3),
            "pair_bytes": [sizes[1], sizes[0]], "shapes_tried": len(FLOOR_SHAPES), "launches_per_graph": K}


# weight copies and steps per workload when every workload is timed: copies * touched bytes
# well above the 256 MB cache. The large batches take 8 and 4 copies although 2 would defeat the
# cache: the grouped gate/up's speed depends on where in DRAM a copy's gate and up tensors land
# (about 222 or 270 µs per batch32 copy), so the figure is a mean over several placements, as a
# model's layers would give.
CONFIG_PLAN = {"tiny_B1_E8_k2_H256_I128": (32, 1000), "wide_B1_E128_k8_H2048_I768": (32, 1000),
               "batch_B8_E128_k8_H2048_I768": (8, 500), "batch_B32_E128_k8_H4096_I1536": (8, 64),
               "skewed_B64_E256_k8_H7168_I2048": (4, 32)}


def profile_entry(L, name):
    """What the committed rocprofv3 summaries of this workload say (MXFP8 weights), while they
    were taken from the current kernel sources: the layer's span under the kernel tracer (median,
    p10, p90; start of gate/up to end of the down step), and per step the HBM bytes per launch
    against the algorithmic bytes, the L2 hit rate and the VALU / MFMA busy percentages."""
    if L.wformat != "mxfp8":
        return None
    files = LAYER_SOURCES if gate_up_kernel_name(L) != "moe_gate_up_grouped_wide_kernel" else GROUPED_SOURCES
    out = {}
    tr = load_profile("kernel_trace", name, files)
    if tr is not None:
        sp = tr["layer_spans"]["after the down step"]
        out["rocprof_layer_us"] = {"median": round(sp["median_ns"] / 1e3, 3), "p10": round(sp["p10_ns"] / 1e3, 3),
                                   "p90": round(sp["p90_ns"] / 1e3, 3), "layers": sp["layers"],
                                   "source": tr["_file"]}
    cn = load_profile("counters_layer", name, files)
    if cn is not None:
        for step in ("gate_up", "down"):
            c = cn[step]
            x = c.get("extra", {})
            out[f"hbm_{step}"] = {"bytes_per_launch": round(c["hbm_bytes_per_launch"]),
                                  "algorithmic_bytes": c["algorithmic_bytes_per_launch"],
                                  "over_algorithmic": round(c["traffic_over_algorithmic"], 4),
                                  "l2_hit_rate": round(x["L2_hit_rate"], 3) if "L2_hit_rate" in x else None,
                                  "valu_busy_pct": round(x["VALUBusy"], 1) if "VALUBusy" in x else None,
                                  "mfma_busy_pct": round(x["MfmaUtil"], 1) if "MfmaUtil" in x else None}
        out["hbm_source"] = cn["_file"]
    return out or None


def config_entry(md, synth, name, wformat, reuse=None, cpu=True, peak=None):
    """One workload: µs per layer (graph of K layers over rotating weight copies; each step alone),
    GB/s on unique routed-weight bytes and its fraction of 8 TB/s (and of the measured read peak,
    when given); accuracy against the float64 oracle on every token (float32 output: max|err|/rms,
    min cosine; bf16 output: max abs; the FP32-accumulate path with BF16 intermediates:
    max|err|/rms), computed outside the timed region; the oracle's own time for the layer on the
    host threads (and on one thread for the three smaller workloads); the committed profiles'
    figures for the workload (profile_entry)."""
    import torch

    R, K = CONFIG_PLAN[name]
    if reuse is not None:
        L, t = reuse
    else:
        L = synth.make_layer(name, device="cuda", wformat=wformat)
        t = measure_steps(md, L, R, K)
    gu_bytes, dn_bytes = kernel_bytes(L)
    us = t["ms_per_step"] * 1e3
    gbs = L.unique_weight_bytes / (us * 1e-6) / 1e9
    sh = L.shape
    e = {"workload": name, "B": sh.B, "E": sh.E, "k": sh.k, "H": sh.H, "I": sh.I,
         "unique_experts": L.unique_experts, "unique_weight_bytes": L.unique_weight_bytes,
         "us_per_layer": round(us, 3), "gbs": round(gbs, 1), "frac_of_8TBps": round(gbs / PEAK_HBM_GBS, 4),
         "us_gate_up": round(t["ms_gate_up"] * 1e3, 3), "us_down": round(t["ms_down"] * 1e3, 3),
         "kernels": {"gate_up": gate_up_kernel_name(L), "down": down_kernel_name(L)},
         "steps": t.get("steps", K), "weight_copies": R if reuse is None else None}
    if peak:
        e["frac_of_measured_read_peak"] = round(gbs / peak, 4)
    e["profile"] = profile_entry(L, name)
    e["accuracy"] = accuracy_entry(md, L, cpu_threads=oracle_threads(), one_thread=cpu and sh.B <= 8)
    return e


def measure_steps(md, L, R, K):
    """Graph-timed µs per layer and per step (gate/up alone, down alone), K launches each."""
    import numpy as np
    import torch

    sh = L.shape
    x, ids, w = md.layer_device_inputs(L)
    copies = weight_copies(L, R)
    out = torch.empty((sh.B, sh.H), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((sh.B, sh.k, sh.I), dtype=torch.float32, device="cuda")
    ws = torch.empty(md.moed_workspace_bytes(sh.B, sh.k, sh.H, sh.I), dtype=torch.uint8, device="cuda")
    y = torch.empty(sh.B * sh.k * sh.H, dtype=torch.float32, device="cuda")
    wf = L.wformat
    fns = {"per_step": lambda r: md.moe_decode(x, ids, w, *copies[r % R], out=out, workspace=ws, wformat=wf),
           "gate_up": lambda r: md.moe_decode_gate_up(x, ids, *copies[r % R][:4], a=a, wformat=wf),
           "down": lambda r: md.moe_decode_down(a, ids, w, *copies[r % R][4:], out=out, wformat=wf, partials=y)}
    res = {"steps": K}
    for key, fn in fns.items():
        for r in range(5):
            fn(r)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(K):
                fn(r)
        g.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / K)
        res["ms_" + key] = float(np.median(ts))
        del g
    del copies
    return res


def oracle_threads():
    """Host threads the oracle runs on: every CPU the process may use, capped by OMP_NUM_THREADS
    when it is set (the GPU machine gives a one-GPU job a share of the host's cores that way)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def accuracy_entry(md, L, cpu_threads, one_thread=False):
    """The HIP path against the float64 oracle on every token of the layer."""
    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    x, ids, w = md.layer_device_inputs(L)
    args = (x, ids, w, L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)
    f32 = md.moe_decode(*args, out_dtype=torch.float32, wformat=L.wformat)
    b16 = md.moe_decode(*args, out_dtype=torch.bfloat16, wformat=L.wformat)
    i16 = md.moe_decode(*args, out_dtype=torch.float32, inter_dtype=torch.bfloat16, wformat=L.wformat)
    torch.cuda.synchronize()
    sel = sorted({int(e) for e in L.ids.ravel()})
    remap = np.full(L.shape.E, -1, np.int64)
    remap[sel] = np.arange(len(sel))
    ids_c = np.ascontiguousarray(remap[L.ids].astype(np.int32))
    idx = torch.tensor(sel, device=L.wg_q.device)
    host = [t.index_select(0, idx).cpu() for t in (L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)]
    used = oracle.threads(cpu_threads)
    t0 = time.perf_counter()
    ref = oracle.moe_decode(np.ascontiguousarray(L.x), ids_c, np.ascontiguousarray(L.w), *host,
                            nthreads=cpu_threads, wformat=L.wformat)
    s_layer = time.perf_counter() - t0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    g = f32.double().cpu().numpy()
    d = g - ref
    cos = np.sum(g * ref, axis=1) / (np.linalg.norm(g, axis=1) * np.linalg.norm(ref, axis=1))
    gi = i16.double().cpu().numpy()
    gb = b16.double().cpu().numpy()
    e = {"tokens": int(L.shape.B), "f32_max_err_over_rms": float(np.abs(d).max() / rms),
         "f32_rms_err_over_rms": float(np.sqrt(np.mean(d ** 2)) / rms),
         "f32_min_cosine": float(cos.min()), "f32_max_abs": float(np.abs(d).max()),
         "bf16_out_max_abs": float(np.abs(gb - ref).max()),
         "bf16_inter_max_err_over_rms": float(np.abs(gi - ref).max() / rms),
         "bf16_inter_rms_err_over_rms": float(np.sqrt(np.mean((gi - ref) ** 2)) / rms),
         "gate_f32_max_err_over_rms": 2e-3, "passes_gate": bool(np.abs(d).max() <= 2e-3 * rms),
         "oracle_s_per_layer": round(s_layer, 5), "oracle_threads": used}
    if one_thread:
        t0 = time.perf_counter()
        oracle.moe_decode(np.ascontiguousarray(L.x), ids_c, np.ascontiguousarray(L.w), *host, nthreads=1,
                          wformat=L.wformat)
        e["oracle_s_per_layer_1thread"] = round(time.perf_counter() - t0, 5)
    return e


COPY_BYTES = 256 << 20      # known-size reference for counter calibration
COUNTER_LAUNCHES = 8


def weight_copies(L, R):
    """R copies of the layer's weight tensors at distinct HBM addresses (copy 0 = L's own)."""
    first = (L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)
    return [first] + [tuple(t.clone() for t in first) for _ in range(R - 1)]


def measure_layer(md, L, R, K, W):
    """Time K layers (HIP graph, R rotating weight copies); also the two kernels alone and
    an eager loop. Returns milliseconds."""
    import numpy as np
    import torch

    sh = L.shape
    x, ids, w = md.layer_device_inputs(L)
    copies = weight_copies(L, R)
    torch.cuda.synchronize()
    out = torch.empty((sh.B, sh.H), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((sh.B, sh.k, sh.I), dtype=torch.float32, device="cuda")
    ws = torch.empty(md.moed_workspace_bytes(sh.B, sh.k, sh.H, sh.I), dtype=torch.uint8, device="cuda")
    y = torch.empty(sh.B * sh.k * sh.H, dtype=torch.float32, device="cuda")   # down's per-slot partials

    wf = L.wformat

    def layer(r):
        md.moe_decode(x, ids, w, *copies[r % R], out=out, workspace=ws, wformat=wf)

    def gate_up(r):
        md.moe_decode_gate_up(x, ids, *copies[r % R][:4], a=a, wformat=wf)

    def down(r):
        md.moe_decode_down(a, ids, w, *copies[r % R][4:], out=out, wformat=wf, partials=y)

    for r in range(W):                       # untimed warm-up steps
        layer(r)
    torch.cuda.synchronize()

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(n):
                fn(r)
        torch.cuda.synchronize()
        return g

    def time_graph(g, n, reps=1):
        res = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) / n)
        return float(np.median(res))

    g_layer = capture(layer, K)
    g_layer.replay()                         # untimed: first replay uploads the graph
    torch.cuda.synchronize()

    # ---- the timed region: exactly K steps ----
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    g_layer.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = ev0.elapsed_time(ev1) / K
    # -------------------------------------------

    g_gu = capture(gate_up, K)
    g_dn = capture(down, K)
    g_gu.replay(); g_dn.replay()
    torch.cuda.synchronize()
    res = {"ms_per_step": ms_per_step, "wall_s": wall,
           "ms_gate_up": time_graph(g_gu, K, reps=3), "ms_down": time_graph(g_dn, K, reps=3),
           "ms_layer_median3": time_graph(g_layer, K, reps=3)}
    del g_layer, g_gu, g_dn
    e0 = torch.cuda.Event(enable_timing=True); e1 = torch.cuda.Event(enable_timing=True)
    n_eager = min(K, 200)
    torch.cuda.synchronize(); e0.record()
    for r in range(n_eager):
        layer(r)
    e1.record(); torch.cuda.synchronize()
    res["ms_eager"] = e0.elapsed_time(e1) / n_eager

    # router front-end: route alone, and route + layer (ids and weights made on the GPU
    # from float32 logits every step), graph-timed like the layer
    logits = torch.from_numpy(synth_router_logits(L)).cuda()
    rid = torch.empty_like(ids)
    rw = torch.empty_like(w)

    def route(r):
        md.moe_route(logits, sh.k, ids=rid, w=rw)

    def routed_layer(r):
        md.moe_route(logits, sh.k, ids=rid, w=rw)
        md.moe_decode(x, rid, rw, *copies[r % R], out=out, workspace=ws, wformat=wf)

    g_rt = capture(route, K)
    g_rl = capture(routed_layer, K)
    g_rt.replay(); g_rl.replay()
    torch.cuda.synchronize()
    res["ms_route"] = time_graph(g_rt, K, reps=3)
    res["ms_routed_layer"] = time_graph(g_rl, K, reps=3)
    del g_rt, g_rl
    return res


def synth_router_logits(L):
    """float32 router logits [B, E] of the layer's workload (same recipe as its routing)."""
    from output_centric_expert_amd import synth
    sh = L.shape
    return synth.make_router_logits(sh.B, sh.E, L.seed, sh.zipf_s).astype("float32")


WEIGHT_DESC = {"mxfp8": "mxfp8 (e4m3 + ue8m0 per 32)", "mxfp4": "mxfp4 (e2m1 two per byte + ue8m0 per 32)"}


def gate_up_kernel_name(L):
    """The gate/up kernel the library's built-in launch table picks for this layer: the
    expert-grouped one once 4*B*k >= 3*E or (H >= 6144 and min(B*k, E)*ceil(I/64) >= 512) --
    the wide form when H is a multiple of 512 -- else the per-slot exact-fit kernel when a row
    is exactly 64*U 16-byte chunks (U <= 8), else the generic per-slot kernel."""
    sh = L.shape
    slots = sh.B * sh.k
    if 4 * slots >= 3 * sh.E or (sh.H >= 6144 and min(slots, sh.E) * -(-sh.I // 64) >= 512):
        return "moe_gate_up_grouped_wide_kernel" if sh.H % 512 == 0 else "moe_gate_up_grouped_kernel"
    nch = sh.H // 32 if L.wformat == "mxfp4" else sh.H // 16
    return "moe_gate_up_exact_kernel" if nch % 64 == 0 and nch // 64 <= 8 else "moe_gate_up_kernel"


def kernel_bytes(L):
    """Algorithmic weight bytes per launch (unique routed experts' codes + scales): gate/up, down."""
    sh = L.shape
    U = L.unique_experts
    per_matrix = sh.I * sh.H * (17 if L.wformat == "mxfp4" else 33) // 32
    return U * 2 * per_matrix, U * per_matrix


def timing_fields(L, t):
    gu_bytes, dn_bytes = kernel_bytes(L)
    return {"us_per_layer": round(t["ms_per_step"] * 1e3, 3),
            "frac_of_peak_hbm": round(L.unique_weight_bytes / (t["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "us_gate_up": round(t["ms_gate_up"] * 1e3, 3), "us_down": round(t["ms_down"] * 1e3, 3),
            "gbs_gate_up": round(gu_bytes / (t["ms_gate_up"] * 1e-3) / 1e9, 1),
            "gbs_down": round(dn_bytes / (t["ms_down"] * 1e-3) / 1e9, 1),
            "us_per_layer_median3": round(t["ms_layer_median3"] * 1e3, 3),
            "us_per_layer_eager": round(t["ms_eager"] * 1e3, 3),
            "us_route": round(t["ms_route"] * 1e3, 3),
            "us_per_layer_with_router": round(t["ms_routed_layer"] * 1e3, 3),
            "wall_s_timed": round(t["wall_s"], 4)}


# weight copies and steps per workload for --all: copies * touched bytes >> 256 MB cache
ALL_PLAN = {"tiny_B1_E8_k2_H256_I128": (32, 2000), "wide_B1_E128_k8_H2048_I768": (32, 2000),
            "batch_B8_E128_k8_H2048_I768": (8, 1000), "batch_B32_E128_k8_H4096_I1536": (8, 96),
            "skewed_B64_E256_k8_H7168_I2048": (4, 40)}


def all_workloads(md, synth, args):
    import torch
    peak = measured_read_peak(md)
    for name in synth.WORKLOAD_ORDER:
        R, K = ALL_PLAN[name]
        L = synth.make_layer(name, device="cuda", wformat=args.wformat)
        t = measure_layer(md, L, R, K, min(args.warmup, 10))
        gbs = L.unique_weight_bytes / (t["ms_per_step"] * 1e-3) / 1e9
        line = {"workload": name, "wformat": L.wformat, "steps": K, "weight_copies": R,
                "unique_experts": L.unique_experts,
                "unique_weight_bytes": L.unique_weight_bytes, "gbs": round(gbs, 1),
                **timing_fields(L, t), "frac_of_measured_read_peak": round(gbs / peak, 4),
                "measured_read_peak_gbs": round(peak, 1)}
        if L.unique_weight_bytes < (1 << 30):
            line["same_size_reads_us"] = same_size_reads(md, *kernel_bytes(L), K=min(K, 2000))
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_baseline(L, L.unique_weight_bytes, min(args.cpu_seconds, 10.0))
        print(json.dumps(line), flush=True)
        del L
        torch.cuda.empty_cache()


def diagnostics(md, synth, args):
    """Labelled measurements beside the metric (none of them is the default line):
    - the single-token layer with its 8 experts at adjacent ids 0..7 against the recipe's
      scattered ids (same weights, same bytes);
    - every workload with one weight copy, so the L2 and the 256 MB MALL keep what fits
      (the metric's runs cycle through copies so that they cannot);
    - the skewed workload with its hot experts at adjacent ids (Zipf ranks r_e = e + 1)."""
    import dataclasses
    import numpy as np
    import torch

    def emit(label, L, R, K):
        t = measure_layer(md, L, R, K, min(args.warmup, 10))
        gbs = L.unique_weight_bytes / (t["ms_per_step"] * 1e-3) / 1e9
        print(json.dumps({"diagnostic": label, "workload": L.shape.name, "wformat": L.wformat,
                          "weight_copies": R, "steps": K, "unique_experts": L.unique_experts,
                          "gbs": round(gbs, 1), **timing_fields(L, t)}), flush=True)

    name = "wide_B1_E128_k8_H2048_I768"
    R, K = ALL_PLAN[name]
    L = synth.make_layer(name, device="cuda", wformat=args.wformat)
    emit("scattered expert ids (the recipe)", L, R, K)
    adj = dataclasses.replace(L, ids=np.arange(L.shape.k, dtype=np.int32)[None, :].repeat(L.shape.B, 0))
    emit("adjacent expert ids 0..k-1", adj, R, K)
    del L, adj
    torch.cuda.empty_cache()
    for name in synth.WORKLOAD_ORDER:
        _, K = ALL_PLAN[name]
        L = synth.make_layer(name, device="cuda", wformat=args.wformat)
        emit("warm cache (one weight copy)", L, 1, K)
        del L
        torch.cuda.empty_cache()
    name = "skewed_B64_E256_k8_H7168_I2048"
    R, K = ALL_PLAN[name]
    L = synth.make_layer(name, device="cuda", wformat=args.wformat, contiguous_hot=True)
    emit("hot experts at adjacent ids", L, R, K)


def counters_run(md, x, ids, w, copies, out, a, workload, wformat="mxfp8"):
    """Launch plan for rocprofv3 --pmc: COUNTER_LAUNCHES copies of COPY_BYTES, then the
    gate/up and down kernels COUNTER_LAUNCHES times each on rotating weight copies."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(COUNTER_LAUNCHES):
        md.moed_bench_copy(src, dst)
        torch.cuda.synchronize()
    R = len(copies)
    y = torch.empty(a.shape[0] * a.shape[1] * out.shape[1], dtype=torch.float32, device="cuda")
    for r in range(COUNTER_LAUNCHES):
        md.moe_decode_gate_up(x, ids, *copies[(r + 1) % R][:4], a=a, wformat=wformat)
        torch.cuda.synchronize()
    for r in range(COUNTER_LAUNCHES):
        md.moe_decode_down(a, ids, w, *copies[(r + 1) % R][4:], out=out, wformat=wformat, partials=y)
        torch.cuda.synchronize()
    print(json.dumps({"counters_plan": {"workload": workload, "copy_bytes": COPY_BYTES,
                                        "launches_each": COUNTER_LAUNCHES,
                                        "source_digest_layer": source_digest(LAYER_SOURCES),
                                        "source_digest_grouped": source_digest(GROUPED_SOURCES)}}), flush=True)


def measured_read_peak(md, nbytes=2 << 30, launches=20):
    """Contiguous streaming-read bandwidth (GB/s) over two alternating 2 GiB buffers."""
    import torch
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    md.moed_bench_read(bufs[0], sink)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(launches):
        md.moed_bench_read(bufs[i % 2], sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    del bufs
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def same_size_reads(md, gu_bytes, dn_bytes, K=2000, min_total=1 << 30):
    """What a pure streaming read of the same byte counts takes with the same launch mechanism
    (a HIP graph of K back-to-back launches over rotating buffers, so the 256 MB cache cannot
    serve them): µs per launch for the gate/up bytes alone, the down bytes alone, and the two as
    a dependent pair (the layer's shape)."""
    import numpy as np
    import torch

    R = max(2, -(-min_total // (gu_bytes + dn_bytes)))
    bufs = [(torch.empty(gu_bytes, dtype=torch.uint8, device="cuda"),
             torch.empty(dn_bytes, dtype=torch.uint8, device="cuda")) for _ in range(R)]
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def timed(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(K):
                fn(r)
        g.replay()
        torch.cuda.synchronize()
        res = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) * 1e3 / K)
        del g
        return float(np.median(res))

    out = {"gate_up_bytes_us": timed(lambda r: md.moed_bench_read(bufs[r % R][0], sink)),
           "down_bytes_us": timed(lambda r: md.moed_bench_read(bufs[r % R][1], sink)),
           "pair_us": timed(lambda r: (md.moed_bench_read(bufs[r % R][0], sink),
                                       md.moed_bench_read(bufs[r % R][1], sink)))}
    del bufs
    torch.cuda.empty_cache()
    return {k: round(v, 3) for k, v in out.items()}


def cpu_baseline(L, uniq, seconds):
    """The float64 oracle, as it stands, on full layers of the same workload: on the host threads
    the process may use (oracle_threads), and on one thread."""
    import numpy as np
    import torch

    import oracle

    oracle.build(force=False)
    B = L.shape.B
    toks = list(range(B)) if B <= 8 else list(range(0, B, B // 4))[:4]   # bounded sample
    ids_t = L.ids[toks]
    sel = sorted(set(int(e) for e in ids_t.ravel()))
    remap = {e: n for n, e in enumerate(sel)}
    ids_c = np.ascontiguousarray(np.vectorize(remap.get)(ids_t).astype(np.int32))
    x_t = np.ascontiguousarray(L.x[toks])
    w_t = np.ascontiguousarray(L.w[toks])
    idx = torch.tensor(sel, device=L.wg_q.device)
    host = [t.index_select(0, idx).cpu() for t in (L.wg_q, L.wg_s, L.wu_q, L.wu_s, L.wd_q, L.wd_s)]

    def run(nthreads, budget):
        oracle.moe_decode(x_t, ids_c, w_t, *host, nthreads=nthreads, wformat=L.wformat)     # warm-up
        n, t = 0, 0.0
        while t < budget or n < 3:
            t0 = time.perf_counter()
            oracle.moe_decode(x_t, ids_c, w_t, *host, nthreads=nthreads, wformat=L.wformat)
            t += time.perf_counter() - t0
            n += 1
        return n, t / n / len(toks) * B          # the oracle's cost is linear in tokens

    nthreads = oracle_threads()
    used = oracle.threads(nthreads)
    n, per = run(nthreads, seconds)
    n1, per1 = run(1, min(seconds, 5.0))
    what = "full layers" if len(toks) == B else f"runs of {len(toks)} of the {B} tokens (cost per layer scaled by B/{len(toks)})"
    return {"value": round(uniq / per / 1e9, 3), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{n} {what} of the same workload (touched experts copied to host)",
            "s_per_layer": round(per, 6),
            "value_1thread": round(uniq / per1 / 1e9, 4), "s_per_layer_1thread": round(per1, 6),
            "runs_1thread": n1, "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "threads_note": "threads = the CPUs this process may use, capped by OMP_NUM_THREADS "
                            "(the GPU box gives a one-GPU job 16)"}


if __name__ == "__main__":
    main()
