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


# The sources the per-slot gate/up kernel (the dominant kernel of the single-token layer) is
# compiled from, with its launch-shape defaults. Its committed HBM counters stay valid while the
# code in these files (comments and blank lines removed) is unchanged.
GATE_UP_SOURCES = ("gate_up.hip", "gate_up_body.h", "launch.h", "mx_device.h")


def _code_only(src: str) -> str:
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.strip() for line in src.splitlines() if line.strip())


# ... and those of the expert-grouped gate/up and the expert-major down (the large-batch kernels).
GROUPED_SOURCES = ("gate_up_grouped.hip", "down_grouped.hip", "grouped_common.h", "launch.h", "mx_device.h")


def source_digest(files=GATE_UP_SOURCES) -> str:
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "output_centric_expert_amd", "csrc", name)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this source."""
    p = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_digest") != source_digest():
        return None
    return d.get("hbm_bytes_per_launch")


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
    t = measure_layer(md, L, R, K, W)
    peak = measured_read_peak(md)
    B, E, k, H, I = shape.B, shape.E, shape.k, shape.H, shape.I
    U = L.unique_experts
    uniq = L.unique_weight_bytes
    gu_bytes, _ = kernel_bytes(L)
    ms_per_step, ms_gu = t["ms_per_step"], t["ms_gate_up"]
    gbs = uniq / (ms_per_step * 1e-3) / 1e9
    gu_gbs = gu_bytes / (ms_gu * 1e-3) / 1e9

    traffic = load_traffic("gate_up", args.workload) if L.wformat == "mxfp8" else None
    _, dn_bytes = kernel_bytes(L)
    floor = same_size_reads(md, gu_bytes, dn_bytes, K=min(K, 2000)) if L.unique_weight_bytes < (1 << 30) else None
    roofline = {"bound": "hbm", "kernel": gate_up_kernel_name(L), "achieved": round(gu_gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gu_gbs / PEAK_HBM_GBS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": gu_bytes,
                "avg_launch_us": round(ms_gu * 1e3, 3)}
    if floor:
        roofline["same_size_read_us"] = floor["gate_up_bytes_us"]
        roofline["frac_of_same_size_read"] = round(floor["gate_up_bytes_us"] / (ms_gu * 1e3), 4)

    cpu = None
    if not args.no_cpu:
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
        "same_size_reads_us": floor,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "tuning": args.tune or "built-in",
    }
    print(json.dumps(res), flush=True)


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
    expert-grouped one once B*k*H >= 2458*E, else the per-slot exact-fit kernel when a row is
    exactly 64*U 16-byte chunks (U <= 8), else the generic per-slot kernel."""
    sh = L.shape
    if sh.B * sh.k * sh.H >= 2458 * sh.E:
        return "moe_gate_up_grouped_wide_kernel"
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
            "batch_B8_E128_k8_H2048_I768": (8, 1000), "batch_B32_E128_k8_H4096_I1536": (2, 100),
            "skewed_B64_E256_k8_H7168_I2048": (2, 40)}


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
                                        "source_digest": source_digest()}}), flush=True)


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
    """The float64 oracle, as it stands, on full layers of the same workload (host cores)."""
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
    nthreads = min(os.cpu_count() or 1, 16)
    used = oracle.threads(nthreads)
    oracle.moe_decode(x_t, ids_c, w_t, *host, nthreads=nthreads, wformat=L.wformat)     # warm-up
    n, t = 0, 0.0
    while t < seconds or n < 3:
        t0 = time.perf_counter()
        oracle.moe_decode(x_t, ids_c, w_t, *host, nthreads=nthreads, wformat=L.wformat)
        t += time.perf_counter() - t0
        n += 1
    per_tok = t / n / len(toks)
    per = per_tok * B                       # the oracle's cost is linear in tokens
    what = "full layers" if len(toks) == B else f"runs of {len(toks)} of the {B} tokens (cost per layer scaled by B/{len(toks)})"
    return {"value": round(uniq / per / 1e9, 3), "unit": "GB/s", "cores": used, "kind": "oracle",
            "sample": f"{n} {what} of the same workload (touched experts copied to host)",
            "s_per_layer": round(per, 6)}


if __name__ == "__main__":
    main()
