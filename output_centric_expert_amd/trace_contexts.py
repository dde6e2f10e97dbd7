"""Per-context kernel durations from a rocprofv3 --kernel-trace CSV of bench.py.

The benchmark launches the layer kernels in several contexts: the timed graph
of K layers (gate/up after down), the graphs of one kernel repeated K times
(gate/up after gate/up, down after down), the routed-layer graph (gate/up
after the router kernel) and an eager loop. The kernel-trace summary averages
over all of them; the benchmark's roofline figure is the launch period in the
one-kernel graph. This splits each layer kernel's dispatches by the layer
kernel that ran just before it, so the trace can be compared context by
context.

It also measures layers the way a trace sees them: for every gate/up dispatch
followed directly by the down step (the down kernel, plus the combine kernel
of the expert-major form), the span from the start of the gate/up to the end
of the down step, reported as median, p10 and p90 per preceding kernel (the
layer graph: after the down step; the routed layer: after the router).

With --workload, --digest and --out it writes the summary as the JSON the
benchmark reads (profiles/kernel_trace_<workload>.json: its roofline entries
take the mean of the "gate_up after gate_up" and "down after down" contexts,
the one-step graphs they time), with the rocprofv3 --stats rows of the run.

    python -m output_centric_expert_amd.trace_contexts <out>/prof_ktrace/bench_kernel_trace.csv \
        [--stats <out>/prof_ktrace/bench_kernel_stats.csv --workload NAME --digest HEX --command CMD --out FILE]
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import statistics

KINDS = (("moe_gate_up_grouped_wide_kernel", "gate_up"), ("moe_gate_up_grouped_kernel", "gate_up"),
         ("moe_gate_up_exact_pair_kernel", "gate_up"), ("moe_gate_up_exact_kernel", "gate_up"),
         ("moe_gate_up_kernel", "gate_up"),
         ("moe_down_rows_kernel", "down"), ("moe_down_staged_kernel", "down"), ("moe_down_onepass_kernel", "down"),
         ("moe_down_blocks_kernel", "down"),
         ("moe_down_kernel", "down"),
         ("moe_down_expert_kernel", "down"), ("moe_down_combine_kernel", "combine"),
         ("moe_route_kernel", "route"))


def kind(name: str):
    for needle, k in KINDS:
        if needle in name:
            return k
    return None


def read_rows(path: str):
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            k = kind(r["Kernel_Name"])
            if k is not None:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), k))
    rows.sort()
    return rows


def percentile(v, q):
    v = sorted(v)
    x = q * (len(v) - 1)
    lo = int(x)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (x - lo)


def layer_spans(rows) -> dict:
    spans = collections.defaultdict(list)
    for n, (start, _, k) in enumerate(rows):
        if k != "gate_up" or n + 1 >= len(rows) or rows[n + 1][2] != "down":
            continue
        end = rows[n + 1][1]
        if n + 2 < len(rows) and rows[n + 2][2] == "combine":
            end = rows[n + 2][1]
        prev = rows[n - 1][2] if n > 0 else None
        spans["after " + ("the down step" if prev in ("down", "combine") else str(prev))].append(end - start)
    return {ctx: {"layers": len(v), "median_ns": round(statistics.median(v), 1),
                  "p10_ns": round(percentile(v, 0.1), 1), "p90_ns": round(percentile(v, 0.9), 1)}
            for ctx, v in sorted(spans.items())}


def contexts(path: str) -> dict:
    rows = read_rows(path)
    per = collections.defaultdict(list)
    prev = None
    for start, end, k in rows:
        per[f"{k} after {prev}"].append(end - start)
        prev = k
    return {ctx: {"dispatches": len(v), "mean_ns": round(statistics.fmean(v), 1),
                  "median_ns": round(statistics.median(v), 1)} for ctx, v in sorted(per.items())}


def stats_rows(path: str) -> list:
    """The rocprofv3 --stats rows (kernel name, calls, average / min / max ns) of the layer kernels."""
    out = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if kind(r["Name"]) is None:
                continue
            out.append({"kernel": r["Name"], "calls": int(r["Calls"]), "average_ns": float(r["AverageNs"]),
                        "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--stats")
    ap.add_argument("--workload")
    ap.add_argument("--digest")
    ap.add_argument("--command")
    ap.add_argument("--out")
    args = ap.parse_args()
    rows = read_rows(args.trace)
    res = {"workload": args.workload, "source_digest": args.digest, "command": args.command,
           "contexts": contexts(args.trace), "layer_spans": layer_spans(rows)}
    if args.stats:
        res["stats"] = stats_rows(args.stats)
    text = json.dumps(res, indent=1)
    if args.out:
        with open(args.out, "w") as fh:
            fh.write(text + "\n")
    print(text)


if __name__ == "__main__":
    main()
