"""Per-context kernel durations from a rocprofv3 --kernel-trace CSV of bench.py.

The benchmark launches the layer kernels in several contexts: the timed graph
of K layers (gate/up after down), the graphs of one kernel repeated K times
(gate/up after gate/up, down after down), the routed-layer graph (gate/up
after the router kernel) and an eager loop. The kernel-trace summary averages
over all of them; the benchmark's roofline figure is the launch period in the
one-kernel graph. This splits each layer kernel's dispatches by the layer
kernel that ran just before it, so the trace can be compared context by
context.

    python -m output_centric_expert_amd.trace_contexts gpurun_out/prof_ktrace/bench_kernel_trace.csv
"""
from __future__ import annotations

import collections
import csv
import json
import statistics
import sys

KINDS = (("moe_gate_up_grouped_kernel", "gate_up_grouped"), ("moe_gate_up_kernel", "gate_up"),
         ("moe_down_rows_kernel", "down"), ("moe_down_staged_kernel", "down"), ("moe_down_kernel", "down"),
         ("moe_down_grouped_kernel", "down"), ("moe_route_kernel", "route"))


def kind(name: str):
    for needle, k in KINDS:
        if needle in name:
            return k
    return None


def contexts(path: str) -> dict:
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            k = kind(r["Kernel_Name"])
            if k is not None:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), k))
    rows.sort()
    per = collections.defaultdict(list)
    prev = None
    for start, end, k in rows:
        per[f"{k} after {prev}"].append(end - start)
        prev = k
    return {ctx: {"dispatches": len(v), "mean_ns": round(statistics.fmean(v), 1),
                  "median_ns": round(statistics.median(v), 1)} for ctx, v in sorted(per.items())}


if __name__ == "__main__":
    print(json.dumps(contexts(sys.argv[1]), indent=1))
