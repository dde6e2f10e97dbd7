"""Turn rocprofv3 --pmc CSV output (FETCH_SIZE pass, WRITE_SIZE pass) of
``bench.py --counters`` into the per-launch HBM-traffic summary the benchmark
reports as roofline.traffic.

The raw counters are scaled by what the same counters read for a copy kernel
of known size (COPY_BYTES read + COPY_BYTES written), launched in the same run.
With --extra DIR, a third pass (any counters, e.g. TCC_HIT_sum TCC_MISS_sum
VALUBusy MfmaUtil) is reported per step as the mean per call, with the L2 hit
rate TCC_HIT / (TCC_HIT + TCC_MISS) when both are there.

    python -m output_centric_expert_amd.counters --fetch DIR --write DIR \\
        --workload NAME --digest HEX --out profiles/counters_layer_NAME.json
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os


def read_counter(d: str, name: str):
    """{kernel-name-prefix: [value per dispatch]} for counter `name` (KiB)."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {d}")
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != name:
                    continue
                per[row["Kernel_Name"]][row.get("Dispatch_Id") or row.get("Correlation_Id")] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def counter_names(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    names = set()
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                names.add(row.get("Counter_Name"))
    return sorted(n for n in names if n)


def pick(per: dict, needle: str):
    vals = [v for k, vs in per.items() if needle in k for v in vs]
    if not vals:
        raise KeyError(f"no dispatch of a kernel matching {needle!r}")
    return sum(vals) / len(vals), len(vals)


# The kernels one call of each layer step launches: the per-slot gate/up (generic or exact-fit) or
# the expert-grouped one (128-byte tile slices or wide loads); the per-output down (staged,
# one-pass, several rows per wave, or direct), or the expert-major down plus its combine.
STEP_KERNELS = {"gate_up": ("moe_gate_up_kernel", "moe_gate_up_exact_kernel", "moe_gate_up_exact_pair_kernel",
                            "moe_gate_up_grouped_kernel", "moe_gate_up_grouped_wide_kernel"),
                "down": ("moe_down_kernel", "moe_down_staged_kernel", "moe_down_onepass_kernel", "moe_down_blocks_kernel",
                         "moe_down_rows_kernel", "moe_down_expert_kernel", "moe_down_combine_kernel")}


def step_counter(per: dict, step: str):
    """Per-call value of one layer step: the mean per dispatch of each of its kernels that ran,
    summed over those kernels. Also returns {kernel: (mean, dispatches)}."""
    parts = {}
    for needle in STEP_KERNELS[step]:
        names = [k for k in per if f"{needle}<" in k or f"{needle}(" in k]
        if names:
            vals = [v for k in names for v in per[k]]
            parts[needle] = (sum(vals) / len(vals), len(vals))
    if not parts:
        raise KeyError(f"no dispatch of a {step} kernel")
    return sum(m for m, _ in parts.values()), parts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--digest", required=True)
    ap.add_argument("--copy-bytes", type=int, default=256 << 20)
    ap.add_argument("--out", required=True)
    ap.add_argument("--gate-up-bytes", type=int, required=True, help="algorithmic bytes per gate/up launch")
    ap.add_argument("--down-bytes", type=int, required=True, help="algorithmic bytes per down launch")
    ap.add_argument("--command", default=None, help="the commands the counter runs came from")
    ap.add_argument("--extra", default=None, help="directory of a third --pmc pass (any counters)")
    args = ap.parse_args()

    fetch = read_counter(args.fetch, "FETCH_SIZE")
    write = read_counter(args.write, "WRITE_SIZE")
    cf, _ = pick(fetch, "moe_bench_copy_kernel")
    cw, _ = pick(write, "moe_bench_copy_kernel")
    f_fetch = args.copy_bytes / (cf * 1024.0)
    f_write = args.copy_bytes / (cw * 1024.0)
    res = {"workload": args.workload, "source_digest": args.digest, "command": args.command,
           "copy_kernel": {"bytes_read": args.copy_bytes, "bytes_written": args.copy_bytes,
                           "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw,
                           "fetch_scale": f_fetch, "write_scale": f_write}}
    for key, alg in (("gate_up", args.gate_up_bytes), ("down", args.down_bytes)):
        fv, fparts = step_counter(fetch, key)
        wv, _ = step_counter(write, key)
        hbm = fv * 1024.0 * f_fetch + wv * 1024.0 * f_write
        res[key] = {"kernels": {k: {"dispatches": n, "FETCH_SIZE_KiB": m} for k, (m, n) in fparts.items()},
                    "FETCH_SIZE_KiB": fv, "WRITE_SIZE_KiB": wv,
                    "hbm_bytes_per_launch": hbm, "algorithmic_bytes_per_launch": alg,
                    "traffic_over_algorithmic": hbm / alg}
    if args.extra:
        for name in counter_names(args.extra):
            per = read_counter(args.extra, name)
            for key in ("gate_up", "down"):
                try:
                    v, parts = step_counter(per, key)
                except KeyError:
                    continue
                res[key].setdefault("extra", {})[name] = v
                res[key].setdefault("extra_per_kernel", {})[name] = {k: m for k, (m, _) in parts.items()}
        for key in ("gate_up", "down"):
            ex = res[key].get("extra", {})
            if "TCC_HIT_sum" in ex and "TCC_MISS_sum" in ex and ex["TCC_HIT_sum"] + ex["TCC_MISS_sum"] > 0:
                ex["L2_hit_rate"] = ex["TCC_HIT_sum"] / (ex["TCC_HIT_sum"] + ex["TCC_MISS_sum"])
    res["hbm_bytes_per_launch"] = res["gate_up"]["hbm_bytes_per_launch"]
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
