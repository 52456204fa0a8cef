"""HBM traffic per kernel launch from rocprofv3 counter runs.

    python -m mixture_experts_router_amd.traffic --workload decode_b1 \
        --fetch <dir of the FETCH_SIZE run> --write <dir of the WRITE_SIZE run> \
        --copy-bytes <bytes the copy kernel reads (= writes) per launch>

FETCH_SIZE and WRITE_SIZE are rocprofv3's derived counters of kilobytes read
from and written to device memory per dispatch.  Each is calibrated against a
plain elementwise copy of known size profiled in the same run (bench.py
--copy-probe-mib): factor = known bytes / (counter KiB * 1024).  The scaled
per-launch means are written to profiles/traffic.json under the workload and
the kernel's plan name, with the hash of the kernel sources they were taken
on, and a short text summary is printed.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
from collections import defaultdict

from . import source_hash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# kernel symbol -> the plan name the library reports for that launch
KERNEL_PLAN = [
    (re.compile(r"router_logits_(small|mfma)_kernel"), "router_logits"),
    (re.compile(r"gemv_up_kernel<\d+, \d+, true>"), "gemv_gate_up_swiglu"),
    (re.compile(r"gemv_down_kernel"), "gemv_down_combine"),
    (re.compile(r"gemm_kernel<\d+, 0,"), "gemm_gate_up_swiglu"),
    (re.compile(r"gemm_kernel<\d+, 2,"), "gemm_down"),
    (re.compile(r"sort_pairs_kernel"), "sort_pairs"),
    (re.compile(r"sort_prep_kernel"), "sort_pairs_prep_a"),
    (re.compile(r"combine_kernel"), "combine"),
]
COPY_KERNEL = re.compile(r"neg")  # torch.neg over fp16: one read and one write per element


def read_counter(run_dir: str, counter: str):
    """{kernel name: [per-dispatch values]} of one counter from a rocprofv3 run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no *counter_collection.csv under %s" % run_dir)
    per = defaultdict(dict)  # kernel -> dispatch -> value
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                key = (f, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                per[row["Kernel_Name"]][key] = per[row["Kernel_Name"]].get(key, 0.0) + float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def plan_name(kernel: str):
    for rx, name in KERNEL_PLAN:
        if rx.search(kernel):
            return name
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-bytes", type=float, required=True)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    args = ap.parse_args()

    fetch = read_counter(args.fetch, "FETCH_SIZE")
    write = read_counter(args.write, "WRITE_SIZE")

    def copy_mean(d):
        vals = [v for k, vs in d.items() if COPY_KERNEL.search(k) for v in vs]
        if not vals:
            raise SystemExit("copy kernel not found among: %s" % ", ".join(sorted(d)))
        return sum(vals) / len(vals)

    f_factor = args.copy_bytes / (copy_mean(fetch) * 1024.0)
    w_factor = args.copy_bytes / (copy_mean(write) * 1024.0)
    print("copy kernel: %.0f bytes read and written per launch; FETCH_SIZE factor %.4f, WRITE_SIZE factor %.4f"
          % (args.copy_bytes, f_factor, w_factor))

    agg = defaultdict(lambda: {"fetch": [], "write": []})
    for k, vs in fetch.items():
        n = plan_name(k)
        if n:
            agg[n]["fetch"] += vs
    for k, vs in write.items():
        n = plan_name(k)
        if n:
            agg[n]["write"] += vs

    data = {}
    if os.path.exists(args.out):
        data = json.load(open(args.out))
    entry = data.setdefault(args.workload, {})
    sh = source_hash()
    print("%-22s %10s %14s %14s %14s" % ("kernel", "dispatches", "fetch B", "write B", "total B"))
    for name, d in sorted(agg.items()):
        if not d["fetch"] or not d["write"]:
            continue
        fb = sum(d["fetch"]) / len(d["fetch"]) * 1024.0 * f_factor
        wb = sum(d["write"]) / len(d["write"]) * 1024.0 * w_factor
        entry[name] = {"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                       "fetch_factor": round(f_factor, 5), "write_factor": round(w_factor, 5),
                       "dispatches": len(d["fetch"]), "source_hash": sh}
        print("%-22s %10d %14.0f %14.0f %14.0f" % (name, len(d["fetch"]), fb, wb, fb + wb))
    os.makedirs(os.path.dirname(args.out), exist_ok=True)
    with open(args.out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")


if __name__ == "__main__":
    main()
