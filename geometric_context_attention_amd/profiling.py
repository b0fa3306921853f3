"""Helpers for the rocprofv3 evidence of the GCA kernels.

* ``kernel_source_digest()``: sha256 of the kernel source, recorded with every
  stored counter measurement so that a figure taken on an older kernel is not
  reported for a newer one.
* ``summarize_kernel_stats(csv)``: the per-kernel table of a
  ``rocprofv3 --kernel-trace --stats --output-format csv`` run.
* ``summarize_pmc(csv, kernel)``: totals and per-dispatch means of the counters
  of a ``rocprofv3 --pmc ... --output-format csv`` run for one kernel.

Command line (run on the GPU host after the profiler):
    python -m geometric_context_attention_amd.profiling stats <kernel_stats.csv>
    python -m geometric_context_attention_amd.profiling pmc <counter_collection.csv> <kernel-substring>
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(PKG, "csrc", "gca_kernels.hip")
TRAFFIC_FILE = os.path.join(os.path.dirname(PKG), "profiles", "k_attn_bf16_gca_stream_traffic.txt")


def kernel_source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def summarize_kernel_stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["kernel | calls | total ms | avg us | min us | max us | share %"]
    for r in rows:
        name = r["Name"].strip('"')
        short = name if len(name) < 70 else name[:67] + "..."
        out.append(f"{short} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                   f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                   f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}")
    return "\n".join(out)


def summarize_pmc(path: str, kernel: str) -> dict:
    acc = collections.defaultdict(float)
    cnt = collections.Counter()
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if kernel not in r["Kernel_Name"]:
                continue
            acc[r["Counter_Name"]] += float(r["Counter_Value"])
            cnt[r["Counter_Name"]] += 1
    return {k: {"total": acc[k], "dispatches": cnt[k], "per_dispatch": acc[k] / max(cnt[k], 1)}
            for k in sorted(acc)}


def read_traffic(path: str = TRAFFIC_FILE):
    """Calibrated HBM bytes per attention launch from the stored counter
    summary, or None if absent or taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_digest():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    b = sub.add_parser("pmc")
    b.add_argument("csv")
    b.add_argument("kernel")
    sub.add_parser("digest")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(summarize_kernel_stats(args.csv))
    elif args.cmd == "pmc":
        for k, v in summarize_pmc(args.csv, args.kernel).items():
            print(f"{k}: total={v['total']:.6g} dispatches={v['dispatches']} "
                  f"per_dispatch={v['per_dispatch']:.6g}")
    else:
        print(kernel_source_digest())
    return 0


if __name__ == "__main__":
    sys.exit(main())
