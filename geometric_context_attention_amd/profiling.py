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
# the same for the intra-frame layers at 64 frames per call (frame mode)
FRAME_TRAFFIC_FILE = os.path.join(os.path.dirname(PKG), "profiles",
                                  "k_attn_bf16_frame_mode_intra_frame_64_per_call_traffic.txt")


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


def trace_report(stats_csv: str, title: str, workload: str, commands, bench_line: str | None = None) -> str:
    """Text summary of a ``rocprofv3 --kernel-trace --stats`` run for
    ``profiles/``: what was run, the kernel source digest, the per-kernel
    table and, if given, the bench JSON line the traced run printed."""
    out = [f"# {title}", "#", f"# Workload: {workload}", "#",
           "# Commands (from the repository root, TMPDIR=/tmp):"]
    out += [f"#   {c}" for c in commands]
    out += ["#", f"# kernel_source_sha256: {kernel_source_digest()}", "", summarize_kernel_stats(stats_csv)]
    if bench_line:
        out += ["", "# Bench line printed by the traced run:", "#   " + bench_line.strip()]
    return "\n".join(out) + "\n"


def pmc_per_dispatch(path: str, kernel: str, counter: str) -> float:
    """Mean per-dispatch value of one counter for the kernels whose name
    contains `kernel` in a ``rocprofv3 --pmc`` CSV."""
    v = summarize_pmc(path, kernel).get(counter)
    if v is None:
        raise KeyError(f"{counter} not found for {kernel} in {path}")
    return v["per_dispatch"]


def counter_total(path: str, kernel: str, counter: str) -> float:
    v = summarize_pmc(path, kernel).get(counter)
    return 0.0 if v is None else v["total"]


def traffic_report(fetch_csv: str, write_csv: str, cal_fetch_csv: str, cal_write_csv: str, kernel: str,
                   kv_bytes: float, cal_read: float, cal_written: float, workload: str, commands,
                   read_label: str = "K/V") -> str:
    """Calibrated HBM bytes per dispatch of `kernel` from two ``--pmc`` runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the copy calibration (``bench.py --copy-calibration``:
    `cal_read` bytes read and `cal_written` written by its elementwise
    kernels).  The result is the traffic file bench.py reads."""
    f = pmc_per_dispatch(fetch_csv, kernel, "FETCH_SIZE")
    w = pmc_per_dispatch(write_csv, kernel, "WRITE_SIZE")
    cf = counter_total(cal_fetch_csv, "elementwise", "FETCH_SIZE")
    cw = counter_total(cal_write_csv, "elementwise", "WRITE_SIZE")
    sf = cal_read / (cf * 1024.0)
    sw = cal_written / (cw * 1024.0)
    fb, wb = f * 1024.0 * sf, w * 1024.0 * sw
    out = [f"# {kernel} HBM traffic per launch (rocprofv3 counters)", "#", f"# Workload: {workload}", "#",
           "# Commands (from the repository root, TMPDIR=/tmp), one counter per run:"]
    out += [f"#   {c}" for c in commands]
    out += ["#",
            f"# Raw (KiB per dispatch): FETCH_SIZE {f:.1f}, WRITE_SIZE {w:.1f}",
            f"# Calibration (elementwise copy kernels): FETCH_SIZE {cf:.6g} KiB for {cal_read:.6g} B read,",
            f"#   WRITE_SIZE {cw:.6g} KiB for {cal_written:.6g} B written => scale x{sf:.4f} / x{sw:.4f}",
            f"# Algorithmic {read_label} bytes per launch: {kv_bytes:.6g}; calibrated fetch is {fb / kv_bytes:.3f}x that",
            "", f"kernel_source_sha256: {kernel_source_digest()}",
            f"fetch_bytes_per_launch: {fb:.6g}", f"write_bytes_per_launch: {wb:.6g}",
            f"hbm_bytes_per_launch: {fb + wb:.6g}"]
    return "\n".join(out) + "\n"


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
    t = sub.add_parser("trace-report")
    t.add_argument("csv")
    t.add_argument("--title", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", action="append", default=[])
    t.add_argument("--bench-json", help="file whose last line is the bench JSON line of the traced run")
    t.add_argument("--out", required=True)
    r = sub.add_parser("traffic-report")
    for name in ("fetch", "write", "cal_fetch", "cal_write"):
        r.add_argument("--" + name.replace("_", "-"), required=True)
    r.add_argument("--kernel", default="k_attn_bf16")
    r.add_argument("--kv-bytes", type=float, required=True, help="algorithmic bytes read per launch")
    r.add_argument("--read-label", default="K/V", help="what those bytes are, for the report")
    r.add_argument("--cal-read", type=float, required=True)
    r.add_argument("--cal-written", type=float, required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--command", action="append", default=[])
    r.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "traffic-report":
        with open(args.out, "w") as fh:
            fh.write(traffic_report(args.fetch, args.write, args.cal_fetch, args.cal_write, args.kernel,
                                    args.kv_bytes, args.cal_read, args.cal_written, args.workload, args.command,
                                    args.read_label))
        return 0
    if args.cmd == "trace-report":
        line = None
        if args.bench_json and os.path.exists(args.bench_json):
            lines = [x for x in open(args.bench_json).read().splitlines() if x.strip().startswith("{")]
            line = lines[-1] if lines else None
        with open(args.out, "w") as fh:
            fh.write(trace_report(args.csv, args.title, args.workload, args.command, line))
        return 0
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
