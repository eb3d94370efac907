"""Summaries of rocprofv3 output for the attention kernel.

    python -m exact_attention_forward_02_amd.profiling stats  RUN_kernel_stats.csv
    python -m exact_attention_forward_02_amd.profiling trace  RUN_kernel_trace.csv [--last K]
    python -m exact_attention_forward_02_amd.profiling pmc    RUN_counter_collection.csv [--kernel NAME]
    python -m exact_attention_forward_02_amd.profiling traffic --fetch F.csv --write W.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --workload NAME [--out PATH]

`stats` prints per-kernel call counts and durations from a --kernel-trace
--stats run (CSV output).  `trace` reads the per-dispatch records of the same
run and prints the durations of the attention kernel over all its dispatches
and over the last K (the timed steps, after the warmup launches that bring
the clocks up).  `pmc` averages every counter per dispatch of the
kernels whose name contains NAME.  `traffic` turns FETCH_SIZE / WRITE_SIZE
(KiB per dispatch) of the attention kernel (or the sum over a sequence of
kernels that one call launches, such as the backward's) into HBM bytes per
launch, each
scaled by what the same counter reads for a plain copy kernel that moves a
known number of bytes, and writes the JSON record bench.py reports while the
kernel source is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCE = os.path.join(ROOT, "exact_attention_forward_02_amd", "csrc",
                             "attn_fwd_kernel.hip")


def kernel_source_digest(path: str = KERNEL_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def read_kernel_stats(path):
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append({
                "name": r.get("Name") or r.get("KERNEL_NAME") or r.get("Kernel_Name"),
                "calls": int(r.get("Calls", 0)),
                "total_ns": float(r.get("TotalDurationNs", 0)),
                "avg_ns": float(r.get("AverageNs", 0)),
                "min_ns": float(r.get("MinNs", 0)),
                "max_ns": float(r.get("MaxNs", 0)),
                "pct": float(r.get("Percentage", 0)),
            })
    return rows


def read_counters(path, kernel="attn_fwd_kernel"):
    """Mean value of each counter per dispatch of the matching kernels."""
    per = defaultdict(lambda: defaultdict(float))
    names = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            kname = r.get("Kernel_Name", "")
            if kernel and kernel not in kname:
                continue
            d = r.get("Dispatch_Id") or r.get("Correlation_Id")
            per[d][r["Counter_Name"]] += float(r["Counter_Value"])
            names[d] = kname
    if not per:
        return {}, 0, ""
    keys = sorted({k for v in per.values() for k in v})
    mean = {k: sum(v.get(k, 0.0) for v in per.values()) / len(per) for k in keys}
    return mean, len(per), next(iter(names.values()))


def cmd_stats(args):
    for r in read_kernel_stats(args.csv):
        print(f"{r['name'][:100]:100s} calls={r['calls']:4d} avg={r['avg_ns'] / 1e3:9.2f} us "
              f"min={r['min_ns'] / 1e3:9.2f} max={r['max_ns'] / 1e3:9.2f} ({r['pct']:.1f}%)")


def read_dispatch_durations(path, kernel="attn_fwd_kernel"):
    """Durations (ns) of the matching kernel's dispatches, in dispatch order."""
    recs = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if kernel and kernel not in r.get("Kernel_Name", ""):
                continue
            recs.append((int(r["Dispatch_Id"]),
                         float(r["End_Timestamp"]) - float(r["Start_Timestamp"])))
    recs.sort()
    return [d for _, d in recs]


def _summary(label, durs):
    n = len(durs)
    avg = sum(durs) / n
    print(f"{label:28s} dispatches={n:4d} avg={avg / 1e3:9.2f} us "
          f"min={min(durs) / 1e3:9.2f} max={max(durs) / 1e3:9.2f}")


def cmd_trace(args):
    durs = read_dispatch_durations(args.csv, args.kernel)
    if not durs:
        print(f"no dispatch of a kernel matching {args.kernel!r}")
        return
    _summary("all dispatches", durs)
    if args.last and args.last < len(durs):
        _summary(f"last {args.last} dispatches", durs[-args.last:])


def cmd_pmc(args):
    mean, n, name = read_counters(args.csv, args.kernel)
    print(f"kernel: {name}\ndispatches: {n}")
    for k, v in mean.items():
        print(f"{k:32s} {v:,.0f}")


def read_counters_sum(path, kernels):
    """Counters per call of a sequence of kernels (names separated by commas):
    the per-dispatch means of each kernel, added up, and the dispatch counts."""
    total, counts = defaultdict(float), []
    for name in kernels.split(","):
        mean, n, _ = read_counters(path, name)
        if not n:
            raise SystemExit(f"{path}: no dispatch of a kernel matching {name!r}")
        for k, v in mean.items():
            total[k] += v
        counts.append(n)
    return dict(total), counts


def cmd_traffic(args):
    fetch, nf = read_counters_sum(args.fetch, args.kernel)
    write, nw = read_counters_sum(args.write, args.kernel)
    cfetch, _, _ = read_counters(args.copy_fetch, args.copy_kernel)
    cwrite, _, _ = read_counters(args.copy_write, args.copy_kernel)
    f_scale = args.copy_bytes / (cfetch["FETCH_SIZE"] * 1024.0)
    w_scale = args.copy_bytes / (cwrite["WRITE_SIZE"] * 1024.0)
    fetch_b = fetch["FETCH_SIZE"] * 1024.0 * f_scale
    write_b = write["WRITE_SIZE"] * 1024.0 * w_scale
    rec = {
        "kernel": args.kernel,
        "workload": args.workload,
        "kernel_source": os.path.basename(args.source),
        "kernel_source_sha256": kernel_source_digest(args.source),
        "fetch_kib_per_dispatch": fetch["FETCH_SIZE"],
        "write_kib_per_dispatch": write["WRITE_SIZE"],
        "dispatches": [nf, nw],  # per kernel of the sequence, FETCH and WRITE runs
        "copy_bytes": args.copy_bytes,
        "copy_fetch_kib": cfetch["FETCH_SIZE"],
        "copy_write_kib": cwrite["WRITE_SIZE"],
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "hbm_bytes_per_launch": fetch_b + write_b,
        "hbm_read_bytes_per_launch": fetch_b,
        "hbm_write_bytes_per_launch": write_b,
    }
    text = json.dumps(rec, indent=2)
    print(text)
    if args.out:
        with open(args.out, "w", encoding="utf-8") as f:
            f.write(text + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.set_defaults(fn=cmd_stats)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("--kernel", default="attn_fwd_kernel")
    t.add_argument("--last", type=int, default=0)
    t.set_defaults(fn=cmd_trace)
    b = sub.add_parser("pmc")
    b.add_argument("csv")
    b.add_argument("--kernel", default="attn_fwd_kernel")
    b.set_defaults(fn=cmd_pmc)
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--copy-bytes", type=float, required=True)
    c.add_argument("--copy-kernel", default="neg")  # the calibration copy is torch.neg
    c.add_argument("--kernel", default="attn_fwd_kernel",
                   help="kernel name, or several separated by commas: one call launches "
                        "each once and the record holds their sum")
    c.add_argument("--source", default=KERNEL_SOURCE,
                   help="the kernel's source file, whose hash the record carries")
    c.add_argument("--workload", required=True)
    c.add_argument("--out")
    c.set_defaults(fn=cmd_traffic)
    args = ap.parse_args(argv)
    args.fn(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
