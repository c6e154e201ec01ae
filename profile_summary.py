"""Summaries of rocprofv3 output for profiles/ (text only; run on the host after a profiled run).

Two kinds of runs feed it:

* kernel traces -- ``rocprofv3 --kernel-trace --stats --output-format csv -d DIR -o prof -- python3 bench.py ...``:
  ``python3 profile_summary.py trace DIR --title T --command C`` prints a Markdown table of
  every kernel's calls and durations (from the ``*_kernel_stats.csv`` file).

* counter passes -- one ``rocprofv3 --pmc <counters> --output-format csv -d DIR -o prof -- python3 bench.py ...``
  per counter group, ``bench.py --copy-calibration-mib N`` adding one plain copy of N MiB
  (``permute_kernel`` with the identity permutation: N MiB read, N MiB written):
  ``python3 profile_summary.py counters --pass DIR ... --kernel NAME=ALG_BYTES ... --calib-mib N``
  prints, per named kernel, the mean of every counter per dispatch, the HBM traffic per
  dispatch with FETCH_SIZE and WRITE_SIZE each scaled by what the same counter reads for the
  copy (bytes / counter KiB), the ratio to the algorithmic bytes, and MFMA utilisation
  as rocprofv3 defines MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / (the GUI-active
  cycles of one XCD x SIMDs); the per-dispatch GRBM_GUI_ACTIVE value sums the 8 XCDs) when
  those counters were taken; ``--json PATH`` also writes the traffic figures for bench.py:
  the first kernel's, or with ``--op NAME,NAME=ALG_BYTES`` the sum over an operation made of
  several launches (one dispatch of each per call).

Kernels are matched by exact name: the demangled function name without its namespace,
argument list or return type, with or without its template arguments
(``decode_bf16_kernel`` matches ``decode_bf16_kernel<2>``; ``prefill_kernel`` does not
match ``score_prefill_kernel``).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
SIMDS = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
XCDS = 8         # GRBM_GUI_ACTIVE as collected per dispatch is the sum of the 8 XCDs' counters


def kernel_key(demangled: str) -> str:
    """'void spa::(anonymous namespace)::decode_bf16_kernel<2>(spa::DecodeArgs, int, int)' -> 'decode_bf16_kernel<2>'."""
    name = demangled.strip()
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):          # the argument list starts at the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not name[i:].startswith("(anonymous"):
            cut = i
            break
    name = name[:cut]
    # drop the return type (text before the last space outside template brackets)
    depth, start = 0, 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == " " and depth == 0:
            start = i + 1
    name = name[start:]
    # drop the namespaces (the last '::' outside template brackets)
    depth, last = 0, 0
    for i in range(len(name) - 1):
        ch = name[i]
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif depth == 0 and name[i:i + 2] == "::":
            last = i + 2
    return name[last:]


def matches(key: str, want: str) -> bool:
    return key == want or key.split("<", 1)[0] == want


def one_file(d: str, suffix: str) -> str:
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return files[-1]


# --------------------------------------------------------------- traces ----

def trace(args):
    path = one_file(args.dir, "_kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    out = [f"# {args.title}", "", "Command (repository root on one MI355X, ROCm 7.2; $R is the repository root):", "",
           "```", args.command, "```", ""]
    if args.note:
        out += [args.note, ""]
    out += ["| kernel | calls | avg us | min us | max us | share of traced GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| `{kernel_key(r['Name'])}` | {int(r['Calls'])} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{100.0 * float(r['TotalDurationNs']) / total:.1f} % |")
    print("\n".join(out))


# ------------------------------------------------------------- counters ----

def read_counters(d: str):
    """Per (kernel key, dispatch id): {counter: value}."""
    path = one_file(d, "_counter_collection.csv")
    per = defaultdict(dict)
    for r in csv.DictReader(open(path)):
        key = kernel_key(r["Kernel_Name"])
        per[(key, int(r["Dispatch_Id"]))][r["Counter_Name"]] = per[(key, int(r["Dispatch_Id"]))].get(
            r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


def mean_of(per, want: str, counter: str):
    vals = [c[counter] for (k, _), c in per.items() if matches(k, want) and counter in c]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "block_sparse_long_int8_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters(args):
    passes = [read_counters(d) for d in args.pass_dirs]
    calib_bytes = args.calib_mib * (1 << 20)
    fetch_f = write_f = None
    for per in passes:
        f, n = mean_of(per, "permute_kernel", "FETCH_SIZE")
        if f:
            fetch_f = calib_bytes / f
        w, n = mean_of(per, "permute_kernel", "WRITE_SIZE")
        if w:
            write_f = calib_bytes / w
    lines = ["| kernel | dispatches | counter | mean per dispatch |", "|---|---|---|---|"]
    summary = {}
    for spec in args.kernel:
        name, _, alg = spec.partition("=")
        alg = float(alg) if alg else None
        entry = {"algorithmic_bytes": alg}
        for per in passes:
            names = sorted({c for (k, _), cs in per.items() if matches(k, name) for c in cs})
            for c in names:
                v, n = mean_of(per, name, c)
                entry[c] = v
                entry.setdefault("dispatches", n)
                lines.append(f"| `{name}` | {n} | {c} | {v:,.1f} |")
        if "FETCH_SIZE" in entry and fetch_f:
            entry["fetch_bytes"] = entry["FETCH_SIZE"] * fetch_f
        if "WRITE_SIZE" in entry and write_f:
            entry["write_bytes"] = entry["WRITE_SIZE"] * write_f
        if "fetch_bytes" in entry and "write_bytes" in entry:
            entry["traffic_bytes"] = entry["fetch_bytes"] + entry["write_bytes"]
            if alg:
                entry["traffic_over_algorithmic"] = entry["traffic_bytes"] / alg
        if entry.get("SQ_VALU_MFMA_BUSY_CYCLES") is not None and entry.get("GRBM_GUI_ACTIVE"):
            # rocprofv3's MfmaUtil: MFMA-busy cycles summed over the SIMDs / (one XCD's GUI-active cycles x SIMDs)
            entry["mfma_util"] = entry["SQ_VALU_MFMA_BUSY_CYCLES"] / (entry["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
        summary[name] = entry
    out = [f"# {args.title}", "", "Commands (repository root on one MI355X, ROCm 7.2; $R is the repository root):", "",
           "```"] + args.command + ["```", ""]
    if args.note:
        out += [args.note, ""]
    out += [f"Calibration: one `permute_kernel` copy of {args.calib_mib} MiB (identity permutation: "
            f"{calib_bytes:,} bytes read and written) in the same runs. "
            f"FETCH_SIZE factor {fetch_f if fetch_f is None else round(fetch_f, 2)} bytes per KiB counted, "
            f"WRITE_SIZE factor {write_f if write_f is None else round(write_f, 2)}.", "", "Raw counters:", ""]
    out += lines + ["", "Derived:", "", "| kernel | algorithmic bytes | HBM read | HBM written | traffic / algorithmic "
                    "| MFMA util |", "|---|---|---|---|---|---|"]

    def fmt(x, unit=""):
        return "—" if x is None else f"{x / 1e6:,.1f} MB" if unit == "MB" else f"{x:.3f}" if unit == "r" else \
            f"{100 * x:.1f} %"
    for name, e in summary.items():
        out.append(f"| `{name}` | {fmt(e.get('algorithmic_bytes'), 'MB')} | {fmt(e.get('fetch_bytes'), 'MB')} | "
                   f"{fmt(e.get('write_bytes'), 'MB')} | {fmt(e.get('traffic_over_algorithmic'), 'r')} | "
                   f"{fmt(e.get('mfma_util'))} |")
    op = None
    if args.op:
        names, _, alg = args.op.partition("=")
        names = names.split(",")
        parts = [summary[n].get("traffic_bytes") for n in names]
        total = sum(parts) if all(p is not None for p in parts) else None
        op = {"kernels": names, "traffic_bytes": total, "algorithmic_bytes": float(alg) if alg else None}
        if total is not None and alg:
            op["traffic_over_algorithmic"] = total / float(alg)
        out += ["", f"Operation {' + '.join(names)}: "
                f"{fmt(total, 'MB')} of HBM traffic per call against {fmt(op['algorithmic_bytes'], 'MB')} "
                f"algorithmic ({fmt(op.get('traffic_over_algorithmic'), 'r')})."]
    print("\n".join(out))
    if args.json:
        main = summary[args.kernel[0].partition("=")[0]]
        with open(args.json, "w") as f:
            json.dump({"kernels": summary, "operation": op, "fetch_factor": fetch_f, "write_factor": write_f,
                       "kernel_source_sha": source_sha(*args.sources) if args.sources else None,
                       "sources": args.sources,
                       "traffic_bytes_per_launch": op["traffic_bytes"] if op else main.get("traffic_bytes"),
                       "commands": args.command}, f, indent=1)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--note", default="")
    c = sub.add_parser("counters")
    c.add_argument("--pass", dest="pass_dirs", action="append", required=True)
    c.add_argument("--kernel", action="append", required=True, help="NAME or NAME=ALGORITHMIC_BYTES (first = main)")
    c.add_argument("--calib-mib", type=int, default=0)
    c.add_argument("--title", required=True)
    c.add_argument("--command", action="append", default=[])
    c.add_argument("--note", default="")
    c.add_argument("--json", default=None)
    c.add_argument("--sources", nargs="*", default=[], help="csrc files whose hash tags the traffic figure")
    c.add_argument("--op", default=None, help="NAME,NAME=ALGORITHMIC_BYTES: an operation of several launches")
    a = ap.parse_args(argv)
    trace(a) if a.what == "trace" else counters(a)


if __name__ == "__main__":
    main()
