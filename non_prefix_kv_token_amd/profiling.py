"""Summaries of rocprofv3 output for the profiles/ folder.

  python -m non_prefix_kv_token_amd.profiling stats  <kernel_stats.csv> --title T --command C --out F
  python -m non_prefix_kv_token_amd.profiling traffic --fetch DIR --write DIR --kernel-substr S \
         --name attention --workload W --source FILE --command-fetch C1 --command-write C2 --out F
  python -m non_prefix_kv_token_amd.profiling counters DIR --title T --command C --out F

`counters` tabulates every counter of a `rocprofv3 --pmc` run per kernel
(mean per dispatch, as rocprofv3 reports them: summed over the device).

`traffic` reads two `rocprofv3 --pmc` runs of the same program (FETCH_SIZE,
then WRITE_SIZE; both in KiB per dispatch) that also ran a 1 GiB device copy
(`bench.py --copy-calib`).  Each counter is scaled by 1 GiB divided by what
it reads for that copy, and the record line carries the sha256 of the
kernel's source so that bench.py reports the figure only while the kernel is
unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics

GIB = 1 << 30


def _rows(path_or_dir: str, pattern: str):
    paths = [path_or_dir] if os.path.isfile(path_or_dir) else \
        glob.glob(os.path.join(path_or_dir, "**", pattern), recursive=True)
    out = []
    for p in paths:
        with open(p) as f:
            out.extend(csv.DictReader(f))
    return out


def short_name(name: str) -> str:
    """Kernel name without its parameter list (the first '(' outside template
    brackets)."""
    name = name.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def kernel_stats_table(stats_csv: str) -> str:
    rows = _rows(stats_csv, "*kernel_stats.csv")
    lines = ["| Kernel | Calls | Average (us) | Total (ms) | Share |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        name = short_name(r["Name"])
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(lines)


def counter_per_dispatch(pmc_dir: str, counter: str, kernel_substr: str):
    vals = [float(r["Counter_Value"]) for r in _rows(pmc_dir, "*counter_collection.csv")
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]]
    return vals


def copy_reading(pmc_dir: str, counter: str) -> float:
    """The counter's reading (KiB) for the 1 GiB calibration copies: the
    largest dispatches of the runtime's copy kernel."""
    vals = counter_per_dispatch(pmc_dir, counter, "copyBuffer")
    if not vals:
        raise SystemExit(f"no copy kernel dispatches with {counter} in {pmc_dir}")
    top = sorted(vals)[-3:]
    return statistics.mean(top)


def counters_table(pmc_dir: str) -> str:
    rows = _rows(pmc_dir, "*counter_collection.csv")
    per = {}
    for r in rows:
        per.setdefault(short_name(r["Kernel_Name"]), {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    names = sorted({c for d in per.values() for c in d})
    kernels = sorted(per)
    lines = ["| Counter | " + " | ".join(f"`{k}`" for k in kernels) + " |",
             "|---|" + "---:|" * len(kernels)]
    lines.append("| dispatches | " + " | ".join(str(len(next(iter(per[k].values())))) for k in kernels) + " |")
    for c in names:
        vals = [f"{statistics.mean(per[k][c]):.4g}" if c in per[k] else "" for k in kernels]
        lines.append(f"| {c} | " + " | ".join(vals) + " |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--note", default="")
    c.add_argument("--out", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--title", required=True)
    a.add_argument("--command", required=True)
    a.add_argument("--note", default="")
    a.add_argument("--out", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel-substr", required=True)
    b.add_argument("--name", required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--source", required=True)
    b.add_argument("--algorithmic-bytes", type=float, default=None)
    b.add_argument("--command-fetch", required=True)
    b.add_argument("--command-write", required=True)
    b.add_argument("--out", required=True)
    args = ap.parse_args()

    if args.cmd == "counters":
        text = f"# {args.title}\n\nCommand (from the repository root, on an MI355X):\n\n    {args.command}\n\n"
        if args.note:
            text += args.note + "\n\n"
        text += counters_table(args.dir) + "\n"
        with open(args.out, "w") as f:
            f.write(text)
        return

    if args.cmd == "stats":
        text = f"# {args.title}\n\nCommand (from the repository root, on an MI355X):\n\n    {args.command}\n\n"
        if args.note:
            text += args.note + "\n\n"
        text += kernel_stats_table(args.csv) + "\n"
        with open(args.out, "w") as f:
            f.write(text)
        return

    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE", args.kernel_substr)
    write = counter_per_dispatch(args.write, "WRITE_SIZE", args.kernel_substr)
    if not fetch or not write:
        raise SystemExit("kernel not found in the counter runs")
    f_kib, w_kib = statistics.mean(fetch), statistics.mean(write)
    f_scale = GIB / (copy_reading(args.fetch, "FETCH_SIZE") * 1024.0)
    w_scale = GIB / (copy_reading(args.write, "WRITE_SIZE") * 1024.0)
    with open(args.source, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    total = f_kib * 1024 * f_scale + w_kib * 1024 * w_scale
    text = (f"# HBM traffic of `{args.name}` ({args.workload})\n\n"
            f"Counters per dispatch, mean over {len(fetch)} / {len(write)} dispatches, each scaled by\n"
            f"1 GiB / (the same counter's reading for a 1 GiB device copy in the same run).\n\n"
            f"| Counter | KiB per dispatch | scale | bytes per launch |\n|---|---:|---:|---:|\n"
            f"| FETCH_SIZE | {f_kib:.0f} | {f_scale:.4f} | {f_kib * 1024 * f_scale:.4g} |\n"
            f"| WRITE_SIZE | {w_kib:.0f} | {w_scale:.4f} | {w_kib * 1024 * w_scale:.4g} |\n"
            f"| total | | | {total:.4g} |\n\n")
    if args.algorithmic_bytes:
        text += f"Algorithmic bytes per launch: {args.algorithmic_bytes:.4g} (ratio {total / args.algorithmic_bytes:.2f}).\n\n"
    text += ("Commands (from the repository root, on an MI355X):\n\n"
             f"    {args.command_fetch}\n    {args.command_write}\n\n"
             f"Kernel source: `{args.source}`.\n\n"
             f"traffic-record: kernel={args.name} workload={args.workload} source_sha256={sha} "
             f"fetch_bytes={f_kib * 1024:.0f} fetch_scale={f_scale:.6f} "
             f"write_bytes={w_kib * 1024:.0f} write_scale={w_scale:.6f}\n")
    with open(args.out, "w") as f:
        f.write(text)


if __name__ == "__main__":
    main()
