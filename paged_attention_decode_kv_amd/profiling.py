"""Summaries of rocprofv3 output for this library's kernels.

* ``trace``: the ``--kernel-trace --stats`` statistics of the library's kernels as a
  markdown table (calls, average, minimum and maximum duration).
* ``traffic``: HBM bytes per launch of one kernel from two counter runs of the same
  command, one with ``--pmc FETCH_SIZE`` and one with ``--pmc WRITE_SIZE`` (KiB per
  dispatch).  Each counter is scaled by what it reads for an elementwise kernel of
  known size in the same run: ``bench.py --copy-calibration`` multiplies a 1 GiB
  float32 tensor by a scalar three times (1 GiB read and 1 GiB written each); on MI355X
  FETCH_SIZE counts half the bytes read and WRITE_SIZE all the bytes written.  The
  record goes into ``profiles/decode_traffic.json`` keyed by workload, layout and the
  sha256 of ``csrc/kernels.hip``, which ``bench.py`` matches before it reports
  ``roofline.traffic``.

Usage (from the repository root)::

    python -m paged_attention_decode_kv_amd.profiling trace <run_kernel_stats.csv>
    python -m paged_attention_decode_kv_amd.profiling traffic --fetch <fetch csv> \\
        --write <write csv> --workload full-width --layout HND --tag full_width_bf16 \\
        --kernel decode_kernel --algorithmic-bytes 7898094632 --update
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_SOURCE = os.path.join(PKG, "csrc", "kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
CALIBRATION_KERNEL = "AUnaryFunctor<float, float"    # torch's multiply by a scalar
CALIBRATION_KIB = 1 << 20                             # 1 GiB read, 1 GiB written


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def short_name(name: str) -> str:
    """``void pkv::decode_kernel<unsigned short, 128, 8, true, 1>(pkv::AttnArgs, ...)``
    -> ``pkv::decode_kernel<unsigned short, 128, 8, true, 1>``."""
    name = name.strip().removeprefix("void ")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def kernel_stats(path: str, prefix: str = "pkv::") -> list[dict]:
    """The statistics rows of this library's kernels, slowest total first."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            name = short_name(r["Name"])
            if not name.startswith(prefix):
                continue
            rows.append({"kernel": name, "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3,
                         "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3,
                         "total_us": float(r["TotalDurationNs"]) / 1e3})
    rows.sort(key=lambda r: -r["total_us"])
    return rows


def stats_table(rows: list[dict]) -> str:
    out = ["| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']:.2f} | "
                   f"{r['min_us']:.2f} | {r['max_us']:.2f} |")
    return "\n".join(out)


def counter_values(path: str, counter: str) -> dict[str, list[float]]:
    """Counter value (KiB) of every dispatch, by full kernel name."""
    out = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return out


def _mean_of(values: dict[str, list[float]], match: str, what: str) -> tuple[str, float, int]:
    names = [n for n in values if match in n]
    if len(names) != 1:
        raise SystemExit(f"{what}: {len(names)} kernels match {match!r}: "
                         f"{[short_name(n) for n in names]}")
    v = values[names[0]]
    return names[0], sum(v) / len(v), len(v)


def traffic_record(fetch_csv: str, write_csv: str, *, kernel: str, workload: str,
                   layout: str, tag: str, algorithmic_bytes: int,
                   commands: list[str]) -> dict:
    """HBM bytes per launch of the kernel whose name contains ``kernel``."""
    fetch = counter_values(fetch_csv, "FETCH_SIZE")
    write = counter_values(write_csv, "WRITE_SIZE")
    name, fetch_kib, n_fetch = _mean_of(fetch, kernel, "FETCH_SIZE")
    _, write_kib, n_write = _mean_of(write, kernel, "WRITE_SIZE")
    _, cal_fetch, _ = _mean_of(fetch, CALIBRATION_KERNEL, "FETCH_SIZE calibration")
    _, cal_write, _ = _mean_of(write, CALIBRATION_KERNEL, "WRITE_SIZE calibration")
    fetch_scale = CALIBRATION_KIB / cal_fetch
    write_scale = CALIBRATION_KIB / cal_write
    fetch_bytes = round(fetch_kib * 1024 * fetch_scale)
    write_bytes = round(write_kib * 1024 * write_scale)
    total = fetch_bytes + write_bytes
    return {
        "workload": workload,
        "layout": layout,
        "tag": tag,
        "kernel": short_name(name),
        "kernel_source_sha256": kernel_source_hash(),
        "dispatches": {"fetch": n_fetch, "write": n_write},
        "fetch_kib_per_dispatch": fetch_kib,
        "write_kib_per_dispatch": write_kib,
        "calibration": {
            "kernel": "torch elementwise multiply over 1 GiB float32 (reads 1 GiB, writes 1 GiB)",
            "fetch_kib": cal_fetch,
            "write_kib": cal_write,
            "fetch_scale": fetch_scale,
            "write_scale": write_scale,
        },
        "fetch_bytes": fetch_bytes,
        "write_bytes": write_bytes,
        "bytes_per_launch": total,
        "algorithmic_bytes_per_launch": int(algorithmic_bytes),
        "traffic_over_algorithmic": total / int(algorithmic_bytes),
        "commands": commands,
    }


def update_records(rec: dict, path: str = TRAFFIC_FILE) -> None:
    """Replace the record of the same workload and layout (any kernel source)."""
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {"records": []}
    data["records"] = [r for r in data.get("records", [])
                       if (r.get("workload"), r.get("layout")) != (rec["workload"], rec["layout"])]
    data["records"].append(rec)
    data["records"].sort(key=lambda r: (r["workload"], r["layout"]))
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace", help="markdown table of a kernel-trace statistics csv")
    t.add_argument("stats")
    c = sub.add_parser("traffic", help="HBM bytes per launch from FETCH/WRITE counter runs")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--kernel", required=True, help="a substring naming the kernel")
    c.add_argument("--workload", required=True)
    c.add_argument("--layout", default="HND")
    c.add_argument("--tag", required=True)
    c.add_argument("--algorithmic-bytes", type=int, required=True)
    c.add_argument("--command", action="append", default=[],
                   help="a command of the counter runs (repeatable)")
    c.add_argument("--update", action="store_true", help=f"write into {TRAFFIC_FILE}")
    args = ap.parse_args(argv)
    if args.cmd == "trace":
        print(stats_table(kernel_stats(args.stats)))
        return
    rec = traffic_record(args.fetch, args.write, kernel=args.kernel, workload=args.workload,
                         layout=args.layout, tag=args.tag,
                         algorithmic_bytes=args.algorithmic_bytes, commands=args.command)
    print(json.dumps(rec, indent=1))
    if args.update:
        update_records(rec)


if __name__ == "__main__":
    main(sys.argv[1:])
