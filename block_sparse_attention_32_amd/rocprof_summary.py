"""Turns rocprofv3 CSV output into the short summaries kept under profiles/.

  python -m block_sparse_attention_32_amd.rocprof_summary trace \
      --stats DIR/trace_kernel_stats.csv --workload W --command "..."
      -> profiles/kernel_trace_<W>.txt

  python -m block_sparse_attention_32_amd.rocprof_summary traffic \
      --fetch DIR1/pmc_counter_collection.csv --write DIR2/pmc_counter_collection.csv \
      --kernel NAME --workload W --files a.hip b.hpp ... \
      --fetch-command "..." --write-command "..."
      -> profiles/<NAME>_<W>_traffic.json

FETCH_SIZE and WRITE_SIZE (KiB per dispatch, L2 <-> memory) of the kernel
are averaged over its dispatches and each scaled by what the same counter
reads for a plain device copy of 256 MiB in the same run (the
`--copy-calibration` dispatch of bench.py).  The JSON records the hash of
the kernel's source files so that bench.py reports the traffic only while
the kernel is unchanged.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20


def source_hash(*files) -> str:
    """Short hash of kernel source files under csrc/."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from a committed traffic summary taken on the
    current kernel source, else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "").strip()


def trace_summary(stats_csv: str, workload: str, command: str) -> str:
    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    lines = [f"# rocprofv3 kernel trace, workload {workload}",
             f"# command: {command}",
             "#",
             f"# {'calls':>7} {'total_ms':>10} {'avg_us':>11} {'min_us':>10} {'max_us':>10} {'%':>6}  kernel"]
    for r in rows:
        lines.append(f"  {int(r['Calls']):>7} {float(r['TotalDurationNs']) / 1e6:>10.3f} "
                     f"{float(r['AverageNs']) / 1e3:>11.2f} {float(r['MinNs']) / 1e3:>10.2f} "
                     f"{float(r['MaxNs']) / 1e3:>10.2f} {float(r['Percentage']):>6.2f}  "
                     f"{_short(r['Name'])}")
    return "\n".join(lines) + "\n"


def _counter(csv_path: str, counter: str):
    """{dispatch id: (kernel name, value)} of one counter."""
    out = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            if d in out:
                out[d] = (name, out[d][1] + v)
            else:
                out[d] = (name, v)
    return out


def _kernel_avg_and_factor(csv_path: str, counter: str, kernel: str):
    vals = _counter(csv_path, counter)
    mine = [v for n, v in vals.values() if _short(n).split("<")[0].endswith(kernel)]
    copies = [v for n, v in vals.values() if "copyBuffer" in n]
    if not mine:
        raise SystemExit(f"no dispatch of {kernel} in {csv_path}")
    if not copies:
        raise SystemExit(f"no copy dispatch in {csv_path} (run bench.py with --copy-calibration)")
    copy_kib = min(copies, key=lambda v: abs(v - COPY_BYTES / 1024.0))
    factor = COPY_BYTES / (copy_kib * 1024.0)
    return sum(mine) / len(mine), len(mine), copy_kib, factor


def traffic_summary(fetch_csv, write_csv, kernel, workload, files, fetch_cmd, write_cmd):
    f_avg, f_n, f_copy, f_fac = _kernel_avg_and_factor(fetch_csv, "FETCH_SIZE", kernel)
    w_avg, w_n, w_copy, w_fac = _kernel_avg_and_factor(write_csv, "WRITE_SIZE", kernel)
    fetch_b = f_avg * 1024.0 * f_fac
    write_b = w_avg * 1024.0 * w_fac
    return {
        "kernel": kernel, "workload": workload,
        "source_files": list(files), "source_hash": source_hash(*files),
        "hbm_bytes_per_launch": round(fetch_b + write_b),
        "fetch_bytes_per_launch": round(fetch_b), "write_bytes_per_launch": round(write_b),
        "fetch_kib_per_dispatch_raw": round(f_avg, 1), "write_kib_per_dispatch_raw": round(w_avg, 1),
        "dispatches": {"fetch_run": f_n, "write_run": w_n},
        "copy_calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": f_copy, "fetch_factor": f_fac,
                             "write_kib": w_copy, "write_factor": w_fac},
        "commands": {"fetch": fetch_cmd, "write": write_cmd},
    }


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--stats", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    m = sub.add_parser("traffic")
    m.add_argument("--fetch", required=True)
    m.add_argument("--write", required=True)
    m.add_argument("--kernel", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--files", nargs="+", required=True)
    m.add_argument("--fetch-command", required=True)
    m.add_argument("--write-command", required=True)
    a = ap.parse_args()
    os.makedirs(PROFILES, exist_ok=True)
    if a.what == "trace":
        path = os.path.join(PROFILES, f"kernel_trace_{a.workload}.txt")
        with open(path, "w") as f:
            f.write(trace_summary(a.stats, a.workload, a.command))
    else:
        d = traffic_summary(a.fetch, a.write, a.kernel, a.workload, a.files,
                            a.fetch_command, a.write_command)
        path = os.path.join(PROFILES, f"{a.kernel}_{a.workload}_traffic.json")
        with open(path, "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
