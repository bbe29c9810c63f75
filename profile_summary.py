#!/usr/bin/env python3
"""Summarise rocprofv3 runs of bench.py into short text files under profiles/.

    python profile_summary.py <run_dir> <workload-name> [<calibration_dir>]

<run_dir> holds, from one GPU session (each a rocprofv3 output directory):
  ktcsv/      --kernel-trace --stats --output-format csv
  fetch/      --pmc FETCH_SIZE        (rocpd database)
  write/      --pmc WRITE_SIZE        (rocpd database)
  cal_fetch/  --pmc FETCH_SIZE of `bench.py --copy-calibration`
  cal_write/  --pmc WRITE_SIZE of `bench.py --copy-calibration`
and commands.txt with the exact commands that produced them.  The two
calibration runs may come from another directory (third argument).

Writes profiles/<kernel>_<workload>.txt (per-kernel durations, HBM bytes
per launch after scaling by the copy calibration) and
profiles/gemm_traffic_<workload>.json, which bench.py reads for the
roofline's `traffic` field when the GEMM source is unchanged since.
"""

from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "fp4_block_scaled_elem_amd", "csrc", "gemm.hip")


def source_hash(path=GEMM_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def short(name: str) -> str:
    n = name.split("(")[0].replace("void ", "").replace("mq::", "")
    return n


def pmc(db_dir: str):
    dbs = glob.glob(os.path.join(db_dir, "**", "*.db"), recursive=True)
    out = collections.defaultdict(list)
    for db in dbs:
        c = sqlite3.connect(db).cursor()
        for name, grid, cnt, val in c.execute(
                "select kernel_name, grid_size, counter_name, value from counters_collection"):
            out[(short(name), grid, cnt)].append(val)
    return out


def main():
    run, workload = sys.argv[1], sys.argv[2]
    cal = sys.argv[3] if len(sys.argv) > 3 else run
    stats = list(csv.DictReader(open(glob.glob(os.path.join(run, "ktcsv", "**", "*kernel_stats.csv"),
                                               recursive=True)[0])))
    fetch, write = pmc(os.path.join(run, "fetch")), pmc(os.path.join(run, "write"))
    calf, calw = pmc(os.path.join(cal, "cal_fetch")), pmc(os.path.join(cal, "cal_write"))
    cal_read = [v for (n, g, c), v in calf.items() if "neg_kernel" in n]
    cal_wr = [v for (n, g, c), v in calw.items() if "neg_kernel" in n]
    gib_kib = float(1 << 20)
    f_fetch = gib_kib / (sum(cal_read[0]) / len(cal_read[0]))
    f_write = gib_kib / (sum(cal_wr[0]) / len(cal_wr[0]))
    commands = open(os.path.join(run, "commands.txt")).read().strip()

    def per_kernel(table, counter, factor):
        acc = collections.defaultdict(list)
        for (n, g, c), v in table.items():
            if c == counter:
                acc[(n, g)].extend(v)
        return {k: factor * 1024.0 * sum(v) / len(v) for k, v in acc.items()}

    fb = per_kernel(fetch, "FETCH_SIZE", f_fetch)
    wb = per_kernel(write, "WRITE_SIZE", f_write)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    lines = [f"# rocprofv3 summary: {workload}", "",
             "Commands (run from the repository root on one MI355X):", "", commands, "",
             f"HBM byte counters scaled by the copy calibration: FETCH_SIZE x {f_fetch:.3f}, "
             f"WRITE_SIZE x {f_write:.3f} (a plain 1 GiB read + 1 GiB write elementwise kernel).",
             f"gemm.hip sha256[:16] = {source_hash()}", "",
             "## Kernel trace (--kernel-trace --stats)", "",
             f"{'kernel':72s} {'calls':>5s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}"]
    for r in stats:
        lines.append(f"{short(r['Name'])[:72]:72s} {int(r['Calls']):5d} {float(r['AverageNs'])/1e3:9.1f} "
                     f"{float(r['MinNs'])/1e3:9.1f} {float(r['MaxNs'])/1e3:9.1f} {float(r['Percentage']):7.2f}")
    g_all = [r for r in stats if short(r["Name"]).startswith("gemm_nvfp4_kernel")]
    if g_all:
        calls = sum(int(r["Calls"]) for r in g_all)
        tot_ns = sum(float(r["TotalDurationNs"]) for r in g_all)
        lines += ["", f"all gemm_nvfp4_kernel launches: {calls} calls, average {tot_ns / calls / 1e3:.1f} us"]
    lines += ["", "## HBM bytes per launch (scaled counters), by kernel and grid size", "",
              f"{'kernel':60s} {'grid':>9s} {'read_MiB':>10s} {'write_MiB':>10s}"]
    for k in sorted(set(fb) | set(wb)):
        lines.append(f"{k[0][:60]:60s} {k[1]:9d} {fb.get(k, 0)/2**20:10.1f} {wb.get(k, 0)/2**20:10.1f}")
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    # traffic for the GEMM launches of one step, per launch (mean over launches)
    launches = collections.Counter()
    for (n, g, c), v in fetch.items():
        if n.startswith("gemm_nvfp4_kernel") and c == "FETCH_SIZE":
            launches[(n, g)] += len(v)
    tot = sum(launches.values())
    if not tot:
        print(path)
        return
    mean_read = sum(fb[k] * launches[k] for k in launches) / tot
    mean_write = sum(wb.get(k, 0) * launches[k] for k in launches) / tot
    json.dump({"workload": workload, "gemm_source_sha256_16": source_hash(),
               "bytes_per_launch": mean_read + mean_write, "read_bytes_per_launch": mean_read,
               "write_bytes_per_launch": mean_write, "fetch_scale": f_fetch, "write_scale": f_write},
              open(os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}.json"), "w"), indent=1)
    print(path)


if __name__ == "__main__":
    main()
