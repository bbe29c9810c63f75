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

    python profile_summary.py --counters <run_dir> <workload-name>

    python profile_summary.py --peak <run_dir>

<run_dir>/peak/ holds a `rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE` run
of `bench.py --peak`; writes profiles/mfma_peak.txt (rate and clock of the
fp16 MFMA rate kernel per VALU load).

<run_dir> holds p1/ and p2/, two `rocprofv3 --kernel-trace --pmc ...` runs
of the same bench.py command with the counter sets COUNTERS_P1 and
COUNTERS_P2, and commands.txt; writes profiles/counters_<workload>.txt
(MFMA, VALU and LDS counters per kind of launch).

    python profile_summary.py --trace <run_dir> <workload-name>

<run_dir>/ktcsv/ holds a --kernel-trace --stats --output-format csv run and
commands.txt its command; writes profiles/kernels_<workload>.txt (kernel
durations only).
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


# the prefill GEMM's kernels: one tile per workgroup, and the fused
# prologue's quantize-once form
GEMM_KERNELS = ("gemm_nvfp4_kernel", "gemm_panel_kernel", "gemm_small_kernel")


def source_hash(path=GEMM_SRC) -> str:
    """Digest of gemm.hip's code (comments and whitespace ignored), the one
    bench.py compares before it reports the traffic figure."""
    from bench import code_digest
    return code_digest(path)


def short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("mq::", "")
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


def trace_main(run: str, workload: str):
    """Kernel durations only (a --kernel-trace --stats run in <run>/ktcsv)."""
    stats = list(csv.DictReader(open(glob.glob(os.path.join(run, "ktcsv", "**", "*kernel_stats.csv"),
                                               recursive=True)[0])))
    commands = open(os.path.join(run, "commands.txt")).read().strip()
    lines = [f"# rocprofv3 summary: {workload}", "",
             "Command (run from the repository root on one MI355X):", "", commands, "",
             f"gemm.hip code digest (sha256[:16], comments and whitespace ignored) = {source_hash()}", "",
             "## Kernel trace (--kernel-trace --stats)", "",
             f"{'kernel':72s} {'calls':>5s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}"]
    for r in stats:
        lines.append(f"{short(r['Name'])[:72]:72s} {int(r['Calls']):5d} {float(r['AverageNs'])/1e3:9.2f} "
                     f"{float(r['MinNs'])/1e3:9.2f} {float(r['MaxNs'])/1e3:9.2f} {float(r['Percentage']):7.2f}")
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


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
             f"gemm.hip code digest (sha256[:16], comments and whitespace ignored) = {source_hash()}", "",
             "## Kernel trace (--kernel-trace --stats)", "",
             f"{'kernel':72s} {'calls':>5s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}"]
    for r in stats:
        lines.append(f"{short(r['Name'])[:72]:72s} {int(r['Calls']):5d} {float(r['AverageNs'])/1e3:9.1f} "
                     f"{float(r['MinNs'])/1e3:9.1f} {float(r['MaxNs'])/1e3:9.1f} {float(r['Percentage']):7.2f}")
    g_all = [r for r in stats if short(r["Name"]).startswith(GEMM_KERNELS)]
    if g_all:
        calls = sum(int(r["Calls"]) for r in g_all)
        tot_ns = sum(float(r["TotalDurationNs"]) for r in g_all)
        lines += ["", f"all GEMM launches: {calls} calls, average {tot_ns / calls / 1e3:.1f} us"]
    lines += ["", "## HBM bytes per launch (scaled counters), by kernel and grid size", "",
              f"{'kernel':60s} {'grid':>9s} {'read_MiB':>10s} {'write_MiB':>10s}"]
    for k in sorted(set(fb) | set(wb)):
        lines.append(f"{k[0][:60]:60s} {k[1]:9d} {fb.get(k, 0)/2**20:10.1f} {wb.get(k, 0)/2**20:10.1f}")
    path = os.path.join(ROOT, "profiles", f"kernels_{workload}.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    # traffic for the GEMM launches of one step, per launch (mean over launches)
    launches = collections.Counter()
    for (n, g, c), v in fetch.items():
        if n.startswith(GEMM_KERNELS) and c == "FETCH_SIZE":
            launches[(n, g)] += len(v)
    tot = sum(launches.values())
    if not tot:
        print(path)
        return
    mean_read = sum(fb[k] * launches[k] for k in launches) / tot
    mean_write = sum(wb.get(k, 0) * launches[k] for k in launches) / tot
    json.dump({"workload": workload, "gemm_code_digest_16": source_hash(),
               "bytes_per_launch": mean_read + mean_write, "read_bytes_per_launch": mean_read,
               "write_bytes_per_launch": mean_write, "fetch_scale": f_fetch, "write_scale": f_write},
              open(os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}.json"), "w"), indent=1)
    print(path)


COUNTERS_P1 = ("GRBM_GUI_ACTIVE SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES "
               "SQ_INSTS_VALU SQ_ACTIVE_INST_VALU")
COUNTERS_P2 = ("GRBM_GUI_ACTIVE SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_VALU_MFMA_COEXEC_CYCLES "
               "SQ_WAIT_INST_ANY SQ_INSTS_SALU SQ_ACTIVE_INST_ANY")
N_SIMD = 1024     # 256 CUs x 4 SIMDs
N_XCD = 8
MFMA_MACS = 32 * 32 * 16  # v_mfma_f32_32x32x16_f16


def dispatches(db_dir: str):
    """[(kernel, grid, duration_ns, {counter: value})] in dispatch order."""
    db = glob.glob(os.path.join(db_dir, "**", "*.db"), recursive=True)[0]
    con = sqlite3.connect(db)
    meta = {d: (n, g, t) for d, n, g, t in con.execute("select dispatch_id, name, grid_x, duration from kernels")}
    ev = collections.defaultdict(dict)
    for d, cn, v in con.execute("select dispatch_id, counter_name, counter_value from pmc_events"):
        ev[d][cn] = ev[d].get(cn, 0.0) + v
    return [(short(meta[d][0]), meta[d][1], meta[d][2], ev[d]) for d in sorted(ev)]


def counters_main(run: str, workload: str):
    p1, p2 = dispatches(os.path.join(run, "p1")), dispatches(os.path.join(run, "p2"))
    if [(a[0], a[1]) for a in p1] != [(b[0], b[1]) for b in p2]:
        raise SystemExit("the two passes dispatched different kernels")
    gemm = lambda n: n.startswith(GEMM_KERNELS)
    tflop = lambda c: 2.0 * MFMA_MACS * c["SQ_INSTS_MFMA"] / 1e12
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for i, ((n, g, t1, c1), (_, _, t2, c2)) in enumerate(zip(p1, p2)):
        if gemm(n):
            label = f"{n} : {tflop(c1):.3f} TFLOP"
        else:
            # an activation's amax and quantize launches precede its GEMM;
            # the set-up quantization of a weight is followed by the next one
            j = i + (1 if n.startswith("quantize") else 2)
            nxt = p1[j] if j < len(p1) and gemm(p1[j][0]) else None
            label = f"{n} : input of the {tflop(nxt[3]):.3f} TFLOP GEMM" if nxt else f"{n} : weights (set-up)"
        r = agg[label]
        r["us"].append((t1 + t2) / 2e3)
        for k, v in c1.items():
            r[k].append(v)
        for k, v in c2.items():
            r[k + "/2"].append(v)
    mean = lambda r, k: sum(r[k]) / len(r[k])
    hdr = ["kernel : launch", "calls", "avg us", "clock GHz", "MFMA instr", "cycles/MFMA", "MFMA busy %",
           "co-exec %", "VALU/MFMA", "LDS conflict/instr", "wait %"]
    rows = []
    for label in sorted(agg):
        r = agg[label]
        us = mean(r, "us")
        cyc = (mean(r, "GRBM_GUI_ACTIVE") + mean(r, "GRBM_GUI_ACTIVE/2")) / 2 / N_XCD
        mf, busy = mean(r, "SQ_INSTS_MFMA"), mean(r, "SQ_VALU_MFMA_BUSY_CYCLES")
        valu, lds = mean(r, "SQ_INSTS_VALU"), mean(r, "SQ_INSTS_LDS/2")
        conf, coex = mean(r, "SQ_LDS_BANK_CONFLICT/2"), mean(r, "SQ_VALU_MFMA_COEXEC_CYCLES/2")
        wait, wc = mean(r, "SQ_WAIT_INST_ANY/2"), mean(r, "SQ_WAVE_CYCLES")
        rows.append([label, str(len(r["us"])), f"{us:.1f}", f"{cyc / (us * 1e3):.2f}", f"{mf:.0f}",
                     f"{busy / mf:.1f}" if mf else "-", f"{100 * busy / (N_SIMD * cyc):.1f}" if mf else "-",
                     f"{100 * coex / busy:.1f}" if busy else "-",
                     f"{valu / mf:.2f}" if mf else f"{valu:.0f} VALU", f"{conf / lds:.2f}" if lds else "-",
                     f"{100 * wait / wc:.1f}" if wc else "-"])
    w = [max(len(hdr[i]), *(len(x[i]) for x in rows)) for i in range(len(hdr))]
    commands = open(os.path.join(run, "commands.txt")).read().strip()
    lines = [f"# rocprofv3 counters: {workload} (MFMA, VALU and LDS per kind of launch)", "",
             "Commands (run from the repository root on one MI355X; two passes with their own counter sets):", "",
             commands, f"python3 profile_summary.py --counters <out> {workload}", "",
             f"gemm.hip code digest (sha256[:16], comments and whitespace ignored) = {source_hash()}", "",
             "Averages over the profiled run's dispatches.  GEMM launches are named by their work",
             "(2 x 32 x 32 x 16 flop per MFMA instruction); quantizer launches by the GEMM they feed.",
             "Reading of the counters:",
             f"- SQ_VALU_MFMA_BUSY_CYCLES is summed over the {N_SIMD} SIMDs; per SQ_INSTS_MFMA it is the pipe time",
             "  of one v_mfma_f32_32x32x16_f16 in cycles (cycles/MFMA).",
             f"- GRBM_GUI_ACTIVE is summed over the {N_XCD} XCDs: GRBM/{N_XCD} over the duration is the clock.  For",
             "  launches of a few microseconds it also counts the profiler's per-dispatch overhead, so their",
             "  clock column is not a clock.",
             f"- MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / ({N_SIMD} x GRBM/{N_XCD}), the share of SIMD-cycles with the",
             "  MFMA pipe busy; it equals the achieved flops over the peak at the clock the launch ran at.",
             "- co-exec % = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (VALU issued while the pipe ran).",
             "- VALU/MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA in wave instructions (kernels without MFMA: the count).",
             "- LDS conflict/instr = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS (cycles).",
             "- wait % = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (waves waiting on memory, LDS or MFMA results).", "",
             " | ".join(h.ljust(w[i]) for i, h in enumerate(hdr)),
             "-|-".join("-" * x for x in w)]
    lines += [" | ".join(c.ljust(w[i]) for i, c in enumerate(x)).rstrip() for x in rows]
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


def peak_main(run: str):
    """profiles/mfma_peak.txt from a `rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE` run of
    `bench.py --peak` (the fp16 MFMA rate kernel with 0, 4 and 6 VALU per MFMA)."""
    rows = collections.defaultdict(list)
    for n, g, dur, c in dispatches(os.path.join(run, "peak")):
        if "mfma_peak_kernel" in n:
            rows[n].append((g, dur, c.get("GRBM_GUI_ACTIVE", 0.0)))
    commands = open(os.path.join(run, "commands.txt")).read().strip()
    lines = ["# rocprofv3: fp16 MFMA rate kernel (bench.py --peak)", "",
             "Commands (run from the repository root on one MI355X):", "", commands,
             "python3 profile_summary.py --peak <out>", "",
             "Each launch: one workgroup of four waves per CU, every wave 20000 x 32 v_mfma_f32_32x32x16_f16",
             "(32768 flop each) on register operands, with 0, 4 or 6 VALU instructions per MFMA (the",
             "dequantization the prefill GEMM issues is 4).  clock = GRBM_GUI_ACTIVE / 8 XCDs / duration;",
             f"peak at clock = {N_SIMD} SIMDs x 1024 flop/cycle x clock (the 2.5 PF/s datasheet figure is 2.4 GHz).", "",
             f"{'kernel':34s} {'calls':>5s} {'avg_us':>9s} {'TFLOP/s':>8s} {'clock_GHz':>9s} {'peak@clk':>9s} {'busy%':>6s}"]
    for n in sorted(rows):
        r = rows[n]
        grid = r[0][0]
        blocks = grid // 256 if grid >= 256 else grid
        flops = blocks * 4 * 20000 * 32 * 32768
        us = sum(x[1] for x in r) / len(r) / 1e3
        ghz = sum(x[2] / 8 / x[1] for x in r) / len(r)
        tf = flops / (us * 1e-6) / 1e12
        at = N_SIMD * 1024 * ghz * 1e9 / 1e12
        lines.append(f"{n[:34]:34s} {len(r):5d} {us:9.1f} {tf:8.1f} {ghz:9.3f} {at:9.1f} {100 * tf / at:6.1f}")
    path = os.path.join(ROOT, "profiles", "mfma_peak.txt")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--counters":
        counters_main(sys.argv[2], sys.argv[3])
    elif len(sys.argv) > 1 and sys.argv[1] == "--trace":
        trace_main(sys.argv[2], sys.argv[3])
    elif len(sys.argv) > 1 and sys.argv[1] == "--peak":
        peak_main(sys.argv[2])
    else:
        main()
