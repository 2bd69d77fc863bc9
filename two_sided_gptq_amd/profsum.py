"""Summarise rocprofv3 output of the benchmark into a short markdown profile.

    python -m two_sided_gptq_amd.profsum --trace DIR --pmc DIR --out profiles/X.md

DIR of --trace holds `bench_kernel_trace.csv` and `bench_kernel_stats.csv`
(`rocprofv3 --kernel-trace --stats --output-format csv -o bench`); DIR of --pmc
holds `FETCH_SIZE/run_counter_collection.csv` and `WRITE_SIZE/...` (one
`rocprofv3 --pmc <counter> -o run` pass each, with `bench.py --copy-probe`)
and, when present, `MFMA/...` (SQ_VALU_MFMA_BUSY_CYCLES,
SQ_INSTS_VALU_MFMA_MOPS_F32 and GRBM_GUI_ACTIVE in one pass) and `MfmaUtil/...`
(rocprofv3's derived utilisation, a pass of its own).

HBM bytes per dispatch: FETCH_SIZE and WRITE_SIZE (KiB) are each scaled so that
the 1 GiB device copy the benchmark runs with --copy-probe reads and writes
exactly 1 GiB.  MFMA work per dispatch: SQ_INSTS_VALU_MFMA_MOPS_F32 counts
fp32 MFMA flops in units of 512; SQ_VALU_MFMA_BUSY_CYCLES counts the cycles
each SIMD's matrix unit is busy (64 per v_mfma_f32_32x32x2f32, 4096 flops, so
the two agree at 64 flops per busy cycle, the fp32 matrix rate of one SIMD).
The busy share of a kernel is its busy cycles over 1024 SIMDs x its average
duration x 2.4 GHz, i.e. its counted MFMA rate over the fp32 MFMA peak.
rocprofv3's MfmaUtil divides by GRBM_GUI_ACTIVE instead, which for dispatches
of some tens of microseconds also spans the counter collection around them.
The summary records a hash of the kernel source; `bench.py` reports the
measured figures only while the source still has that hash.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(HERE, "csrc", "quantize.hip")
COPY_BYTES = 1 << 30
SIMDS = 256 * 4
CLOCK_HZ = 2.4e9
MFMA_KERNELS = ("band_gemm_kernel", "band_side_kernel", "leaf_kernel<false>", "leaf_kernel<true>")


def source_hash(path: str = KERNEL_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def short_name(n: str) -> str:
    m = re.match(r"(?:void )?(?:[\w:]*\(anonymous namespace\)::)?([\w:<>, ]+?)\(", n)
    return m.group(1) if m else n[:48]


def _windows(rows):
    """The last timed graph solve, the timing pass after it (the same plan in
    order on one stream), each from its first parameter kernel to its final
    reduction, and the band replays that follow (the critical band launches
    alone, then the deferred ones), from which the benchmark takes the band
    kernels' average launch durations.  A solve with a side stream launches its
    parameter kernel twice (the first tile rows, then the rest beside the first
    leaves), so solves are told apart by their final reductions."""
    rows = sorted(rows, key=lambda r: int(r["Start_Timestamp"]))
    fin = [i for i, r in enumerate(rows) if "sumsq_final_kernel" in r["Kernel_Name"]]
    if len(fin) >= 2:
        def start(after):
            return next(i for i in range(after + 1, len(rows)) if "qparams_kernel" in rows[i]["Kernel_Name"])
        g0, t0 = start(fin[-3] if len(fin) >= 3 else -1), start(fin[-2])
        return rows[g0:fin[-2] + 1], rows[t0:fin[-1] + 1], rows[fin[-1] + 1:]
    q = [i for i, r in enumerate(rows) if "qparams_kernel" in r["Kernel_Name"]]
    if len(q) < 2:
        return rows, rows, []
    end = next((i for i in range(q[-1], len(rows)) if "sumsq_final_kernel" in rows[i]["Kernel_Name"]),
               len(rows) - 1)
    return rows[q[-2]:q[-1]], rows[q[-1]:end + 1], rows[end + 1:]


def _table(out, win, title):
    per = collections.defaultdict(list)
    for r in win:
        per[short_name(r["Kernel_Name"])].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    span = max(int(r["End_Timestamp"]) for r in win) - int(win[0]["Start_Timestamp"])
    out.append(f"### {title}: {span / 1e3:.1f} us over {len(win)} dispatches\n")
    out.append("| kernel | launches | total us | avg us | min us | max us |")
    out.append("|---|---|---|---|---|---|")
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| {k} | {len(v)} | {sum(v) / 1e3:.1f} | {statistics.mean(v) / 1e3:.2f} | "
                   f"{min(v) / 1e3:.2f} | {max(v) / 1e3:.2f} |")
    out.append("")


def _factor_windows(rows):
    """The factor calls in a benchmark trace: each runs from its
    load_reversed_kernel to its write_l_kernel (the side stream's products fall
    inside that span).  The benchmark calls the input side's factor twice (one
    warm-up, one timed), then the output side's."""
    rows = sorted(rows, key=lambda r: int(r["Start_Timestamp"]))
    wins, start = [], None
    for i, r in enumerate(rows):
        if "load_reversed_kernel" in r["Kernel_Name"]:
            start = i
        elif "write_l_kernel" in r["Kernel_Name"] and start is not None:
            wins.append(rows[start:i + 1])
            start = None
    return wins


def summarise(trace_dir: str, pmc_dir: str, command: str, pmc_command: str,
              mfma_command: str = "") -> str:
    out = []
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "bench_kernel_trace.csv"))))
    graph_win, timing_win, replay_win = _windows(rows)
    out.append(f"Kernel trace command: `{command}`\n")
    _table(out, graph_win, "One timed solve (graph replay; deferred products overlap the leaves)")
    _table(out, timing_win, "Timing pass (the same plan in order on one stream, an event after every step)")
    if replay_win:
        _table(out, replay_win, "Band replays (critical, then deferred launches alone; bench.py's band averages)")
    fwins = _factor_windows(rows)
    if len(fwins) >= 2:
        _table(out, fwins[1], "One bakron_factor call (the input side's timed call; T products on a side stream)")
    out.append("\n### rocprofv3 --stats (whole command)\n")
    out.append("| kernel | calls | average ns | % |")
    out.append("|---|---|---|---|")
    avg_ns = {}
    for r in csv.DictReader(open(os.path.join(trace_dir, "bench_kernel_stats.csv"))):
        avg_ns[short_name(r["Name"])] = float(r["AverageNs"])
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                   f"{float(r['Percentage']):.2f} |")
    # counters
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        for r in csv.DictReader(open(os.path.join(pmc_dir, c, "run_counter_collection.csv"))):
            vals[short_name(r["Kernel_Name"])][c].append(float(r["Counter_Value"]))
    copies = vals.get("__amd_rocclr_copyBuffer", {})
    f_copy = max(copies.get("FETCH_SIZE", [0.0]))
    w_copy = max(copies.get("WRITE_SIZE", [0.0]))
    f_scale = COPY_BYTES / (f_copy * 1024) if f_copy else float("nan")
    w_scale = COPY_BYTES / (w_copy * 1024) if w_copy else float("nan")
    out.append(f"\n### HBM bytes (counter command: `{pmc_command}`)\n")
    out.append(f"1 GiB copy probe: FETCH_SIZE {f_copy:.0f} KiB, WRITE_SIZE {w_copy:.0f} KiB "
               f"-> scale x{f_scale:.3f} (fetch), x{w_scale:.3f} (write).\n")
    out.append("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes per dispatch (scaled) |")
    out.append("|---|---|---|---|---|")
    traffic = {}
    for k, d in vals.items():
        if not d.get("FETCH_SIZE") or not d.get("WRITE_SIZE"):
            continue
        f = statistics.mean(d["FETCH_SIZE"])
        w = statistics.mean(d["WRITE_SIZE"])
        b = (f * f_scale + w * w_scale) * 1024
        traffic[k] = b
        out.append(f"| {k} | {len(d['FETCH_SIZE'])} | {f:.1f} | {w:.1f} | {b:.4g} |")
    mfma = _mfma_section(out, pmc_dir, avg_ns, mfma_command)
    out.append("\nMachine-readable (read by bench.py):\n")
    out.append(f"    source_sha256_16: {source_hash()}")
    for k in MFMA_KERNELS:
        if k in traffic:
            out.append(f"    traffic_bytes_per_dispatch: {k} {traffic[k]:.6g}")
    for k in MFMA_KERNELS:
        if k in mfma:
            out.append(f"    mfma_flops_per_dispatch: {k} {mfma[k]:.6g}")
    return "\n".join(out) + "\n"


def _per_kernel(path):
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        vals[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return vals


def _mfma_section(out, pmc_dir, avg_ns, command):
    """Counted fp32 MFMA flops and busy cycles per dispatch of each kernel that
    issues MFMA; returns {kernel: counted flops per dispatch}."""
    path = os.path.join(pmc_dir, "MFMA", "run_counter_collection.csv")
    if not os.path.exists(path):
        return {}
    vals = _per_kernel(path)
    upath = os.path.join(pmc_dir, "MfmaUtil", "run_counter_collection.csv")
    util = _per_kernel(upath) if os.path.exists(upath) else {}
    out.append(f"\n### MFMA work (counter command: `{command}`)\n")
    out.append("Busy share = busy cycles / (1024 SIMDs x kernel average duration from the trace x 2.4 GHz).\n")
    out.append("| kernel | dispatches | fp32 MFMA flops (MOPS_F32 x 512) | MFMA busy cycles | "
               "flops / busy cycle / SIMD | avg us (trace) | busy share | rocprofv3 MfmaUtil % |")
    out.append("|---|---|---|---|---|---|---|---|")
    flops = {}
    for k, d in vals.items():
        mops = d.get("SQ_INSTS_VALU_MFMA_MOPS_F32")
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES")
        if not mops or not busy or statistics.mean(mops) == 0:
            continue  # no fp32 MFMA (the factor's fp64 products count elsewhere)
        f = statistics.mean(mops) * 512
        b = statistics.mean(busy)
        flops[k] = f
        avg = avg_ns.get(k)
        share = f"{b / (SIMDS * avg * 1e-9 * CLOCK_HZ):.3f}" if avg else "-"
        u = util.get(k, {}).get("MfmaUtil")
        out.append(f"| {k} | {len(mops)} | {f:.4g} | {b:.4g} | {f / b:.1f} | "
                   f"{avg / 1e3 if avg else float('nan'):.2f} | {share} | "
                   f"{statistics.mean(u) if u else float('nan'):.1f} |")
    return flops


def read_figure(md_path: str, key: str, kernel: str):
    """A per-dispatch figure (`key`: traffic_bytes_per_dispatch or
    mfma_flops_per_dispatch) of `kernel` from a summary, or None when the
    summary is missing, lacks it or was taken from a different kernel source."""
    try:
        text = open(md_path).read()
    except OSError:
        return None
    m = re.search(r"source_sha256_16: (\w+)", text)
    if not m or m.group(1) != source_hash():
        return None
    m = re.search(re.escape(key) + r": " + re.escape(kernel) + r" ([\d.e+]+)", text)
    return float(m.group(1)) if m else None


def read_traffic(md_path: str, kernel: str):
    """HBM bytes per dispatch of `kernel` (see read_figure)."""
    return read_figure(md_path, "traffic_bytes_per_dispatch", kernel)


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--trace", required=True)
    p.add_argument("--pmc", required=True)
    p.add_argument("--out", required=True)
    p.add_argument("--command", default="rocprofv3 --kernel-trace --stats --output-format csv "
                   "-d <trace dir> -o bench -- python3 bench.py --steps 3 --warmup 1 --cpu-sample 0")
    p.add_argument("--pmc-command", default="rocprofv3 --pmc <FETCH_SIZE|WRITE_SIZE> --output-format csv "
                   "-d <pmc dir>/<counter> -o run -- python3 bench.py --steps 1 --warmup 0 "
                   "--cpu-sample 0 --copy-probe")
    p.add_argument("--mfma-command", default="rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                   "SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE (then, in a run of its own, MfmaUtil) "
                   "--output-format csv -d <pmc dir>/<MFMA|MfmaUtil> -o run -- python3 bench.py "
                   "--steps 1 --warmup 0 --cpu-sample 0")
    a = p.parse_args()
    text = summarise(a.trace, a.pmc, a.command, a.pmc_command, a.mfma_command)
    with open(a.out, "w") as f:
        f.write(text)
    print(a.out)


if __name__ == "__main__":
    main()
