"""Summaries of rocprofv3 output for the benchmark (measurement tooling).

Reads the CSV files rocprofv3 writes (``--kernel-trace --stats`` and
``--pmc`` passes with ``--output-format csv``), averages counters per kernel
dispatch, scales the HBM byte counters by what the same counters read for a
plain device copy of known size, and writes short text summaries.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict
from typing import Dict, List


def kernel_short_name(name: str) -> str:
    m = re.search(r"(k_\w+)(<[^>]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return name.split("(")[0].strip()[:60]


def kernel_stats(trace_dir: str) -> List[dict]:
    files = glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))
    if not files:
        return []
    out = []
    for r in csv.DictReader(open(files[0])):
        out.append({
            "kernel": kernel_short_name(r["Name"]),
            "calls": int(r["Calls"]),
            "avg_us": float(r["AverageNs"]) / 1e3,
            "min_us": float(r["MinNs"]) / 1e3,
            "max_us": float(r["MaxNs"]) / 1e3,
            "percent": float(r["Percentage"]),
        })
    return out


def counters_per_dispatch(pmc_dir: str) -> Dict[str, Dict[str, float]]:
    """kernel -> counter -> mean value per dispatch (summed over dimensions)."""
    per = defaultdict(lambda: defaultdict(float))
    names = {}
    for f in glob.glob(os.path.join(pmc_dir, "*counter_collection.csv")):
        for r in csv.DictReader(open(f)):
            per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = kernel_short_name(r["Kernel_Name"])
    acc = defaultdict(lambda: defaultdict(list))
    for d, cs in per.items():
        for c, v in cs.items():
            acc[names[d]][c].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


COMPUTE_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                    "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_WAVE_CYCLES "
                    "SQ_WAVES GRBM_GUI_ACTIVE")
N_CU, N_SIMD = 256, 1024


def compute_counters(pmc_dir: str) -> Dict[str, dict]:
    """Per kernel: mean counters per dispatch and mean duration, from a
    `--pmc <COMPUTE_COUNTERS> --kernel-trace` run, with derived figures:
    MFMA busy fraction (MFMA-busy cycles per SIMD over CU-busy cycles per
    CU), effective shader clock (CU-busy cycles per CU over the dispatch's
    duration) and MFMA TFLOP/s (MOPS count units of 512 flops)."""
    per = counters_per_dispatch(pmc_dir)
    durs = defaultdict(list)
    for f in glob.glob(os.path.join(pmc_dir, "*kernel_trace.csv")):
        for r in csv.DictReader(open(f)):
            durs[kernel_short_name(r["Kernel_Name"])].append(
                (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3)
    out = {}
    for k, cs in per.items():
        d = sum(durs[k]) / len(durs[k]) if durs.get(k) else None
        e = {"counters": cs, "duration_us": d}
        busy = cs.get("SQ_BUSY_CU_CYCLES", 0.0) / N_CU
        mfma = cs.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / N_SIMD
        if busy > 0:
            e["mfma_busy_frac"] = mfma / busy
        if d:
            e["shader_clock_ghz"] = busy / (d * 1e3)
            e["mfma_tflops"] = cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / (d * 1e-6) / 1e12
        out[k] = e
    return out


def copy_factor(pmc_dir: str, counter: str, copy_bytes: int) -> float:
    """Counter reading (KiB) per byte actually moved, from the copy kernel."""
    cs = counters_per_dispatch(pmc_dir)
    vals = [v[counter] for k, v in cs.items() if "copyBuffer" in k and counter in v]
    if not vals:
        raise ValueError("no copy kernel in " + pmc_dir)
    return max(vals) * 1024.0 / copy_bytes


def summarize(root: str, out_dir: str, bench_cmd: str, copy_mib: int, gemm_source: str,
              workload: str) -> dict:
    """Write the kernel-trace and traffic summaries for one profiling run.

    root holds trace/, fetch/, write/, cfetch/, cwrite/ (rocprofv3 -d dirs)."""
    os.makedirs(out_dir, exist_ok=True)
    stats = kernel_stats(os.path.join(root, "trace"))
    fetch = counters_per_dispatch(os.path.join(root, "fetch"))
    write = counters_per_dispatch(os.path.join(root, "write"))
    copy_bytes = copy_mib << 20
    f_fac = copy_factor(os.path.join(root, "cfetch"), "FETCH_SIZE", copy_bytes)
    w_fac = copy_factor(os.path.join(root, "cwrite"), "WRITE_SIZE", copy_bytes)
    lines = ["# Kernel trace and HBM traffic: %s" % workload, ""]
    lines.append("Commands (run from the repository root on one MI355X; `cd /tmp` and "
                 "`TMPDIR=/tmp` first):")
    lines.append("")
    for sub, extra in (("trace", "--kernel-trace --stats"), ("fetch", "--pmc FETCH_SIZE"),
                       ("write", "--pmc WRITE_SIZE")):
        lines.append("    rocprofv3 %s --output-format csv -d <out>/%s -o %s -- %s" %
                     (extra, sub, sub, bench_cmd))
    for sub, c in (("cfetch", "FETCH_SIZE"), ("cwrite", "WRITE_SIZE")):
        lines.append("    rocprofv3 --pmc %s --output-format csv -d <out>/%s -o %s -- "
                     "python3 bench.py --copy-calibration %d" % (c, sub, sub, copy_mib))
    lines += ["", "## Kernel durations (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | max us | % |", "|---|---|---|---|---|---|"]
    for s in stats:
        lines.append("| %s | %d | %.2f | %.2f | %.2f | %.1f |" % (s["kernel"], s["calls"], s["avg_us"],
                                                               s["min_us"], s["max_us"], s["percent"]))
    lines += ["", "## HBM traffic per dispatch (FETCH_SIZE / WRITE_SIZE)", "",
              "Counter calibration: for a %d MiB device copy, FETCH_SIZE reads %.3f x and "
              "WRITE_SIZE %.3f x the bytes the copy moved; kernel bytes below = counter KiB x "
              "1024 / that factor." % (copy_mib, f_fac, w_fac), "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB |",
              "|---|---|---|---|---|"]
    traffic = {}
    for k in sorted(set(fetch) | set(write)):
        fk = fetch.get(k, {}).get("FETCH_SIZE", 0.0)
        wk = write.get(k, {}).get("WRITE_SIZE", 0.0)
        fb = fk * 1024.0 / f_fac
        wb = wk * 1024.0 / w_fac
        traffic[k] = {"fetch_bytes": fb, "write_bytes": wb}
        lines.append("| %s | %.1f | %.1f | %.2f | %.2f |" % (k, fk, wk, fb / 1e6, wb / 1e6))
    cdir = os.path.join(root, "compute")
    compute = compute_counters(cdir) if os.path.isdir(cdir) else {}
    if compute:
        lines += ["", "## MFMA, clock and LDS counters per dispatch", "",
                  "    rocprofv3 --kernel-trace --pmc %s --output-format csv -d <out>/compute "
                  "-o compute -- %s" % (COMPUTE_COUNTERS, bench_cmd), "",
                  "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / %d SIMDs over SQ_BUSY_CU_CYCLES / %d CUs; "
                  "shader clock = SQ_BUSY_CU_CYCLES / %d CUs over the dispatch duration of the same "
                  "run; MFMA TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops over the duration."
                  % (N_SIMD, N_CU, N_CU), "",
                  "| kernel | us (this run) | MFMA busy | shader clock GHz | MFMA TFLOP/s | "
                  "LDS active cyc / CU | LDS bank-conflict cyc / CU | waves |",
                  "|---|---|---|---|---|---|---|---|"]
        for k, e in sorted(compute.items(), key=lambda kv: -(kv[1]["duration_us"] or 0)):
            c = e["counters"]
            lines.append("| %s | %s | %s | %s | %s | %.0f | %.0f | %.0f |" % (
                k, "%.2f" % e["duration_us"] if e["duration_us"] else "-",
                "%.3f" % e["mfma_busy_frac"] if "mfma_busy_frac" in e else "-",
                "%.2f" % e["shader_clock_ghz"] if "shader_clock_ghz" in e else "-",
                "%.1f" % e["mfma_tflops"] if "mfma_tflops" in e else "-",
                c.get("SQ_LDS_IDX_ACTIVE", 0) / N_CU, c.get("SQ_LDS_BANK_CONFLICT", 0) / N_CU,
                c.get("SQ_WAVES", 0)))
    md = os.path.join(out_dir, "c3_proj70b_kernels.md")
    open(md, "w").write("\n".join(lines) + "\n")
    # the headline step's GEMM: the split-K pairs with the shrink folded in
    # (template argument true), then the plain split, then unsplit tiles
    gemm = sorted((k for k in traffic if k.startswith("k_gemm_bf16_split<144") or
                   k.startswith("k_gemm_bf16_pipe")),
                  key=lambda k: (not k.startswith("k_gemm_bf16_split"), "true" not in k, k))
    result = {"workload": workload, "kernel_trace": stats, "traffic": traffic,
              "fetch_factor": f_fac, "write_factor": w_fac,
              "compute": {k: {kk: vv for kk, vv in e.items() if kk != "counters"}
                          for k, e in compute.items()}}
    if gemm:
        g = gemm[0]
        tj = {
            "kernel": g,
            "source": os.path.relpath(gemm_source, os.path.dirname(out_dir)),
            "source_sha256": hashlib.sha256(open(gemm_source, "rb").read()).hexdigest(),
            "bytes_per_launch": traffic[g]["fetch_bytes"] + traffic[g]["write_bytes"],
            "fetch_bytes_per_launch": traffic[g]["fetch_bytes"],
            "write_bytes_per_launch": traffic[g]["write_bytes"],
            "workload": workload,
            "command": bench_cmd,
        }
        json.dump(tj, open(os.path.join(out_dir, "traffic_c3_gemm.json"), "w"), indent=1)
        result["gemm_traffic"] = tj
    return result
