"""Summaries of rocprofv3 output for the library's kernels.

    python -m exact_io_aware_07_amd.profiling stats CSV --cmd "..." --out FILE.md
    python -m exact_io_aware_07_amd.profiling traffic --fetch CSV --write CSV \
        --copy-fetch CSV --copy-write CSV --copy-bytes N --workload NAME \
        --cmd "..." --out-md FILE.md --out-json profiles/traffic.json

    python -m exact_io_aware_07_amd.profiling counters CSV [CSV ...] --workload NAME \
        --cmd "..." --out FILE.md

``stats`` turns a ``--kernel-trace --stats`` kernel_stats.csv into a short
markdown table. ``counters`` merges ``--pmc`` passes (one CSV each) into one
table per kernel: MFMA-busy share of SIMD cycles, share of CU cycles with a
wave resident, share of SIMD cycles with MFMA and VALU both executing, share
of wave cycles issuing VALU, waiting (s_waitcnt, barriers) or waiting to
issue (dependencies, arbitration), LDS
bank-conflict cycles per LDS-active cycle, L2 hit rate, and VALU /
transcendental / LDS instructions per MFMA instruction. ``traffic`` turns two ``--pmc`` runs (FETCH_SIZE, then
WRITE_SIZE, KiB per dispatch) into HBM bytes per launch, each counter scaled
by what it reads for a plain device copy of known size, and records the hash
of the kernel sources the counters were taken on, so a stale figure is
never reported for a changed kernel; the JSON file keeps one record per
workload.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
from typing import Dict, List

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# short name -> (substring of the demangled kernel name, defining source)
KERNELS = {
    "fwd": ("fwd_mfma_kernel", "fa_fwd_mfma.hip"),
    "dsum": ("dsum_kernel", "fa_bwd_mfma.hip"),
    "dkdv": ("dkdv_kernel", "fa_bwd_mfma.hip"),
    "dq": ("dq_kernel", "fa_bwd_mfma.hip"),
    "dkv_reduce": ("dkv_reduce_kernel", "fa_bwd_mfma.hip"),
    "merge": ("merge_kernel", "fa_merge.hip"),
    "fp8_attn": ("fwd_fp8_kernel", "fa_fp8.hip"),
    "fp8_qk": ("fp8_qk_kernel", "fa_fp8.hip"),
    "fp8_v": ("fp8_v_kernel", "fa_fp8.hip"),
}


def source_sha(short: str) -> str:
    """sha256 of the source that defines kernel ``short`` plus the shared header."""
    h = hashlib.sha256()
    for f in (KERNELS[short][1], "fa_internal.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(kernel_name: str) -> str:
    for short, (sub, _) in KERNELS.items():
        if f"::{sub}<" in kernel_name or kernel_name.startswith(sub):
            return short
    return kernel_name


def _counter_means(path: str, counter: str) -> Dict[str, float]:
    vals: Dict[str, List[float]] = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def _copy_factor(path: str, counter: str, nbytes: int) -> float:
    means = _counter_means(path, counter)
    copies = [v for k, v in means.items() if "copy" in k.lower()]
    if not copies:
        raise SystemExit(f"no copy kernel found in {path}")
    return nbytes / (max(copies) * 1024.0)


def stats_md(csv_path: str, cmd: str) -> str:
    lines = ["# Kernel time (rocprofv3 --kernel-trace --stats)", "", "Command:", "", "```",
             cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    with open(csv_path) as fh:
        for r in csv.DictReader(fh):
            lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
    return "\n".join(lines) + "\n"


# Every XCD has its own GRBM and SQs, and rocprofv3 sums each counter over
# the eight: GRBM_GUI_ACTIVE reads eight times the kernel's cycles, and
# SQ_BUSY_CU_CYCLES / GRBM_GUI_ACTIVE comes to about 30 on full-chip kernels
# (32 CUs per GRBM). So per-CU and per-SIMD ratios divide the GRBM count by
# the units of one XCD.
CUS_PER_XCD = 32
SIMDS_PER_CU = 4

# derived ratio -> (numerator, denominator[, units the denominator counts])
RATIOS = {
    "MFMA busy / SIMD cycles": ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", CUS_PER_XCD * SIMDS_PER_CU),
    "CUs with a wave / CU cycles": ("SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE", CUS_PER_XCD),
    "MFMA and VALU together / SIMD cycles": ("SQ_VALU_MFMA_COEXEC_CYCLES", "GRBM_GUI_ACTIVE",
                                             CUS_PER_XCD * SIMDS_PER_CU),
    "VALU issuing / wave cycles": ("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
    "waiting (s_waitcnt, barrier) / wave cycles": ("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
    "LDS issuing / wave cycles": ("SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
    "waiting to issue / wave cycles": ("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    "LDS bank-conflict / LDS-active cycles": ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
    "VALU insts / MFMA inst": ("SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
    "transcendental insts / MFMA inst": ("SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA"),
    "LDS insts / MFMA inst": ("SQ_INSTS_LDS", "SQ_INSTS_MFMA"),
}


def counters_md(paths: List[str], workload: str, cmd: str) -> str:
    per: Dict[str, Dict[str, float]] = collections.defaultdict(dict)
    for path in paths:
        vals: Dict[tuple, List[float]] = collections.defaultdict(list)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                short = short_name(r["Kernel_Name"])
                if short in KERNELS:
                    vals[(short, r["Counter_Name"])].append(float(r["Counter_Value"]))
        for (short, c), v in vals.items():
            per[short][c] = sum(v) / len(v)
    lines = ["# Shader counters per kernel (rocprofv3 --pmc)", "", f"Workload: `{workload}`.", "",
             "Commands (one pass each):", "", "```", cmd, "```", "",
             "| kernel | " + " | ".join(RATIOS) + " | L2 hit rate |",
             "|---|" + "---|" * (len(RATIOS) + 1)]
    for short in sorted(per):
        c = per[short]
        cells = []
        for num, den, *units in RATIOS.values():
            n_units = units[0] if units else 1
            cells.append(f"{c[num] / (c[den] * n_units):.3f}" if num in c and c.get(den) else "—")
        hit = c.get("TCC_HIT_sum", c.get("TCC_HIT"))
        miss = c.get("TCC_MISS_sum", c.get("TCC_MISS"))
        cells.append(f"{hit / (hit + miss):.3f}" if hit is not None and miss is not None and hit + miss > 0 else "—")
        lines.append(f"| `{short}` | " + " | ".join(cells) + " |")
    lines += ["", "Raw means per dispatch:", "", "| kernel | counter | value |", "|---|---|---|"]
    for short in sorted(per):
        for cname, v in sorted(per[short].items()):
            lines.append(f"| `{short}` | {cname} | {v:.4g} |")
    return "\n".join(lines) + "\n"


def traffic(args) -> None:
    ff = _copy_factor(args.copy_fetch, "FETCH_SIZE", args.copy_bytes)
    fw = _copy_factor(args.copy_write, "WRITE_SIZE", args.copy_bytes)
    fetch = _counter_means(args.fetch, "FETCH_SIZE")
    write = _counter_means(args.write, "WRITE_SIZE")
    out = {"copy_bytes": args.copy_bytes, "fetch_scale": ff, "write_scale": fw, "cmd": args.cmd,
           "kernels": {}}
    md = ["# HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)", "",
          f"Workload: `{args.workload}`.", "", "Commands:", "", "```", args.cmd, "```", "",
          f"Scale factors from a plain {args.copy_bytes} B device copy (the copy reads and "
          f"writes exactly that many bytes): FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {fw:.4f}.", "",
          "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB |",
          "|---|---|---|---|---|"]
    for name in sorted(set(fetch) | set(write)):
        short = short_name(name)
        fb = fetch.get(name, 0.0) * 1024.0 * ff
        wb = write.get(name, 0.0) * 1024.0 * fw
        md.append(f"| `{short}` | {fetch.get(name, 0.0):.1f} | {write.get(name, 0.0):.1f} | "
                  f"{fb / 1e6:.2f} | {wb / 1e6:.2f} |")
        if short in KERNELS:
            out["kernels"][short] = {"workload": args.workload, "kernel_name": name,
                                     "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                                     "source_sha256": source_sha(short)}
    with open(args.out_md, "w") as fh:
        fh.write("\n".join(md) + "\n")
    # one record per workload; records of other workloads are kept
    try:
        with open(args.out_json) as fh:
            allrec = json.load(fh)
        if "workloads" not in allrec:
            allrec = {"workloads": {}}
    except (OSError, ValueError):
        allrec = {"workloads": {}}
    allrec["workloads"][args.workload] = out
    with open(args.out_json, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
        fh.write("\n")


def traffic_record(path: str, workload: str, short: str):
    """(fetch, write) bytes per launch of kernel ``short`` on ``workload`` from
    a traffic file, or None when there is none or the kernel's source has
    changed since the counters were taken."""
    try:
        with open(path) as fh:
            rec = json.load(fh)["workloads"][workload]["kernels"][short]
    except (OSError, KeyError, ValueError, TypeError):
        return None
    if rec.get("source_sha256") != source_sha(short):
        return None
    return rec.get("fetch_bytes_per_launch", 0.0), rec.get("write_bytes_per_launch", 0.0)


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for name in ("fetch", "write", "copy_fetch", "copy_write", "workload", "cmd", "out_md", "out_json"):
        t.add_argument("--" + name.replace("_", "-"), dest=name, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--workload", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "stats":
        with open(a.out, "w") as fh:
            fh.write(stats_md(a.csv, a.cmd))
    elif a.what == "counters":
        with open(a.out, "w") as fh:
            fh.write(counters_md(a.csv, a.workload, a.cmd))
    else:
        traffic(a)


if __name__ == "__main__":
    main()
