"""Summaries of rocprofv3 runs of the benchmark (kernel-trace statistics and the
FETCH_SIZE / WRITE_SIZE byte counters), written as short text under profiles/.

The byte counters are scaled by what the same counter reads for a plain device
copy of 256 MiB (``bench.py --calibrate-copy``): the copy reads and writes exactly
268435456 bytes, so ``factor = 262144 KiB / counter(copy)`` per counter.

Usage (from the repository root, after the three rocprofv3 runs):
    python -m quantized_decode_gemv_02_amd.profiling TRACE_DIR FETCH_DIR WRITE_DIR OUT.md OUT.json
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

COPY_BYTES = 256 << 20
COPY_KERNEL = "__amd_rocclr_copyBuffer"
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def kernel_source_sha() -> str:
    """Hash of the kernel sources, so a stored byte count is used only for the code it was taken on."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def _one(directory: str, pattern: str) -> str:
    """The one file matching `pattern` anywhere under `directory` (rocprofv3 may nest its output)."""
    hits = sorted(glob.glob(os.path.join(directory, "**", pattern), recursive=True))
    if len(hits) != 1:
        raise FileNotFoundError(f"{len(hits)} files match {pattern} under {directory}")
    return hits[0]


def kernel_stats(trace_dir: str) -> list[dict]:
    rows = list(csv.DictReader(open(_one(trace_dir, "*kernel_stats.csv"))))
    return [{"name": r["Name"], "calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
             "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]), "pct": float(r["Percentage"])} for r in rows]


def trace_by_grid(trace_dir: str) -> dict:
    """Mean / min / max duration (ns) and count per (kernel, total work-items) from the kernel trace."""
    acc = defaultdict(list)
    for r in csv.DictReader(open(_one(trace_dir, "*kernel_trace.csv"))):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        acc[(short(r["Kernel_Name"]), grid)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: (sum(v) / len(v), min(v), max(v), len(v)) for k, v in acc.items()}


def counters(pmc_dir: str) -> list[dict]:
    return list(csv.DictReader(open(_one(pmc_dir, "*counter_collection.csv"))))


def short(name: str) -> str:
    name = name.replace("qdg::(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "")


def scale_factor(rows: list[dict]) -> float:
    """KiB-to-bytes factor from the largest copy dispatch (the 256 MiB calibration copy)."""
    best = max(float(r["Counter_Value"]) for r in rows if r["Kernel_Name"].startswith(COPY_KERNEL))
    return COPY_BYTES / best


def per_kernel_grid(rows: list[dict]) -> dict:
    """Mean counter value (KiB) per (kernel, grid size), with the dispatch count."""
    acc = defaultdict(list)
    for r in rows:
        acc[(short(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v), min(v), max(v)) for k, v in acc.items()}


def summarize(trace_dir, fetch_dir, write_dir, out_md, out_json, command: str, dominant: tuple[str, int]):
    ks = kernel_stats(trace_dir)
    fr, wr = counters(fetch_dir), counters(write_dir)
    ff, wf = scale_factor(fr), scale_factor(wr)
    fk, wk = per_kernel_grid(fr), per_kernel_grid(wr)
    lines = [f"# rocprofv3 summary: {os.path.basename(out_md)[:-3]}", "",
             "Commands (from the repository root):", "", "```", command, "```", "",
             "## Kernel trace (--kernel-trace --stats)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for k in ks:
        lines.append(f"| {short(k['name'])} | {k['calls']} | {k['avg_ns'] / 1e3:.2f} | {k['min_ns'] / 1e3:.2f} | "
                     f"{k['max_ns'] / 1e3:.2f} | {k['pct']:.1f} |")
    tg = trace_by_grid(trace_dir)
    lines += ["", "### Per launch shape (kernel trace: End - Start per dispatch)", "",
              "| kernel | grid (work-items) | dispatches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for key in sorted(tg):
        a, lo, hi, n = tg[key]
        lines.append(f"| {key[0]} | {key[1]} | {n} | {a / 1e3:.2f} | {lo / 1e3:.2f} | {hi / 1e3:.2f} |")
    lines += ["", "## HBM bytes per dispatch (--pmc FETCH_SIZE, then --pmc WRITE_SIZE)", "",
              f"Scale: the 256 MiB calibration copy reads FETCH_SIZE x {ff:.4f} and WRITE_SIZE x {wf:.4f} "
              "bytes per KiB counted.", "",
              "| kernel | grid (work-items) | dispatches | fetch MB (mean) | fetch MB (min..max) | write MB (mean) |",
              "|---|---|---|---|---|---|"]
    for key in sorted(fk):
        f_mean, n, f_min, f_max = fk[key]
        w_mean = wk.get(key, (0.0, 0, 0.0, 0.0))[0]
        lines.append(f"| {key[0]} | {key[1]} | {n} | {f_mean * ff / 1e6:.3f} | {f_min * ff / 1e6:.3f}..{f_max * ff / 1e6:.3f} "
                     f"| {w_mean * wf / 1e6:.4f} |")
    dom = {"kernel": dominant[0], "grid": dominant[1], "kernel_source_sha": kernel_source_sha()}
    if (dominant[0], dominant[1]) in tg:
        dom["trace_avg_us"] = tg[(dominant[0], dominant[1])][0] / 1e3
    if (dominant[0], dominant[1]) in fk:
        dom["fetch_bytes"] = fk[dominant][0] * ff
        dom["write_bytes"] = wk[dominant][0] * wf
        dom["traffic_bytes"] = dom["fetch_bytes"] + dom["write_bytes"]
        lines += ["", f"Dominant kernel {dominant[0]} (grid {dominant[1]}): {dom['traffic_bytes'] / 1e6:.3f} MB "
                      "per launch (mean fetch + mean write)"
                      + (f", {dom['trace_avg_us']:.2f} us per launch in the kernel trace." if "trace_avg_us" in dom
                         else ".")]
    open(out_md, "w").write("\n".join(lines) + "\n")
    json.dump(dom, open(out_json, "w"), indent=1)
    return dom


if __name__ == "__main__":
    t, f, w, md, js, kern, grid = sys.argv[1:8]
    cmd = sys.argv[8] if len(sys.argv) > 8 else ""
    print(summarize(t, f, w, md, js, cmd, (kern, int(grid))))
