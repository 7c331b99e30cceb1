"""Summaries of rocprofv3 runs of the benchmark (kernel-trace statistics and the
FETCH_SIZE / WRITE_SIZE byte counters), written as short text under profiles/.

FETCH_SIZE is scaled by what it reads for the library's own streaming read of
1 GiB (k_stream_read over exactly 2^30 bytes, the benchmark's read-ceiling
pass): factor = 2^30 bytes / counter(that dispatch).  On gfx950 the counter
gives half the bytes for every kernel of this library (the streaming read, the
GEMVs, the LDS-DMA batched kernel alike), which are all 16-byte loads; the
runtime's copy kernel reads 1.0-1.6x its bytes on the same counter, so it is
not used.  WRITE_SIZE is reported as counted (KiB x 1024): the library's
kernels write only their outputs.

Usage (from the repository root, after the rocprofv3 runs):
    python -m quantized_decode_gemv_02_amd.profiling TRACE_DIR FETCH_DIR WRITE_DIR OUT.md OUT.json \
        KERNEL GRID "COMMAND" [OCC_DIR]
    python -m quantized_decode_gemv_02_amd.profiling counters OUT.md "COMMAND" PASS_DIR [PASS_DIR ...]
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

READ_BYTES = 1 << 30
READ_KERNEL = "k_stream_read"
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


# The translation unit of the step's dominant kernel (the in-workgroup split-K GEMV):
# a stored byte count stands only while these sources are unchanged.
DOMINANT_SOURCES = (os.path.join(CSRC, "qdg_wsplit.hip"), os.path.join(CSRC, "qdg_device.h"),
                    os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qdg.h"))


def sources_for(kernel: str) -> tuple:
    """The translation unit of a traced kernel, for the hash stored beside its byte count."""
    unit = {"k_gemv_fmt": "qdg_formats.hip", "k_gemv_dq_seg": "qdg_dequant_seg.hip",
            "k_gemv_dq_glu": "qdg_dequant_seg.hip", "k_gemv_glu": "qdg_glu.hip", "k_gemv_mma": "qdg_mma_tiled.hip",
            "k_gemv_mfma": "qdg_mfma.hip", "k_gemv_dot4": "qdg_gemv.hip"}
    for prefix, f in unit.items():
        if kernel.startswith(prefix):
            return (os.path.join(CSRC, f),) + DOMINANT_SOURCES[1:]
    return DOMINANT_SOURCES


def kernel_source_sha(paths=DOMINANT_SOURCES) -> str:
    """Hash of the dominant kernel's sources, so a stored byte count is used only for the code it was taken on."""
    h = hashlib.sha256()
    for p in paths:
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


# MI355X (gfx950): 256 CUs of 4 SIMDs; 512 VGPRs (arch + accumulation) a SIMD lane,
# allocated in granules of 8; at most 8 waves a SIMD; 160 KiB of LDS a CU.
CUS, SIMDS, VGPR_FILE, VGPR_GRANULE, WAVES_PER_SIMD, LDS_BYTES = 256, 4, 512, 8, 8, 160 * 1024
# rocprofv3's VGPR_Count for these gfx950 dispatches is half the allocation: the
# compiler's resource report (hipcc -Rpass-analysis=kernel-resource-usage) gives
# 60, 66 and 72 VGPRs for kernels the trace lists at 32, 36 and 36 (allocations
# 64, 72, 72 in granules of 8), so the trace's figure is doubled here.
TRACE_VGPR_SCALE = 2


def occupancy(vgpr: int, agpr: int, lds: int, wg_size: int, grid: int) -> dict:
    """Resident capacity of one launch shape and how its grid fills it (theoretical)."""
    regs = -(-(vgpr + agpr) // VGPR_GRANULE) * VGPR_GRANULE
    per_simd = min(WAVES_PER_SIMD, VGPR_FILE // max(regs, 1))
    wpw = -(-wg_size // 64)  # waves a workgroup
    wg_cu = (SIMDS * per_simd) // wpw
    if lds > 0:
        wg_cu = min(wg_cu, LDS_BYTES // lds)
    wgs = -(-grid // wg_size)
    cap = wg_cu * CUS
    rounds = wgs / cap if cap else float("inf")
    return {"waves_per_simd": per_simd, "wg_per_cu": wg_cu, "workgroups": wgs, "capacity": cap,
            "fill": min(1.0, wgs / cap) if cap else 0.0, "rounds": rounds,
            "tail": rounds - int(rounds) if rounds > 1 and rounds != int(rounds) else 0.0}


def trace_shapes(trace_dir: str) -> dict:
    """(kernel, total work-items) -> resources of the dispatch, from the kernel trace."""
    out = {}
    for r in csv.DictReader(open(_one(trace_dir, "*kernel_trace.csv"))):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
        out[(short(r["Kernel_Name"]), grid)] = (TRACE_VGPR_SCALE * int(r["VGPR_Count"]),
                                                TRACE_VGPR_SCALE * int(r["Accum_VGPR_Count"]),
                                                int(r["LDS_Block_Size"]), wg)
    return out


def counters(pmc_dir: str) -> list[dict]:
    return list(csv.DictReader(open(_one(pmc_dir, "*counter_collection.csv"))))


def short(name: str) -> str:
    name = name.replace("qdg::(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "")


def scale_factor(rows: list[dict]) -> float:
    """KiB-to-bytes factor from the largest streaming-read dispatch (the 1 GiB read)."""
    best = max(float(r["Counter_Value"]) for r in rows if short(r["Kernel_Name"]) == READ_KERNEL)
    return READ_BYTES / best


def per_kernel_grid(rows: list[dict]) -> dict:
    """Mean counter value (KiB) per (kernel, grid size), with the dispatch count."""
    acc = defaultdict(list)
    for r in rows:
        acc[(short(r["Kernel_Name"]), int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v), min(v), max(v)) for k, v in acc.items()}


def per_kernel_counters(pmc_dir: str) -> dict:
    """(kernel, grid) -> {counter: mean value per dispatch} for a multi-counter run."""
    acc = defaultdict(lambda: defaultdict(list))
    for r in counters(pmc_dir):
        acc[(short(r["Kernel_Name"]), int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}


def summarize(trace_dir, fetch_dir, write_dir, out_md, out_json, command: str, dominant: tuple[str, int],
              occ_dir: str | None = None):
    ks = kernel_stats(trace_dir)
    fr, wr = counters(fetch_dir), counters(write_dir)
    ff, wf = scale_factor(fr), 1024.0
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
              f"Scale: FETCH_SIZE x {ff:.2f} bytes per KiB counted (the 1 GiB streaming read, k_stream_read, "
              "counts 2^30 bytes); WRITE_SIZE x 1024 (as counted).", "",
              "| kernel | grid (work-items) | dispatches | fetch MB (mean) | fetch MB (min..max) | write MB (mean) |",
              "|---|---|---|---|---|---|"]
    for key in sorted(fk):
        f_mean, n, f_min, f_max = fk[key]
        w_mean = wk.get(key, (0.0, 0, 0.0, 0.0))[0]
        lines.append(f"| {key[0]} | {key[1]} | {n} | {f_mean * ff / 1e6:.3f} | {f_min * ff / 1e6:.3f}..{f_max * ff / 1e6:.3f} "
                     f"| {w_mean * wf / 1e6:.4f} |")
    shapes = trace_shapes(trace_dir)
    occ_meas = per_kernel_counters(occ_dir) if occ_dir else {}
    lines += ["", "## Occupancy and split-K block fill", "",
              "Theoretical residency from each dispatch's registers (VGPR + AGPR, granule 8, 512 a lane; the "
              "kernel trace's counts doubled, as they are half the allocation the compiler reports on gfx950), "
              "its LDS (160 KiB a CU; the trace reports the static allocation only -- the split-K workgroup's "
              "dynamic window, K/32 x (36 or 68 + 2 x rows) bytes, at most 79 KiB, allows two workgroups a CU, "
              "as its waves do) and workgroup size, on 256 "
              "CUs x 4 SIMDs with at most 8 waves a SIMD; fill = workgroups / resident capacity (capped at 1), "
              "rounds = workgroups / capacity.  Waves launched: SQ_WAVES from a third pass (--pmc SQ_WAVES "
              "SQ_WAVE_CYCLES GRBM_GUI_ACTIVE), which checks the grid.", "",
              "| kernel | grid | VGPR+AGPR | LDS B | waves/SIMD | WG/CU | WGs | fill | rounds | waves launched |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    for key in sorted(shapes):
        if not key[0].startswith("k_gemv"):
            continue
        v, a, l, wg = shapes[key]
        o = occupancy(v, a, l, wg, key[1])
        m = occ_meas.get(key, {})
        waves = f"{m['SQ_WAVES']:.0f}" if "SQ_WAVES" in m else "-"
        lines.append(f"| {key[0]} | {key[1]} | {v}+{a} | {l} | {o['waves_per_simd']} | {o['wg_per_cu']} | "
                     f"{o['workgroups']} | {o['fill']:.2f} | {o['rounds']:.2f} | {waves} |")
    dom = {"kernel": dominant[0], "grid": dominant[1], "kernel_source_sha": kernel_source_sha(sources_for(dominant[0]))}
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


# Per-wave instruction counts and wave-cycle fractions from SQ counter passes
# (each pass its own rocprofv3 --pmc run of the same command).
COUNTER_COLUMNS = (
    ("VALU/wave", lambda c: c["SQ_INSTS_VALU"] / c["SQ_WAVES"]),
    ("SALU/wave", lambda c: c["SQ_INSTS_SALU"] / c["SQ_WAVES"]),
    ("VMEM rd/wave", lambda c: c["SQ_INSTS_VMEM_RD"] / c["SQ_WAVES"]),
    ("LDS/wave", lambda c: c["SQ_INSTS_LDS"] / c["SQ_WAVES"]),
    ("f64 FMA/wave", lambda c: c["SQ_INSTS_VALU_FMA_F64"] / c["SQ_WAVES"]),
    ("CVT/wave", lambda c: c["SQ_INSTS_VALU_CVT"] / c["SQ_WAVES"]),
    ("wait any", lambda c: c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]),
    ("wait issue", lambda c: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
    ("active", lambda c: c["SQ_ACTIVE_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
    ("LDS bank confl./wave", lambda c: c["SQ_LDS_BANK_CONFLICT"] / c["SQ_WAVES"]),
    ("LDS unaligned stall/wave", lambda c: c["SQ_LDS_UNALIGNED_STALL"] / c["SQ_WAVES"]),
)


def summarize_counters(out_md: str, command: str, pass_dirs: list[str], prefix: str = "k_gemv") -> None:
    merged = defaultdict(dict)
    for d in pass_dirs:
        for key, vals in per_kernel_counters(d).items():
            merged[key].update(vals)
    lines = [f"# rocprofv3 counters: {os.path.basename(out_md)[:-3]}", "",
             "Commands (from the repository root; one --pmc pass each):", "", "```", command, "```", "",
             "Per dispatch, mean over the dispatches of each kernel and grid. The wave-cycle fractions are "
             "SQ_WAIT_ANY (waiting on a load, LDS or other counter), SQ_WAIT_INST_ANY (ready, waiting for "
             "its instruction to issue) and SQ_ACTIVE_INST_ANY (issuing), each over SQ_WAVE_CYCLES; they "
             "overlap and need not add to 1.", ""]
    cols = [name for name, _ in COUNTER_COLUMNS]
    lines += ["| kernel | grid | waves | " + " | ".join(cols) + " |", "|---|---|---|" + "---|" * len(cols)]
    for key in sorted(merged):
        if not key[0].startswith(prefix):
            continue
        c = merged[key]
        cells = []
        for _, fn in COUNTER_COLUMNS:
            try:
                v = fn(c)
                cells.append(f"{v:.2f}" if v < 10 else f"{v:.0f}")
            except (KeyError, ZeroDivisionError):
                cells.append("-")
        lines.append(f"| {key[0]} | {key[1]} | {c.get('SQ_WAVES', 0):.0f} | " + " | ".join(cells) + " |")
    open(out_md, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "counters":
        summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4:])
        sys.exit(0)
    t, f, w, md, js, kern, grid = sys.argv[1:8]
    cmd = sys.argv[8] if len(sys.argv) > 8 else ""
    occ = sys.argv[9] if len(sys.argv) > 9 else None
    print(summarize(t, f, w, md, js, cmd, (kern, int(grid)), occ))
