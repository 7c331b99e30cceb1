"""Phase stamps of the in-workgroup split-K GEMV (k_gemv_wsplit) on the narrow
projections: where a launch's time goes.

A debug build of the library (every kernel source compiled with
-DQDG_PHASE_STAMPS into a directory of its own, never the release libqdg.so) has
each wave of k_gemv_wsplit record the 100 MHz constant clock at five points:
entry, all first loads issued, its workgroup's staged bytes landed (after the
barrier), its chunk's terms done, and exit, plus the XCC it ran on.  Each launch
is also timed by its own dispatch (qdg_time_next_launch).  The summary gives,
per projection and mode, the launch duration, the spread of wave entries, the
staging latency, the streaming time of a wave, and the spread of exits.

Each timed launch follows the buffer clearing and the stamp set-up (a fill
kernel and a copy).  With --step it also follows a fresh run of the activation
quantizer into the words the GEMV stages, as in the benchmark's step.  With
--pair the same GEMV (another weight copy) runs once more right before it, so
the timed launch follows a launch of itself, as in back-to-back timing; the
stamps are those of the second launch, which overwrites the first's.

Usage (from the repository root, on a GPU):
    python -m quantized_decode_gemv_02_amd.phases [OUT.md] [--reps N] [--step | --pair]
"""
from __future__ import annotations

import json
import os
import shutil
import statistics
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
VARIANT = os.path.join(ROOT, "_build", "phase_stamps")
TICK_NS = 10.0  # s_memrealtime runs at 100 MHz


def build_variant() -> str:
    """libqdg.so with the phase stamps, in _build/phase_stamps/quantized_decode_gemv_02_amd/."""
    sys.path.insert(0, HERE)
    import build as B  # noqa: E402  (the package's own build script, loaded by path)
    pkg = os.path.join(VARIANT, "quantized_decode_gemv_02_amd")
    obj = os.path.join(VARIANT, "obj")
    os.makedirs(pkg, exist_ok=True)
    os.makedirs(obj, exist_ok=True)
    shutil.copy(os.path.join(HERE, "__init__.py"), pkg)
    from concurrent.futures import ThreadPoolExecutor

    def comp(src):
        o = os.path.join(obj, os.path.basename(src) + ".o")
        subprocess.run([B.HIPCC, *B.FLAGS, "-DQDG_PHASE_STAMPS", "-c", src, "-o", o], check=True,
                       capture_output=True)
        return o

    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(comp, B.sources()))
    lib = os.path.join(pkg, "libqdg.so")
    subprocess.run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib, *objs], check=True)
    return VARIANT


def pct(v, p):
    v = sorted(v)
    return v[min(len(v) - 1, int(p / 100 * len(v)))]


def measure(reps: int, step: bool = False, pair: bool = False) -> dict:
    """Runs in the process whose sys.path starts with the variant build."""
    import ctypes

    import numpy as np
    import torch

    import quantized_decode_gemv_02_amd as q
    import workloads

    lib = q.raw()
    lib.qdg_debug_phase_stamps.argtypes = [ctypes.c_void_p]
    dev = torch.device("cuda:0")
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()
    out = {}
    for si, sh in enumerate(workloads.CONFIGS[workloads.NARROW]):
        d = workloads.make(workloads.NARROW, si)
        w0 = torch.from_numpy(d["wq"]).to(dev)
        s0 = torch.from_numpy(d["ws"].view(np.int16)).to(dev)
        R = max(2, int(1.2e9 // (w0.numel() * 1.0625)))
        wsets = [(w0, s0)] + [(w0.clone(), s0.clone()) for _ in range(R - 1)]
        x = torch.from_numpy(d["x"]).to(dev)
        buf = torch.zeros(-(-sh.N // 4) * 16 * 8, dtype=torch.int64, device=dev)
        for mode, S in ((1, 4), (2, 4), (1, 5), (2, 5)):
            xq = torch.empty((1, sh.K), dtype=torch.int8, device=dev)
            xl = torch.empty_like(xq) if mode == 2 else None
            xs = torch.empty((1, sh.K // 32), dtype=torch.float32, device=dev)
            q.quantize_act(mode, x, xq, xl, xs)
            y = torch.empty((1, sh.N), dtype=torch.float32, device=dev)
            rows_m, waves_m = q.sk_workgroup_shape(mode, sh.K, S)
            calls = [q.bind_gemv_q8_sk(mode, w, s, y, xq, xl, xs, S, q.sk_workspace(sh.N, S)) for w, s in wsets]
            for c in calls[:4]:
                c()
            rec = {"dur": [], "entry": [], "issued": [], "staged": [], "stream": [], "exit": [], "span": [],
                   "last_entry": [], "first_exit": [], "xcc_exit": {}}
            for i in range(reps):
                buf.zero_()
                if step:
                    q.quantize_act(mode, x, xq, xl, xs)
                lib.qdg_debug_phase_stamps(ctypes.c_void_p(buf.data_ptr()))
                if pair:
                    calls[(i + 1) % len(calls)]()
                q.time_next_launch(*ev)
                calls[i % len(calls)]()
                lib.qdg_debug_phase_stamps(None)
                torch.cuda.synchronize()
                dur_us = ev[0].elapsed_time(ev[1]) * 1e3
                nwg_m = -(-sh.N // rows_m)
                st = buf.view(-1, 16, 8)[:nwg_m, :waves_m].cpu().numpy().reshape(-1, 8)
                t = st[:, :5].astype(np.float64)
                t0 = t[:, 0].min()
                rel = (t - t0) * TICK_NS / 1e3  # µs from the first wave's entry
                xcc = (st[:, 5] >> 32) & 0xF
                rec["dur"].append(dur_us)
                rec["entry"] += list(rel[:, 0])
                rec["issued"] += list(rel[:, 1] - rel[:, 0])
                rec["staged"] += list(rel[:, 2] - rel[:, 0])
                rec["stream"] += list(rel[:, 3] - rel[:, 2])
                rec["exit"] += list(rel[:, 4])
                rec["span"].append(rel[:, 4].max())
                rec["last_entry"].append(rel[:, 0].max())
                rec["first_exit"].append(rel[:, 4].min())
                for xi in range(8):
                    sel = rel[xcc == xi, 4]
                    if len(sel):
                        rec["xcc_exit"].setdefault(str(xi), []).append(float(np.median(sel)))
            summ = {"workgroups": nwg_m, "waves_per_workgroup": waves_m, "rows_per_workgroup": rows_m,
                    "launches": reps,
                    "launch_us_median": round(statistics.median(rec["dur"]), 3),
                    "wave_span_us_median": round(statistics.median(rec["span"]), 3)}
            for k in ("entry", "issued", "staged", "stream", "exit"):
                v = rec[k]
                summ[k + "_us"] = {f"p{p}": round(float(pct(v, p)), 3) for p in (0, 10, 50, 90, 100)}
            summ["last_entry_us_median"] = round(statistics.median(rec["last_entry"]), 3)
            summ["first_exit_us_median"] = round(statistics.median(rec["first_exit"]), 3)
            summ["median_exit_us_by_xcc"] = {k: round(statistics.median(v), 3) for k, v in sorted(rec["xcc_exit"].items())}
            out[f"{sh.name} {sh.N}x{sh.K} {'int8act' if mode == 1 else 'twopass'} S={S}"] = summ
        del wsets, w0, s0
        torch.cuda.empty_cache()
    return out


def to_markdown(res: dict, cmd: str, step: bool = False, pair: bool = False) -> str:
    title = "# Phase stamps of k_gemv_wsplit (in-workgroup split-K GEMV), narrow projections" + \
        (", each launch right after the activation quantizer" if step else "") + \
        (", each launch right after a launch of itself" if pair else "")
    lines = [title, "",
             "Command (from the repository root, on one MI355X):", "", "```", cmd, "```", "",
             "A debug build (`-DQDG_PHASE_STAMPS`, built by the command into `_build/phase_stamps/`) has every "
             "wave record the 100 MHz constant clock at its entry, after issuing its first loads, when its "
             "workgroup's staged bytes have landed, when its chunk's terms are done, and at exit. Times are µs "
             "from the launch's first wave entry; percentiles are over all waves of all timed launches. "
             "`launch` is the dispatch's own duration (events bound to the dispatch).", ""]
    lines.append("| launch | launch µs | wave span µs | entry p50 / p90 / max | first loads issued p50 | "
                 "staged p50 / p90 | stream p10 / p50 / p90 | exit p0 / p50 / max |")
    lines.append("|---|---|---|---|---|---|---|---|")
    for k, v in res.items():
        e, i, s, st, x = v["entry_us"], v["issued_us"], v["staged_us"], v["stream_us"], v["exit_us"]
        lines.append(f"| {k} ({v['workgroups']} WGs x {v['waves_per_workgroup']} waves) | {v['launch_us_median']} | "
                     f"{v['wave_span_us_median']} | {e['p50']} / {e['p90']} / {e['p100']} | {i['p50']} | "
                     f"{s['p50']} / {s['p90']} | {st['p10']} / {st['p50']} / {st['p90']} | "
                     f"{x['p0']} / {x['p50']} / {x['p100']} |")
    lines += ["", "Median exit per XCC (µs):", ""]
    for k, v in res.items():
        lines.append(f"- {k}: " + ", ".join(f"XCC{a} {b}" for a, b in v["median_exit_us_by_xcc"].items()))
    lines += ["", "Raw summary:", "", "```json", json.dumps(res, indent=1), "```", ""]
    return "\n".join(lines)


def main(argv: list[str]) -> int:
    if len(argv) > 1 and argv[1] == "--child":
        reps = int(argv[2])
        print("PHASES_JSON " + json.dumps(measure(reps, "--step" in argv, "--pair" in argv)), flush=True)
        return 0
    out_md = argv[1] if len(argv) > 1 and not argv[1].startswith("--") else None
    reps = int(argv[argv.index("--reps") + 1]) if "--reps" in argv else 30
    variant = build_variant()
    print(f"phase-stamp build in {variant}", flush=True)
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([variant, ROOT]))
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--child", str(reps)] +
                       [a for a in ("--step", "--pair") if a in argv],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    sys.stderr.write(r.stderr[-2000:])
    if r.returncode != 0:
        return r.returncode
    res = json.loads(next(l for l in r.stdout.splitlines() if l.startswith("PHASES_JSON "))[len("PHASES_JSON "):])
    if out_md:
        open(os.path.splitext(out_md)[0] + ".json", "w").write(json.dumps(res, indent=1))
    cmd = "python -m quantized_decode_gemv_02_amd.phases " + " ".join(argv[1:])
    md = to_markdown(res, cmd, "--step" in argv, "--pair" in argv)
    if out_md:
        os.makedirs(os.path.dirname(os.path.abspath(out_md)), exist_ok=True)
        open(out_md, "w").write(md)
    print(md)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
