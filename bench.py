#!/usr/bin/env python3
"""Benchmark of the Q8_0 decode GEMV hot path on one MI355X.

One step is one decode pass over the narrow projections (o-proj 5120x8192 and
down-proj 5120x25600, batch 1): for each of the Int8Act and TwoPass numerics and
each projection, quantize the activation, run the split-K GEMV and the ascending
combine.  The default path makes two calls (qdg_quantize_act, then
qdg_gemv_q8_sk: the split-K GEMV whose chunks are the waves of one workgroup and
meet in LDS for the ascending combine); --path staged makes the three calls of
the pages' own structure (qdg_quantize_act, qdg_gemv_q8 with S chunks,
qdg_sk_combine) and --path single one (qdg_gemv_q8_fused, the quantizer in every
workgroup).  All three give the same bits.  Inputs are seeded synthetic tensors
resident in HBM before timing; the weights rotate over enough copies (>= 1 GiB
between reuses of a copy) that the 256 MB Infinity Cache cannot serve them.

Timing.  The step (``value``) is timed over K whole steps with nothing else in
the stream.  Every kernel figure is a device duration: the library binds a pair
of HIP events to the measured kernel's own dispatch (qdg_time_next_launch,
hipExtLaunchKernel), so the events add no stream work and give the time a
kernel trace reports; each figure is the median over the measured launches
(>= 50 after >= 5 warm-up launches, rotated weight copies).

Prints ONE JSON line:
  value      = algorithmic GEMV bytes of a step / step time (GB/s); algorithmic
               bytes per GEMV = N*K weight bytes + N*K/16 scale bytes + the
               activation in the mode's encoding (4K Dequant, K + K/8 Int8Act,
               2K + K/8 TwoPass) + 4N output bytes (split-K partials not counted);
  roofline   = the down-proj TwoPass GEMV (the step's dominant kernel): its
               algorithmic bytes / its median device duration over the K steps of
               a second pass of the same step with the events bound, against 8 TB/s;
  config.modes   = per mode and projection of the step: S, device µs, GB/s, % of
               peak and of the read ceiling (Dequant: qdg_gemv_q8_fused beside it);
  config.configs = every workload configuration (tiny, 8B projections, narrow
               projections with S in {1,2,4,8}, LM head + arg-max, 16-row batch)
               in its modes: device µs, GB/s, % of peak, and end-to-end times;
  config.read_ceiling = qdg_stream_read over each projection's bytes and 1 GiB;
  cpu_baseline = the CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0  # MI355X HBM3E
NAMES = {0: "dequant", 1: "int8act", 2: "twopass"}


def alg_bytes(mode: int, N: int, K: int, B: int = 1) -> int:
    act = {0: 4 * K, 1: K + K // 8, 2: 2 * K + K // 8}[mode]
    return N * K + N * K // 16 + B * act + 4 * B * N


def rate(nbytes: int, us: float) -> dict:
    gbs = nbytes / us / 1e3
    return {"us": round(us, 3), "GBs": round(gbs, 1), "pct_of_peak": round(100 * gbs / PEAK_GBS, 2)}


def dominant_kernel(path: str, mode: int, sh, S: int, tiled: bool = False) -> tuple[str, int]:
    """The GEMV kernel a path launches for one projection, as the kernel trace names
    it, and its grid in threads (the library's defaults: no tuning knob set)."""
    import quantized_decode_gemv_02_amd as q
    shape = q.sk_workgroup_shape(mode, sh.K, S) if path == "fused" else None
    if shape is not None:
        rows, waves = shape
        # the staging rule of the library (its STAGE template argument): per-wave copies (1) for one
        # row group, else LDS DMA (2) when K is a multiple of 256 (torch's buffers are 256-byte
        # aligned), else the workgroup copy (0)
        stage = 1 if rows == 4 else (2 if sh.K % 256 == 0 else 0)
        tl = "true" if tiled else "false"
        return f"k_gemv_wsplit<{mode}, {rows // 4}, 1, 4, {stage}, {tl}, false>", 64 * waves * -(-sh.N // rows)
    flags = {"staged": "false, false", "fused": "true, false", "single": "true, true"}[path]
    return f"k_gemv_dot4<{mode}, 4, 4, {flags}, false>", 256 * -(-sh.N // 16) * S


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps before the timed ones (about 75 ms by default: the clocks settle)")
    ap.add_argument("--splits", default=None,
                    help="split-K chunks: one S for both projections, or 'S_o,S_down'; default per path: 5,5 "
                         "for the in-workgroup combine (fused), 4,16 otherwise")
    ap.add_argument("--modes", default="1,2")
    ap.add_argument("--launches", type=int, default=60, help="timed launches per kernel figure (after 5 warm-up)")
    ap.add_argument("--cpu-seconds", type=float, default=2.0, help="length of one timed CPU-baseline run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-rotate-bytes", type=float, default=1.1 * 2 ** 30)
    ap.add_argument("--path", choices=("single", "fused", "staged"), default="fused")
    ap.add_argument("--weights", choices=("plain", "tiled"), default="plain",
                    help="the step's weight layout: plain [N][K], or row tiles of four rows by 256 values "
                         "(qdg_q8_tile_rows, done before timing; --path fused only)")
    ap.add_argument("--no-other-paths", action="store_true", help="skip the other paths' step times")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workload configurations (tiny, 8B, LM head, batch 16, the S sweep)")
    ap.add_argument("--only-configs", default=None,
                    help="comma list among tiny,8b,narrow,lm_head,batched: time only these beside the step")
    ap.add_argument("--no-dequant", action="store_true", help="skip the Dequant timing beside the step")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling measurement")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the timing of the other GGUF block formats beside the step")
    ap.add_argument("--no-producers", action="store_true",
                    help="skip the timing of the fused producers (RMSNorm / SwiGLU + quantizer)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain device copy of 256 MiB (a reference dispatch for the profiler's byte "
                         "counters; the summaries scale by the 1 GiB streaming read instead)")
    return ap.parse_args()


class DeviceTimer:
    """Device durations of library kernels: a pool of HIP event pairs, each bound to one
    launch's own dispatch by qdg_time_next_launch (the first kernel the call launches)."""

    def __init__(self, torch, q, n: int):
        self.torch, self.q = torch, q
        self.pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(n)]
        for a, b in self.pairs:  # torch creates the HIP events at their first record
            a.record()
            b.record()
        torch.cuda.synchronize()

    def bind(self, i: int) -> None:
        self.q.time_next_launch(*self.pairs[i])

    def ms(self, i: int) -> float:
        a, b = self.pairs[i]
        return a.elapsed_time(b)

    def median_us(self, calls, launches: int, warm: int = 300) -> float:
        """Median device duration (µs) of the first kernel of ``calls[i % len(calls)]()`` over
        ``launches`` launches after ``warm`` untimed ones -- and at least one untimed launch on
        every rotated copy, so that no timed launch is a copy's first touch.  A few untimed
        launches are not enough: the same kernel, timed again later in one process, ran up to 6%
        faster (TwoPass, 16 rows) until several milliseconds of launches had passed."""
        for i in range(max(warm, len(calls))):
            calls[i % len(calls)]()
        self.torch.cuda.synchronize()
        n = min(launches, len(self.pairs))
        for i in range(n):
            self.bind(i)
            calls[i % len(calls)]()
        self.torch.cuda.synchronize()
        return statistics.median(self.ms(i) for i in range(n)) * 1e3

    def wall_us(self, calls, launches: int, warm: int = 300) -> float:
        """Mean time a call takes in a back-to-back sequence: one event pair around ``launches``
        calls (every kernel of the call, and the gaps between launches, counted), after one untimed
        launch on every rotated copy."""
        for i in range(max(warm, len(calls))):
            calls[i % len(calls)]()
        e0, e1 = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
        self.torch.cuda.synchronize()
        e0.record()
        for i in range(launches):
            calls[i % len(calls)]()
        e1.record()
        self.torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / launches


def rotation(nbytes: int, min_bytes: float) -> int:
    return max(2, math.ceil(min_bytes / nbytes))


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path shards by output "
              "rows across GPUs, but only the one-GPU path is implemented and timed)", file=sys.stderr)
        return 2
    if args.weights == "tiled" and args.path != "fused":
        print("bench.py: --weights tiled needs --path fused (the in-workgroup split-K GEMV)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import quantized_decode_gemv_02_amd as q
    import workloads

    dev = torch.device("cuda:0")
    modes = [int(m) for m in args.modes.split(",")]
    shapes = workloads.CONFIGS[workloads.NARROW]
    timer = DeviceTimer(torch, q, max(args.steps * len(modes) * len(shapes), args.launches, 64))

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---- inputs (seeded, uploaded once), rotated copies of the weights
    t0 = time.time()
    host = []
    base = []
    for si, sh in enumerate(shapes):
        d = workloads.make(workloads.NARROW, si)
        host.append(d)
        base.append((torch.from_numpy(d["wq"]).to(dev), torch.from_numpy(d["ws"].view(np.int16)).to(dev)))
    set_bytes = sum(w.numel() + 2 * s.numel() for w, s in base)
    R = rotation(set_bytes, args.min_rotate_bytes)
    copies = [[(w.clone(), s.clone()) for (w, s) in base] for _ in range(R)]
    if args.weights == "tiled":  # each copy also in row tiles (the other legs keep the plain weights)
        for cs in copies:
            for i, (w, s) in enumerate(cs):
                wt = torch.empty_like(w)
                q.q8_tile_rows(w, wt)
                cs[i] = (w, s, wt)
    del base
    acts = [torch.from_numpy(d["x"]).to(dev) for d in host]
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    progress(f"narrow projections uploaded ({R} copies, {setup_s:.1f} s)")

    buffers = {}

    def ensure_buffers(mode, si, S):
        if (mode, si, S) in buffers:
            return
        sh = shapes[si]
        buffers[(mode, si, S)] = {
            "xq": torch.empty((1, sh.K), dtype=torch.int8, device=dev),
            "xl": torch.empty((1, sh.K), dtype=torch.int8, device=dev) if mode == 2 else None,
            "xs": torch.empty((1, sh.K // 32), dtype=torch.float32, device=dev),
            "y": torch.empty((1, sh.N), dtype=torch.float32, device=dev),
            "part": torch.empty((S, 1, sh.N), dtype=torch.float32, device=dev) if S > 1 else None,
            "fws": q.sk_workspace(sh.N, S),
        }

    def make_calls(mode, si, S, copy_idx, path):
        """The calls of one projection; the GEMV is the last call but one (staged) or the last."""
        bufs = buffers[(mode, si, S)]
        w, s = copies[copy_idx][si][:2]
        if path == "fused" and args.weights == "tiled":
            return [q.bind_quantize_act(mode, acts[si], bufs["xq"], bufs["xl"], bufs["xs"]),
                    q.bind_gemv_q8_sk_tiled(mode, copies[copy_idx][si][2], s, bufs["y"], bufs["xq"], bufs["xl"],
                                            bufs["xs"], S)]
        if path == "single":
            return [q.bind_gemv_q8_fused(mode, w, s, bufs["y"], acts[si], S, bufs["fws"])]
        calls = [q.bind_quantize_act(mode, acts[si], bufs["xq"], bufs["xl"], bufs["xs"])]
        if path == "fused":
            calls.append(q.bind_gemv_q8_sk(mode, w, s, bufs["y"], bufs["xq"], bufs["xl"], bufs["xs"], S, bufs["fws"]))
            return calls
        out = bufs["y"] if S == 1 else bufs["part"]
        calls.append(q.bind_gemv_q8(mode, w, s, out, xq=bufs["xq"], xl=bufs["xl"], xs=bufs["xs"], splits=S))
        if S > 1:
            calls.append(q.bind_sk_combine(bufs["part"], bufs["y"]))
        return calls

    # S per (mode, shape).  Measured best: the in-workgroup combine at S = 5 on both projections
    # (5120x25600: five chunks of 5120 values, three row groups, one round of 427 workgroups of 15
    # waves; 5120x8192: four non-empty chunks, 427 workgroups of 12 waves); the workspace paths at
    # 4 and 16.
    default_splits = {"fused": "5,5", "staged": "4,16", "single": "4,16"}

    def splits_for(path):
        v = [int(t) for t in (args.splits or default_splits[path]).split(",")]
        return {(mode, si): v[min(si, len(v) - 1)] for mode in modes for si in range(len(shapes))}

    chosen = splits_for(args.path)
    for key, S in chosen.items():
        ensure_buffers(key[0], key[1], S)

    dom_key = (2 if 2 in modes else modes[-1], len(shapes) - 1)
    keys = [(mode, si) for mode in modes for si in range(len(shapes))]

    def build_steps(path):
        ch = chosen if path == args.path else splits_for(path)
        for key, S in ch.items():
            ensure_buffers(key[0], key[1], S)
        steps = []
        for copy_pair in range(R):
            seq = []
            for mi, mode in enumerate(modes):
                cidx = (copy_pair * len(modes) + mi) % R
                for si in range(len(shapes)):
                    seq.append(((mode, si), make_calls(mode, si, ch[(mode, si)], cidx, path)))
            steps.append(seq)
        return steps

    steps_calls = build_steps(args.path)
    step_bytes = sum(alg_bytes(m, shapes[si].N, shapes[si].K) for m in modes for si in range(len(shapes)))
    dom_bytes = alg_bytes(dom_key[0], shapes[dom_key[1]].N, shapes[dom_key[1]].K)

    def run_step(i, steps=None):
        for _, calls in (steps or steps_calls)[i % R]:
            for f in calls:
                f()

    def gemv_position(calls):
        return 0 if len(calls) == 1 else 1  # single: the only call; else after the quantizer

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Timed region (value): K whole steps, nothing else in the stream.
    K = args.steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        run_step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / K
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    progress(f"step: {ms_per_step * 1e3:.2f} us, {value:.0f} GB/s")

    # Second pass of the same K steps with the events bound to each GEMV's and each quantizer's
    # own dispatch (no stream work added): the device duration of every launch of the step.
    quant_ms = {key: [] for key in keys}
    torch.cuda.synchronize()
    t_h = time.perf_counter()
    for i in range(K):
        for ki, (key, calls) in enumerate(steps_calls[i % R]):
            g = gemv_position(calls)
            for ci, f in enumerate(calls):
                if ci == g:
                    timer.bind(i * len(keys) + ki)
                f()
    torch.cuda.synchronize()
    hook_pass_ms = (time.perf_counter() - t_h) * 1e3 / K
    gemv_ms = {key: [timer.ms(i * len(keys) + ki) for i in range(K)] for ki, key in enumerate(keys)}
    if args.path != "single":  # the quantizer launches on their own (the same calls as in the step)
        for key in keys:
            qcalls = [seq[keys.index(key)][1][0] for seq in steps_calls]
            quant_ms[key] = timer.median_us(qcalls, args.launches) / 1e3
    dom_us = statistics.median(gemv_ms[dom_key]) * 1e3
    achieved = dom_bytes / dom_us / 1e3

    # the other paths' step times, for reference (same steps, same rotation)
    other_ms = {}
    if not args.no_other_paths:
        for other in ("single", "fused", "staged"):
            if other == args.path:
                continue
            other_steps = build_steps(other)
            for i in range(args.warmup):
                run_step(i, other_steps)
            torch.cuda.synchronize()
            t_o = time.perf_counter()
            for i in range(K):
                run_step(i, other_steps)
            torch.cuda.synchronize()
            other_ms[f"{other}_ms_per_step"] = round((time.perf_counter() - t_o) * 1e3 / K, 5)

    # HBM bytes per launch of the dominant kernel from the committed profiler counters, used
    # only if they were taken on the current kernel sources at the same launch shape
    traffic = None
    dom_name, dom_grid = dominant_kernel(args.path, dom_key[0], shapes[dom_key[1]], chosen[dom_key],
                                         args.weights == "tiled")
    tpath = os.path.join(ROOT, "profiles", "gemv_q8_narrow_projections_traffic.json")
    if os.path.exists(tpath):
        from quantized_decode_gemv_02_amd import profiling
        t = json.load(open(tpath))
        if (t.get("kernel_source_sha") == profiling.kernel_source_sha() and t.get("grid") == dom_grid
                and t.get("kernel") == dom_name and "traffic_bytes" in t):
            traffic = int(round(t["traffic_bytes"]))

    # ---- the streaming-read ceiling (qdg_stream_read: contiguous 64 KiB slabs a workgroup, only
    # 16-byte nontemporal loads), over as many bytes as each GEMV moves and over 1 GiB
    ceiling = {}
    if not args.no_ceiling:
        pool = torch.empty(3 << 29, dtype=torch.uint8, device=dev)  # 1.5 GiB
        sink = torch.zeros(256, dtype=torch.int32, device=dev)
        sizes = {sh.name: alg_bytes(2, sh.N, sh.K) // 16 * 16 for sh in shapes}
        sizes["1GiB"] = 1 << 30
        for name, nb_ in sizes.items():
            regions = max(1, pool.numel() // nb_)
            calls = [q.bind_stream_read(pool[r * nb_:], nb_, sink) for r in range(regions)]
            ceiling[name] = {"bytes": nb_, **rate(nb_, timer.median_us(calls, args.launches))}
        del pool
        progress("read ceiling done")

    # ---- per mode and projection of the step
    per_mode = {}
    for mode in modes:
        per_mode[NAMES[mode]] = {}
        for si, sh in enumerate(shapes):
            b = alg_bytes(mode, sh.N, sh.K)
            rec = {"splits": chosen[(mode, si)], "alg_bytes": b,
                   **rate(b, statistics.median(gemv_ms[(mode, si)]) * 1e3),
                   "launches": len(gemv_ms[(mode, si)])}
            if quant_ms[(mode, si)]:
                rec["quantize_us"] = round(quant_ms[(mode, si)] * 1e3, 3)
            if sh.name in ceiling:
                rec["pct_of_read_ceiling"] = round(100 * rec["GBs"] / ceiling[sh.name]["GBs"], 1)
            per_mode[NAMES[mode]][sh.name] = rec

    # Dequant on the same projections, beside the step: one launch with binary64 chunk partials
    # added in ascending order in the workgroup (qdg_gemv_q8_fused)
    if not args.no_dequant:
        per_mode["dequant"] = {}
        for si, sh in enumerate(shapes):
            y0 = torch.empty((1, sh.N), dtype=torch.float32, device=dev)
            S = (5, 4)[min(si, 1)]  # Dequant's measured best: five chunks (o-proj), four (down-proj)
            dws = q.sk_workspace(sh.N, S)
            calls = [q.bind_gemv_q8_fused(0, copies[c][si][0], copies[c][si][1], y0, acts[si], S, dws)
                     for c in range(R)]
            b = alg_bytes(0, sh.N, sh.K)
            rec = {"splits": S, "alg_bytes": b, **rate(b, timer.median_us(calls, args.launches))}
            if sh.name in ceiling:
                rec["pct_of_read_ceiling"] = round(100 * rec["GBs"] / ceiling[sh.name]["GBs"], 1)
            per_mode["dequant"][sh.name] = rec

    # ---- every workload configuration, device-timed
    configs = {}
    only = set(args.only_configs.split(",")) if args.only_configs else None

    def want(name):
        return not args.no_configs and (only is None or name in only)

    def upload_set(config, si, rot_min=args.min_rotate_bytes):
        d = workloads.make(config, si)
        w = torch.from_numpy(d["wq"]).to(dev)
        s = torch.from_numpy(d["ws"].view(np.int16)).to(dev)
        n = rotation(w.numel() + 2 * s.numel(), rot_min)
        ws_ = [(w, s)] + [(w.clone(), s.clone()) for _ in range(n - 1)]
        return d, ws_

    def quantized(mode, x):
        B, Kx = x.shape
        xq = torch.empty((B, Kx), dtype=torch.int8, device=dev)
        xl = torch.empty((B, Kx), dtype=torch.int8, device=dev) if mode == 2 else None
        xs = torch.empty((B, Kx // 32), dtype=torch.float32, device=dev)
        q.quantize_act(mode, x, xq, xl, xs)
        return xq, xl, xs

    def projection_record(mode, sh, wsets, x, S):
        """One projection in one mode through its default call: Dequant qdg_gemv_q8_fused,
        the quantized modes qdg_gemv_q8_sk (in-workgroup combine where it fits) after the
        quantizer.  Device µs of the GEMV, plus the quantizer's."""
        y = torch.empty((1, sh.N), dtype=torch.float32, device=dev)
        wsp = q.sk_workspace(sh.N, S)
        rec = {"splits": S, "alg_bytes": alg_bytes(mode, sh.N, sh.K)}
        if mode == 0:
            calls = [q.bind_gemv_q8_fused(0, w, s, y, x, S, wsp) for w, s in wsets]
        else:
            xq, xl, xs = quantized(mode, x)
            calls = [q.bind_gemv_q8_sk(mode, w, s, y, xq, xl, xs, S, wsp) for w, s in wsets]
            rec["in_workgroup"] = q.sk_combines_in_workgroup(mode, sh.K, S)
            rec["quantize_us"] = round(timer.median_us([q.bind_quantize_act(mode, x, xq, xl, xs)], args.launches), 3)
        rec.update(rate(rec["alg_bytes"], timer.median_us(calls, args.launches)))
        return rec

    def glu_record(mode, sh, wsets, x):
        """The stacked gate+up matrix (gate rows first, then up) as the gate and up GEMVs
        with the SwiGLU epilogue in one launch -- Dequant qdg_gemv_glu_dequant (h in f32),
        the quantized modes qdg_gemv_glu_q8 (h's words) -- against the three calls it
        equals: two unsplit qdg_gemv_q8 calls and the producer."""
        F = sh.N // 2
        g = torch.empty((1, F), dtype=torch.float32, device=dev)
        u = torch.empty_like(g)
        halves = [(w[:F], s[:F], w[F:], s[F:]) for w, s in wsets]
        if mode == 0:
            h = torch.empty((F,), dtype=torch.float32, device=dev)
            fused = [q.bind_gemv_glu_dequant(0, *hv, x.view(-1), h) for hv in halves]
            gemv = [q.bind_gemv_q8(0, hv[0], hv[1], g, x=x) for hv in halves]
            prod = q.bind_glu_quantize(0, 0, g, u, h.view(1, F))
            ups = [q.bind_gemv_q8(0, hv[2], hv[3], u, x=x) for hv in halves]
        else:
            xq, xl, xs = quantized(mode, x)
            hq = torch.empty((F,), dtype=torch.int8, device=dev)
            hl = torch.empty_like(hq) if mode == 2 else None
            hs = torch.empty((F // 32,), dtype=torch.float32, device=dev)
            fused = [q.bind_gemv_glu_q8(mode, *hv, xq, xl, xs, hq, hl, hs) for hv in halves]
            gemv = [q.bind_gemv_q8(mode, hv[0], hv[1], g, xq=xq, xl=xl, xs=xs) for hv in halves]
            ups = [q.bind_gemv_q8(mode, hv[2], hv[3], u, xq=xq, xl=xl, xs=xs) for hv in halves]
            prod = q.bind_swiglu_quantize(mode, g, u, None, hq.view(1, F), None if hl is None else hl.view(1, F),
                                          hs.view(1, F // 32))
        f_us = timer.median_us(fused, args.launches)
        g_us = timer.median_us(gemv, args.launches)
        p_us = timer.median_us([prod], args.launches)
        three = [lambda a=a, b=b: (a(), b(), prod()) for a, b in zip(gemv, ups)]
        return {"F": F, "fused_us": round(f_us, 2), "gemv_us": round(g_us, 2), "producer_us": round(p_us, 2),
                "three_calls_us": round(2 * g_us + p_us, 2),
                "fused_wall_us": round(timer.wall_us(fused, args.launches), 2),
                "three_calls_wall_us": round(timer.wall_us(three, args.launches), 2),
                # both matrices, the activation once, and h (f32, or its words and scales)
                **rate(2 * (F * sh.K + F * sh.K // 16) + alg_bytes(mode, 0, sh.K)
                       + {0: 4 * F, 1: F + F // 8, 2: 2 * F + F // 8}[mode], f_us)}

    if want("tiny"):
        sh = workloads.CONFIGS[workloads.TINY][0]
        d, wsets = upload_set(workloads.TINY, 0, 0)
        x = torch.from_numpy(d["x"]).to(dev)
        rec = {}
        for mode in (0, 1, 2):
            y = torch.empty((1, sh.N), dtype=torch.float32, device=dev)
            if mode == 0:
                calls = [q.bind_gemv_q8(0, w, s, y, x=x) for w, s in wsets]
            else:
                xq, xl, xs = quantized(mode, x)
                calls = [q.bind_gemv_q8(mode, w, s, y, xq=xq, xl=xl, xs=xs) for w, s in wsets]
            rec[NAMES[mode]] = {"splits": 1, **rate(alg_bytes(mode, sh.N, sh.K), timer.median_us(calls, args.launches))}
        configs["tiny_512x256"] = rec
        progress("tiny done")

    if want("8b"):
        # S per projection (measured best, in-workgroup combine / Dequant chunk waves)
        s_q8 = {"qkv": 2, "gate_up": 2, "down": 6}
        s_dq = {"qkv": 3, "gate_up": 2, "down": 2}
        for si, sh in enumerate(workloads.CONFIGS[workloads.DECODE_8B]):
            d, wsets = upload_set(workloads.DECODE_8B, si)
            x = torch.from_numpy(d["x"]).to(dev)
            rec = {}
            for mode in (0, 1, 2):
                rec[NAMES[mode]] = projection_record(mode, sh, wsets, x, s_dq[sh.name] if mode == 0 else s_q8[sh.name])
            if sh.name == "gate_up":
                rec["glu"] = {NAMES[mode]: glu_record(mode, sh, wsets, x) for mode in (0, 1, 2)}
            configs[f"8b_{sh.name}_{sh.N}x{sh.K}"] = rec
            del wsets
        torch.cuda.empty_cache()
        progress("8B projections done")

    if want("narrow"):
        # the configuration's own split counts S in {1, 2, 4, 8} through qdg_gemv_q8_sk (the
        # in-workgroup combine where it serves the shape, else the last-arriving workgroup)
        for si, sh in enumerate(shapes):
            rec = {}
            for mode in modes:
                rec[NAMES[mode]] = {}
                xq, xl, xs = quantized(mode, acts[si])
                for S in (1, 2, 4, 8):
                    y = torch.empty((1, sh.N), dtype=torch.float32, device=dev)
                    wsp = q.sk_workspace(sh.N, S)
                    calls = [q.bind_gemv_q8_sk(mode, copies[c][si][0], copies[c][si][1], y, xq, xl, xs, S, wsp)
                             for c in range(R)]
                    rec[NAMES[mode]][f"S{S}"] = {"in_workgroup": q.sk_combines_in_workgroup(mode, sh.K, S),
                                                 **rate(alg_bytes(mode, sh.N, sh.K), timer.median_us(calls, args.launches))}
            configs[f"narrow_{sh.name}_{sh.N}x{sh.K}_splits"] = rec
        progress("narrow S sweep done")

    if want("lm_head"):
        sh = workloads.CONFIGS[workloads.LM_HEAD][0]
        d = workloads.make(workloads.LM_HEAD, 0)
        a, b = workloads.tie_rows(sh.N, workloads.seed_of(workloads.LM_HEAD, 0, 4))
        workloads.plant_tie(d["wq"], d["ws"], d["x"][0], a, b)
        w = torch.from_numpy(d["wq"]).to(dev)
        s = torch.from_numpy(d["ws"].view(np.int16)).to(dev)
        wsets = [(w, s), (w.clone(), s.clone())]
        x = torch.from_numpy(d["x"]).to(dev)
        del d
        y = torch.empty((1, sh.N), dtype=torch.float32, device=dev)
        idx = torch.empty(1, dtype=torch.int32, device=dev)
        kws = q.gemv_argmax_workspace(sh.N)
        rec = {"tie_rows": [a, b]}
        for mode in (0, 1, 2):
            if mode == 0:
                calls = [q.bind_gemv_q8_argmax(0, ww, ss, y, idx, kws, x=x) for ww, ss in wsets]
                qus = 0.0
            else:
                xq, xl, xs = quantized(mode, x)
                calls = [q.bind_gemv_q8_argmax(mode, ww, ss, y, idx, kws, xq=xq, xl=xl, xs=xs) for ww, ss in wsets]
                qus = timer.median_us([q.bind_quantize_act(mode, x, xq, xl, xs)], args.launches)
            r = {"gemv": rate(alg_bytes(mode, sh.N, sh.K), timer.median_us(calls, args.launches))}
            r["end_to_end_us"] = round(timer.wall_us(calls, args.launches) + qus, 3)
            if qus:
                r["quantize_us"] = round(qus, 3)
            torch.cuda.synchronize()
            r["index"] = int(idx.item())
            r["index_is_first_tie"] = r["index"] == a
            rec[NAMES[mode]] = r
        configs[f"lm_head_{sh.N}x{sh.K}_argmax"] = rec
        del wsets, w, s
        torch.cuda.empty_cache()
        progress("LM head done")

    if want("batched"):
        sh = workloads.CONFIGS[workloads.BATCHED][0]
        d, wsets = upload_set(workloads.BATCHED, 0)
        x = torch.from_numpy(d["x"]).to(dev)
        rec = {}
        for mode in (1, 2):
            xq, xl, xs = quantized(mode, x)
            y = torch.empty((sh.B, sh.N), dtype=torch.float32, device=dev)
            calls = [q.bind_gemv_q8(mode, w, s, y, xq=xq, xl=xl, xs=xs) for w, s in wsets]
            rec[NAMES[mode]] = {"B": sh.B, "alg_bytes": alg_bytes(mode, sh.N, sh.K, sh.B),
                                **rate(alg_bytes(mode, sh.N, sh.K, sh.B), timer.median_us(calls, args.launches))}
        # a 64-row prefill chunk on the same weights (seeded rows of the same
        # distribution), plain and MFMA-ordered, beside the 16-row batch
        PB = 64
        xp = torch.from_numpy(workloads.batch_activation(PB, sh.K, 4000, True, 4001)).to(dev)
        prefill = {"plain": {}, "mma_tiled": {}}
        for mode in (1, 2):
            xq, xl, xs = quantized(mode, xp)
            y = torch.empty((PB, sh.N), dtype=torch.float32, device=dev)
            calls = [q.bind_gemv_q8(mode, w, s, y, xq=xq, xl=xl, xs=xs) for w, s in wsets]
            b = alg_bytes(mode, sh.N, sh.K, PB)
            prefill["plain"][NAMES[mode]] = {"B": PB, "alg_bytes": b, **rate(b, timer.median_us(calls, args.launches))}
        # the same batch over MFMA-ordered operands: the weights repacked once
        # (qdg_q8_tile_mma), the activations quantized into the MFMA order
        # (qdg_quantize_act_mma, timed beside), the GEMV qdg_gemv_q8_mma_tiled
        tiles, halves = [], []
        F = sh.N // 2
        for w, s in wsets:
            wt = torch.empty(q.q8_tile_mma_bytes(sh.N, sh.K), dtype=torch.uint8, device=dev)
            q.q8_tile_mma(w, s, wt)
            tiles.append(wt)
            pair = []
            for lo in (0, F):  # the gate rows, then the up rows, each repacked on its own
                ht = torch.empty(q.q8_tile_mma_bytes(F, sh.K), dtype=torch.uint8, device=dev)
                q.q8_tile_mma(w[lo:lo + F], s[lo:lo + F], ht)
                pair.append(ht)
            halves.append(pair)
        del wsets
        torch.cuda.empty_cache()
        tiled = {}
        for mode in (1, 2):
            tq = torch.empty(16 * sh.K, dtype=torch.int8, device=dev)
            tl = torch.empty(16 * sh.K, dtype=torch.int8, device=dev) if mode == 2 else None
            ts = torch.empty(16 * (sh.K // 32), dtype=torch.float32, device=dev)
            qcall = q.bind_quantize_act_mma(mode, x, tq, tl, ts)
            qcall()
            y = torch.empty((sh.B, sh.N), dtype=torch.float32, device=dev)
            calls = [q.bind_gemv_q8_mma_tiled(mode, wt, sh.N, sh.K, y, tq, tl, ts, sh.B) for wt in tiles]
            b = alg_bytes(mode, sh.N, sh.K, sh.B)
            tiled[NAMES[mode]] = {"B": sh.B, "alg_bytes": b, **rate(b, timer.median_us(calls, args.launches)),
                                  "quantize_us": round(timer.median_us([qcall], args.launches), 3)}
        rec["mma_tiled"] = tiled
        for mode in (1, 2):
            Rp = q.mma_act_rows(PB)
            tq = torch.empty(Rp * sh.K, dtype=torch.int8, device=dev)
            tl = torch.empty(Rp * sh.K, dtype=torch.int8, device=dev) if mode == 2 else None
            ts = torch.empty(Rp * (sh.K // 32), dtype=torch.float32, device=dev)
            q.quantize_act_mma(mode, xp, tq, tl, ts)
            y = torch.empty((PB, sh.N), dtype=torch.float32, device=dev)
            calls = [q.bind_gemv_q8_mma_tiled(mode, wt, sh.N, sh.K, y, tq, tl, ts, PB) for wt in tiles]
            b = alg_bytes(mode, sh.N, sh.K, PB)
            prefill["mma_tiled"][NAMES[mode]] = {"B": PB, "alg_bytes": b, **rate(b, timer.median_us(calls, args.launches))}
        # the two halves as gate and up with the SwiGLU and the quantizer into the down
        # projection's MFMA-ordered words (qdg_gemv_glu_mma_tiled), against the four calls it
        # equals: two tiled GEMVs, the producer (f32 h) and the MFMA-order quantizer
        glu = {}
        for mode in (1, 2):
            for Bg in (sh.B, PB):
                xg = x if Bg == sh.B else xp
                Rg = q.mma_act_rows(Bg)
                tq = torch.empty(Rg * sh.K, dtype=torch.int8, device=dev)
                tl = torch.empty(Rg * sh.K, dtype=torch.int8, device=dev) if mode == 2 else None
                ts = torch.empty(Rg * (sh.K // 32), dtype=torch.float32, device=dev)
                q.quantize_act_mma(mode, xg, tq, tl, ts)
                hq = torch.empty(Rg * F, dtype=torch.int8, device=dev)
                hl = torch.empty(Rg * F, dtype=torch.int8, device=dev) if mode == 2 else None
                hs = torch.empty(Rg * (F // 32), dtype=torch.float32, device=dev)
                fused = [q.bind_gemv_glu_mma_tiled(0, mode, a, b, F, sh.K, tq, tl, ts, Bg, hq, hl, hs)
                         for a, b in halves]
                g = torch.empty((Bg, F), dtype=torch.float32, device=dev)
                u = torch.empty_like(g)
                hf = torch.empty_like(g)
                gcalls = [q.bind_gemv_q8_mma_tiled(mode, a, F, sh.K, g, tq, tl, ts, Bg) for a, _ in halves]
                ucalls = [q.bind_gemv_q8_mma_tiled(mode, b, F, sh.K, u, tq, tl, ts, Bg) for _, b in halves]
                prod = q.bind_glu_quantize(0, 0, g, u, hf)
                qcall = q.bind_quantize_act_mma(mode, hf, hq, hl, hs)
                f_us = timer.median_us(fused, args.launches)
                g_us = timer.median_us(gcalls, args.launches)
                p_us = timer.median_us([prod], args.launches)
                q_us = timer.median_us([qcall], args.launches)
                four = [lambda a=a, b=b: (a(), b(), prod(), qcall()) for a, b in zip(gcalls, ucalls)]
                nb = 2 * (F * sh.K + F * sh.K // 16) + Bg * {1: sh.K + sh.K // 8, 2: 2 * sh.K + sh.K // 8}[mode] \
                    + Bg * {1: F + F // 8, 2: 2 * F + F // 8}[mode]
                glu[f"{NAMES[mode]}_B{Bg}"] = {
                    "F": F, "fused_us": round(f_us, 2), "gemv_us": round(g_us, 2), "producer_us": round(p_us, 2),
                    "quantize_us": round(q_us, 2), "four_calls_us": round(2 * g_us + p_us + q_us, 2),
                    "fused_wall_us": round(timer.wall_us(fused, args.launches), 2),
                    "four_calls_wall_us": round(timer.wall_us(four, args.launches), 2), **rate(nb, f_us)}
        rec["glu_mma_tiled"] = glu
        configs[f"batched_B{sh.B}_{sh.N}x{sh.K}"] = rec
        configs[f"prefill_B{PB}_{sh.N}x{sh.K}"] = prefill
        del tiles, halves
        torch.cuda.empty_cache()
        progress("batched done")

    # ---- the producers of the activation words, beside the step: the residual add + RMSNorm
    # and SwiGLU, each fused with the quantizer, against the same work in two launches
    producers = {}
    if not args.no_producers:
        hid, inter = shapes[0].N, shapes[-1].K
        xr = torch.from_numpy(workloads.batch_activation(1, hid, 11, True, 12)).to(dev)
        rr = torch.from_numpy(workloads.batch_activation(1, hid, 13)).to(dev)
        wn = torch.from_numpy(workloads.norm_weight(hid, 14)).to(dev)
        gg, uu = (torch.from_numpy(a_).to(dev) for a_ in workloads.glu_inputs(1, inter, 15))
        for mode in modes:
            for name, K_, fused, f32_only, f32 in (
                    ("rmsnorm", hid,
                     lambda xq, xl, xs: q.bind_rmsnorm_quantize(mode, xr, wn, rr, None, None, xq, xl, xs),
                     lambda y: q.bind_rmsnorm_quantize(0, xr, wn, rr, None, y), torch.empty_like(xr)),
                    ("swiglu", inter,
                     lambda xq, xl, xs: q.bind_swiglu_quantize(mode, gg, uu, None, xq, xl, xs),
                     lambda y: q.bind_swiglu_quantize(0, gg, uu, y), torch.empty_like(gg))):
                xq_ = torch.empty((1, K_), dtype=torch.int8, device=dev)
                xl_ = torch.empty_like(xq_) if mode == 2 else None
                xs_ = torch.empty((1, K_ // 32), dtype=torch.float32, device=dev)
                one = fused(xq_, xl_, xs_)
                a_, b_ = f32_only(f32), q.bind_quantize_act(mode, f32, xq_, xl_, xs_)
                producers[f"{name}_{NAMES[mode]}_K{K_}"] = {
                    "fused_us": round(timer.median_us([one], args.launches), 2),
                    "f32_producer_us": round(timer.median_us([a_], args.launches), 2),
                    "quantize_us": round(timer.median_us([b_], args.launches), 2)}
        # the projection that feeds the norm, with the residual add, RMSNorm and quantizer as its
        # epilogue (qdg_gemv_q8_rmsnorm), against the GEMV alone and against the GEMV followed by
        # the norm producer (two launches), on each narrow projection at the step's S
        for si, sh in enumerate(shapes):
            rn = torch.from_numpy(workloads.activation(sh.N, 21 + si)).to(dev)
            wn2 = torch.from_numpy(workloads.norm_weight(sh.N, 23 + si)).to(dev)
            for mode in modes:
                S = chosen[(mode, si)]
                if not q.sk_combines_in_workgroup(mode, sh.K, S):
                    continue
                xq, xl, xs = quantized(mode, acts[si])
                y = torch.empty((1, sh.N), dtype=torch.float32, device=dev)
                s_ = torch.empty_like(y)
                hq = torch.empty((1, sh.N), dtype=torch.int8, device=dev)
                hl = torch.empty_like(hq) if mode == 2 else None
                hs = torch.empty((1, sh.N // 32), dtype=torch.float32, device=dev)
                nws = q.gemv_rmsnorm_workspace(sh.N)
                sws = q.sk_workspace(sh.N, S)
                fused_calls = [q.bind_gemv_q8_rmsnorm(mode, copies[c][si][0], copies[c][si][1], xq, xl, xs, S, nws,
                                                      y=y, r=rn, s=s_, w=wn2, qmode=mode, hq=hq, hl=hl, hs=hs)
                               for c in range(R)]
                gemv_calls = [q.bind_gemv_q8_sk(mode, copies[c][si][0], copies[c][si][1], y, xq, xl, xs, S, sws)
                              for c in range(R)]
                norm_call = q.bind_rmsnorm_quantize(mode, y, wn2, rn, s_, None, hq, hl, hs)
                two = [lambda g=g: (g(), norm_call()) for g in gemv_calls]
                f_us = timer.median_us(fused_calls, args.launches)
                g_us = timer.median_us(gemv_calls, args.launches)
                n_us = timer.median_us([norm_call], args.launches)
                producers[f"gemv_rmsnorm_{NAMES[mode]}_{sh.name}_{sh.N}x{sh.K}_S{S}"] = {
                    "fused_us": round(f_us, 2), "gemv_us": round(g_us, 2), "rmsnorm_quantize_us": round(n_us, 2),
                    "two_launches_us": round(g_us + n_us, 2),
                    "fused_wall_us": round(timer.wall_us(fused_calls, args.launches), 2),
                    "two_launches_wall_us": round(timer.wall_us(two, args.launches), 2),
                    # the GEMV's bytes plus the norm's: r, s and w (4 bytes a row each) and the words
                    **rate(alg_bytes(mode, sh.N, sh.K) + 12 * sh.N + (2 if mode == 2 else 1) * sh.N + sh.N // 8,
                           f_us)}
        progress("producers done")

    # ---- the other GGUF block formats on the down-proj's shape: qdg_gemv_fmt in the two
    # quantized modes at S=8 (one round of 1280 five-wave workgroups), over rotated copies
    formats = {}
    if not args.no_formats:
        fsh = shapes[-1]
        fnames = {2: "Q4_0", 3: "Q4_1", 6: "Q5_0", 7: "Q5_1", 20: "IQ4_NL", 39: "MXFP4", 10: "Q2_K",
                  11: "Q3_K", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K", 23: "IQ4_XS"}
        fx = acts[-1]
        fy = torch.empty((fsh.N,), dtype=torch.float32, device=dev)
        fq = {mode: quantized(mode, fx) for mode in modes}
        for fmt, fname in fnames.items():
            Kf = fsh.K // workloads.BLOCK_FORMATS[fmt][0] * workloads.BLOCK_FORMATS[fmt][0]
            wb = torch.from_numpy(workloads.block_matrix(fmt, fsh.N, Kf, 2000 + fmt).reshape(-1)).to(dev)
            nbytes = wb.numel()
            fc = [wb] + [wb.clone() for _ in range(max(1, int(args.min_rotate_bytes // nbytes)))]
            rec = {"K": Kf, "bytes": nbytes, "S": 8}
            for mode in modes:
                xq_, xl_, xs_ = fq[mode]
                calls = [q.bind_gemv_fmt(fmt, mode, c, fsh.N, Kf, fy, xq=xq_, xl=xl_, xs=xs_, splits=8) for c in fc]
                rec[NAMES[mode]] = rate(nbytes, timer.median_us(calls, args.launches))
            formats[fname] = rec
            del fc, wb
        torch.cuda.empty_cache()
        progress("formats done")

    # ---- CPU baseline: the oracle on the same step.  One warm-up run, then five timed runs of
    # whole steps (each run as many steps as fill --cpu-seconds); the median run's throughput.
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = min(16, os.cpu_count() or 1)

        def oracle_step(nthreads):
            for mode in modes:
                for si in range(len(shapes)):
                    d = host[si]
                    xq, xl, xs = oracle.quantize(mode, d["x"])
                    oracle.combine(oracle.gemv_split(mode, d["wq"], d["ws"], xq, xl, xs, chosen[(mode, si)],
                                                     nthreads=nthreads))

        def cpu_runs(nthreads):
            tb = time.perf_counter()
            oracle_step(nthreads)  # warm-up run of one step also sizes the runs
            per = max(1, int(args.cpu_seconds / max(time.perf_counter() - tb, 1e-3)))
            rates = []
            for _ in range(5):
                tb = time.perf_counter()
                for _ in range(per):
                    oracle_step(nthreads)
                rates.append(step_bytes * per / (time.perf_counter() - tb) / 1e9)
            return statistics.median(rates), per

        v_all, per_all = cpu_runs(threads)
        v_one, per_one = cpu_runs(1)
        model = ""
        try:
            model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
        except (OSError, StopIteration):
            pass
        cpu = {"value": round(v_all, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"median of 5 runs of {per_all} whole steps each after one warm-up step: quantize + "
                         f"split-K GEMV + combine of both projections in every mode, OpenMP over rows",
               "single_thread_value": round(v_one, 3),
               "single_thread_sample": f"median of 5 runs of {per_one} whole steps on one thread",
               "host": {"cpu_count": os.cpu_count(), "model": model}}
        progress("cpu baseline done")

    line = {
        "metric": "Q8_0 GEMV achieved HBM GB/s and % of peak per mode (Dequant/Int8/TwoPass)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 dot / f32 sum",
        "data": "synthetic (seeded; int8 weights uniform [-127,127], fp16 scales U[1e-3,1e-2), N(0,1) activations "
                "with 1% x20 outliers)",
        "config": {"workload": "narrow projections with split-K: o-proj K=8192 N=5120 and down-proj K=25600 N=5120, "
                               "batch 1, Int8Act + TwoPass, quantize + GEMV + ascending combine",
                   "path": args.path, "weights": args.weights, **other_ms,
                   "timed_pass_ms_per_step": round(hook_pass_ms, 5),
                   "global_batch": 1, "seq_len": 1, "parallelism": "single GPU",
                   "weight_copies": R, "rotated_bytes": R * set_bytes, "modes": per_mode,
                   "configs": configs, "read_ceiling": ceiling, "producers": producers, "formats": formats,
                   "step_alg_bytes": step_bytes, "pct_of_peak": round(100 * value / PEAK_GBS, 2),
                   "timing": "device durations: events bound to each kernel's own dispatch "
                             "(qdg_time_next_launch), median over the measured launches"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"{dom_name} ({args.path} path) down-proj 5120x25600 TwoPass S={chosen[dom_key]}",
                     "alg_bytes_per_launch": dom_bytes, "median_launch_us": round(dom_us, 3),
                     "launches": len(gemv_ms[dom_key])},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
