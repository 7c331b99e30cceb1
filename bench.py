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
workgroup).  All three give the same bits.  Each run reports the other paths'
step times beside its own, and times Dequant (qdg_gemv_q8_fused with the
same S) on the same projections.  Inputs are seeded synthetic tensors resident in HBM before
timing; the weights rotate over enough copies (>= 1 GiB between reuses of a
copy) that the 256 MB Infinity Cache cannot serve them.

Prints ONE JSON line:
  value      = algorithmic GEMV bytes of a step / step time (GB/s), timed over K
               steps with no events in the stream; algorithmic
               bytes per GEMV = N*K weight bytes + N*K/16 scale bytes + the
               activation in the mode's encoding (K + K/8 Int8Act, 2K + K/8
               TwoPass) + 4N output bytes (split-K partial traffic not counted);
  roofline   = the down-proj TwoPass GEMV (the step's dominant kernel): its
               algorithmic bytes / its mean launch duration from HIP events
               around each of its launches in a second timed pass of the same K
               steps (events around every GEMV), against 8 TB/s;
  config.modes = per mode and projection: S, the GEMV's mean launch time (the
               same second pass), GB/s, and its share of the read ceiling;
  config.read_ceiling = qdg_stream_read over each projection's bytes and 1 GiB:
               the practical ceiling of a launch that only reads;
  cpu_baseline = the CPU oracle on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0  # MI355X HBM3E


def alg_bytes(mode: int, N: int, K: int, B: int = 1) -> int:
    act = {0: 4 * K, 1: K + K // 8, 2: 2 * K + K // 8}[mode]
    return N * K + N * K // 16 + B * act + 4 * B * N


def dominant_kernel(path: str, mode: int, sh, S: int, tiled: bool = False) -> tuple[str, int]:
    """The GEMV kernel a path launches for one projection, as the kernel trace names
    it, and its grid in threads."""
    import quantized_decode_gemv_02_amd as q
    shape = q.sk_workgroup_shape(mode, sh.K, S) if path == "fused" else None
    if os.environ.get("QDG_SK_WSPLIT", "1").startswith("0"):  # the library's override of the placement
        shape = None
    if shape is not None:
        rows, waves = shape
        # the library's staging rule (its STAGE template argument): per-wave copies (1) for one
        # row group, else LDS DMA (2) when K is a multiple of 256 (torch's buffers are 256-byte
        # aligned), else the workgroup copy (0); QDG_WS_LOCAL / QDG_WS_DMA override as in the library
        loc = os.environ.get("QDG_WS_LOCAL")
        dma = sh.K % 256 == 0 and not os.environ.get("QDG_WS_DMA", "1").startswith("0")
        stage = 1 if (loc.startswith("1") if loc else rows == 4) else (2 if dma else 0)
        # template arguments: mode, row groups, steps a weight group (1), groups in flight (4), staging
        tl = "true" if tiled else "false"
        return f"k_gemv_wsplit<{mode}, {rows // 4}, 1, 4, {stage}, {tl}>", 64 * waves * -(-sh.N // rows)
    flags = {"staged": "false, false", "fused": "true, false", "single": "true, true"}[path]
    return f"k_gemv_dot4<{mode}, 4, 4, {flags}, false>", 256 * -(-sh.N // 16) * S


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--splits", default=None,
                    help="split-K chunks: 'auto' (timed choice), one S for both projections, or 'S_o,S_down'; "
                         "default per path: 5,5 for the in-workgroup combine (fused), 4,16 otherwise")
    ap.add_argument("--modes", default="1,2")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-rotate-bytes", type=float, default=1.1 * 2 ** 30)
    ap.add_argument("--path", choices=("single", "fused", "staged"), default="fused")
    ap.add_argument("--weights", choices=("plain", "tiled"), default="plain",
                    help="the step's weight layout: plain [N][K], or row tiles of four rows by 256 values "
                         "(qdg_q8_tile_rows, done before timing; --path fused only)")
    ap.add_argument("--no-dequant", action="store_true", help="skip the Dequant timing beside the step")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling measurement")
    ap.add_argument("--no-sweep", action="store_true", help="skip the S in {1,2,4,8} sweep beside the step")
    ap.add_argument("--no-formats", action="store_true",
                    help="skip the timing of the other GGUF block formats beside the step")
    ap.add_argument("--no-producers", action="store_true",
                    help="skip the timing of the fused producers (RMSNorm / SwiGLU + quantizer)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain device copy of 256 MiB (for scaling profiler byte counters)")
    return ap.parse_args()


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
    shapes = workloads.CONFIGS[2]

    # ---- inputs (seeded, uploaded once), rotated copies of the weights
    t0 = time.time()
    host = []
    base = []
    for si, sh in enumerate(shapes):
        d = workloads.make(2, si)
        host.append(d)
        base.append((torch.from_numpy(d["wq"]).to(dev), torch.from_numpy(d["ws"].view(np.int16)).to(dev),
                     torch.from_numpy(d["x"]).to(dev)))
    set_bytes = sum(w.numel() + 2 * s.numel() for w, s, _ in base)
    R = max(2, math.ceil(args.min_rotate_bytes / set_bytes))
    copies = [[(w.clone(), s.clone()) for (w, s, _) in base] for _ in range(R)]
    if args.weights == "tiled":  # each copy also in row tiles (the other legs keep the plain weights)
        for cs in copies:
            for i, (w, s) in enumerate(cs):
                wt = torch.empty_like(w)
                q.q8_tile_rows(w, wt)
                cs[i] = (w, s, wt)
    del base  # keep only the rotated copies (the x tensors live in `acts`)
    acts = [torch.from_numpy(d["x"]).to(dev) for d in host]
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    # ---- per (mode, shape) buffers and pre-bound launches
    def make_calls(mode, si, S, copy_idx, path="staged"):
        # the GEMV is always the last call but one (staged) or the last call
        sh = shapes[si]
        N, K = sh.N, sh.K
        bufs = buffers[(mode, si, S)]
        w, s = copies[copy_idx][si][:2]
        if path == "fused" and args.weights == "tiled":
            calls = [q.bind_quantize_act(mode, acts[si], bufs["xq"], bufs["xl"], bufs["xs"])]
            calls.append(q.bind_gemv_q8_sk_tiled(mode, copies[copy_idx][si][2], s, bufs["y"], bufs["xq"], bufs["xl"],
                                                 bufs["xs"], S))
            return calls
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

    # ---- S per (mode, shape): fixed (default 4 for the o-proj, 8 for the down-proj), or timed
    # Measured best: the in-workgroup combine at S = 5 on both projections (5120x25600: five
    # chunks of 5120 values, three row groups, one round of 427 workgroups of 15 waves;
    # 5120x8192: four non-empty chunks, 427 workgroups of 12 waves); the workspace paths at 4
    # and 16.  Back-to-back launches of the o-proj alone favour S = 3 by 2-4%, but whole steps
    # at S = 3 on the o-proj ran 1-2% slower than at S = 5.
    default_splits = {"fused": "5,5", "staged": "4,16", "single": "4,16"}

    def splits_for(path):
        spec = args.splits or default_splits[path]
        if spec == "auto":
            return None
        v = [int(t) for t in spec.split(",")]
        return {(mode, si): v[min(si, len(v) - 1)] for mode in modes for si in range(len(shapes))}

    chosen = {}
    fixed = splits_for(args.path)
    for mode in modes:
        for si in range(len(shapes)):
            if fixed is not None:
                chosen[(mode, si)] = fixed[(mode, si)]
                ensure_buffers(mode, si, chosen[(mode, si)])
                continue
            best = None
            for S in (1, 2, 3, 4, 5, 6, 8, 10, 12, 13, 16):
                ensure_buffers(mode, si, S)
                seqs = [make_calls(mode, si, S, c, args.path) for c in range(R)]
                for c in seqs:
                    for f in c:
                        f()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 8 * R
                skip = 0 if args.path == "single" else 1  # the quantizer does not depend on S
                e0.record()
                for i in range(reps):
                    for f in seqs[i % R][skip:]:
                        f()
                e1.record()
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                if best is None or ms < best[1]:
                    best = (S, ms)
            chosen[(mode, si)] = best[0]

    # ---- the step: every (mode, shape) once, each mode on its own weight copy
    dom_key = (2 if 2 in modes else modes[-1], len(shapes) - 1)

    def build_steps(path):
        ch = chosen if path == args.path else (splits_for(path) or chosen)
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

    keys = [(mode, si) for mode in modes for si in range(len(shapes))]

    def run_step(i, events=None, steps=None):
        # events: {key: list of (start, end)} -- one pair around every GEMV launch of the step
        for key, calls in (steps or steps_calls)[i % R]:
            if events is not None and key in events:
                g = 0 if len(calls) == 1 else 1  # the GEMV's position (single: the only call)
                for f in calls[:g]:
                    f()
                ev0, ev1 = events[key][i]
                ev0.record()
                calls[g]()
                ev1.record()
                for f in calls[g + 1:]:
                    f()
            else:
                for f in calls:
                    f()

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Timed region 1 (value): K steps with no events.  HIP events between the kernels of a
    # step add stream work of their own (about 7 us a step here), so the step is timed bare.
    K = args.steps
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        run_step(i)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1e3 / K

    # Timed region 2 (roofline and the per-mode table): the same K steps again, with a HIP event
    # pair around every GEMV launch; the dominant kernel's mean launch time comes from here.
    ev_all = {key: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in range(K)] for key in keys}
    for i in range(K):
        run_step(i, ev_all)
    torch.cuda.synchronize()
    gemv_ms = {key: sum(a.elapsed_time(b) for a, b in ev_all[key]) / K for key in keys}
    dom_ms = gemv_ms[dom_key]

    # the other paths' step times, for reference (same steps, same rotation)
    other_ms = {}
    for other in ("single", "fused", "staged"):
        if other == args.path:
            continue
        other_steps = build_steps(other)
        for i in range(args.warmup):
            run_step(i, steps=other_steps)
        torch.cuda.synchronize()
        t_o = time.perf_counter()
        for i in range(K):
            run_step(i, steps=other_steps)
        torch.cuda.synchronize()
        other_ms[f"{other}_ms_per_step"] = round((time.perf_counter() - t_o) * 1e3 / K, 5)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

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

    # per mode and projection: the GEMV launch's mean duration (HIP events in the timed region)
    names = {0: "dequant", 1: "int8act", 2: "twopass"}
    per_mode = {}
    for mode in modes:
        per_mode[names[mode]] = {}
        for si in range(len(shapes)):
            b = alg_bytes(mode, shapes[si].N, shapes[si].K)
            us = gemv_ms[(mode, si)] * 1e3
            per_mode[names[mode]][shapes[si].name] = {
                "splits": chosen[(mode, si)], "alg_bytes": b, "gemv_us": round(us, 3),
                "gemv_GBs": round(b / us / 1e3, 1), "pct_of_peak": round(100 * b / us / 1e3 / PEAK_GBS, 2)}

    def mean_launch_us(calls, reps):
        for c in calls:
            c()
        torch.cuda.synchronize()
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            pairs[i][0].record()
            calls[i % len(calls)]()
            pairs[i][1].record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in pairs) / reps * 1e3

    # Dequant on the same projections, beside the step: one launch with the same S (binary64
    # chunk partials and an ascending binary64 combine in the last workgroup of each row tile)
    if not args.no_dequant:
        per_mode["dequant"] = {}
        for si, sh in enumerate(shapes):
            y0 = torch.empty((1, sh.N), dtype=torch.float32, device=dev)
            S = (4, 8)[min(si, 1)]  # Dequant's measured best: four chunks (o-proj), eight (down-proj)
            dws = q.sk_workspace(sh.N, S)
            calls = [q.bind_gemv_q8_fused(0, copies[c][si][0], copies[c][si][1], y0, acts[si], S, dws)
                     for c in range(R)]
            for c in calls:
                c()
            torch.cuda.synchronize()
            reps = max(K // 4, 2 * R)
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(reps)]
            for i in range(reps):
                pairs[i][0].record()
                calls[i % R]()
                pairs[i][1].record()
            torch.cuda.synchronize()
            us = sum(a.elapsed_time(b) for a, b in pairs) / reps * 1e3
            b = alg_bytes(0, sh.N, sh.K)
            per_mode["dequant"][sh.name] = {"splits": S, "alg_bytes": b, "gemv_us": round(us, 3),
                                            "gemv_GBs": round(b / us / 1e3, 1),
                                            "pct_of_peak": round(100 * b / us / 1e3 / PEAK_GBS, 2)}

    # The configuration's own split counts, S in {1, 2, 4, 8}, beside the chosen S: the GEMV with
    # its combine (the default path's qdg_gemv_q8_sk) per mode and projection, events around
    # each launch, rotated copies.
    splits_sweep = {}
    if not args.no_sweep:
        for mode in modes:
            for si, sh in enumerate(shapes):
                rec = {}
                for S in (1, 2, 4, 8):
                    ensure_buffers(mode, si, S)
                    b = buffers[(mode, si, S)]
                    calls = [q.bind_gemv_q8_sk(mode, copies[c][si][0], copies[c][si][1], b["y"], b["xq"], b["xl"],
                                               b["xs"], S, b["fws"]) for c in range(R)]
                    q.quantize_act(mode, acts[si], b["xq"], b["xl"], b["xs"])
                    us = mean_launch_us(calls, max(40, 4 * R))
                    rec[str(S)] = {"gemv_us": round(us, 3),
                                   "gemv_GBs": round(alg_bytes(mode, sh.N, sh.K) / us / 1e3, 1),
                                   "in_workgroup": q.sk_combines_in_workgroup(mode, sh.K, S)}
                splits_sweep[f"{names[mode]}_{sh.name}"] = rec

    # The practical read ceiling: qdg_stream_read (contiguous 64 KiB slabs a workgroup, nothing
    # but 16-byte nontemporal loads) over as many bytes as each GEMV launch moves, rotated over
    # a pool larger than the Infinity Cache, and over 1 GiB.
    ceiling = {}
    if not args.no_ceiling:
        pool = torch.empty(3 << 29, dtype=torch.uint8, device=dev)  # 1.5 GiB
        sink = torch.zeros(256, dtype=torch.int32, device=dev)
        sizes = {sh.name: alg_bytes(2, sh.N, sh.K) // 16 * 16 for sh in shapes}
        sizes["1GiB"] = 1 << 30
        for name, nb_ in sizes.items():
            regions = max(1, pool.numel() // nb_)
            calls = [q.bind_stream_read(pool[r * nb_:], nb_, sink) for r in range(regions)]
            us = mean_launch_us(calls, max(20, 4 * regions))
            ceiling[name] = {"bytes": nb_, "us": round(us, 3), "GBs": round(nb_ / us / 1e3, 1)}
        del pool
        for mname, per_shape in per_mode.items():
            for sname, rec in per_shape.items():
                if sname in ceiling:
                    rec["pct_of_read_ceiling"] = round(100 * rec["gemv_GBs"] / ceiling[sname]["GBs"], 1)

    # The producers of the activation words, beside the step: the residual add + RMSNorm and
    # SwiGLU, each fused with the quantizer, against the same work in two launches (the f32
    # result, then qdg_quantize_act).  Inputs of the projections' shapes: the norm over the
    # hidden size (the o-proj's N), SwiGLU over the down-proj's K.
    producers = {}
    if not args.no_producers:
        hid, inter = shapes[0].N, shapes[-1].K
        xr = torch.from_numpy(workloads.batch_activation(1, hid, 11, True, 12)).to(dev)
        rr = torch.from_numpy(workloads.batch_activation(1, hid, 13)).to(dev)
        wn = torch.from_numpy(workloads.norm_weight(hid, 14)).to(dev)
        gg, uu = (torch.from_numpy(a).to(dev) for a in workloads.glu_inputs(1, inter, 15))
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
                a, b = f32_only(f32), q.bind_quantize_act(mode, f32, xq_, xl_, xs_)
                producers[f"{name}_{names[mode]}_K{K_}"] = {
                    "fused_us": round(mean_launch_us([one], 200), 2),
                    "two_launches_us": round(mean_launch_us([lambda: (a(), b())], 200), 2)}

    # The other GGUF block formats on the down-proj's shape, beside the step: qdg_gemv_fmt in the
    # two quantized modes at S=8 (one round of 1280 five-wave workgroups), over rotated copies.
    formats = {}
    if not args.no_formats:
        fsh = shapes[-1]
        fnames = {2: "Q4_0", 3: "Q4_1", 6: "Q5_0", 7: "Q5_1", 20: "IQ4_NL", 39: "MXFP4", 10: "Q2_K",
                  11: "Q3_K", 12: "Q4_K", 13: "Q5_K", 14: "Q6_K", 23: "IQ4_XS"}
        fx = acts[-1]
        fy = torch.empty((fsh.N,), dtype=torch.float32, device=dev)
        fq = {}
        for mode in modes:
            xq_ = torch.empty((1, fsh.K), dtype=torch.int8, device=dev)
            xl_ = torch.empty_like(xq_) if mode == 2 else None
            xs_ = torch.empty((1, fsh.K // 32), dtype=torch.float32, device=dev)
            q.quantize_act(mode, fx, xq_, xl_, xs_)
            fq[mode] = (xq_, xl_, xs_)
        for fmt, fname in fnames.items():
            Kf = fsh.K // workloads.BLOCK_FORMATS[fmt][0] * workloads.BLOCK_FORMATS[fmt][0]
            wb = torch.from_numpy(workloads.block_matrix(fmt, fsh.N, Kf, 2000 + fmt).reshape(-1)).to(dev)
            nbytes = wb.numel()
            fc = [wb] + [wb.clone() for _ in range(max(1, int(args.min_rotate_bytes // nbytes)))]
            rec = {"K": Kf, "bytes": nbytes, "S": 8}
            for mode in modes:
                xq_, xl_, xs_ = fq[mode]
                calls = [q.bind_gemv_fmt(fmt, mode, c, fsh.N, Kf, fy, xq=xq_, xl=xl_, xs=xs_, splits=8) for c in fc]
                us = mean_launch_us(calls, max(40, 2 * len(fc)))
                rec[names[mode]] = {"us": round(us, 2), "GBs": round(nbytes / us / 1e3, 1),
                                    "pct_of_peak": round(100 * nbytes / us / 1e3 / PEAK_GBS, 1)}
            formats[fname] = rec
            del fc, wb
        torch.cuda.empty_cache()

    # ---- CPU baseline: the oracle on the same step (whole steps, repeated for a bounded time)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = min(16, os.cpu_count() or 1)
        t_cpu, n_steps = 0.0, 0
        while n_steps == 0 or t_cpu < args.cpu_seconds:
            tb = time.perf_counter()
            for mode in modes:
                for si, sh in enumerate(shapes):
                    d = host[si]
                    xq, xl, xs = oracle.quantize(mode, d["x"])
                    part = oracle.gemv_split(mode, d["wq"], d["ws"], xq, xl, xs, chosen[(mode, si)],
                                             nthreads=threads)
                    oracle.combine(part)
            t_cpu += time.perf_counter() - tb
            n_steps += 1
        # the same steps on one thread (row-parallel OpenMP does not change any row's order), for a
        # quarter of the budget
        t1, n1 = 0.0, 0
        while n1 == 0 or t1 < args.cpu_seconds / 4:
            tb = time.perf_counter()
            for mode in modes:
                for si, sh in enumerate(shapes):
                    d = host[si]
                    xq, xl, xs = oracle.quantize(mode, d["x"])
                    oracle.combine(oracle.gemv_split(mode, d["wq"], d["ws"], xq, xl, xs, chosen[(mode, si)],
                                                     nthreads=1))
            t1 += time.perf_counter() - tb
            n1 += 1
        model = ""
        try:
            model = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
        except (OSError, StopIteration):
            pass
        cpu = {"value": round(step_bytes * n_steps / t_cpu / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{n_steps} whole steps ({t_cpu:.1f} s): quantize + split-K GEMV + combine of both "
                         f"projections in every mode, OpenMP over rows",
               "single_thread_value": round(step_bytes * n1 / t1 / 1e9, 3),
               "single_thread_sample": f"{n1} whole steps ({t1:.1f} s) on one thread",
               "host": {"cpu_count": os.cpu_count(), "model": model}}

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
        "data": "synthetic (seeded; int8 weights uniform [-127,127], fp16 scales U[1e-3,1e-2), N(0,1) activations with 1% x20 outliers)",
        "config": {"workload": "narrow projections with split-K: o-proj K=8192 N=5120 and down-proj K=25600 N=5120, "
                               "batch 1, Int8Act + TwoPass, quantize + GEMV + ascending combine",
                   "path": args.path, "weights": args.weights, **other_ms,
                   "global_batch": 1, "seq_len": 1, "parallelism": "single GPU",
                   "weight_copies": R, "rotated_bytes": R * set_bytes, "modes": per_mode,
                   "read_ceiling": ceiling, "producers": producers, "formats": formats, "splits_sweep": splits_sweep,
                   "step_alg_bytes": step_bytes, "pct_of_peak": round(100 * value / PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                     "kernel": f"{dom_name} ({args.path} path) down-proj 5120x25600 TwoPass S={chosen[dom_key]}",
                     "alg_bytes_per_launch": dom_bytes, "mean_launch_us": round(dom_ms * 1e3, 3)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
