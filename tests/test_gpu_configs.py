"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times (quantize -> GEMV [-> combine] [-> arg-max] through the C ABI), against the
whole oracle output (every row; the C oracle runs row-parallel on the host).

Workloads: tiny 256x512 (all modes); 8B-class decode projections qkv 6144x4096,
gate+up 24576x4096, down 4096x12288 with 1% x20 outliers (all modes); narrow
5120x8192 and 5120x25600 projections with split-K S in {1, 2, 4, 8} (Int8Act,
TwoPass); the 151936x5120 LM head with planted equal maxima (all modes); and a
16-row batch against 25600x5120 (Int8Act, TwoPass).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_gemv_02_amd as q
import workloads
from quantized_decode_gemv_02_amd.path import DecodeBuffers, Q8Matrix

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
THREADS = min(16, os.cpu_count() or 1)


def announce(msg):
    print(f"[case] {msg}", flush=True)


def oracle_y(mode, wq, ws, x, splits=1):
    if mode == 0:
        return oracle.gemv(0, wq, ws, x=x, nthreads=THREADS)
    xq, xl, xs = oracle.quantize(mode, x)
    if splits == 1:
        return oracle.gemv(mode, wq, ws, xq=xq, xl=xl, xs=xs, nthreads=THREADS)
    return oracle.combine(oracle.gemv_split(mode, wq, ws, xq, xl, xs, splits, nthreads=THREADS))


def check(mode, y_gpu, wq, ws, x, splits=1):
    if mode == 0:
        Y, tn = oracle.reference_f64(0, wq, ws, x=x, nthreads=THREADS)
        assert oracle.within_tolerance(y_gpu, Y, tn).all()
        assert (y_gpu == oracle_y(0, wq, ws, x)).mean() > 0.99
    else:
        np.testing.assert_array_equal(y_gpu, oracle_y(mode, wq, ws, x, splits))


def run_path(mode, w, x, splits=1, with_argmax=False):
    B, K = x.shape
    buf = DecodeBuffers(mode, w.N, K, B=B, splits=splits, with_argmax=with_argmax)
    y = buf.run(w, torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    return buf, y.cpu().numpy()


@pytest.mark.parametrize("config,shape_index", [(workloads.TINY, 0), (workloads.DECODE_8B, 0), (workloads.DECODE_8B, 1),
                                                 (workloads.DECODE_8B, 2)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_decode_projections(config, shape_index, mode):
    announce(f"config {config}.{shape_index} mode {mode}")
    d = workloads.make(config, shape_index)
    w = Q8Matrix.from_numpy(d["wq"], d["ws"])
    _, y = run_path(mode, w, d["x"])
    check(mode, y, d["wq"], d["ws"], d["x"])


@pytest.mark.parametrize("shape_index", [0, 1])
@pytest.mark.parametrize("mode", [1, 2])
def test_narrow_projections_split_k(shape_index, mode):
    d = workloads.make(workloads.NARROW, shape_index)
    w = Q8Matrix.from_numpy(d["wq"], d["ws"])
    for S in (1, 2, 4, 8):
        announce(f"config 2.{shape_index} mode {mode} S={S}")
        buf, y = run_path(mode, w, d["x"], splits=S)
        check(mode, y, d["wq"], d["ws"], d["x"], splits=S)
        if S > 1:
            xq, xl, xs = oracle.quantize(mode, d["x"])
            want = oracle.gemv_split(mode, d["wq"], d["ws"], xq, xl, xs, S, nthreads=THREADS)
            np.testing.assert_array_equal(buf.part.cpu().numpy(), want)


@pytest.fixture(scope="module")
def lm_head():
    announce("generating the 151936x5120 LM head")
    d = workloads.make(workloads.LM_HEAD, 0)
    return d


def test_lm_head_argmax_planted_ties(lm_head):
    d = lm_head
    wq, ws, x = d["wq"], d["ws"], d["x"]
    N = wq.shape[0]
    w = Q8Matrix.from_numpy(wq, ws)
    a0, b0 = workloads.tie_rows(N, workloads.seed_of(workloads.LM_HEAD, 0, 4))
    placements = [(a0, b0), (0, N - 1), (15, 16), (2025, 2026), (N - 2, N - 1), (1, N - 1)]
    for a, b in placements:
        saved = (wq[[a, b]].copy(), ws[[a, b]].copy())
        workloads.plant_tie(wq, ws, x[0], a, b)
        w.wq[[a, b]] = torch.from_numpy(wq[[a, b]]).to(DEV)
        w.ws[[a, b]] = torch.from_numpy(ws[[a, b]].view(np.int16)).to(DEV)
        for mode in (0, 1, 2):
            announce(f"lm head tie ({a}, {b}) mode {mode}")
            buf, y = run_path(mode, w, x, with_argmax=True)
            idx = int(buf.idx.cpu().numpy()[0])
            assert y[0, a] == y[0, b]
            assert idx == a, (idx, a, b)
            assert idx == int(oracle.argmax(y)[0])      # the index is exact on the GPU's own logits
            # the two-launch tail (keys from the GEMV's epilogue): same logits, same index
            y2 = torch.empty((1, N), dtype=torch.float32, device=DEV)
            i2 = torch.empty(1, dtype=torch.int32, device=DEV)
            wsp = q.gemv_argmax_workspace(N)
            xd = torch.from_numpy(x).to(DEV)
            if mode == 0:
                q.gemv_q8_argmax(0, w.wq, w.ws, y2, i2, wsp, x=xd)
            else:
                xq = torch.empty((1, x.shape[1]), dtype=torch.int8, device=DEV)
                xl = torch.empty_like(xq) if mode == 2 else None
                xs = torch.empty((1, x.shape[1] // 32), dtype=torch.float32, device=DEV)
                q.quantize_act(mode, xd, xq, xl, xs)
                q.gemv_q8_argmax(mode, w.wq, w.ws, y2, i2, wsp, xq=xq, xl=xl, xs=xs)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(y2.cpu().numpy(), y)
            assert int(i2.cpu().numpy()[0]) == a
            if (a, b) == (a0, b0):
                check(mode, y, wq, ws, x)
                assert int(oracle.argmax(oracle_y(mode, wq, ws, x))[0]) == a
        wq[[a, b]], ws[[a, b]] = saved
        w.wq[[a, b]] = torch.from_numpy(saved[0]).to(DEV)
        w.ws[[a, b]] = torch.from_numpy(saved[1].view(np.int16)).to(DEV)


@pytest.mark.parametrize("mode", [1, 2])
def test_batched_decode_b16(mode):
    announce(f"batched B=16 25600x5120 mode {mode}")
    d = workloads.make(workloads.BATCHED, 0)
    w = Q8Matrix.from_numpy(d["wq"], d["ws"])
    _, y = run_path(mode, w, d["x"])
    check(mode, y, d["wq"], d["ws"], d["x"])
    # batch invariance: row t alone gives the same bits
    for t in (0, 7, 15):
        _, y1 = run_path(mode, w, d["x"][t:t + 1])
        np.testing.assert_array_equal(y1[0], y[t])
