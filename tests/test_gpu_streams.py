"""Concurrent calls on two HIP streams (default priority), each with its own
buffers and workspace: the library keeps no state between calls, so the calls
interleave freely on the GPU and every result equals the same call made alone.

Covered: the split-K GEMV with the combine in the workgroup, the workspace form
with the last-arriving workgroup's combine (whose tickets live in the caller's
workspace), the single launch with the quantizer, and the block-format GEMV.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_gemv_02_amd as q
import workloads
from gguf_blocks import encode

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def _q8_inputs(N, K, seed):
    wq, ws = workloads.weights(N, K, seed, seed + 1)
    x = workloads.activation(K, seed + 2, True, seed + 3)[None, :]
    return (torch.from_numpy(wq).to(DEV), torch.from_numpy(ws.view(np.int16)).to(DEV),
            torch.from_numpy(x).to(DEV))


@pytest.mark.parametrize("mode", [1, 2])
def test_two_streams_q8(mode):
    announce(f"two streams q8 mode={mode}")
    N, K = 5120, 8192
    cases = [_q8_inputs(N, K, 900 + 10 * i) for i in range(2)]

    def run(wq, ws, x, S, fused, ws_bytes):
        xq = torch.empty((1, K), dtype=torch.int8, device=DEV)
        xl = torch.empty_like(xq) if mode == 2 else None
        xs = torch.empty((1, K // 32), dtype=torch.float32, device=DEV)
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        wsp = q.sk_workspace(N, S)
        if fused:
            q.gemv_q8_fused(mode, wq, ws, y, x, S, wsp)
        else:
            q.quantize_act(mode, x, xq, xl, xs)
            q.gemv_q8_sk(mode, wq, ws, y, xq, xl, xs, S, wsp)
        return y

    # alone, on the default stream
    alone = {}
    for i, (wq, ws, x) in enumerate(cases):
        for S, fused in ((5, False), (16, False), (4, True)):
            alone[(i, S, fused)] = run(wq, ws, x, S, fused, None)
    torch.cuda.synchronize()
    # the same calls issued alternately on two streams, several rounds
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = {}
    for rnd in range(3):
        for S, fused in ((5, False), (16, False), (4, True)):
            for i, (wq, ws, x) in enumerate(cases):
                with torch.cuda.stream(streams[i]):
                    got[(rnd, i, S, fused)] = run(wq, ws, x, S, fused, None)
    torch.cuda.synchronize()
    for (rnd, i, S, fused), y in got.items():
        assert torch.equal(y.view(torch.int32), alone[(i, S, fused)].view(torch.int32)), (rnd, i, S, fused)


@pytest.mark.parametrize("fmt", [2, 12, 39])
def test_two_streams_block_formats(fmt):
    announce(f"two streams gemv_fmt fmt={fmt}")
    N, K, S = 300, 5120, 5
    rng = np.random.default_rng(950 + fmt)
    mats = [encode(fmt, N, K, rng)[0] for _ in range(2)]
    x = rng.standard_normal((1, K)).astype(np.float32)
    oq, _, os_ = oracle.quantize(1, x)
    want = [oracle.gemv_fmt(fmt, 1, w, N, K, xq=oq, xs=os_, splits=S, nthreads=8)[0] for w in mats]
    dws = [torch.from_numpy(w.reshape(-1)).to(DEV) for w in mats]
    xq, xs = torch.from_numpy(oq).to(DEV), torch.from_numpy(os_).to(DEV)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rnd in range(4):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
                q.gemv_fmt(fmt, 1, dws[i], N, K, y, xq=xq, xs=xs, splits=S)
                outs.append((i, y))
    torch.cuda.synchronize()
    for i, y in outs:
        np.testing.assert_array_equal(y.cpu().numpy(), want[i])
