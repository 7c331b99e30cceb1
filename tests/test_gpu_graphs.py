"""Calls captured in a HIP graph (torch.cuda.CUDAGraph over the library's launches
on the capturing stream) and replayed: every replay, with eager library calls and
synchronizations between the replays, gives the eager call's bytes.

Covered: the quantizer and the split-K GEMV whose chunks meet inside a workgroup
(no workspace is touched), and the MFMA-ordered batched path (the quantizer into
MFMA order and the GEMV).  None of these issues a memset; the inputs are written
outside the graph, before capture.
"""
import numpy as np
import pytest
import torch

import quantized_decode_gemv_02_amd as q
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def replay_and_check(graph, out, want, eager):
    for rep in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == want, rep
        eager()  # the program's own work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("mode", [1, 2])
def test_graph_split_k_in_workgroup(mode):
    announce(f"graph quantize + gemv_q8_sk mode={mode}")
    N, K, S = 5120, 8192, 5
    assert q.sk_combines_in_workgroup(mode, K, S)
    wq, ws = workloads.weights(N, K, 501, 502)
    wq, ws = torch.from_numpy(wq).to(DEV), torch.from_numpy(ws.view(np.int16)).to(DEV)
    x = torch.from_numpy(workloads.activation(K, 503, True, 504)[None, :]).to(DEV)
    xq = torch.empty((1, K), dtype=torch.int8, device=DEV)
    xl = torch.empty_like(xq) if mode == 2 else None
    xs = torch.empty((1, K // 32), dtype=torch.float32, device=DEV)
    wsp = q.sk_workspace(N, S)
    y = torch.empty((1, N), dtype=torch.float32, device=DEV)

    def call(out):
        q.quantize_act(mode, x, xq, xl, xs)
        q.gemv_q8_sk(mode, wq, ws, out, xq, xl, xs, S, wsp)

    call(y)
    torch.cuda.synchronize()
    want = y.cpu().numpy().tobytes()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call(y)  # one call on the capturing stream before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            call(y)
    torch.cuda.synchronize()
    other = torch.empty((1, N), dtype=torch.float32, device=DEV)
    replay_and_check(g, y, want, lambda: call(other))
    assert other.cpu().numpy().tobytes() == want
    assert not wsp.any().item()


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B", [16, 40])
def test_graph_mma_tiled(mode, B):
    announce(f"graph quantize_act_mma + gemv_q8_mma_tiled mode={mode} B={B}")
    N, K = 4096, 5120
    wq, ws = workloads.weights(N, K, 511, 512)
    wq, ws = torch.from_numpy(wq).to(DEV), torch.from_numpy(ws.view(np.int16)).to(DEV)
    wt = torch.empty(q.q8_tile_mma_bytes(N, K), dtype=torch.uint8, device=DEV)
    q.q8_tile_mma(wq, ws, wt)
    x = torch.from_numpy(workloads.batch_activation(B, K, 513, True, 514)).to(DEV)
    R = q.mma_act_rows(B)
    tq = torch.empty(R * K, dtype=torch.int8, device=DEV)
    tl = torch.empty(R * K, dtype=torch.int8, device=DEV) if mode == 2 else None
    ts = torch.empty(R * (K // 32), dtype=torch.float32, device=DEV)
    y = torch.empty((B, N), dtype=torch.float32, device=DEV)

    def call(out):
        q.quantize_act_mma(mode, x, tq, tl, ts)
        q.gemv_q8_mma_tiled(mode, wt, N, K, out, tq, tl, ts, B)

    call(y)
    torch.cuda.synchronize()
    want = y.cpu().numpy().tobytes()
    # the plain batched path agrees
    xq = torch.empty((B, K), dtype=torch.int8, device=DEV)
    xl = torch.empty_like(xq) if mode == 2 else None
    xs = torch.empty((B, K // 32), dtype=torch.float32, device=DEV)
    q.quantize_act(mode, x, xq, xl, xs)
    plain = torch.empty((B, N), dtype=torch.float32, device=DEV)
    q.gemv_q8(mode, wq, ws, plain, xq=xq, xl=xl, xs=xs)
    torch.cuda.synchronize()
    assert plain.cpu().numpy().tobytes() == want
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call(y)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            call(y)
    torch.cuda.synchronize()
    other = torch.empty((B, N), dtype=torch.float32, device=DEV)
    replay_and_check(g, y, want, lambda: call(other))
    assert other.cpu().numpy().tobytes() == want


@pytest.mark.parametrize("mode", [1, 2])
def test_graph_glu_mma_tiled(mode):
    """The MFMA-order quantizer and the batched gate/up kernel with the gated-product
    and quantizer epilogue, captured and replayed: the words and h every replay."""
    announce(f"graph quantize_act_mma + gemv_glu_mma_tiled mode={mode}")
    B, F, K = 16, 1024, 2048
    wg, sg = workloads.weights(F, K, 521, 522)
    wu, su = workloads.weights(F, K, 523, 524)
    tiles = []
    for w, s in ((wg, sg), (wu, su)):
        t = torch.empty(q.q8_tile_mma_bytes(F, K), dtype=torch.uint8, device=DEV)
        q.q8_tile_mma(torch.from_numpy(w).to(DEV), torch.from_numpy(s.view(np.int16)).to(DEV), t)
        tiles.append(t)
    x = torch.from_numpy(workloads.batch_activation(B, K, 525, True, 526)).to(DEV)
    R = q.mma_act_rows(B)
    tq = torch.empty(R * K, dtype=torch.int8, device=DEV)
    tl = torch.empty(R * K, dtype=torch.int8, device=DEV) if mode == 2 else None
    ts = torch.empty(R * (K // 32), dtype=torch.float32, device=DEV)
    # every output in one buffer, so one fill and one comparison cover them all
    nw = R * F * (2 if mode == 2 else 1)
    out = torch.empty(B * F + nw // 4 + R * (F // 32), dtype=torch.float32, device=DEV)

    def views(o):
        h = o[:B * F].view(B, F)
        words = o[B * F:B * F + nw // 4].view(torch.int8)
        hq, hl = words[:R * F], (words[R * F:] if mode == 2 else None)
        return h, hq, hl, o[B * F + nw // 4:]

    def call(o):
        h, hq, hl, hs = views(o)
        q.quantize_act_mma(mode, x, tq, tl, ts)
        q.gemv_glu_mma_tiled(0, mode, tiles[0], tiles[1], F, K, tq, tl, ts, B, hq, hl, hs, h=h)

    call(out)
    torch.cuda.synchronize()
    want = out.cpu().numpy().tobytes()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call(out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            call(out)
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    replay_and_check(g, out, want, lambda: call(other))
    assert other.cpu().numpy().tobytes() == want


def test_graph_glu_dequant():
    """The Dequant gate/up kernel with the gated product, captured and replayed."""
    announce("graph gemv_glu_dequant")
    F, K = 4096, 5120
    wg, sg = workloads.weights(F, K, 531, 532)
    wu, su = workloads.weights(F, K, 533, 534)
    args = [torch.from_numpy(a).to(DEV) for a in (wg, sg.view(np.int16), wu, su.view(np.int16))]
    x = torch.from_numpy(workloads.activation(K, 535, True, 536)).to(DEV)
    h = torch.empty(F, dtype=torch.float32, device=DEV)

    def call(out):
        q.gemv_glu_dequant(1, *args, x, out)

    call(h)
    torch.cuda.synchronize()
    want = h.cpu().numpy().tobytes()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call(h)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            call(h)
    torch.cuda.synchronize()
    other = torch.empty_like(h)
    replay_and_check(g, h, want, lambda: call(other))
    assert other.cpu().numpy().tobytes() == want
