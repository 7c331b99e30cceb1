"""GPU parity of the batched GEMV over MFMA-ordered operands: the weight records
of qdg_q8_tile_mma and the activation records of qdg_quantize_act_mma, both
checked byte for byte against the layout the header defines (restated here in
numpy from that definition, not from the kernels), and qdg_gemv_q8_mma_tiled
against the oracle bit for bit, equal to qdg_gemv_q8 over the plain operands,
batch-invariant, in both workgroup shapes (one or two 64-row record groups)."""
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_gemv_02_amd as q
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
THREADS = min(16, os.cpu_count() or 1)


def announce(msg):
    print(f"[case] {msg}", flush=True)


def dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def records_weights(wq, ws):
    """The weight records by the header's definition: record (q, s, r) holds, at
    byte 1024*m + 16*l + 8*h + j, byte 8*(l//16) + j of block 8s + r + 4h of row
    64q + 16m + l%16, then the 16-bit scales at word 2048 + 8*c + 2*m + h."""
    N, K = wq.shape
    G, S = -(-N // 64), K // 256
    w = np.zeros((G * 64, K), np.int8)
    w[:N] = wq
    s = np.zeros((G * 64, K // 32), np.uint16)
    s[:N] = ws
    out = np.zeros((G, S, 4, 4352), np.uint8)
    for qg in range(G):
        for st in range(S):
            for r in range(4):
                rec = out[qg, st, r]
                for m in range(4):
                    for l in range(64):
                        row, u = 64 * qg + 16 * m + l % 16, l // 16
                        for h in range(2):
                            b = 8 * st + r + 4 * h
                            o = 1024 * m + 16 * l + 8 * h
                            rec[o:o + 8] = w[row, 32 * b + 8 * u:32 * b + 8 * u + 8].view(np.uint8)
                words = rec[4096:].view(np.uint16)
                for c in range(16):
                    for m in range(4):
                        for h in range(2):
                            words[8 * c + 2 * m + h] = s[64 * qg + 16 * m + c, 8 * st + r + 4 * h]
    return out.reshape(-1)


def records_acts(xq, xs, B, zero_scale):
    """The activation records by the header's definition: tiles of 16 rows (1, 2
    or 4 of them), each a run of records (s, r) holding, at byte 16*l + 8*h + j,
    word 8*(l//16) + j of block 8s + r + 4h of row l%16 of the tile, then scale
    16*h + t of that block and tile row t; rows past B are a zero row's."""
    K = xq.shape[1]
    R = 16 if B <= 16 else 32 if B <= 32 else 64
    full = np.zeros((R, K), np.int8)
    full[:B] = xq
    sc = np.full((R, K // 32), zero_scale, np.float32)
    sc[:B] = xs
    S = K // 256
    words = np.zeros((R // 16, S, 4, 1024), np.int8)
    scales = np.zeros((R // 16, S, 4, 32), np.float32)
    for a in range(R // 16):
        for st in range(S):
            for r in range(4):
                for l in range(64):
                    t, u = 16 * a + l % 16, l // 16
                    for h in range(2):
                        b = 8 * st + r + 4 * h
                        words[a, st, r, 16 * l + 8 * h:16 * l + 8 * h + 8] = full[t, 32 * b + 8 * u:32 * b + 8 * u + 8]
                for h in range(2):
                    for t in range(16):
                        scales[a, st, r, 16 * h + t] = sc[16 * a + t, 8 * st + r + 4 * h]
    return words.reshape(-1), scales.reshape(-1)


def zero_row_scale(mode):
    # the quantizer's scale of an all-zero block: 1 (Int8Act), 1e-30/127 (TwoPass)
    return np.float32(1.0) if mode == 1 else np.float32(np.float32(1e-30) / np.float32(127.0))


def tile(wq, ws):
    N, K = wq.shape
    wt = torch.full((q.q8_tile_mma_bytes(N, K),), 0xA5, dtype=torch.uint8, device=DEV)
    q.q8_tile_mma(dev(wq), dev(ws), wt)
    return wt


def acts(mode, x):
    B, K = x.shape
    R = q.mma_act_rows(B)
    xd = dev(x)
    tq = torch.full((R * K,), 77, dtype=torch.int8, device=DEV)
    tl = torch.full((R * K,), 77, dtype=torch.int8, device=DEV) if mode == 2 else None
    ts = torch.full((R * (K // 32),), float("nan"), dtype=torch.float32, device=DEV)
    q.quantize_act_mma(mode, xd, tq, tl, ts)
    return tq, tl, ts


@pytest.mark.parametrize("N,K", [(64, 256), (100, 512), (5, 768), (130, 1536)])
def test_tile_mma_layout(N, K):
    announce(f"tile_mma N={N} K={K}")
    wq, ws = workloads.weights(N, K, N + K, N + K + 1)
    got = host(tile(wq, ws))
    np.testing.assert_array_equal(got, records_weights(wq, ws))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,K", [(16, 512), (1, 256), (5, 1280), (16, 2048), (17, 512), (32, 256), (33, 768),
                                 (64, 512)])
def test_quantize_act_mma_layout(mode, B, K):
    """The words and scales are the oracle quantizer's, in the MFMA order, with a
    zero row's words and scale past the batch."""
    announce(f"quantize_act_mma mode={mode} B={B} K={K}")
    x = workloads.batch_activation(B, K, 40 + B + K, True, 41 + B + K)
    x[0, :32] = 0.0  # a zero block inside the batch
    oq, ol, os_ = oracle.quantize(mode, x)
    tq, tl, ts = acts(mode, x)
    wq_, ws_ = records_acts(oq, os_, B, zero_row_scale(mode))
    np.testing.assert_array_equal(host(tq), wq_)
    np.testing.assert_array_equal(host(ts).view(np.int32), ws_.view(np.int32))
    if mode == 2:
        wl_, _ = records_acts(ol, os_, B, zero_row_scale(mode))
        np.testing.assert_array_equal(host(tl), wl_)


CASES = [(16, 256, 5120, 1), (2, 33, 512, 1), (5, 100, 1536, 2), (16, 130, 768, 3), (11, 64, 25600, 4),
         (1, 77, 256, 1), (16, 200, 5120, 3), (7, 192, 1024, 1),
         (3, 40, 256, 2), (16, 64, 256, 4),  # these two: empty chunks
         (17, 100, 512, 1), (32, 64, 2048, 2), (40, 130, 768, 1), (64, 200, 1024, 3), (64, 16, 256, 2)]  # prefill


@pytest.mark.parametrize("groups", [1, 2])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,N,K,S", CASES)
def test_mma_tiled_bit_exact(B, N, K, S, mode, groups, tune):
    """Against the oracle bit for bit (y, or the chunk partials for S > 1), equal
    to qdg_gemv_q8 over the plain operands, and row t alone gives row t's bits."""
    announce(f"gemv_q8_mma_tiled mode={mode} B={B} N={N} K={K} S={S} groups={groups}")
    tune(mt_groups=groups)
    wq, ws, x = (*workloads.weights(N, K, 3 * N + K, 3 * N + K + 1),
                 workloads.batch_activation(B, K, 5 * B + K, True, 6 * B + K))
    oq, ol, os_ = oracle.quantize(mode, x)
    want = (oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_, nthreads=THREADS) if S == 1
            else oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=THREADS))
    wt = tile(wq, ws)
    tq, tl, ts = acts(mode, x)
    out = torch.full((S, B, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_mma_tiled(mode, wt, N, K, out, tq, tl, ts, B, splits=S)
    got = host(out)
    np.testing.assert_array_equal(got[0] if S == 1 else got, want)
    # the plain batched path on the plain operands gives the same bits
    xd = dev(x)
    pq = torch.empty((B, K), dtype=torch.int8, device=DEV)
    pl = torch.empty((B, K), dtype=torch.int8, device=DEV) if mode == 2 else None
    ps = torch.empty((B, K // 32), dtype=torch.float32, device=DEV)
    q.quantize_act(mode, xd, pq, pl, ps)
    plain = torch.full((S, B, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8(mode, dev(wq), dev(ws), plain, xq=pq, xl=pl, xs=ps, splits=S)
    assert host(plain).tobytes() == got.tobytes()
    for t in sorted({0, B - 1, min(16, B - 1)}):
        tq1, tl1, ts1 = acts(mode, x[t:t + 1])
        one = torch.full((S, 1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_mma_tiled(mode, wt, N, K, one, tq1, tl1, ts1, 1, splits=S)
        assert host(one)[:, 0].tobytes() == got[:, t].tobytes(), t


@pytest.mark.parametrize("mode", [1, 2])
def test_mma_tiled_decode_b16_full(mode):
    """The 16-row batch against 25600x5120 in the benchmark's launch: every output
    against the oracle, and a repeat gives the same bytes."""
    announce(f"gemv_q8_mma_tiled B=16 25600x5120 mode {mode}")
    d = workloads.make(workloads.BATCHED, 0)
    wq, ws, x = d["wq"], d["ws"], d["x"]
    B, K = x.shape
    N = wq.shape[0]
    oq, ol, os_ = oracle.quantize(mode, x)
    want = oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_, nthreads=THREADS)
    wt = tile(wq, ws)
    tq, tl, ts = acts(mode, x)
    outs = []
    for _ in range(2):
        y = torch.full((B, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_mma_tiled(mode, wt, N, K, y, tq, tl, ts, B)
        outs.append(host(y))
    np.testing.assert_array_equal(outs[0], want)
    assert outs[0].tobytes() == outs[1].tobytes()


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B", [40, 64])
def test_mma_tiled_prefill_full(mode, B):
    """A prefill chunk of B rows against 25600x5120: every output against the
    oracle, and the first 16 rows equal a 16-row call."""
    announce(f"gemv_q8_mma_tiled B={B} 25600x5120 mode {mode}")
    N, K = 25600, 5120
    wq, ws = workloads.weights(N, K, 71, 72)
    x = workloads.batch_activation(B, K, 73 + B, True, 74 + B)
    oq, ol, os_ = oracle.quantize(mode, x)
    want = oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_, nthreads=THREADS)
    wt = tile(wq, ws)
    tq, tl, ts = acts(mode, x)
    y = torch.full((B, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_mma_tiled(mode, wt, N, K, y, tq, tl, ts, B)
    got = host(y)
    np.testing.assert_array_equal(got, want)
    tq16, tl16, ts16 = acts(mode, x[:16])
    y16 = torch.full((16, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_mma_tiled(mode, wt, N, K, y16, tq16, tl16, ts16, 16)
    assert host(y16).tobytes() == got[:16].tobytes()


def ulp_diff(a, b):
    """Distance in binary32 units in the last place (sign-magnitude bit patterns)."""
    def key(v):
        i = np.asarray(v, np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7fffffff), i)
    return np.abs(key(a) - key(b))


def glu_outputs(mode, B, F, fill=True):
    R = q.mma_act_rows(B)
    hq = torch.full((R * F,), 77, dtype=torch.int8, device=DEV)
    hl = torch.full((R * F,), 77, dtype=torch.int8, device=DEV) if mode == 2 else None
    hs = torch.full((R * (F // 32),), float("nan"), dtype=torch.float32, device=DEV)
    return hq, hl, hs


def glu_three_calls(act, mode, wgt, wut, F, K, tq, tl, ts, B):
    """g and u by qdg_gemv_q8_mma_tiled, h by qdg_glu_quantize (f32 only), h's words
    by qdg_quantize_act_mma."""
    g = torch.full((B, F), float("nan"), dtype=torch.float32, device=DEV)
    u = torch.full((B, F), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_mma_tiled(mode, wgt, F, K, g, tq, tl, ts, B)
    q.gemv_q8_mma_tiled(mode, wut, F, K, u, tq, tl, ts, B)
    h = torch.empty((B, F), dtype=torch.float32, device=DEV)
    q.glu_quantize(act, 0, g, u, h)
    rq, rl, rs = glu_outputs(mode, B, F)
    q.quantize_act_mma(mode, h, rq, rl, rs)
    return g, u, h, rq, rl, rs


GLU_CASES = [(1, 256, 256), (5, 512, 768), (16, 768, 1024), (17, 256, 512), (33, 512, 256), (64, 256, 1280),
             (16, 1280, 5120)]


@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,F,K", GLU_CASES)
def test_glu_mma_tiled(B, F, K, mode, act):
    """qdg_gemv_glu_mma_tiled: h and its MFMA-ordered words equal two tiled GEMVs, the
    producer and the MFMA-order quantizer bit for bit; g and u of those calls equal the
    oracle's, h is within one ulp of the oracle's gated product of them, and the words
    are the oracle quantizer's on the kernel's h in the header's order (zero rows past
    the batch).  Without h the words are the same."""
    announce(f"gemv_glu_mma_tiled act={act} mode={mode} B={B} F={F} K={K}")
    wg, sg = workloads.weights(F, K, 7 * F + K, 7 * F + K + 1)
    wu, su = workloads.weights(F, K, 9 * F + K, 9 * F + K + 1)
    x = workloads.batch_activation(B, K, 11 * B + K, True, 12 * B + K)
    wgt, wut = tile(wg, sg), tile(wu, su)
    tq, tl, ts = acts(mode, x)
    hq, hl, hs = glu_outputs(mode, B, F)
    h = torch.full((B, F), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_glu_mma_tiled(act, mode, wgt, wut, F, K, tq, tl, ts, B, hq, hl, hs, h=h)
    g, u, h2, rq, rl, rs = glu_three_calls(act, mode, wgt, wut, F, K, tq, tl, ts, B)
    got = host(h)
    assert got.tobytes() == host(h2).tobytes()
    assert host(hq).tobytes() == host(rq).tobytes()
    assert host(hs).tobytes() == host(rs).tobytes()
    if mode == 2:
        assert host(hl).tobytes() == host(rl).tobytes()
    # against the oracle
    oq, ol, os_ = oracle.quantize(mode, x)
    og = oracle.gemv(mode, wg, sg, xq=oq, xl=ol, xs=os_, nthreads=THREADS)
    ou = oracle.gemv(mode, wu, su, xq=oq, xl=ol, xs=os_, nthreads=THREADS)
    np.testing.assert_array_equal(host(g), og)
    np.testing.assert_array_equal(host(u), ou)
    d = ulp_diff(got, oracle.glu(act, og, ou))
    assert d.max() <= 1 and np.count_nonzero(d) <= max(2, d.size // 1000)
    hq_o, hl_o, hs_o = oracle.quantize(mode, got)
    w_, s_ = records_acts(hq_o, hs_o, B, zero_row_scale(mode))
    np.testing.assert_array_equal(host(hq), w_)
    np.testing.assert_array_equal(host(hs).view(np.int32), s_.view(np.int32))
    if mode == 2:
        wl_, _ = records_acts(hl_o, hs_o, B, zero_row_scale(mode))
        np.testing.assert_array_equal(host(hl), wl_)
    # no h: the same words
    hq2, hl2, hs2 = glu_outputs(mode, B, F)
    q.gemv_glu_mma_tiled(act, mode, wgt, wut, F, K, tq, tl, ts, B, hq2, hl2, hs2)
    assert host(hq2).tobytes() == host(hq).tobytes() and host(hs2).tobytes() == host(hs).tobytes()
    if mode == 2:
        assert host(hl2).tobytes() == host(hl).tobytes()


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B", [16, 64])
def test_glu_mma_tiled_full(mode, B):
    """The gate and up halves of the 25600x5120 batched gate+up matrix (F = 12800): the
    words and h equal the three calls and the quantizer bit for bit, and the down
    projection over them (5120 rows, K = 12800) gives the same bytes either way."""
    announce(f"gemv_glu_mma_tiled full B={B} mode={mode}")
    F, K = 12800, 5120
    wq, ws = workloads.weights(2 * F, K, 81, 82)
    x = workloads.batch_activation(B, K, 83 + B, True, 84 + B)
    wgt, wut = tile(wq[:F], ws[:F]), tile(wq[F:], ws[F:])
    tq, tl, ts = acts(mode, x)
    hq, hl, hs = glu_outputs(mode, B, F)
    h = torch.full((B, F), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_glu_mma_tiled(0, mode, wgt, wut, F, K, tq, tl, ts, B, hq, hl, hs, h=h)
    _, _, h2, rq, rl, rs = glu_three_calls(0, mode, wgt, wut, F, K, tq, tl, ts, B)
    assert host(h).tobytes() == host(h2).tobytes()
    assert host(hq).tobytes() == host(rq).tobytes() and host(hs).tobytes() == host(rs).tobytes()
    if mode == 2:
        assert host(hl).tobytes() == host(rl).tobytes()
    wd, sd = workloads.weights(K, F, 85, 86)
    wdt = tile(wd, sd)
    y = torch.full((B, K), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_mma_tiled(mode, wdt, K, F, y, hq, hl, hs, B)
    y2 = torch.full((B, K), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_mma_tiled(mode, wdt, K, F, y2, rq, rl, rs, B)
    assert host(y).tobytes() == host(y2).tobytes()
    assert not np.isnan(host(y)).any()


def test_glu_mma_tiled_overlap_refused():
    """An output over an input is refused before any launch; outputs right after the inputs are not."""
    announce("gemv_glu_mma_tiled overlap")
    B, F, K, mode = 16, 256, 512, 1
    wg, sg = workloads.weights(F, K, 91, 92)
    wu, su = workloads.weights(F, K, 93, 94)
    x = workloads.batch_activation(B, K, 95)
    wgt, wut = tile(wg, sg), tile(wu, su)
    R = q.mma_act_rows(B)
    buf = torch.zeros(R * K + R * F, dtype=torch.int8, device=DEV)
    tq, hq = buf[:R * K], buf[R * K:]
    ts = torch.empty(R * (K // 32), dtype=torch.float32, device=DEV)
    q.quantize_act_mma(mode, dev(x), tq, None, ts)
    hs = torch.empty(R * (F // 32), dtype=torch.float32, device=DEV)
    q.gemv_glu_mma_tiled(0, mode, wgt, wut, F, K, tq, None, ts, B, hq, None, hs)
    _, _, _, rq, _, rs = glu_three_calls(0, mode, wgt, wut, F, K, tq, None, ts, B)
    assert host(hq).tobytes() == host(rq).tobytes() and host(hs).tobytes() == host(rs).tobytes()
    with pytest.raises(q.QdgError) as e:
        q.gemv_glu_mma_tiled(0, mode, wgt, wut, F, K, tq, None, ts, B, buf[R * K - 4:R * K - 4 + R * F], None, hs)
    assert e.value.status == -1
