"""GPU parity: every hot-path call of libqdg.so against the CPU oracle on the same
seeded inputs.

Bar: quantized words, scales, block dots, arg-max indices and the f32 outputs of
the quantized modes (whose order the kernels share with the oracle) are compared
bit for bit; Dequant outputs (a binary64 sum in the kernel's own order) within
|y - Y| <= 1e-5 * max(|Y|, ||t||_2) of the oracle's binary64 reference, and
almost always bit-equal to the oracle's own binary32 result.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_gemv_02_amd as q
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def dev(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def quantize_gpu(mode, x):
    xd = dev(x.reshape(-1, x.shape[-1]))
    B, K = xd.shape
    xq = torch.empty((B, K), dtype=torch.int8, device=DEV)
    xl = torch.empty((B, K), dtype=torch.int8, device=DEV) if mode == 2 else None
    xs = torch.empty((B, K // 32), dtype=torch.float32, device=DEV)
    q.quantize_act(mode, xd, xq, xl, xs)
    return xq, xl, xs


def gemv_gpu(mode, wqd, wsd, B, N, splits=1, x=None, xq=None, xl=None, xs=None):
    out = torch.full((splits, B, N) if splits > 1 else (B, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8(mode, wqd, wsd, out, x=x, xq=xq, xl=xl, xs=xs, splits=splits)
    return out


# ---------------------------------------------------------------- quantizer

@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,K,kind", [(1, 512, "normal"), (1, 25600, "outliers"), (16, 5120, "normal"),
                                      (3, 1600, "special"), (1, 32, "special")])
def test_quantize_bit_exact(mode, B, K, kind):
    announce(f"quantize mode={mode} B={B} K={K} {kind}")
    rng = np.random.default_rng(100 + K + B)
    x = rng.standard_normal((B, K)).astype(np.float32)
    if kind == "outliers":
        x = workloads.activation(K, 1, outliers=True, seed_out=2)[None, :]
    if kind == "special":
        x[:, :32] = 0.0                                   # zero block
        if K >= 128:
            x[:, 32:64] = np.arange(32) - 15.5            # ties after scaling
            x[:, 32] = 127.0
            x[:, 64:96] *= np.float32(1e-20)              # tiny but inside the contract
            x[:, 96:128] *= np.float32(1e20)              # huge
        x[:, 5] = -0.0
    xq, xl, xs = quantize_gpu(mode, x)
    oq, ol, os_ = oracle.quantize(mode, x)
    np.testing.assert_array_equal(host(xq), oq)
    np.testing.assert_array_equal(host(xs), os_)
    if mode == 2:
        np.testing.assert_array_equal(host(xl), ol)


# ---------------------------------------------------------------- block dots

@pytest.mark.parametrize("mode,B", [(1, 1), (2, 1), (1, 3), (2, 2)])
def test_block_dots_bit_exact(mode, B):
    announce(f"block_dots mode={mode} B={B}")
    rng = np.random.default_rng(7 * B + mode)
    N, K = 45, 32 * 37
    wq = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    xq = rng.integers(-128, 128, size=(B, K), dtype=np.int8)
    xl = rng.integers(-128, 128, size=(B, K), dtype=np.int8) if mode == 2 else None
    dh = torch.empty((B, N, K // 32), dtype=torch.int32, device=DEV)
    dl = torch.empty((B, N, K // 32), dtype=torch.int32, device=DEV) if mode == 2 else None
    q.block_dots(mode, dev(wq), dev(xq), dev(xl), dh, dl)
    rh, rl = oracle.block_dots(mode, wq, xq, xl)
    np.testing.assert_array_equal(host(dh), rh)
    if mode == 2:
        np.testing.assert_array_equal(host(dl), rl)


# ---------------------------------------------------------------- quantized GEMV

def _quant_case(N, K, B, seed, outliers=False):
    wq, ws = workloads.weights(N, K, seed, seed + 1)
    x = workloads.batch_activation(B, K, seed + 2, outliers, seed + 3 if outliers else None)
    return wq, ws, x


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("N,K", [(256, 512), (1, 32), (7, 96), (33, 544), (129, 1600), (70, 4096), (300, 25600),
                                 (40, 28672)])  # rows longer than one LDS window in both modes
def test_gemv_quantized_bit_exact(mode, N, K):
    announce(f"gemv mode={mode} N={N} K={K}")
    wq, ws, x = _quant_case(N, K, 1, 10 * N + K)
    oq, ol, os_ = oracle.quantize(mode, x)
    want = oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_, nthreads=8)
    xq, xl, xs = quantize_gpu(mode, x)
    y = gemv_gpu(mode, dev(wq), dev(ws), 1, N, xq=xq, xl=xl, xs=xs)
    np.testing.assert_array_equal(host(y), want)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("N,K", [(100, 25600), (64, 8192), (17, 1600), (9, 256), (50, 12288)])
@pytest.mark.parametrize("S", [1, 2, 3, 4, 8, 64])
def test_split_partials_and_combine_bit_exact(mode, N, K, S):
    announce(f"split mode={mode} N={N} K={K} S={S}")
    wq, ws, x = _quant_case(N, K, 1, 3 * N + K + S, outliers=True)
    oq, ol, os_ = oracle.quantize(mode, x)
    want_part = oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8)
    xq, xl, xs = quantize_gpu(mode, x)
    part = gemv_gpu(mode, dev(wq), dev(ws), 1, N, splits=S, xq=xq, xl=xl, xs=xs)
    if S == 1:
        part = part.reshape(1, 1, N)
    np.testing.assert_array_equal(host(part), want_part)
    y = torch.empty((1, N), dtype=torch.float32, device=DEV)
    q.sk_combine(part, y)
    np.testing.assert_array_equal(host(y), oracle.combine(want_part))
    if S == 1:
        np.testing.assert_array_equal(host(y), oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_))


def test_combine_golden_and_random(golden_dir):
    import json
    for c in json.load(open(os.path.join(golden_dir, "combine_order.json")))["cases"]:
        p = np.array(c["partials"], np.float32).reshape(-1, 1, 1)
        y = torch.empty((1, 1), dtype=torch.float32, device=DEV)
        q.sk_combine(dev(p), y)
        assert host(y)[0, 0] == np.float32(c["y"])
    rng = np.random.default_rng(5)
    p = (rng.standard_normal((7, 3, 1001)) * 10.0 ** rng.integers(-8, 8, size=(7, 3, 1001))).astype(np.float32)
    y = torch.empty((3, 1001), dtype=torch.float32, device=DEV)
    q.sk_combine(dev(p), y)
    np.testing.assert_array_equal(host(y), oracle.combine(p))


# ---------------------------------------------------------------- batched (MFMA)

@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,N,K,S", [(16, 256, 5120, 1), (2, 33, 512, 1), (5, 100, 1600, 2), (16, 40, 96, 1),
                                     (11, 64, 25600, 4), (3, 17, 32, 1), (16, 96, 8192, 3),
                                     (3, 40, 256, 2), (16, 64, 480, 4)])  # the last two: empty chunks
def test_batched_bit_exact_and_batch_invariant(mode, B, N, K, S):
    announce(f"batched mode={mode} B={B} N={N} K={K} S={S}")
    wq, ws, x = _quant_case(N, K, B, 5 * B + N + K)
    oq, ol, os_ = oracle.quantize(mode, x)
    xq, xl, xs = quantize_gpu(mode, x)
    wqd, wsd = dev(wq), dev(ws)
    out = gemv_gpu(mode, wqd, wsd, B, N, splits=S, xq=xq, xl=xl, xs=xs)
    if S == 1:
        np.testing.assert_array_equal(host(out), oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_, nthreads=8))
    else:
        np.testing.assert_array_equal(host(out), oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8))
    # row t of the batch equals the batch-1 kernel on row t, bit for bit
    for t in (0, B - 1):
        y1 = gemv_gpu(mode, wqd, wsd, 1, N, splits=S, xq=xq[t:t + 1].contiguous(),
                      xl=None if xl is None else xl[t:t + 1].contiguous(), xs=xs[t:t + 1].contiguous())
        got = host(out)
        np.testing.assert_array_equal(got[:, t] if S > 1 else got[t], host(y1)[:, 0] if S > 1 else host(y1)[0])


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,N,K,S", [(64, 100, 5120, 1), (17, 33, 256, 1), (32, 64, 2048, 2), (33, 65, 512, 1),
                                     (48, 130, 8192, 3), (64, 16, 256, 2), (40, 300, 25600, 4)])
def test_prefill_chunk_bit_exact_and_batch_invariant(mode, B, N, K, S):
    """More than 16 activation rows (a prefill chunk): every weight step meets 2 or
    4 activation tiles.  Bit-exact with the oracle; each row equals the batch-1
    kernel's result, and the first 16 rows equal a 16-row call."""
    announce(f"prefill chunk mode={mode} B={B} N={N} K={K} S={S}")
    wq, ws, x = _quant_case(N, K, B, 13 * B + N + K)
    oq, ol, os_ = oracle.quantize(mode, x)
    xq, xl, xs = quantize_gpu(mode, x)
    wqd, wsd = dev(wq), dev(ws)
    got = host(gemv_gpu(mode, wqd, wsd, B, N, splits=S, xq=xq, xl=xl, xs=xs))
    want = (oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_, nthreads=8) if S == 1
            else oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8))
    np.testing.assert_array_equal(got, want)
    for t in (0, 16, B - 1):
        y1 = host(gemv_gpu(mode, wqd, wsd, 1, N, splits=S, xq=xq[t:t + 1].contiguous(),
                           xl=None if xl is None else xl[t:t + 1].contiguous(), xs=xs[t:t + 1].contiguous()))
        np.testing.assert_array_equal(got[:, t] if S > 1 else got[t], y1[:, 0] if S > 1 else y1[0])
    y16 = host(gemv_gpu(mode, wqd, wsd, 16, N, splits=S, xq=xq[:16].contiguous(),
                        xl=None if xl is None else xl[:16].contiguous(), xs=xs[:16].contiguous()))
    np.testing.assert_array_equal(got[:, :16] if S > 1 else got[:16], y16)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B", [1, 16])
def test_weight_scales_at_a_two_byte_offset(mode, B):
    """The header asks only 2-byte alignment of ws: scales that start 2 bytes past a
    16-byte boundary (K a multiple of 256, where 16-byte scale words would otherwise
    be used) give the same bits."""
    N, K = 70, 5120
    announce(f"ws offset mode={mode} B={B} N={N} K={K}")
    wq, ws, x = _quant_case(N, K, B, 77 + B)
    oq, ol, os_ = oracle.quantize(mode, x)
    want = oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_, nthreads=8)
    buf = torch.empty(N * (K // 32) + 8, dtype=torch.int16, device=DEV)
    wsd = buf[1:1 + N * (K // 32)].view(N, K // 32)
    wsd.copy_(dev(ws))
    assert wsd.data_ptr() % 16 == 2
    xq, xl, xs = quantize_gpu(mode, x)
    y = gemv_gpu(mode, dev(wq), wsd, B, N, xq=xq, xl=xl, xs=xs)
    np.testing.assert_array_equal(host(y), want)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("B,N,K,S", [(16, 100, 5120, 1), (7, 64, 2048, 2), (16, 33, 256, 2)])
def test_batched_general_path_on_fast_path_shapes(mode, B, N, K, S, tune):
    """Shapes with K a multiple of 256 take the LDS-direct batched kernel; the
    general kernel (forced by the mfma_general tuning knob) must give the same bits there."""
    announce(f"batched general path mode={mode} B={B} N={N} K={K} S={S}")
    wq, ws, x = _quant_case(N, K, B, 9 * B + N + K)
    oq, ol, os_ = oracle.quantize(mode, x)
    want = (oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_, nthreads=8) if S == 1
            else oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8))
    xq, xl, xs = quantize_gpu(mode, x)
    wqd, wsd = dev(wq), dev(ws)
    fast = host(gemv_gpu(mode, wqd, wsd, B, N, splits=S, xq=xq, xl=xl, xs=xs))
    tune(mfma_general=1)
    general = host(gemv_gpu(mode, wqd, wsd, B, N, splits=S, xq=xq, xl=xl, xs=xs))
    np.testing.assert_array_equal(fast, want)
    np.testing.assert_array_equal(general, want)


# ---------------------------------------------------------------- Dequant

@pytest.mark.parametrize("N,K", [(256, 512), (1, 32), (37, 1600), (64, 12288), (20, 5120), (5, 25600)])
@pytest.mark.parametrize("kernel", ["chunk-waves", "workspace"])
def test_dequant_tolerance(N, K, kernel, tune):
    announce(f"dequant N={N} K={K} {kernel}")
    if kernel == "workspace":
        tune(dq_seg=0)
    wq, ws, x = _quant_case(N, K, 1, N + 3 * K, outliers=True)
    y = host(gemv_gpu(0, dev(wq), dev(ws), 1, N, x=dev(x)))
    Y, tn = oracle.reference_f64(0, wq, ws, x=x)
    assert oracle.within_tolerance(y, Y, tn).all()
    same = (y == oracle.gemv(0, wq, ws, x=x)).mean()
    if N >= 20:
        assert same >= 0.95, same


# ---------------------------------------------------------------- arg-max

def argmax_gpu(y):
    y = np.atleast_2d(y).astype(np.float32)
    B, N = y.shape
    idx = torch.empty(B, dtype=torch.int32, device=DEV)
    wsp = torch.empty(q.argmax_workspace_bytes(B, N) // 8, dtype=torch.int64, device=DEV)
    q.argmax(dev(y), idx, wsp)
    return host(idx)


def test_argmax_random_and_ties():
    announce("argmax random")
    for seed in range(60):
        rng = np.random.default_rng(seed)
        N = int(rng.choice([1, 2, 63, 2047, 2048, 2049, 4096, 10000, 151936]))
        B = int(rng.integers(1, 4))
        y = rng.standard_normal((B, N)).astype(np.float32)
        if seed % 3 == 0:
            y = np.round(y).astype(np.float32)  # many exact ties
        np.testing.assert_array_equal(argmax_gpu(y), oracle.argmax(y))


@pytest.mark.parametrize("N", [151936, 4096, 5000])
def test_argmax_planted_ties_adversarial(N):
    announce(f"argmax planted N={N}")
    G = -(-N // 2048)
    G = min(max(G, 1), 256)
    per = -(-N // G)
    pairs = [(0, N - 1), (per - 1, per), (per, min(2 * per - 1, N - 1)), (N - 2, N - 1), (1, 0)]
    rng = np.random.default_rng(N)
    for a, b in pairs:
        y = rng.standard_normal(N).astype(np.float32)
        y[a] = y[b] = np.float32(9.0)
        assert argmax_gpu(y)[0] == min(a, b)
    y = np.zeros(N, np.float32)
    assert argmax_gpu(y)[0] == 0
    y = np.full(N, -3.0, np.float32)
    y[N // 2] = -0.0
    y[N // 3] = 0.0
    assert argmax_gpu(y)[0] == min(N // 2, N // 3)
    y = np.full(N, -np.inf, np.float32)
    assert argmax_gpu(y)[0] == 0


# ---------------------------------------------------------------- determinism

def test_repeat_and_fresh_buffers_bitwise():
    announce("determinism")
    N, K = 1000, 8192
    wq, ws, x = _quant_case(N, K, 1, 77, outliers=True)
    for mode in (0, 1, 2):
        outs = []
        for rep in range(5):
            wqd, wsd = dev(wq), dev(ws)  # fresh allocations each time
            if mode == 0:
                outs.append(host(gemv_gpu(0, wqd, wsd, 1, N, x=dev(x))))
            else:
                xq, xl, xs = quantize_gpu(mode, x)
                part = gemv_gpu(mode, wqd, wsd, 1, N, splits=4, xq=xq, xl=xl, xs=xs)
                y = torch.empty((1, N), dtype=torch.float32, device=DEV)
                q.sk_combine(part, y)
                outs.append(host(y))
        for o in outs[1:]:
            assert o.tobytes() == outs[0].tobytes()


# ---------------------------------------------------------------- split-K with in-kernel combine

@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("N,K,S", [(256, 512, 1), (100, 25600, 8), (33, 1600, 4), (70, 8192, 3), (9, 256, 2),
                                   (17, 1600, 64), (129, 4096, 1), (1, 32, 1), (5, 544, 5), (5120, 8192, 4)])
@pytest.mark.parametrize("path", ["default", "workspace"])
def test_in_kernel_combine_bit_exact(mode, N, K, S, path, tune):
    announce(f"gemv_q8_sk mode={mode} N={N} K={K} S={S} {path}")
    if path == "workspace":
        tune(sk_wsplit=0)
    wq, ws, x = _quant_case(N, K, 1, 11 * N + K + S, outliers=True)
    oq, ol, os_ = oracle.quantize(mode, x)
    want = oracle.combine(oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8))
    wqd, wsd = dev(wq), dev(ws)
    xq, xl, xs = quantize_gpu(mode, x)
    wsp = q.sk_workspace(N, S)
    for rep in range(3):  # the workspace must come back to zero after every call
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_sk(mode, wqd, wsd, y, xq, xl, xs, S, wsp)
        np.testing.assert_array_equal(host(y), want)
    assert not host(wsp).any()  # tickets and partial slots all back at zero


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("N,K,S", [(5120, 25600, 16), (5120, 8192, 4), (77, 8192, 8), (4097, 1600, 16),
                                   (33, 544, 4), (9, 256, 8), (1, 32, 16), (130, 12288, 8), (20, 25632, 16),
                                   (5120, 25600, 5), (640, 25600, 10), (300, 25600, 13), (50, 25632, 12),
                                   (21, 8192, 3), (64, 4608, 2), (19, 1056, 7),
                                   # the largest TwoPass rows the LDS budget takes (three, two, one row groups)
                                   (24, 28128, 5), (24, 30720, 8), (8, 34048, 16)])
@pytest.mark.parametrize("variant", ["dma", "barrier", "wave-local"])
def test_in_workgroup_split_bit_exact(mode, N, K, S, variant, tune):
    """The split-K GEMV whose chunks are the waves of one workgroup (partials
    combined in LDS) against the oracle's chunk partials and ascending combine,
    with each staging of the activation: LDS DMA (K a multiple of 256; other K
    fall back to the workgroup copy), the workgroup-wide copy, the per-wave copy."""
    announce(f"gemv_q8_sk in-workgroup split mode={mode} N={N} K={K} S={S} {variant}")
    if variant == "dma":
        tune(ws_dma=-1)
        tune(ws_local=0)
    else:
        tune(ws_dma=0)
        tune(ws_local=1 if variant == "wave-local" else 0)
    wq, ws, x = _quant_case(N, K, 1, 17 * N + K + S, outliers=True)
    oq, ol, os_ = oracle.quantize(mode, x)
    if N > 1000:  # the oracle on every 7th row (the rows are independent)
        rows = np.arange(0, N, 7)
        want = oracle.combine(oracle.gemv_split(mode, wq[rows], ws[rows], oq, ol, os_, S, nthreads=8))
    else:
        rows, want = np.arange(N), oracle.combine(oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8))
    wqd, wsd = dev(wq), dev(ws)
    xq, xl, xs = quantize_gpu(mode, x)
    wsp = q.sk_workspace(N, S)
    for rep in range(2):
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_sk(mode, wqd, wsd, y, xq, xl, xs, S, wsp)
        np.testing.assert_array_equal(host(y)[:, rows], want)
    tune(sk_wsplit=0)  # the workspace path: the same bits
    y2 = torch.empty((1, N), dtype=torch.float32, device=DEV)
    q.gemv_q8_sk(mode, wqd, wsd, y2, xq, xl, xs, S, wsp)
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("N,K,S", [(70, 5120, 5), (300, 25600, 5), (21, 8192, 3)])
def test_in_workgroup_split_unaligned_scales(mode, N, K, S):
    """The in-workgroup split-K GEMV with the weight scales 2 bytes and the activation
    scales 4 bytes past a 16-byte boundary (what the header allows): K is a multiple
    of 256, so aligned inputs would be staged by LDS DMA; these fall back to the
    copy through registers and give the oracle's bits, and the aligned call's."""
    announce(f"gemv_q8_sk unaligned scales mode={mode} N={N} K={K} S={S}")
    assert q.sk_combines_in_workgroup(mode, K, S)
    wq, ws, x = _quant_case(N, K, 1, 31 * N + K + S, outliers=True)
    oq, ol, os_ = oracle.quantize(mode, x)
    want = oracle.combine(oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8))
    nb = K // 32
    wbuf = torch.empty(N * nb + 8, dtype=torch.int16, device=DEV)
    wsd = wbuf[1:1 + N * nb].view(N, nb)
    wsd.copy_(dev(ws))
    assert wsd.data_ptr() % 16 == 2
    xq, xl, xs = quantize_gpu(mode, x)
    sbuf = torch.empty(nb + 4, dtype=torch.float32, device=DEV)
    xs_off = sbuf[1:1 + nb].view(1, nb)
    xs_off.copy_(xs.view(1, nb))
    assert xs_off.data_ptr() % 16 == 4
    wsp = q.sk_workspace(N, S)
    wqd = dev(wq)
    y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_sk(mode, wqd, wsd, y, xq, xl, xs_off, S, wsp)
    np.testing.assert_array_equal(host(y), want)
    y2 = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_sk(mode, wqd, dev(ws), y2, xq, xl, xs, S, wsp)  # aligned: the DMA staging
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("N,K", [(4, 256), (8, 512), (20, 2304), (516, 5120), (5120, 25600)])
def test_tile_rows_bit_exact(N, K):
    """Row tiles of four rows by 256 values: every byte where the oracle's layout puts it."""
    announce(f"q8_tile_rows N={N} K={K}")
    wq = np.random.default_rng(N + K).integers(-128, 128, size=(N, K), dtype=np.int8)
    wt = torch.empty((N, K), dtype=torch.int8, device=DEV)
    q.q8_tile_rows(dev(wq), wt)
    np.testing.assert_array_equal(host(wt), oracle.tile_rows(wq))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("N,K,S", [(5120, 25600, 5), (5120, 8192, 5), (5120, 25600, 16), (640, 25600, 10),
                                   (40, 25600, 5), (100, 8192, 4), (4, 1024, 2), (12, 768, 3), (36, 1280, 5),
                                   (24, 27904, 5), (8, 33792, 16), (64, 4608, 2)])
@pytest.mark.parametrize("variant", ["dma", "barrier", "wave-local"])
def test_in_workgroup_split_tiled_bit_exact(mode, N, K, S, variant, tune):
    """The in-workgroup split-K GEMV over row-tiled weights: the oracle's chunk
    partials and ascending combine bit for bit, and the plain-layout call's bits,
    with each staging of the activation (the weight addressing is the same in all)."""
    announce(f"gemv_q8_sk_tiled mode={mode} N={N} K={K} S={S} {variant}")
    if variant == "dma":
        tune(ws_dma=-1)
        tune(ws_local=0)
    else:
        tune(ws_dma=0)
        tune(ws_local=1 if variant == "wave-local" else 0)
    assert q.sk_combines_in_workgroup(mode, K, S)
    wq, ws, x = _quant_case(N, K, 1, 23 * N + K + S, outliers=True)
    oq, ol, os_ = oracle.quantize(mode, x)
    rows = np.arange(0, N, 7) if N > 1000 else np.arange(N)
    want = oracle.combine(oracle.gemv_split(mode, wq[rows], ws[rows], oq, ol, os_, S, nthreads=8))
    wqd, wsd = dev(wq), dev(ws)
    wt = torch.empty_like(wqd)
    q.q8_tile_rows(wqd, wt)
    xq, xl, xs = quantize_gpu(mode, x)
    for rep in range(2):
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_sk_tiled(mode, wt, wsd, y, xq, xl, xs, S)
        np.testing.assert_array_equal(host(y)[:, rows], want)
    y2 = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_sk(mode, wqd, wsd, y2, xq, xl, xs, S, q.sk_workspace(N, S))
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("N,K,S", [(256, 512, 1), (100, 25600, 16), (33, 1600, 4), (70, 8192, 3), (9, 256, 2),
                                   (17, 1600, 64), (129, 4096, 1), (1, 32, 1), (5, 544, 5), (5120, 8192, 4),
                                   (40, 25632, 7)])
def test_fused_single_launch_bit_exact(mode, N, K, S):
    """qdg_gemv_q8_fused (quantize in the workgroup + split-K GEMV + in-kernel
    combine) against the oracle's quantize -> chunk partials -> ascending combine."""
    announce(f"gemv_q8_fused mode={mode} N={N} K={K} S={S}")
    wq, ws, x = _quant_case(N, K, 1, 13 * N + K + S, outliers=True)
    oq, ol, os_ = oracle.quantize(mode, x)
    want = oracle.combine(oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8))
    wqd, wsd, xd = dev(wq), dev(ws), dev(x.reshape(1, K))
    wsp = q.sk_workspace(N, S)
    for rep in range(3):  # the workspace must come back to zero after every call
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_fused(mode, wqd, wsd, y, xd, S, wsp)
        np.testing.assert_array_equal(host(y), want)
    assert not host(wsp).any()  # tickets and partial slots all back at zero


def test_fused_single_launch_dequant_and_edge_inputs():
    """Dequant through the fused entry point (S = 1), and quantizer edge blocks
    (zero, tiny, huge, ties) reaching the in-workgroup quantizer."""
    N, K = 37, 1600
    announce(f"gemv_q8_fused dequant + edge inputs N={N} K={K}")
    wq, ws, x = _quant_case(N, K, 1, 4242)
    y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8_fused(0, dev(wq), dev(ws), y, dev(x.reshape(1, K)))
    Y, tn = oracle.reference_f64(0, wq, ws, x=x)
    assert oracle.within_tolerance(host(y), Y, tn).all()
    x = x.copy()
    x[0, :32] = 0.0
    x[0, 32:64] = 1e-20
    x[0, 64:96] = 3e4
    x[0, 96:128] = np.arange(32, dtype=np.float32) - 15.5
    for mode in (1, 2):
        oq, ol, os_ = oracle.quantize(mode, x)
        want = oracle.combine(oracle.gemv_split(mode, wq, ws, oq, ol, os_, 2, nthreads=8))
        wsp = q.sk_workspace(N, 2)
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_fused(mode, dev(wq), dev(ws), y, dev(x.reshape(1, K)), 2, wsp)
        np.testing.assert_array_equal(host(y), want)


@pytest.mark.parametrize("N,K,S", [(37, 1600, 2), (100, 25600, 16), (5120, 8192, 4), (9, 256, 2), (65, 25632, 7)])
@pytest.mark.parametrize("kernel", ["chunk-waves", "workspace"])
def test_fused_dequant_split_k(N, K, S, kernel, tune):
    """Dequant split-K (binary64 chunk partials, ascending binary64 combine, one
    rounding): within the Dequant tolerance of the binary64 reference, and almost
    always the oracle's own binary32 result."""
    announce(f"gemv_q8_fused dequant N={N} K={K} S={S} {kernel}")
    if kernel == "workspace":
        tune(dq_seg=0)
    wq, ws, x = _quant_case(N, K, 1, 17 * N + K + S, outliers=True)
    Y, tn = oracle.reference_f64(0, wq, ws, x=x, nthreads=8)
    want32 = oracle.gemv(0, wq, ws, x=x, nthreads=8)
    wsp = q.sk_workspace(N, S)
    for rep in range(3):
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_fused(0, dev(wq), dev(ws), y, dev(x.reshape(1, K)), S, wsp)
        got = host(y)
        assert oracle.within_tolerance(got, Y, tn).all()
        assert (got == want32).mean() > 0.99
    assert not host(wsp).any()  # tickets and partial slots all back at zero


@pytest.mark.parametrize("N,K,S", [(300, 25600, 8), (300, 25632, 5), (37, 8192, 16)])
def test_dequant_chunk_waves_several_chunks_a_wave(N, K, S, tune):
    """Waves that sum several chunks of the Dequant chunk-wave kernel one after
    another (the wave count forced below the chunk count): the same bits as a
    wave a chunk, and within the Dequant tolerance of the binary64 reference."""
    wq, ws, x = _quant_case(N, K, 1, 31 * N + K + S, outliers=True)
    Y, tn = oracle.reference_f64(0, wq, ws, x=x, nthreads=8)
    wsp = q.sk_workspace(N, S)
    outs = {}
    for W in (16, 1, 2, 3):
        announce(f"dequant chunk waves N={N} K={K} S={S} W={W}")
        tune(dq_waves=W)
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_fused(0, dev(wq), dev(ws), y, dev(x.reshape(1, K)), S, wsp)
        outs[W] = host(y)
    assert oracle.within_tolerance(outs[16], Y, tn).all()
    for W in (1, 2, 3):
        assert outs[W].tobytes() == outs[16].tobytes(), W


@pytest.mark.parametrize("N,K,S", [(37, 1600, 2), (100, 25600, 16), (5120, 8192, 4), (9, 256, 2), (65, 25632, 7),
                                   (5120, 25600, 5), (300, 25600, 1), (1, 32, 1), (130, 12288, 8), (21, 4608, 3)])
@pytest.mark.parametrize("variant", ["R1", "R2", "R3", "R4"])
def test_dequant_chunk_waves(N, K, S, variant, tune):
    """The Dequant GEMV whose chunks are waves of one workgroup (8 values a lane,
    binary64 throughout, chunk partials added in LDS): within the Dequant
    tolerance of the binary64 reference, almost always the oracle's binary32
    result, and bit-identical on repeat."""
    announce(f"dequant chunk waves N={N} K={K} S={S} {variant}")
    tune(dq_rows=int(variant[1]))
    wq, ws, x = _quant_case(N, K, 1, 23 * N + K + S, outliers=True)
    rows = np.arange(0, N, 7) if N > 1000 else np.arange(N)
    Y, tn = oracle.reference_f64(0, wq[rows], ws[rows], x=x, nthreads=8)
    want32 = oracle.gemv(0, wq[rows], ws[rows], x=x, nthreads=8)
    wsp = q.sk_workspace(N, S)
    outs = []
    for rep in range(2):
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_q8_fused(0, dev(wq), dev(ws), y, dev(x.reshape(1, K)), S, wsp)
        outs.append(host(y))
    got = outs[0][:, rows]
    assert oracle.within_tolerance(got, Y, tn).all()
    if len(rows) >= 20:
        assert (got == want32).mean() > 0.95
    assert outs[0].tobytes() == outs[1].tobytes()


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("N,K", [(4097, 512), (33, 1600), (5000, 544), (16, 96)])
def test_gemv_argmax_epilogue(mode, N, K):
    """qdg_gemv_q8_argmax: the logits equal qdg_gemv_q8's bit for bit, and the index
    is the first of the maxima -- planted exact ties inside one 16-row tile, across
    a tile boundary, and at (0, N-1), each with the later row in the later tile."""
    announce(f"gemv_q8_argmax mode={mode} N={N} K={K}")
    wq, ws, x = _quant_case(N, K, 1, 19 * N + K + mode)
    wsp = q.gemv_argmax_workspace(N)
    for a, b in [(2, 5), (15, 16), (0, N - 1), (N // 2, N - 2)]:
        if not 0 <= a < b < N:
            continue
        w2, s2, x2 = wq.copy(), ws.copy(), x.copy()
        workloads.plant_tie(w2, s2, x2[0], a, b)
        wqd, wsd = dev(w2), dev(s2)
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        idx = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        y_ref = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        if mode == 0:
            xd = dev(x2)
            q.gemv_q8_argmax(0, wqd, wsd, y, idx, wsp, x=xd)
            q.gemv_q8(0, wqd, wsd, y_ref, x=xd)
        else:
            xq, xl, xs = quantize_gpu(mode, x2)
            q.gemv_q8_argmax(mode, wqd, wsd, y, idx, wsp, xq=xq, xl=xl, xs=xs)
            q.gemv_q8(mode, wqd, wsd, y_ref, xq=xq, xl=xl, xs=xs)
        got = host(y)
        np.testing.assert_array_equal(got, host(y_ref))
        assert int(host(idx)[0]) == int(oracle.argmax(got)[0]) == a


# ---------------------------------------------------------------- several matrices in one launch

@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("Ns,K,S", [((4096, 1024, 1024), 4096, 4), ((37, 1, 200), 1600, 2),
                                    ((12288, 12288), 4096, 2), ((5, 7, 9, 11, 13, 15), 544, 4),
                                    ((300,), 25600, 5), ((64, 65), 8192, 8)])
def test_parts_match_single_calls(mode, Ns, K, S):
    """qdg_gemv_q8_parts: every part's output is bit-identical to the single-matrix
    call with the same splits, and (quantized modes) to the oracle's chunk
    partials and ascending combine; Dequant within its tolerance."""
    announce(f"gemv_q8_parts mode={mode} Ns={Ns} K={K} S={S}")
    x = workloads.batch_activation(1, K, 31 + K, True, 32 + K)
    mats = [workloads.weights(n, K, 100 * i + n, 100 * i + n + 1) for i, n in enumerate(Ns)]
    dev_m = [(dev(wq), dev(ws)) for wq, ws in mats]
    ys = [torch.full((n,), float("nan"), dtype=torch.float32, device=DEV) for n in Ns]
    if mode == 0:
        xd = dev(x.reshape(1, K))
        q.gemv_q8_parts(0, [(w, s, y) for (w, s), y in zip(dev_m, ys)], x=xd, splits=S)
    else:
        xq, xl, xs = quantize_gpu(mode, x)
        q.gemv_q8_parts(mode, [(w, s, y) for (w, s), y in zip(dev_m, ys)], xq=xq, xl=xl, xs=xs, splits=S)
        oq, ol, os_ = oracle.quantize(mode, x)
    for i, n in enumerate(Ns):
        single = torch.empty((1, n), dtype=torch.float32, device=DEV)
        wsp = q.sk_workspace(n, S)
        if mode == 0:
            q.gemv_q8_fused(0, dev_m[i][0], dev_m[i][1], single, xd, S, wsp)
        else:
            q.gemv_q8_sk(mode, dev_m[i][0], dev_m[i][1], single, xq, xl, xs, S, wsp)
        got = host(ys[i]).reshape(1, n)
        assert got.tobytes() == host(single).tobytes(), i
        rows = np.arange(0, n, 7) if n > 2000 else np.arange(n)
        wq, ws = mats[i]
        if mode == 0:
            Y, tn = oracle.reference_f64(0, wq[rows], ws[rows], x=x, nthreads=8)
            assert oracle.within_tolerance(got[:, rows], Y, tn).all()
        else:
            want = oracle.combine(oracle.gemv_split(mode, wq[rows], ws[rows], oq, ol, os_, S, nthreads=8))
            np.testing.assert_array_equal(got[:, rows], want)
