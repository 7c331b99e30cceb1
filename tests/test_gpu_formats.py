"""GPU parity of the block-format GEMV (qdg_gemv_fmt) against the CPU oracle,
for all twelve GGUF formats and all three numerics modes.

Bar: the quantized modes bit-exact (the kernel runs the oracle's order); Dequant
(a binary64 sum in the kernel's own fixed order) within one unit in the last
place of the oracle's binary32 result and equal to it almost everywhere; every
call byte-identical on repeat.  Row sizes include ones that leave rows 2 bytes
off a 4-byte boundary (the loaders' 2-byte path).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_gemv_02_amd as q
from gguf_blocks import SUPER, encode

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def shapes(fmt):
    if fmt in SUPER:
        return [(37, 256), (5, 512), (70, 2560), (300, 5120)]
    return [(37, 288), (5, 512), (70, 1600), (300, 5120)]


CASES = [(f, N, K) for f in oracle.FORMATS for (N, K) in shapes(f)]


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("fmt,N,K", CASES)
def test_fmt_quantized_bit_exact(fmt, N, K, mode):
    announce(f"gemv_fmt fmt={fmt} mode={mode} N={N} K={K}")
    rng = np.random.default_rng(1000 * fmt + N + K + mode)
    w, _, _, _ = encode(fmt, N, K, rng)
    x = rng.standard_normal((1, K)).astype(np.float32)
    x[0, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    oq, ol, os_ = oracle.quantize(mode, x)
    want = oracle.gemv_fmt(fmt, mode, w, N, K, xq=oq, xl=ol, xs=os_, nthreads=8)
    dw = dev(w.reshape(-1))
    xq, xl, xs = dev(oq), None if ol is None else dev(ol), dev(os_)
    outs = []
    for rep in range(2):
        y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
        q.gemv_fmt(fmt, mode, dw, N, K, y, xq=xq, xl=xl, xs=xs)
        outs.append(host(y))
    np.testing.assert_array_equal(outs[0], want[0])
    assert outs[0].tobytes() == outs[1].tobytes()


@pytest.mark.parametrize("fmt,N,K", CASES)
def test_fmt_dequant(fmt, N, K):
    announce(f"gemv_fmt fmt={fmt} dequant N={N} K={K}")
    rng = np.random.default_rng(2000 * fmt + N + K)
    w, _, _, _ = encode(fmt, N, K, rng)
    x = rng.standard_normal((1, K)).astype(np.float32)
    want = oracle.gemv_fmt(fmt, 0, w, N, K, x=x, nthreads=8)[0]
    y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_fmt(fmt, 0, dev(w.reshape(-1)), N, K, y, x=dev(x))
    got = host(y)
    d = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert d.max() <= 1, (int(d.max()), int(d.argmax()))
    if N >= 20:
        assert np.mean(d == 0) >= 0.95
    y2 = torch.empty_like(y)
    q.gemv_fmt(fmt, 0, dev(w.reshape(-1)), N, K, y2, x=dev(x))
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))


def split_cases(fmt):
    ragged = 2816 if fmt in SUPER else 1600          # whole 512-value groups plus a tail
    small = 256 if fmt in SUPER else 288             # below one group: all of it in the last chunk
    return [(300, 5120, 5), (300, 5120, 16), (70, ragged, 3), (37, small, 4), (45, 4608, 2)]


SPLIT_CASES = [(f, N, K, S) for f in oracle.FORMATS for (N, K, S) in split_cases(f)]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("fmt,N,K,S", SPLIT_CASES)
def test_fmt_split(fmt, N, K, S, mode):
    """Split-K chunks as waves of a workgroup, added in ascending order: the
    quantized modes bit-exact with the oracle's chunked sum, Dequant within one
    unit in the last place of it."""
    announce(f"gemv_fmt split fmt={fmt} mode={mode} N={N} K={K} S={S}")
    rng = np.random.default_rng(3000 * fmt + N + K + 7 * S + mode)
    w, _, _, _ = encode(fmt, N, K, rng)
    x = rng.standard_normal((1, K)).astype(np.float32)
    dw = dev(w.reshape(-1))
    y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    y2 = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    if mode == 0:
        want = oracle.gemv_fmt(fmt, 0, w, N, K, x=x, splits=S, nthreads=8)[0]
        for t in (y, y2):
            q.gemv_fmt(fmt, 0, dw, N, K, t, x=dev(x), splits=S)
        got = host(y)
        d = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
        assert d.max() <= 1, (int(d.max()), int(d.argmax()))
    else:
        oq, ol, os_ = oracle.quantize(mode, x)
        want = oracle.gemv_fmt(fmt, mode, w, N, K, xq=oq, xl=ol, xs=os_, splits=S, nthreads=8)[0]
        xq, xl, xs = dev(oq), None if ol is None else dev(ol), dev(os_)
        for t in (y, y2):
            q.gemv_fmt(fmt, mode, dw, N, K, t, xq=xq, xl=xl, xs=xs, splits=S)
        np.testing.assert_array_equal(host(y), want)
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))


def test_chunk_wave_queries(tune):
    """The wave counts the launches use: within 1..min(chunks, 16), the knobs
    reflected (clamped to the chunk count), QDG_EMODE where the Dequant
    chunk-wave kernel does not serve the shape."""
    announce("chunk-wave queries")
    for fmt, mode, N, K, S, ceff in ((11, 1, 5120, 25600, 8, 8), (2, 2, 5120, 25600, 16, 13), (14, 0, 300, 4096, 5, 4),
                                     (10, 1, 70, 512 * 40 + 256, 40, 40), (23, 2, 8, 256, 1, 1)):
        w = q.fmt_chunk_waves(fmt, mode, N, K, S)
        assert 1 <= w <= min(ceff, 16), (fmt, mode, N, K, S, w)
        tune(fmt_waves=3)
        assert q.fmt_chunk_waves(fmt, mode, N, K, S) == min(3, ceff)
        tune(fmt_waves=-1)
    for N, K, S, ceff in ((5120, 25600, 8, 8), (5120, 8192, 5, 4), (300, 25632, 5, 5)):
        w = q.dq_chunk_waves(N, K, S)
        assert 1 <= w <= ceff, (N, K, S, w)
        tune(dq_waves=2)
        assert q.dq_chunk_waves(N, K, S) == 2
        tune(dq_waves=-1)
    with pytest.raises(q.QdgError) as e:
        q.dq_chunk_waves(64, 512 * 17, 17)   # 17 chunk waves: not this kernel
    assert e.value.status == -4


def wave_cases(fmt):
    """(N, K, S, W): W chunk waves forced below the chunk count, and more chunks
    than a workgroup has waves (S = 40, the last chunk with the K mod 512 tail)."""
    tail = 256 if fmt in SUPER else 32
    return [(300, 5120, 8, 1), (300, 5120, 8, 3), (300, 5120, 5, 2), (70, 512 * 40 + tail, 40, -1),
            (37, 512 * 64, 64, 5)]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_fmt_several_chunks_a_wave(fmt, mode):
    """A wave that sums several chunks one after another, each into its own
    partial: the quantized modes bit-exact with the oracle's chunked sum, Dequant
    within one unit in the last place of it, and every wave count the same bits."""
    for N, K, S, W in wave_cases(fmt):
        announce(f"gemv_fmt chunks a wave fmt={fmt} mode={mode} N={N} K={K} S={S} W={W}")
        rng = np.random.default_rng(7000 * fmt + N + K + 7 * S + mode)
        w, _, _, _ = encode(fmt, N, K, rng)
        x = rng.standard_normal((1, K)).astype(np.float32)
        dw = dev(w.reshape(-1))
        y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
        y1 = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
        if mode == 0:
            args = dict(x=dev(x))
            want = oracle.gemv_fmt(fmt, 0, w, N, K, x=x, splits=S, nthreads=8)[0]
        else:
            oq, ol, os_ = oracle.quantize(mode, x)
            args = dict(xq=dev(oq), xl=None if ol is None else dev(ol), xs=dev(os_))
            want = oracle.gemv_fmt(fmt, mode, w, N, K, xq=oq, xl=ol, xs=os_, splits=S, nthreads=8)[0]
        with q.tuning(fmt_waves=W):
            q.gemv_fmt(fmt, mode, dw, N, K, y, splits=S, **args)
        with q.tuning(fmt_waves=1):
            q.gemv_fmt(fmt, mode, dw, N, K, y1, splits=S, **args)
        got = host(y)
        if mode == 0:
            d = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
            assert d.max() <= 1, (N, K, S, W, int(d.max()))
        else:
            np.testing.assert_array_equal(got, want, err_msg=f"N={N} K={K} S={S} W={W}")
        assert torch.equal(y1.view(torch.int32), y.view(torch.int32)), (N, K, S, W)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_fmt_bench_shape(fmt, mode):
    """The down-projection's shape, 5120 x 25600 (25600 is a whole number of
    super-blocks), at the launch configuration the benchmark times (S=8), on the
    benchmark's generator: sampled rows bit-exact with the oracle."""
    import workloads
    N, K, S = 5120, 25600, 8
    announce(f"gemv_fmt bench shape fmt={fmt} mode={mode} N={N} K={K} S={S}")
    w = workloads.block_matrix(fmt, N, K, 2000 + fmt)
    x = workloads.activation(K, 77, True, 78)[None, :]
    oq, ol, os_ = oracle.quantize(mode, x)
    y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_fmt(fmt, mode, dev(w.reshape(-1)), N, K, y, xq=dev(oq), xl=None if ol is None else dev(ol), xs=dev(os_),
               splits=S)
    got = host(y)
    rows = np.unique(np.concatenate([[0, 1, 2, 3, 4095, N - 1], np.random.default_rng(fmt).choice(N, 58, False)]))
    want = oracle.gemv_fmt(fmt, mode, np.ascontiguousarray(w[rows]), len(rows), K, xq=oq, xl=ol, xs=os_, splits=S,
                           nthreads=8)[0]
    np.testing.assert_array_equal(got[rows], want)
    assert np.all(np.isfinite(got))


def tiny_cases():
    out = []
    for f in oracle.FORMATS:
        k1 = 256 if f in SUPER else 32          # one block: the matrix is 17..210 bytes
        for N, K in ((1, k1), (2, k1), (3, 2 * k1), (5, 3 * k1), (1, 768 if f in SUPER else 544)):
            out.append((f, N, K))
    return out


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("fmt,N,K", tiny_cases())
def test_fmt_tiny(fmt, N, K, mode):
    """The smallest matrices: one block a row (the last 16-byte piece of the
    matrix ends past it and is read as the 16 bytes that end at the matrix end),
    fewer rows than a wave's four, and K past one 512-value group with S=2 (a
    tail chunk)."""
    announce(f"gemv_fmt tiny fmt={fmt} mode={mode} N={N} K={K}")
    rng = np.random.default_rng(5000 * fmt + 10 * N + K + mode)
    w, _, _, _ = encode(fmt, N, K, rng)
    x = rng.standard_normal((1, K)).astype(np.float32)
    dw = dev(w.reshape(-1))
    assert dw.numel() == N * q.fmt_row_bytes(fmt, K)
    for S in (1, 2):
        y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
        if mode == 0:
            want = oracle.gemv_fmt(fmt, 0, w, N, K, x=x, splits=S)[0]
            q.gemv_fmt(fmt, 0, dw, N, K, y, x=dev(x), splits=S)
            got = host(y)
            d = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
            assert d.max() <= 1, (S, int(d.max()))
        else:
            oq, ol, os_ = oracle.quantize(mode, x)
            want = oracle.gemv_fmt(fmt, mode, w, N, K, xq=oq, xl=ol, xs=os_, splits=S)[0]
            q.gemv_fmt(fmt, mode, dw, N, K, y, xq=dev(oq), xl=None if ol is None else dev(ol), xs=dev(os_), splits=S)
            np.testing.assert_array_equal(host(y), want, err_msg=f"S={S}")


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_fmt_mxfp4_scale_extremes(mode):
    """MXFP4 blocks whose E8M0 scale byte is 0 or 1 (binary32 subnormal scales),
    2, 127 or 200, mixed along the rows: the GPU keeps binary32 subnormals as the
    oracle does (quantized modes bit-exact, Dequant within one ulp)."""
    from gguf_blocks import MXFP4
    N, K = 40, 1024
    announce(f"gemv_fmt mxfp4 scale extremes mode={mode}")
    rng = np.random.default_rng(77 + mode)
    w, _, _, _ = encode(MXFP4, N, K, rng)
    blocks = w.reshape(N, K // 32, 17)
    blocks[:, :, 0] = rng.choice(np.array([0, 1, 2, 127, 200], np.uint8), size=(N, K // 32))
    blocks[:8, :, 0] = 0  # whole rows of subnormal scales
    w = blocks.reshape(N, -1)
    x = rng.standard_normal((1, K)).astype(np.float32)
    y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    if mode == 0:
        want = oracle.gemv_fmt(MXFP4, 0, w, N, K, x=x)[0]
        q.gemv_fmt(MXFP4, 0, dev(w.reshape(-1)), N, K, y, x=dev(x))
        got = host(y)
        d = np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
        assert d.max() <= 1, int(d.max())
    else:
        oq, ol, os_ = oracle.quantize(mode, x)
        want = oracle.gemv_fmt(MXFP4, mode, w, N, K, xq=oq, xl=ol, xs=os_)[0]
        q.gemv_fmt(MXFP4, mode, dev(w.reshape(-1)), N, K, y, xq=dev(oq), xl=None if ol is None else dev(ol), xs=dev(os_))
        np.testing.assert_array_equal(host(y), want)
    assert np.all(np.isfinite(want)) and np.any(np.abs(want[:8]) < 1e-30)
