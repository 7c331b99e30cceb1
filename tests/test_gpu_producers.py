"""GPU parity of the producers of the quantized activation (the residual add with
RMSNorm, and SwiGLU, each fused with the quantizer) against the CPU oracle.

Bar:
* the residual sum s is bit-exact (one binary32 addition);
* the f32 result (y of the norm, h of SwiGLU) is within one unit in the last place
  of the oracle's and equal to it almost everywhere.  Both sides evaluate the
  formula in binary64 and round once, so they can only differ where the exact
  value sits within a few binary64 units of a binary32 midpoint;
* the words and scales are bit-exact against the oracle's quantizer applied to the
  kernel's own f32 result (the integer decision is taken in the same precision on
  both sides, as for the arg-max), and equal to qdg_quantize_act's on it;
* every call is byte-identical on repeat.
"""
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
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in binary32 units in the last place (sign-magnitude bit patterns)."""
    def key(v):
        i = v.astype(np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7fffffff), i)
    return np.abs(key(a) - key(b))


def check_f32(got, want, what):
    d = ulp_diff(got, want)
    assert d.max() <= 1, f"{what}: {int(d.max())} ulp at {np.unravel_index(d.argmax(), d.shape)}"
    n_off = int(np.count_nonzero(d))
    assert n_off <= max(2, d.size // 1000), f"{what}: {n_off} of {d.size} values one ulp off"


def words(mode, B, K):
    xq = torch.empty((B, K), dtype=torch.int8, device=DEV)
    xl = torch.empty((B, K), dtype=torch.int8, device=DEV) if mode == 2 else None
    xs = torch.empty((B, K // 32), dtype=torch.float32, device=DEV)
    return xq, xl, xs


def check_words(mode, f32, xq, xl, xs, what):
    oq, ol, os_ = oracle.quantize(mode, f32)
    assert np.array_equal(host(xq), oq), f"{what}: xq"
    assert np.array_equal(host(xs).view(np.uint32), os_.view(np.uint32)), f"{what}: xs"
    if mode == 2:
        assert np.array_equal(host(xl), ol), f"{what}: xl"
    # the same words as the standalone quantizer on the same f32 values
    gq, gl, gs = words(mode, *f32.shape)
    q.quantize_act(mode, dev(f32), gq, gl, gs)
    assert torch.equal(gq, xq) and torch.equal(gs.view(torch.int32), xs.view(torch.int32))
    if mode == 2:
        assert torch.equal(gl, xl)


RMS_CASES = [  # (B, K, residual, weight, eps)
    (1, 32, True, True, 1e-6),
    (3, 96, False, True, 1e-5),
    (2, 544, True, False, 1e-6),
    (1, 4128, True, True, 1e-6),      # a second, partial round of chunks
    (16, 5120, True, True, 1e-6),     # the hidden size, 16 rows
    (1, 16384, True, True, 1e-6),     # the largest K held in registers
    (2, 20480, True, True, 1e-6),     # read again in the second pass
    (1, 32768, False, True, 0.5),     # the largest K
]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("B,K,res,wt,eps", RMS_CASES)
def test_rmsnorm_quantize(mode, B, K, res, wt, eps):
    announce(f"rmsnorm_quantize mode={mode} B={B} K={K} r={res} w={wt} eps={eps}")
    x = workloads.batch_activation(B, K, 700 + K, outliers=True, seed_out=701 + K)
    r = workloads.batch_activation(B, K, 900 + K) if res else None
    w = workloads.norm_weight(K, 800 + K) if wt else None
    os_, oy = oracle.rmsnorm(x, r, w, eps)
    dx, dr, dw = dev(x), dev(r), dev(w)
    s = torch.empty_like(dx) if res else None
    y = torch.empty_like(dx)
    xq, xl, xs = words(mode, B, K) if mode else (None, None, None)
    q.rmsnorm_quantize(mode, dx, dw, dr, s, y, xq, xl, xs, eps)
    gy = host(y)
    check_f32(gy, oy, "y")
    if res:
        assert np.array_equal(host(s).view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(host(dx), x)                      # x untouched when s is elsewhere
    if mode:
        check_words(mode, gy, xq, xl, xs, "rmsnorm")
        # without the f32 output, and without the residual write-back: the same words
        xq2, xl2, xs2 = words(mode, B, K)
        q.rmsnorm_quantize(mode, dx, dw, dr, None, None, xq2, xl2, xs2, eps)
        assert torch.equal(xq2, xq) and torch.equal(xs2.view(torch.int32), xs.view(torch.int32))
        if mode == 2:
            assert torch.equal(xl2, xl)
    # repeat: byte-identical
    y2 = torch.empty_like(dx)
    q.rmsnorm_quantize(mode, dx, dw, dr, torch.empty_like(dx) if res else None, y2,
                       *(words(mode, B, K) if mode else (None, None, None)), eps)
    assert torch.equal(y2.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("K", [5120, 20480])
def test_rmsnorm_in_place_residual(mode, K):
    """s = x (the residual stream updated in place), y = x too for Dequant's layout."""
    announce(f"rmsnorm in place mode={mode} K={K}")
    B = 2
    x = workloads.batch_activation(B, K, 31, outliers=True, seed_out=32)
    r = workloads.batch_activation(B, K, 33)
    w = workloads.norm_weight(K, 34)
    os_, oy = oracle.rmsnorm(x, r, w, 1e-6)
    dx = dev(x)
    xq, xl, xs = words(mode, B, K)
    q.rmsnorm_quantize(mode, dx, dev(w), dev(r), dx, None, xq, xl, xs, 1e-6)
    assert np.array_equal(host(dx).view(np.uint32), os_.view(np.uint32))
    # y over the same buffer as well: x <- y after s was formed in registers or in s
    dx2 = dev(x)
    xq2, xl2, xs2 = words(mode, B, K)
    q.rmsnorm_quantize(mode, dx2, dev(w), dev(r), None, dx2, xq2, xl2, xs2, 1e-6)
    check_f32(host(dx2), oy, "y in place")
    assert torch.equal(xq2, xq) and torch.equal(xs2.view(torch.int32), xs.view(torch.int32))


@pytest.mark.parametrize("mode", [1, 2])
def test_rmsnorm_special_rows(mode):
    """A zero row (eps > 0), a constant row, a one-hot row, and a row whose norm
    output is subnormal (tiny values, eps = 1)."""
    announce(f"rmsnorm special rows mode={mode}")
    K = 256
    x = np.zeros((4, K), np.float32)
    x[1] = 3.0
    x[2, 17] = -5.0
    x[3] = workloads.activation(K, 5) * np.float32(1e-39)
    for eps in (1e-6, 1.0):
        _, oy = oracle.rmsnorm(x, None, None, eps)
        y = torch.empty((4, K), dtype=torch.float32, device=DEV)
        xq, xl, xs = words(mode, 4, K)
        q.rmsnorm_quantize(mode, dev(x), None, None, None, y, xq, xl, xs, eps)
        gy = host(y)
        assert np.array_equal(gy.view(np.uint32), oy.view(np.uint32)), eps
        check_words(mode, gy, xq, xl, xs, f"special eps={eps}")


GLU_CASES = [(1, 32), (3, 544), (1, 25600), (16, 5120)]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("B,K", GLU_CASES)
def test_swiglu_quantize(mode, B, K):
    announce(f"swiglu_quantize mode={mode} B={B} K={K}")
    g, u = workloads.glu_inputs(B, K, 40 + K)
    oh = oracle.swiglu(g, u)
    dg, du = dev(g), dev(u)
    h = torch.empty_like(dg)
    xq, xl, xs = words(mode, B, K) if mode else (None, None, None)
    q.swiglu_quantize(mode, dg, du, h, xq, xl, xs)
    gh = host(h)
    check_f32(gh, oh, "h")
    if mode:
        check_words(mode, gh, xq, xl, xs, "swiglu")
        xq2, xl2, xs2 = words(mode, B, K)
        q.swiglu_quantize(mode, dg, du, None, xq2, xl2, xs2)
        assert torch.equal(xq2, xq) and torch.equal(xs2.view(torch.int32), xs.view(torch.int32))
        if mode == 2:
            assert torch.equal(xl2, xl)
    h2 = torch.empty_like(dg)
    q.swiglu_quantize(mode, dg, du, h2, *(words(mode, B, K) if mode else (None, None, None)))
    assert torch.equal(h2.view(torch.int32), h.view(torch.int32))


@pytest.mark.parametrize("mode", [1, 2])
def test_swiglu_special_values_and_in_place(mode):
    announce(f"swiglu special values mode={mode}")
    K = 64
    g = np.zeros((1, K), np.float32)
    u = np.ones((1, K), np.float32)
    g[0, :12] = [0.0, -0.0, 88.0, -88.0, 100.0, -100.0, -800.0, 1e-30, -1e-30, 3e38, -3e38, 20.0]
    u[0, 5] = 3.0          # silu(-100) * 3 is a binary32 subnormal
    u[0, 12:] = np.linspace(-4, 4, K - 12, dtype=np.float32)
    g[0, 12:] = np.linspace(-30, 30, K - 12, dtype=np.float32)
    oh = oracle.swiglu(g, u)
    dg = dev(g)
    xq, xl, xs = words(mode, 1, K)
    q.swiglu_quantize(mode, dg, dev(u), dg, xq, xl, xs)      # h over g
    gh = host(dg)
    check_f32(gh, oh, "special h")
    assert np.array_equal(gh[0, :12].view(np.uint32), oh[0, :12].view(np.uint32))
    check_words(mode, gh, xq, xl, xs, "swiglu special")


@pytest.mark.parametrize("mode", [1, 2])
def test_producer_words_drive_the_gemv(mode):
    """The fused producer's words give the GEMV the same output as quantizing the
    producer's f32 result separately (down-projection input, 2 row tiles)."""
    announce(f"producer -> gemv mode={mode}")
    N, K = 40, 25600
    g, u = workloads.glu_inputs(1, K, 77)
    wq, ws = workloads.weights(N, K, 78, 79)
    dg, du = dev(g), dev(u)
    h = torch.empty_like(dg)
    xq, xl, xs = words(mode, 1, K)
    q.swiglu_quantize(mode, dg, du, h, xq, xl, xs)
    y = torch.empty((1, N), dtype=torch.float32, device=DEV)
    dwq, dws = dev(wq), dev(ws.view(np.int16))
    q.gemv_q8(mode, dwq, dws, y, xq=xq, xl=xl, xs=xs)
    oq, ol, os_ = oracle.quantize(mode, host(h))
    want = oracle.gemv(mode, wq, ws, xq=oq, xl=ol, xs=os_)
    assert np.array_equal(host(y).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("F,K", [(32, 32), (64, 544), (12288, 4096), (96, 13184), (160, 15776), (64, 256),
                                 (96, 12800)])
@pytest.mark.parametrize("staging", ["default", "copy"])
def test_glu_matches_the_three_calls(mode, F, K, staging, tune):
    """qdg_gemv_glu_q8 (gate and up GEMVs with the SwiGLU and quantizer epilogue)
    against two qdg_gemv_q8 calls and qdg_swiglu_quantize, bit for bit, and the
    oracle: g and u bit-exact, h within one ulp, words bit-exact on the kernel's h.
    "default" stages by LDS DMA where K is a multiple of 256, "copy" through registers."""
    if mode == 2 and K > 13184:
        # the TwoPass activation row and 64 rows of scales exceed the LDS budget: the call is
        # refused before anything is enqueued
        xq, xl, xs = words(mode, 1, K)
        hq, hl, hs = words(mode, 1, F)
        w0 = torch.zeros((F, K), dtype=torch.int8, device=DEV)
        s0 = torch.zeros((F, K // 32), dtype=torch.int16, device=DEV)
        with pytest.raises(q.QdgError) as err:
            q.gemv_glu_q8(mode, w0, s0, w0, s0, xq, xl, xs, hq, hl, hs)
        assert err.value.status == -4  # QDG_EMODE
        return
    if staging == "copy":
        tune(ws_dma=0)
    else:
        tune(ws_dma=-1)
    announce(f"gemv_glu mode={mode} F={F} K={K} {staging}")
    wg, sg = workloads.weights(F, K, 71 + K, 72 + K)
    wu, su = workloads.weights(F, K, 73 + K, 74 + K)
    x = workloads.batch_activation(1, K, 75 + K, True, 76 + K)
    dwg, dsg = dev(wg), dev(sg.view(np.int16))
    dwu, dsu = dev(wu), dev(su.view(np.int16))
    xq, xl, xs = words(mode, 1, K)
    q.quantize_act(mode, dev(x), xq, xl, xs)
    h = torch.empty((F,), dtype=torch.float32, device=DEV)
    hq, hl, hs = words(mode, 1, F)
    q.gemv_glu_q8(mode, dwg, dsg, dwu, dsu, xq, xl, xs, hq, hl, hs, h=h)
    # the three calls
    g = torch.empty((1, F), dtype=torch.float32, device=DEV)
    u = torch.empty((1, F), dtype=torch.float32, device=DEV)
    q.gemv_q8(mode, dwg, dsg, g, xq=xq, xl=xl, xs=xs)
    q.gemv_q8(mode, dwu, dsu, u, xq=xq, xl=xl, xs=xs)
    h2 = torch.empty((1, F), dtype=torch.float32, device=DEV)
    hq2, hl2, hs2 = words(mode, 1, F)
    q.swiglu_quantize(mode, g, u, h2, hq2, hl2, hs2)
    assert torch.equal(h.view(torch.int32), h2.view(-1).view(torch.int32))
    assert torch.equal(hq.view(-1), hq2.view(-1)) and torch.equal(hs.view(torch.int32).view(-1), hs2.view(torch.int32).view(-1))
    if mode == 2:
        assert torch.equal(hl.view(-1), hl2.view(-1))
    # the oracle
    oq, ol, os_ = oracle.quantize(mode, x)
    og = oracle.gemv(mode, wg, sg, xq=oq, xl=ol, xs=os_, nthreads=8)
    ou = oracle.gemv(mode, wu, su, xq=oq, xl=ol, xs=os_, nthreads=8)
    assert np.array_equal(host(g), og) and np.array_equal(host(u), ou)
    gh = host(h).reshape(1, F)
    check_f32(gh, oracle.swiglu(og, ou), "glu h")
    check_words(mode, gh, hq.view(1, F), None if hl is None else hl.view(1, F), hs.view(1, F // 32), "glu")


@pytest.mark.parametrize("mode", [1, 2])
def test_glu_unaligned_scales(mode):
    """qdg_gemv_glu_q8 with the gate and up scales 2 bytes past a 16-byte boundary (K a
    multiple of 256, so aligned scales would be staged by LDS DMA): the register-copy
    staging gives the aligned call's bits."""
    F, K = 96, 4096
    announce(f"gemv_glu unaligned scales mode={mode} F={F} K={K}")
    wg, sg = workloads.weights(F, K, 81, 82)
    wu, su = workloads.weights(F, K, 83, 84)
    x = workloads.batch_activation(1, K, 85, True, 86)
    nb = K // 32

    def offset_copy(s):
        buf = torch.empty(F * nb + 8, dtype=torch.int16, device=DEV)
        v = buf[1:1 + F * nb].view(F, nb)
        v.copy_(dev(s.view(np.int16)))
        assert v.data_ptr() % 16 == 2
        return v

    dwg, dwu = dev(wg), dev(wu)
    xq, xl, xs = words(mode, 1, K)
    q.quantize_act(mode, dev(x), xq, xl, xs)
    outs = []
    for sgd, sud in ((dev(sg.view(np.int16)), dev(su.view(np.int16))), (offset_copy(sg), offset_copy(su))):
        h = torch.empty((F,), dtype=torch.float32, device=DEV)
        hq, hl, hs = words(mode, 1, F)
        q.gemv_glu_q8(mode, dwg, sgd, dwu, sud, xq, xl, xs, hq, hl, hs, h=h)
        outs.append((host(h), host(hq), None if hl is None else host(hl), host(hs)))
    for a, b in zip(*outs):
        if a is not None:
            assert a.tobytes() == b.tobytes()


# ---- the gated product with the other activations of lk_act: sigmoid and the tanh-form GELU

@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("B,K", [(1, 32), (3, 544), (1, 25600), (16, 5120)])
def test_glu_quantize(act, mode, B, K):
    """qdg_glu_quantize against the oracle's gated product (h within one ulp, almost
    always equal) and its words against the oracle's quantizer on the kernel's h;
    act 0 bit for bit the SwiGLU call."""
    announce(f"glu_quantize act={act} mode={mode} B={B} K={K}")
    g, u = workloads.glu_inputs(B, K, 140 + K + act)
    if act == 2:
        g = g * np.float32(2.5)   # reach the GELU's saturated tails too
    oh = oracle.glu(act, g, u)
    dg, du = dev(g), dev(u)
    h = torch.empty_like(dg)
    xq, xl, xs = words(mode, B, K) if mode else (None, None, None)
    q.glu_quantize(act, mode, dg, du, h, xq, xl, xs)
    gh = host(h)
    check_f32(gh, oh, f"act {act} h")
    if mode:
        check_words(mode, gh, xq, xl, xs, f"glu act {act}")
    if act == 0:
        h2 = torch.empty_like(dg)
        q.swiglu_quantize(mode, dg, du, h2, *(words(mode, B, K) if mode else (None, None, None)))
        assert torch.equal(h2.view(torch.int32), h.view(torch.int32))


@pytest.mark.parametrize("act", [1, 2])
@pytest.mark.parametrize("mode", [1, 2])
def test_glu_special_values_and_in_place(act, mode):
    """Zeros, the saturated tails (overflowing exponentials, subnormal and zero
    results) and h written over g."""
    announce(f"glu special values act={act} mode={mode}")
    K = 64
    g = np.zeros((1, K), np.float32)
    u = np.ones((1, K), np.float32)
    g[0, :12] = [0.0, -0.0, 20.0, -20.0, 100.0, -100.0, -800.0, 1e-30, -1e-30, 3e38, -3e38, 5.0]
    u[0, 5] = 3.0
    u[0, 12:] = np.linspace(-4, 4, K - 12, dtype=np.float32)
    g[0, 12:] = np.linspace(-12, 12, K - 12, dtype=np.float32)
    oh = oracle.glu(act, g, u)
    dg = dev(g)
    xq, xl, xs = words(mode, 1, K)
    q.glu_quantize(act, mode, dg, dev(u), dg, xq, xl, xs)      # h over g
    gh = host(dg)
    check_f32(gh, oh, "special h")
    assert np.array_equal(gh[0, :11].view(np.uint32), oh[0, :11].view(np.uint32))
    check_words(mode, gh, xq, xl, xs, f"glu act {act} special")


@pytest.mark.parametrize("act", [1, 2])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("F,K", [(32, 32), (64, 544), (12288, 4096), (96, 12800)])
def test_glu_act_matches_the_three_calls(act, mode, F, K):
    """qdg_gemv_glu_act_q8 against two qdg_gemv_q8 calls and qdg_glu_quantize, bit
    for bit, and the oracle: g and u bit-exact, h within one ulp, words bit-exact on
    the kernel's h."""
    announce(f"gemv_glu act={act} mode={mode} F={F} K={K}")
    wg, sg = workloads.weights(F, K, 171 + K, 172 + K)
    wu, su = workloads.weights(F, K, 173 + K, 174 + K)
    x = workloads.batch_activation(1, K, 175 + K, True, 176 + K)
    dwg, dsg = dev(wg), dev(sg.view(np.int16))
    dwu, dsu = dev(wu), dev(su.view(np.int16))
    xq, xl, xs = words(mode, 1, K)
    q.quantize_act(mode, dev(x), xq, xl, xs)
    h = torch.empty((F,), dtype=torch.float32, device=DEV)
    hq, hl, hs = words(mode, 1, F)
    q.gemv_glu_act_q8(act, mode, dwg, dsg, dwu, dsu, xq, xl, xs, hq, hl, hs, h=h)
    g = torch.empty((1, F), dtype=torch.float32, device=DEV)
    u = torch.empty((1, F), dtype=torch.float32, device=DEV)
    q.gemv_q8(mode, dwg, dsg, g, xq=xq, xl=xl, xs=xs)
    q.gemv_q8(mode, dwu, dsu, u, xq=xq, xl=xl, xs=xs)
    h2 = torch.empty((1, F), dtype=torch.float32, device=DEV)
    hq2, hl2, hs2 = words(mode, 1, F)
    q.glu_quantize(act, mode, g, u, h2, hq2, hl2, hs2)
    assert torch.equal(h.view(torch.int32), h2.view(-1).view(torch.int32))
    assert torch.equal(hq.view(-1), hq2.view(-1)) and torch.equal(hs.view(torch.int32).view(-1),
                                                                  hs2.view(torch.int32).view(-1))
    if mode == 2:
        assert torch.equal(hl.view(-1), hl2.view(-1))
    oq, ol, os_ = oracle.quantize(mode, x)
    og = oracle.gemv(mode, wg, sg, xq=oq, xl=ol, xs=os_, nthreads=8)
    ou = oracle.gemv(mode, wu, su, xq=oq, xl=ol, xs=os_, nthreads=8)
    assert np.array_equal(host(g), og) and np.array_equal(host(u), ou)
    gh = host(h).reshape(1, F)
    check_f32(gh, oracle.glu(act, og, ou), f"glu act {act} h")
    check_words(mode, gh, hq.view(1, F), None if hl is None else hl.view(1, F), hs.view(1, F // 32), "glu act")


def glu_dequant_three_calls(act, dwg, dsg, dwu, dsu, dx, F):
    """g and u by two qdg_gemv_q8 Dequant calls, h by qdg_glu_quantize under
    Dequant over g and u padded with zeros to whole 32-value blocks."""
    K = dx.numel()
    g = torch.full((1, F), float("nan"), dtype=torch.float32, device=DEV)
    u = torch.full((1, F), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_q8(0, dwg, dsg, g, x=dx.view(1, K))
    q.gemv_q8(0, dwu, dsu, u, x=dx.view(1, K))
    Fp = -(-F // 32) * 32
    gp = torch.zeros((1, Fp), dtype=torch.float32, device=DEV)
    up = torch.zeros((1, Fp), dtype=torch.float32, device=DEV)
    gp[:, :F], up[:, :F] = g, u
    h = torch.empty((1, Fp), dtype=torch.float32, device=DEV)
    q.glu_quantize(act, 0, gp, up, h)
    return host(g)[0], host(u)[0], host(h)[0, :F]


@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("F,K", [(32, 32), (3, 544), (7, 1536), (101, 4096), (5120, 5120), (8191, 1056),
                                 (8192, 1056), (12289, 800), (12288, 4096), (25600, 5120)])
def test_glu_dequant_matches_the_three_calls(act, F, K):
    """qdg_gemv_glu_dequant against two qdg_gemv_q8 Dequant calls and qdg_glu_quantize,
    bit for bit (both sides of the 8192-row change of chunk count, ragged F, K with
    a tail past the last 512-value superblock); the calls' g and u within the Dequant
    tolerance of the binary64 reference, h within one ulp of the oracle's gated
    product of them."""
    announce(f"gemv_glu_dequant act={act} F={F} K={K}")
    wg, sg = workloads.weights(F, K, 181 + K + F, 182 + K)
    wu, su = workloads.weights(F, K, 183 + K + F, 184 + K)
    x = workloads.activation(K, 185 + K, True, 186 + K)
    dwg, dsg = dev(wg), dev(sg.view(np.int16))
    dwu, dsu = dev(wu), dev(su.view(np.int16))
    dx = dev(x)
    h = torch.full((F,), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_glu_dequant(act, dwg, dsg, dwu, dsu, dx, h)
    gh, uh, want = glu_dequant_three_calls(act, dwg, dsg, dwu, dsu, dx, F)
    got = host(h)
    assert got.view(np.int32).tobytes() == want.view(np.int32).tobytes()
    for w, s, y in ((wg, sg, gh), (wu, su, uh)):
        Y, tn = oracle.reference_f64(0, w, s, x=x[None, :], nthreads=16)
        assert oracle.within_tolerance(y[None, :], Y, tn).all()
    check_f32(got[None, :], oracle.glu(act, gh[None, :], uh[None, :]), f"glu dequant act {act}")
    # a repeat gives the same bytes
    h2 = torch.full((F,), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_glu_dequant(act, dwg, dsg, dwu, dsu, dx, h2)
    assert host(h2).tobytes() == got.tobytes()


def test_glu_dequant_h_beside_x():
    """h may sit right after x in one buffer; one value over x is refused before any launch."""
    announce("gemv_glu_dequant h beside x")
    F, K = 96, 1024
    wg, sg = workloads.weights(F, K, 191, 192)
    wu, su = workloads.weights(F, K, 193, 194)
    x = workloads.activation(K, 195, True, 196)
    dwg, dsg = dev(wg), dev(sg.view(np.int16))
    dwu, dsu = dev(wu), dev(su.view(np.int16))
    buf = torch.full((K + F,), float("nan"), dtype=torch.float32, device=DEV)
    buf[:K] = dev(x)
    q.gemv_glu_dequant(0, dwg, dsg, dwu, dsu, buf[:K], buf[K:])
    alone = torch.empty((F,), dtype=torch.float32, device=DEV)
    q.gemv_glu_dequant(0, dwg, dsg, dwu, dsu, dev(x), alone)
    assert host(buf[K:]).tobytes() == host(alone).tobytes()
    assert host(buf[:K]).tobytes() == x.tobytes()
    with pytest.raises(q.QdgError) as e:
        q.gemv_glu_dequant(0, dwg, dsg, dwu, dsu, buf[:K], buf[K - 1:K - 1 + F])
    assert e.value.status == -1
