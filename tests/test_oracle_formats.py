"""Pins of the oracle's GGUF block-format decoders and block-format GEMV (lane
kernel library page: module doc on the other formats, BLOCKS, lk_sub,
lk_row_dot, lk_sub_dot).

* Decoders: blocks packed by an encoder written separately from the layouts
  (tests/gguf_blocks.py) decode back to the levels, scales and offsets that were
  packed, for every format, at every sub-block position of a super-block.
* Identities between formats: Q4_1 with offset -8d is Q4_0, Q5_1 with -16d is
  Q5_0, and IQ4_NL and MXFP4 levels come from their published tables.
* The GEMV: exact in integers when every scale and offset is an integer (the
  row is then the integer matrix product, whatever the rounding order); the
  TwoPass low words count 1/128; Dequant is the exactly rounded sum of the
  dequantized weights times x within one unit in the last place; negating the
  activation negates the result and doubling the binary16 scales doubles it,
  bit for bit.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.exact import f32_round

from gguf_blocks import encode, E2M1X2, IQ4, Q4_0, Q4_1, Q5_0, Q5_1, IQ4_NL, MXFP4, SUPER

ALL = oracle.FORMATS


@pytest.mark.parametrize("fmt", ALL)
def test_decoder_recovers_the_packed_fields(fmt):
    rng = np.random.default_rng(fmt)
    N, K = 3, 512
    w, lv, d, c = encode(fmt, N, K, rng)
    assert w.shape[1] == oracle.fmt_row_bytes(fmt, K)
    glv, gd, gc = oracle.fmt_decode(fmt, w, N, K)
    np.testing.assert_array_equal(glv, lv)
    np.testing.assert_array_equal(gd.view(np.uint32), d.view(np.uint32))
    np.testing.assert_array_equal(gc, c)


def test_format_identities():
    rng = np.random.default_rng(7)
    K = 256
    for lo, hi, off in ((Q4_0, Q4_1, 8), (Q5_0, Q5_1, 16)):
        w0, lv0, d0, _ = encode(lo, 1, K, rng)
        g = oracle.fmt_geometry(hi)[1]
        gl = oracle.fmt_geometry(lo)[1]
        # the same levels + off with offset -off*d: insert the binary16 offset after d
        rows = []
        for b in range(K // 32):
            blk = w0[0, b * gl:(b + 1) * gl]
            dd = np.frombuffer(blk[:2].tobytes(), np.float16)[0]
            m = np.float16(-off * np.float32(dd))
            assert np.float32(m) == -off * np.float32(dd)  # exact in binary16 for these scales
            rows += list(blk[:2]) + list(np.array([m], np.float16).view(np.uint8)) + list(blk[2:])
        w1 = np.array([rows], np.uint8)
        assert w1.shape[1] == K // 32 * g
        l1, d1, c1 = oracle.fmt_decode(hi, w1, 1, K)
        wt0 = (d0[0].repeat(16) * lv0[0].astype(np.float32))
        wt1 = (d1[0].repeat(16) * l1[0].astype(np.float32)) + c1[0].repeat(16)
        np.testing.assert_array_equal(wt0, wt1)
    # table formats: every nibble maps to its table level
    nib = np.arange(16)
    blk = np.array([0x00, 0x3c] + [int(a) | (int(b) << 4) for a, b in zip(nib, nib[::-1])], np.uint8)  # d = 1.0
    lv, d, _ = oracle.fmt_decode(IQ4_NL, blk[None, :], 1, 32)
    np.testing.assert_array_equal(lv[0, :16], IQ4) and np.testing.assert_array_equal(lv[0, 16:], IQ4[::-1])
    assert d[0, 0] == 1.0
    blk = np.array([130] + [int(a) | (int(b) << 4) for a, b in zip(nib, nib[::-1])], np.uint8)
    lv, d, _ = oracle.fmt_decode(MXFP4, blk[None, :], 1, 32)
    np.testing.assert_array_equal(lv[0, :16], E2M1X2)
    assert d[0, 0] == 4.0  # E8M0 130 is 2^3, halved for the doubled levels
    # the E2M1 values themselves: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives
    assert list(E2M1X2[:8] / 2) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _act(mode, K, rng, small):
    if small:
        xq = rng.integers(-20, 21, (1, K)).astype(np.int8)
        xl = rng.integers(-20, 21, (1, K)).astype(np.int8) if mode == 2 else None
        xs = np.full((1, K // 32), 128.0 if mode == 2 else 1.0, np.float32)
        return xq, xl, xs
    x = rng.standard_normal((1, K)).astype(np.float32)
    return oracle.quantize(mode, x)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("mode", [1, 2])
def test_quantized_gemv_integer_case(fmt, mode):
    """Integer scales and offsets, activation scale 1 (Int8Act) or 128 (TwoPass):
    every product and sum is an exact integer, so y is the integer product
    sum_k w_k * (h_k [* 128] + l_k) for any order of the f32 operations."""
    rng = np.random.default_rng(100 + fmt + mode)
    N, K = 5, 512
    w, lv, d, c = encode(fmt, N, K, rng, small=True)
    xq, xl, xs = _act(mode, K, rng, True)
    wt = (d.repeat(16, axis=1).astype(np.int64) * lv + c.repeat(16, axis=1).astype(np.int64))
    assert np.all(d == np.round(d)) and np.all(c == np.round(c))
    act = xq[0].astype(np.int64) * (128 if mode == 2 else 1) + (xl[0].astype(np.int64) if mode == 2 else 0)
    want = wt @ act
    assert np.abs(want).max() < 2 ** 24
    y = oracle.gemv_fmt(fmt, mode, w, N, K, xq=xq, xl=xl, xs=xs)
    np.testing.assert_array_equal(y[0], want.astype(np.float32))


@pytest.mark.parametrize("fmt", ALL)
def test_dequant_gemv_exact_rational(fmt):
    rng = np.random.default_rng(200 + fmt)
    N, K = 4, 512
    w, lv, d, c = encode(fmt, N, K, rng)
    x = rng.standard_normal((1, K)).astype(np.float32)
    y = oracle.gemv_fmt(fmt, 0, w, N, K, x=x)
    for o in range(N):
        wt = (d[o].repeat(16) * lv[o].astype(np.float32)).astype(np.float32) + c[o].repeat(16)  # fl(fl(d*l)+c)
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(wt, x[0]))
        want = float(f32_round(exact))
        assert abs(float(y[0, o]) - want) <= np.spacing(np.float32(abs(want))), (o, y[0, o], want)


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("mode", [1, 2])
def test_quantized_gemv_symmetries(fmt, mode):
    rng = np.random.default_rng(300 + fmt + mode)
    N, K = 6, 512
    w, lv, d, c = encode(fmt, N, K, rng)
    xq, xl, xs = _act(mode, K, rng, False)
    y = oracle.gemv_fmt(fmt, mode, w, N, K, xq=xq, xl=xl, xs=xs)
    # negating the words (none is -128 for quantized activations) negates every step exactly
    assert np.all(xq > -128) and (xl is None or np.all(xl > -128))
    yn = oracle.gemv_fmt(fmt, mode, w, N, K, xq=(-xq).astype(np.int8), xl=None if xl is None else (-xl).astype(np.int8),
                         xs=xs)
    np.testing.assert_array_equal(yn, -y)
    # doubling the activation scales doubles every term: y doubles bit for bit
    y2 = oracle.gemv_fmt(fmt, mode, w, N, K, xq=xq, xl=xl, xs=(2 * xs).astype(np.float32))
    np.testing.assert_array_equal(y2, 2 * y)


def test_twopass_low_words_weigh_one_128th():
    rng = np.random.default_rng(5)
    N, K = 3, 256
    w, lv, d, c = encode(Q4_0, N, K, rng, small=True)
    xq = np.zeros((1, K), np.int8)
    xl = rng.integers(-20, 21, (1, K)).astype(np.int8)
    xs = np.ones((1, K // 32), np.float32)
    y = oracle.gemv_fmt(Q4_0, 2, w, N, K, xq=xq, xl=xl, xs=xs)
    want = (d.repeat(16, axis=1) * lv) @ xl[0].astype(np.float64) / 128.0
    np.testing.assert_array_equal(y[0], want.astype(np.float32))


@pytest.mark.parametrize("fmt", [Q4_0, 12, 14, MXFP4])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_split_integer_case(fmt, mode):
    """Split into chunks (the split-K chunk rule) and added in ascending order: in
    the integer case every split count gives the exact integer product, so every
    sub-block is summed once, in one chunk."""
    rng = np.random.default_rng(400 + fmt + mode)
    N, K = 4, 2560
    w, lv, d, c = encode(fmt, N, K, rng, small=True)
    wt = (d.repeat(16, axis=1).astype(np.int64) * lv + c.repeat(16, axis=1).astype(np.int64))
    if mode == 0:
        x = rng.integers(-20, 21, (1, K)).astype(np.float32)
        want = wt @ x[0].astype(np.int64)
        kw = dict(x=x)
    else:
        xq, xl, xs = _act(mode, K, rng, True)
        want = wt @ (xq[0].astype(np.int64) * (128 if mode == 2 else 1) + (xl[0].astype(np.int64) if mode == 2 else 0))
        kw = dict(xq=xq, xl=xl, xs=xs)
    for S in (1, 2, 3, 5, 16):
        y = oracle.gemv_fmt(fmt, mode, w, N, K, splits=S, **kw)
        np.testing.assert_array_equal(y[0], want.astype(np.float32), err_msg=f"S={S}")


@pytest.mark.parametrize("fmt", ALL)
def test_workload_block_matrix_is_a_valid_matrix(fmt):
    """The seeded block-format generator (random bytes, binary16 scales drawn on
    [1e-3, 1e-2), E8M0 on [118, 134)) makes rows of the format's size whose every
    scale and offset decodes finite, and is reproducible from its seed."""
    import workloads
    K = 512
    b = workloads.block_matrix(fmt, 4, K, 9)
    assert b.dtype == np.uint8 and b.shape == (4, oracle.fmt_row_bytes(fmt, K))
    _, d, c = oracle.fmt_decode(fmt, b, 4, K)
    assert np.all(np.isfinite(d)) and np.all(np.isfinite(c)) and np.any(d != 0)
    np.testing.assert_array_equal(b, workloads.block_matrix(fmt, 4, K, 9))


def test_mxfp4_e8m0_extremes():
    """MXFP4's E8M0 byte e gives the scale 2^(e-128) for the doubled E2M1 levels:
    e = 0 and 1 are binary32 subnormals (2^-128, 2^-127), 127 and 128 are 1/2
    and 1, and 255 (E8M0's NaN code) decodes as 2^127 like every other byte."""
    nib = np.arange(16)
    for e, want in ((0, 2.0 ** -128), (1, 2.0 ** -127), (127, 0.5), (128, 1.0), (254, 2.0 ** 126), (255, 2.0 ** 127)):
        blk = np.array([e] + [int(a) | (int(b) << 4) for a, b in zip(nib, nib[::-1])], np.uint8)
        _, d, c = oracle.fmt_decode(MXFP4, blk[None, :], 1, 32)
        assert float(d[0, 0]) == want and float(d[0, 1]) == want and not np.any(c), (e, d[0])
