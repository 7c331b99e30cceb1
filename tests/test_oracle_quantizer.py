"""Pins of the oracle's activation quantizer (CPU only).

What fixes the quantizer other than the oracle itself:
* hand-derived blocks (tests/golden/quantizer_cases.json) -- exact scales and
  words, ties-to-even, the zero block;
* closed-form identities every block satisfies (word ranges, the block maximum
  maps to +-127, the reconstruction error bounds s/2 and s/256);
* metamorphic relations (scaling by 2^k, negation);
* an exact-rational brute force (oracle/exact.py) of the same steps, which
  fixes that each float operation is one IEEE binary32 rounding.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import exact

pytestmark = pytest.mark.filterwarnings("ignore")


def _block_from_spec(values: dict) -> np.ndarray:
    x = np.zeros(32, np.float32)
    for k, v in values.items():
        x[int(k)] = np.float32(v)
    return x


def test_golden_quantizer_cases(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "quantizer_cases.json")))["cases"]
    for c in cases:
        x = _block_from_spec(c["values"])
        xq, xl, xs = oracle.quantize(c["mode"], x)
        if "s" in c:
            assert xs[0, 0] == np.float32(c["s"]), c["derivation"]
        else:
            assert xs[0, 0] == np.float32(np.float32(1e-30) / np.float32(127)), c["derivation"]
        want_h = np.zeros(32, np.int8)
        for k, v in c["h"].items():
            want_h[int(k)] = v
        np.testing.assert_array_equal(xq[0], want_h, err_msg=c["derivation"])
        if c["mode"] == 2:
            want_l = np.zeros(32, np.int8)
            for k, v in c["l"].items():
                want_l[int(k)] = v
            np.testing.assert_array_equal(xl[0], want_l, err_msg=c["derivation"])


def _blocks(rng, nblocks, kind):
    if kind == "normal":
        return rng.standard_normal((nblocks, 32)).astype(np.float32)
    if kind == "wide":
        mant = rng.standard_normal((nblocks, 32))
        ex = rng.integers(-30, 30, size=(nblocks, 1))
        return (mant * 2.0 ** ex).astype(np.float32)
    if kind == "sparse":
        x = np.zeros((nblocks, 32), np.float32)
        pos = rng.integers(0, 32, size=nblocks)
        x[np.arange(nblocks), pos] = rng.standard_normal(nblocks).astype(np.float32) * 10
        return x
    if kind == "outliers":
        x = rng.standard_normal((nblocks, 32)).astype(np.float32)
        x[:, 5] *= np.float32(20.0)
        return x
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "wide", "sparse", "outliers"])
@pytest.mark.parametrize("mode", [1, 2])
def test_identities(mode, kind):
    rng = np.random.default_rng(7 + mode)
    x = _blocks(rng, 4000, kind)
    xq, xl, xs = oracle.quantize(mode, x.reshape(1, -1))
    h = xq.reshape(-1, 32).astype(np.int64)
    s = xs.reshape(-1).astype(np.float64)
    xv = x.astype(np.float64)
    a = np.abs(xv).max(axis=1)
    nz = a > 0
    # the block maximum maps to +-127 and no word exceeds it
    assert np.all(np.abs(h) <= 127)
    amax = np.abs(xv).argmax(axis=1)
    assert np.all(np.abs(h[np.arange(len(h)), amax][nz]) == 127)
    # the scale is the rounded a/127 (or the floor)
    if mode == 1:
        assert np.all(s[nz] == (a[nz].astype(np.float32) / np.float32(127)).astype(np.float64))
        assert np.all(s[~nz] == 1.0)
        # |v - s h| <= s/2 (the quotient rounds once, so allow its 2^-24 relative)
        err = np.abs(xv - s[:, None] * h)
        assert np.all(err <= s[:, None] * (0.5 + 128 * 2.0 ** -24))
    else:
        l = xl.reshape(-1, 32).astype(np.int64)
        assert np.all(np.abs(l) <= 64)
        # two-word reconstruction: |v - s (h + l/128)| <= s/256, plus the roundings of the
        # residual (2^-24 |r|, r = v when h = 0) and of the low-word quotient (s 2^-25)
        rec = s[:, None] * (h + l / 128.0)
        err = np.abs(xv - rec)
        bound = s[:, None] / 256.0 * (1 + 2.0 ** -16) + np.abs(xv) * 2.0 ** -24
        assert np.all(err <= bound)


@pytest.mark.parametrize("mode", [1, 2])
def test_metamorphic_scale_and_sign(mode):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((500, 32)).astype(np.float32)
    xq, xl, xs = oracle.quantize(mode, x.reshape(1, -1))
    for k in (-20, -3, 1, 9):
        y = (x * np.float32(2.0 ** k)).astype(np.float32)
        yq, yl, ys = oracle.quantize(mode, y.reshape(1, -1))
        np.testing.assert_array_equal(yq, xq)
        if mode == 2:
            np.testing.assert_array_equal(yl, xl)
        np.testing.assert_array_equal(ys, (xs * np.float32(2.0 ** k)).astype(np.float32))
    nq, nl, ns = oracle.quantize(mode, (-x).reshape(1, -1))
    np.testing.assert_array_equal(nq.astype(np.int16), -xq.astype(np.int16))
    if mode == 2:
        np.testing.assert_array_equal(nl.astype(np.int16), -xl.astype(np.int16))
    np.testing.assert_array_equal(ns, xs)


def test_half_even_ties_constructed():
    # a = 127 gives s = 1, so v/s = v: exact .5 quotients round to the even integer
    x = np.zeros(32, np.float32)
    x[0] = 127
    ties = np.arange(-62.5, 63.0, 4.0, dtype=np.float32)[:31]
    x[1:1 + len(ties)] = ties
    xq, _, _ = oracle.quantize(1, x)
    want = [int(2 * round(float(t) / 2)) for t in ties]  # half-even by construction
    assert list(xq[0, 1:1 + len(ties)].astype(int)) == want
    for t, q in zip(ties, xq[0, 1:1 + len(ties)]):
        assert abs(float(t) - int(q)) == 0.5 and int(q) % 2 == 0


@pytest.mark.parametrize("mode", [1, 2])
def test_exact_rational_brute_force(mode):
    rng = np.random.default_rng(3)
    parts = [_blocks(rng, 12, "normal"), _blocks(rng, 12, "wide"), _blocks(rng, 4, "sparse"),
             np.zeros((1, 32), np.float32)]
    x = np.concatenate(parts).reshape(1, -1)
    xq, xl, xs = oracle.quantize(mode, x)
    eq, el, es = exact.quantize(mode, x)
    np.testing.assert_array_equal(xq, eq)
    np.testing.assert_array_equal(xs, es)
    if mode == 2:
        np.testing.assert_array_equal(xl, el)


@settings(max_examples=60, deadline=None)
@given(st.lists(st.floats(min_value=-1e6, max_value=1e6, allow_nan=False, width=32), min_size=32, max_size=32),
       st.sampled_from([1, 2]))
def test_hypothesis_against_exact(vals, mode):
    x = np.array(vals, np.float32)
    a = float(np.abs(x).max())
    if 0 < a < 1e-30:
        return  # outside the contract: scale floor / subnormal scales
    xq, xl, xs = oracle.quantize(mode, x)
    eq, el, es = exact.quantize(mode, x)
    np.testing.assert_array_equal(xq, eq)
    np.testing.assert_array_equal(xs, es)
    if mode == 2:
        np.testing.assert_array_equal(xl, el)


def test_half_decode_matches_numpy():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    fin = np.isfinite(ref)
    got = np.array([oracle.half_to_float(int(b)) for b in bits[fin][::37]], np.float32)
    np.testing.assert_array_equal(got, ref[fin][::37])
    assert math.isinf(oracle.half_to_float(0x7C00))
