"""Pins of the oracle's GEMV, split-K, combine and arg-max (CPU only).

Each oracle function is fixed by something other than itself:
* hand-derived cases (tests/golden/gemv_order_pins.json): the fixed order of the
  four partials, the ascending chain, the single rounding of a step, the 2^-7
  weight of the low word, the TwoPass and Int8Act factorisations;
* the integer special case (scale 1, activation already integer) where every
  order is exact and the result is numpy's int64 matrix product;
* block dots against numpy's int64 matrix product;
* Dequant against the exact rational sum (Fractions) rounded once to binary32;
* the binary64 reference within the f32 criterion on seeded workloads;
* split-K: hand-derived chunk boundaries and ascending-combine cases, S = 1
  equal to the unsplit row, the integer case exact for every S;
* arg-max against numpy.argmax (first occurrence) and planted ties.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from oracle import exact


def _one_hot(spec, key, all_key):
    v = np.zeros(32, np.int64)
    if all_key in spec:
        v[:] = spec[all_key]
    for k, x in spec.get(key, {}).items():
        v[int(k)] = x
    return v


def _build_pin(case):
    K = case["K"]
    nb = K // 32
    w = np.zeros(K, np.int8)
    h = np.zeros(K, np.int8)
    l = np.zeros(K, np.int8)
    ws = np.full(nb, 0x3C00, np.uint16)
    xs = np.ones(nb, np.float32)
    for g, b in enumerate(case["blocks"]):
        sl = slice(32 * g, 32 * g + 32)
        w[sl] = _one_hot(b, "w", "w_all")
        h[sl] = _one_hot(b, "h", "h_all")
        l[sl] = _one_hot(b, "l", "l_all")
        if "ws" in b:
            ws[g] = int(b["ws"], 16)
        if "s" in b:
            xs[g] = np.float32(b["s"])
    return w.reshape(1, K), ws.reshape(1, nb), h.reshape(1, K), l.reshape(1, K), xs.reshape(1, nb)


def test_golden_order_pins(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "gemv_order_pins.json")))["cases"]
    assert len(cases) >= 6
    for c in cases:
        w, ws, h, l, xs = _build_pin(c)
        mode = c["mode"]
        y = oracle.gemv(mode, w, ws, xq=h, xl=l if mode == 2 else None, xs=xs)
        assert y[0, 0] == np.float32(c["y"]), (c["name"], float(y[0, 0]), c["derivation"])
        for other in c["other_orders"].values():
            assert np.float32(other) != np.float32(c["y"]), c["name"]
        # the exact-rational statement of the same steps agrees
        ex = exact.row_quant(mode, w[0], ws[0], h[0], l[0], xs[0])
        assert float(ex) == float(y[0, 0]), c["name"]


def test_block_dots_match_int64_matmul():
    rng = np.random.default_rng(5)
    N, K, B = 37, 32 * 13, 3
    wq = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    xq = rng.integers(-128, 128, size=(B, K), dtype=np.int8)
    xl = rng.integers(-128, 128, size=(B, K), dtype=np.int8)
    dh, dl = oracle.block_dots(2, wq, xq, xl)
    for g in range(K // 32):
        sl = slice(32 * g, 32 * g + 32)
        ref_h = xq[:, sl].astype(np.int64) @ wq[:, sl].astype(np.int64).T
        ref_l = xl[:, sl].astype(np.int64) @ wq[:, sl].astype(np.int64).T
        np.testing.assert_array_equal(dh[:, :, g], ref_h)
        np.testing.assert_array_equal(dl[:, :, g], ref_l)
    # extreme block: every product (-128)*(-128)
    w = np.full((1, 32), -128, np.int8)
    x = np.full((1, 32), -128, np.int8)
    assert oracle.block_dots(1, w, x)[0][0, 0, 0] == 32 * 128 * 128


def _integer_case(rng, N, K, B):
    """Scale 1, integer activations with a block max of exactly 127 (so s = 1, h = x, l = 0)."""
    wq = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    ws = np.full((N, K // 32), 0x3C00, np.uint16)
    x = rng.integers(-126, 127, size=(B, K)).astype(np.float32)
    x[:, ::32] = 127.0
    return wq, ws, x


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_integer_special_case_exact(mode):
    rng = np.random.default_rng(17 + mode)
    N, K, B = 64, 32 * 40, 2
    wq, ws, x = _integer_case(rng, N, K, B)
    ref = x.astype(np.int64) @ wq.astype(np.int64).T
    assert np.abs(ref).max() < 2 ** 24
    if mode == 0:
        y = oracle.gemv(0, wq, ws, x=x)
    else:
        xq, xl, xs = oracle.quantize(mode, x)
        assert np.all(xs == 1.0)
        np.testing.assert_array_equal(xq, x.astype(np.int8))
        if mode == 2:
            assert not xl.any()
        y = oracle.gemv(mode, wq, ws, xq=xq, xl=xl, xs=xs)
        for S in (1, 2, 3, 4, 8):
            part = oracle.gemv_split(mode, wq, ws, xq, xl, xs, S)
            np.testing.assert_array_equal(oracle.combine(part), ref.astype(np.float32))
    np.testing.assert_array_equal(y, ref.astype(np.float32))


def test_dequant_matches_exact_rational_rounding():
    rng = np.random.default_rng(23)
    N, K = 24, 96
    wq, ws = workloads.weights(N, K, 1, 2)
    x = rng.standard_normal(K).astype(np.float32)
    x[5] = np.float32(3.0e-7)
    y = oracle.gemv(0, wq, ws, x=x)
    mism = 0
    for o in range(N):
        ex = exact.dequant_exact(wq[o], ws[o], x)
        want = exact.f32_round(ex)
        if Fraction(float(y[0, o])) != want:
            # only a binary64 rounding that lands next to a binary32 tie may move it, by one ulp
            mism += 1
            assert abs(Fraction(float(y[0, o])) - want) <= abs(want) * Fraction(1, 2 ** 23)
    assert mism <= 1


@pytest.mark.parametrize("mode", [1, 2])
def test_quantized_rows_exact_rational(mode):
    rng = np.random.default_rng(29 + mode)
    N, K = 6, 32 * 9
    wq, ws = workloads.weights(N, K, 3, 4)
    x = (rng.standard_normal(K) * 3).astype(np.float32)
    xq, xl, xs = oracle.quantize(mode, x)
    y = oracle.gemv(mode, wq, ws, xq=xq, xl=xl, xs=xs)
    for o in range(N):
        ex = exact.row_quant(mode, wq[o], ws[o], xq[0], xl[0] if mode == 2 else np.zeros(K, np.int8), xs[0])
        assert float(ex) == float(y[0, o])
    # a sub-range of blocks, as a split chunk uses
    part = oracle.gemv_split(mode, wq, ws, xq, xl, xs, 1)
    np.testing.assert_array_equal(part[0], y)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("config,shape_index", [(workloads.TINY, 0), (workloads.DECODE_8B, 0)])
def test_within_f64_tolerance(mode, config, shape_index):
    d = workloads.make(config, shape_index)
    wq, ws, x = d["wq"], d["ws"], d["x"]
    if config == 1:
        wq, ws = wq[:512], ws[:512]
    if mode == 0:
        y = oracle.gemv(0, wq, ws, x=x, nthreads=4)
        Y, tn = oracle.reference_f64(0, wq, ws, x=x, nthreads=4)
    else:
        xq, xl, xs = oracle.quantize(mode, x)
        y = oracle.gemv(mode, wq, ws, xq=xq, xl=xl, xs=xs, nthreads=4)
        Y, tn = oracle.reference_f64(mode, wq, ws, xq=xq, xl=xl, xs=xs, nthreads=4)
    ok = oracle.within_tolerance(y, Y, tn)
    assert ok.all(), np.abs(y - Y).max()
    # against the unquantized product the encoding error is visible but bounded
    if mode != 0:
        Yd, tnd = oracle.reference_f64(0, wq, ws, x=x, nthreads=4)
        rel = np.abs(y - Yd) / np.maximum(np.abs(Yd), tnd)
        assert rel.max() < (1e-1 if mode == 1 else 2e-3)


def test_reference_tnorm_closed_forms():
    """The tolerance scale tnorm is the root-sum-square of a row's block terms
    (sigma * the block's exact dot), pinned on rows whose terms are known: equal
    terms give Y = nb*T and tnorm = sqrt(nb)*|T|; alternating signs give Y = 0
    with the same tnorm (so tnorm is not |Y|); one nonzero block gives
    tnorm = |Y|; a TwoPass row whose low words carry the whole term weighs them
    by 1/128."""
    nb = 16
    K = 32 * nb
    ones = np.ones((3, K), np.int8)
    ones[1].reshape(nb, 32)[1::2] = -1          # alternating block signs
    ones[2].reshape(nb, 32)[1:] = 0             # one nonzero block
    ws = np.full((3, nb), 0x3C00, np.uint16)     # sigma = 1
    # Dequant: x = 0.5 everywhere, T = 32 * 0.5 = 16 per block
    x = np.full((1, K), 0.5, np.float32)
    Y, tn = oracle.reference_f64(0, ones, ws, x=x)
    assert Y[0, 0] == 16.0 * nb and tn[0, 0] == 16.0 * np.sqrt(nb)
    assert Y[0, 1] == 0.0 and tn[0, 1] == 16.0 * np.sqrt(nb)
    assert Y[0, 2] == 16.0 and tn[0, 2] == 16.0
    # Int8Act: the words of x = 0.5 are 127 with s = fl32(0.5/127), T = 32*127*s
    xq, xl, xs = oracle.quantize(1, x)
    assert (xq == 127).all() and (xs == np.float32(0.5) / np.float32(127.0)).all()
    T = 32 * 127 * float(xs[0, 0])
    Y, tn = oracle.reference_f64(1, ones, ws, xq=xq, xl=xl, xs=xs)
    assert Y[0, 0] == pytest.approx(T * nb, rel=1e-15) and tn[0, 0] == pytest.approx(T * np.sqrt(nb), rel=1e-15)
    assert Y[0, 1] == 0.0 and tn[0, 1] == pytest.approx(T * np.sqrt(nb), rel=1e-15)
    assert tn[0, 2] == pytest.approx(abs(Y[0, 2]), rel=1e-15)
    # TwoPass with high words zero and low words 64: T = s * (0 + 32*64/128) = 16 s
    hq = np.zeros((1, K), np.int8)
    lq = np.full((1, K), 64, np.int8)
    s = np.full((1, nb), 0.25, np.float32)
    Y, tn = oracle.reference_f64(2, ones, ws, xq=hq, xl=lq, xs=s)
    assert Y[0, 0] == 4.0 * nb and tn[0, 0] == 4.0 * np.sqrt(nb)
    assert Y[0, 1] == 0.0 and tn[0, 1] == 4.0 * np.sqrt(nb)


def test_tolerance_catches_low_word_1_over_127():
    # the f64 criterion with the low word weighted 1/127 instead of 1/128 fails on a
    # low-word-dominated row: a mistake of that kind in the oracle would show
    K = 32 * 16
    rng = np.random.default_rng(31)
    x = (rng.standard_normal(K) * 0.004).astype(np.float32)
    x[::32] = 1.0
    wq = rng.integers(-127, 128, size=(4, K), dtype=np.int8)
    wq[:, ::32] = 0
    ws = np.full((4, K // 32), 0x3C00, np.uint16)
    xq, xl, xs = oracle.quantize(2, x)
    y = oracle.gemv(2, wq, ws, xq=xq, xl=xl, xs=xs)
    Y, tn = oracle.reference_f64(2, wq, ws, xq=xq, xl=xl, xs=xs)
    assert oracle.within_tolerance(y, Y, tn).all()
    dh, dl = oracle.block_dots(2, wq, xq, xl)
    wrong = (xs[0][None, :] * (dh[0] + dl[0] / 127.0)).sum(axis=1)
    assert not oracle.within_tolerance(wrong[None, :].astype(np.float32), Y, tn).all()


def test_split_bounds_golden(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "split_bounds.json")))["cases"]
    for c in cases:
        assert list(oracle.split_bounds(c["K"], c["S"])) == c["first"], c["derivation"]


def test_split_partials_are_chunk_rows():
    rng = np.random.default_rng(37)
    N, K = 16, 1600  # 3 superblocks and a 64-value tail
    wq, ws = workloads.weights(N, K, 5, 6)
    x = rng.standard_normal(K).astype(np.float32)
    for mode in (1, 2):
        xq, xl, xs = oracle.quantize(mode, x)
        y1 = oracle.gemv(mode, wq, ws, xq=xq, xl=xl, xs=xs)
        np.testing.assert_array_equal(oracle.gemv_split(mode, wq, ws, xq, xl, xs, 1)[0], y1)
        for S in (2, 4, 8):
            first = oracle.split_bounds(K, S)
            part = oracle.gemv_split(mode, wq, ws, xq, xl, xs, S)
            for s in range(S):
                g0, g1 = int(first[s]), int(first[s + 1])
                for o in (0, 7, 15):
                    ex = exact.row_quant(mode, wq[o], ws[o], xq[0],
                                         xl[0] if mode == 2 else np.zeros(K, np.int8), xs[0], g0, g1)
                    assert float(ex) == float(part[s, 0, o])
                if g0 == g1:
                    assert not part[s].any()


def test_combine_golden(golden_dir):
    cases = json.load(open(os.path.join(golden_dir, "combine_order.json")))["cases"]
    for c in cases:
        p = np.array(c["partials"], np.float32).reshape(-1, 1, 1)
        y = oracle.combine(p)
        assert y[0, 0] == np.float32(c["y"]), c["derivation"]
        assert not np.signbit(y[0, 0]) or c["y"] < 0


def test_argmax_matches_numpy_first_occurrence():
    for seed in range(200):
        rng = np.random.default_rng(seed)
        N = int(rng.integers(1, 3000))
        y = rng.standard_normal(N).astype(np.float32)
        if seed % 3 == 0:
            y = np.round(y * 2).astype(np.float32)  # many exact ties
        if seed % 5 == 0:
            y[:] = y[0]
        assert oracle.argmax(y)[0] == int(np.argmax(y))


def test_argmax_special_cases():
    assert oracle.argmax(np.array([-0.0, 0.0], np.float32))[0] == 0
    assert oracle.argmax(np.array([0.0, -0.0], np.float32))[0] == 0
    assert oracle.argmax(np.array([-1.0, -0.0, 0.0, -0.0], np.float32))[0] == 1
    assert oracle.argmax(np.array([5.0], np.float32))[0] == 0
    assert oracle.argmax(np.array([-np.inf, -np.inf], np.float32))[0] == 0
    y = np.zeros((3, 10), np.float32)
    y[1, 4] = y[1, 9] = 2.0
    y[2, 0] = y[2, 9] = -1.0
    assert list(oracle.argmax(y)) == [0, 4, 1]


def test_planted_tie_is_first_index():
    N, K = 3000, 512
    wq, ws = workloads.weights(N, K, 41, 42)
    x = workloads.activation(K, 43)
    a, b = 1234, 2345
    workloads.plant_tie(wq, ws, x, a, b)
    for mode in (0, 1, 2):
        if mode == 0:
            y = oracle.gemv(0, wq, ws, x=x)
        else:
            xq, xl, xs = oracle.quantize(mode, x)
            y = oracle.gemv(mode, wq, ws, xq=xq, xl=xl, xs=xs)
        assert y[0, a] == y[0, b]
        assert oracle.argmax(y)[0] == a
