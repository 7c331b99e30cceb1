"""Pins of the oracle's producers of the quantized activation: the RMSNorm with its
residual add, and SwiGLU (lane kernel library page: RMSNORM and lk_act; QWEN38
page: gk_add_rmsnorm_q8f, gk_silu_had_q8).

The oracle evaluates both in binary64 and rounds once to binary32.  The pins
below do not reuse that route.  They evaluate the same formulas with 50-digit
decimal arithmetic and round the result to binary32 exactly.  They also check
closed forms (a 3-4-5 row, the logistic at 1), exact invariants (scaling by a
power of two, a one-hot row) and the limits of silu.  A dropped eps, a sum in
place of the mean, a missing weight or residual, or a wrong sign in the
exponent each fails one of them."""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.exact import f32_round

getcontext().prec = 50


def dec(v) -> Decimal:
    return Decimal(float(v))  # exact: every binary32/binary64 value is a finite decimal


def f32_of(d: Decimal) -> float:
    return float(f32_round(Fraction(d)))


def near_midpoint(d: Decimal, rel=Decimal("1e-14")) -> bool:
    """True when d lies within rel of a binary32 rounding midpoint.  The binary64
    route may then round the other way (its own error is some 1e-16 relative).
    For example, g * u of two binary32 values can fall on a midpoint exactly, and
    silu(88) * u is that product less a relative 6e-39."""
    f = Fraction(d)
    a = f32_round(f)
    if f == a or f == 0:
        return False
    m, e = np.frexp(abs(float(a)))
    ulp = Fraction(2) ** (int(e) - 24)
    mid = a + (ulp / 2 if f > a else -ulp / 2)
    return abs(f - mid) <= abs(f) * Fraction(rel)


def check_rounded(got, want: Decimal, where) -> int:
    """got is the binary32 rounding of want; within one unit in the last place
    where want sits on (or next to) a rounding midpoint.  Returns 1 there, else 0."""
    if near_midpoint(want):
        assert abs(float(got) - f32_of(want)) <= np.spacing(np.float32(abs(f32_of(want)))), where
        return 1
    assert got == f32_of(want), where
    return 0


def rms_decimal(x, r, w, eps):
    v = [dec(np.float32(a) + np.float32(b)) if r is not None else dec(a)
         for a, b in zip(x, r if r is not None else x)]
    mean = sum(t * t for t in v) / Decimal(len(v))
    den = (mean + dec(np.float32(eps))).sqrt()
    out = []
    for i, t in enumerate(v):
        o = t / den
        if w is not None:
            o = o * dec(w[i])
        out.append(o)
    return out


def test_rmsnorm_three_four_five_row():
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 1] = 3.0, 4.0
    _, y = oracle.rmsnorm(x, eps=0.0)
    root32 = Decimal(32).sqrt()
    assert y[0, 0] == f32_of(3 * root32 / 5)
    assert y[0, 1] == f32_of(4 * root32 / 5)
    assert np.all(y[0, 2:] == 0)
    # the same row reached through the residual add: (1 + 2, 2.5 + 1.5)
    xr, rr = np.zeros((1, 32), np.float32), np.zeros((1, 32), np.float32)
    xr[0, :2], rr[0, :2] = (1.0, 2.5), (2.0, 1.5)
    s, y2 = oracle.rmsnorm(xr, rr, eps=0.0)
    assert np.array_equal(s, x) and np.array_equal(y2, y)


@pytest.mark.parametrize("K,eps,with_r,with_w", [(32, 1e-6, True, True), (96, 0.5, False, True),
                                                  (100, 1e-6, True, False), (7, 1e-5, True, True)])
def test_rmsnorm_against_fifty_digits(K, eps, with_r, with_w):
    rng = np.random.default_rng(K)
    B = 3
    x = (rng.standard_normal((B, K)) * rng.choice([0.01, 1.0, 30.0], (B, 1))).astype(np.float32)
    r = rng.standard_normal((B, K)).astype(np.float32) if with_r else None
    w = (1 + 0.25 * rng.standard_normal(K)).astype(np.float32) if with_w else None
    s, y = oracle.rmsnorm(x, r, w, eps)
    for t in range(B):
        want = rms_decimal(x[t], None if r is None else r[t], w, eps)
        near = sum(check_rounded(y[t, i], want[i], (t, i)) for i in range(K))
        assert near <= 1
        if r is not None:
            for i in range(K):
                assert s[t, i] == f32_of(dec(x[t, i]) + dec(r[t, i]))


def test_rmsnorm_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 160)).astype(np.float32)
    w = (1 + 0.25 * rng.standard_normal(160)).astype(np.float32)
    _, y = oracle.rmsnorm(x, None, w, 0.0)
    for k in (-20, -3, 5, 30):
        _, yk = oracle.rmsnorm(np.ldexp(x, k).astype(np.float32), None, w, 0.0)
        assert np.array_equal(yk, y), k
    _, y4 = oracle.rmsnorm(x, None, (4 * w).astype(np.float32), 0.0)
    assert np.array_equal(y4, 4 * y)


def test_rmsnorm_unit_rms_and_one_hot():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    _, y = oracle.rmsnorm(x, eps=0.0)
    assert np.allclose(np.mean(y.astype(np.float64) ** 2, axis=1), 1.0, rtol=1e-6)
    for a in (-7.5, 1e-20, 3e30):
        h = np.zeros((1, 4), np.float32)
        h[0, 2] = a
        _, yh = oracle.rmsnorm(h, eps=0.0)
        assert yh[0, 2] == np.sign(a) * 2.0 and np.all(yh[0, [0, 1, 3]] == 0)


def test_rmsnorm_zero_row_with_eps_and_the_eps_term():
    _, y = oracle.rmsnorm(np.zeros((1, 64), np.float32), eps=1e-6)
    assert np.all(y == 0)
    # mean(v^2) = 1 and eps = 3: y = v / 2 exactly
    _, y = oracle.rmsnorm(np.ones((1, 64), np.float32), eps=3.0)
    assert np.all(y == 0.5)


def silu_decimal(g, u):
    gd = dec(g)
    return gd / (1 + (-gd).exp()) * dec(u)


def test_swiglu_logistic_at_one():
    h = oracle.swiglu(np.array([1.0, 2.0], np.float32), np.array([1.0, -3.0], np.float32))
    # the logistic function at 1 is 0.73105857863000487925...
    assert h[0] == np.float32(0.7310585786300049)
    assert h[1] == f32_of(Decimal(2) / (1 + Decimal(-2).exp()) * -3)


def test_swiglu_against_fifty_digits():
    rng = np.random.default_rng(3)
    g = np.concatenate([rng.uniform(-20, 20, 400), rng.standard_normal(400) * 1e-3,
                        [0.5, -0.5, 88.0, -88.0, 1e-30]]).astype(np.float32)
    u = rng.standard_normal(g.size).astype(np.float32)
    h = oracle.swiglu(g, u)
    near = sum(check_rounded(h[i], silu_decimal(g[i], u[i]), (i, g[i], u[i])) for i in range(g.size))
    assert near <= 3


def test_swiglu_limits_and_symmetry():
    one = np.ones(5, np.float32)
    h = oracle.swiglu(np.array([0.0, -0.0, 100.0, -800.0, -1e38], np.float32), one)
    assert h[0] == 0 and h[1] == 0
    assert h[2] == 100.0                                 # e^-100 vanishes next to 1 in binary64
    assert h[3] == 0 and np.signbit(h[3]) and h[4] == 0 and np.signbit(h[4])
    # silu(g) - silu(-g) = g: g * (sigma(g) + sigma(-g)) with sigma(g) + sigma(-g) = 1
    g = np.random.default_rng(4).uniform(-30, 30, 1000).astype(np.float32)
    d = oracle.swiglu(g, np.ones_like(g)).astype(np.float64) - oracle.swiglu(-g, np.ones_like(g))
    assert np.all(np.abs(d - g) <= 4 * np.spacing(np.abs(g)).astype(np.float64))


def test_swiglu_scipy_logistic():
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(5)
    g = rng.uniform(-40, 40, 20000).astype(np.float32)
    u = rng.standard_normal(20000).astype(np.float32)
    h = oracle.swiglu(g, u)
    ref = (g.astype(np.float64) * special.expit(g.astype(np.float64)) * u).astype(np.float32)
    diff = np.abs(h.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert diff.max() <= 1 and np.mean(diff == 0) > 0.999


# The gated product with the other activations of the lane kernel library
# page's lk_act: sigmoid and the GELU in its tanh form.
PI50 = Decimal("3.1415926535897932384626433832795028841971693993751")


def glu_decimal(act, g, u):
    gd = dec(g)
    if act == 0:
        a = gd / (1 + (-gd).exp())
    elif act == 1:
        a = 1 / (1 + (-gd).exp())
    else:
        z = (2 / PI50).sqrt() * (gd + Decimal("0.044715") * gd * gd * gd)
        a = gd / (1 + (-2 * z).exp())
    return a * dec(u)


def test_glu_silu_is_the_swiglu():
    rng = np.random.default_rng(6)
    g = rng.uniform(-30, 30, 2000).astype(np.float32)
    u = rng.standard_normal(2000).astype(np.float32)
    assert np.array_equal(oracle.glu(oracle.SILU, g, u).view(np.uint32), oracle.swiglu(g, u).view(np.uint32))


@pytest.mark.parametrize("act", [1, 2])
def test_glu_against_fifty_digits(act):
    rng = np.random.default_rng(7 + act)
    g = np.concatenate([rng.uniform(-12, 12, 400), rng.standard_normal(400) * 1e-3,
                        [0.5, -0.5, 3.0, -3.0, 1e-30, -1e-30]]).astype(np.float32)
    u = rng.standard_normal(g.size).astype(np.float32)
    h = oracle.glu(act, g, u)
    near = sum(check_rounded(h[i], glu_decimal(act, g[i], u[i]), (act, i, g[i], u[i])) for i in range(g.size))
    assert near <= 3


def test_glu_sigmoid_closed_forms_symmetry_and_limits():
    u = np.array([3.0, -7.25, 1e-30, 6e37], np.float32)
    h = oracle.glu(oracle.SIGMOID, np.zeros(4, np.float32), u)
    assert np.array_equal(h, u / 2)                            # the logistic at 0 is exactly 1/2
    one = np.ones(4, np.float32)
    lim = oracle.glu(oracle.SIGMOID, np.array([100.0, -800.0, -1e38, 1e38], np.float32), one)
    assert lim[0] == 1.0 and lim[3] == 1.0                     # e^-100 vanishes next to 1 in binary64
    assert lim[1] == 0 and not np.signbit(lim[1]) and lim[2] == 0
    # sigma(g) + sigma(-g) = 1
    g = np.random.default_rng(8).uniform(-15, 15, 1000).astype(np.float32)
    s = oracle.glu(oracle.SIGMOID, g, np.ones_like(g)).astype(np.float64) + \
        oracle.glu(oracle.SIGMOID, -g, np.ones_like(g))
    assert np.all(np.abs(s - 1.0) <= 2 * np.spacing(np.float32(1.0)))


def test_glu_gelu_identities_and_limits():
    one = np.ones(6, np.float32)
    h = oracle.glu(oracle.GELU_TANH, np.array([0.0, -0.0, 20.0, -20.0, 1e38, -1e38], np.float32), one)
    assert h[0] == 0 and h[1] == 0
    assert h[2] == 20.0                                        # e^-2z is some e^-1e3 there
    assert h[3] == 0 and np.signbit(h[3])                     # -20 / e^600: below every binary32
    assert h[4] == np.float32(1e38) and h[5] == 0 and np.signbit(h[5])
    # gelu(g) - gelu(-g) = g, since 1 / (1 + e^-2z) + 1 / (1 + e^2z) = 1
    g = np.random.default_rng(9).uniform(-8, 8, 1000).astype(np.float32)
    d = oracle.glu(oracle.GELU_TANH, g, np.ones_like(g)).astype(np.float64) - \
        oracle.glu(oracle.GELU_TANH, -g, np.ones_like(g))
    assert np.all(np.abs(d - g) <= 4 * np.spacing(np.abs(g)).astype(np.float64))
    # the same function as 0.5 g (1 + tanh z), evaluated through tanh instead of
    # exp, where that form is well conditioned (z > -1/2: no cancellation in
    # 1 + tanh z; below, the fifty-digit pin above covers it)
    rng = np.random.default_rng(10)
    g = rng.uniform(-0.6, 6, 20000).astype(np.float32)
    gd = g.astype(np.float64)
    z = np.sqrt(2 / np.pi) * (gd + 0.044715 * gd ** 3)
    g, gd, z = g[z > -0.5], gd[z > -0.5], z[z > -0.5]
    u = rng.standard_normal(g.size).astype(np.float32)
    ref = (0.5 * gd * (1 + np.tanh(z)) * u).astype(np.float32)
    hh = oracle.glu(oracle.GELU_TANH, g, u)
    diff = np.abs(hh.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert diff.max() <= 1 and np.mean(diff == 0) > 0.999


def test_glu_sigmoid_scipy_logistic():
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(11)
    g = rng.uniform(-40, 40, 20000).astype(np.float32)
    u = rng.standard_normal(20000).astype(np.float32)
    h = oracle.glu(oracle.SIGMOID, g, u)
    ref = (special.expit(g.astype(np.float64)) * u).astype(np.float32)
    diff = np.abs(h.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert diff.max() <= 1 and np.mean(diff == 0) > 0.999


def test_glu_rejects_an_unknown_activation():
    with pytest.raises(Exception):
        oracle.glu(3, np.zeros(4, np.float32), np.zeros(4, np.float32))
