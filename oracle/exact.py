"""Exact-arithmetic brute force for tiny inputs -- TEST INFRASTRUCTURE ONLY.

Every value here is a ``fractions.Fraction``; each IEEE binary32 rounding the
method prescribes is carried out by ``f32_round`` (nearest, ties to even, written
from the binary32 format: 24-bit significand, exponents -126..127, subnormals
down to 2^-149).  Nothing is computed in hardware floating point, so these
functions check that the C oracle's float operations are single IEEE roundings
(no extended precision, no contraction, a real fused multiply-add) on the inputs
they are given.  Pure Python loops: only for a few thousand values.

Steps follow the same passages as ``qdg_oracle.c``: the quantizer of the module
doc / ``lk_quant_lane`` / ``lk_two_words`` of the lane kernel library page, the
block step ``lk_q8_term`` and the fixed order of ``lk_q8_rows_dot`` /
``lk_q8_sum4``, and the binary64 Dequant sum.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

_EMIN = -126
_P = 24


def f32_round(v: Fraction) -> Fraction:
    """Nearest binary32 value to the rational ``v``, ties to even (no overflow handling)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, _EMIN) - (_P - 1)  # spacing 2^q of the binade (subnormals share 2^-149)
    scaled = a / (Fraction(2) ** q)
    n = round_half_even(scaled)
    return sign * Fraction(n) * (Fraction(2) ** q)


def round_half_even(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def f64_round(v: Fraction) -> Fraction:
    """Nearest binary64 value, ties to even (normal range only, which is all the tests use)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = e - 52
    n = round_half_even(a / (Fraction(2) ** q))
    return sign * Fraction(n) * (Fraction(2) ** q)


def half_value(bits: int) -> Fraction:
    """IEEE binary16 from its bit pattern (finite values only)."""
    sign = -1 if (bits >> 15) & 1 else 1
    e = (bits >> 10) & 31
    f = bits & 1023
    if e == 31:
        raise ValueError("inf/nan scale")
    if e == 0:
        return sign * Fraction(f, 2 ** 24)
    return sign * Fraction(1024 + f) * Fraction(2) ** (e - 25)


def F(v) -> Fraction:
    return Fraction(float(v))


def clamp8(v: int) -> int:
    return max(-128, min(127, v))


def quantize_block(mode: int, x) -> tuple[list[int], list[int], Fraction]:
    """One 32-value block: ``(h, l, s)``; ``l`` is all zeros for Int8Act."""
    xv = [F(v) for v in x]
    a = max(abs(v) for v in xv)
    if mode == 1:
        s = f32_round(a / 127) if a > 0 else Fraction(1)
    else:
        floor = F(np.float32(1e-30))
        s = f32_round((a if a > floor else floor) / 127)
    h, l = [], []
    for v in xv:
        hv = round_half_even(f32_round(v / s))
        if mode == 2:
            hv = clamp8(hv)
            r = f32_round(v - hv * s)                     # one rounding of x - h*s
            lsc = f32_round(s / 128)
            lv = clamp8(round_half_even(f32_round(r / lsc)))
        else:
            lv = 0
        h.append(hv)
        l.append(lv)
    return h, l, s


def quantize(mode: int, x: np.ndarray):
    x = np.atleast_2d(np.asarray(x, np.float32))
    B, K = x.shape
    xq = np.zeros((B, K), np.int8)
    xl = np.zeros((B, K), np.int8)
    xs = np.zeros((B, K // 32), np.float32)
    for t in range(B):
        for g in range(K // 32):
            h, l, s = quantize_block(mode, x[t, 32 * g:32 * g + 32])
            xq[t, 32 * g:32 * g + 32] = h
            xl[t, 32 * g:32 * g + 32] = l
            xs[t, g] = float(s)
    return xq, (xl if mode == 2 else None), xs


def row_quant(mode: int, w, ws_bits, h, l, s, g0: int = 0, g1: int | None = None) -> Fraction:
    """A quantized row dot over blocks [g0, g1) with every rounding made explicit."""
    nb = len(w) // 32
    g1 = nb if g1 is None else g1
    p = [Fraction(0)] * 4
    for g in range(g0, g1):
        sig = half_value(int(ws_bits[g]))
        sg = F(s[g])
        d = sum(int(w[32 * g + i]) * int(h[32 * g + i]) for i in range(32))
        if mode == 1:
            alpha = f32_round(sig * sg)
            beta = Fraction(d)
        else:
            e = sum(int(w[32 * g + i]) * int(l[32 * g + i]) for i in range(32))
            lo = f32_round(f32_round(sg / 128) * e)
            alpha = sig
            beta = f32_round(sg * d + lo)                 # fma(s, D, lo): one rounding
        p[g % 4] = f32_round(alpha * beta + p[g % 4])     # fma(alpha, beta, p): one rounding
    return f32_round(f32_round(p[0] + p[2]) + f32_round(p[1] + p[3]))


def dequant_exact(w, ws_bits, x) -> Fraction:
    """The exact value of sum_k sigma*w*x (no rounding at all)."""
    K = len(w)
    return sum(half_value(int(ws_bits[k // 32])) * int(w[k]) * F(x[k]) for k in range(K))
