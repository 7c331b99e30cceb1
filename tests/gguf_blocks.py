"""Test infrastructure: an encoder for the GGUF block formats, written from the
byte layouts independently of the oracle's C decoders (lane kernel library page,
BLOCKS: lk_sub and its helpers describe each layout).  Each encoder takes chosen
raw fields (levels, sub-scales, binary16 scales), packs them into blocks, and
returns the packed rows together with what a decoder must recover: the int8
levels [N][K] and each half's scale d and offset c [N][K/16] in binary32.

Nothing here is used by the library; the GPU tests also use it to build
block-format matrices of a chosen shape and distribution.
"""
from __future__ import annotations

import numpy as np

Q4_0, Q4_1, Q5_0, Q5_1, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, IQ4_NL, IQ4_XS, MXFP4 = 2, 3, 6, 7, 10, 11, 12, 13, 14, 20, 23, 39
SUPER = {Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, IQ4_XS}
BYTES = {Q4_0: 18, Q4_1: 20, Q5_0: 22, Q5_1: 24, IQ4_NL: 18, MXFP4: 17,
         Q2_K: 84, Q3_K: 110, Q4_K: 144, Q5_K: 176, Q6_K: 210, IQ4_XS: 136}
IQ4 = np.array([-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113], np.int8)
E2M1X2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int8)


def f16(v) -> np.ndarray:
    return np.asarray(v, np.float16)


def f16_bytes(h: np.float16) -> list[int]:
    b = int(np.asarray(h, np.float16).view(np.uint16))
    return [b & 255, b >> 8]


def f32(v) -> np.float32:
    return np.float32(v)


def row_bytes(fmt: int, K: int) -> int:
    return K // (256 if fmt in SUPER else 32) * BYTES[fmt]


def _pack_nibbles(lo: np.ndarray, hi: np.ndarray) -> list[int]:
    return [int(a) | (int(b) << 4) for a, b in zip(lo, hi)]


def encode(fmt: int, N: int, K: int, rng: np.random.Generator, small: bool = False):
    """Random fields for an N x K matrix -> (bytes uint8 [N][row_bytes], levels, d, c).
    small=True draws integer scales and offsets (every product and sum exact)."""
    rb = row_bytes(fmt, K)
    out = np.zeros((N, rb), np.uint8)
    lv = np.zeros((N, K), np.int8)
    d = np.zeros((N, K // 16), np.float32)
    c = np.zeros((N, K // 16), np.float32)

    def scale16(lo=1e-3, hi=1e-2):
        return f16(rng.integers(1, 4)) if small else f16(rng.uniform(lo, hi))

    for o in range(N):
        blob = []
        if fmt not in SUPER:
            for g in range(K // 32):
                sl = slice(32 * g, 32 * g + 32)
                hs = slice(2 * g, 2 * g + 2)
                if fmt in (Q4_0, Q4_1, IQ4_NL):
                    n = rng.integers(0, 16, 32)
                    dd = scale16()
                    blk = f16_bytes(dd)
                    if fmt == Q4_1:
                        m = f16(rng.integers(-3, 4)) if small else f16(rng.uniform(-0.05, 0.05))
                        blk += f16_bytes(m)
                        c[o, hs] = f32(m)
                    blk += _pack_nibbles(n[:16], n[16:])
                    lv[o, sl] = IQ4[n] if fmt == IQ4_NL else n - (8 if fmt == Q4_0 else 0)
                    d[o, hs] = f32(dd)
                elif fmt in (Q5_0, Q5_1):
                    q = rng.integers(0, 32, 32)
                    dd = scale16()
                    blk = f16_bytes(dd)
                    if fmt == Q5_1:
                        m = f16(rng.integers(-3, 4)) if small else f16(rng.uniform(-0.05, 0.05))
                        blk += f16_bytes(m)
                        c[o, hs] = f32(m)
                    qh = sum(int(q[i] >> 4) << i for i in range(32))
                    blk += [(qh >> (8 * i)) & 255 for i in range(4)]
                    blk += _pack_nibbles(q[:16] & 15, q[16:] & 15)
                    lv[o, sl] = q - (16 if fmt == Q5_0 else 0)
                    d[o, hs] = f32(dd)
                else:  # MXFP4
                    e = 128 if small else int(rng.integers(118, 134))
                    n = rng.integers(0, 16, 32)
                    blk = [e] + _pack_nibbles(n[:16], n[16:])
                    lv[o, sl] = E2M1X2[n]
                    d[o, hs] = f32(2.0 ** (e - 128))
                blob += blk
        else:
            for sbk in range(K // 256):
                base = 256 * sbk
                if fmt in (Q4_K, Q5_K):
                    dd, dm = scale16(), scale16()
                    sc = rng.integers(0, 4 if small else 64, 8)
                    mn = rng.integers(0, 4 if small else 64, 8)
                    sp = [0] * 12
                    for j in range(4):
                        sp[j] = int(sc[j]) | ((int(sc[j + 4]) >> 4) << 6)
                        sp[j + 4] = int(mn[j]) | ((int(mn[j + 4]) >> 4) << 6)
                        sp[j + 8] = (int(sc[j + 4]) & 15) | ((int(mn[j + 4]) & 15) << 4)
                    q = rng.integers(0, 32 if fmt == Q5_K else 16, 256)
                    blk = f16_bytes(dd) + f16_bytes(dm) + sp
                    if fmt == Q5_K:
                        qh = [0] * 32
                        for j in range(8):
                            for ell in range(32):
                                qh[ell] |= (int(q[32 * j + ell]) >> 4) << j
                        blk += qh
                    for p in range(4):
                        blk += _pack_nibbles(q[64 * p:64 * p + 32] & 15, q[64 * p + 32:64 * p + 64] & 15)
                    for j in range(8):
                        lv[o, base + 32 * j:base + 32 * j + 32] = q[32 * j:32 * j + 32]
                        hs = slice((base + 32 * j) // 16, (base + 32 * j) // 16 + 2)
                        d[o, hs] = f32(dd) * f32(sc[j])
                        c[o, hs] = -(f32(dm) * f32(mn[j]))
                elif fmt == Q6_K:
                    dd = scale16()
                    sc = rng.integers(-4, 5, 16) if small else rng.integers(-128, 128, 16)
                    q = rng.integers(0, 64, 256)
                    ql, qh = [0] * 128, [0] * 64
                    for j in range(8):
                        half, k = j // 4, j % 4
                        for ell in range(32):
                            v = int(q[32 * j + ell])
                            lo, hi2 = v & 15, v >> 4
                            idx = 64 * half + ell + (32 if k & 1 else 0)
                            ql[idx] |= lo << (4 if k & 2 else 0)
                            qh[32 * half + ell] |= hi2 << (2 * k)
                    blk = ql + qh + [int(v) & 255 for v in sc] + f16_bytes(dd)
                    for j in range(8):
                        half, k = j // 4, j % 4
                        lv[o, base + 32 * j:base + 32 * j + 32] = q[32 * j:32 * j + 32] - 32
                        for h in range(2):
                            d[o, (base + 32 * j) // 16 + h] = f32(dd) * f32(sc[8 * half + 2 * k + h])
                elif fmt == Q2_K:
                    dd, dm = scale16(), scale16()
                    scb = rng.integers(0, 256, 16)
                    q = rng.integers(0, 4, 256)
                    qs = [0] * 64
                    for j in range(8):
                        half, k = j // 4, j % 4
                        for ell in range(32):
                            qs[32 * half + ell] |= int(q[32 * j + ell]) << (2 * k)
                    blk = [int(v) for v in scb] + qs + f16_bytes(dd) + f16_bytes(dm)
                    for j in range(8):
                        half, k = j // 4, j % 4
                        lv[o, base + 32 * j:base + 32 * j + 32] = q[32 * j:32 * j + 32]
                        for h in range(2):
                            sbyte = int(scb[8 * half + 2 * k + h])
                            d[o, (base + 32 * j) // 16 + h] = f32(dd) * f32(sbyte & 15)
                            c[o, (base + 32 * j) // 16 + h] = -(f32(dm) * f32(sbyte >> 4))
                elif fmt == Q3_K:
                    dd = scale16()
                    s6 = rng.integers(28, 37, 16) if small else rng.integers(0, 64, 16)
                    lvl = rng.integers(-4, 4, 256)
                    hmask, qs, sp = [0] * 32, [0] * 64, [0] * 12
                    for j in range(8):
                        half, k = j // 4, j % 4
                        for ell in range(32):
                            v = int(lvl[32 * j + ell])
                            hb = 1 if v >= 0 else 0
                            low2 = v if hb else v + 4
                            qs[32 * half + ell] |= low2 << (2 * k)
                            hmask[ell] |= hb << (4 * half + k)
                    for i in range(16):
                        sp[i & 7] |= (int(s6[i]) & 15) << (4 * (i >> 3))
                        sp[8 + (i & 3)] |= (int(s6[i]) >> 4) << (2 * (i >> 2))
                    blk = hmask + qs + sp + f16_bytes(dd)
                    for j in range(8):
                        half, k = j // 4, j % 4
                        lv[o, base + 32 * j:base + 32 * j + 32] = lvl[32 * j:32 * j + 32]
                        for h in range(2):
                            d[o, (base + 32 * j) // 16 + h] = f32(dd) * f32(int(s6[8 * half + 2 * k + h]) - 32)
                else:  # IQ4_XS
                    dd = scale16()
                    ls = rng.integers(30, 35, 8) if small else rng.integers(0, 64, 8)
                    n = rng.integers(0, 16, 256)
                    sh = sum((int(ls[ib]) >> 4) << (2 * ib) for ib in range(8))
                    sl = [0] * 4
                    for ib in range(8):
                        sl[ib >> 1] |= (int(ls[ib]) & 15) << (4 * (ib & 1))
                    blk = f16_bytes(dd) + [sh & 255, sh >> 8] + sl
                    for ib in range(8):
                        blk += _pack_nibbles(n[32 * ib:32 * ib + 16], n[32 * ib + 16:32 * ib + 32])
                        lv[o, base + 32 * ib:base + 32 * ib + 32] = IQ4[n[32 * ib:32 * ib + 32]]
                        hs = slice((base + 32 * ib) // 16, (base + 32 * ib) // 16 + 2)
                        d[o, hs] = f32(dd) * f32(int(ls[ib]) - 32)
                blob += blk
        assert len(blob) == rb, (fmt, len(blob), rb)
        out[o] = np.array(blob, np.uint8)
    return out, lv, d, c
