"""The CPU oracle of the Q8_0 decode GEMV -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C, see
``qdg_oracle.c``) with numpy arrays and shares no code with the GPU library.

Functions (each mirrors one step of the method; citations in ``qdg_oracle.c``):

* ``quantize(mode, x)`` -> ``(xq, xl, xs)``
* ``block_dots(mode, wq, xq, xl)`` -> ``(dh, dl)`` exact int32 per-block dots
* ``gemv(mode, wq, ws, x=None, xq=None, xl=None, xs=None)`` -> ``y[B][N]``
* ``split_bounds(K, S)`` -> block boundaries of the split-K chunks
* ``gemv_split(mode, wq, ws, xq, xl, xs, S)`` -> partials ``[S][B][N]``
* ``combine(part)`` -> ``y``
* ``argmax(y)`` -> first index of the maximum, per row
* ``tile_rows(wq)`` -> the weight values in row tiles of four rows by 256 values
* ``reference_f64(mode, ...)`` -> ``(Y, tnorm)`` binary64 anchor of the tolerance
* ``rmsnorm(x, r=None, w=None, eps)`` -> ``(s, y)``: residual sum and RMSNorm
* ``swiglu(g, u)`` -> ``h = silu(g) * u``
* ``glu(act, g, u)`` -> ``h = act(g) * u`` (silu, sigmoid or the tanh-form GELU)
* ``fmt_geometry(fmt)``, ``fmt_row_bytes(fmt, K)``, ``fmt_decode(fmt, w, N, K)`` ->
  ``(levels [N][K], d [N][K/16], c [N][K/16])``, ``gemv_fmt(fmt, mode, w, N, K, ...)``:
  the other GGUF block formats
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

DEQUANT, INT8ACT, TWOPASS = 0, 1, 2
QK = 32

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.orc_quantize.argtypes = [I, P, I64, I64, P, P, P]
        lib.orc_block_dots.argtypes = [I, P, I64, I64, P, P, I64, P, P]
        lib.orc_gemv.argtypes = [I, P, P, I64, I64, P, P, P, P, I64, P, I]
        lib.orc_split_bounds.argtypes = [I64, I, P]
        lib.orc_gemv_split.argtypes = [I, P, P, I64, I64, P, P, P, I64, I, P, I]
        lib.orc_combine.argtypes = [P, I, I64, I64, P]
        lib.orc_argmax.argtypes = [P, I64, I64, P]
        lib.orc_reference_f64.argtypes = [I, P, P, I64, I64, P, P, P, P, I64, P, P, I]
        lib.orc_rmsnorm.argtypes = [P, P, P, ctypes.c_float, I64, I64, P, P]
        lib.orc_swiglu.argtypes = [P, P, I64, P]
        lib.orc_glu.argtypes = [I, P, P, I64, P]
        lib.orc_fmt_geometry.argtypes = [I, P, P]
        lib.orc_fmt_row_bytes.argtypes = [I, I64]
        lib.orc_fmt_row_bytes.restype = I64
        lib.orc_fmt_decode.argtypes = [I, P, I64, I64, P, P, P]
        lib.orc_gemv_fmt.argtypes = [I, I, P, I64, I64, P, P, P, P, I, P, I]
        lib.orc_half_to_float.argtypes = [ctypes.c_uint16]
        lib.orc_half_to_float.restype = ctypes.c_float
        for name in ("orc_quantize", "orc_block_dots", "orc_gemv", "orc_split_bounds",
                     "orc_gemv_split", "orc_combine", "orc_argmax", "orc_reference_f64",
                     "orc_rmsnorm", "orc_swiglu", "orc_glu", "orc_fmt_geometry", "orc_fmt_decode", "orc_gemv_fmt"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def default_threads() -> int:
    return 1


def half_to_float(bits: int) -> float:
    return float(_load().orc_half_to_float(int(bits)))


def quantize(mode: int, x: np.ndarray):
    x = _c(np.atleast_2d(x), np.float32)
    B, K = x.shape
    xq = np.empty((B, K), np.int8)
    xl = np.empty((B, K), np.int8) if mode == TWOPASS else None
    xs = np.empty((B, K // QK), np.float32)
    _check(_load().orc_quantize(mode, _p(x), B, K, _p(xq), _p(xl), _p(xs)), "quantize")
    return xq, xl, xs


def block_dots(mode: int, wq: np.ndarray, xq: np.ndarray, xl: np.ndarray | None = None):
    wq = _c(wq, np.int8)
    xq = _c(np.atleast_2d(xq), np.int8)
    xl = _c(None if xl is None else np.atleast_2d(xl), np.int8)
    N, K = wq.shape
    B = xq.shape[0]
    dh = np.empty((B, N, K // QK), np.int32)
    dl = np.empty((B, N, K // QK), np.int32) if mode == TWOPASS else None
    _check(_load().orc_block_dots(mode, _p(wq), N, K, _p(xq), _p(xl), B, _p(dh), _p(dl)), "block_dots")
    return dh, dl


def _gemv_args(wq, ws, x, xq, xl, xs):
    wq = _c(wq, np.int8)
    ws = _c(ws, np.uint16)
    N, K = wq.shape
    x = _c(None if x is None else np.atleast_2d(x), np.float32)
    xq = _c(None if xq is None else np.atleast_2d(xq), np.int8)
    xl = _c(None if xl is None else np.atleast_2d(xl), np.int8)
    xs = _c(None if xs is None else np.atleast_2d(xs), np.float32)
    B = (x if x is not None else xq).shape[0]
    return wq, ws, N, K, x, xq, xl, xs, B


def gemv(mode, wq, ws, x=None, xq=None, xl=None, xs=None, nthreads: int = 1):
    wq, ws, N, K, x, xq, xl, xs, B = _gemv_args(wq, ws, x, xq, xl, xs)
    y = np.empty((B, N), np.float32)
    _check(_load().orc_gemv(mode, _p(wq), _p(ws), N, K, _p(x), _p(xq), _p(xl), _p(xs), B, _p(y),
                            int(nthreads)), "gemv")
    return y


def split_bounds(K: int, S: int) -> np.ndarray:
    first = np.empty(S + 1, np.int32)
    _check(_load().orc_split_bounds(K, S, _p(first)), "split_bounds")
    return first


def gemv_split(mode, wq, ws, xq, xl, xs, S: int, nthreads: int = 1):
    wq, ws, N, K, _, xq, xl, xs, B = _gemv_args(wq, ws, None, xq, xl, xs)
    part = np.empty((S, B, N), np.float32)
    _check(_load().orc_gemv_split(mode, _p(wq), _p(ws), N, K, _p(xq), _p(xl), _p(xs), B, S, _p(part),
                                  int(nthreads)), "gemv_split")
    return part


def combine(part: np.ndarray) -> np.ndarray:
    part = _c(part, np.float32)
    S, B, N = part.shape
    y = np.empty((B, N), np.float32)
    _check(_load().orc_combine(_p(part), S, B, N, _p(y)), "combine")
    return y


def argmax(y: np.ndarray) -> np.ndarray:
    y = _c(np.atleast_2d(y), np.float32)
    B, N = y.shape
    idx = np.empty(B, np.int32)
    _check(_load().orc_argmax(_p(y), B, N, _p(idx)), "argmax")
    return idx


def tile_rows(wq: np.ndarray) -> np.ndarray:
    """The row-tiled weight layout: the values of four consecutive rows and 256
    consecutive columns are stored together, tile after tile.

    The megakernel page ("model-as-a-kernel mak_cuda/megakernel.cu", the GEMV's
    tiled-weights option) stores bf16 weights as [N/8][K/8][8][8] so that the
    eight warps of a block, on eight consecutive rows, read one contiguous
    stream; only addresses change, each lane reads the same values in the same
    order.  Here the tile is four rows by 256 values: byte
    ((t*(K/256) + s)*4 + r)*256 + c holds row 4t + r, column 256s + c.  N must
    be a multiple of 4 and K of 256.  The scales keep their plain layout.
    """
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    N, K = wq.shape
    if N % 4 or K % 256:
        raise ValueError("tile_rows: N must be a multiple of 4 and K of 256")
    return np.ascontiguousarray(wq.reshape(N // 4, 4, K // 256, 256).transpose(0, 2, 1, 3)).reshape(N, K)


def reference_f64(mode, wq, ws, x=None, xq=None, xl=None, xs=None, nthreads: int = 1):
    wq, ws, N, K, x, xq, xl, xs, B = _gemv_args(wq, ws, x, xq, xl, xs)
    Y = np.empty((B, N), np.float64)
    tn = np.empty((B, N), np.float64)
    _check(_load().orc_reference_f64(mode, _p(wq), _p(ws), N, K, _p(x), _p(xq), _p(xl), _p(xs), B,
                                     _p(Y), _p(tn), int(nthreads)), "reference_f64")
    return Y, tn


def within_tolerance(y: np.ndarray, Y: np.ndarray, tnorm: np.ndarray, rel: float = 1e-5) -> np.ndarray:
    """The f32 criterion: ``|y - Y| <= rel * max(|Y|, ||t||_2)`` elementwise."""
    y = np.asarray(y, np.float64)
    return np.abs(y - Y) <= rel * np.maximum(np.abs(Y), tnorm)


def rmsnorm(x: np.ndarray, r: np.ndarray | None = None, w: np.ndarray | None = None, eps: float = 1e-6):
    """``(s, y)`` for rows ``x[B][K]``: ``s = fl32(x + r)`` (``None`` without ``r``) and
    ``y = fl32((s / sqrt(mean(s^2) + eps)) * w)`` evaluated in binary64."""
    x = _c(np.atleast_2d(x), np.float32)
    B, K = x.shape
    r = None if r is None else _c(np.atleast_2d(r), np.float32)
    w = None if w is None else _c(w, np.float32)
    if r is not None and r.shape != x.shape or w is not None and w.shape != (K,):
        raise ValueError("rmsnorm: shapes of x, r and w disagree")
    s = np.empty_like(x) if r is not None else None
    y = np.empty_like(x)
    _check(_load().orc_rmsnorm(_p(x), _p(r), _p(w), ctypes.c_float(eps), B, K, _p(s), _p(y)), "rmsnorm")
    return s, y


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """``h = fl32((g / (1 + exp(-g))) * u)`` evaluated in binary64, elementwise."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    if g.shape != u.shape:
        raise ValueError("swiglu: g and u differ in shape")
    h = np.empty_like(g)
    _check(_load().orc_swiglu(_p(g), _p(u), g.size, _p(h)), "swiglu")
    return h


# Activation numbers of the gated product (the lane kernel library page's lk_act)
SILU, SIGMOID, GELU_TANH = 0, 1, 2


def glu(act: int, g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """``h = fl32(act(g) * u)`` evaluated in binary64, elementwise: act 0 silu
    ``g / (1 + exp(-g))``, 1 sigmoid ``1 / (1 + exp(-g))``, 2 the tanh-form GELU
    ``g / (1 + exp(-2z))``, ``z = sqrt(2/pi) * (g + 0.044715 g^3)``."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    if g.shape != u.shape:
        raise ValueError("glu: g and u differ in shape")
    h = np.empty_like(g)
    _check(_load().orc_glu(int(act), _p(g), _p(u), g.size, _p(h)), "glu")
    return h


# GGUF type numbers of the block formats
Q4_0, Q4_1, Q5_0, Q5_1, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, IQ4_NL, IQ4_XS, MXFP4 = 2, 3, 6, 7, 10, 11, 12, 13, 14, 20, 23, 39
FORMATS = (Q4_0, Q4_1, Q5_0, Q5_1, Q2_K, Q3_K, Q4_K, Q5_K, Q6_K, IQ4_NL, IQ4_XS, MXFP4)


def fmt_geometry(fmt: int) -> tuple[int, int]:
    """``(values, bytes)`` per block of the format."""
    v, b = ctypes.c_int(), ctypes.c_int()
    _check(_load().orc_fmt_geometry(fmt, ctypes.byref(v), ctypes.byref(b)), "fmt_geometry")
    return v.value, b.value


def fmt_row_bytes(fmt: int, K: int) -> int:
    return int(_load().orc_fmt_row_bytes(fmt, K))


def fmt_decode(fmt: int, w: np.ndarray, N: int, K: int):
    """``(levels int8 [N][K], d f32 [N][K/16], c f32 [N][K/16])``: weight k of row o is
    ``fl(fl(d[o][k/16] * levels[o][k]) + c[o][k/16])``."""
    w = _c(w, np.uint8)
    lv = np.empty((N, K), np.int8)
    d = np.empty((N, K // 16), np.float32)
    c = np.empty((N, K // 16), np.float32)
    _check(_load().orc_fmt_decode(fmt, _p(w), N, K, _p(lv), _p(d), _p(c)), "fmt_decode")
    return lv, d, c


def gemv_fmt(fmt: int, mode: int, w: np.ndarray, N: int, K: int, x=None, xq=None, xl=None, xs=None,
             splits: int = 1, nthreads: int = 1) -> np.ndarray:
    """``y [1][N]`` of a block-format matrix (batch 1) under the mode's numerics; with
    ``splits`` > 1 the chunk partials of the split rule added in ascending order."""
    w = _c(w, np.uint8)
    x, xq, xl, xs = _c(x, np.float32), _c(xq, np.int8), _c(xl, np.int8), _c(xs, np.float32)
    y = np.empty((1, N), np.float32)
    _check(_load().orc_gemv_fmt(fmt, mode, _p(w), N, K, _p(x), _p(xq), _p(xl), _p(xs), splits, _p(y), nthreads),
           "gemv_fmt")
    return y
