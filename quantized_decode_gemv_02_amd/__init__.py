"""Python binding of libqdg.so, the MI355X (gfx950) Q8_0 decode GEMV library.

Argument marshalling only: every step of the computation runs in the library's
HIP kernels.  PyTorch supplies device memory and the current HIP stream.  The
functions carry the names of the C entry points in ``include/qdg.h`` without the
``qdg_`` prefix:

* ``quantize_act(mode, x, xq, xl, xs)``
* ``gemv_q8(mode, wq, ws, out, x=None, xq=None, xl=None, xs=None, splits=1)``
* ``sk_combine(partials, y)``
* ``gemv_q8_sk(mode, wq, ws, y, xq, xl, xs, splits, workspace)`` / ``gemv_sk_workspace_bytes(B, N, S)``
* ``gemv_q8_fused(mode, wq, ws, y, x, splits, workspace)`` (quantize + GEMV + combine, one launch)
* ``q8_tile_rows(wq, wt)`` / ``gemv_q8_sk_tiled(mode, wt, ws, y, xq, xl, xs, splits)`` (row-tiled weights)
* ``argmax(y, idx, workspace)`` / ``argmax_workspace_bytes(B, N)``
* ``gemv_q8_argmax(mode, wq, ws, y, idx, workspace, x=, xq=, xl=, xs=)`` / ``gemv_argmax_workspace(N)``
* ``block_dots(mode, wq, xq, xl, dh, dl)``
* ``split_bounds(K, splits)`` (host only)

Every array is a contiguous torch tensor on the GPU (except ``split_bounds``),
with the dtypes of the header: int8 weights/words, int16-viewed binary16 weight
scales (``torch.float16`` tensors are accepted and reinterpreted), float32
activations, scales and outputs.  A non-zero status raises ``QdgError``.  If
``libqdg.so`` is missing, importing this package raises ``ImportError``: there is
no fallback implementation.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

DEQUANT, INT8ACT, TWOPASS = 0, 1, 2
QK = 32
MAX_B = 64
MAX_SPLITS = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqdg.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                      "or `python quantized_decode_gemv_02_amd/build.py`")

# The library and PyTorch must share one HIP runtime: PyTorch's libamdhip64.so
# has the soname libamdhip64.so.7 that libqdg.so needs, so loading torch first
# makes the dynamic linker bind libqdg.so to that copy.  Loaded the other way
# round, torch brings a second runtime into the process and the library's own
# runtime then finds no device (hipErrorNoDevice at the first launch).
import torch  # noqa: E402,F401  (load order only)

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int

_SIGS = {
    "qdg_abi_version": ([], _I),
    "qdg_status_str": ([_I], ctypes.c_char_p),
    "qdg_last_hip_error": ([], _I),
    "qdg_quantize_act": ([_I, _P, _I64, _I64, _P, _P, _P, _P], _I),
    "qdg_gemv_q8": ([_I, _P, _P, _I64, _I64, _P, _P, _P, _P, _I64, _I, _P, _P], _I),
    "qdg_sk_combine": ([_P, _I, _I64, _I64, _P, _P], _I),
    "qdg_gemv_sk_workspace_bytes": ([_I64, _I64, _I], ctypes.c_size_t),
    "qdg_gemv_sk_combines_in_workgroup": ([_I, _I64, _I, _P], _I),
    "qdg_gemv_q8_sk": ([_I, _P, _P, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P, ctypes.c_size_t, _P], _I),
    "qdg_gemv_q8_fused": ([_I, _P, _P, _I64, _I64, _P, _I, _P, _P, ctypes.c_size_t, _P], _I),
    "qdg_q8_tile_rows": ([_P, _I64, _I64, _P, _P], _I),
    "qdg_gemv_q8_sk_tiled": ([_I, _P, _P, _I64, _I64, _P, _P, _P, _I, _P, _P], _I),
    "qdg_q8_tile_mma_bytes": ([_I64, _I64], _I64),
    "qdg_q8_tile_mma": ([_P, _P, _I64, _I64, _P, _P], _I),
    "qdg_gemv_q8_mma_tiled": ([_I, _P, _I64, _I64, _P, _P, _P, _I64, _I, _P, _P], _I),
    "qdg_quantize_act_mma": ([_I, _P, _I64, _I64, _P, _P, _P, _P], _I),
    "qdg_gemv_argmax_workspace_bytes": ([_I64], ctypes.c_size_t),
    "qdg_gemv_q8_argmax": ([_I, _P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P], _I),
    "qdg_argmax_workspace_bytes": ([_I64, _I64], ctypes.c_size_t),
    "qdg_argmax": ([_P, _I64, _I64, _P, _P, ctypes.c_size_t, _P], _I),
    "qdg_block_dots": ([_I, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P], _I),
    "qdg_split_bounds": ([_I64, _I, _P], _I),
    "qdg_stream_read": ([_P, _I64, _P, _P], _I),
    "qdg_rmsnorm_quantize": ([_I, _P, _P, _P, _P, ctypes.c_float, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "qdg_rmsnorm_max_k": ([], _I64),
    "qdg_gemv_rmsnorm_workspace_bytes": ([_I64], ctypes.c_size_t),
    "qdg_gemv_rmsnorm_max_n": ([], _I64),
    "qdg_gemv_q8_rmsnorm": ([_I, _P, _P, _I64, _I64, _P, _P, _P, _I, _P, _P, _P, _P, ctypes.c_float, _I, _P, _P, _P,
                             _P, _P, ctypes.c_size_t, _P], _I),
    "qdg_swiglu_quantize": ([_I, _P, _P, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "qdg_glu_quantize": ([_I, _I, _P, _P, _I64, _I64, _P, _P, _P, _P, _P], _I),
    "qdg_gemv_q8_parts": ([_I, _P, _I, _I64, _P, _P, _P, _P, _I, _P], _I),
    "qdg_gemv_glu_q8": ([_I, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "qdg_gemv_glu_act_q8": ([_I, _I, _P, _P, _P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "qdg_gemv_glu_dequant": ([_I, _P, _P, _P, _P, _I64, _I64, _P, _P, _P], _I),
    "qdg_gemv_glu_mma_tiled": ([_I, _I, _P, _P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _P, _P, _P], _I),
    "qdg_fmt_row_bytes": ([_I, _I64], _I64),
    "qdg_gemv_fmt": ([_I, _I, _P, _I64, _I64, _P, _P, _P, _P, _I, _P, _P], _I),
    "qdg_gemv_fmt_chunk_waves": ([_I, _I, _I64, _I64, _I], _I),
    "qdg_gemv_dq_chunk_waves": ([_I64, _I64, _I], _I),
    "qdg_gemv_q8_argmax_noalloc": ([_I, _P, _P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P], _I),
    "qdg_set_tuning": ([_I, _I], _I),
    "qdg_get_tuning": ([_I], _I),
    "qdg_time_next_launch": ([_P, _P], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTS = tuple(_SIGS)


class QdgError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.qdg_status_str(status).decode()
        if status == -6:
            msg += f" (hipError_t {_lib.qdg_last_hip_error()})"
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise QdgError(fn, status)


# qdg_set_tuning's knobs (include/qdg.h): they choose among kernels, stagings and
# launch shapes that give the same bits; -1 is the library's own choice.
TUNE = {"sk_wsplit": 0, "ws_dma": 1, "ws_local": 2, "ws_rows": 3, "dq_seg": 4, "dq_rows": 5, "dq_x64": 6,
        "mfma_general": 7, "mfma_shape": 8, "mfma_wide": 9, "gemv_order": 10, "gemv_rpw": 11,
        "gemv_unroll": 12, "reject_launch": 13, "fmt_waves": 14, "dq_waves": 15, "mt_groups": 16}


def set_tuning(knob: str, value: int) -> None:
    _check("qdg_set_tuning", _lib.qdg_set_tuning(TUNE[knob], int(value)))


def get_tuning(knob: str) -> int:
    return int(_lib.qdg_get_tuning(TUNE[knob]))


@contextlib.contextmanager
def tuning(**knobs):
    """Sets the named knobs (``tuning(ws_dma=0, ws_local=1)``) for the block and restores them after."""
    old = {k: get_tuning(k) for k in knobs}
    try:
        for k, v in knobs.items():
            set_tuning(k, -1 if v is None else v)
        yield
    finally:
        for k, v in old.items():
            set_tuning(k, v)


def time_next_launch(start, stop) -> None:
    """Binds two recorded ``torch.cuda.Event(enable_timing=True)`` to the next kernel this thread's
    calls launch: ``start.elapsed_time(stop)`` is then that kernel's device duration."""
    _check("qdg_time_next_launch", _lib.qdg_time_next_launch(ctypes.c_void_p(start.cuda_event),
                                                              ctypes.c_void_p(stop.cuda_event)))


def abi_version() -> int:
    return _lib.qdg_abi_version()


def status_str(status: int) -> str:
    return _lib.qdg_status_str(status).decode()


def raw():
    """The ctypes handle of libqdg.so (for tests that call the C ABI directly)."""
    return _lib


def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in dtype:
        raise TypeError(f"{name} must have dtype in {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _need(**sized) -> None:
    """Host-side size checks before a call: each keyword is ``name=(tensor, elements)``; a tensor
    (when given) holding fewer elements than the call reads or writes raises ValueError, so an
    undersized buffer never reaches the device."""
    for name, (t, n) in sized.items():
        if t is not None and t.numel() < n:
            raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _gemv_sizes(mode, wq_shape, ws, B, x=None, xq=None, xl=None, xs=None, **outs) -> None:
    """The sizes every GEMV entry point assumes: ws [N][K/32], the activation of B rows in the
    mode's encoding, and each output's element count (``outs``: name=(tensor, elements))."""
    N, K = wq_shape
    if ws is not None and tuple(ws.shape) != (N, K // QK) and ws.numel() != N * (K // QK):
        raise ValueError(f"ws must hold [N][K/32] = [{N}][{K // QK}] scales, got shape {tuple(ws.shape)}")
    _need(x=(x, B * K), xq=(xq, B * K), xl=(xl, B * K), xs=(xs, B * (K // QK)), **outs)


def _i8():
    return (_torch().int8,)


def _f32():
    return (_torch().float32,)


def _scales():
    torch = _torch()
    return (torch.int16, torch.float16, torch.uint16) if hasattr(torch, "uint16") else (torch.int16, torch.float16)


def quantize_act(mode: int, x, xq, xl, xs) -> None:
    """``x [B][K]`` float32 -> ``xq`` (and ``xl`` under TwoPass) int8 ``[B][K]``, ``xs [B][K/32]``."""
    B, K = x.shape if x.dim() == 2 else (1, x.shape[0])
    _need(xq=(xq, B * K), xl=(xl, B * K), xs=(xs, B * (K // QK)))
    _check("qdg_quantize_act", _lib.qdg_quantize_act(
        mode, _ptr(x, _f32(), "x"), B, K, _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"),
        _stream()))


def _rows(t):
    return t.shape if t.dim() == 2 else (1, t.shape[0])


def _rmsnorm_args(mode, x, w, r, s, y, xq, xl, xs, eps):
    B, K = _rows(x)
    return (mode, _ptr(x, _f32(), "x"), _ptr(r, _f32(), "r"), _ptr(s, _f32(), "s"), _ptr(w, _f32(), "w"),
            float(eps), B, K, _ptr(y, _f32(), "y"), _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"),
            _ptr(xs, _f32(), "xs"), _stream())


def rmsnorm_quantize(mode: int, x, w=None, r=None, s=None, y=None, xq=None, xl=None, xs=None,
                     eps: float = 1e-6) -> None:
    """Residual add + RMSNorm + the activation quantizer in one launch: ``s = x + r``
    (optional), ``y = (x + r) / sqrt(mean((x + r)^2) + eps) * w`` (optional output
    under the quantized modes, the only output under Dequant), then ``xq/xl/xs``."""
    _check("qdg_rmsnorm_quantize", _lib.qdg_rmsnorm_quantize(*_rmsnorm_args(mode, x, w, r, s, y, xq, xl, xs, eps)))


def bind_rmsnorm_quantize(mode: int, x, w=None, r=None, s=None, y=None, xq=None, xl=None, xs=None,
                          eps: float = 1e-6) -> Bound:
    return Bound("qdg_rmsnorm_quantize", *_rmsnorm_args(mode, x, w, r, s, y, xq, xl, xs, eps))


def rmsnorm_max_k() -> int:
    return int(_lib.qdg_rmsnorm_max_k())


def _swiglu_args(mode, g, u, h, xq, xl, xs):
    B, K = _rows(g)
    if tuple(u.shape) != tuple(g.shape):
        raise ValueError("swiglu_quantize: g and u differ in shape")
    return (mode, _ptr(g, _f32(), "g"), _ptr(u, _f32(), "u"), B, K, _ptr(h, _f32(), "h"),
            _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), _stream())


def swiglu_quantize(mode: int, g, u, h=None, xq=None, xl=None, xs=None) -> None:
    """``h = silu(g) * u`` (optional output under the quantized modes) and its quantized words."""
    _check("qdg_swiglu_quantize", _lib.qdg_swiglu_quantize(*_swiglu_args(mode, g, u, h, xq, xl, xs)))


def bind_swiglu_quantize(mode: int, g, u, h=None, xq=None, xl=None, xs=None) -> Bound:
    return Bound("qdg_swiglu_quantize", *_swiglu_args(mode, g, u, h, xq, xl, xs))


# The activations of the gated product (include/qdg.h: QDG_ACT_*, the lane kernel library page's lk_act numbers)
ACT_SILU, ACT_SIGMOID, ACT_GELU_TANH = 0, 1, 2


def glu_quantize(act: int, mode: int, g, u, h=None, xq=None, xl=None, xs=None) -> None:
    """``h = act(g) * u`` (silu, sigmoid or the tanh-form GELU; optional output under the
    quantized modes) and its quantized words."""
    _check("qdg_glu_quantize", _lib.qdg_glu_quantize(act, *_swiglu_args(mode, g, u, h, xq, xl, xs)))


def bind_glu_quantize(act: int, mode: int, g, u, h=None, xq=None, xl=None, xs=None) -> Bound:
    return Bound("qdg_glu_quantize", act, *_swiglu_args(mode, g, u, h, xq, xl, xs))


def _glu_args(mode, wg, sg, wu, su, xq, xl, xs, h, hq, hl, hs):
    F, K = wg.shape
    if tuple(wu.shape) != (F, K):
        raise ValueError("gemv_glu_q8: gate and up must have the same shape")
    _need(sg=(sg, F * (K // QK)), su=(su, F * (K // QK)), xq=(xq, K), xl=(xl, K), xs=(xs, K // QK), h=(h, F),
          hq=(hq, F), hl=(hl, F), hs=(hs, F // QK))
    return (mode, _ptr(wg, _i8(), "wg"), _ptr(sg, _scales(), "sg"), _ptr(wu, _i8(), "wu"), _ptr(su, _scales(), "su"),
            F, K, _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), _ptr(h, _f32(), "h"),
            _ptr(hq, _i8(), "hq"), _ptr(hl, _i8(), "hl"), _ptr(hs, _f32(), "hs"), _stream())


def gemv_glu_q8(mode: int, wg, sg, wu, su, xq, xl, xs, hq, hl, hs, h=None) -> None:
    """Gate and up GEMVs with the SwiGLU and quantizer epilogue: ``(hq, hl, hs)`` is
    ``silu(Wg x) * (Wu x)`` quantized (``h``, optional, the f32 SwiGLU output)."""
    _check("qdg_gemv_glu_q8", _lib.qdg_gemv_glu_q8(*_glu_args(mode, wg, sg, wu, su, xq, xl, xs, h, hq, hl, hs)))


def bind_gemv_glu_q8(mode: int, wg, sg, wu, su, xq, xl, xs, hq, hl, hs, h=None) -> Bound:
    return Bound("qdg_gemv_glu_q8", *_glu_args(mode, wg, sg, wu, su, xq, xl, xs, h, hq, hl, hs))


def gemv_glu_act_q8(act: int, mode: int, wg, sg, wu, su, xq, xl, xs, hq, hl, hs, h=None) -> None:
    """``gemv_glu_q8`` with any of the gated product's activations (``ACT_*``)."""
    _check("qdg_gemv_glu_act_q8",
           _lib.qdg_gemv_glu_act_q8(act, *_glu_args(mode, wg, sg, wu, su, xq, xl, xs, h, hq, hl, hs)))


def bind_gemv_glu_act_q8(act: int, mode: int, wg, sg, wu, su, xq, xl, xs, hq, hl, hs, h=None) -> Bound:
    return Bound("qdg_gemv_glu_act_q8", act, *_glu_args(mode, wg, sg, wu, su, xq, xl, xs, h, hq, hl, hs))


def _glu_dequant_args(act, wg, sg, wu, su, x, h):
    F, K = wg.shape
    if tuple(wu.shape) != (F, K):
        raise ValueError("gemv_glu_dequant: gate and up must have the same shape")
    if x.numel() != K or h.numel() != F:
        raise ValueError("gemv_glu_dequant: x must hold K values and h F values")
    _need(sg=(sg, F * (K // QK)), su=(su, F * (K // QK)))
    return (act, _ptr(wg, _i8(), "wg"), _ptr(sg, _scales(), "sg"), _ptr(wu, _i8(), "wu"), _ptr(su, _scales(), "su"),
            F, K, _ptr(x, _f32(), "x"), _ptr(h, _f32(), "h"), _stream())


def gemv_glu_dequant(act: int, wg, sg, wu, su, x, h) -> None:
    """Gate and up GEMVs under the Dequant numerics with the gated product as the
    epilogue: ``h = act(Wg x) * (Wu x)`` in f32, the down projection's input."""
    _check("qdg_gemv_glu_dequant", _lib.qdg_gemv_glu_dequant(*_glu_dequant_args(act, wg, sg, wu, su, x, h)))


def bind_gemv_glu_dequant(act: int, wg, sg, wu, su, x, h) -> Bound:
    return Bound("qdg_gemv_glu_dequant", *_glu_dequant_args(act, wg, sg, wu, su, x, h))


# GGUF type numbers of the other block formats
FMT_Q4_0, FMT_Q4_1, FMT_Q5_0, FMT_Q5_1, FMT_Q2_K, FMT_Q3_K = 2, 3, 6, 7, 10, 11
FMT_Q4_K, FMT_Q5_K, FMT_Q6_K, FMT_IQ4_NL, FMT_IQ4_XS, FMT_MXFP4 = 12, 13, 14, 20, 23, 39


def fmt_row_bytes(fmt: int, K: int) -> int:
    return int(_lib.qdg_fmt_row_bytes(fmt, K))


def _fmt_args(fmt, mode, w, N, K, y, x, xq, xl, xs, splits):
    if w.numel() < N * fmt_row_bytes(fmt, K):
        raise ValueError("gemv_fmt: w is smaller than N rows of the format")
    return (fmt, mode, _ptr(w, (_torch().uint8, _torch().int8), "w"), N, K, _ptr(x, _f32(), "x"),
            _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), splits, _ptr(y, _f32(), "y"),
            _stream())


def gemv_fmt(fmt: int, mode: int, w, N: int, K: int, y, x=None, xq=None, xl=None, xs=None, splits: int = 1) -> None:
    """``y [N] = W x`` for ``w``, N rows of K values in GGUF block format ``fmt`` (bytes as stored),
    the row cut into ``splits`` split-K chunks added in ascending order."""
    _check("qdg_gemv_fmt", _lib.qdg_gemv_fmt(*_fmt_args(fmt, mode, w, N, K, y, x, xq, xl, xs, splits)))


def bind_gemv_fmt(fmt: int, mode: int, w, N: int, K: int, y, x=None, xq=None, xl=None, xs=None,
                  splits: int = 1) -> Bound:
    return Bound("qdg_gemv_fmt", *_fmt_args(fmt, mode, w, N, K, y, x, xq, xl, xs, splits))


MAX_PARTS = 6


class _Part(ctypes.Structure):
    _fields_ = [("wq", ctypes.c_void_p), ("ws", ctypes.c_void_p), ("N", ctypes.c_int64), ("y", ctypes.c_void_p)]


def _parts_args(mode, parts, x, xq, xl, xs, splits):
    if not 1 <= len(parts) <= MAX_PARTS:
        raise ValueError(f"gemv_q8_parts: 1 to {MAX_PARTS} parts")
    K = parts[0][0].shape[1]
    arr = (_Part * len(parts))()
    for i, (wq, ws, y) in enumerate(parts):
        if wq.shape[1] != K:
            raise ValueError("gemv_q8_parts: every part must have the same K")
        arr[i] = _Part(_ptr(wq, _i8(), "wq"), _ptr(ws, _scales(), "ws"), wq.shape[0], _ptr(y, _f32(), "y"))
    return (mode, ctypes.cast(arr, ctypes.c_void_p), len(parts), K, _ptr(x, _f32(), "x"), _ptr(xq, _i8(), "xq"),
            _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), int(splits), _stream()), arr


def gemv_q8_parts(mode: int, parts, x=None, xq=None, xl=None, xs=None, splits: int = 4) -> None:
    """``parts``: list of ``(wq [N_p][K], ws, y [N_p])``; one launch computes every ``y_p = W_p x``."""
    args, _keep = _parts_args(mode, parts, x, xq, xl, xs, splits)
    _check("qdg_gemv_q8_parts", _lib.qdg_gemv_q8_parts(*args))


def bind_gemv_q8_parts(mode: int, parts, x=None, xq=None, xl=None, xs=None, splits: int = 4) -> Bound:
    args, keep = _parts_args(mode, parts, x, xq, xl, xs, splits)
    b = Bound("qdg_gemv_q8_parts", *args)
    b.keep = keep  # the host part table must outlive the bound call
    return b


def gemv_q8(mode: int, wq, ws, out, x=None, xq=None, xl=None, xs=None, splits: int = 1) -> None:
    """``out = Y [B][N]`` (``splits == 1``) or the partials ``[splits][B][N]``."""
    N, K = wq.shape
    act = x if mode == DEQUANT else xq
    B = act.shape[0] if act.dim() == 2 else 1
    _gemv_sizes(mode, wq.shape, ws, B, x, xq, xl, xs, out=(out, int(splits) * B * N))
    _check("qdg_gemv_q8", _lib.qdg_gemv_q8(
        mode, _ptr(wq, _i8(), "wq"), _ptr(ws, _scales(), "ws"), N, K, _ptr(x, _f32(), "x"),
        _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), B, int(splits),
        _ptr(out, _f32(), "out"), _stream()))


def gemv_sk_workspace_bytes(B: int, N: int, splits: int) -> int:
    return int(_lib.qdg_gemv_sk_workspace_bytes(B, N, splits))


def sk_combines_in_workgroup(mode: int, K: int, splits: int) -> bool:
    """Whether ``gemv_q8_sk`` adds the chunk partials inside a workgroup (LDS) for this shape."""
    return sk_workgroup_shape(mode, K, splits) is not None


def sk_workgroup_shape(mode: int, K: int, splits: int):
    """``(rows, waves)`` per workgroup of the in-workgroup launch, or ``None`` (workspace path)."""
    arr = (ctypes.c_int32 * 2)()
    r = int(_lib.qdg_gemv_sk_combines_in_workgroup(mode, K, splits, ctypes.cast(arr, ctypes.c_void_p)))
    if r < 0:
        _check("qdg_gemv_sk_combines_in_workgroup", r)
    return (int(arr[0]), int(arr[1])) if r == 1 else None


def fmt_chunk_waves(fmt: int, mode: int, N: int, K: int, splits: int) -> int:
    """Chunk waves a workgroup's rows get in ``gemv_fmt`` for this shape on the current device."""
    r = int(_lib.qdg_gemv_fmt_chunk_waves(fmt, mode, N, K, splits))
    _check("qdg_gemv_fmt_chunk_waves", r if r < 0 else 0)
    return r


def dq_chunk_waves(N: int, K: int, splits: int) -> int:
    """Chunk waves a workgroup's rows get in the Dequant chunk-wave kernel on the current device."""
    r = int(_lib.qdg_gemv_dq_chunk_waves(N, K, splits))
    _check("qdg_gemv_dq_chunk_waves", r if r < 0 else 0)
    return r


def sk_workspace(N: int, splits: int):
    """A zero-filled device workspace for ``gemv_q8_sk`` (int64 words; torch allocations are 256-byte aligned)."""
    torch = _torch()
    nbytes = max(gemv_sk_workspace_bytes(1, N, splits), 8)
    return torch.zeros((nbytes + 7) // 8, dtype=torch.int64, device="cuda")


def gemv_q8_sk(mode: int, wq, ws, y, xq, xl, xs, splits: int, workspace) -> None:
    """Split-K GEMV whose last-arriving workgroups do the ascending combine: ``y [1][N]``."""
    N, K = wq.shape
    B = xq.shape[0] if xq.dim() == 2 else 1
    _gemv_sizes(mode, wq.shape, ws, B, None, xq, xl, xs, y=(y, B * N))
    nbytes = workspace.numel() * workspace.element_size()
    _check("qdg_gemv_q8_sk", _lib.qdg_gemv_q8_sk(
        mode, _ptr(wq, _i8(), "wq"), _ptr(ws, _scales(), "ws"), N, K, _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"),
        _ptr(xs, _f32(), "xs"), B, int(splits), _ptr(y, _f32(), "y"), _ptr(workspace, None, "workspace"), nbytes,
        _stream()))


def q8_tile_rows(wq, wt) -> None:
    """The weight values ``wq [N][K]`` in row tiles of four rows by 256 values, into ``wt`` (same shape)."""
    N, K = wq.shape
    if tuple(wt.shape) != (N, K):
        raise ValueError("q8_tile_rows: wt must have the shape of wq")
    _check("qdg_q8_tile_rows", _lib.qdg_q8_tile_rows(_ptr(wq, _i8(), "wq"), N, K, _ptr(wt, _i8(), "wt"), _stream()))


def gemv_q8_sk_tiled(mode: int, wt, ws, y, xq, xl, xs, splits: int) -> None:
    """``gemv_q8_sk``'s in-workgroup placement over row-tiled weights ``wt`` (from ``q8_tile_rows``)."""
    N, K = wt.shape
    _gemv_sizes(mode, wt.shape, ws, 1, None, xq, xl, xs, y=(y, N))
    _check("qdg_gemv_q8_sk_tiled", _lib.qdg_gemv_q8_sk_tiled(
        mode, _ptr(wt, _i8(), "wt"), _ptr(ws, _scales(), "ws"), N, K, _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"),
        _ptr(xs, _f32(), "xs"), int(splits), _ptr(y, _f32(), "y"), _stream()))


def _u8():
    torch = _torch()
    return (torch.uint8, torch.int8)


def q8_tile_mma_bytes(N: int, K: int) -> int:
    """Bytes of the MFMA-tiled form of an ``[N][K]`` Q8_0 matrix (0: shape not served)."""
    return int(_lib.qdg_q8_tile_mma_bytes(N, K))


def q8_tile_mma(wq, ws, wt) -> None:
    """The weights ``wq [N][K]`` and scales ``ws [N][K/32]`` as MFMA-tiled records, into the byte array ``wt``."""
    N, K = wq.shape
    _gemv_sizes(1, wq.shape, ws, 1)
    _need(wt=(wt, q8_tile_mma_bytes(N, K) // wt.element_size()))
    _check("qdg_q8_tile_mma", _lib.qdg_q8_tile_mma(
        _ptr(wq, _i8(), "wq"), _ptr(ws, _scales(), "ws"), N, K, _ptr(wt, _u8(), "wt"), _stream()))


def mma_act_rows(B: int) -> int:
    """Rows of the MFMA-ordered activations for a batch of B: 16 activation-tile rows times 1, 2 or 4."""
    return 16 if B <= 16 else 32 if B <= 32 else 64


def quantize_act_mma(mode: int, x, xq, xl, xs) -> None:
    """``x [B][K]`` quantized as ``quantize_act`` does, written in the MFMA order ``gemv_q8_mma_tiled``
    reads: ``xq``, ``xl`` hold ``mma_act_rows(B)*K`` int8, ``xs`` ``mma_act_rows(B)*K/32`` float32."""
    B, K = x.shape if x.dim() == 2 else (1, x.shape[0])
    R = mma_act_rows(B)
    _need(xq=(xq, R * K), xl=(xl, R * K), xs=(xs, R * (K // QK)))
    _check("qdg_quantize_act_mma", _lib.qdg_quantize_act_mma(
        mode, _ptr(x, _f32(), "x"), B, K, _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"),
        _stream()))


def gemv_q8_mma_tiled(mode: int, wt, N: int, K: int, out, xq, xl, xs, B: int, splits: int = 1) -> None:
    """``gemv_q8`` for B <= 16 activation rows over MFMA-tiled weights ``wt`` (from ``q8_tile_mma``) and
    MFMA-ordered activations (from ``quantize_act_mma``): ``out = Y [B][N]`` (``splits == 1``) or the
    partials ``[splits][B][N]``."""
    R = mma_act_rows(B)
    _need(xq=(xq, R * K), xl=(xl, R * K), xs=(xs, R * (K // QK)), out=(out, int(splits) * B * N))
    _need(wt=(wt, q8_tile_mma_bytes(N, K) // wt.element_size()))
    _check("qdg_gemv_q8_mma_tiled", _lib.qdg_gemv_q8_mma_tiled(
        mode, _ptr(wt, _u8(), "wt"), N, K, _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"),
        B, int(splits), _ptr(out, _f32(), "out"), _stream()))


def _glu_mma_args(act, mode, wgt, wut, F, K, xq, xl, xs, B, hq, hl, hs, h):
    R = mma_act_rows(B)
    _need(xq=(xq, R * K), xl=(xl, R * K), xs=(xs, R * (K // QK)), hq=(hq, R * F), hl=(hl, R * F),
          hs=(hs, R * (F // QK)))
    if h is not None:
        _need(h=(h, B * F))
    _need(wgt=(wgt, q8_tile_mma_bytes(F, K) // wgt.element_size()), wut=(wut, q8_tile_mma_bytes(F, K) // wut.element_size()))
    return (act, mode, _ptr(wgt, _u8(), "wgt"), _ptr(wut, _u8(), "wut"), F, K, _ptr(xq, _i8(), "xq"),
            _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), B, _ptr(h, _f32(), "h"), _ptr(hq, _i8(), "hq"),
            _ptr(hl, _i8(), "hl"), _ptr(hs, _f32(), "hs"), _stream())


def gemv_glu_mma_tiled(act: int, mode: int, wgt, wut, F: int, K: int, xq, xl, xs, B: int, hq, hl, hs,
                       h=None) -> None:
    """Gate and up GEMVs of B <= 64 rows over MFMA-tiled weights (``q8_tile_mma`` of each ``[F][K]``
    matrix) and MFMA-ordered activations, with the gated product and the quantizer as the epilogue:
    ``(hq, hl, hs)`` hold ``act(g) * u`` quantized in the MFMA order ``quantize_act_mma`` writes for
    K = F (``mma_act_rows(B)*F`` words, ``mma_act_rows(B)*F/32`` scales); ``h`` (optional) is ``[B][F]``."""
    _check("qdg_gemv_glu_mma_tiled", _lib.qdg_gemv_glu_mma_tiled(
        *_glu_mma_args(act, mode, wgt, wut, F, K, xq, xl, xs, B, hq, hl, hs, h)))


def bind_gemv_glu_mma_tiled(act: int, mode: int, wgt, wut, F: int, K: int, xq, xl, xs, B: int, hq, hl, hs,
                            h=None) -> Bound:
    return Bound("qdg_gemv_glu_mma_tiled", *_glu_mma_args(act, mode, wgt, wut, F, K, xq, xl, xs, B, hq, hl, hs, h))


def gemv_q8_fused(mode: int, wq, ws, y, x, splits: int = 1, workspace=None) -> None:
    """One launch for a batch-1 projection: quantize ``x [1][K]`` (f32), split-K GEMV and ascending
    combine into ``y [1][N]`` (``workspace`` from ``sk_workspace(N, splits)``; may be None when S == 1)."""
    N, K = wq.shape
    _gemv_sizes(mode, wq.shape, ws, 1, x, y=(y, N))
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("qdg_gemv_q8_fused", _lib.qdg_gemv_q8_fused(
        mode, _ptr(wq, _i8(), "wq"), _ptr(ws, _scales(), "ws"), N, K, _ptr(x, _f32(), "x"), int(splits),
        _ptr(y, _f32(), "y"), _ptr(workspace, None, "workspace"), nbytes, _stream()))


def sk_combine(partials, y) -> None:
    """``y [B][N]`` = ascending sum over the leading axis of ``partials [S][B][N]``."""
    S = partials.shape[0]
    N = partials.shape[-1]
    B = partials.numel() // (S * N)
    _check("qdg_sk_combine", _lib.qdg_sk_combine(_ptr(partials, _f32(), "partials"), S, B, N,
                                                 _ptr(y, _f32(), "y"), _stream()))


def gemv_argmax_workspace_bytes(N: int) -> int:
    return int(_lib.qdg_gemv_argmax_workspace_bytes(N))


def gemv_argmax_workspace(N: int):
    """A device workspace for ``gemv_q8_argmax`` (int64 words)."""
    return _torch().empty((gemv_argmax_workspace_bytes(N) + 7) // 8, dtype=_torch().int64, device="cuda")


def gemv_q8_argmax(mode: int, wq, ws, y, idx, workspace, x=None, xq=None, xl=None, xs=None) -> None:
    """LM-head tail: ``y [1][N]`` logits and ``idx [1]`` int32 first index of their maximum, in two launches."""
    N, K = wq.shape
    _gemv_sizes(mode, wq.shape, ws, 1, x, xq, xl, xs, y=(y, N), idx=(idx, 1))
    nbytes = workspace.numel() * workspace.element_size()
    _check("qdg_gemv_q8_argmax", _lib.qdg_gemv_q8_argmax(
        mode, _ptr(wq, _i8(), "wq"), _ptr(ws, _scales(), "ws"), N, K, _ptr(x, _f32(), "x"), _ptr(xq, _i8(), "xq"),
        _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), _ptr(y, _f32(), "y"), _ptr(idx, (_torch().int32,), "idx"),
        _ptr(workspace, None, "workspace"), nbytes, _stream()))


def bind_gemv_q8_argmax(mode: int, wq, ws, y, idx, workspace, x=None, xq=None, xl=None, xs=None) -> Bound:
    N, K = wq.shape
    _gemv_sizes(mode, wq.shape, ws, 1, x, xq, xl, xs, y=(y, N), idx=(idx, 1))
    for t, n in ((wq, "wq"), (ws, "ws"), (y, "y"), (idx, "idx"), (workspace, "workspace"), (x, "x"), (xq, "xq"),
                 (xl, "xl"), (xs, "xs")):
        _ptr(t, None, n)
    nbytes = workspace.numel() * workspace.element_size()
    return Bound("qdg_gemv_q8_argmax", mode, wq, ws, N, K, x, xq, xl, xs, y, idx, workspace, nbytes, _stream())


def gemv_q8_argmax_noalloc(mode: int, wq, ws, y, idx, x=None, xq=None, xl=None, xs=None) -> None:
    """``gemv_q8_argmax`` with the keys in the library's own per-GPU array (no workspace,
    nothing allocated; calls on one GPU must not overlap in time)."""
    N, K = wq.shape
    _gemv_sizes(mode, wq.shape, ws, 1, x, xq, xl, xs, y=(y, N), idx=(idx, 1))
    _check("qdg_gemv_q8_argmax_noalloc", _lib.qdg_gemv_q8_argmax_noalloc(
        mode, _ptr(wq, _i8(), "wq"), _ptr(ws, _scales(), "ws"), N, K, _ptr(x, _f32(), "x"), _ptr(xq, _i8(), "xq"),
        _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), _ptr(y, _f32(), "y"), _ptr(idx, (_torch().int32,), "idx"),
        _stream()))


def gemv_rmsnorm_workspace_bytes(N: int) -> int:
    return int(_lib.qdg_gemv_rmsnorm_workspace_bytes(N))


def gemv_rmsnorm_max_n() -> int:
    return int(_lib.qdg_gemv_rmsnorm_max_n())


def gemv_rmsnorm_workspace(N: int):
    """A zero-filled device workspace for ``gemv_q8_rmsnorm`` (int64 words, 256-byte aligned)."""
    torch = _torch()
    nbytes = max(gemv_rmsnorm_workspace_bytes(N), 8)
    return torch.zeros((nbytes + 7) // 8, dtype=torch.int64, device="cuda")


def _gemv_rmsnorm_args(mode, wq, ws, xq, xl, xs, splits, y, r, s, w, eps, qmode, yn, hq, hl, hs, workspace):
    N, K = wq.shape
    _gemv_sizes(mode, wq.shape, ws, 1, None, xq, xl, xs, y=(y, N), r=(r, N), s=(s, N), w=(w, N), yn=(yn, N),
                hq=(hq, N), hl=(hl, N), hs=(hs, N // QK))
    nbytes = workspace.numel() * workspace.element_size()
    return (mode, _ptr(wq, _i8(), "wq"), _ptr(ws, _scales(), "ws"), N, K, _ptr(xq, _i8(), "xq"),
            _ptr(xl, _i8(), "xl"), _ptr(xs, _f32(), "xs"), int(splits), _ptr(y, _f32(), "y"), _ptr(r, _f32(), "r"),
            _ptr(s, _f32(), "s"), _ptr(w, _f32(), "w"), float(eps), int(qmode), _ptr(yn, _f32(), "yn"),
            _ptr(hq, _i8(), "hq"), _ptr(hl, _i8(), "hl"), _ptr(hs, _f32(), "hs"), _ptr(workspace, None, "workspace"),
            nbytes, _stream())


def gemv_q8_rmsnorm(mode: int, wq, ws, xq, xl, xs, splits: int, workspace, y=None, r=None, s=None, w=None,
                    eps: float = 1e-6, qmode: int = INT8ACT, yn=None, hq=None, hl=None, hs=None) -> None:
    """One launch: the split-K projection ``y = W x`` (``gemv_q8_sk``), then in its last workgroup
    ``s = y + r``, the RMSNorm ``yn`` and its words ``hq/hl/hs`` in mode ``qmode``
    (``rmsnorm_quantize``); ``workspace`` from ``gemv_rmsnorm_workspace(N)``."""
    _check("qdg_gemv_q8_rmsnorm", _lib.qdg_gemv_q8_rmsnorm(*_gemv_rmsnorm_args(
        mode, wq, ws, xq, xl, xs, splits, y, r, s, w, eps, qmode, yn, hq, hl, hs, workspace)))


def bind_gemv_q8_rmsnorm(mode: int, wq, ws, xq, xl, xs, splits: int, workspace, y=None, r=None, s=None, w=None,
                         eps: float = 1e-6, qmode: int = INT8ACT, yn=None, hq=None, hl=None, hs=None) -> "Bound":
    return Bound("qdg_gemv_q8_rmsnorm", *_gemv_rmsnorm_args(
        mode, wq, ws, xq, xl, xs, splits, y, r, s, w, eps, qmode, yn, hq, hl, hs, workspace))


def argmax_workspace_bytes(B: int, N: int) -> int:
    return int(_lib.qdg_argmax_workspace_bytes(B, N))


def argmax(y, idx, workspace) -> None:
    """``idx [B]`` int32 = first index of each row's maximum of ``y [B][N]``."""
    B, N = (y.shape if y.dim() == 2 else (1, y.shape[0]))
    nbytes = workspace.numel() * workspace.element_size()
    _check("qdg_argmax", _lib.qdg_argmax(_ptr(y, _f32(), "y"), B, N, _ptr(idx, (_torch().int32,), "idx"),
                                         _ptr(workspace, None, "workspace"), nbytes, _stream()))


def block_dots(mode: int, wq, xq, xl, dh, dl) -> None:
    """Exact int32 per-block dots ``dh``/``dl [B][N][K/32]`` (test hook)."""
    N, K = wq.shape
    B = xq.shape[0] if xq.dim() == 2 else 1
    i32 = (_torch().int32,)
    _check("qdg_block_dots", _lib.qdg_block_dots(
        mode, _ptr(wq, _i8(), "wq"), N, K, _ptr(xq, _i8(), "xq"), _ptr(xl, _i8(), "xl"), B,
        _ptr(dh, i32, "dh"), _ptr(dl, i32, "dl"), _stream()))


def split_bounds(K: int, splits: int) -> list[int]:
    arr = (ctypes.c_int32 * (splits + 1))()
    _check("qdg_split_bounds", _lib.qdg_split_bounds(K, splits, ctypes.cast(arr, ctypes.c_void_p)))
    return list(arr)


class Bound:
    """A C entry point with its ctypes arguments converted once (pointers, sizes,
    stream), for loops that launch the same call many times.  Calling it checks
    the status like the functions above."""

    def __init__(self, name: str, *args):
        self.name = name
        self.fn = getattr(_lib, name)
        self.args = tuple(self._conv(a) for a in args)

    @staticmethod
    def _conv(a):
        if a is None or isinstance(a, (int, ctypes.c_void_p)):
            return a
        if hasattr(a, "data_ptr"):
            return ctypes.c_void_p(a.data_ptr())
        return a

    def __call__(self) -> None:
        _check(self.name, self.fn(*self.args))


def bind_gemv_q8(mode: int, wq, ws, out, x=None, xq=None, xl=None, xs=None, splits: int = 1) -> Bound:
    N, K = wq.shape
    act = x if mode == DEQUANT else xq
    B = act.shape[0] if act.dim() == 2 else 1
    _gemv_sizes(mode, wq.shape, ws, B, x, xq, xl, xs, out=(out, int(splits) * B * N))
    for t, n in ((wq, "wq"), (ws, "ws"), (out, "out"), (x, "x"), (xq, "xq"), (xl, "xl"), (xs, "xs")):
        _ptr(t, None, n)
    return Bound("qdg_gemv_q8", mode, wq, ws, N, K, x, xq, xl, xs, B, int(splits), out, _stream())


def bind_gemv_q8_sk(mode: int, wq, ws, y, xq, xl, xs, splits: int, workspace) -> Bound:
    N, K = wq.shape
    B = xq.shape[0] if xq.dim() == 2 else 1
    _gemv_sizes(mode, wq.shape, ws, B, None, xq, xl, xs, y=(y, B * N))
    for t, n in ((wq, "wq"), (ws, "ws"), (y, "y"), (xq, "xq"), (xl, "xl"), (xs, "xs"), (workspace, "workspace")):
        _ptr(t, None, n)
    nbytes = workspace.numel() * workspace.element_size()
    return Bound("qdg_gemv_q8_sk", mode, wq, ws, N, K, xq, xl, xs, B, int(splits), y, workspace, nbytes, _stream())


def bind_gemv_q8_sk_tiled(mode: int, wt, ws, y, xq, xl, xs, splits: int) -> Bound:
    N, K = wt.shape
    _gemv_sizes(mode, wt.shape, ws, 1, None, xq, xl, xs, y=(y, N))
    for t, n in ((wt, "wt"), (ws, "ws"), (y, "y"), (xq, "xq"), (xl, "xl"), (xs, "xs")):
        _ptr(t, None, n)
    return Bound("qdg_gemv_q8_sk_tiled", mode, wt, ws, N, K, xq, xl, xs, int(splits), y, _stream())


def bind_gemv_q8_mma_tiled(mode: int, wt, N: int, K: int, out, xq, xl, xs, B: int, splits: int = 1) -> Bound:
    R = mma_act_rows(B)
    _need(xq=(xq, R * K), xl=(xl, R * K), xs=(xs, R * (K // QK)), out=(out, int(splits) * B * N))
    _need(wt=(wt, q8_tile_mma_bytes(N, K) // wt.element_size()))
    for t, n in ((wt, "wt"), (out, "out"), (xq, "xq"), (xl, "xl"), (xs, "xs")):
        _ptr(t, None, n)
    return Bound("qdg_gemv_q8_mma_tiled", mode, wt, N, K, xq, xl, xs, B, int(splits), out, _stream())


def bind_gemv_q8_fused(mode: int, wq, ws, y, x, splits: int = 1, workspace=None) -> Bound:
    N, K = wq.shape
    _gemv_sizes(mode, wq.shape, ws, 1, x, y=(y, N))
    for t, n in ((wq, "wq"), (ws, "ws"), (y, "y"), (x, "x"), (workspace, "workspace")):
        _ptr(t, None, n)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return Bound("qdg_gemv_q8_fused", mode, wq, ws, N, K, x, int(splits), y, workspace, nbytes, _stream())


def bind_stream_read(buf, nbytes: int, sink) -> Bound:
    """The measurement hook: read ``nbytes`` of ``buf`` once (the practical read ceiling)."""
    _ptr(buf, None, "buf")
    _ptr(sink, None, "sink")
    return Bound("qdg_stream_read", buf, int(nbytes), sink, _stream())


def bind_quantize_act_mma(mode: int, x, xq, xl, xs) -> Bound:
    B, K = x.shape if x.dim() == 2 else (1, x.shape[0])
    R = mma_act_rows(B)
    _need(xq=(xq, R * K), xl=(xl, R * K), xs=(xs, R * (K // QK)))
    for t, n in ((x, "x"), (xq, "xq"), (xl, "xl"), (xs, "xs")):
        _ptr(t, None, n)
    return Bound("qdg_quantize_act_mma", mode, x, B, K, xq, xl, xs, _stream())


def bind_quantize_act(mode: int, x, xq, xl, xs) -> Bound:
    B, K = x.shape if x.dim() == 2 else (1, x.shape[0])
    _need(xq=(xq, B * K), xl=(xl, B * K), xs=(xs, B * (K // QK)))
    for t, n in ((x, "x"), (xq, "xq"), (xl, "xl"), (xs, "xs")):
        _ptr(t, None, n)
    return Bound("qdg_quantize_act", mode, x, B, K, xq, xl, xs, _stream())


def bind_argmax(y, idx, workspace) -> Bound:
    B, N = (y.shape if y.dim() == 2 else (1, y.shape[0]))
    for t, n in ((y, "y"), (idx, "idx"), (workspace, "workspace")):
        _ptr(t, None, n)
    nbytes = workspace.numel() * workspace.element_size()
    return Bound("qdg_argmax", y, B, N, idx, workspace, nbytes, _stream())


def bind_sk_combine(partials, y) -> Bound:
    S, N = partials.shape[0], partials.shape[-1]
    B = partials.numel() // (S * N)
    _ptr(partials, None, "partials")
    _ptr(y, None, "y")
    return Bound("qdg_sk_combine", partials, S, B, N, y, _stream())
