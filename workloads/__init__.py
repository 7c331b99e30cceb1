"""Seeded synthetic inputs for the Q8_0 decode GEMV workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no quantizer, no dot, no sum).  Both the CPU oracle's tests
and the GPU path's tests/bench take their inputs from here, so the two sides see
byte-identical operands.

Recipe (all draws from ``numpy.random.Generator(PCG64(seed))``):

* ``seed = 1000*config + 10*shape_index + role``; roles: 0 weights, 1 weight
  scales, 2 activation, 3 outlier positions, 4 tie rows.  Row ``t`` of a batched
  activation uses role 2 with ``seed + 100*t``.
* weights ``wq``: int8 uniform on [-127, 127] inclusive, row-major ``[N][K]``.
* weight scales ``ws``: uniform on [1e-3, 1e-2) in float64, rounded once to
  IEEE binary16 (round-to-nearest-even); the binary16 value is the truth and is
  handed over as its 16-bit pattern, ``[N][K/32]``.
* activation ``x``: float32 standard normal.  Where a workload asks for
  outliers, ``round(0.01*K)`` distinct positions are drawn and multiplied by 20
  in float32.
* planted ties (LM head): row ``a`` gets ``wq = 127*sign(x)`` (``+127`` where
  ``x == 0``) with every scale set to binary16(1e-2), and row ``b`` becomes a
  byte copy of row ``a``; the first of the two equal maxima is row ``min(a, b)``.

The shapes are those of the Q8_0 workloads of the pages (decode projections of
an 8B-class model, narrow 5120-row projections, a 151936-row LM head, and a
16-row batched decode against a 25600x5120 gate+up weight).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

QK = 32  # values per Q8_0 block


@dataclass(frozen=True)
class Shape:
    name: str
    K: int
    N: int
    B: int = 1
    outliers: bool = False


# The workload sets, each a seed base (it enters every seed, so the inputs stay
# fixed) and its shapes (the position in the list is the shape_index of the seed).
TINY = 0        # 256x512, one tile's worth: the case the oracle finishes in a blink
DECODE_8B = 1   # the projections of an 8B-class decoder layer
NARROW = 2      # o-proj 5120x8192 and down-proj 5120x25600, batch 1
LM_HEAD = 3     # 151936x5120 with an arg-max
BATCHED = 4     # the 25600x5120 gate+up matrix with 16 activation rows

CONFIGS: dict[int, list[Shape]] = {
    TINY: [Shape("tiny", K=512, N=256)],
    DECODE_8B: [
        Shape("qkv", K=4096, N=6144, outliers=True),
        Shape("gate_up", K=4096, N=24576, outliers=True),
        Shape("down", K=12288, N=4096, outliers=True),
    ],
    NARROW: [
        Shape("o_proj", K=8192, N=5120, outliers=True),
        Shape("down_proj", K=25600, N=5120, outliers=True),
    ],
    LM_HEAD: [Shape("lm_head", K=5120, N=151936)],
    BATCHED: [Shape("batched_gate_up", K=5120, N=25600, B=16)],
}


def seed_of(config: int, shape_index: int, role: int) -> int:
    return 1000 * config + 10 * shape_index + role


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def weights(N: int, K: int, seed_w: int, seed_s: int) -> tuple[np.ndarray, np.ndarray]:
    """``wq`` int8 ``[N][K]`` uniform on [-127, 127]; ``ws`` binary16 bits ``[N][K/32]``."""
    if K % QK:
        raise ValueError("K must be a multiple of 32")
    wq = _rng(seed_w).integers(-127, 128, size=(N, K), dtype=np.int8)
    ws = scales(N, K // QK, seed_s)
    return wq, ws


def scales(N: int, nb: int, seed: int) -> np.ndarray:
    s = _rng(seed).uniform(1e-3, 1e-2, size=(N, nb))
    return s.astype(np.float16).view(np.uint16)


def activation(K: int, seed: int, outliers: bool = False, seed_out: int | None = None) -> np.ndarray:
    x = _rng(seed).standard_normal(K, dtype=np.float32)
    if outliers:
        n_out = int(round(0.01 * K))
        pos = _rng(seed_out if seed_out is not None else seed + 1).choice(K, size=n_out, replace=False)
        x[pos] = x[pos] * np.float32(20.0)
    return x


def batch_activation(B: int, K: int, seed: int, outliers: bool = False, seed_out: int | None = None) -> np.ndarray:
    """``B`` independent rows; row ``t`` seeded with ``seed + 100*t``."""
    rows = []
    for t in range(B):
        so = None if seed_out is None else seed_out + 100 * t
        rows.append(activation(K, seed + 100 * t, outliers, so))
    return np.stack(rows).astype(np.float32)


def make(config: int, shape_index: int) -> dict:
    """All operands of one workload shape: ``wq``, ``ws``, ``x`` (``[B][K]``) and the shape."""
    sh = CONFIGS[config][shape_index]
    wq, ws = weights(sh.N, sh.K, seed_of(config, shape_index, 0), seed_of(config, shape_index, 1))
    x = batch_activation(sh.B, sh.K, seed_of(config, shape_index, 2), sh.outliers,
                         seed_of(config, shape_index, 3) if sh.outliers else None)
    return {"shape": sh, "wq": wq, "ws": ws, "x": x}


def tie_rows(N: int, seed: int) -> tuple[int, int]:
    """A seeded pair ``a < b`` of distinct rows."""
    a, b = sorted(int(v) for v in _rng(seed).choice(N, size=2, replace=False))
    return a, b


FP16_1EM2 = int(np.array(1e-2, dtype=np.float16).view(np.uint16))


def plant_tie(wq: np.ndarray, ws: np.ndarray, x: np.ndarray, a: int, b: int) -> None:
    """In place: row ``a`` dominates every random row and row ``b`` is its exact copy."""
    sgn = np.where(x < 0, -127, 127).astype(np.int8)
    wq[a, :] = sgn
    ws[a, :] = FP16_1EM2
    wq[b, :] = wq[a, :]
    ws[b, :] = ws[a, :]


def random_logits(N: int, seed: int) -> np.ndarray:
    return _rng(seed).standard_normal(N, dtype=np.float32)


def norm_weight(K: int, seed: int) -> np.ndarray:
    """An RMSNorm weight ``[K]``: 1 + 0.25 * N(0, 1), so a few entries are small or negative."""
    return (1.0 + 0.25 * _rng(seed).standard_normal(K)).astype(np.float32)


def glu_inputs(B: int, K: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Gate and up projections ``[B][K]`` of one activation: the gate N(0, 2^2) with 1%
    of its entries 8x larger (silu's linear and vanishing tails), the up N(0, 1)."""
    rng = _rng(seed)
    g = (2.0 * rng.standard_normal((B, K))).astype(np.float32)
    tail = rng.random((B, K)) < 0.01
    g[tail] *= np.float32(8.0)
    u = rng.standard_normal((B, K)).astype(np.float32)
    return g, u


# Other GGUF block formats: GGUF type number -> (values per block, bytes per block,
# byte offsets of the binary16 scale fields inside a block).  Only where the
# scale fields sit, so that random bytes make a valid matrix: the levels, sub-scales
# and masks of every format are valid for any byte values.  MXFP4's one-byte E8M0
# scale sits at offset 0.
BLOCK_FORMATS = {
    2: (32, 18, (0,)), 3: (32, 20, (0, 2)), 6: (32, 22, (0,)), 7: (32, 24, (0, 2)),
    20: (32, 18, (0,)), 39: (32, 17, ()),
    10: (256, 84, (80, 82)), 11: (256, 110, (108,)), 12: (256, 144, (0, 2)), 13: (256, 176, (0, 2)),
    14: (256, 210, (208,)), 23: (256, 136, (0,)),
}


def block_matrix(fmt: int, N: int, K: int, seed: int) -> np.ndarray:
    """``N`` rows of ``K`` values in GGUF block format ``fmt`` as uint8 ``[N][row bytes]``:
    uniform random bytes, with every binary16 scale field drawn uniform on
    [1e-3, 1e-2) (rounded once to binary16) and MXFP4's E8M0 scales uniform on
    [118, 134) (2^-10 .. 2^5)."""
    vals, nbytes, fields = BLOCK_FORMATS[fmt]
    if K % vals:
        raise ValueError("K must be a whole number of the format's blocks")
    nblk = K // vals
    rng = _rng(seed)
    b = rng.integers(0, 256, size=(N, nblk, nbytes), dtype=np.uint8)
    for off in fields:
        h = rng.uniform(1e-3, 1e-2, size=(N, nblk)).astype(np.float16).view(np.uint16)
        b[:, :, off] = (h & 0xFF).astype(np.uint8)
        b[:, :, off + 1] = (h >> 8).astype(np.uint8)
    if fmt == 39:
        b[:, :, 0] = rng.integers(118, 134, size=(N, nblk), dtype=np.uint8)
    return b.reshape(N, nblk * nbytes)
