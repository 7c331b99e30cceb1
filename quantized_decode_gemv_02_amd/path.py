"""The hot path as a sequence of library calls, with device buffers from PyTorch.

``Q8Matrix`` holds a Q8_0 weight on the GPU (int8 values ``[N][K]`` and binary16
scale bits ``[N][K/32]``, the split upload of the lane kernel library page).
``DecodeBuffers`` owns the activation words and outputs of one projection so
repeated steps allocate nothing.  Every arithmetic step runs in libqdg.so.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (DEQUANT, INT8ACT, TWOPASS, QK, argmax, argmax_workspace_bytes, gemv_q8, quantize_act,
               sk_combine)


@dataclass
class Q8Matrix:
    wq: torch.Tensor  # int8 [N][K]
    ws: torch.Tensor  # int16 (binary16 bits) [N][K/32]

    @property
    def N(self) -> int:
        return self.wq.shape[0]

    @property
    def K(self) -> int:
        return self.wq.shape[1]

    @staticmethod
    def from_numpy(wq, ws, device="cuda") -> "Q8Matrix":
        return Q8Matrix(torch.from_numpy(wq).to(device), torch.from_numpy(ws.view("int16")).to(device))


class DecodeBuffers:
    """Buffers of one projection: ``quantize_act`` -> ``gemv_q8`` [-> ``sk_combine``] [-> ``argmax``]."""

    def __init__(self, mode: int, N: int, K: int, B: int = 1, splits: int = 1, with_argmax: bool = False,
                 device="cuda"):
        self.mode, self.N, self.K, self.B, self.splits = mode, N, K, B, splits
        dev = torch.device(device)
        self.xq = torch.empty((B, K), dtype=torch.int8, device=dev) if mode != DEQUANT else None
        self.xl = torch.empty((B, K), dtype=torch.int8, device=dev) if mode == TWOPASS else None
        self.xs = torch.empty((B, K // QK), dtype=torch.float32, device=dev) if mode != DEQUANT else None
        self.y = torch.empty((B, N), dtype=torch.float32, device=dev)
        self.part = torch.empty((splits, B, N), dtype=torch.float32, device=dev) if splits > 1 else None
        self.idx = torch.empty((B,), dtype=torch.int32, device=dev) if with_argmax else None
        nbytes = argmax_workspace_bytes(B, N) if with_argmax else 0
        self.ws_argmax = torch.empty((max(nbytes, 8) + 7) // 8, dtype=torch.int64, device=dev) if with_argmax else None

    def quantize(self, x: torch.Tensor) -> None:
        if self.mode != DEQUANT:
            quantize_act(self.mode, x, self.xq, self.xl, self.xs)

    def gemv(self, w: Q8Matrix, x: torch.Tensor) -> None:
        out = self.y if self.splits == 1 else self.part
        if self.mode == DEQUANT:
            gemv_q8(DEQUANT, w.wq, w.ws, out, x=x)
        else:
            gemv_q8(self.mode, w.wq, w.ws, out, xq=self.xq, xl=self.xl, xs=self.xs, splits=self.splits)

    def combine(self) -> None:
        if self.splits > 1:
            sk_combine(self.part, self.y)

    def run(self, w: Q8Matrix, x: torch.Tensor) -> torch.Tensor:
        """One pass: quantize (quantized modes), GEMV, combine (splits > 1), arg-max (if asked)."""
        self.quantize(x)
        self.gemv(w, x)
        self.combine()
        if self.idx is not None:
            argmax(self.y, self.idx, self.ws_argmax)
        return self.y


__all__ = ["Q8Matrix", "DecodeBuffers", "DEQUANT", "INT8ACT", "TWOPASS"]
