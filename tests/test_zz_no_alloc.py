"""qdg_gemv_q8_argmax_noalloc (the LM-head GEMV + arg-max with the keys in the
library's own per-GPU array) against qdg_gemv_q8_argmax with a caller's
workspace, through the C ABI: the logits bit for bit and the index, in every
mode, on two calls in a row -- the second with a smaller input, so keys left
from the first call would show if the second read any it did not write -- and
the size limit, refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_decode_gemv_02_amd as q
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
P = ctypes.c_void_p


def _ptr(t):
    return None if t is None else P(t.data_ptr())


def _case(N, K, seed, a, b):
    wq, ws = workloads.weights(N, K, seed, seed + 1)
    x = workloads.activation(K, seed + 2)
    workloads.plant_tie(wq, ws, x, a, b)
    return (torch.from_numpy(wq).to(DEV), torch.from_numpy(ws.view(np.int16)).to(DEV),
            torch.from_numpy(x[None, :]).to(DEV))


def _words(mode, x):
    K = x.shape[1]
    xq = torch.empty((1, K), dtype=torch.int8, device=DEV)
    xl = torch.empty((1, K), dtype=torch.int8, device=DEV) if mode == 2 else None
    xs = torch.empty((1, K // 32), dtype=torch.float32, device=DEV)
    q.quantize_act(mode, x, xq, xl, xs)
    return xq, xl, xs


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_noalloc_matches_workspace_call(mode):
    lib = q.raw()
    stream = P(torch.cuda.current_stream().cuda_stream)
    # (N, K, tie rows): a large call, then a smaller one whose keys are a prefix of the first's
    for N, K, a, b in ((40000, 5120, 39001, 39980), (1000, 512, 17, 999)):
        print(f"[case] noalloc mode={mode} N={N} K={K} ties=({a},{b})", flush=True)
        wq, ws, x = _case(N, K, 500 + N + K + mode, a, b)
        xq = xl = xs = None
        if mode != 0:
            xq, xl, xs = _words(mode, x)
        xd = x if mode == 0 else None
        y_ref = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        i_ref = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        wsp = q.gemv_argmax_workspace(N)
        rc = lib.qdg_gemv_q8_argmax(mode, _ptr(wq), _ptr(ws), N, K, _ptr(xd), _ptr(xq), _ptr(xl), _ptr(xs),
                                    _ptr(y_ref), _ptr(i_ref), _ptr(wsp), wsp.numel() * 8, stream)
        assert rc == 0
        y = torch.full((1, N), float("nan"), dtype=torch.float32, device=DEV)
        idx = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        rc = lib.qdg_gemv_q8_argmax_noalloc(mode, _ptr(wq), _ptr(ws), N, K, _ptr(xd), _ptr(xq), _ptr(xl), _ptr(xs),
                                            _ptr(y), _ptr(idx), stream)
        assert rc == 0
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
        assert int(idx.item()) == int(i_ref.item()) == a


def test_noalloc_size_limit():
    lib = q.raw()
    dummy = torch.zeros(64, dtype=torch.int64, device=DEV)
    p = _ptr(dummy)
    # 2,097,152 rows is the largest N the 1 MiB array serves; one more tile is refused up front
    assert lib.qdg_gemv_q8_argmax_noalloc(1, p, p, 2097152 + 16, 32, None, p, None, p, p, p, None) == -5
    assert lib.qdg_gemv_q8_argmax_noalloc(1, p, p, 0, 32, None, p, None, p, p, p, None) == -2
    assert lib.qdg_gemv_q8_argmax_noalloc(1, None, p, 64, 32, None, p, None, p, p, p, None) == -1
