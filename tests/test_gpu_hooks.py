"""The library's error path and its measurement hook, on the GPU.

QDG_EHIP: with the reject_launch tuning knob set, every launch asks the HIP
runtime for a 2048-thread workgroup, which it refuses before anything is
enqueued; the call must return QDG_EHIP with that hipError_t, leave the output
untouched, leave no pending error for the next HIP call, and the next call
without the knob must run normally.  Nothing reaches the GPU in the refused
calls.

qdg_time_next_launch: the events it binds take the timed kernel's own dispatch
timestamps, so the duration they give is positive, no longer than an event pair
recorded around the same call, and the binding covers one launch only.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_gemv_02_amd as q
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
HIP_ERROR_INVALID_CONFIGURATION, HIP_ERROR_INVALID_VALUE = 9, 1


def test_refused_launch_returns_qdg_ehip(tune):
    print("[case] reject_launch -> QDG_EHIP on quantize, gemv_q8_sk and argmax", flush=True)
    K, N = 1024, 64
    x = torch.from_numpy(workloads.activation(K, 31)[None, :]).to(DEV)
    xq = torch.full((1, K), 7, dtype=torch.int8, device=DEV)
    xs = torch.full((1, K // 32), 3.0, dtype=torch.float32, device=DEV)
    wq, ws = workloads.weights(N, K, 32, 33)
    wqd, wsd = torch.from_numpy(wq).to(DEV), torch.from_numpy(ws.view(np.int16)).to(DEV)
    y = torch.full((1, N), 5.0, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    tune(reject_launch=1)
    calls = [lambda: q.quantize_act(q.INT8ACT, x, xq, None, xs),
             lambda: q.gemv_q8_sk(q.INT8ACT, wqd, wsd, y, xq, None, xs, 4, q.sk_workspace(N, 4)),
             lambda: q.gemv_q8(q.INT8ACT, wqd, wsd, y, xq=xq, xs=xs)]
    for c in calls:
        with pytest.raises(q.QdgError) as err:
            c()
        assert err.value.status == -6
        assert q.raw().qdg_last_hip_error() in (HIP_ERROR_INVALID_CONFIGURATION, HIP_ERROR_INVALID_VALUE)
    # nothing ran, and no error is left pending for torch's next launch
    torch.cuda.synchronize()
    assert (xq == 7).all() and (xs == 3.0).all() and (y == 5.0).all()
    z = torch.zeros(4, device=DEV) + 1
    torch.cuda.synchronize()
    assert z.sum().item() == 4.0
    tune(reject_launch=-1)
    q.quantize_act(q.INT8ACT, x, xq, None, xs)
    oq, _, os_ = oracle.quantize(1, x.cpu().numpy())
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), oq) and np.array_equal(xs.cpu().numpy(), os_)


def test_timed_launch_gives_the_kernels_own_duration():
    print("[case] qdg_time_next_launch on gemv_q8_sk 5120x25600", flush=True)
    N, K, S = 5120, 25600, 5
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=DEV)
    ws = torch.full((N, K // 32), 0x1c00, dtype=torch.int16, device=DEV)  # binary16 0.00390625
    xq = torch.randint(-127, 128, (1, K), dtype=torch.int8, device=DEV)
    xs = torch.ones((1, K // 32), dtype=torch.float32, device=DEV)
    y = torch.empty((1, N), dtype=torch.float32, device=DEV)
    wsp = q.sk_workspace(N, S)
    call = q.bind_gemv_q8_sk(q.INT8ACT, wq, ws, y, xq, None, xs, S, wsp)
    call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    durations, outer = [], []
    for _ in range(5):
        ev[2].record()
        q.time_next_launch(ev[0], ev[1])
        call()
        ev[3].record()
        call()  # not timed: the binding covered one launch
        torch.cuda.synchronize()
        durations.append(ev[0].elapsed_time(ev[1]))
        outer.append(ev[2].elapsed_time(ev[3]))
    for d, o in zip(durations, outer):
        assert 0.005 < d <= o + 1e-3, (d, o)  # ms: more than 5 us, no more than the enclosing pair
    same = q.raw().qdg_time_next_launch(None, None)
    assert same == 0
