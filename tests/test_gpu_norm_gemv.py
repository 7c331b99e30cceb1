"""GPU parity of qdg_gemv_q8_rmsnorm: the split-K projection with the residual
add, the RMSNorm and the next projection's quantizer in its last workgroup.

Bar:
* bit-exact against the two calls it fuses, qdg_gemv_q8_sk (same splits) then
  qdg_rmsnorm_quantize over its output: y, s, yn and the words;
* against the oracle, orc_gemv_split + orc_combine (the split GEMV) then
  orc_rmsnorm then orc_quantize: y and s bit-exact, yn within one unit in the
  last place and equal almost everywhere (the producer's bar: both sides round
  one binary64 evaluation), the words bit-exact against the oracle's quantizer
  on the kernel's own yn;
* the workspace is zero again after every call (the next call, a smaller row on
  the same workspace, relies on it).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_gemv_02_amd as q
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[case] {msg}", flush=True)


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ulp_diff(a, b):
    def key(v):
        i = v.astype(np.float32).view(np.int32).astype(np.int64)
        return np.where(i < 0, -(i & 0x7fffffff), i)
    return np.abs(key(a) - key(b))


def words(mode, n):
    if mode == 0:
        return None, None, None
    hq = torch.empty(n, dtype=torch.int8, device=DEV)
    hl = torch.empty(n, dtype=torch.int8, device=DEV) if mode == 2 else None
    hs = torch.empty(n // 32, dtype=torch.float32, device=DEV)
    return hq, hl, hs


def act_words(mode, x):
    K = x.shape[-1]
    xq = torch.empty((1, K), dtype=torch.int8, device=DEV)
    xl = torch.empty((1, K), dtype=torch.int8, device=DEV) if mode == 2 else None
    xs = torch.empty((1, K // 32), dtype=torch.float32, device=DEV)
    q.quantize_act(mode, dev(x.reshape(1, K)), xq, xl, xs)
    return xq, xl, xs


def same(a, b):
    if a is None or b is None:
        return a is None and b is None
    return torch.equal(a.view(torch.int8) if a.dtype == torch.int8 else a.view(torch.int32),
                       b.view(torch.int8) if b.dtype == torch.int8 else b.view(torch.int32))


def inputs(N, K, seed):
    wq, ws = workloads.weights(N, K, seed, seed + 1)
    x = workloads.activation(K, seed + 2, outliers=True, seed_out=seed + 3)
    r = workloads.activation(N, seed + 4)
    w = workloads.norm_weight(N, seed + 5)
    return wq, ws, x, r, w


def two_calls(mode, dwq, dws, xq, xl, xs, S, N, dr, dw, eps, qmode, with_s):
    """qdg_gemv_q8_sk then qdg_rmsnorm_quantize: the reference the fused launch must equal."""
    y = torch.empty((1, N), dtype=torch.float32, device=DEV)
    q.gemv_q8_sk(mode, dwq, dws, y, xq, xl, xs, S, q.sk_workspace(N, S))
    s = torch.empty_like(y) if with_s else None
    yn = torch.empty_like(y)
    hq, hl, hs = words(qmode, N)
    q.rmsnorm_quantize(qmode, y, dw, dr, s, yn, *(t if t is None else t.view(1, -1) for t in (hq, hl, hs)), eps=eps)
    return y.view(-1), (s.view(-1) if with_s else None), yn.view(-1), hq, hl, hs


CASES = [  # (mode, qmode, N, K, splits): small rows, ragged tiles and K tails, the largest N, the two projections
    (1, 1, 32, 1024, 2),
    (2, 2, 96, 4128, 3),         # K tail of 32 values; register-copy staging
    (1, 2, 544, 2048, 4),        # 544 rows: a ragged last row tile of 12
    (2, 1, 4128, 1056, 2),       # a second, partial round of the norm's chunks
    (1, 0, 1024, 8192, 16),      # one row group (per-wave staging); Dequant words: yn only
    (2, 2, 2048, 8192, 8),       # two row groups
    (1, 1, 20224, 1024, 2),      # the largest N: five rounds of chunks, the row's 79 KiB in LDS
    (1, 1, 5120, 8192, 4),       # the attention output projection
    (2, 2, 5120, 8192, 4),
    (1, 1, 5120, 25600, 5),      # the MLP down projection
    (2, 2, 5120, 25600, 5),
]


@pytest.mark.parametrize("mode,qmode,N,K,S", CASES)
def test_gemv_rmsnorm_matches_the_two_calls_and_the_oracle(mode, qmode, N, K, S):
    announce(f"gemv_q8_rmsnorm mode={mode} qmode={qmode} N={N} K={K} S={S}")
    assert N <= q.gemv_rmsnorm_max_n()
    assert q.sk_workgroup_shape(mode, K, S) is not None
    eps = 1e-6
    wq, ws, x, r, w = inputs(N, K, 4000 + N + K)
    dwq, dws, dr, dw = dev(wq), dev(ws.view(np.int16)), dev(r), dev(w)
    xq, xl, xs = act_words(mode, x)
    wsp = q.gemv_rmsnorm_workspace(N)
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    s = torch.empty(N, dtype=torch.float32, device=DEV)
    yn = torch.empty(N, dtype=torch.float32, device=DEV)
    hq, hl, hs = words(qmode, N)
    q.gemv_q8_rmsnorm(mode, dwq, dws, xq, xl, xs, S, wsp, y=y, r=dr, s=s, w=dw, eps=eps, qmode=qmode, yn=yn,
                      hq=hq, hl=hl, hs=hs)
    assert int(torch.count_nonzero(wsp)) == 0, "workspace not left zero"

    # the two calls it fuses: every output bit-identical
    ry, rs, ryn, rq, rl, rsc = two_calls(mode, dwq, dws, xq, xl, xs, S, N, dr, dw, eps, qmode, True)
    assert same(y, ry), "y differs from qdg_gemv_q8_sk"
    assert same(s, rs), "s differs from qdg_rmsnorm_quantize"
    assert same(yn, ryn), "yn differs from qdg_rmsnorm_quantize"
    assert same(hq, rq) and same(hl, rl) and same(hs, rsc), "words differ from qdg_rmsnorm_quantize"

    # the oracle: split GEMV + ascending combine, then the norm, then the quantizer
    oq, ol, os_ = oracle.quantize(mode, x.reshape(1, K))
    oy = oracle.combine(oracle.gemv_split(mode, wq, ws, oq, ol, os_, S, nthreads=8)).reshape(-1)
    gy = host(y)
    assert np.array_equal(gy.view(np.uint32), oy.view(np.uint32)), "y differs from the oracle"
    o_s, o_yn = oracle.rmsnorm(oy.reshape(1, N), r.reshape(1, N), w, eps)
    assert np.array_equal(host(s).view(np.uint32), o_s.reshape(-1).view(np.uint32)), "s differs from the oracle"
    gyn = host(yn)
    d = ulp_diff(gyn, o_yn.reshape(-1))
    assert d.max() <= 1 and np.count_nonzero(d) <= max(2, N // 1000), f"yn: {int(d.max())} ulp, {np.count_nonzero(d)} off"
    if qmode:
        wq_, wl_, ws_ = oracle.quantize(qmode, gyn.reshape(1, N))
        assert np.array_equal(host(hq), wq_.reshape(-1)), "hq differs from the oracle's quantizer"
        assert np.array_equal(host(hs).view(np.uint32), ws_.reshape(-1).view(np.uint32)), "hs"
        if qmode == 2:
            assert np.array_equal(host(hl), wl_.reshape(-1)), "hl"


@pytest.mark.parametrize("mode", [1, 2])
def test_gemv_rmsnorm_optional_outputs_and_reuse(mode):
    """No y, no s, no weight, s over r in place; then a smaller row on the same workspace."""
    N, K, S = 3072, 4096, 4
    announce(f"gemv_q8_rmsnorm options mode={mode} N={N} K={K} S={S}")
    wq, ws, x, r, w = inputs(N, K, 9100 + mode)
    dwq, dws, dr = dev(wq), dev(ws.view(np.int16)), dev(r)
    xq, xl, xs = act_words(mode, x)
    wsp = q.gemv_rmsnorm_workspace(N)
    full = two_calls(mode, dwq, dws, xq, xl, xs, S, N, dr, None, 1e-5, mode, True)

    # neither y nor yn nor the weight: the words alone
    hq, hl, hs = words(mode, N)
    q.gemv_q8_rmsnorm(mode, dwq, dws, xq, xl, xs, S, wsp, r=dr, eps=1e-5, qmode=mode, hq=hq, hl=hl, hs=hs)
    assert same(hq, full[3]) and same(hl, full[4]) and same(hs, full[5])
    assert int(torch.count_nonzero(wsp)) == 0

    # s written over r (the residual stream updated in place)
    r2 = dr.clone()
    yn = torch.empty(N, dtype=torch.float32, device=DEV)
    q.gemv_q8_rmsnorm(mode, dwq, dws, xq, xl, xs, S, wsp, r=r2, s=r2, eps=1e-5, qmode=0, yn=yn)
    assert same(r2, full[1]) and same(yn, full[2])

    # no residual: the norm of y itself
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    hq2, hl2, hs2 = words(mode, N)
    q.gemv_q8_rmsnorm(mode, dwq, dws, xq, xl, xs, S, wsp, y=y, eps=1e-5, qmode=mode, yn=yn, hq=hq2, hl=hl2, hs=hs2)
    ref_yn = torch.empty((1, N), dtype=torch.float32, device=DEV)
    rq, rl, rs = words(mode, N)
    q.rmsnorm_quantize(mode, y.view(1, N), None, None, None, ref_yn, rq.view(1, -1),
                       None if rl is None else rl.view(1, -1), rs.view(1, -1), eps=1e-5)
    assert same(y, full[0]) and same(yn, ref_yn.view(-1)) and same(hq2, rq) and same(hs2, rs) and same(hl2, rl)

    # a smaller row on the same workspace, twice: the ticket and the slots were left zero
    n2, k2 = 1024, 2048
    wq2, ws2, x2, r3, w3 = inputs(n2, k2, 9200 + mode)
    d2, s2, dr3, dw3 = dev(wq2), dev(ws2.view(np.int16)), dev(r3), dev(w3)
    a2 = act_words(mode, x2)
    ref = two_calls(mode, d2, s2, *a2, S, n2, dr3, dw3, 1e-6, mode, True)
    for _ in range(2):
        y3 = torch.empty(n2, dtype=torch.float32, device=DEV)
        s3 = torch.empty(n2, dtype=torch.float32, device=DEV)
        yn3 = torch.empty(n2, dtype=torch.float32, device=DEV)
        hq3, hl3, hs3 = words(mode, n2)
        q.gemv_q8_rmsnorm(mode, d2, s2, *a2, S, wsp, y=y3, r=dr3, s=s3, w=dw3, eps=1e-6, qmode=mode, yn=yn3,
                          hq=hq3, hl=hl3, hs=hs3)
        assert same(y3, ref[0]) and same(s3, ref[1]) and same(yn3, ref[2])
        assert same(hq3, ref[3]) and same(hl3, ref[4]) and same(hs3, ref[5])
        assert int(torch.count_nonzero(wsp)) == 0


def test_gemv_rmsnorm_rejects_an_unsplit_launch():
    N, K = 64, 1024
    wq, ws, x, r, w = inputs(N, K, 9300)
    xq, xl, xs = act_words(1, x)
    hq, hl, hs = words(1, N)
    with pytest.raises(q.QdgError) as e:
        q.gemv_q8_rmsnorm(1, dev(wq), dev(ws.view(np.int16)), xq, xl, xs, 1, q.gemv_rmsnorm_workspace(N),
                          r=dev(r), eps=1e-6, qmode=1, hq=hq, hs=hs)
    assert e.value.status == -4
