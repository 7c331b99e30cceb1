"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments with the documented status before it touches
the HIP runtime.  The host-only chunk rule matches the oracle and the hand-derived
boundaries."""
import ctypes
import json
import os
import re

import pytest

import oracle
import quantized_decode_gemv_02_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qdg.h")

OK, EINVAL, ESHAPE, EALIGN, EMODE, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5, -6
A = 0x10000  # a 64 KiB-aligned fake device address: every check passes on alignment
lib = q.raw()
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qdg_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) == 43
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(q.EXPORTS)


def test_abi_version_and_status_strings():
    assert q.abi_version() == 1
    for s in (OK, EINVAL, ESHAPE, EALIGN, EMODE, EWORKSPACE, EHIP, 12345):
        assert isinstance(q.status_str(s), str) and q.status_str(s)


def test_split_bounds_match_oracle_and_golden(golden_dir):
    for c in json.load(open(os.path.join(golden_dir, "split_bounds.json")))["cases"]:
        assert q.split_bounds(c["K"], c["S"]) == c["first"]
    for K in (32, 480, 512, 544, 1600, 4096, 5120, 8192, 12288, 25600, 25632):
        for S in (1, 2, 3, 4, 5, 7, 8, 16, 64):
            assert q.split_bounds(K, S) == list(oracle.split_bounds(K, S)), (K, S)


def gemv(mode=1, wq=A, ws=A, N=64, K=512, x=None, xq=A, xl=None, xs=A, B=1, S=1, out=A):
    return lib.qdg_gemv_q8(mode, P(wq), P(ws), N, K, P(x), P(xq), P(xl), P(xs), B, S, P(out), None)


def test_gemv_validation():
    assert gemv(mode=3) == EINVAL
    assert gemv(mode=-1) == EINVAL
    assert gemv(wq=None) == EINVAL
    assert gemv(out=None) == EINVAL
    assert gemv(mode=0, x=None, xq=None, xs=None) == EINVAL      # Dequant needs x
    assert gemv(mode=0, x=A) == EINVAL                           # ... and no quantized words
    assert gemv(mode=1, x=A) == EINVAL
    assert gemv(mode=2) == EINVAL                                # TwoPass needs xl
    assert gemv(mode=1, xl=A) == EINVAL
    assert gemv(K=33) == ESHAPE
    assert gemv(K=0) == ESHAPE
    assert gemv(K=16) == ESHAPE
    assert gemv(N=0) == ESHAPE
    assert gemv(B=0) == ESHAPE
    assert gemv(B=65) == ESHAPE
    assert gemv(B=17, K=544) == EMODE                         # prefill chunks need K % 256 == 0
    assert gemv(B=17, K=512, ws=A + 2) == EMODE               # ... and 16-byte weight-scale words
    assert gemv(S=0) == ESHAPE
    assert gemv(S=65) == ESHAPE
    assert gemv(wq=A + 8) == EALIGN
    assert gemv(xq=A + 4) == EALIGN
    assert gemv(ws=A + 1) == EALIGN
    assert gemv(xs=A + 2) == EALIGN
    assert gemv(out=A + 2) == EALIGN
    assert gemv(mode=2, xl=A + 8) == EALIGN
    assert gemv(mode=0, x=A, xq=None, xs=None, B=2) == EMODE
    assert gemv(mode=0, x=A, xq=None, xs=None, S=2) == EMODE


def test_quantize_validation():
    f = lib.qdg_quantize_act
    assert f(0, P(A), 1, 512, P(A), None, P(A), None) == EINVAL    # Dequant has no quantizer
    assert f(1, None, 1, 512, P(A), None, P(A), None) == EINVAL
    assert f(2, P(A), 1, 512, P(A), None, P(A), None) == EINVAL    # TwoPass needs xl
    assert f(1, P(A), 1, 512, P(A), P(A), P(A), None) == EINVAL    # Int8Act takes no xl
    assert f(1, P(A), 1, 500, P(A), None, P(A), None) == ESHAPE
    assert f(1, P(A), 0, 512, P(A), None, P(A), None) == ESHAPE
    assert f(1, P(A + 4), 1, 512, P(A), None, P(A), None) == EALIGN
    assert f(1, P(A), 1, 512, P(A), None, P(A + 1), None) == EALIGN


def test_combine_argmax_blockdots_validation():
    assert lib.qdg_sk_combine(None, 2, 1, 8, P(A), None) == EINVAL
    assert lib.qdg_sk_combine(P(A), 0, 1, 8, P(A), None) == ESHAPE
    assert lib.qdg_sk_combine(P(A), 65, 1, 8, P(A), None) == ESHAPE
    assert lib.qdg_sk_combine(P(A + 2), 2, 1, 8, P(A), None) == EALIGN
    need = q.argmax_workspace_bytes(1, 151936)
    assert need >= 8 and need % 8 == 0
    assert q.argmax_workspace_bytes(0, 10) == 0
    assert lib.qdg_argmax(P(A), 1, 151936, P(A), P(A), need - 8, None) == EWORKSPACE
    assert lib.qdg_argmax(P(A), 1, 0, P(A), P(A), need, None) == ESHAPE
    assert lib.qdg_argmax(P(A), 1, 100, P(A), None, need, None) == EINVAL
    assert lib.qdg_argmax(P(A), 1, 100, P(A), P(A + 4), need, None) == EALIGN
    bd = lib.qdg_block_dots
    assert bd(0, P(A), 4, 64, P(A), None, 1, P(A), None, None) == EINVAL
    assert bd(2, P(A), 4, 64, P(A), None, 1, P(A), P(A), None) == EINVAL
    assert bd(1, P(A), 4, 64, P(A), None, 1, P(A), P(A), None) == EINVAL
    assert bd(1, P(A), 4, 60, P(A), None, 1, P(A), None, None) == ESHAPE
    assert bd(1, P(A), 4, 64, P(A), None, 65, P(A), None, None) == ESHAPE


def test_fused_validation():
    f = lib.qdg_gemv_q8_fused
    need = q.gemv_sk_workspace_bytes(1, 64, 4)

    def call(mode=1, wq=A, ws=A, N=64, K=512, x=A, S=4, y=A, wsp=A, nbytes=None):
        return f(mode, P(wq), P(ws), N, K, P(x), S, P(y), P(wsp), need if nbytes is None else nbytes, None)

    assert call(mode=3) == EINVAL
    assert call(x=None) == EINVAL
    assert call(y=None) == EINVAL
    assert call(wsp=None) == EINVAL                  # S > 1 needs the workspace
    assert call(K=500) == ESHAPE
    assert call(S=0) == ESHAPE
    assert call(S=65) == ESHAPE
    assert call(mode=0, S=2, wsp=None) == EINVAL     # Dequant splits K too, with the workspace
    assert call(x=A + 4) == EALIGN
    assert call(wq=A + 8) == EALIGN
    assert call(wsp=A + 8) == EALIGN
    assert call(nbytes=need - 4) == EWORKSPACE


def test_sk_placement_query():
    def f(mode, K, S):
        return lib.qdg_gemv_sk_combines_in_workgroup(mode, K, S, None)
    assert f(0, 512, 4) == EINVAL
    assert f(1, 500, 4) == ESHAPE
    assert f(1, 512, 0) == ESHAPE
    assert f(1, 25600, 16) == 1 and f(2, 25600, 16) == 1
    assert f(1, 25600, 4) == 1 and f(2, 25600, 4) == 1
    assert f(1, 8192, 1) == 0                                  # no split, nothing to combine
    assert f(1, 8192, 3) == 1 and f(2, 12288, 5) == 1
    assert f(1, 8192, 17) == 0 and f(1, 8192, 64) == 0       # more chunk waves than a workgroup holds
    assert f(1, 512, 16) == 0                                  # one non-empty chunk
    assert f(2, 65536, 16) == 0                                # the staged row exceeds the LDS budget
    # the LDS budget's edges: K/32 x (68 + 8 x row groups) bytes of at most 79 KiB under TwoPass
    assert f(2, 28128, 5) == 1 and f(2, 28160, 5) == 0         # three row groups
    assert f(2, 30816, 8) == 1 and f(2, 30848, 8) == 0         # two row groups
    assert f(2, 34048, 16) == 1 and f(2, 34080, 16) == 0       # one row group
    assert f(1, 28160, 5) == 1                                 # Int8Act stages half the words
    # launch shape: one wave per non-empty chunk, row groups of four rows up to 16 waves
    assert q.sk_workgroup_shape(2, 25600, 16) == (4, 13)       # 13 chunks of 4 superblocks, 3 empty
    assert q.sk_workgroup_shape(2, 25600, 5) == (12, 15)       # 5 chunks, three row groups
    assert q.sk_workgroup_shape(1, 8192, 5) == (12, 12)        # 4 chunks of 4 superblocks, 1 empty
    assert q.sk_workgroup_shape(1, 25600, 8) == (8, 16)        # 8 chunks: two row groups fit
    assert q.sk_workgroup_shape(1, 25632, 16) == (4, 14)       # the tail makes chunk 15 non-empty
    assert q.sk_workgroup_shape(1, 8192, 1) is None


def test_gemv_argmax_validation():
    f = lib.qdg_gemv_q8_argmax
    need = q.gemv_argmax_workspace_bytes(151936)
    assert need == 8 * (151936 // 16)
    assert q.gemv_argmax_workspace_bytes(0) == 0

    def call(mode=1, wq=A, ws=A, N=64, K=512, x=None, xq=A, xl=None, xs=A, y=A, idx=A, wsp=A, nbytes=8 * 4):
        return f(mode, P(wq), P(ws), N, K, P(x), P(xq), P(xl), P(xs), P(y), P(idx), P(wsp), nbytes, None)

    assert call(mode=3) == EINVAL
    assert call(idx=None) == EINVAL
    assert call(wsp=None) == EINVAL
    assert call(mode=0) == EINVAL                     # Dequant reads x, not words
    assert call(mode=2) == EINVAL                     # TwoPass needs xl
    assert call(K=500) == ESHAPE
    assert call(idx=A + 2) == EALIGN
    assert call(wsp=A + 4) == EALIGN
    assert call(nbytes=8 * 3) == EWORKSPACE


def test_rmsnorm_quantize_validation():
    f = lib.qdg_rmsnorm_quantize
    kmax = q.rmsnorm_max_k()
    assert kmax >= 16384 and kmax % 32 == 0

    def call(mode=1, x=A, r=A, s=A, w=A, eps=1e-6, B=1, K=512, y=None, xq=A, xl=None, xs=A):
        return f(mode, P(x), P(r), P(s), P(w), eps, B, K, P(y), P(xq), P(xl), P(xs), None)

    assert call(mode=3) == EINVAL
    assert call(x=None) == EINVAL
    assert call(r=None) == EINVAL                         # s needs r
    assert call(mode=0) == EINVAL                         # Dequant writes y only
    assert call(mode=0, y=A, xq=None, xs=None, xl=A) == EINVAL
    assert call(mode=1, xl=A) == EINVAL
    assert call(mode=2) == EINVAL                         # TwoPass needs xl
    assert call(xs=None) == EINVAL
    assert call(eps=-1.0) == EINVAL
    assert call(eps=float("nan")) == EINVAL
    assert call(eps=float("inf")) == EINVAL
    assert call(K=500) == ESHAPE
    assert call(K=0) == ESHAPE
    assert call(K=kmax + 32) == ESHAPE
    assert call(B=0) == ESHAPE
    assert call(x=A + 4) == EALIGN
    assert call(w=A + 8) == EALIGN
    assert call(s=A + 4) == EALIGN
    assert call(xq=A + 4) == EALIGN
    assert call(xs=A + 2) == EALIGN
    assert call(mode=0, y=A + 4, xq=None, xs=None) == EALIGN


def test_gemv_rmsnorm_validation():
    f = lib.qdg_gemv_q8_rmsnorm
    nmax = q.gemv_rmsnorm_max_n()
    assert nmax % 32 == 0 and 16384 <= nmax <= q.rmsnorm_max_k()
    assert q.gemv_rmsnorm_workspace_bytes(5120) == 5120 * 4
    assert q.gemv_rmsnorm_workspace_bytes(96) == 512                # one word a row, in 256-byte lines
    assert q.gemv_rmsnorm_workspace_bytes(0) == 0
    assert q.gemv_rmsnorm_workspace_bytes(100) == 0                 # not whole 32-value blocks
    assert q.gemv_rmsnorm_workspace_bytes(nmax + 32) == 0
    need = q.gemv_rmsnorm_workspace_bytes(512)

    def call(mode=1, wq=A, ws=A, N=512, K=8192, xq=A, xl=None, xs=A, S=4, y=A, r=A, s=A, w=A, eps=1e-6, qm=1,
             yn=None, hq=A, hl=None, hs=A, wsp=A, nbytes=None):
        return f(mode, P(wq), P(ws), N, K, P(xq), P(xl), P(xs), S, P(y), P(r), P(s), P(w), eps, qm, P(yn), P(hq),
                 P(hl), P(hs), P(wsp), need if nbytes is None else nbytes, None)

    assert call(mode=0) == EMODE                          # the GEMV side reads words
    assert call(mode=3) == EINVAL
    assert call(mode=2) == EINVAL                         # TwoPass needs xl
    assert call(xl=A) == EINVAL
    assert call(wq=None) == EINVAL
    assert call(wsp=None) == EINVAL
    assert call(qm=3) == EINVAL
    assert call(qm=2) == EINVAL                           # TwoPass words need hl
    assert call(qm=1, hl=A) == EINVAL
    assert call(qm=0) == EINVAL                           # Dequant writes yn only
    assert call(qm=0, yn=A, hq=None, hs=None, N=500) == ESHAPE   # Dequant outputs pass to the shape checks
    assert call(qm=0, yn=A + 4, hq=None, hs=None) == EALIGN
    assert call(hs=None) == EINVAL
    assert call(r=None) == EINVAL                         # s needs r
    assert call(eps=-1.0) == EINVAL
    assert call(eps=float("nan")) == EINVAL
    assert call(N=500) == ESHAPE                          # whole 32-value blocks of the norm
    assert call(N=nmax + 32) == ESHAPE
    assert call(K=500) == ESHAPE
    assert call(S=0) == ESHAPE
    assert call(S=65) == ESHAPE
    assert call(S=1) == EMODE                             # no split: nothing meets in a workgroup
    assert call(S=17) == EMODE
    assert call(mode=2, xl=A, K=65536, S=16) == EMODE     # the staged row exceeds the LDS budget
    assert call(wq=A + 8) == EALIGN
    assert call(ws=A + 1) == EALIGN
    assert call(y=A + 2) == EALIGN
    assert call(r=A + 4) == EALIGN
    assert call(s=A + 8) == EALIGN
    assert call(w=A + 4) == EALIGN
    assert call(hq=A + 4) == EALIGN
    assert call(hs=A + 2) == EALIGN
    assert call(wsp=A + 8) == EALIGN
    assert call(nbytes=need - 4) == EWORKSPACE


def test_swiglu_quantize_validation():
    f = lib.qdg_swiglu_quantize

    def call(mode=1, g=A, u=A, B=1, K=512, h=None, xq=A, xl=None, xs=A):
        return f(mode, P(g), P(u), B, K, P(h), P(xq), P(xl), P(xs), None)

    assert call(mode=-1) == EINVAL
    assert call(g=None) == EINVAL
    assert call(u=None) == EINVAL
    assert call(mode=0) == EINVAL                         # Dequant writes h only
    assert call(mode=2) == EINVAL
    assert call(mode=1, xl=A) == EINVAL
    assert call(K=48) == ESHAPE
    assert call(B=0) == ESHAPE
    assert call(g=A + 4) == EALIGN
    assert call(u=A + 8) == EALIGN
    assert call(h=A + 4) == EALIGN
    assert call(mode=2, xl=A + 4) == EALIGN


@pytest.mark.parametrize("act", [0, 1, 2])
def test_glu_quantize_validation(act):
    """qdg_glu_quantize checks as qdg_swiglu_quantize does, and rejects an unknown activation first."""
    f = lib.qdg_glu_quantize

    def call(act=act, mode=1, g=A, u=A, B=1, K=512, h=None, xq=A, xl=None, xs=A):
        return f(act, mode, P(g), P(u), B, K, P(h), P(xq), P(xl), P(xs), None)

    assert call(act=3) == EINVAL and call(act=-1) == EINVAL
    assert call(g=None) == EINVAL
    assert call(mode=0) == EINVAL
    assert call(K=48) == ESHAPE
    assert call(u=A + 8) == EALIGN


@pytest.mark.parametrize("act", [0, 1, 2])
def test_glu_act_validation(act):
    f = lib.qdg_gemv_glu_act_q8

    def call(act=act, mode=1, wg=A, sg=A, wu=A, su=A, F=128, K=4096, xq=A, xl=None, xs=A, h=None, hq=A, hl=None,
             hs=A):
        return f(act, mode, P(wg), P(sg), P(wu), P(su), F, K, P(xq), P(xl), P(xs), P(h), P(hq), P(hl), P(hs), None)

    assert call(act=3) == EINVAL and call(act=-2) == EINVAL
    assert call(mode=0) == EINVAL
    assert call(F=100) == ESHAPE
    assert call(h=A + 4) == EALIGN
    assert call(mode=1, K=15808) == EMODE


def test_parts_validation():
    f = lib.qdg_gemv_q8_parts
    Part = q._Part

    def table(n=3, wq=A, ws=A, N=64, y=A):
        arr = (Part * max(n, 1))()
        for i in range(max(n, 1)):
            arr[i] = Part(wq, ws, N, y)
        return arr

    def call(mode=1, parts=None, n=3, K=8192, x=None, xq=A, xl=None, xs=A, S=4, **kw):
        arr = parts if parts is not None else table(n, **kw)
        return f(mode, ctypes.cast(arr, P), n, K, P(x), P(xq), P(xl), P(xs), S, None)

    assert f(1, None, 1, 8192, None, P(A), None, P(A), 4, None) == EINVAL
    assert call(mode=3) == EINVAL
    assert call(n=0) == ESHAPE
    assert call(n=7) == ESHAPE
    assert call(wq=None) == EINVAL
    assert call(y=None) == EINVAL
    assert call(x=A) == EINVAL                          # quantized modes take words, not x
    assert call(mode=2) == EINVAL                       # TwoPass needs xl
    assert call(mode=0, xq=None, xs=None) == EINVAL     # Dequant needs x
    assert call(N=0) == ESHAPE
    assert call(K=500) == ESHAPE
    assert call(wq=A + 8) == EALIGN
    assert call(ws=A + 1) == EALIGN
    assert call(xq=A + 4) == EALIGN
    assert call(S=1) == EMODE                           # no split: nothing to combine in a workgroup
    assert call(S=64) == EMODE                          # more chunk waves than a workgroup holds
    assert call(mode=2, xl=A, K=65536, S=16) == EMODE   # the staged row exceeds the LDS budget
    assert call(mode=0, x=A + 4, xq=None, xs=None) == EALIGN


def test_glu_validation():
    f = lib.qdg_gemv_glu_q8

    def call(mode=1, wg=A, sg=A, wu=A, su=A, F=128, K=4096, xq=A, xl=None, xs=A, h=None, hq=A, hl=None, hs=A):
        return f(mode, P(wg), P(sg), P(wu), P(su), F, K, P(xq), P(xl), P(xs), P(h), P(hq), P(hl), P(hs), None)

    assert call(mode=0) == EINVAL
    assert call(wu=None) == EINVAL
    assert call(hq=None) == EINVAL
    assert call(mode=2, xl=A) == EINVAL                 # TwoPass needs hl too
    assert call(mode=1, hl=A) == EINVAL
    assert call(F=100) == ESHAPE                        # one quantized block per 32 outputs
    assert call(F=0) == ESHAPE
    assert call(K=4100) == ESHAPE
    assert call(wg=A + 8) == EALIGN
    assert call(h=A + 4) == EALIGN
    assert call(hs=A + 2) == EALIGN
    assert call(mode=2, xl=A, hl=A, K=13216) == EMODE   # the activation and 64 rows of scales exceed LDS
    assert call(mode=1, K=15808) == EMODE


@pytest.mark.parametrize("act", [0, 1, 2])
def test_glu_dequant_validation(act):
    """qdg_gemv_glu_dequant: each operand at an address of its own, then one bad argument
    at a time; h may not overlap x, a weight matrix or a scale array."""
    f = lib.qdg_gemv_glu_dequant
    X, WG, WU, SG, SU, H = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000
    F, K = 128, 4096  # spans: x 16 KiB, weights 512 KiB, scales 32 KiB

    def call(act=act, wg=WG, sg=SG, wu=WU, su=SU, F=F, K=K, x=X, h=H):
        return f(act, P(wg), P(sg), P(wu), P(su), F, K, P(x), P(h), None)

    assert call(act=3) == EINVAL and call(act=-1) == EINVAL
    assert call(x=None) == EINVAL
    assert call(h=None) == EINVAL
    assert call(wu=None) == EINVAL and call(su=None) == EINVAL
    assert call(F=0) == ESHAPE
    assert call(K=48) == ESHAPE and call(K=0) == ESHAPE
    assert call(F=1 << 33, K=32) == ESHAPE              # more than 2^31 four-row workgroups
    assert call(wg=WG + 8) == EALIGN
    assert call(wu=WU + 8) == EALIGN
    assert call(sg=SG + 1) == EALIGN
    assert call(x=X + 4) == EALIGN
    assert call(h=H + 2) == EALIGN
    assert call(h=X + 16) == EINVAL                     # h over x
    assert call(h=X - 4 * F + 4) == EINVAL              # h's last value on x's first
    assert call(h=WU + 0x80000 - 4) == EINVAL           # h's first value on the up matrix's last word
    assert call(h=SG + 0x8000 - 4) == EINVAL
    assert call(h=SU) == EINVAL
    assert call(h=WG, act=act, F=F) == EINVAL


@pytest.mark.parametrize("act", [0, 1, 2])
def test_glu_mma_tiled_validation(act):
    """qdg_gemv_glu_mma_tiled: operands at addresses of their own, one bad argument at a time;
    no output may overlap an input."""
    f = lib.qdg_gemv_glu_mma_tiled
    WG, WU, XQ, XL, XS, H, HQ, HL, HS = (0x1000000 * (i + 1) for i in range(9))
    F, K, B = 512, 1024, 16  # records (512/64)*(1024/256)*4*4352 = 557056 bytes; words 16*K bytes

    def call(act=act, mode=1, wgt=WG, wut=WU, F=F, K=K, xq=XQ, xl=None, xs=XS, B=B, h=H, hq=HQ, hl=None, hs=HS):
        return f(act, mode, P(wgt), P(wut), F, K, P(xq), P(xl), P(xs), B, P(h), P(hq), P(hl), P(hs), None)

    assert call(act=3) == EINVAL and call(act=-1) == EINVAL
    assert call(mode=0) == EINVAL and call(mode=3) == EINVAL
    assert call(wut=None) == EINVAL and call(hq=None) == EINVAL and call(hs=None) == EINVAL
    assert call(mode=2, xl=XL) == EINVAL                # TwoPass needs hl too
    assert call(mode=1, hl=HL) == EINVAL
    assert call(F=320) == ESHAPE                        # F a multiple of 256
    assert call(K=288) == ESHAPE and call(K=0) == ESHAPE
    assert call(B=0) == ESHAPE and call(B=65) == ESHAPE
    assert call(wgt=WG + 8) == EALIGN
    assert call(xq=XQ + 4) == EALIGN
    assert call(h=H + 4) == EALIGN
    assert call(hq=HQ + 2) == EALIGN
    assert call(mode=2, xl=XL, hl=HL + 1) == EALIGN
    assert call(hq=XQ + 16 * K - 4) == EINVAL          # hq's first word on xq's last
    assert call(hs=XS) == EINVAL
    assert call(h=WU + 557056 - 16) == EINVAL          # h on the up records' last bytes
    assert call(mode=2, xl=XL, hl=XL + 64) == EINVAL
    assert call(hq=WG - 16 * F + 4) == EINVAL          # hq's last word on the gate records' first


def test_fmt_validation():
    for fmt in oracle.FORMATS:
        for K in (256, 512, 5120):
            assert q.fmt_row_bytes(fmt, K) == oracle.fmt_row_bytes(fmt, K), (fmt, K)
    assert q.fmt_row_bytes(8, 256) == 0            # Q8_0 is the split layout, not this call's
    assert q.fmt_row_bytes(12, 300) == 0
    f = lib.qdg_gemv_fmt

    def call(fmt=2, mode=1, w=A, N=64, K=512, x=None, xq=A, xl=None, xs=A, y=A, splits=1):
        return f(fmt, mode, P(w), N, K, P(x), P(xq), P(xl), P(xs), splits, P(y), None)

    assert call(fmt=8) == EINVAL
    assert call(mode=3) == EINVAL
    assert call(w=None) == EINVAL
    assert call(mode=0) == EINVAL                       # Dequant reads x
    assert call(mode=2) == EINVAL                       # TwoPass needs xl
    assert call(K=500) == ESHAPE
    assert call(fmt=12, K=480) == ESHAPE                # Q4_K needs whole 256-value super-blocks
    assert call(N=0) == ESHAPE
    assert call(w=A + 8) == EALIGN
    assert call(xq=A + 4) == EALIGN
    assert call(y=A + 2) == EALIGN
    assert call(splits=0) == EINVAL
    assert call(splits=65) == EINVAL


def test_chunk_wave_queries_validate():
    """The wave-count queries reject what the launches reject, before asking the device."""
    fw, dw = lib.qdg_gemv_fmt_chunk_waves, lib.qdg_gemv_dq_chunk_waves
    assert fw(8, 1, 64, 512, 8) == EINVAL        # unknown format
    assert fw(2, 3, 64, 512, 8) == EINVAL        # unknown mode
    assert fw(2, 1, 64, 512, 0) == EINVAL
    assert fw(12, 1, 64, 480, 8) == ESHAPE       # Q4_K needs whole 256-value super-blocks
    assert fw(2, 1, 0, 512, 8) == ESHAPE
    assert dw(0, 512, 8) == ESHAPE
    assert dw(64, 500, 8) == ESHAPE
    assert dw(64, 512, 65) == ESHAPE


def test_stream_read_validation():
    f = lib.qdg_stream_read
    assert f(None, 1024, P(A), None) == EINVAL
    assert f(P(A), 1024, None, None) == EINVAL
    assert f(P(A), 8, P(A), None) == ESHAPE
    assert f(P(A), 1000, P(A), None) == ESHAPE
    assert f(P(A + 8), 1024, P(A), None) == EALIGN


def test_split_bounds_validation():
    arr = (ctypes.c_int32 * 66)()
    assert lib.qdg_split_bounds(512, 0, ctypes.cast(arr, P)) == ESHAPE
    assert lib.qdg_split_bounds(500, 2, ctypes.cast(arr, P)) == ESHAPE
    assert lib.qdg_split_bounds(512, 2, None) == EINVAL
    assert lib.qdg_split_bounds(512, 64, ctypes.cast(arr, P)) == OK


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    w = torch.zeros((4, 64), dtype=torch.int8)
    with pytest.raises(ValueError):
        q.gemv_q8(q.INT8ACT, w, torch.zeros((4, 2), dtype=torch.int16), torch.zeros((1, 4)),
                  xq=torch.zeros((1, 64), dtype=torch.int8), xs=torch.zeros((1, 2)))


def test_one_hip_runtime_in_the_process():
    """The package alone must not bring a second HIP runtime next to PyTorch's:
    a fresh process that imports only the package maps one libamdhip64 (two
    copies leave the library's runtime without a device at its first launch)."""
    import subprocess
    import sys
    code = ("import quantized_decode_gemv_02_amd, torch, re\n"
            "paths = set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l)\n"
            "print(len(paths), sorted(paths))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[0] == "1", r.stdout


def test_tiled_layout_validation():
    tile = lib.qdg_q8_tile_rows
    assert tile(None, 8, 512, P(A), None) == EINVAL
    assert tile(P(A), 8, 512, None, None) == EINVAL
    assert tile(P(A), 6, 512, P(A + 8192), None) == ESHAPE  # N not a multiple of 4
    assert tile(P(A), 8, 288, P(A + 8192), None) == ESHAPE  # K not a multiple of 256
    assert tile(P(A), 0, 512, P(A + 8192), None) == ESHAPE
    assert tile(P(A + 8), 8, 512, P(A + 8192), None) == EALIGN
    assert tile(P(A), 8, 512, P(A + 4080), None) == EINVAL  # overlaps wq's 4096 bytes
    assert tile(P(A + 4080), 8, 512, P(A), None) == EINVAL

    def sk(mode=1, wt=A, N=64, K=5120, xl=None, S=5, xs=A, y=A):
        return lib.qdg_gemv_q8_sk_tiled(mode, P(wt), P(A), N, K, P(A), P(xl), P(xs), S, P(y), None)

    assert sk(mode=0) == EMODE
    assert sk(mode=3) == EINVAL
    assert sk(wt=None) == EINVAL
    assert sk(mode=2) == EINVAL            # TwoPass without xl
    assert sk(mode=1, xl=A) == EINVAL      # Int8Act with xl
    assert sk(N=66) == ESHAPE
    assert sk(K=5120 + 32) == ESHAPE
    assert sk(S=1) == EMODE                # not an in-workgroup split
    assert sk(S=17) == EMODE               # more than 16 chunk waves
    assert sk(S=0) == ESHAPE
    assert sk(mode=2, xl=A, K=32768, S=5) == EMODE  # the staged row exceeds the LDS budget
    assert sk(wt=A + 4) == EALIGN
    assert sk(xs=A + 2) == EALIGN


def test_tuning_knobs():
    """The tuning hooks start at the library's own choice (-1), never read the
    environment, reject unknown knobs, and the binding's context manager puts
    every knob back."""
    for k in range(17):
        assert lib.qdg_get_tuning(k) == -1, k
    assert lib.qdg_get_tuning(17) == EINVAL
    assert lib.qdg_get_tuning(-1) == EINVAL
    assert lib.qdg_set_tuning(17, 0) == EINVAL
    assert lib.qdg_set_tuning(2, 1) == OK and lib.qdg_get_tuning(2) == 1
    assert lib.qdg_set_tuning(2, -7) == OK and lib.qdg_get_tuning(2) == -1
    with q.tuning(ws_dma=0, ws_local=1):
        assert q.get_tuning("ws_dma") == 0 and q.get_tuning("ws_local") == 1
        with q.tuning(ws_local=0):
            assert q.get_tuning("ws_local") == 0
        assert q.get_tuning("ws_local") == 1
    assert q.get_tuning("ws_dma") == -1 and q.get_tuning("ws_local") == -1
    assert sorted(q.TUNE.values()) == list(range(17))
    assert lib.qdg_time_next_launch(None, None) == OK


def test_knobs_ignore_the_environment():
    """A process whose environment names the old variables still starts with every knob at -1
    and the same in-workgroup placement."""
    import subprocess
    import sys
    code = ("import quantized_decode_gemv_02_amd as q\n"
            "print([q.get_tuning(k) for k in q.TUNE], q.sk_workgroup_shape(2, 25600, 5))\n")
    env = dict(os.environ, QDG_WS_ROWS="1", QDG_SK_WSPLIT="0", QDG_WS_DMA="0", QDG_MFMA_GENERAL="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == str([-1] * 17) + " (12, 15)", r.stdout


def test_binding_checks_sizes_before_the_call():
    """Undersized buffers raise ValueError on the host, before any pointer reaches the library."""
    torch = pytest.importorskip("torch")
    N, K = 8, 512
    w = torch.zeros((N, K), dtype=torch.int8)
    ws = torch.zeros((N, K // 32), dtype=torch.int16)
    xq, xl = torch.zeros((1, K), dtype=torch.int8), torch.zeros((1, K), dtype=torch.int8)
    xs, y = torch.zeros((1, K // 32)), torch.zeros((1, N))
    wsp = torch.zeros(64, dtype=torch.int64)
    cases = [
        lambda: q.gemv_q8_sk(q.TWOPASS, w, ws, torch.zeros(N - 1), xq, xl, xs, 4, wsp),
        lambda: q.gemv_q8_sk(q.TWOPASS, w, torch.zeros((N, K // 64), dtype=torch.int16), y, xq, xl, xs, 4, wsp),
        lambda: q.gemv_q8_sk(q.TWOPASS, w, ws, y, xq[:, :K - 32].contiguous(), xl, xs, 4, wsp),
        lambda: q.gemv_q8_sk(q.TWOPASS, w, ws, y, xq, xl[:, :16].contiguous(), xs, 4, wsp),
        lambda: q.gemv_q8_sk(q.TWOPASS, w, ws, y, xq, xl, xs[:, :3].contiguous(), 4, wsp),
        lambda: q.gemv_q8_sk_tiled(q.INT8ACT, w, ws, torch.zeros(4), xq, None, xs, 4),
        lambda: q.bind_gemv_q8_sk(q.INT8ACT, w, ws, torch.zeros(3), xq, None, xs, 4, wsp),
        lambda: q.bind_gemv_q8_sk_tiled(q.INT8ACT, w, ws, y, xq, None, xs[:, :1].contiguous(), 4),
        lambda: q.gemv_q8(q.INT8ACT, w, ws, torch.zeros((3, 1, N)), xq=xq, xs=xs, splits=4),
        lambda: q.gemv_q8_fused(q.INT8ACT, w, ws, y, torch.zeros((1, K - 32)), 4, wsp),
        lambda: q.quantize_act(q.TWOPASS, torch.zeros((1, K)), xq, xl[:, :8].contiguous(), xs),
        lambda: q.gemv_q8_argmax(q.INT8ACT, w, ws, torch.zeros(N - 2), torch.zeros(1, dtype=torch.int32), wsp,
                                 xq=xq, xs=xs),
    ]
    # the gate/up epilogues: F = 64 outputs
    F = 64
    wg = torch.zeros((F, K), dtype=torch.int8)
    sg = torch.zeros((F, K // 32), dtype=torch.int16)
    hq, hs = torch.zeros(F, dtype=torch.int8), torch.zeros(F // 32)
    R = q.mma_act_rows(16)
    wt = torch.zeros(q.q8_tile_mma_bytes(F, K), dtype=torch.uint8)
    tq, ts = torch.zeros(R * K, dtype=torch.int8), torch.zeros(R * (K // 32))
    cases += [
        lambda: q.gemv_glu_q8(q.INT8ACT, wg, sg[:F // 2].contiguous(), wg, sg, xq, None, xs, hq, None, hs),
        lambda: q.gemv_glu_q8(q.INT8ACT, wg, sg, wg, sg, xq, None, xs, hq[:F - 4].contiguous(), None, hs),
        lambda: q.gemv_glu_act_q8(q.ACT_SIGMOID, q.INT8ACT, wg, sg, wg, sg, xq, None, xs[:, :2].contiguous(), hq,
                                  None, hs),
        lambda: q.gemv_glu_dequant(0, wg, sg, wg, sg[:3].contiguous(), torch.zeros(K), torch.zeros(F)),
        lambda: q.gemv_glu_mma_tiled(0, q.INT8ACT, wt, wt, F, K, tq, None, ts, 16, torch.zeros(R * F - 4,
                                     dtype=torch.int8), None, torch.zeros(R * (F // 32))),
        lambda: q.gemv_glu_mma_tiled(0, q.INT8ACT, wt[:100].contiguous(), wt, F, K, tq, None, ts, 16,
                                     torch.zeros(R * F, dtype=torch.int8), None, torch.zeros(R * (F // 32))),
    ]
    for i, c in enumerate(cases):
        with pytest.raises(ValueError, match="holds|ws must"):
            c()


def test_mma_tiled_validation():
    """The MFMA-tiled batched path: sizes, modes, shapes, alignment and overlap are
    rejected on the host with the documented status."""
    nbytes = lib.qdg_q8_tile_mma_bytes
    nbytes.restype = ctypes.c_int64
    nbytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
    assert nbytes(64, 256) == 4 * 4352
    assert nbytes(65, 512) == 2 * 2 * 4 * 4352
    assert nbytes(25600, 5120) == 400 * 20 * 4 * 4352
    for N, K in ((64, 32), (64, 288), (0, 256), (64, 0), (1, 1 << 30)):
        assert nbytes(N, K) == 0, (N, K)

    def tile(wq=A, ws=A, N=64, K=512, wt=A + (1 << 30)):
        return lib.qdg_q8_tile_mma(P(wq), P(ws), N, K, P(wt), None)

    assert tile(wq=None) == EINVAL and tile(ws=None) == EINVAL and tile(wt=None) == EINVAL
    assert tile(K=288) == ESHAPE and tile(N=0) == ESHAPE and tile(K=32) == ESHAPE
    assert tile(wq=A + 8) == EALIGN and tile(ws=A + 1) == EALIGN and tile(wt=A + (1 << 30) + 8) == EALIGN
    assert tile(wt=A) == EINVAL                      # overlaps wq
    assert tile(ws=A + (1 << 30) + 4096) == EINVAL   # ws inside wt

    def quant(mode=1, x=A, B=4, K=512, xq=A, xl=None, xs=A):
        return lib.qdg_quantize_act_mma(mode, P(x), B, K, P(xq), P(xl), P(xs), None)

    assert quant(mode=0) == EINVAL and quant(mode=3) == EINVAL
    assert quant(x=None) == EINVAL and quant(xq=None) == EINVAL and quant(xs=None) == EINVAL
    assert quant(mode=2) == EINVAL                   # TwoPass needs xl
    assert quant(xl=A) == EINVAL                     # Int8Act takes no xl
    assert quant(B=0) == ESHAPE and quant(B=65) == ESHAPE and quant(K=288) == ESHAPE
    assert quant(x=A + 4) == EALIGN and quant(xq=A + 8) == EALIGN and quant(xs=A + 2) == EALIGN
    assert quant(mode=2, xl=A + 8) == EALIGN

    def mt(mode=1, wt=A, N=64, K=512, xq=A, xl=None, xs=A, B=4, S=1, out=A):
        return lib.qdg_gemv_q8_mma_tiled(mode, P(wt), N, K, P(xq), P(xl), P(xs), B, S, P(out), None)

    assert mt(mode=0) == EMODE                       # Dequant is not served
    assert mt(mode=3) == EINVAL and mt(wt=None) == EINVAL and mt(out=None) == EINVAL
    assert mt(mode=2) == EINVAL and mt(xl=A) == EINVAL
    assert mt(K=288) == ESHAPE and mt(N=0) == ESHAPE and mt(B=0) == ESHAPE and mt(S=0) == ESHAPE
    assert mt(S=65) == ESHAPE and mt(B=65) == ESHAPE
    assert mt(wt=A + 8) == EALIGN and mt(xq=A + 4) == EALIGN and mt(xs=A + 2) == EALIGN and mt(out=A + 1) == EALIGN
