"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/*.h declares,
and reject bad arguments with the documented status codes before making any
HIP call (so these run on a machine without a GPU).
"""
import ctypes
import os
import re

import pytest

import fp4_block_scaled_amax_amd as F
from fp4_block_scaled_amax_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = ctypes.c_void_p
A = P(4096)  # a 16-byte aligned, never dereferenced stand-in pointer
MIS = P(4097)
NULL = None


@pytest.fixture(scope="module")
def L():
    if B.is_stale():
        B.build()
    return F.lib()


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b((?:nvfp4|mxfp4)_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(F.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in F.STATUS:
        s = F.nvfp4_status_string(code)
        assert isinstance(s, str) and s
    assert F.nvfp4_status_string(12345) == "unknown status"


def test_amax_validation(L):
    assert L.nvfp4_amax(NULL, 16, 16, 0, 0, A, NULL) == -1
    assert L.nvfp4_amax(A, 16, 16, 0, 0, NULL, NULL) == -1
    assert L.nvfp4_amax(A, 0, 16, 0, 0, A, NULL) == -2
    assert L.nvfp4_amax(A, 16, -1, 0, 0, A, NULL) == -2
    assert L.nvfp4_amax(A, 16, 16, 0x80, 0, A, NULL) == -4
    assert L.nvfp4_amax(MIS, 16, 16, 0, 0, A, NULL) == -3
    assert L.nvfp4_amax(A, 24, 16, F.RHT, 0, A, NULL) == -2  # rows not a multiple of 16
    assert L.nvfp4_amax(A, 1 << 40, 1 << 40, 0, 0, A, NULL) == -6
    assert L.nvfp4_amax(A, 16, 16, F.AMAX_BOTH, 0, A, NULL) == -4  # both amaxes need the transform


def q1(L, x=A, rows=64, cols=64, amax=A, flags=F.ROWWISE, cr=A, sr_=A, cc=A, sc=A):
    return L.nvfp4_quantize_1d(x, rows, cols, amax, flags, 0, 0, cr, sr_, cc, sc, NULL, NULL)


def test_quantize_1d_validation(L):
    assert q1(L, flags=0) == -4
    assert q1(L, flags=0x40 | F.ROWWISE) == -4
    assert q1(L, flags=F.RHT | F.ROWWISE | F.COLWISE) == -4  # RHT is columnwise only
    assert q1(L, flags=F.RHT | F.ROWWISE) == -4
    assert q1(L, x=NULL) == -1
    assert q1(L, amax=NULL) == -1
    assert q1(L, cr=NULL) == -1
    assert q1(L, flags=F.COLWISE, sc=NULL) == -1
    assert q1(L, rows=24) == -2
    assert q1(L, cols=8) == -2
    assert q1(L, rows=0) == -2
    assert q1(L, x=MIS) == -3
    assert q1(L, flags=F.COLWISE, cc=MIS) == -3
    assert q1(L, rows=1 << 40, cols=1 << 40) == -6


def q1f(L, x=A, rows=64, cols=64, flags=F.ROWWISE, ws=A, cr=A, sr_=A, cc=A, sc=A):
    return L.nvfp4_quantize_1d_fused(x, rows, cols, flags, 0, ws, cr, sr_, cc, sc, NULL, NULL)


def test_quantize_1d_fused_validation(L):
    assert q1f(L, flags=0) == -4
    assert q1f(L, flags=F.ROWWISE | F.RHT) == -4  # the transform's amax is nvfp4_amax's
    assert q1f(L, flags=F.COLWISE | F.RHT) == -4
    assert q1f(L, flags=F.ROWWISE | 0x10) == -4  # unknown flag
    assert q1f(L, x=NULL) == -1
    assert q1f(L, ws=NULL) == -1
    assert q1f(L, cr=NULL) == -1
    assert q1f(L, flags=F.COLWISE, sc=NULL) == -1
    assert q1f(L, rows=24) == -2
    assert q1f(L, x=MIS) == -3
    assert q1f(L, ws=MIS) == -3
    assert q1f(L, rows=1 << 40, cols=1 << 40) == -6
    # nvfp4_quantize_1d itself no longer takes a workspace flag
    assert q1(L, flags=F.ROWWISE | 0x10) == -4


def test_quantize_1d_fused_noalloc_validation(L):
    f = lambda **k: L.nvfp4_quantize_1d_fused_noalloc(
        k.get("x", A), k.get("rows", 64), k.get("cols", 64), k.get("flags", F.ROWWISE), 0, k.get("cr", A),
        k.get("sr", A), k.get("cc", A), k.get("sc", A), NULL, k.get("amax", NULL), NULL)
    assert f(flags=0) == -4
    assert f(flags=F.COLWISE | F.RHT) == -4
    assert f(x=NULL) == -1
    assert f(cr=NULL) == -1
    assert f(rows=40) == -2
    assert f(x=MIS) == -3
    assert f(amax=P(4098)) == -3
    assert f(rows=1 << 40, cols=1 << 40) == -6


def test_quantize_2d_validation(L):
    assert L.nvfp4_quantize_2d(A, 32, 32, A, NULL, NULL, A, NULL, NULL) == -1
    assert L.nvfp4_quantize_2d(A, 32, 32, A, A, A, NULL, NULL, NULL) == -1
    assert L.nvfp4_quantize_2d(A, 40, 32, A, A, A, A, NULL, NULL) == -2
    assert L.nvfp4_quantize_2d(A, 32, 32, A, MIS, A, A, NULL, NULL) == -3
    assert L.nvfp4_quantize_2d_tscales(A, 32, 32, A, A, A, A, NULL, NULL, NULL) == -1  # scales_t required
    assert L.nvfp4_quantize_2d_tscales(A, 40, 32, A, A, A, A, A, NULL, NULL) == -2


def test_rht_dequant_gemm_validation(L):
    assert L.nvfp4_rht16(A, 32, 32, 2, 0, A, NULL) == -4
    assert L.nvfp4_rht16(A, 24, 32, 0, 0, A, NULL) == -2
    assert L.nvfp4_rht16(A, 24, 24, 1, 0, A, NULL) == -2
    assert L.nvfp4_rht16(A, 32, 32, 0, 0, MIS, NULL) == -3
    assert L.nvfp4_dequantize(A, A, 3, A, 32, 32, A, 0, NULL) == -4
    assert L.nvfp4_dequantize(A, A, 1, A, 32, 32, A, 7, NULL) == -4
    assert L.nvfp4_dequantize(A, A, 1, NULL, 32, 32, A, 0, NULL) == -1
    assert L.nvfp4_dequantize(A, A, 1, A, 33, 32, A, 0, NULL) == -2
    g = lambda **k: L.nvfp4_gemm(k.get("ac", A), A, k.get("am", 1), A, A, A, k.get("bm", 2), A,
                                 k.get("c", A), k.get("dt", 0), k.get("M", 32), k.get("N", 32),
                                 k.get("K", 32), NULL)
    assert g(ac=NULL) == -1
    assert g(am=0) == -4
    assert g(dt=3) == -4
    assert g(K=24) == -2
    assert g(M=0) == -2
    assert g(c=MIS) == -3
    ga = lambda amax: L.nvfp4_gemm_amax(A, A, 1, A, A, A, 2, A, A, 0, 32, 32, 32, amax, NULL)
    assert ga(NULL) == -1
    assert ga(P(4098)) == -3


def test_gemm_quantize_validation(L):
    def gq(**k):
        return L.nvfp4_gemm_quantize(k.get("ac", A), A, 1, A, A, A, 2, A, k.get("M", 32), k.get("N", 32),
                                     k.get("K", 32), k.get("amax", A), k.get("f", F.ROWWISE | F.COLWISE),
                                     k.get("cr", A), k.get("sr", A), k.get("cc", A), k.get("sc", A),
                                     NULL, k.get("camax", NULL), NULL)
    assert gq(f=0) == -4
    assert gq(f=F.ROWWISE | F.SR) == -4  # round to nearest only
    assert gq(amax=NULL) == -1
    assert gq(cr=NULL) == -1
    assert gq(f=F.COLWISE, cr=NULL, sr=NULL, M=24) == -2  # rowwise outputs not needed: the shape fails next
    assert gq(f=F.ROWWISE, cc=NULL, sc=NULL, M=24) == -2  # nor columnwise ones
    assert gq(cc=NULL) == -1
    assert gq(ac=NULL) == -1
    assert gq(M=24) == -2
    assert gq(K=0) == -2
    assert gq(cr=MIS) == -3
    assert gq(sc=MIS) == -3
    assert gq(camax=P(4098)) == -3


def test_mxfp4_validation(L):
    q = lambda **k: L.mxfp4_quantize(k.get("x", A), k.get("R", 64), k.get("C", 64), k.get("f", F.ROWWISE), 0,
                                     k.get("cr", A), k.get("sr", A), k.get("cc", A), k.get("sc", A), NULL)
    assert q(f=0) == -4
    assert q(f=F.ROWWISE | F.SR) == -4                    # no stochastic rounding
    assert q(f=F.ROWWISE | F.RHT) == -4                   # the transform is columnwise only
    assert q(f=F.ROWWISE | F.COLWISE | F.RHT) == -4
    assert q(x=NULL) == -1
    assert q(cr=NULL) == -1
    assert q(f=F.COLWISE, sc=NULL) == -1
    assert q(f=F.COLWISE, R=48) == -2                     # columnwise: rows a multiple of 32
    assert q(f=F.COLWISE, C=12) == -2                     # ... and cols of 8
    assert q(C=16) == -2                                  # rowwise: cols a multiple of 32
    assert q(x=MIS) == -3
    assert q(R=1 << 40, C=1 << 40) == -6
    assert L.mxfp4_dequantize(NULL, A, 32, 32, A, 0, NULL) == -1
    assert L.mxfp4_dequantize(A, A, 32, 32, A, 2, NULL) == -4
    assert L.mxfp4_dequantize(A, A, 32, 48, A, 0, NULL) == -2
    assert L.mxfp4_dequantize(A, A, 32, 32, MIS, 0, NULL) == -3
    g = lambda **k: L.mxfp4_gemm(k.get("ac", A), A, A, k.get("bs", A), k.get("c", A), k.get("dt", 0),
                                 k.get("M", 32), k.get("N", 32), k.get("K", 64), NULL)
    assert g(ac=NULL) == -1
    assert g(bs=NULL) == -1
    assert g(dt=5) == -4
    assert g(K=48) == -2
    assert g(M=0) == -2
    assert g(c=MIS) == -3
    assert g(M=1 << 40, N=1 << 40, K=1 << 20) == -6


def test_oracle_is_not_reachable_from_product():
    """The product package never imports or links the oracle."""
    pkg = os.path.join(ROOT, "fp4_block_scaled_amax_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
