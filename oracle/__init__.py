"""NVFP4 reference oracle -- TEST INFRASTRUCTURE ONLY.

Python face of the plain-C oracle in ``nvfp4_oracle.c``. Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it. It shares no code with the HIP library and never imports it.

All tensors are numpy arrays; bf16 tensors are ``uint16`` bit patterns.
The C side computes every value; this module only marshals arguments,
except for the contraction, whose double-precision matrix product of the
exactly reconstructed operands is a library matmul (numpy).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")

# IEEE binary32 semantics: no contraction into FMA, no fast-math.
CFLAGS = ["-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-std=c11"]

_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    U64 = ctypes.c_uint64
    sig = {
        "nvfp4_oracle_e2m1_decode": (ctypes.c_double, [ctypes.c_uint8]),
        "nvfp4_oracle_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
        "nvfp4_oracle_e4m3_encode": (ctypes.c_uint8, [F]),
        "nvfp4_oracle_e2m1_rne": (ctypes.c_int, [F]),
        "nvfp4_oracle_e2m1_sr": (ctypes.c_int, [F, ctypes.c_uint16]),
        "nvfp4_oracle_philox4x32_10": (None, [P, P, P]),
        "nvfp4_oracle_sr_draw": (ctypes.c_uint16, [U64, U64]),
        "nvfp4_oracle_rht16": (None, [P, ctypes.c_uint16, P]),
        "nvfp4_oracle_rht16_tensor": (None, [P, I64, I64, ctypes.c_int, ctypes.c_uint16, P]),
        "nvfp4_oracle_amax_bf16": (F, [P, I64]),
        "nvfp4_oracle_amax_rht_axis0": (F, [P, I64, I64, ctypes.c_uint16]),
        "nvfp4_oracle_global_scale": (F, [F]),
        "nvfp4_oracle_quantize_1d_rows": (None, [P, I64, I64, F, ctypes.c_int, U64, I64, I64, P, P]),
        "nvfp4_oracle_quantize_1d_cols": (
            None,
            [P, I64, I64, F, ctypes.c_int, U64, ctypes.c_int, ctypes.c_uint16, I64, I64, P, P],
        ),
        "nvfp4_oracle_quantize_2d": (None, [P, I64, I64, F, I64, I64, P, P, P]),
        "nvfp4_oracle_dequantize": (None, [P, P, ctypes.c_int, F, I64, I64, I64, I64, P]),
        "nvfp4_oracle_dequantize_bf16": (None, [P, P, ctypes.c_int, F, I64, I64, I64, I64, P]),
        "nvfp4_oracle_dequantize_f64_rows": (None, [P, P, ctypes.c_int, F, I64, I64, P, I64, P]),
        "nvfp4_oracle_e2m1_rne_array": (None, [P, I64, P]),
        "nvfp4_oracle_e2m1_sr_array": (None, [P, P, I64, P]),
        "nvfp4_oracle_e4m3_encode_array": (None, [P, I64, P]),
        "nvfp4_oracle_sr_draw_array": (None, [U64, P, I64, P]),
        "mxfp4_oracle_e8m0_decode": (ctypes.c_double, [ctypes.c_uint8]),
        "mxfp4_oracle_scale_byte": (ctypes.c_uint8, [F]),
        "mxfp4_oracle_quantize_rows": (None, [P, I64, I64, I64, I64, P, P]),
        "mxfp4_oracle_quantize_cols": (None, [P, I64, I64, ctypes.c_int, ctypes.c_uint16, I64, I64, P, P]),
        "mxfp4_oracle_dequantize": (None, [P, P, I64, I64, I64, I64, P]),
        "mxfp4_oracle_dequantize_f64_rows": (None, [P, P, I64, I64, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- scalars

def e2m1_decode(code: int) -> float:
    return _load().nvfp4_oracle_e2m1_decode(code)


def e4m3_decode(b: int) -> float:
    return _load().nvfp4_oracle_e4m3_decode(b)


def e4m3_encode(v: float) -> int:
    return int(_load().nvfp4_oracle_e4m3_encode(v))


def e2m1_rne(v: float) -> int:
    return int(_load().nvfp4_oracle_e2m1_rne(v))


def e2m1_sr(v: float, h: int) -> int:
    return int(_load().nvfp4_oracle_e2m1_sr(v, h))


def global_scale(amax: float) -> np.float32:
    return np.float32(_load().nvfp4_oracle_global_scale(float(amax)))


def philox4x32_10(ctr, key) -> np.ndarray:
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.zeros(4, np.uint32)
    _load().nvfp4_oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_draw(seed: int, i: int) -> int:
    return int(_load().nvfp4_oracle_sr_draw(seed, i))


# ----------------------------------------------------------------- arrays

def e2m1_rne_array(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().nvfp4_oracle_e2m1_rne_array(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_sr_array(v: np.ndarray, h: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    h = _c(h, np.uint16)
    assert v.shape == h.shape
    out = np.empty(v.shape, np.uint8)
    _load().nvfp4_oracle_e2m1_sr_array(_ptr(v), _ptr(h), v.size, _ptr(out))
    return out


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().nvfp4_oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def sr_draw_array(seed: int, idx: np.ndarray) -> np.ndarray:
    idx = _c(idx, np.uint64)
    out = np.empty(idx.shape, np.uint16)
    _load().nvfp4_oracle_sr_draw_array(seed, _ptr(idx), idx.size, _ptr(out))
    return out


def rht16(x16, mask: int) -> np.ndarray:
    x = _c(x16, np.float32)
    assert x.size == 16
    y = np.empty(16, np.float32)
    _load().nvfp4_oracle_rht16(_ptr(x), mask, _ptr(y))
    return y


def rht16_tensor(x: np.ndarray, axis: int, mask: int) -> np.ndarray:
    x = _c(x, np.uint16)
    R, C = x.shape
    y = np.empty((R, C), np.float32)
    _load().nvfp4_oracle_rht16_tensor(_ptr(x), R, C, axis, mask, _ptr(y))
    return y


# -------------------------------------------------------------- the path

def amax(x: np.ndarray) -> np.float32:
    x = _c(x, np.uint16)
    return np.float32(_load().nvfp4_oracle_amax_bf16(_ptr(x), x.size))


def amax_rht(x: np.ndarray, mask: int) -> np.float32:
    x = _c(x, np.uint16)
    R, C = x.shape
    return np.float32(_load().nvfp4_oracle_amax_rht_axis0(_ptr(x), R, C, mask))


def quantize_1d_rows(x: np.ndarray, sg, sr: bool = False, seed: int = 0, r0: int = 0, r1=None):
    """Rowwise 1D codes [r1-r0][C/2] and scales [r1-r0][C/16]."""
    x = _c(x, np.uint16)
    R, C = x.shape
    r1 = R if r1 is None else r1
    codes = np.empty((r1 - r0, C // 2), np.uint8)
    scales = np.empty((r1 - r0, C // 16), np.uint8)
    _load().nvfp4_oracle_quantize_1d_rows(
        _ptr(x), R, C, float(sg), int(bool(sr)), seed, r0, r1, _ptr(codes), _ptr(scales)
    )
    return codes, scales


def quantize_1d_cols(x: np.ndarray, sg, sr: bool = False, seed: int = 0, rht: bool = False,
                     mask: int = 0, c0: int = 0, c1=None):
    """Columnwise 1D codes [c1-c0][R/2] and scales [c1-c0][R/16]."""
    x = _c(x, np.uint16)
    R, C = x.shape
    c1 = C if c1 is None else c1
    codes = np.empty((c1 - c0, R // 2), np.uint8)
    scales = np.empty((c1 - c0, R // 16), np.uint8)
    _load().nvfp4_oracle_quantize_1d_cols(
        _ptr(x), R, C, float(sg), int(bool(sr)), seed, int(bool(rht)), mask, c0, c1,
        _ptr(codes), _ptr(scales)
    )
    return codes, scales


def quantize_2d(x: np.ndarray, sg, tr0: int = 0, tr1=None):
    """2D codes_row [R][C/2], codes_col [C][R/2], tile scales [R/16][C/16]
    (only tile rows [tr0, tr1) are filled; the rest stays zero)."""
    x = _c(x, np.uint16)
    R, C = x.shape
    tr1 = R // 16 if tr1 is None else tr1
    codes_row = np.zeros((R, C // 2), np.uint8)
    codes_col = np.zeros((C, R // 2), np.uint8)
    scales = np.zeros((R // 16, C // 16), np.uint8)
    _load().nvfp4_oracle_quantize_2d(
        _ptr(x), R, C, float(sg), tr0, tr1, _ptr(codes_row), _ptr(codes_col), _ptr(scales)
    )
    return codes_row, codes_col, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, scale_mode: int, sg, R: int, C: int,
               r0: int = 0, r1=None) -> np.ndarray:
    """binary32 reconstruction of rows [r0, r1); scale_mode 1 = 1D, 2 = 2D."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    r1 = R if r1 is None else r1
    out = np.empty((r1 - r0, C), np.float32)
    _load().nvfp4_oracle_dequantize(_ptr(codes), _ptr(scales), scale_mode, float(sg), R, C, r0, r1,
                                    _ptr(out))
    return out


def dequantize_bf16(codes: np.ndarray, scales: np.ndarray, scale_mode: int, sg, R: int, C: int,
                    r0: int = 0, r1=None) -> np.ndarray:
    """bf16 bit patterns of the reconstruction (binary32 value rounded to
    nearest even)."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    r1 = R if r1 is None else r1
    out = np.empty((r1 - r0, C), np.uint16)
    _load().nvfp4_oracle_dequantize_bf16(_ptr(codes), _ptr(scales), scale_mode, float(sg), R, C, r0,
                                         r1, _ptr(out))
    return out


def dequantize_f64_rows(codes: np.ndarray, scales: np.ndarray, scale_mode: int, sg, R: int, C: int,
                        rows) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, C), np.float64)
    _load().nvfp4_oracle_dequantize_f64_rows(_ptr(codes), _ptr(scales), scale_mode, float(sg), R, C,
                                             _ptr(rows), rows.size, _ptr(out))
    return out


def gemm_rows(a_codes, a_scales, a_mode, a_sg, b_codes, b_scales, b_mode, b_sg, M, N, K, rows):
    """Reference product rows: C[m][n] = sum_k A^[m][k] B^[n][k] in double,
    with A^ and B^ the exact reconstructions (TN layout)."""
    a = dequantize_f64_rows(a_codes, a_scales, a_mode, a_sg, M, K, rows)
    b = dequantize_f64_rows(b_codes, b_scales, b_mode, b_sg, N, K, np.arange(N, dtype=np.int64))
    return a @ b.T


# ------------------------------------------------- whole-call conveniences

def quantize_1d(x: np.ndarray, rowwise=True, colwise=False, sr=False, seed=0, rht=False, mask=0):
    """The whole 1D call: amax (of the transformed tensor when rht), global
    scale, then the requested layouts. Returns a dict."""
    a = amax_rht(x, mask) if rht else amax(x)
    sg = global_scale(a)
    out = {"amax": a, "sg": sg}
    if rowwise:
        out["codes_row"], out["scales_row"] = quantize_1d_rows(x, sg, sr, seed)
    if colwise:
        out["codes_col"], out["scales_col"] = quantize_1d_cols(x, sg, sr, seed, rht, mask)
    return out


# ------------------------------------------ MXFP4, the comparator format

def e8m0_decode(b: int) -> float:
    return _load().mxfp4_oracle_e8m0_decode(b)


def mx_scale_byte(amax: float) -> int:
    return int(_load().mxfp4_oracle_scale_byte(float(amax)))


def mx_quantize_rows(x: np.ndarray, r0: int = 0, r1=None):
    """MXFP4 rowwise codes [r1-r0][C/2] and E8M0 scales [r1-r0][C/32]."""
    x = _c(x, np.uint16)
    R, C = x.shape
    r1 = R if r1 is None else r1
    codes = np.empty((r1 - r0, C // 2), np.uint8)
    scales = np.empty((r1 - r0, C // 32), np.uint8)
    _load().mxfp4_oracle_quantize_rows(_ptr(x), R, C, r0, r1, _ptr(codes), _ptr(scales))
    return codes, scales


def mx_quantize_cols(x: np.ndarray, rht: bool = False, mask: int = 0, c0: int = 0, c1=None):
    """MXFP4 columnwise codes [c1-c0][R/2] and scales [c1-c0][R/32]."""
    x = _c(x, np.uint16)
    R, C = x.shape
    c1 = C if c1 is None else c1
    codes = np.empty((c1 - c0, R // 2), np.uint8)
    scales = np.empty((c1 - c0, R // 32), np.uint8)
    _load().mxfp4_oracle_quantize_cols(_ptr(x), R, C, int(bool(rht)), mask, c0, c1, _ptr(codes),
                                       _ptr(scales))
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, R: int, C: int, r0: int = 0,
                  r1=None) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    r1 = R if r1 is None else r1
    out = np.empty((r1 - r0, C), np.float32)
    _load().mxfp4_oracle_dequantize(_ptr(codes), _ptr(scales), R, C, r0, r1, _ptr(out))
    return out


def mx_dequantize_f64_rows(codes: np.ndarray, scales: np.ndarray, R: int, C: int,
                           rows) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, C), np.float64)
    _load().mxfp4_oracle_dequantize_f64_rows(_ptr(codes), _ptr(scales), R, C, _ptr(rows), rows.size,
                                             _ptr(out))
    return out


def mx_gemm_rows(a_codes, a_scales, b_codes, b_scales, M, N, K, rows):
    """MXFP4 reference product rows: C[m][n] = sum_k A^[m][k] B^[n][k] in
    double from the exact reconstructions (TN layout)."""
    a = mx_dequantize_f64_rows(a_codes, a_scales, M, K, rows)
    b = mx_dequantize_f64_rows(b_codes, b_scales, N, K, np.arange(N, dtype=np.int64))
    return a @ b.T


# ------------------------------------------- the same functions on all cores
#
# The C functions take row, column or tile-row ranges and release the
# interpreter lock, so threads run them side by side on disjoint ranges of
# one output array. The arithmetic is the single-threaded functions'; only
# the work is split (whole 16-row blocks for the transform, whole tiles for
# 2D), so the bytes are the same.

def host_threads(limit: int = 16) -> int:
    """Threads for the multi-threaded drivers: the CPUs this process may
    use, at most `limit`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(limit, n))


def _ranges(n: int, parts: int, align: int = 1):
    step = -(-n // max(1, parts))
    step = max(align, -(-step // align) * align)
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)]


def _run(fn, ranges, threads):
    from concurrent.futures import ThreadPoolExecutor

    if len(ranges) == 1:
        return [fn(ranges[0])]
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, ranges))


def _at(a: np.ndarray, offset: int):
    return ctypes.c_void_p(a.ctypes.data + offset)


def amax_mt(x: np.ndarray, threads: int | None = None) -> np.float32:
    x = _c(x, np.uint16)
    t = threads or host_threads()
    parts = _run(lambda r: amax(x[r[0]:r[1]]), _ranges(x.shape[0], t), t)
    return np.float32(np.nan) if any(np.isnan(p) for p in parts) else np.float32(max(parts))


def amax_rht_mt(x: np.ndarray, mask: int, threads: int | None = None) -> np.float32:
    x = _c(x, np.uint16)
    t = threads or host_threads()
    parts = _run(lambda r: amax_rht(x[r[0]:r[1]], mask), _ranges(x.shape[0], t, 16), t)
    return np.float32(np.nan) if any(np.isnan(p) for p in parts) else np.float32(max(parts))


def quantize_1d_rows_mt(x: np.ndarray, sg, sr: bool = False, seed: int = 0, threads: int | None = None):
    """quantize_1d_rows over the whole tensor, row ranges on threads."""
    x = _c(x, np.uint16)
    R, C = x.shape
    codes = np.empty((R, C // 2), np.uint8)
    scales = np.empty((R, C // 16), np.uint8)
    lib = _load()
    t = threads or host_threads()

    def work(r):
        lib.nvfp4_oracle_quantize_1d_rows(_ptr(x), R, C, float(sg), int(bool(sr)), seed, r[0], r[1],
                                          _at(codes, r[0] * (C // 2)), _at(scales, r[0] * (C // 16)))

    _run(work, _ranges(R, t), t)
    return codes, scales


def quantize_1d_cols_mt(x: np.ndarray, sg, sr: bool = False, seed: int = 0, rht: bool = False,
                        mask: int = 0, threads: int | None = None):
    """quantize_1d_cols over the whole tensor, column ranges on threads."""
    x = _c(x, np.uint16)
    R, C = x.shape
    codes = np.empty((C, R // 2), np.uint8)
    scales = np.empty((C, R // 16), np.uint8)
    lib = _load()
    t = threads or host_threads()

    def work(c):
        lib.nvfp4_oracle_quantize_1d_cols(_ptr(x), R, C, float(sg), int(bool(sr)), seed, int(bool(rht)), mask,
                                          c[0], c[1], _at(codes, c[0] * (R // 2)), _at(scales, c[0] * (R // 16)))

    _run(work, _ranges(C, t), t)
    return codes, scales


def mx_quantize_rows_mt(x: np.ndarray, threads: int | None = None):
    """mx_quantize_rows over the whole tensor, row ranges on threads."""
    x = _c(x, np.uint16)
    R, C = x.shape
    codes = np.empty((R, C // 2), np.uint8)
    scales = np.empty((R, C // 32), np.uint8)
    lib = _load()
    t = threads or host_threads()

    def work(r):
        lib.mxfp4_oracle_quantize_rows(_ptr(x), R, C, r[0], r[1], _at(codes, r[0] * (C // 2)),
                                       _at(scales, r[0] * (C // 32)))

    _run(work, _ranges(R, t), t)
    return codes, scales


def mx_quantize_cols_mt(x: np.ndarray, rht: bool = False, mask: int = 0, threads: int | None = None):
    """mx_quantize_cols over the whole tensor, column ranges on threads."""
    x = _c(x, np.uint16)
    R, C = x.shape
    codes = np.empty((C, R // 2), np.uint8)
    scales = np.empty((C, R // 32), np.uint8)
    lib = _load()
    t = threads or host_threads()

    def work(c):
        lib.mxfp4_oracle_quantize_cols(_ptr(x), R, C, int(bool(rht)), mask, c[0], c[1],
                                       _at(codes, c[0] * (R // 2)), _at(scales, c[0] * (R // 32)))

    _run(work, _ranges(C, t), t)
    return codes, scales


def quantize_2d_mt(x: np.ndarray, sg, threads: int | None = None):
    """quantize_2d over the whole tensor, tile-row ranges on threads."""
    x = _c(x, np.uint16)
    R, C = x.shape
    codes_row = np.zeros((R, C // 2), np.uint8)
    codes_col = np.zeros((C, R // 2), np.uint8)
    scales = np.zeros((R // 16, C // 16), np.uint8)
    lib = _load()
    t = threads or host_threads()

    def work(tr):
        lib.nvfp4_oracle_quantize_2d(_ptr(x), R, C, float(sg), tr[0], tr[1], _ptr(codes_row), _ptr(codes_col),
                                     _ptr(scales))

    _run(work, _ranges(R // 16, t), t)
    return codes_row, codes_col, scales


def dequantize_mt(codes: np.ndarray, scales: np.ndarray, scale_mode: int, sg, R: int, C: int,
                  bf16: bool = False, threads: int | None = None) -> np.ndarray:
    """dequantize (binary32) or dequantize_bf16 over the whole tensor."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    out = np.empty((R, C), np.uint16 if bf16 else np.float32)
    lib = _load()
    fn = lib.nvfp4_oracle_dequantize_bf16 if bf16 else lib.nvfp4_oracle_dequantize
    t = threads or host_threads()

    def work(r):
        fn(_ptr(codes), _ptr(scales), scale_mode, float(sg), R, C, r[0], r[1], _at(out, r[0] * C * out.itemsize))

    _run(work, _ranges(R, t, 16), t)
    return out
