"""NVFP4 quantization on MI355X (gfx950): Python binding of libnvfp4.so.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in include/nvfp4.h. PyTorch provides device memory (output
tensors are allocated here with torch.empty) and the current stream. There
is no fallback: if the library is missing, every call raises.

Names follow the C ABI: nvfp4_amax, nvfp4_quantize_1d, nvfp4_quantize_1d_fused,
nvfp4_quantize_2d, nvfp4_rht16, nvfp4_dequantize, nvfp4_gemm, nvfp4_status_string, and the
MXFP4 comparator format's mxfp4_quantize, mxfp4_dequantize, mxfp4_gemm
(include/mxfp4.h).
"""
from __future__ import annotations

import ctypes
import os

from . import build as _build

ROWWISE = 0x1
COLWISE = 0x2
SR = 0x4
RHT = 0x8
AMAX_BOTH = 0x20
WORKSPACE_BYTES = 32832
SCALE_1D = 1
SCALE_2D = 2
SCALE_2D_T = 3  # 2D tile scales of the transposed operand (GEMM only)
F32 = 0
BF16 = 1

STATUS = {
    0: "NVFP4_OK",
    -1: "NVFP4_ERR_NULL",
    -2: "NVFP4_ERR_SHAPE",
    -3: "NVFP4_ERR_ALIGN",
    -4: "NVFP4_ERR_FLAGS",
    -5: "NVFP4_ERR_HIP",
    -6: "NVFP4_ERR_SIZE",
}

EXPORTS = (
    "nvfp4_status_string",
    "nvfp4_amax",
    "nvfp4_quantize_1d",
    "nvfp4_quantize_1d_fused",
    "nvfp4_quantize_1d_fused_noalloc",
    "nvfp4_quantize_2d",
    "nvfp4_quantize_2d_tscales",
    "nvfp4_rht16",
    "nvfp4_dequantize",
    "nvfp4_gemm",
    "nvfp4_gemm_amax",
    "nvfp4_gemm_quantize",
    "mxfp4_quantize",
    "mxfp4_dequantize",
    "mxfp4_gemm",
)


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded C library (ctypes). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB_PATH):
        raise ImportError(
            f"{_build.LIB_PATH} is missing: build it with "
            "`python -m fp4_block_scaled_amax_amd.build` (hipcc, gfx950)"
        )
    L = ctypes.CDLL(_build.LIB_PATH)
    P, I64, U32, U16, U64, I = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint16,
                                ctypes.c_uint64, ctypes.c_int)
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_status_string.argtypes = [I]
    L.nvfp4_amax.restype = I
    L.nvfp4_amax.argtypes = [P, I64, I64, U32, U16, P, P]
    L.nvfp4_quantize_1d.restype = I
    L.nvfp4_quantize_1d.argtypes = [P, I64, I64, P, U32, U16, U64, P, P, P, P, P, P]
    L.nvfp4_quantize_1d_fused.restype = I
    L.nvfp4_quantize_1d_fused.argtypes = [P, I64, I64, U32, U64, P, P, P, P, P, P, P]
    L.nvfp4_quantize_1d_fused_noalloc.restype = I
    L.nvfp4_quantize_1d_fused_noalloc.argtypes = [P, I64, I64, U32, U64, P, P, P, P, P, P, P]
    L.nvfp4_quantize_2d.restype = I
    L.nvfp4_quantize_2d.argtypes = [P, I64, I64, P, P, P, P, P, P]
    L.nvfp4_quantize_2d_tscales.restype = I
    L.nvfp4_quantize_2d_tscales.argtypes = [P, I64, I64, P, P, P, P, P, P, P]
    L.nvfp4_rht16.restype = I
    L.nvfp4_rht16.argtypes = [P, I64, I64, I, U16, P, P]
    L.nvfp4_dequantize.restype = I
    L.nvfp4_dequantize.argtypes = [P, P, I, P, I64, I64, P, I, P]
    L.nvfp4_gemm.restype = I
    L.nvfp4_gemm.argtypes = [P, P, I, P, P, P, I, P, P, I, I64, I64, I64, P]
    L.nvfp4_gemm_amax.restype = I
    L.nvfp4_gemm_amax.argtypes = [P, P, I, P, P, P, I, P, P, I, I64, I64, I64, P, P]
    L.nvfp4_gemm_quantize.restype = I
    L.nvfp4_gemm_quantize.argtypes = [P, P, I, P, P, P, I, P, I64, I64, I64, P, U32, P, P, P, P, P, P, P]
    L.mxfp4_quantize.restype = I
    L.mxfp4_quantize.argtypes = [P, I64, I64, U32, U16, P, P, P, P, P]
    L.mxfp4_dequantize.restype = I
    L.mxfp4_dequantize.argtypes = [P, P, I64, I64, P, I, P]
    L.mxfp4_gemm.restype = I
    L.mxfp4_gemm.argtypes = [P, P, P, P, P, I, I64, I64, I64, P]
    _lib = L
    return L


def nvfp4_status_string(status: int) -> str:
    return lib().nvfp4_status_string(status).decode()


def _check(status: int):
    if status != 0:
        raise Nvfp4Error(status, nvfp4_status_string(status))


# --------------------------------------------------------------- marshalling

def _torch():
    import torch

    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _bits16(x, name="x"):
    """bf16 tensor (or its int16/uint16 bit patterns) -> 2-D tensor."""
    torch = _torch()
    _dev_tensor(x, name)
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16 (or its 16-bit patterns)")
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows][cols]")
    return x


def _empty(shape, dtype, device, out=None):
    torch = _torch()
    if out is not None:
        return out
    return torch.empty(shape, dtype=dtype, device=device)


# ------------------------------------------------------------------ the API

def nvfp4_amax(x, rht: bool = False, rht_mask: int = 0, out=None, stream=None, both: bool = False):
    """Tensor amax (of the axis-0 Hadamard transform when rht) -> float32 [1];
    with both=True (and rht), float32 [2]: the plain amax and the
    transform's, from one read of x."""
    torch = _torch()
    _bits16(x)
    out = _empty((2 if both else 1,), torch.float32, x.device, out)
    flags = (RHT if rht else 0) | (AMAX_BOTH if both else 0)
    _check(lib().nvfp4_amax(_ptr(x), x.shape[0], x.shape[1], flags, rht_mask & 0xFFFF,
                            _ptr(out), _stream(stream)))
    return out


def nvfp4_workspace(device=None):
    """A zero-filled workspace for nvfp4_quantize_1d_fused."""
    torch = _torch()
    return torch.zeros(WORKSPACE_BYTES // 4, dtype=torch.int32, device=device or "cuda")


def _q1_outputs(x, rowwise, colwise, out):
    R, C = x.shape
    return _q1_outputs_of(R, C, x.device, rowwise, colwise, out)


def _q1_outputs_of(R, C, dev, rowwise, colwise, out):
    torch = _torch()
    out = dict(out or {})
    if rowwise:
        out["codes_row"] = _empty((R, C // 2), torch.uint8, dev, out.get("codes_row"))
        out["scales_row"] = _empty((R, C // 16), torch.uint8, dev, out.get("scales_row"))
    if colwise:
        out["codes_col"] = _empty((C, R // 2), torch.uint8, dev, out.get("codes_col"))
        out["scales_col"] = _empty((C, R // 16), torch.uint8, dev, out.get("scales_col"))
    out["global_scale"] = _empty((1,), torch.float32, dev, out.get("global_scale"))
    return out


def nvfp4_quantize_1d(x, amax, rowwise: bool = True, colwise: bool = False, sr: bool = False,
                      rht: bool = False, rht_mask: int = 0, seed: int = 0, out: dict | None = None,
                      stream=None):
    """1D NVFP4 quantization with the amax given (float32 [1] from
    nvfp4_amax). Returns a dict with codes_row [R][C/2], scales_row
    [R][C/16], codes_col [C][R/2], scales_col [C][R/16] (the requested
    layouts) and global_scale (float32 [1])."""
    torch = _torch()
    _bits16(x)
    _dev_tensor(amax, "amax", torch.float32)
    R, C = x.shape
    out = _q1_outputs(x, rowwise, colwise, out)
    flags = ((ROWWISE if rowwise else 0) | (COLWISE if colwise else 0) | (SR if sr else 0)
             | (RHT if rht else 0))
    _check(lib().nvfp4_quantize_1d(
        _ptr(x), R, C, _ptr(amax), flags, rht_mask & 0xFFFF, seed & ((1 << 64) - 1),
        _ptr(out.get("codes_row")), _ptr(out.get("scales_row")),
        _ptr(out.get("codes_col")), _ptr(out.get("scales_col")),
        _ptr(out["global_scale"]), _stream(stream)))
    return out


def nvfp4_quantize_1d_fused(x, workspace, rowwise: bool = True, colwise: bool = False,
                            sr: bool = False, seed: int = 0, out: dict | None = None, stream=None):
    """1D NVFP4 quantization that finds the amax in the same call (one pass
    over x when it fits on chip). workspace: from nvfp4_workspace(); the amax
    lands in its first float (ws.view(torch.float32)[0]). Outputs as
    nvfp4_quantize_1d."""
    _bits16(x)
    _dev_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < WORKSPACE_BYTES:
        raise ValueError(f"workspace must hold {WORKSPACE_BYTES} bytes")
    R, C = x.shape
    out = _q1_outputs(x, rowwise, colwise, out)
    flags = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0) | (SR if sr else 0)
    _check(lib().nvfp4_quantize_1d_fused(
        _ptr(x), R, C, flags, seed & ((1 << 64) - 1), _ptr(workspace),
        _ptr(out.get("codes_row")), _ptr(out.get("scales_row")),
        _ptr(out.get("codes_col")), _ptr(out.get("scales_col")),
        _ptr(out["global_scale"]), _stream(stream)))
    return out


def nvfp4_quantize_1d_fused_noalloc(x, rowwise: bool = True, colwise: bool = False, sr: bool = False,
                                    seed: int = 0, out: dict | None = None, amax=None, stream=None):
    """nvfp4_quantize_1d_fused on the library's own static workspace (no
    device allocation by the library; pass preallocated outputs in `out` to
    allocate nothing here either). amax: optional float32 [1] that receives
    the amax. Calls that overlap in time on one device race."""
    torch = _torch()
    _bits16(x)
    if amax is not None:
        _dev_tensor(amax, "amax", torch.float32)
    R, C = x.shape
    out = _q1_outputs(x, rowwise, colwise, out)
    flags = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0) | (SR if sr else 0)
    _check(lib().nvfp4_quantize_1d_fused_noalloc(
        _ptr(x), R, C, flags, seed & ((1 << 64) - 1),
        _ptr(out.get("codes_row")), _ptr(out.get("scales_row")),
        _ptr(out.get("codes_col")), _ptr(out.get("scales_col")),
        _ptr(out["global_scale"]), _ptr(amax), _stream(stream)))
    return out


def nvfp4_quantize_2d(x, amax, rowwise: bool = True, colwise: bool = True, out: dict | None = None,
                      stream=None, transposed_scales: bool = False):
    """2D (16x16 tile) NVFP4 weight quantization -> dict with codes_row,
    codes_col (requested layouts), scales [R/16][C/16], global_scale; with
    transposed_scales also scales_t [C/16][R/16] (nvfp4_quantize_2d_tscales:
    the scales under which codes_col is a plain 2D-scaled operand)."""
    torch = _torch()
    _bits16(x)
    _dev_tensor(amax, "amax", torch.float32)
    R, C = x.shape
    out = dict(out or {})
    dev = x.device
    if rowwise:
        out["codes_row"] = _empty((R, C // 2), torch.uint8, dev, out.get("codes_row"))
    if colwise:
        out["codes_col"] = _empty((C, R // 2), torch.uint8, dev, out.get("codes_col"))
    out["scales"] = _empty((R // 16, C // 16), torch.uint8, dev, out.get("scales"))
    out["global_scale"] = _empty((1,), torch.float32, dev, out.get("global_scale"))
    if transposed_scales:
        out["scales_t"] = _empty((C // 16, R // 16), torch.uint8, dev, out.get("scales_t"))
        _check(lib().nvfp4_quantize_2d_tscales(
            _ptr(x), R, C, _ptr(amax), _ptr(out.get("codes_row")), _ptr(out.get("codes_col")),
            _ptr(out["scales"]), _ptr(out["scales_t"]), _ptr(out["global_scale"]), _stream(stream)))
        return out
    _check(lib().nvfp4_quantize_2d(
        _ptr(x), R, C, _ptr(amax), _ptr(out.get("codes_row")), _ptr(out.get("codes_col")),
        _ptr(out["scales"]), _ptr(out["global_scale"]), _stream(stream)))
    return out


def nvfp4_rht16(x, axis: int = 0, rht_mask: int = 0, out=None, stream=None):
    """Random-sign 16-point Hadamard transform along `axis` -> float32."""
    torch = _torch()
    _bits16(x)
    out = _empty(tuple(x.shape), torch.float32, x.device, out)
    _check(lib().nvfp4_rht16(_ptr(x), x.shape[0], x.shape[1], axis, rht_mask & 0xFFFF, _ptr(out),
                             _stream(stream)))
    return out


def nvfp4_dequantize(codes, scales, scale_mode: int, global_scale, rows: int, cols: int,
                     out_dtype=None, out=None, stream=None):
    """Reconstruct [rows][cols] (float32 or bfloat16) from one layout."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    _dev_tensor(codes, "codes", torch.uint8)
    _dev_tensor(scales, "scales", torch.uint8)
    _dev_tensor(global_scale, "global_scale", torch.float32)
    dt = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    out = _empty((rows, cols), out_dtype, codes.device, out)
    _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), scale_mode, _ptr(global_scale), rows,
                                  cols, _ptr(out), dt, _stream(stream)))
    return out


def nvfp4_gemm(a_codes, a_scales, a_scale_mode: int, a_global_scale, b_codes, b_scales,
               b_scale_mode: int, b_global_scale, M: int, N: int, K: int, out_dtype=None, out=None,
               stream=None, out_amax=None):
    """C [M][N] = A * B^T from packed NVFP4 operands (TN). out_amax: a
    float32 [1] tensor that also receives max |C| of the stored values
    (nvfp4_gemm_amax: the amax pass of C's own quantization, fused into the
    epilogue)."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    for name, t in (("a_codes", a_codes), ("a_scales", a_scales), ("b_codes", b_codes),
                    ("b_scales", b_scales)):
        _dev_tensor(t, name, torch.uint8)
    _dev_tensor(a_global_scale, "a_global_scale", torch.float32)
    _dev_tensor(b_global_scale, "b_global_scale", torch.float32)
    dt = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    out = _empty((M, N), out_dtype, a_codes.device, out)
    if out_amax is not None:
        _dev_tensor(out_amax, "out_amax", torch.float32)
        _check(lib().nvfp4_gemm_amax(_ptr(a_codes), _ptr(a_scales), a_scale_mode, _ptr(a_global_scale),
                                     _ptr(b_codes), _ptr(b_scales), b_scale_mode, _ptr(b_global_scale),
                                     _ptr(out), dt, M, N, K, _ptr(out_amax), _stream(stream)))
        return out
    _check(lib().nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), a_scale_mode, _ptr(a_global_scale),
                            _ptr(b_codes), _ptr(b_scales), b_scale_mode, _ptr(b_global_scale),
                            _ptr(out), dt, M, N, K, _stream(stream)))
    return out


def nvfp4_gemm_quantize(a_codes, a_scales, a_scale_mode: int, a_global_scale, b_codes, b_scales,
                        b_scale_mode: int, b_global_scale, M: int, N: int, K: int, amax,
                        rowwise: bool = True, colwise: bool = True, out: dict | None = None,
                        out_amax=None, stream=None):
    """The NVFP4 quantization of the bf16 product A * B^T, made by the GEMM's
    epilogue (C is never stored): the dict nvfp4_quantize_1d(Y, amax, ...)
    returns for Y = nvfp4_gemm(..., out_dtype=bfloat16). amax: float32 [1],
    the tensor amax the quantization takes (for instance the previous
    product's out_amax). out_amax: optional float32 [1] that receives max |Y|
    of this product."""
    torch = _torch()
    for name, t in (("a_codes", a_codes), ("a_scales", a_scales), ("b_codes", b_codes),
                    ("b_scales", b_scales)):
        _dev_tensor(t, name, torch.uint8)
    _dev_tensor(a_global_scale, "a_global_scale", torch.float32)
    _dev_tensor(b_global_scale, "b_global_scale", torch.float32)
    _dev_tensor(amax, "amax", torch.float32)
    if out_amax is not None:
        _dev_tensor(out_amax, "out_amax", torch.float32)
    out = _q1_outputs_of(M, N, a_codes.device, rowwise, colwise, out)
    flags = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    _check(lib().nvfp4_gemm_quantize(
        _ptr(a_codes), _ptr(a_scales), a_scale_mode, _ptr(a_global_scale),
        _ptr(b_codes), _ptr(b_scales), b_scale_mode, _ptr(b_global_scale), M, N, K,
        _ptr(amax), flags, _ptr(out.get("codes_row")), _ptr(out.get("scales_row")),
        _ptr(out.get("codes_col")), _ptr(out.get("scales_col")), _ptr(out["global_scale"]),
        _ptr(out_amax), _stream(stream)))
    return out


# ------------------------------------------------- MXFP4 comparator format

def mxfp4_quantize(x, rowwise: bool = True, colwise: bool = False, rht: bool = False,
                   rht_mask: int = 0, out: dict | None = None, stream=None):
    """MXFP4 quantization (E8M0 scale per 32 elements) -> dict with codes_row
    [R][C/2], scales_row [R][C/32], codes_col [C][R/2], scales_col [C][R/32]
    (the requested layouts). rht: columnwise only, after the axis-0
    Hadamard transform with sign mask rht_mask."""
    torch = _torch()
    _bits16(x)
    R, C = x.shape
    out = dict(out or {})
    dev = x.device
    if rowwise:
        out["codes_row"] = _empty((R, C // 2), torch.uint8, dev, out.get("codes_row"))
        out["scales_row"] = _empty((R, C // 32), torch.uint8, dev, out.get("scales_row"))
    if colwise:
        out["codes_col"] = _empty((C, R // 2), torch.uint8, dev, out.get("codes_col"))
        out["scales_col"] = _empty((C, R // 32), torch.uint8, dev, out.get("scales_col"))
    flags = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0) | (RHT if rht else 0)
    _check(lib().mxfp4_quantize(
        _ptr(x), R, C, flags, rht_mask & 0xFFFF, _ptr(out.get("codes_row")), _ptr(out.get("scales_row")),
        _ptr(out.get("codes_col")), _ptr(out.get("scales_col")), _stream(stream)))
    return out


def mxfp4_dequantize(codes, scales, rows: int, cols: int, out_dtype=None, out=None, stream=None):
    """Reconstruct [rows][cols] (float32 or bfloat16) from MXFP4 codes and
    E8M0 scales [rows][cols/32]."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    _dev_tensor(codes, "codes", torch.uint8)
    _dev_tensor(scales, "scales", torch.uint8)
    dt = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    out = _empty((rows, cols), out_dtype, codes.device, out)
    _check(lib().mxfp4_dequantize(_ptr(codes), _ptr(scales), rows, cols, _ptr(out), dt, _stream(stream)))
    return out


def mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, M: int, N: int, K: int, out_dtype=None, out=None,
               stream=None):
    """C [M][N] = A * B^T from MXFP4 operands (TN) on the block-scaled
    matrix cores."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    for name, t in (("a_codes", a_codes), ("a_scales", a_scales), ("b_codes", b_codes),
                    ("b_scales", b_scales)):
        _dev_tensor(t, name, torch.uint8)
    dt = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    out = _empty((M, N), out_dtype, a_codes.device, out)
    _check(lib().mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), _ptr(out), dt,
                            M, N, K, _stream(stream)))
    return out
