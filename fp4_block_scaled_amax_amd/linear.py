"""NVFP4 linear layer y = x W^T, composed from the library's calls.

The three GEMMs of a linear layer in the NVFP4 training recipe, each with
the quantization its operands take (page "Melatih model dalam 4 bit:
pengaman numerik di balik NVFP4", section "Empat pengaman"; page "NVFP4 Is a
Scaling System, Not Just a 4-Bit Number", section "A format is not a
training recipe"):

  fprop  Y  = X W^T    X rowwise 1D RNE;  W 2D tiles (rowwise copy)
  dgrad  dX = dY W     dY rowwise 1D stochastic;  W 2D tiles (columnwise copy)
  wgrad  dW = dY^T X   dY and X columnwise (blocks along the tokens) after the
                       random-sign Hadamard transform with one shared sign
                       mask; dY stochastic, X round-to-nearest-even

The shared mask makes the transform cancel in dW: (H D a)^T (H D b) / 16 =
a^T b, since H^T H = 16 I and D^2 = I. The weight is quantized once with
2D tiles, so its two copies hold identical codes and the same tile scales
(read transposed by the dgrad GEMM, NVFP4_SCALE_2D_T).

Every step runs in the library's kernels; this module only sequences calls
on one stream. Shapes: x [tokens][in], w [out][in], dy [tokens][out], all
bf16 bit patterns (int16/uint16 tensors), every dimension a multiple of 16.
"""
from __future__ import annotations

from . import (SCALE_1D, SCALE_2D, SCALE_2D_T, _torch, nvfp4_amax, nvfp4_gemm,
               nvfp4_quantize_1d, nvfp4_quantize_2d, nvfp4_workspace)


def quantize_weight(w, stream=None) -> dict:
    """W [out][in] -> 2D-tiled NVFP4 in both layouts: codes_row [out][in/2],
    codes_col [in][out/2], scales [out/16][in/16], global_scale."""
    return nvfp4_quantize_2d(w, nvfp4_amax(w, stream=stream), rowwise=True, colwise=True,
                             stream=stream)


def fprop(x, wq: dict, ws=None, out_dtype=None, stream=None):
    """Y [tokens][out] = X W^T: X rowwise 1D RNE (amax and quantization in
    one pass through the workspace `ws`, allocated if None)."""
    tokens, k = x.shape
    n = wq["codes_row"].shape[0]
    ws = nvfp4_workspace(x.device) if ws is None else ws
    xq = nvfp4_quantize_1d(x, ws, rowwise=True, fused_amax=True, stream=stream)
    return nvfp4_gemm(xq["codes_row"], xq["scales_row"], SCALE_1D, xq["global_scale"],
                      wq["codes_row"], wq["scales"], SCALE_2D, wq["global_scale"],
                      tokens, n, k, out_dtype=out_dtype, stream=stream)


def dgrad(dy, wq: dict, seed: int, ws=None, out_dtype=None, stream=None):
    """dX [tokens][in] = dY W: dY rowwise 1D stochastic (seed), W's
    columnwise copy with its tile scales read transposed."""
    tokens, k = dy.shape
    n = wq["codes_col"].shape[0]
    ws = nvfp4_workspace(dy.device) if ws is None else ws
    dyq = nvfp4_quantize_1d(dy, ws, rowwise=True, sr=True, seed=seed, fused_amax=True,
                            stream=stream)
    return nvfp4_gemm(dyq["codes_row"], dyq["scales_row"], SCALE_1D, dyq["global_scale"],
                      wq["codes_col"], wq["scales"], SCALE_2D_T, wq["global_scale"],
                      tokens, n, k, out_dtype=out_dtype, stream=stream)


def wgrad_operands(dy, x, rht_mask: int, seed: int, x_sr: bool = False, stream=None):
    """The two columnwise operands of dW = dY^T X, blocks along the tokens,
    after the Hadamard transform with the shared sign mask: dY stochastic,
    X round-to-nearest-even (or stochastic with x_sr)."""
    a_dy = nvfp4_amax(dy, rht=True, rht_mask=rht_mask, stream=stream)
    dyq = nvfp4_quantize_1d(dy, a_dy, rowwise=False, colwise=True, sr=True, rht=True,
                            rht_mask=rht_mask, seed=seed, stream=stream)
    a_x = nvfp4_amax(x, rht=True, rht_mask=rht_mask, stream=stream)
    xq = nvfp4_quantize_1d(x, a_x, rowwise=False, colwise=True, sr=x_sr, rht=True,
                           rht_mask=rht_mask, seed=seed, stream=stream)
    return dyq, xq


def wgrad(dy, x, rht_mask: int, seed: int, x_sr: bool = False, out_dtype=None, stream=None):
    """dW [out][in] = dY^T X from the Hadamard-transformed columnwise
    operands (the transform cancels in the product)."""
    tokens, n_out = dy.shape
    n_in = x.shape[1]
    dyq, xq = wgrad_operands(dy, x, rht_mask, seed, x_sr, stream)
    return nvfp4_gemm(dyq["codes_col"], dyq["scales_col"], SCALE_1D, dyq["global_scale"],
                      xq["codes_col"], xq["scales_col"], SCALE_1D, xq["global_scale"],
                      n_out, n_in, tokens, out_dtype=out_dtype, stream=stream)


def training_step(x, w, dy, rht_mask: int, seed: int, out_dtype=None, stream=None) -> dict:
    """One linear layer's forward and backward GEMMs with their
    quantizations: {"y", "dx", "dw", "wq"}."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    wq = quantize_weight(w, stream=stream)
    ws = nvfp4_workspace(x.device)
    y = fprop(x, wq, ws=ws, out_dtype=out_dtype, stream=stream)
    dx = dgrad(dy, wq, seed, ws=ws, out_dtype=out_dtype, stream=stream)
    dw = wgrad(dy, x, rht_mask, seed, out_dtype=out_dtype, stream=stream)
    return {"y": y, "dx": dx, "dw": dw, "wq": wq}
