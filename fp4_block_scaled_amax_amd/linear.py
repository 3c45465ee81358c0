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
2D tiles, so its two copies hold identical codes and the same tile scales;
the quantizer also writes the tile grid transposed, under which the
columnwise copy is a plain 2D-scaled dgrad operand with contiguous scale
reads (NVFP4_SCALE_2D_T on the untransposed grid gives the same product).

Fused passes: dY's two amaxes (plain, for its rowwise dgrad operand, and of
its Hadamard transform, for its columnwise wgrad operand) come from one read
of dY (nvfp4_amax with both=True), and the forward can hand its output to
the next layer already quantized, the output's amax reduced in the GEMM's
epilogue (forward_quantized) so the quantization reads Y once; with the amax
known beforehand (the layer's previous max |Y|), the GEMM's epilogue
quantizes Y itself and Y never reaches memory (forward_quantized_delayed).

Every step runs in the library's kernels; this module only sequences calls
on one stream. Shapes: x [tokens][in], w [out][in], dy [tokens][out], all
bf16 bit patterns (int16/uint16 tensors), every dimension a multiple of 16.
"""
from __future__ import annotations

from . import (SCALE_1D, SCALE_2D, SCALE_2D_T, _torch, nvfp4_amax, nvfp4_gemm, nvfp4_gemm_quantize,
               nvfp4_quantize_1d, nvfp4_quantize_1d_fused, nvfp4_quantize_2d, nvfp4_workspace)


def quantize_weight(w, stream=None) -> dict:
    """W [out][in] -> 2D-tiled NVFP4 in both layouts: codes_row [out][in/2],
    codes_col [in][out/2], scales [out/16][in/16], the same grid transposed
    scales_t [in/16][out/16], global_scale."""
    return nvfp4_quantize_2d(w, nvfp4_amax(w, stream=stream), rowwise=True, colwise=True,
                             stream=stream, transposed_scales=True)


def fprop(x, wq: dict, ws=None, out_dtype=None, stream=None):
    """Y [tokens][out] = X W^T: X rowwise 1D RNE (amax and quantization in
    one pass through the workspace `ws`, allocated if None)."""
    tokens, k = x.shape
    n = wq["codes_row"].shape[0]
    ws = nvfp4_workspace(x.device) if ws is None else ws
    xq = nvfp4_quantize_1d_fused(x, ws, rowwise=True, stream=stream)
    return nvfp4_gemm(xq["codes_row"], xq["scales_row"], SCALE_1D, xq["global_scale"],
                      wq["codes_row"], wq["scales"], SCALE_2D, wq["global_scale"],
                      tokens, n, k, out_dtype=out_dtype, stream=stream)


def forward_quantized(x, wq: dict, ws=None, stream=None):
    """Y = X W^T in bf16 and Y's own NVFP4 quantization for the next layer
    (rowwise and columnwise 1D, round-to-nearest-even): the GEMM's epilogue
    reduces max |Y| of the stored bf16 values, so the quantization takes it
    as its amax and reads Y once. Returns (y, yq)."""
    torch = _torch()
    tokens, k = x.shape
    n = wq["codes_row"].shape[0]
    ws = nvfp4_workspace(x.device) if ws is None else ws
    xq = nvfp4_quantize_1d_fused(x, ws, rowwise=True, stream=stream)
    y_amax = torch.empty(1, dtype=torch.float32, device=x.device)
    y = nvfp4_gemm(xq["codes_row"], xq["scales_row"], SCALE_1D, xq["global_scale"],
                   wq["codes_row"], wq["scales"], SCALE_2D, wq["global_scale"],
                   tokens, n, k, out_dtype=torch.bfloat16, stream=stream, out_amax=y_amax)
    yq = nvfp4_quantize_1d(y, y_amax, rowwise=True, colwise=True, stream=stream)
    return y, yq


def forward_quantized_delayed(x, wq: dict, y_amax, ws=None, stream=None, out_amax=None):
    """Y's NVFP4 quantization (rowwise and columnwise 1D, round to nearest
    even) made by the fprop GEMM's own epilogue, with the amax given (for
    instance the previous step's max |Y| of this layer): Y is never stored.
    Returns (yq, out_amax), out_amax = max |Y| of this product (float32 [1],
    allocated if not given), the amax for the next call. With y_amax equal to
    this product's own max |Y| the bytes equal forward_quantized's yq."""
    torch = _torch()
    tokens, k = x.shape
    n = wq["codes_row"].shape[0]
    ws = nvfp4_workspace(x.device) if ws is None else ws
    xq = nvfp4_quantize_1d_fused(x, ws, rowwise=True, stream=stream)
    if out_amax is None:
        out_amax = torch.empty(1, dtype=torch.float32, device=x.device)
    yq = nvfp4_gemm_quantize(xq["codes_row"], xq["scales_row"], SCALE_1D, xq["global_scale"],
                             wq["codes_row"], wq["scales"], SCALE_2D, wq["global_scale"],
                             tokens, n, k, y_amax, rowwise=True, colwise=True, out_amax=out_amax,
                             stream=stream)
    return yq, out_amax


def gradient_amaxes(dy, rht_mask: int, stream=None):
    """dY's plain amax and its Hadamard transform's, from one read: float32
    [2] (views [0:1] and [1:2] serve dgrad and wgrad)."""
    return nvfp4_amax(dy, rht=True, rht_mask=rht_mask, both=True, stream=stream)


def dgrad(dy, wq: dict, seed: int, ws=None, out_dtype=None, stream=None, dy_amax=None):
    """dX [tokens][in] = dY W: dY rowwise 1D stochastic (seed), W's
    columnwise copy with the transposed tile grid (a plain 2D operand; a wq
    without scales_t is read with NVFP4_SCALE_2D_T, same product). dy_amax:
    dY's amax if already known (gradient_amaxes(...)[0:1]); otherwise the
    call computes it."""
    tokens, k = dy.shape
    n = wq["codes_col"].shape[0]
    if dy_amax is not None:
        dyq = nvfp4_quantize_1d(dy, dy_amax, rowwise=True, sr=True, seed=seed, stream=stream)
    else:
        ws = nvfp4_workspace(dy.device) if ws is None else ws
        dyq = nvfp4_quantize_1d_fused(dy, ws, rowwise=True, sr=True, seed=seed, stream=stream)
    if "scales_t" in wq:
        b_scales, b_mode = wq["scales_t"], SCALE_2D
    else:
        b_scales, b_mode = wq["scales"], SCALE_2D_T
    return nvfp4_gemm(dyq["codes_row"], dyq["scales_row"], SCALE_1D, dyq["global_scale"],
                      wq["codes_col"], b_scales, b_mode, wq["global_scale"],
                      tokens, n, k, out_dtype=out_dtype, stream=stream)


def wgrad_operands(dy, x, rht_mask: int, seed: int, x_sr: bool = False, stream=None,
                   dy_amax_rht=None):
    """The two columnwise operands of dW = dY^T X, blocks along the tokens,
    after the Hadamard transform with the shared sign mask: dY stochastic,
    X round-to-nearest-even (or stochastic with x_sr). dy_amax_rht: the
    transform's amax of dY if already known (gradient_amaxes(...)[1:2])."""
    a_dy = nvfp4_amax(dy, rht=True, rht_mask=rht_mask, stream=stream) if dy_amax_rht is None else dy_amax_rht
    dyq = nvfp4_quantize_1d(dy, a_dy, rowwise=False, colwise=True, sr=True, rht=True,
                            rht_mask=rht_mask, seed=seed, stream=stream)
    a_x = nvfp4_amax(x, rht=True, rht_mask=rht_mask, stream=stream)
    xq = nvfp4_quantize_1d(x, a_x, rowwise=False, colwise=True, sr=x_sr, rht=True,
                           rht_mask=rht_mask, seed=seed, stream=stream)
    return dyq, xq


def wgrad(dy, x, rht_mask: int, seed: int, x_sr: bool = False, out_dtype=None, stream=None,
          dy_amax_rht=None):
    """dW [out][in] = dY^T X from the Hadamard-transformed columnwise
    operands (the transform cancels in the product)."""
    tokens, n_out = dy.shape
    n_in = x.shape[1]
    dyq, xq = wgrad_operands(dy, x, rht_mask, seed, x_sr, stream, dy_amax_rht)
    return nvfp4_gemm(dyq["codes_col"], dyq["scales_col"], SCALE_1D, dyq["global_scale"],
                      xq["codes_col"], xq["scales_col"], SCALE_1D, xq["global_scale"],
                      n_out, n_in, tokens, out_dtype=out_dtype, stream=stream)


def training_step(x, w, dy, rht_mask: int, seed: int, out_dtype=None, stream=None) -> dict:
    """One linear layer's forward and backward GEMMs with their
    quantizations: {"y", "dx", "dw", "wq"}. dY is read once for both of its
    amaxes."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    wq = quantize_weight(w, stream=stream)
    ws = nvfp4_workspace(x.device)
    y = fprop(x, wq, ws=ws, out_dtype=out_dtype, stream=stream)
    a_dy = gradient_amaxes(dy, rht_mask, stream=stream)
    dx = dgrad(dy, wq, seed, out_dtype=out_dtype, stream=stream, dy_amax=a_dy[0:1])
    dw = wgrad(dy, x, rht_mask, seed, out_dtype=out_dtype, stream=stream, dy_amax_rht=a_dy[1:2])
    return {"y": y, "dx": dx, "dw": dw, "wq": wq}
