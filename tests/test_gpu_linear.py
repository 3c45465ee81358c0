"""GPU: the NVFP4 linear layer composed from the library (fprop, dgrad,
wgrad), each GEMM against the double-precision product of its exactly
reconstructed operands (||C - C_ref||_F / ||C_ref||_F <= 1e-5), each
operand's codes and scales against the oracle bit for bit, and the layer's
outputs against the unquantized products within the format's error (which
also shows the Hadamard transform cancelling in dW)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

F = None
L = None

# tokens, in, out: multiples of 16, ragged against the GEMM's 256 x 256 tiles
T, N_IN, N_OUT = 272, 528, 784
SEED = 42


def setup_module(module):
    global F, L
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_block_scaled_amax_amd as pkg
    from fp4_block_scaled_amax_amd import linear

    pkg.lib()  # raises if the HIP library is missing: no fallback
    F, L = pkg, linear


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def tensors():
    x = W.activation(T, N_IN, seed=31, n_outlier_cols=2)
    w = W.weight(N_OUT, N_IN, seed=32)
    dy = W.gradient(T, N_OUT, seed=33)
    return x, w, dy


def rel_fro(c, ref):
    return np.linalg.norm(c.astype(np.float64) - ref) / np.linalg.norm(ref)


def recon(codes, scales, mode, sg, R, C):
    """Double reconstruction by the oracle of oracle-made codes and scales."""
    return oracle.dequantize_f64_rows(codes, scales, mode, sg, R, C, np.arange(R, dtype=np.int64))


def to_gpu(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def sg_gpu(sg) -> torch.Tensor:
    return torch.tensor([float(np.float32(sg))], dtype=torch.float32, device="cuda")


def f32_bits(a) -> int:
    return int(np.float32(a).view(np.uint32))


def test_fprop():
    x, w, _ = tensors()
    log("[test_linear] fprop")
    xd, wd = dev(x), dev(w)
    wq = L.quantize_weight(wd)
    y = host(L.fprop(xd, wq))
    # the operands are the library's own quantizations, equal to the oracle's
    xq = F.nvfp4_quantize_1d(xd, F.nvfp4_amax(xd), rowwise=True)
    sg = oracle.global_scale(oracle.amax(x))
    c, s = oracle.quantize_1d_rows(x, sg)
    assert np.array_equal(host(xq["codes_row"]), c) and np.array_equal(host(xq["scales_row"]), s)
    assert f32_bits(host(xq["global_scale"])[0]) == f32_bits(sg)
    sgw = oracle.global_scale(oracle.amax(w))
    cr, cc, s2 = oracle.quantize_2d(w, sgw)
    assert np.array_equal(host(wq["scales"]), s2)
    assert np.array_equal(host(wq["codes_row"]), cr) and np.array_equal(host(wq["codes_col"]), cc)
    assert f32_bits(host(wq["global_scale"])[0]) == f32_bits(sgw)
    # so the reference is the oracle's product of the oracle's operands
    ref = recon(c, s, 1, sg, T, N_IN) @ recon(cr, s2, 2, sgw, N_OUT, N_IN).T
    assert rel_fro(y, ref) <= 1e-5
    exact = W.bf16_bits_to_f32(x).astype(np.float64) @ W.bf16_bits_to_f32(w).astype(np.float64).T
    assert rel_fro(y, exact) < 0.15  # 4-bit operands


def test_dgrad_reads_the_weight_column_copy():
    x, w, dy = tensors()
    log("[test_linear] dgrad")
    wd, dyd = dev(w), dev(dy)
    wq = L.quantize_weight(wd)
    dx = host(L.dgrad(dyd, wq, SEED))
    dyq = F.nvfp4_quantize_1d(dyd, F.nvfp4_amax(dyd), rowwise=True, sr=True, seed=SEED)
    sg = oracle.global_scale(oracle.amax(dy))
    c, s = oracle.quantize_1d_rows(dy, sg, True, SEED)
    assert np.array_equal(host(dyq["codes_row"]), c) and np.array_equal(host(dyq["scales_row"]), s)
    assert f32_bits(host(dyq["global_scale"])[0]) == f32_bits(sg)
    sgw = oracle.global_scale(oracle.amax(w))
    cr, _, s2 = oracle.quantize_2d(w, sgw)
    assert np.array_equal(host(wq["codes_row"]), cr) and np.array_equal(host(wq["scales"]), s2)
    assert f32_bits(host(wq["global_scale"])[0]) == f32_bits(sgw)
    ref = recon(c, s, 1, sg, T, N_OUT) @ recon(cr, s2, 2, sgw, N_OUT, N_IN)
    assert rel_fro(dx, ref) <= 1e-5
    # the column copy holds the same codes, transposed (one code per element)
    lo_hi = lambda a: np.stack([a & 15, a >> 4], -1).reshape(a.shape[0], -1)
    assert np.array_equal(lo_hi(host(wq["codes_col"])), lo_hi(host(wq["codes_row"])).T)
    exact = W.bf16_bits_to_f32(dy).astype(np.float64) @ W.bf16_bits_to_f32(w).astype(np.float64)
    assert rel_fro(dx, exact) < 0.2


def test_transposed_tile_grid_and_dgrad_operand_modes_agree():
    """nvfp4_quantize_2d_tscales writes the oracle's tile scales transposed;
    the column copy read as a 2D operand with them gives the product of the
    NVFP4_SCALE_2D_T reading bit for bit (K = 14336 past the LDS-staged K,
    and a small K that stages)."""
    for (tok, n_out, n_in) in ((256, 14336, 512), (T, N_OUT, N_IN)):
        w = W.weight(n_out, n_in, seed=39)
        dy = W.gradient(tok, n_out, seed=40)
        wq = L.quantize_weight(dev(w))
        cr, cc, s2 = oracle.quantize_2d(w, oracle.global_scale(oracle.amax(w)))
        assert np.array_equal(host(wq["scales"]), s2)
        assert np.array_equal(host(wq["scales_t"]), np.ascontiguousarray(s2.T))
        dyq = F.nvfp4_quantize_1d(dev(dy), F.nvfp4_amax(dev(dy)), sr=True, seed=SEED)
        args = (dyq["codes_row"], dyq["scales_row"], 1, dyq["global_scale"], wq["codes_col"])
        c2 = host(F.nvfp4_gemm(*args, wq["scales_t"], F.SCALE_2D, wq["global_scale"], tok, n_in, n_out))
        c3 = host(F.nvfp4_gemm(*args, wq["scales"], F.SCALE_2D_T, wq["global_scale"], tok, n_in, n_out))
        assert np.array_equal(c2.view(np.uint32), c3.view(np.uint32))


def test_gemm_transposed_tile_scales_match_dequantized_reference():
    """NVFP4_SCALE_2D_T on either operand, with K not a multiple of 32."""
    w = W.weight(N_OUT, 784, seed=34)  # the operand's K is N_OUT = 784 = 24.5 x 32
    a = W.activation(T, N_OUT, seed=35, n_outlier_cols=1)
    sgw = oracle.global_scale(oracle.amax(w))
    wr, wc, ws = oracle.quantize_2d(w, sgw)         # [784][784]: the column copy is W^T
    sga = oracle.global_scale(oracle.amax(a))
    ac, as_ = oracle.quantize_1d_rows(a, sga)
    w_hat_t = recon(wr, ws, 2, sgw, 784, 784).T
    a_hat = recon(ac, as_, 1, sga, T, N_OUT)
    wcd, wsd, wgd = to_gpu(wc), to_gpu(ws), sg_gpu(sgw)
    acd, asd, agd = to_gpu(ac), to_gpu(as_), sg_gpu(sga)
    c = host(F.nvfp4_gemm(acd, asd, 1, agd, wcd, wsd, F.SCALE_2D_T, wgd, T, 784, 784))
    assert rel_fro(c, a_hat @ w_hat_t.T) <= 1e-5
    c2 = host(F.nvfp4_gemm(wcd, wsd, F.SCALE_2D_T, wgd, acd, asd, 1, agd, 784, T, 784))
    assert rel_fro(c2, w_hat_t @ a_hat.T) <= 1e-5


@pytest.mark.parametrize("x_sr", [False, True])
def test_wgrad_hadamard_operands_cancel(x_sr):
    x, _, dy = tensors()
    log(f"[test_linear] wgrad x_sr={x_sr}")
    xd, dyd = dev(x), dev(dy)
    mask = W.rht_sign_mask()
    dw = host(L.wgrad(dyd, xd, mask, SEED, x_sr=x_sr))
    dyq, xq = L.wgrad_operands(dyd, xd, mask, SEED, x_sr=x_sr)
    hats = []
    for t, q, sr in ((dy, dyq, True), (x, xq, x_sr)):
        sg = oracle.global_scale(oracle.amax_rht(t, mask))
        c, s = oracle.quantize_1d_cols(t, sg, sr, SEED, True, mask)
        assert np.array_equal(host(q["codes_col"]), c) and np.array_equal(host(q["scales_col"]), s)
        assert f32_bits(host(q["global_scale"])[0]) == f32_bits(sg)
        hats.append(recon(c, s, 1, sg, t.shape[1], T))
    ref = hats[0] @ hats[1].T
    assert rel_fro(dw, ref) <= 1e-5
    # (H D dY)^T (H D X) / 16 = dY^T X: the transform cancels
    exact = W.bf16_bits_to_f32(dy).astype(np.float64).T @ W.bf16_bits_to_f32(x).astype(np.float64)
    assert rel_fro(dw, exact) < 0.2


def test_wgrad_with_mismatched_masks_does_not_cancel():
    """Control for the cancellation check: different sign masks on the two
    operands leave a product far from dY^T X."""
    x, _, dy = tensors()
    xd, dyd = dev(x), dev(dy)
    mask = W.rht_sign_mask()
    a_dy = F.nvfp4_amax(dyd, rht=True, rht_mask=mask)
    dyq = F.nvfp4_quantize_1d(dyd, a_dy, rowwise=False, colwise=True, sr=True, rht=True, rht_mask=mask, seed=SEED)
    a_x = F.nvfp4_amax(xd, rht=True, rht_mask=mask ^ 0x0F0F)
    xq = F.nvfp4_quantize_1d(xd, a_x, rowwise=False, colwise=True, rht=True, rht_mask=mask ^ 0x0F0F)
    dw = host(F.nvfp4_gemm(dyq["codes_col"], dyq["scales_col"], 1, dyq["global_scale"],
                           xq["codes_col"], xq["scales_col"], 1, xq["global_scale"], N_OUT, N_IN, T))
    exact = W.bf16_bits_to_f32(dy).astype(np.float64).T @ W.bf16_bits_to_f32(x).astype(np.float64)
    assert rel_fro(dw, exact) > 0.5


def test_training_step_outputs():
    x, w, dy = tensors()
    out = L.training_step(dev(x), dev(w), dev(dy), W.rht_sign_mask(), SEED, out_dtype=torch.bfloat16)
    assert tuple(out["y"].shape) == (T, N_OUT) and out["y"].dtype == torch.bfloat16
    assert tuple(out["dx"].shape) == (T, N_IN)
    assert tuple(out["dw"].shape) == (N_OUT, N_IN)
    for k in ("y", "dx", "dw"):
        assert torch.isfinite(out[k].float()).all()


def quantize_operand_2d(x):
    """2D codes and tile scales of a [R][K] operand, and its double reconstruction."""
    sg = oracle.global_scale(oracle.amax(x))
    codes, _, scales = oracle.quantize_2d(x, sg)
    return codes, scales, sg, recon(codes, scales, 2, sg, x.shape[0], x.shape[1])


@pytest.mark.parametrize("mode, K, a_mode", [(2, 16400, 1), (3, 16400, 1), (2, 16448, 1), (3, 16448, 1),
                                              (2, 16400, 2)])
def test_gemm_2d_scales_beyond_the_lds_staged_k(mode, K, a_mode):
    """2D and transposed 2D B operands around the K whose tile scales a
    workgroup stages in LDS. With 32-deep stages (K = 16400, an odd multiple
    of 16) the region holds 16384 scale columns per operand, twice that for a
    lone 2D operand: a 1D A keeps B staged, a 2D A (both operands 2D) sends
    both to the per-row scale loads. With 64-deep stages (K = 16448) a lone 2D
    operand is staged up to K = 16384, so B takes the per-row loads."""
    M, N = 48, 64
    a = W.activation(M, K, seed=36, n_outlier_cols=1)
    if a_mode == 1:
        sga = oracle.global_scale(oracle.amax(a))
        ac, as_ = oracle.quantize_1d_rows(a, sga)
        a_hat = recon(ac, as_, 1, sga, M, K)
    else:
        ac, as_, sga, a_hat = quantize_operand_2d(a)
    if mode == 2:
        w = W.weight(N, K, seed=37)                     # B = W [N][K], 2D scales [N/16][K/16]
        sgw = oracle.global_scale(oracle.amax(w))
        b_codes, _, b_scales = oracle.quantize_2d(w, sgw)
        b_hat = recon(b_codes, b_scales, 2, sgw, N, K)
    else:
        w = W.weight(K, N, seed=38)                     # B = W^T: W's column copy, scales [K/16][N/16]
        sgw = oracle.global_scale(oracle.amax(w))
        w_rows, b_codes, b_scales = oracle.quantize_2d(w, sgw)
        b_hat = recon(w_rows, b_scales, 2, sgw, K, N).T
    c = host(F.nvfp4_gemm(to_gpu(ac), to_gpu(as_), a_mode, sg_gpu(sga),
                          to_gpu(b_codes), to_gpu(b_scales), mode, sg_gpu(sgw), M, N, K))
    assert rel_fro(c, a_hat @ b_hat.T) <= 1e-5
