"""GPU parity of the MXFP4 comparator format (E2M1 codes, one E8M0 scale per
32 elements) through the C ABI, against the CPU oracle.

Codes and scale bytes must match bit for bit (rowwise, columnwise, both in
one call, columnwise after the Hadamard transform), dequantization bit for
bit in binary32 and bf16, and the GEMM on the block-scaled matrix cores must
satisfy ||C - C_ref||_F / ||C_ref||_F <= 1e-5 (every row separately too)
against the double product of the exactly reconstructed operands. Every
byte is compared, at small and ragged shapes and at the full-size 8192x4096
activation and 8192x14336 gradient; the 8192x14336x4096 product on sampled
rows, in the launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

F = None
MASK = W.rht_sign_mask()


def setup_module(module):
    global F
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_block_scaled_amax_amd as pkg

    pkg.lib()  # raises if the HIP library is missing: no fallback
    F = pkg


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()


def to_gpu(a: np.ndarray) -> torch.Tensor:
    """An oracle-made array (codes, scales) on the device."""
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def special_tensor(R, C, seed):
    """Normal values with zeros, -0, bf16 subnormals, NaN, +-inf, values
    near the bf16 maximum and exact grid points planted in separate blocks."""
    x = W.normal_tensor(R, C, seed)
    x[0, 0:32] = 0                              # an all-zero block
    x[0, 40] = 0x8000                           # -0
    x[1, 0:32] = np.arange(1, 33, dtype=np.uint16)       # subnormal block
    x[2, 5] = 0x7FC0                            # NaN
    x[3, 70] = 0xFF80                           # -inf
    x[4, 0:32] = 0x7F7F                         # the bf16 maximum
    x[5, 0:32] = W.f32_to_bf16_bits(np.array([5.0, 3.0, 0.75, 0.25] * 8, np.float32))  # ties
    x[6:10, 32:64] = 0x3F80                     # constant 1.0 in a 4 x 32 patch
    return x


CASES = {
    "ragged_act": lambda: W.activation(160, 224, seed=60, n_outlier_cols=3),
    "ragged_grad": lambda: W.gradient(288, 96, seed=61),
    "weight": lambda: W.weight(256, 384, seed=62),
    "one_block": lambda: W.normal_tensor(32, 32, seed=63),
    "special": lambda: special_tensor(96, 160, seed=64),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("layouts", [(True, False), (False, True), (True, True)])
def test_quantize_matches_oracle(name, layouts):
    x = CASES[name]()
    row, col = layouts
    log(f"[test_mx_quantize] {name} {x.shape} row={row} col={col}")
    got = {k: host(v) for k, v in F.mxfp4_quantize(dev(x), rowwise=row, colwise=col).items()}
    if row:
        c, s = oracle.mx_quantize_rows(x)
        assert np.array_equal(got["scales_row"], s)
        assert np.array_equal(got["codes_row"], c)
    if col:
        c, s = oracle.mx_quantize_cols(x)
        assert np.array_equal(got["scales_col"], s)
        assert np.array_equal(got["codes_col"], c)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("mask", [MASK, 0])
def test_quantize_columnwise_hadamard_matches_oracle(name, mask):
    x = CASES[name]()
    log(f"[test_mx_quantize_rht] {name} {x.shape} mask={mask:#x}")
    got = {k: host(v) for k, v in F.mxfp4_quantize(dev(x), rowwise=False, colwise=True, rht=True,
                                                    rht_mask=mask).items()}
    c, s = oracle.mx_quantize_cols(x, rht=True, mask=mask)
    assert np.array_equal(got["scales_col"], s)
    assert_codes_equal_up_to_nan_signs(got["codes_col"], c, oracle.rht16_tensor(x, 0, mask).T)


def unpack(codes):
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


def assert_codes_equal_up_to_nan_signs(got, want, values):
    """Bit-exact codes, except the sign bit of elements whose transformed
    value is NaN: IEEE arithmetic leaves the sign of a NaN produced by an
    addition unspecified (the host keeps an operand's, the GPU gives the
    default NaN), so those codes (magnitude 0) are compared by magnitude."""
    g, w = unpack(got), unpack(want)
    nan = np.isnan(values)
    assert np.array_equal(g & 7, w & 7)
    assert np.array_equal(g[~nan], w[~nan])


def test_quantize_layout_specific_shapes():
    """Rowwise needs only cols % 32 (rows ragged against the 128-row tile);
    columnwise needs rows % 32 and cols % 8 (here 40 columns)."""
    x = W.activation(272, 96, seed=65, n_outlier_cols=1)
    got = F.mxfp4_quantize(dev(x))
    c, s = oracle.mx_quantize_rows(x)
    assert np.array_equal(host(got["codes_row"]), c) and np.array_equal(host(got["scales_row"]), s)
    x = W.gradient(64, 40, seed=66)
    for rht in (False, True):
        got = F.mxfp4_quantize(dev(x), rowwise=False, colwise=True, rht=rht, rht_mask=MASK)
        c, s = oracle.mx_quantize_cols(x, rht=rht, mask=MASK)
        assert np.array_equal(host(got["codes_col"]), c) and np.array_equal(host(got["scales_col"]), s)


def test_quantize_full_activation():
    """8192 x 4096 activation, both layouts in one call: every byte against
    the oracle (threaded over row and column ranges)."""
    x = W.activation()
    log("[test_mx_quantize_full] 8192x4096 activation, row+col")
    q = F.mxfp4_quantize(dev(x), rowwise=True, colwise=True)
    cr, sr, cc, sc = (host(q[k]) for k in ("codes_row", "scales_row", "codes_col", "scales_col"))
    c, s = oracle.mx_quantize_rows_mt(x)
    assert np.array_equal(cr, c) and np.array_equal(sr, s)
    c, s = oracle.mx_quantize_cols_mt(x)
    assert np.array_equal(cc, c) and np.array_equal(sc, s)


def test_quantize_full_gradient_hadamard():
    x = W.gradient()
    log("[test_mx_quantize_full] 8192x14336 gradient, columnwise + Hadamard")
    q = F.mxfp4_quantize(dev(x), rowwise=False, colwise=True, rht=True, rht_mask=MASK)
    cc, sc = host(q["codes_col"]), host(q["scales_col"])
    c, s = oracle.mx_quantize_cols_mt(x, rht=True, mask=MASK)
    assert np.array_equal(cc, c) and np.array_equal(sc, s)


@pytest.mark.parametrize("name", ["ragged_act", "special"])
def test_dequantize_bit_exact(name):
    x = CASES[name]()
    R, C = x.shape
    codes, scales = oracle.mx_quantize_rows(x)     # the oracle's bytes, decoded on the GPU
    cd, sd = to_gpu(codes), to_gpu(scales)
    want = oracle.mx_dequantize(codes, scales, R, C)
    got32 = host(F.mxfp4_dequantize(cd, sd, R, C))
    assert np.array_equal(got32.view(np.uint32), want.view(np.uint32))
    got16 = host(F.mxfp4_dequantize(cd, sd, R, C, out_dtype=torch.bfloat16).view(torch.int16)).view(np.uint16)
    nan = np.isnan(want)
    assert np.array_equal(got16[~nan], (want.view(np.uint32)[~nan] >> 16).astype(np.uint16))
    assert np.all((got16[nan] & 0x7F80) == 0x7F80) and np.all(got16[nan] & 0x7F)


def test_dequantize_every_code_and_scale_byte():
    """All 16 codes under every scale byte 0..254 and 0xFF."""
    R, C = 256, 32
    # elements 0..15 and 16..31 of every row are the codes 0..15 in order
    codes = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] * 2, np.uint8), (R, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(R, 1)
    want = oracle.mx_dequantize(codes, scales, R, C)
    got = host(F.mxfp4_dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), R, C))
    both = ~np.isnan(want)
    assert np.array_equal(got[both].view(np.uint32), want[both].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(want))


# ------------------------------------------------------------------ GEMM

def gemm_check(a, b, rows, out_dtype=None):
    """The oracle's MXFP4 operands multiplied on the GPU, against the
    oracle's double product of the same operands."""
    M, K = a.shape
    N = b.shape[0]
    ac, as_ = oracle.mx_quantize_rows(a)
    bc, bs = oracle.mx_quantize_rows(b)
    c = F.mxfp4_gemm(to_gpu(ac), to_gpu(as_), to_gpu(bc), to_gpu(bs), M, N, K, out_dtype=out_dtype)
    if out_dtype == torch.bfloat16:
        c = W.bf16_bits_to_f32(host(c.view(torch.int16)).view(np.uint16))
    else:
        c = host(c)
    ref = oracle.mx_gemm_rows(ac, as_, bc, bs, M, N, K, np.asarray(rows))
    got = c[np.asarray(rows)].astype(np.float64)
    err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    row_err = np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return err, row_err.max(), c


@pytest.mark.parametrize("M,N,K", [
    (272, 528, 1024),    # ragged tiles, K a multiple of 128 (one scale word per stage)
    (272, 528, 800),     # K = 25 blocks: a partial last stage
    (5, 7, 32),          # one block, one partial tile
    (300, 40, 4160),     # long K, N under one fragment width
])
def test_gemm_matches_double_reference(M, N, K):
    log(f"[test_mx_gemm] {M}x{N}x{K}")
    a = W.activation(M, K, seed=70, n_outlier_cols=2) if M >= 8 else W.normal_tensor(M, K, seed=70)
    b = W.weight(N, K, seed=71)
    err, row_err, _ = gemm_check(a, b, np.arange(M))
    log(f"[test_mx_gemm] rel_fro={err:.3e} worst row {row_err:.3e}")
    assert err <= 1e-5 and row_err <= 1e-5


def test_gemm_more_tiles_than_workgroups():
    """More 256 x 256 tiles than resident workgroups (each walks several)."""
    M, N, K = 2064, 8208, 96   # 9 x 33 = 297 tiles
    a = W.normal_tensor(M, K, seed=72)
    b = W.normal_tensor(N, K, seed=73, std=0.02)
    err, row_err, _ = gemm_check(a, b, np.arange(M))
    assert err <= 1e-5 and row_err <= 1e-5


def test_gemm_full_size_sampled_rows():
    log("[test_mx_gemm_full] 8192x14336x4096")
    a, b = W.gemm_operands()
    err, row_err, _ = gemm_check(a, b, W.gemm_sample_rows())
    log(f"[test_mx_gemm_full] rel_fro={err:.3e} worst row {row_err:.3e}")
    assert err <= 1e-5 and row_err <= 1e-5


def test_gemm_bf16_output_is_rounded_fp32():
    a = W.normal_tensor(272, 544, seed=74)
    b = W.normal_tensor(400, 544, seed=75, std=0.02)
    _, _, c32 = gemm_check(a, b, np.arange(8))
    err16, _, c16 = gemm_check(a, b, np.arange(272), out_dtype=torch.bfloat16)
    assert np.array_equal(W.f32_to_bf16_bits(c32), W.f32_to_bf16_bits(c16))
    assert err16 <= 2.0 ** -8


def test_nvfp4_quantizes_with_less_error_than_mxfp4_on_gpu():
    """The pages' claim, on the library's own outputs for the activation
    (rowwise) and the gradient (columnwise after the Hadamard transform)."""
    x = W.activation(1024, 4096, seed=76)
    xd = dev(x)
    xf = torch.from_numpy(W.bf16_bits_to_f32(x)).cuda().double()
    q = F.nvfp4_quantize_1d(xd, F.nvfp4_amax(xd))
    nv = F.nvfp4_dequantize(q["codes_row"], q["scales_row"], 1, q["global_scale"], 1024, 4096).double()
    m = F.mxfp4_quantize(xd)
    mx = F.mxfp4_dequantize(m["codes_row"], m["scales_row"], 1024, 4096).double()
    e_nv = float(torch.linalg.norm(nv - xf) / torch.linalg.norm(xf))
    e_mx = float(torch.linalg.norm(mx - xf) / torch.linalg.norm(xf))
    log(f"[test_mx_error] activation rowwise: nvfp4 {e_nv:.4f} mxfp4 {e_mx:.4f}")
    assert e_nv < e_mx
