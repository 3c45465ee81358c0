"""GPU: the fused passes of the linear layer, against the oracle and
against the unfused calls.

- nvfp4_amax with NVFP4_RHT | NVFP4_AMAX_BOTH: the plain amax and the
  Hadamard transform's from one read, each bit-equal to the oracle's.
- nvfp4_gemm_amax: the GEMM's epilogue reduces max |C| of the stored values;
  C is bit-identical to nvfp4_gemm's and the amax bit-equal to nvfp4_amax of
  C (bf16) or the host maximum (fp32).
- nvfp4_gemm_quantize: the GEMM's epilogue quantizes the bf16 product with a
  given amax instead of storing it; every output byte equals the unfused
  nvfp4_gemm (bf16) + nvfp4_quantize_1d with that amax and the oracle's
  quantization of that bf16 product, for the true amax, a smaller one
  (saturating blocks) and a larger one; its reported amax is max |Y|.
- linear.forward_quantized: Y's quantization from the epilogue amax equals
  the oracle's quantization of Y; linear.training_step (one read of dY for
  both amaxes) equals the calls composed without the fusion, bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

F = None
L = None
MASK = W.rht_sign_mask()


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


def host16(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.int16)).view(np.uint16)


def bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


def special(R, C, seed, what):
    x = W.gradient(R, C, seed=seed)
    if what == "nan":
        x[R // 2, C // 3] = 0x7FC0
    if what == "inf":
        x[3, 5] = 0xFF80
    if what == "zeros":
        x[:] = 0
    return x


AMAX_CASES = {
    "activation": lambda: W.activation(512, 1024, seed=80, n_outlier_cols=4),
    "gradient_ragged": lambda: W.gradient(304, 400, seed=81),
    "gradient_full": lambda: W.gradient(),
    "nan": lambda: special(64, 96, 82, "nan"),
    "inf": lambda: special(64, 96, 83, "inf"),
    "zeros": lambda: special(32, 48, 84, "zeros"),
}


@pytest.mark.parametrize("name", list(AMAX_CASES))
def test_amax_both_from_one_read(name):
    x = AMAX_CASES[name]()
    log(f"[test_amax_both] {name} {x.shape}")
    a = host(F.nvfp4_amax(dev(x), rht=True, rht_mask=MASK, both=True))
    plain, rht = oracle.amax(x), oracle.amax_rht(x, MASK)
    if np.isnan(plain):
        assert np.isnan(a[0]) and np.isnan(a[1])
        return
    assert bits(a[0]) == bits(plain)
    if np.isnan(rht):
        assert np.isnan(a[1])
    else:
        assert bits(a[1]) == bits(rht)
    # the single-amax calls agree
    assert bits(host(F.nvfp4_amax(dev(x)))[0]) == bits(a[0])


@pytest.mark.parametrize("M,N,K", [(272, 400, 528), (2064, 8208, 48), (8192, 14336, 4096)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gemm_amax_epilogue(M, N, K, dtype):
    log(f"[test_gemm_amax] {M}x{N}x{K} {dtype}")
    a = W.normal_tensor(M, K, seed=85)
    b = W.normal_tensor(N, K, seed=86, std=0.02)
    ad, bd = dev(a), dev(b)
    qa = F.nvfp4_quantize_1d(ad, F.nvfp4_amax(ad))
    qb = F.nvfp4_quantize_2d(bd, F.nvfp4_amax(bd), colwise=False)
    args = (qa["codes_row"], qa["scales_row"], 1, qa["global_scale"], qb["codes_row"], qb["scales"], 2,
            qb["global_scale"], M, N, K)
    ref = F.nvfp4_gemm(*args, out_dtype=dtype)
    amax = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")  # reset by the call
    c = F.nvfp4_gemm(*args, out_dtype=dtype, out_amax=amax)
    if dtype == torch.bfloat16:
        cb, rb = host16(c), host16(ref)
        assert np.array_equal(cb, rb)
        assert bits(host(amax)[0]) == bits(host(F.nvfp4_amax(c))[0])
        # max |C| by definition: the largest bf16 magnitude pattern, widened
        assert bits(host(amax)[0]) == int((cb & 0x7FFF).max()) << 16
    else:
        cf, rf = host(c), host(ref)
        assert np.array_equal(cf.view(np.uint32), rf.view(np.uint32))
        assert bits(host(amax)[0]) == int((cf.view(np.uint32) & 0x7FFFFFFF).max())


def test_forward_quantized_equals_the_unfused_quantization_of_y():
    """The epilogue amax and the quantization of Y that uses it give the
    same bytes as quantizing the plain fprop output with the library's own
    amax + quantize calls (whose agreement with the oracle is tested on
    generated inputs), and the amax is max |Y| by definition."""
    T, N_IN, N_OUT = 272, 528, 784
    x = W.activation(T, N_IN, seed=87, n_outlier_cols=2)
    w = W.weight(N_OUT, N_IN, seed=88)
    wq = L.quantize_weight(dev(w))
    y, yq = L.forward_quantized(dev(x), wq)
    yb = host16(y)
    # Y itself is the plain fprop's output
    y_plain = L.fprop(dev(x), wq, out_dtype=torch.bfloat16)
    assert np.array_equal(yb, host16(y_plain))
    a = F.nvfp4_amax(y_plain)
    assert bits(host(a)[0]) == int((yb & 0x7FFF).max()) << 16
    ref = F.nvfp4_quantize_1d(y_plain, a, rowwise=True, colwise=True)
    for k in ("global_scale", "codes_row", "scales_row", "codes_col", "scales_col"):
        assert np.array_equal(host(yq[k]), host(ref[k])), k


def test_training_step_equals_unfused_calls():
    T, N_IN, N_OUT = 272, 528, 784
    x = W.activation(T, N_IN, seed=89, n_outlier_cols=2)
    w = W.weight(N_OUT, N_IN, seed=90)
    dy = W.gradient(T, N_OUT, seed=91)
    xd, wd, dyd = dev(x), dev(w), dev(dy)
    out = L.training_step(xd, wd, dyd, MASK, 42)
    wq = L.quantize_weight(wd)
    y = L.fprop(xd, wq)
    dx = L.dgrad(dyd, wq, 42)                    # its own amax (fused single-pass quantize)
    dw = L.wgrad(dyd, xd, MASK, 42)              # its own transform amax
    for k, ref in (("y", y), ("dx", dx), ("dw", dw)):
        assert np.array_equal(host(out[k]).view(np.uint32), host(ref).view(np.uint32)), k


GQ_CASES = [
    # (M, N, K, b_scale_mode, layouts)
    (272, 400, 528, 2, "both"),     # ragged tiles in M and N, 64-deep stages
    (2064, 8208, 48, 1, "both"),    # K an odd multiple of 16 (32-deep stages, one-block tail)
    (528, 784, 96, 1, "row"),
    (528, 784, 96, 2, "col"),
    (256, 256, 64, 2, "both"),      # one whole tile
    (8192, 14336, 4096, 2, "both"),  # the linear layer's fprop shape
]


@pytest.mark.parametrize("M,N,K,bmode,layouts", GQ_CASES)
def test_gemm_quantize_epilogue(M, N, K, bmode, layouts):
    log(f"[test_gemm_quantize_epilogue] {M}x{N}x{K} b_mode {bmode} {layouts}")
    rowwise, colwise = layouts in ("both", "row"), layouts in ("both", "col")
    a = W.normal_tensor(M, K, seed=92)
    b = W.normal_tensor(N, K, seed=93, std=0.02)
    ad, bd = dev(a), dev(b)
    qa = F.nvfp4_quantize_1d(ad, F.nvfp4_amax(ad))
    if bmode == 2:
        qb = F.nvfp4_quantize_2d(bd, F.nvfp4_amax(bd), colwise=False)
        bc, bs = qb["codes_row"], qb["scales"]
    else:
        qb = F.nvfp4_quantize_1d(bd, F.nvfp4_amax(bd))
        bc, bs = qb["codes_row"], qb["scales_row"]
    args = (qa["codes_row"], qa["scales_row"], 1, qa["global_scale"], bc, bs, bmode, qb["global_scale"], M, N, K)
    y = F.nvfp4_gemm(*args, out_dtype=torch.bfloat16)
    y_amax = F.nvfp4_amax(y)
    yh = host16(y)
    for scale_by in (1.0, 0.25, 3.0):
        # the oracle over every element (at the largest shape for the true amax only)
        full = M * N <= 40 << 20 or scale_by == 1.0
        given = y_amax * scale_by
        out_amax = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        got = F.nvfp4_gemm_quantize(*args, given, rowwise=rowwise, colwise=colwise, out_amax=out_amax)
        ref = F.nvfp4_quantize_1d(y, given, rowwise=rowwise, colwise=colwise)
        keys = ["global_scale"] + (["codes_row", "scales_row"] if rowwise else []) + \
            (["codes_col", "scales_col"] if colwise else [])
        for k in keys:
            assert np.array_equal(host(got[k]), host(ref[k])), (k, scale_by)
        assert bits(host(out_amax)[0]) == bits(host(y_amax)[0])
        sg = oracle.global_scale(np.float32(host(given)[0]))
        assert bits(host(got["global_scale"])[0]) == bits(sg)
        if full:
            if rowwise:
                c, s_ = oracle.quantize_1d_rows_mt(yh, sg)
                assert np.array_equal(host(got["codes_row"]), c) and np.array_equal(host(got["scales_row"]), s_)
            if colwise:
                c, s_ = oracle.quantize_1d_cols_mt(yh, sg)
                assert np.array_equal(host(got["codes_col"]), c) and np.array_equal(host(got["scales_col"]), s_)
        else:
            rows = np.arange(0, M, 61)
            c, s_ = oracle.quantize_1d_rows(yh[rows], sg)
            assert np.array_equal(host(got["codes_row"])[rows], c) and np.array_equal(host(got["scales_row"])[rows], s_)


def test_forward_quantized_delayed_equals_forward_quantized():
    """With the amax from a first call, the epilogue-quantized forward gives
    forward_quantized's bytes, and reports the same max |Y|."""
    T, N_IN, N_OUT = 272, 528, 784
    x = W.activation(T, N_IN, seed=94, n_outlier_cols=2)
    w = W.weight(N_OUT, N_IN, seed=95)
    xd = dev(x)
    wq = L.quantize_weight(dev(w))
    y, yq = L.forward_quantized(xd, wq)
    y_amax = F.nvfp4_amax(y)
    dq, out_amax = L.forward_quantized_delayed(xd, wq, y_amax)
    assert bits(host(out_amax)[0]) == bits(host(y_amax)[0])
    for k in ("global_scale", "codes_row", "scales_row", "codes_col", "scales_col"):
        assert np.array_equal(host(dq[k]), host(yq[k])), k


@pytest.mark.parametrize("given", [0.0, float("inf"), float("nan"), 1e-30])
def test_gemm_quantize_epilogue_degenerate_amax(given):
    """A given amax of 0, infinity, NaN or a tiny value: the epilogue's bytes
    still equal nvfp4_quantize_1d's of the bf16 product with that amax (both
    run the same item code, here down its exact and non-finite paths)."""
    M, N, K = 272, 400, 96
    log(f"[test_gemm_quantize_epilogue_degenerate_amax] amax {given}")
    a = W.normal_tensor(M, K, seed=96)
    b = W.normal_tensor(N, K, seed=97, std=0.02)
    ad, bd = dev(a), dev(b)
    qa = F.nvfp4_quantize_1d(ad, F.nvfp4_amax(ad))
    qb = F.nvfp4_quantize_2d(bd, F.nvfp4_amax(bd), colwise=False)
    args = (qa["codes_row"], qa["scales_row"], 1, qa["global_scale"], qb["codes_row"], qb["scales"], 2,
            qb["global_scale"], M, N, K)
    y = F.nvfp4_gemm(*args, out_dtype=torch.bfloat16)
    amax = torch.full((1,), given, dtype=torch.float32, device="cuda")
    got = F.nvfp4_gemm_quantize(*args, amax)
    ref = F.nvfp4_quantize_1d(y, amax, rowwise=True, colwise=True)
    for k in ("global_scale", "codes_row", "scales_row", "codes_col", "scales_col"):
        g_, r_ = host(got[k]), host(ref[k])
        assert np.array_equal(g_.view(np.uint8), r_.view(np.uint8)), k
