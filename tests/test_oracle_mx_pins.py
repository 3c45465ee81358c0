"""CPU pins of the oracle's MXFP4 comparator format (E2M1 payload, one
E8M0 power-of-two scale per 32 values; page "NVFP4 Is a Scaling System, Not
Just a 4-Bit Number", section "Generic FP4, MXFP4, and NVFP4").

Each check holds the oracle against something other than itself: torch's
own E8M0 decoder, an exact-rational brute force of the scale rule
(X = 2^(floor(log2 amax) - 2), from the exponent that frexp returns, not
from log2) and of nearest-even E2M1 rounding, a closed form of the Hadamard
transform of a constant column, the pages' storage figure, and the pages'
claim that NVFP4 quantizes with less error than MXFP4.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _unpack(codes):
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


def _e8m0_torch(b):
    t = torch.tensor(np.asarray(b, np.uint8)).view(torch.float8_e8m0fnu)
    return t.to(torch.float64).numpy()


def _expected_block(vals):
    """(scale byte, codes) of one block of binary32 values, brute force."""
    vals = [float(np.float32(v)) for v in vals]
    if any(not math.isfinite(v) for v in vals):
        return 0xFF, [8 if math.copysign(1.0, v) < 0 else 0 for v in vals]
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        e = -127
    else:
        e = max(-127, min(127, math.frexp(amax)[1] - 1 - 2))
    X = Fraction(2) ** e
    codes = []
    for v in vals:
        r = abs(Fraction(v)) / X
        d = [abs(r - g) for g in GRID]
        best = min(range(8), key=lambda k: (d[k], k & 1))
        codes.append(best | (8 if math.copysign(1.0, v) < 0 else 0))
    return e + 127, codes


def _check_rows(vals_f32, codes, scales):
    R, C = vals_f32.shape
    q = _unpack(codes)
    for r in range(R):
        for b in range(C // 32):
            sb, cs = _expected_block(vals_f32[r, 32 * b:32 * b + 32])
            assert scales[r, b] == sb, (r, b)
            assert list(q[r, 32 * b:32 * b + 32]) == cs, (r, b)


def test_e8m0_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    mine = np.array([oracle.e8m0_decode(int(v)) for v in b])
    ref = _e8m0_torch(b)
    assert np.isnan(mine[255]) and np.isnan(ref[255])
    assert np.array_equal(mine[:255], ref[:255])
    assert mine[127] == 1.0


def test_scale_rule_brackets_the_block_maximum():
    """4 <= amax / X < 8 wherever the rule is not clamped; bf16 maxima at
    every binade, both ends of each, zero and the subnormals."""
    rng = np.random.default_rng(1)
    bits = np.concatenate([
        np.arange(0, 0x7F80, 97, dtype=np.uint32),
        np.array([1, 0x7F, 0x80, 0x3F80, 0x3FFF, 0x4000, 0x7F7F], np.uint32),
        rng.integers(0, 0x7F80, 3000).astype(np.uint32),
    ])
    for h in bits:
        a = float(np.uint32(h << 16).view(np.float32))
        b = oracle.mx_scale_byte(a)
        want, _ = _expected_block([a] + [0.0] * 31)
        assert b == want, hex(h)
        if 1 <= b <= 253:
            q = Fraction(a) / (Fraction(2) ** (b - 127))
            assert 4 <= q < 8
    assert oracle.mx_scale_byte(float("inf")) == 0xFF
    assert oracle.mx_scale_byte(float("nan")) == 0xFF


@pytest.mark.parametrize("maker", [
    lambda: W.activation(8, 96, seed=40, n_outlier_cols=2),
    lambda: W.gradient(4, 128, seed=41),
    lambda: W.normal_tensor(4, 64, seed=42, std=3e-39),   # subnormal-range blocks
])
def test_rows_match_bruteforce(maker):
    x = maker()
    codes, scales = oracle.mx_quantize_rows(x)
    assert codes.shape == (x.shape[0], x.shape[1] // 2) and scales.shape == (x.shape[0], x.shape[1] // 32)
    _check_rows(W.bf16_bits_to_f32(x), codes, scales)


def test_cols_is_rows_of_transpose():
    x = W.activation(64, 48, seed=43, n_outlier_cols=1)
    cc, sc = oracle.mx_quantize_cols(x)
    cr, sr = oracle.mx_quantize_rows(np.ascontiguousarray(x.T))
    assert np.array_equal(cc, cr) and np.array_equal(sc, sr)


def test_cols_with_hadamard_quantize_the_transformed_values():
    x = W.gradient(64, 24, seed=44)
    mask = W.rht_sign_mask()
    cc, sc = oracle.mx_quantize_cols(x, rht=True, mask=mask)
    y = oracle.rht16_tensor(x, 0, mask)          # [R][C] binary32
    _check_rows(np.ascontiguousarray(y.T), cc, sc)


def test_hadamard_of_constant_column_is_one_spike_per_segment():
    """mask 0: (1/4) H16 (c, ..., c) = (4c, 0, ..., 0), so each 32-row block
    decodes to 4c rounded by the format at rows 0 and 16 and zero elsewhere;
    c = 1.25 puts 4c = 5 on a tie (4 and 6), which goes to 4."""
    R, C = 64, 4
    cvals = np.array([1.0, 1.25, -0.75, 3.0], np.float32)
    x = W.f32_to_bf16_bits(np.tile(cvals, (R, 1)))
    cc, sc = oracle.mx_quantize_cols(x, rht=True, mask=0)
    deq = oracle.mx_dequantize(cc, sc, C, R)
    want_spike = {1.0: 4.0, 1.25: 4.0, -0.75: -3.0, 3.0: 12.0}
    for c, v in enumerate(cvals):
        col = deq[c]
        spikes = np.zeros(R, np.float32)
        spikes[0::16] = want_spike[float(v)]
        assert np.array_equal(col, spikes), (v, col[:17])


def test_zero_nan_inf_blocks():
    x = np.zeros((2, 96), np.uint16)
    x[0, 5] = 0x8000                      # -0 in an all-zero block
    x[0, 40] = 0x7FC0                     # NaN in block 1
    x[1, 70] = 0xFF80                     # -inf in block 2
    x[1, 71] = 0x3F80                     # 1.0 beside it
    codes, scales = oracle.mx_quantize_rows(x)
    assert scales[0].tolist() == [0, 0xFF, 0] and scales[1].tolist() == [0, 0, 0xFF]
    q = _unpack(codes)
    assert q[0, 5] == 8 and q[1, 70] == 8 and q[1, 71] == 0
    assert np.count_nonzero(q) == 2
    deq = oracle.mx_dequantize(codes, scales, 2, 96)
    assert np.all(np.isnan(deq[0, 32:64])) and np.all(np.isnan(deq[1, 64:96]))
    assert np.all(deq[0, :32] == 0) and np.signbit(deq[0, 5])


def test_dequantize_matches_torch_decoders_and_is_exact():
    x = W.activation(16, 128, seed=45, n_outlier_cols=2)
    codes, scales = oracle.mx_quantize_rows(x)
    q = _unpack(codes)
    mags = np.array([float(g) for g in GRID])
    want = np.where(q & 8, -1.0, 1.0) * mags[q & 7] * np.repeat(_e8m0_torch(scales), 32, axis=1)
    f32 = oracle.mx_dequantize(codes, scales, 16, 128)
    f64 = oracle.mx_dequantize_f64_rows(codes, scales, 16, 128, np.arange(16))
    assert np.array_equal(f64, want) and np.array_equal(f32.astype(np.float64), want)


def test_storage_bits(golden):
    exp = {k: (float(v), float(t)) for k, v, t in golden("storage_bits.txt")}
    x = W.normal_tensor(64, 256, seed=46)
    codes, scales = oracle.mx_quantize_rows(x)
    v, tol = exp["bits_per_element_mxfp4"]
    assert abs(8 * (codes.nbytes + scales.nbytes) / x.size - v) <= tol


def _rel_err(ref, deq):
    ref = ref.astype(np.float64)
    return np.linalg.norm(ref - deq) / np.linalg.norm(ref)


@pytest.mark.parametrize("maker", [
    lambda: W.activation(128, 512, seed=47),
    lambda: W.weight(128, 512, seed=48),
    lambda: W.gradient(128, 512, seed=49),
])
def test_nvfp4_quantizes_with_less_error_than_mxfp4(maker):
    """The pages' claim (page "MXFP4 和 NVFP4 的区别", section "NVFP4:NVIDIA
    专有,精度更优"; page "NVFP4 Is a Scaling System, Not Just a 4-Bit
    Number", section "Generic FP4, MXFP4, and NVFP4"), rowwise on the three
    workload tensors, and columnwise after the Hadamard transform."""
    x = maker()
    R, C = x.shape
    xf = W.bf16_bits_to_f32(x)
    r = oracle.quantize_1d(x, rowwise=True)
    e_nv = _rel_err(xf, oracle.dequantize(r["codes_row"], r["scales_row"], 1, r["sg"], R, C))
    mc, ms = oracle.mx_quantize_rows(x)
    e_mx = _rel_err(xf, oracle.mx_dequantize(mc, ms, R, C))
    assert e_nv < e_mx
    mask = W.rht_sign_mask()
    y = oracle.rht16_tensor(x, 0, mask).T
    r = oracle.quantize_1d(x, rowwise=False, colwise=True, rht=True, mask=mask)
    e_nv_h = _rel_err(y, oracle.dequantize(r["codes_col"], r["scales_col"], 1, r["sg"], C, R))
    mc, ms = oracle.mx_quantize_cols(x, rht=True, mask=mask)
    e_mx_h = _rel_err(y, oracle.mx_dequantize(mc, ms, C, R))
    assert e_nv_h < e_mx_h


def test_gemm_reference_tiny_bruteforce():
    M, N, K = 8, 8, 64
    a = W.activation(M, K, seed=50, n_outlier_cols=1)
    b = W.weight(N, K, seed=51)
    ca, sa = oracle.mx_quantize_rows(a)
    cb, sb = oracle.mx_quantize_rows(b)
    ref = oracle.mx_gemm_rows(ca, sa, cb, sb, M, N, K, np.arange(M))
    qa, qb = _unpack(ca), _unpack(cb)

    def val(q, s, r, k):
        v = GRID[q[r, k] & 7] * Fraction(2) ** (int(s[r, k // 32]) - 127)
        return -v if q[r, k] & 8 else v

    for m in range(M):
        for n in (0, 3, 7):
            exact = sum(val(qa, sa, m, k) * val(qb, sb, n, k) for k in range(K))
            assert abs(float(exact) - ref[m, n]) <= 1e-12 * max(1.0, abs(float(exact)))


def test_threaded_drivers_equal_single_thread():
    """The threaded drivers the full-size GPU tests use split rows or
    columns over threads and must give the single call's bytes."""
    x = W.gradient(320, 96, seed=5)
    for a, b in zip(oracle.mx_quantize_rows(x), oracle.mx_quantize_rows_mt(x, threads=4)):
        assert np.array_equal(a, b)
    for rht in (False, True):
        single = oracle.mx_quantize_cols(x, rht=rht, mask=0x5A3C)
        for a, b in zip(single, oracle.mx_quantize_cols_mt(x, rht=rht, mask=0x5A3C, threads=5)):
            assert np.array_equal(a, b)
