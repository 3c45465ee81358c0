"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Codes, scale bytes, amax and global scales must match bit for bit; the
Hadamard transform must match the oracle's binary32 butterfly bit for bit
(and the dense double-precision transform within 1e-6 relative); the GEMM
must satisfy ||C - C_ref||_F / ||C_ref||_F <= 1e-5 against the double
reference on the dequantized operands.

Every quantizer output is compared whole, the full-size workloads (8192x4096
activation, 14336x4096 weight, 8192x14336 gradient) included, against the
oracle run on all host cores (the same C functions over disjoint row,
column or tile-row ranges), in the launch configurations bench.py times.
The 8192x14336x4096 product is checked on 256 sampled rows in full, as its
workload states.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

F = None


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


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f32_bits(a) -> int:
    return int(np.float32(a).view(np.uint32))


def to_gpu(a: np.ndarray) -> torch.Tensor:
    """An oracle-made array (codes, scales) on the device, as the input of
    the kernel under test."""
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def sg_gpu(sg) -> torch.Tensor:
    return torch.tensor([float(np.float32(sg))], dtype=torch.float32, device="cuda")


def oracle_operand(x: np.ndarray, mode: int):
    """The oracle's NVFP4 encoding of x as a TN GEMM operand: (codes,
    scales, S_g). mode 1: 1D rowwise; 2: 2D tiles, rowwise codes; 3: the
    column copy of x^T (codes [R][C/2], the transposed tensor's tile
    scales [C/16][R/16])."""
    if mode == 1:
        sg = oracle.global_scale(oracle.amax(x))
        c, s = oracle.quantize_1d_rows(x, sg)
        return c, s, sg
    if mode == 2:
        sg = oracle.global_scale(oracle.amax(x))
        cr, _, s = oracle.quantize_2d(x, sg)
        return cr, s, sg
    xt = np.ascontiguousarray(x.T)
    sg = oracle.global_scale(oracle.amax(xt))
    _, cc, s = oracle.quantize_2d(xt, sg)
    return cc, s, sg


# ------------------------------------------------------------- workloads

@functools.lru_cache(maxsize=None)
def wl(name):
    log(f"[workload] generating {name}")
    if name == "act_small":
        return W.activation_small()
    if name == "act":
        return W.activation()
    if name == "weight":
        return W.weight()
    if name == "grad":
        return W.gradient()
    if name == "ragged_act":
        return W.activation(272, 528, seed=101)
    if name == "ragged_grad":
        return W.gradient(304, 400, seed=102)
    if name == "ragged_weight":
        return W.weight(272, 400, seed=103)
    raise KeyError(name)


MASK = W.rht_sign_mask()
SEED = W.SR_SEED


def same_rows(got, want, what):
    """Whole-array byte equality, naming the first rows that differ."""
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.nonzero(np.any(got != want, axis=tuple(range(1, got.ndim))))[0]
        raise AssertionError(f"{what} differ in {bad.size} rows, first {bad[:8].tolist()}")


# ------------------------------------------------------------------ amax

@pytest.mark.parametrize("name", ["act_small", "ragged_act", "act", "grad"])
def test_amax(name):
    x = wl(name)
    log(f"[test_amax] {name} {x.shape}")
    got = host(F.nvfp4_amax(dev(x)))[0]
    assert f32_bits(got) == f32_bits(oracle.amax(x))


def test_amax_odd_length_tail():
    x = W.normal_tensor(13, 17, seed=5)  # 221 elements: 27 vectors + a 5-element tail
    x[12, 16] = W.f32_to_bf16_bits(np.array([-77.0], np.float32))[0]
    got = host(F.nvfp4_amax(dev(x)))[0]
    assert got == 77.0 and f32_bits(got) == f32_bits(oracle.amax(x))


@pytest.mark.parametrize("pos", ["first", "middle", "last"])
def test_amax_planted_max_reused_output(pos):
    """The one-workgroup-per-CU amax launches read the running maximum before
    their atomic and skip it when it cannot raise the output. A maximum
    planted at either end of an 8192x4096 tensor (the first or last
    workgroup's span), with the output buffer holding a larger value from the
    previous call, must still come out exact: the plain amax, the transform's
    amax and both amaxes of the one-read variant."""
    x = W.normal_tensor(8192, 4096, seed=31)
    r, c = {"first": (0, 0), "middle": (4100, 2049), "last": (8191, 4095)}[pos]
    x[r, c] = W.f32_to_bf16_bits(np.array([-640.0], np.float32))[0]
    big = x.copy()
    big[17, 5] = W.f32_to_bf16_bits(np.array([1.0e6], np.float32))[0]
    log(f"[test_amax_planted_max_reused_output] {pos}")
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    F.nvfp4_amax(dev(big), out=out)
    got = host(F.nvfp4_amax(dev(x), out=out))[0]
    assert got == 640.0 and f32_bits(got) == f32_bits(oracle.amax(x))
    rht_ref = oracle.amax_rht_mt(x, MASK)
    F.nvfp4_amax(dev(big), rht=True, rht_mask=MASK, out=out)
    got_rht = host(F.nvfp4_amax(dev(x), rht=True, rht_mask=MASK, out=out))[0]
    assert f32_bits(got_rht) == f32_bits(rht_ref)
    out2 = torch.empty(2, dtype=torch.float32, device="cuda")
    F.nvfp4_amax(dev(big), rht=True, rht_mask=MASK, both=True, out=out2)
    got2 = host(F.nvfp4_amax(dev(x), rht=True, rht_mask=MASK, both=True, out=out2))
    assert f32_bits(got2[0]) == f32_bits(oracle.amax(x))
    assert f32_bits(got2[1]) == f32_bits(rht_ref)


@pytest.mark.parametrize("pos", [(8192, 0), (10000, 1234), (12287, 4095)])
def test_amax_partial_last_round(pos):
    """12288x4096 is one and a half rounds of the plain amax's grid-stride
    loop (256 workgroups x 1024 threads x 16 vectors): rows 8192 onwards are
    read by the last, partial round, whose loads past the end repeat the
    last vector. A maximum planted at the start, inside and at the very end
    of that region must come out exact."""
    x = W.normal_tensor(12288, 4096, seed=37)
    x[pos] = W.f32_to_bf16_bits(np.array([-512.0], np.float32))[0]
    log(f"[test_amax_partial_last_round] {pos}")
    got = host(F.nvfp4_amax(dev(x)))[0]
    assert got == 512.0 and f32_bits(got) == f32_bits(oracle.amax(x))


@pytest.mark.parametrize("name", ["ragged_grad", "grad", "act"])
def test_amax_rht(name):
    x = wl(name)
    log(f"[test_amax_rht] {name} {x.shape}")
    got = host(F.nvfp4_amax(dev(x), rht=True, rht_mask=MASK))[0]
    assert f32_bits(got) == f32_bits(oracle.amax_rht(x, MASK))


# -------------------------------------------------------------- 1D quantize

def run_q1(x, rowwise, colwise, sr=False, rht=False):
    xd = dev(x)
    a = F.nvfp4_amax(xd, rht=rht, rht_mask=MASK)
    out = F.nvfp4_quantize_1d(xd, a, rowwise=rowwise, colwise=colwise, sr=sr, rht=rht,
                              rht_mask=MASK, seed=SEED)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}, host(a)[0]


def check_q1(x, got, amax_gpu, rowwise, colwise, sr, rht):
    """Every byte of the requested layouts, the amax and S_g, against the
    oracle on the whole tensor."""
    amax = oracle.amax_rht_mt(x, MASK) if rht else oracle.amax_mt(x)
    assert f32_bits(amax_gpu) == f32_bits(amax)
    sg = oracle.global_scale(amax)
    assert f32_bits(got["global_scale"][0]) == f32_bits(sg)
    if rowwise:
        c, s = oracle.quantize_1d_rows_mt(x, sg, sr, SEED)
        same_rows(got["codes_row"], c, "rowwise codes")
        same_rows(got["scales_row"], s, "rowwise scales")
    if colwise:
        c, s = oracle.quantize_1d_cols_mt(x, sg, sr, SEED, rht, MASK)
        same_rows(got["codes_col"], c, "columnwise codes (rows = input columns)")
        same_rows(got["scales_col"], s, "columnwise scales")


CASES_SMALL = [
    # (workload, rowwise, colwise, sr, rht)
    ("act_small", True, False, False, False),
    ("act_small", False, True, False, False),
    ("act_small", True, True, False, False),
    ("ragged_act", True, True, False, False),
    ("ragged_act", False, True, False, False),
    ("ragged_act", True, False, True, False),
    ("ragged_act", False, True, True, False),
    ("ragged_act", True, True, True, False),
    ("ragged_grad", False, True, True, True),
    ("ragged_grad", False, True, False, True),
    ("ragged_grad", True, True, True, False),
]


@pytest.mark.parametrize("case", CASES_SMALL, ids=lambda c: "-".join(str(v) for v in c))
def test_quantize_1d_small(case):
    name, rowwise, colwise, sr, rht = case
    x = wl(name)
    log(f"[test_quantize_1d_small] {case} {x.shape}")
    got, a = run_q1(x, rowwise, colwise, sr, rht)
    check_q1(x, got, a, rowwise, colwise, sr, rht)


FULL_CASES = [
    # (workload, rowwise, colwise, sr, rht): the activation's layouts as the
    # bench rows time them (round-to-nearest with columnwise output takes the
    # paired-tile kernel, rowwise only and stochastic rounding the one-tile
    # kernel), the gradient path of the wgrad operands (transform +
    # stochastic rounding, columnwise, seed 42, gradient and activation),
    # the transform with round-to-nearest, stochastic rounding without the
    # transform, and the gradient's rowwise dgrad operand.
    ("act", True, True, False, False),
    ("act", True, False, False, False),
    ("act", False, True, False, False),
    ("act", True, True, True, False),
    ("act", False, True, True, True),
    ("act", False, True, False, True),
    ("grad", False, True, True, True),
    ("grad", False, True, True, False),
    ("grad", True, False, True, False),
    ("grad", True, True, False, False),
]


@pytest.mark.parametrize("case", FULL_CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_quantize_1d_full_size(case):
    """The full-size workloads, every byte of every requested output."""
    name, rowwise, colwise, sr, rht = case
    x = wl(name)
    log(f"[test_quantize_1d_full_size] {case} {x.shape}")
    got, a = run_q1(x, rowwise, colwise, sr, rht)
    check_q1(x, got, a, rowwise, colwise, sr, rht)


def wide_range_blocks(rows, cols, seed):
    """Every 16-element block (along rows and along columns) spans a huge
    dynamic range: its ratios |x|/(s*S_g) cover 2^-42 .. 6, both signs,
    exact grid points and midpoints included, so stochastic rounding meets
    tiny ratios (no fraction bits left for a 22-bit window), ratios in
    [0.5, 1) with odd last mantissa bits, and saturation."""
    rng = np.random.default_rng(seed)
    mag = np.exp2(rng.uniform(-44.0, 2.6, size=(rows, cols))).astype(np.float32)
    grid = np.array([0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.5, 3.0, 3.5, 4.0, 5.0, 6.0],
                    np.float32) / np.float32(6.0)
    pick = rng.random((rows, cols)) < 0.1
    mag[pick] = rng.choice(grid, size=int(pick.sum()))
    mag[::16, :] = 1.0  # a block maximum in every column block
    mag[:, ::16] = 1.0  # and in every row block
    sign = np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0).astype(np.float32)
    return W.f32_to_bf16_bits(mag * sign)


@pytest.mark.parametrize("layouts", [(True, False), (False, True), (True, True)])
def test_sr_wide_dynamic_range(layouts):
    """Stochastic rounding over ratios from 2^-42 to 6: bit-identical to the
    oracle in both layouts (the rule 'round up iff h < p * 2^16' at every
    magnitude)."""
    rowwise, colwise = layouts
    x = wide_range_blocks(512, 1024, 77)
    log(f"[test_sr_wide_dynamic_range] {layouts}")
    got, a = run_q1(x, rowwise, colwise, sr=True)
    check_q1(x, got, a, rowwise, colwise, True, False)


def scale_straddlers(amax):
    """Positive bf16 block maxima b <= amax whose E4M3 scale byte differs
    between fl(b / t), the rule, and fl(b * fl(1/t)), a multiply by the
    reciprocal (t = 6 * S_g): the blocks where that shortcut would round
    the scale the wrong way."""
    b = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    b = b[b <= amax]
    t = np.float32(6.0) * np.float32(oracle.global_scale(amax))
    by_rcp = oracle.e4m3_encode_array(b * (np.float32(1.0) / t))
    by_div = oracle.e4m3_encode_array(b / t)
    return b[by_rcp != by_div]


def straddle_tensor(rows, cols, seed):
    """amax 0.00189208984375 (bf16 0x3AF8) has a straddling block maximum in
    each of 15 binades. Every 16x16 tile carries one on its diagonal (so it is
    the maximum of one row block and one column block), over noise 16x
    smaller; every fifth tile is all zeros, and one element is the amax."""
    amax = np.float32(0.00189208984375)
    hits = scale_straddlers(amax)
    assert hits.size >= 10
    rng = np.random.default_rng(seed)
    x = (rng.uniform(-1.0, 1.0, size=(rows, cols)) * float(hits.min()) / 16.0).astype(np.float32)
    i = np.arange(rows)
    for c0 in range(0, cols, 16):
        diag = rng.choice(hits, size=rows) * np.where(rng.random(rows) < 0.5, -1.0, 1.0)
        x[i, c0 + (i % 16)] = diag
    for t, (r0, c0) in enumerate((r, c) for r in range(0, rows, 16) for c in range(0, cols, 16)):
        if t % 5 == 3:
            x[r0:r0 + 16, c0:c0 + 16] = 0.0
    x[1, 1] = amax
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("layouts", [(True, True), (True, False), (False, True)])
def test_scale_bytes_near_rounding_midpoints(layouts, fused):
    """Block maxima whose scale sits next to an E4M3 rounding midpoint, all
    through the tensor and mixed with all-zero blocks in the same waves:
    scale bytes and codes bit-identical to the oracle (division rule)."""
    rowwise, colwise = layouts
    x = straddle_tensor(128, 512, 31)
    log(f"[test_scale_bytes_near_rounding_midpoints] {layouts} fused={fused}")
    if fused:
        out = F.nvfp4_quantize_1d_fused(dev(x), F.nvfp4_workspace(), rowwise=rowwise, colwise=colwise)
        torch.cuda.synchronize()
        got = {k: host(v) for k, v in out.items()}
        a = np.float32(oracle.amax(x))
    else:
        got, a = run_q1(x, rowwise, colwise)
    assert a == np.float32(0.00189208984375)
    check_q1(x, got, a, rowwise, colwise, False, False)


def test_quantize_deterministic():
    x = wl("ragged_grad")
    g1, _ = run_q1(x, True, True, sr=True)
    g2, _ = run_q1(x, True, True, sr=True)
    for k in g1:
        assert np.array_equal(g1[k], g2[k])


# ------------------------------------------------------------- edge cases

def edge_tensors():
    z = np.zeros((32, 48), np.uint16)
    neg0 = z.copy()
    neg0[5, 7] = 0x8000
    denorm = (np.arange(32 * 48, dtype=np.uint32) % 120 + 1).astype(np.uint16).reshape(32, 48)
    denorm[::3] |= 0x8000
    tiny = W.f32_to_bf16_bits(W.bf16_bits_to_f32(W.normal_tensor(32, 48, 9)) * np.float32(1e-36))
    withnan = W.normal_tensor(32, 48, 10)
    withnan[7, 9] = 0x7FC1
    withinf = W.normal_tensor(32, 48, 11)
    withinf[3, 3] = 0xFF80
    return {"zeros": z, "neg_zero": neg0, "denormals": denorm, "tiny": tiny, "nan": withnan,
            "inf": withinf}


@pytest.mark.parametrize("name", list(edge_tensors().keys()))
@pytest.mark.parametrize("sr", [False, True])
def test_edge_cases_1d(name, sr):
    x = edge_tensors()[name]
    log(f"[test_edge_cases_1d] {name} sr={sr}")
    got, a = run_q1(x, True, True, sr=sr)
    amax = oracle.amax(x)
    if np.isnan(amax):
        assert np.isnan(a)
        sg = oracle.global_scale(amax)
        c, s = oracle.quantize_1d_rows(x, sg, sr, SEED)
        assert np.array_equal(got["codes_row"], c) and np.array_equal(got["scales_row"], s)
        c, s = oracle.quantize_1d_cols(x, sg, sr, SEED)
        assert np.array_equal(got["codes_col"], c) and np.array_equal(got["scales_col"], s)
    else:
        check_q1(x, got, a, True, True, sr, False)


@pytest.mark.parametrize("name", ["zeros", "denormals", "tiny", "inf"])
def test_edge_cases_rht(name):
    x = edge_tensors()[name]
    got, a = run_q1(x, False, True, sr=True, rht=True)
    check_q1(x, got, a, False, True, True, True)


# -------------------------------------------------------------------- 2D

def run_q2(x):
    xd = dev(x)
    a = F.nvfp4_amax(xd)
    out = F.nvfp4_quantize_2d(xd, a)
    return {k: host(v) for k, v in out.items()}, host(a)[0]


def test_quantize_2d_ragged_full_compare():
    x = wl("ragged_weight")
    got, a = run_q2(x)
    sg = oracle.global_scale(oracle.amax(x))
    assert f32_bits(a) == f32_bits(oracle.amax(x))
    assert f32_bits(got["global_scale"][0]) == f32_bits(sg)
    cr, cc, s = oracle.quantize_2d(x, sg)
    assert np.array_equal(got["scales"], s)
    assert np.array_equal(got["codes_row"], cr)
    assert np.array_equal(got["codes_col"], cc)


def test_quantize_2d_full_weight():
    """The 14336x4096 weight: every tile scale and every code of both
    layouts; the transposed tile grid equals the grid transposed."""
    x = wl("weight")
    log("[test_quantize_2d_full_weight]")
    xd = dev(x)
    a = F.nvfp4_amax(xd)
    got = {k: host(v) for k, v in F.nvfp4_quantize_2d(xd, a, transposed_scales=True).items()}
    amax = oracle.amax_mt(x)
    assert f32_bits(host(a)[0]) == f32_bits(amax)
    sg = oracle.global_scale(amax)
    assert f32_bits(got["global_scale"][0]) == f32_bits(sg)
    cr, cc, s = oracle.quantize_2d_mt(x, sg)
    same_rows(got["scales"], s, "tile scales")
    same_rows(got["scales_t"], np.ascontiguousarray(s.T), "transposed tile scales")
    same_rows(got["codes_row"], cr, "rowwise codes")
    same_rows(got["codes_col"], cc, "columnwise codes")


def test_quantize_2d_single_layout_outputs():
    x = wl("ragged_weight")
    xd = dev(x)
    a = F.nvfp4_amax(xd)
    both = F.nvfp4_quantize_2d(xd, a)
    rows_only = F.nvfp4_quantize_2d(xd, a, rowwise=True, colwise=False)
    cols_only = F.nvfp4_quantize_2d(xd, a, rowwise=False, colwise=True)
    sg = oracle.global_scale(oracle.amax(x))
    cr, cc, s = oracle.quantize_2d(x, sg)
    assert np.array_equal(host(rows_only["codes_row"]), cr) and np.array_equal(host(rows_only["scales"]), s)
    assert np.array_equal(host(cols_only["codes_col"]), cc) and np.array_equal(host(cols_only["scales"]), s)
    assert torch.equal(both["codes_row"], rows_only["codes_row"])
    assert torch.equal(both["codes_col"], cols_only["codes_col"])


# ------------------------------------------------------------------- RHT

@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("name", ["ragged_grad", "act_small"])
def test_rht16_standalone(name, axis):
    x = wl(name)
    y = host(F.nvfp4_rht16(dev(x), axis=axis, rht_mask=MASK))
    ref = oracle.rht16_tensor(x, axis, MASK)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))
    # against the dense double-precision transform
    H = np.array([[(-1) ** bin(j & k).count("1") for k in range(16)] for j in range(16)], float) / 4
    d = np.array([-1.0 if (MASK >> j) & 1 else 1.0 for j in range(16)])
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    if axis == 0:
        dense = np.einsum("jk,rkc->rjc", H, d[None, :, None] * xf.reshape(-1, 16, xf.shape[1])).reshape(xf.shape)
    else:
        dense = np.einsum("jk,rck->rcj", H, d[None, None, :] * xf.reshape(xf.shape[0], -1, 16)).reshape(xf.shape)
    assert np.linalg.norm(y - dense) / np.linalg.norm(dense) <= 1e-6


# ------------------------------------------------------------ dequantize

@pytest.mark.parametrize("mode", [1, 2])
def test_dequantize(mode):
    """The oracle's codes and scales, decoded on the GPU: bit-identical to
    the oracle's decode of the same bytes."""
    x = wl("ragged_weight") if mode == 2 else wl("ragged_act")
    R, C = x.shape
    codes, scales, sg = oracle_operand(x, mode)
    cd, sd, gd = to_gpu(codes), to_gpu(scales), sg_gpu(sg)
    y32 = host(F.nvfp4_dequantize(cd, sd, mode, gd, R, C))
    y16 = host(F.nvfp4_dequantize(cd, sd, mode, gd, R, C, out_dtype=torch.bfloat16).view(torch.int16))
    ref = oracle.dequantize(codes, scales, mode, sg, R, C)
    assert np.array_equal(y32.view(np.uint32), ref.view(np.uint32))
    ref16 = oracle.dequantize_bf16(codes, scales, mode, sg, R, C)
    assert np.array_equal(y16.view(np.uint16), ref16)


@pytest.mark.parametrize("mode", [1, 2])
def test_dequantize_every_code_and_scale_byte(mode):
    """Arbitrary codes and all 256 scale bytes (negative, zero, subnormal,
    448, NaN): bit-identical to the oracle, NaN results compared as NaN with
    the oracle's sign (the payload is not a property of the method)."""
    rng = np.random.default_rng(7)
    R, C = 272, 4096  # a 2D tile row covers all 256 scale bytes per 16 rows
    codes = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    if mode == 1:
        scales = np.tile(np.arange(256, dtype=np.uint8), R * (C // 16) // 256 + 1)[: R * (C // 16)]
        scales = scales.reshape(R, C // 16)
    else:
        scales = np.tile(np.arange(256, dtype=np.uint8), (R // 16) * (C // 16) // 256 + 1)
        scales = scales[: (R // 16) * (C // 16)].reshape(R // 16, C // 16)
    sg = np.array([0.37109375], dtype=np.float32)
    cd, sd, gd = (torch.from_numpy(a).to("cuda") for a in (codes, scales, sg))
    y32 = host(F.nvfp4_dequantize(cd, sd, mode, gd, R, C))
    y16 = host(F.nvfp4_dequantize(cd, sd, mode, gd, R, C, out_dtype=torch.bfloat16).view(torch.int16))
    ref = oracle.dequantize(codes, scales, mode, sg[0], R, C)
    ref16 = oracle.dequantize_bf16(codes, scales, mode, sg[0], R, C)
    for got, want, top in ((y32.view(np.uint32), ref.view(np.uint32), np.uint32(0x80000000)),
                           (y16.view(np.uint16), ref16.view(np.uint16), np.uint16(0x8000))):
        nan_w = (want & ~top) > (np.uint32(0x7F800000) if top == 0x80000000 else np.uint16(0x7F80))
        nan_g = (got & ~top) > (np.uint32(0x7F800000) if top == 0x80000000 else np.uint16(0x7F80))
        assert nan_w.any()
        assert np.array_equal(nan_w, nan_g)
        assert np.array_equal(got[~nan_w], want[~nan_w])
        assert np.array_equal(got[nan_w] & top, want[nan_w] & top)


# ------------------------------------------------------------------- GEMM

def gemm_check(a_bits, b_bits, rows, out_dtype=torch.float32):
    """The oracle's operands (A 1D, B 2D) multiplied on the GPU, against the
    oracle's double product of the same operands on the given rows."""
    M, K = a_bits.shape
    N = b_bits.shape[0]
    ac, as_, ag = oracle_operand(a_bits, 1)
    bc, bs, bg = oracle_operand(b_bits, 2)
    c = F.nvfp4_gemm(to_gpu(ac), to_gpu(as_), 1, sg_gpu(ag), to_gpu(bc), to_gpu(bs), 2, sg_gpu(bg),
                     M, N, K, out_dtype=out_dtype)
    c = host(c.float() if out_dtype == torch.bfloat16 else c)
    ref = oracle.gemm_rows(ac, as_, 1, ag, bc, bs, 2, bg, M, N, K, np.asarray(rows, np.int64))
    got = c[np.asarray(rows)].astype(np.float64)
    return np.linalg.norm(got - ref) / np.linalg.norm(ref), c


def test_gemm_ragged_full():
    a = W.normal_tensor(272, 528, seed=40)
    b = W.normal_tensor(400, 528, seed=41, std=0.02)
    err, _ = gemm_check(a, b, np.arange(272))
    assert err <= 1e-5


def test_gemm_full_size_sampled_rows():
    log("[test_gemm_full_size_sampled_rows] generating 8192x4096 and 14336x4096 operands")
    a, b = W.gemm_operands()
    rows = W.gemm_sample_rows()
    err, c32 = gemm_check(a, b, rows)
    log(f"[test_gemm_full_size_sampled_rows] rel_fro={err:.3e}")
    assert err <= 1e-5


@pytest.mark.parametrize("a_mode,b_mode", [(1, 2), (2, 1)])
def test_gemm_more_tiles_than_workgroups(a_mode, b_mode):
    """More 256 x 256 output tiles than resident workgroups (each workgroup
    walks several), ragged in M and N, K an odd multiple of 16, and both
    assignments of 1D / 2D scales to the operands: every output row checked."""
    M, N, K = 2064, 8208, 48  # 9 x 33 = 297 tiles
    a = W.normal_tensor(M, K, seed=44)
    b = W.normal_tensor(N, K, seed=45, std=0.02)
    log(f"[test_gemm_more_tiles_than_workgroups] modes=({a_mode},{b_mode})")
    ac, as_, ag = oracle_operand(a, a_mode)
    bc, bs, bg = oracle_operand(b, b_mode)
    c = host(F.nvfp4_gemm(to_gpu(ac), to_gpu(as_), a_mode, sg_gpu(ag), to_gpu(bc), to_gpu(bs), b_mode,
                          sg_gpu(bg), M, N, K))
    ref = oracle.gemm_rows(ac, as_, a_mode, ag, bc, bs, b_mode, bg, M, N, K, np.arange(M, dtype=np.int64))
    err = np.linalg.norm(c.astype(np.float64) - ref) / np.linalg.norm(ref)
    assert err <= 1e-5
    # each row separately too, so a wrong tile cannot hide in the norm
    row_err = np.linalg.norm(c.astype(np.float64) - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    assert row_err.max() <= 1e-5


def reference_rows(codes, scales, mode, sg, R, C):
    """Double reconstruction by the oracle of an oracle-made operand in any
    scale mode: mode 3 is decoded as the 2D rowwise layout of the
    transposed tensor's tiles."""
    if mode != 3:
        return oracle.dequantize_f64_rows(codes, scales, mode, sg, R, C, np.arange(R))
    # codes_col [R][C/2] of x^T [C][R] with scales [C/16][R/16]: element (r, c) has scale [c/16][r/16]
    st = np.ascontiguousarray(scales.T)      # [R/16][C/16]
    return oracle.dequantize_f64_rows(codes, st, 2, sg, R, C, np.arange(R))


@pytest.mark.parametrize("K", [1024, 4160])
@pytest.mark.parametrize("a_mode,b_mode", [(1, 2), (2, 1), (1, 3), (3, 1), (1, 1)])
def test_gemm_64_element_stages(K, a_mode, b_mode):
    """K a multiple of 64: 64-element stages, tile scales staged in LDS up to
    K = 4096 and read per row beyond it; ragged M and N."""
    M, N = 304, 560
    log(f"[test_gemm_64] K={K} modes=({a_mode},{b_mode})")
    a = W.normal_tensor(M, K, seed=46)
    b = W.normal_tensor(N, K, seed=47, std=0.02)
    ac, as_, ag = oracle_operand(a, a_mode)
    bc, bs, bg = oracle_operand(b, b_mode)
    c = host(F.nvfp4_gemm(to_gpu(ac), to_gpu(as_), a_mode, sg_gpu(ag), to_gpu(bc), to_gpu(bs), b_mode,
                          sg_gpu(bg), M, N, K))
    ref = reference_rows(ac, as_, a_mode, ag, M, K) @ reference_rows(bc, bs, b_mode, bg, N, K).T
    err = np.linalg.norm(c.astype(np.float64) - ref) / np.linalg.norm(ref)
    row_err = np.linalg.norm(c.astype(np.float64) - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    assert err <= 1e-5 and row_err.max() <= 1e-5


def test_gemm_unaligned_scales_take_the_32_element_stages():
    """Scale arrays that are not 4-byte aligned (here a view one byte into a
    buffer) run the 32-element-stage kernel; same product."""
    M, N, K = 272, 400, 1024
    a = W.normal_tensor(M, K, seed=48)
    b = W.normal_tensor(N, K, seed=49, std=0.02)
    ac, as_, ag = oracle_operand(a, 1)
    bc, bs, bg = oracle_operand(b, 2)
    acd, asd, agd, bcd, bsd, bgd = to_gpu(ac), to_gpu(as_), sg_gpu(ag), to_gpu(bc), to_gpu(bs), sg_gpu(bg)
    shifted = torch.empty(asd.numel() + 1, dtype=torch.uint8, device="cuda")[1:].view(asd.shape)
    shifted.copy_(asd)
    c_ref = host(F.nvfp4_gemm(acd, asd, 1, agd, bcd, bsd, 2, bgd, M, N, K))
    c = host(F.nvfp4_gemm(acd, shifted, 1, agd, bcd, bsd, 2, bgd, M, N, K))
    ref = reference_rows(ac, as_, 1, ag, M, K) @ reference_rows(bc, bs, 2, bg, N, K).T
    for cc in (c, c_ref):
        assert np.linalg.norm(cc.astype(np.float64) - ref) / np.linalg.norm(ref) <= 1e-5


def test_minimum_shape_16x16():
    """The smallest tensor the 1D and 2D layouts take (one block per row and
    column, one tile, one workgroup holding a fraction of a tile): every
    path bit-identical to the oracle, and the 16 x 16 x 16 product within
    1e-5 of the oracle's."""
    x = W.normal_tensor(16, 16, seed=98)
    for rowwise, colwise, sr, rht in ((True, True, False, False), (True, True, True, False),
                                      (False, True, True, True)):
        got, a = run_q1(x, rowwise, colwise, sr, rht)
        check_q1(x, got, a, rowwise, colwise, sr, rht)
    ws = F.nvfp4_workspace()
    out = F.nvfp4_quantize_1d_fused(dev(x), ws, rowwise=True, colwise=True)
    got = {k: host(v) for k, v in out.items()}
    check_q1(x, got, host(ws)[:1].view(np.float32)[0], True, True, False, False)
    sg = oracle.global_scale(oracle.amax(x))
    cr, cc, s2 = oracle.quantize_2d(x, sg)
    q2 = F.nvfp4_quantize_2d(dev(x), F.nvfp4_amax(dev(x)))
    assert np.array_equal(host(q2["codes_row"]), cr) and np.array_equal(host(q2["codes_col"]), cc)
    assert np.array_equal(host(q2["scales"]), s2)
    codes, scales = oracle.quantize_1d_rows(x, sg)
    y = host(F.nvfp4_dequantize(to_gpu(codes), to_gpu(scales), 1, sg_gpu(sg), 16, 16))
    assert np.array_equal(y.view(np.uint32), oracle.dequantize(codes, scales, 1, sg, 16, 16).view(np.uint32))
    b = W.normal_tensor(16, 16, seed=99, std=0.02)
    err, _ = gemm_check(x, b, np.arange(16))
    assert err <= 1e-5


def test_gemm_half_tiles_equal_whole_tiles():
    """A last round of at most half the grid runs as 256 x 128 half tiles:
    the 1024 x 2048 product (32 tiles, all halved) equals the same block of
    the 4096 x 4096 product (256 whole tiles, one full round on 256 CUs)
    bit for bit, from the same operand bytes; both within 1e-5 of the
    oracle."""
    K = 512
    a = W.normal_tensor(4096, K, seed=93)
    b = W.normal_tensor(4096, K, seed=94, std=0.02)
    ac, as_, ag = oracle_operand(a, 1)
    bc, bs, bg = oracle_operand(b, 2)
    big = host(F.nvfp4_gemm(to_gpu(ac), to_gpu(as_), 1, sg_gpu(ag), to_gpu(bc), to_gpu(bs), 2, sg_gpu(bg),
                            4096, 4096, K))
    small = host(F.nvfp4_gemm(to_gpu(ac[:1024]), to_gpu(as_[:1024]), 1, sg_gpu(ag), to_gpu(bc[:2048]),
                              to_gpu(bs[:128]), 2, sg_gpu(bg), 1024, 2048, K))
    assert np.array_equal(small.view(np.uint32), big[:1024, :2048].view(np.uint32))
    rows = np.arange(0, 1024, 37, dtype=np.int64)
    ref = oracle.gemm_rows(ac, as_, 1, ag, bc[:2048], bs[:128], 2, bg, 4096, 2048, K, rows)
    assert np.linalg.norm(small[rows] - ref) / np.linalg.norm(ref) <= 1e-5


def test_gemm_bf16_output_is_rounded_fp32():
    a = W.normal_tensor(272, 528, seed=42)
    b = W.normal_tensor(400, 528, seed=43, std=0.02)
    _, c32 = gemm_check(a, b, np.arange(16))
    err16, c16 = gemm_check(a, b, np.arange(272), out_dtype=torch.bfloat16)
    assert np.array_equal(W.f32_to_bf16_bits(c32), W.f32_to_bf16_bits(c16))
    assert err16 <= 2.0 ** -8


# ------------------------------------------------ fused amax + quantize

@pytest.mark.parametrize("name,sr", [("act_small", False), ("ragged_act", False), ("ragged_act", True),
                                     ("act", False), ("act", True), ("grad", False)])
@pytest.mark.parametrize("layouts", [(True, True), (True, False), (False, True)])
def test_fused_amax_quantize(name, sr, layouts):
    """One call computes the amax and quantizes (a single pass over the
    tensor when it fits on chip, else the two-pass path): bit-identical to
    the oracle, and to the two-call path."""
    rowwise, colwise = layouts
    x = wl(name)
    log(f"[test_fused_amax_quantize] {name} sr={sr} layouts={layouts}")
    xd = dev(x)
    ws = F.nvfp4_workspace()
    got = None
    for rep in range(2):  # the workspace is reused as is
        out = F.nvfp4_quantize_1d_fused(xd, ws, rowwise=rowwise, colwise=colwise, sr=sr, seed=SEED)
        torch.cuda.synchronize()
        got = {k: host(v) for k, v in out.items()}
        wsh = host(ws)
        assert wsh[2] == 0, "in-kernel exchange fell back to the slow path"
        # a single pass moves the generation by one per call (the two-pass
        # path, for tensors that do not fit on chip, leaves it); with no
        # expired wait nothing is counted in words 4..5
        assert wsh[1] in (0, rep + 1) and wsh[4] == 0 and wsh[5] == 0, (wsh[1], wsh[4], wsh[5])
        amax_gpu = wsh[:1].view(np.float32)[0]
        check_q1(x, got, amax_gpu, rowwise, colwise, sr, False)
    two, _ = run_q1(x, rowwise, colwise, sr=sr)
    for k in two:
        assert np.array_equal(got[k], two[k]), k


@pytest.mark.parametrize("sr,layouts", [(False, (True, True)), (True, (True, True)), (False, (True, False)),
                                       (False, (False, True))])
def test_fused_exchange_fallback_forced(sr, layouts):
    """Word 3 of the workspace set to one tick makes the exchange's waits
    expire at once, so workgroups take the direct amax: the outputs are
    still bit-identical to the oracle, the slow-path counter moves, and the
    same workspace then serves a normal call (word 3 back to 0)."""
    rowwise, colwise = layouts
    x = W.activation(1024, 1280, seed=17)  # 4 x 5 workgroups: the release is never there in time
    log(f"[test_fused_exchange_fallback_forced] sr={sr} layouts={layouts}")
    xd = dev(x)
    ws = F.nvfp4_workspace()
    ws[3] = 1
    out = F.nvfp4_quantize_1d_fused(xd, ws, rowwise=rowwise, colwise=colwise, sr=sr, seed=SEED)
    torch.cuda.synchronize()
    wsh = host(ws)
    assert wsh[2] > 0, "no workgroup took the direct amax"
    got = {k: host(v) for k, v in out.items()}
    check_q1(x, got, wsh[:1].view(np.float32)[0], rowwise, colwise, sr, False)
    slow = int(wsh[2])
    ws[3] = 0
    out = F.nvfp4_quantize_1d_fused(xd, ws, rowwise=rowwise, colwise=colwise, sr=sr, seed=SEED)
    torch.cuda.synchronize()
    wsh = host(ws)
    assert int(wsh[2]) == slow, "the exchange fell back again with the default wait"
    got2 = {k: host(v) for k, v in out.items()}
    for k in got:
        assert np.array_equal(got[k], got2[k]), k


@pytest.mark.parametrize("sr,layouts", [(False, (True, True)), (True, (True, True)), (False, (True, False)),
                                       (True, (False, True))])
def test_fused_fallback_then_smaller_tensor(sr, layouts):
    """A call whose exchange waits all expire (word 3 = one tick) on a tensor
    with a large amax, then a normal call on another tensor with a much
    smaller amax through the same workspace. The generation advances only
    after every workgroup of a call has read it, so no workgroup of the
    first call can post its maximum under the second call's generation: the
    second call's amax and every code and scale byte are the oracle's for
    its own tensor. The generation word moves by one per call; after the
    expired call, words 4..5 hold its generation as the tag and the number
    of its workgroups that went through an expired wait (all 20 when
    workgroup 0's own wait expired; fewer when workgroup 0 still saw every
    arrival on its first look), and the normal call leaves them."""
    rowwise, colwise = layouts
    log(f"[test_fused_fallback_then_smaller_tensor] sr={sr} layouts={layouts}")
    big = W.f32_to_bf16_bits(W.bf16_bits_to_f32(W.activation(1024, 1280, seed=31)) * np.float32(1e4))
    small = W.activation(1024, 1280, seed=32)
    ws = F.nvfp4_workspace()
    ws[3] = 1
    out = F.nvfp4_quantize_1d_fused(dev(big), ws, rowwise=rowwise, colwise=colwise, sr=sr, seed=SEED)
    wsh = host(ws)
    assert wsh[2] > 0, "no workgroup took the direct amax"
    grid = 4 * 5  # pairs of 128-row tiles x 256-column tiles
    assert wsh[1] == 1 and wsh[4] == 1 and 1 <= wsh[5] <= grid, (wsh[1], wsh[4], wsh[5])
    expired = int(wsh[5])
    check_q1(big, {k: host(v) for k, v in out.items()}, wsh[:1].view(np.float32)[0], rowwise, colwise, sr,
             False)
    ws[3] = 0
    out = F.nvfp4_quantize_1d_fused(dev(small), ws, rowwise=rowwise, colwise=colwise, sr=sr, seed=SEED)
    wsh = host(ws)
    assert wsh[1] == 2 and wsh[4] == 1 and wsh[5] == expired, (wsh[1], wsh[4], wsh[5])
    a = wsh[:1].view(np.float32)[0]
    assert f32_bits(a) == f32_bits(oracle.amax(small))
    check_q1(small, {k: host(v) for k, v in out.items()}, a, rowwise, colwise, sr, False)


def test_fused_workspace_across_tensors():
    """Consecutive fused calls on different tensors through one workspace."""
    ws = F.nvfp4_workspace()
    for seed, scale in ((21, 1.0), (22, 1e-3), (23, 300.0)):
        x = W.f32_to_bf16_bits(W.bf16_bits_to_f32(W.activation(640, 768, seed=seed)) * np.float32(scale))
        out = F.nvfp4_quantize_1d_fused(dev(x), ws, rowwise=True, colwise=True)
        torch.cuda.synchronize()
        got = {k: host(v) for k, v in out.items()}
        check_q1(x, got, host(ws)[:1].view(np.float32)[0], True, True, False, False)
