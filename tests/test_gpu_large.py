"""A tensor past 2^31 elements (65552 x 32768 bf16, 4.3 GB): every element
offset in the 1D path is 64-bit. The amax (plain and of the 16-point
Hadamard transform) must equal the oracle's over the whole tensor; rowwise
and columnwise codes and scales (round-to-nearest-even and stochastic) must
equal the oracle's on sampled rows and columns, the rows taken on both
sides of element 2^31 (row 65536); the bf16 dequantization of those rows
must equal the oracle's decode of its own codes."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

F = None
SEED = W.SR_SEED
ROWS = [0, 1, 15, 16, 30001, 65519, 65535, 65536, 65537, 65550, 65551]
COLS = [0, 1, 4095, 16384, 32766, 32767]


def setup_module(module):
    global F
    import fp4_block_scaled_amax_amd as pkg

    pkg.lib()  # raises if the HIP library is missing: no fallback
    F = pkg


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(v) -> int:
    return int(np.float32(v).view(np.uint32))


def threaded_max(fn, R: int):
    """max of fn(r0, r1) over 16-row-aligned ranges of R rows, in threads."""
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    step = -(-(-(-R // n)) // 16) * 16
    with ThreadPoolExecutor(n) as ex:
        return max(ex.map(lambda r0: fn(r0, min(R, r0 + step)), range(0, R, step)))


def test_past_2_31_elements():
    log("[test_past_2_31_elements] generating 65552x32768")
    x = W.large_tensor()
    R, C = x.shape
    assert R * C > 2 ** 31 and ROWS[-1] < R and COLS[-1] < C
    xd = torch.from_numpy(x.view(np.int16)).cuda()

    log("[test_past_2_31_elements] amax")
    a_ref = threaded_max(lambda r0, r1: oracle.amax(x[r0:r1]), R)
    amax = F.nvfp4_amax(xd)
    assert bits(host(amax)[0]) == bits(a_ref)
    sg = oracle.global_scale(a_ref)

    for sr in (False, True):
        log(f"[test_past_2_31_elements] quantize rowwise + columnwise sr={sr}")
        q = F.nvfp4_quantize_1d(xd, amax, rowwise=True, colwise=True, sr=sr, seed=SEED)
        assert bits(host(q["global_scale"])[0]) == bits(sg)
        rows = torch.tensor(ROWS, device="cuda")
        cr, sr_ = host(q["codes_row"][rows]), host(q["scales_row"][rows])
        for i, r in enumerate(ROWS):
            c, s = oracle.quantize_1d_rows(x, sg, sr, SEED, r, r + 1)
            assert np.array_equal(cr[i], c[0]) and np.array_equal(sr_[i], s[0]), f"row {r}"
            if not sr and r in (65535, 65536, 65551):
                log(f"[test_past_2_31_elements] dequantize row {r}")
                y = F.nvfp4_dequantize(q["codes_row"], q["scales_row"], 1, q["global_scale"], R, C,
                                       out_dtype=torch.bfloat16)
                got = host(y[r].view(torch.int16)).view(np.uint16)
                want = oracle.dequantize_bf16(c, s, 1, sg, 1, C)[0]
                assert np.array_equal(got, want), f"dequantized row {r}"
                del y
        cols = torch.tensor(COLS, device="cuda")
        cc, sc = host(q["codes_col"][cols]), host(q["scales_col"][cols])
        for i, col in enumerate(COLS):
            c, s = oracle.quantize_1d_cols(x, sg, sr, SEED, False, 0, col, col + 1)
            assert np.array_equal(cc[i], c[0]) and np.array_equal(sc[i], s[0]), f"column {col}"
        del q
        torch.cuda.empty_cache()

    mask = W.rht_sign_mask()
    log("[test_past_2_31_elements] amax of the Hadamard transform")
    a_rht = threaded_max(lambda r0, r1: oracle.amax_rht(x[r0:r1], mask), R)
    amax_t = F.nvfp4_amax(xd, rht=True, rht_mask=mask)
    assert bits(host(amax_t)[0]) == bits(a_rht)
    sg_t = oracle.global_scale(a_rht)
    log("[test_past_2_31_elements] columnwise Hadamard + stochastic rounding")
    q = F.nvfp4_quantize_1d(xd, amax_t, rowwise=False, colwise=True, sr=True, seed=SEED, rht=True, rht_mask=mask)
    cols = torch.tensor(COLS, device="cuda")
    cc, sc = host(q["codes_col"][cols]), host(q["scales_col"][cols])
    for i, col in enumerate(COLS):
        c, s = oracle.quantize_1d_cols(x, sg_t, True, SEED, True, mask, col, col + 1)
        assert np.array_equal(cc[i], c[0]) and np.array_equal(sc[i], s[0]), f"transformed column {col}"


def rel_rows(got, ref):
    return (np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)).max()


def test_gemm_output_past_2_31_elements():
    """C of 65552 x 32768 (2^31 + 2^19 elements) from K = 64: NVFP4 (fp32 and
    bf16 C) and MXFP4 products of the oracle's operands, rows either side of
    element 2^31 within 1e-5 of the oracle's double product."""
    M, N, K = 65552, 32768, 64
    a = W.normal_tensor(M, K, seed=91)
    b = W.normal_tensor(N, K, seed=92, std=0.02)
    rows = np.array([0, 1, 30001, 65535, 65536, 65537, 65551], np.int64)
    to_gpu = lambda v: torch.from_numpy(np.ascontiguousarray(v)).cuda()
    sg_gpu = lambda v: torch.tensor([float(np.float32(v))], dtype=torch.float32, device="cuda")
    ag = oracle.global_scale(oracle.amax(a))
    ac, as_ = oracle.quantize_1d_rows(a, ag)
    bg = oracle.global_scale(oracle.amax(b))
    bc, _, bs = oracle.quantize_2d(b, bg)
    ref = oracle.gemm_rows(ac, as_, 1, ag, bc, bs, 2, bg, M, N, K, rows)
    sel = torch.tensor(rows, device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        log(f"[test_gemm_output_past_2_31_elements] NVFP4 {dt}")
        c = F.nvfp4_gemm(to_gpu(ac), to_gpu(as_), 1, sg_gpu(ag), to_gpu(bc), to_gpu(bs), 2, sg_gpu(bg),
                         M, N, K, out_dtype=dt)
        got = host(c[sel].float()).astype(np.float64)
        del c
        torch.cuda.empty_cache()
        assert rel_rows(got, ref) <= (1e-5 if dt == torch.float32 else 2.0 ** -8)
    log("[test_gemm_output_past_2_31_elements] MXFP4 float32")
    mac, mas = oracle.mx_quantize_rows(a)
    mbc, mbs = oracle.mx_quantize_rows(b)
    mref = oracle.mx_gemm_rows(mac, mas, mbc, mbs, M, N, K, rows)
    c = F.mxfp4_gemm(to_gpu(mac), to_gpu(mas), to_gpu(mbc), to_gpu(mbs), M, N, K)
    got = host(c[sel]).astype(np.float64)
    assert rel_rows(got, mref) <= 1e-5
