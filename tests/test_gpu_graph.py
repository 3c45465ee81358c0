"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph):
the fused amax + quantize, the transform + stochastic-rounding quantize and
the GEMM with its epilogue amax are captured once and replayed several
times, with eager work and synchronizations between the replays; every
replay must equal the eager result bit for bit. The library records no
memset node: its resets are kernels."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import workloads as W

pytestmark = pytest.mark.gpu

F = None
SEED = W.SR_SEED


def setup_module(module):
    global F
    import fp4_block_scaled_amax_amd as pkg

    pkg.lib()  # raises if the HIP library is missing: no fallback
    F = pkg


def dev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()


def snapshot(tensors):
    torch.cuda.synchronize()
    return [t.clone() for t in tensors]


def test_replays_equal_eager():
    x = dev(W.activation(2048, 4096, seed=95))
    g = dev(W.gradient(1024, 2048, seed=96))
    b = dev(W.weight(1024, 4096, seed=97))
    mask = W.rht_sign_mask()
    ws = F.nvfp4_workspace()
    qb = F.nvfp4_quantize_2d(b, F.nvfp4_amax(b), colwise=False)
    ga = torch.empty(1, dtype=torch.float32, device="cuda")
    c_amax = torch.empty(1, dtype=torch.float32, device="cuda")

    def work():
        q = F.nvfp4_quantize_1d_fused(x, ws, rowwise=True, colwise=True)
        F.nvfp4_amax(g, rht=True, rht_mask=mask, out=ga)
        qg = F.nvfp4_quantize_1d(g, ga, rowwise=False, colwise=True, sr=True, rht=True, rht_mask=mask,
                                 seed=SEED)
        c = F.nvfp4_gemm(q["codes_row"], q["scales_row"], 1, q["global_scale"], qb["codes_row"], qb["scales"],
                         2, qb["global_scale"], 2048, 1024, 4096, out_dtype=torch.bfloat16, out_amax=c_amax)
        return [q["codes_row"], q["scales_row"], q["codes_col"], q["scales_col"], q["global_scale"],
                qg["codes_col"], qg["scales_col"], c, c_amax]

    eager = snapshot(work())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as capture requires
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = work()
    for rep in range(4):
        for t in outs:
            t.zero_()  # the replay must rewrite every output
        graph.replay()
        got = snapshot(outs)
        for i, (a, e) in enumerate(zip(got, eager)):
            assert torch.equal(a.view(torch.uint8), e.view(torch.uint8)), f"replay {rep}, output {i}"
        # eager work of the program between replays
        F.nvfp4_quantize_1d_fused(x, ws, rowwise=True, colwise=False)
        torch.cuda.synchronize()
