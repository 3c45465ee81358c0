"""nvfp4_quantize_1d_fused_noalloc (the library's static workspace) against
nvfp4_quantize_1d_fused (a caller's workspace): bit-identical outputs and
amax, over consecutive calls whose second input is smaller, through the C
ABI. Outputs are preallocated, so the calls under test allocate nothing."""
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

F = None


def setup_module(module):
    global F
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_block_scaled_amax_amd as pkg

    pkg.lib()
    F = pkg


def dev(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda()


def outputs(R, C, rowwise, colwise):
    o = {"global_scale": torch.empty(1, dtype=torch.float32, device="cuda")}
    if rowwise:
        o["codes_row"] = torch.empty((R, C // 2), dtype=torch.uint8, device="cuda")
        o["scales_row"] = torch.empty((R, C // 16), dtype=torch.uint8, device="cuda")
    if colwise:
        o["codes_col"] = torch.empty((C, R // 2), dtype=torch.uint8, device="cuda")
        o["scales_col"] = torch.empty((C, R // 16), dtype=torch.uint8, device="cuda")
    return o


@pytest.mark.parametrize("sr,layouts", [(False, (True, True)), (True, (True, True)), (False, (True, False)),
                                       (True, (False, True))])
def test_noalloc_equals_workspace_call(sr, layouts):
    rowwise, colwise = layouts
    # the benchmarked activation (single pass), then a smaller tensor with a
    # different amax, then a tensor too large for one pass (two-pass path),
    # then a small one again
    inputs = [W.activation(8192, 4096, seed=1), W.activation_small(256, 1024, seed=0),
              W.gradient(8192, 14336, seed=3), W.activation(528, 784, seed=12)]
    ws = F.nvfp4_workspace()
    for i, x in enumerate(inputs):
        print(f"[test_noalloc_equals_workspace_call] sr={sr} layouts={layouts} input {i} {x.shape}", flush=True)
        sys.stdout.flush()
        xd = dev(x)
        R, C = x.shape
        want = outputs(R, C, rowwise, colwise)
        got = outputs(R, C, rowwise, colwise)
        amax = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        F.nvfp4_quantize_1d_fused(xd, ws, rowwise=rowwise, colwise=colwise, sr=sr, seed=42, out=want)
        F.nvfp4_quantize_1d_fused_noalloc(xd, rowwise=rowwise, colwise=colwise, sr=sr, seed=42, out=got,
                                          amax=amax)
        torch.cuda.synchronize()
        assert torch.equal(amax.view(torch.int32), ws[:1]), "amax differs"
        for k in want:
            assert torch.equal(got[k].view(torch.uint8), want[k].view(torch.uint8)), f"{k} differs"
        del xd, want, got
    # the amax output is optional
    x = W.activation(256, 512, seed=13)
    o = outputs(256, 512, True, True)
    F.nvfp4_quantize_1d_fused_noalloc(dev(x), rowwise=True, colwise=True, out=o)
    w = outputs(256, 512, True, True)
    F.nvfp4_quantize_1d_fused(dev(x), ws, rowwise=True, colwise=True, out=w)
    torch.cuda.synchronize()
    for k in w:
        assert torch.equal(o[k].view(torch.uint8), w[k].view(torch.uint8)), k
