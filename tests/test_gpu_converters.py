"""The gfx950 E2M1 converters, as the quantize kernels call them, against
the oracle's rounding rules on every input.

Round to nearest even ("MXFP4 和 NVFP4 的区别", section "随机舍入": weights
and activations round to nearest): every non-NaN binary32 pattern goes
through the library's encoder on the GPU (tests/native/converter_probe.hip
includes the library's own encode.h), which reports the patterns where the
code changes. Within each such run the hardware code is constant; the
oracle's rule is a nondecreasing step function of the value (pinned on the
CPU), so it equals the hardware on the whole run when it does at both ends.
The oracle is evaluated at every run's first and last pattern.

Stochastic rounding (same section: gradients round up with probability
(v - lo)/(hi - lo)): for each of about 77,000 values, every one of the 65,536
16-bit draws goes through the hardware converter with the library's input
mapping (both halves of a Philox word; the 2^23 operand scaling applied by
the encoder, or carried by the multiplier as the columnwise kernels fold it)
and through the software encoder.
The probe reports the code at h = 0 and h = 65535 and the number of draws
giving the h = 0 code, and checks that those draws come first and that the
encoders agree. The oracle's rule rounds up exactly for the lowest draws
(pinned on the CPU), so it equals the hardware on all draws when it does at
h = 0, h = 65535 and on both sides of the threshold.
"""
import ctypes
import importlib.util
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))

P = None


def setup_module(module):
    global P
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec = importlib.util.spec_from_file_location("converter_probe_build", os.path.join(HERE, "native", "build.py"))
    probe_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(probe_build)

    if not os.path.exists(probe_build.LIB_PATH):
        probe_build.build()
    P = ctypes.CDLL(probe_build.LIB_PATH)
    P.probe_rne_runs.restype = ctypes.c_int
    P.probe_rne_runs.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint32,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P.probe_sr_thresholds.restype = ctypes.c_int
    P.probe_sr_thresholds.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def log(msg):
    print(msg, flush=True)


def rne_runs(lo, hi, cap=1 << 16):
    runs = torch.zeros(2 * cap, dtype=torch.int32, device="cuda")
    counters = torch.zeros(2, dtype=torch.int32, device="cuda")
    st = P.probe_rne_runs(lo, hi, ctypes.c_void_p(runs.data_ptr()), cap, ctypes.c_void_p(counters.data_ptr()),
                          ctypes.c_void_p(counters.data_ptr() + 4), stream())
    assert st == 0
    torch.cuda.synchronize()
    count, mismatch = (int(v) for v in counters.cpu().numpy())
    assert count <= cap
    r = runs.cpu().numpy()[: 2 * count].view(np.uint32).reshape(count, 2)
    return r[np.argsort(r[:, 0])], mismatch


@pytest.mark.parametrize("sign", [0, 1])
def test_rne_converter_every_pattern(sign):
    base = np.uint32(sign << 31)
    lo, hi = int(base), int(base | np.uint32(0x7F800000))  # +-0 .. +-inf, every finite value between
    log(f"[test_rne_converter_every_pattern] patterns {lo:#x}..{hi:#x}")
    runs, mismatch = rne_runs(lo, hi)
    assert mismatch == 0, "a byte position or nibble of the encoder gave another code"
    assert runs[0, 0] == lo
    starts = runs[:, 0].astype(np.uint64)
    ends = np.append(starts[1:] - 1, hi).astype(np.uint32)
    codes = runs[:, 1]
    # every run's code carries the sign, and the magnitudes rise run by run
    assert np.all((codes >> 3) == sign)
    assert np.all(np.diff(codes & 7) > 0)
    for pats in (starts.astype(np.uint32), ends):
        v = pats.view(np.float32)
        want = oracle.e2m1_rne_array(np.abs(v)) | np.uint8(sign << 3)
        assert np.array_equal(codes.astype(np.uint8), want), (pats, codes, want)
    assert len(runs) == 8  # one run per magnitude code 0..7
    log(f"  runs start at {[hex(int(s)) for s in starts]}")


def sr_values():
    rng = np.random.default_rng(12)
    parts = []
    for e in range(-40, 3):  # random mantissas in every binade 2^-40 .. 8
        parts.append((np.float32(2.0 ** e) * (1 + rng.random(600, dtype=np.float32))).astype(np.float32))
    pts = [0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6]
    for p in pts:  # every float within 300 ulp of each grid point and midpoint
        u = int(np.float32(p).view(np.uint32))
        parts.append(np.arange(u - 300, u + 301, dtype=np.uint32).view(np.float32))
    parts.append(np.arange(0, 1 << 12, dtype=np.uint32).view(np.float32))  # zero and subnormals
    parts.append(np.array([6.5, 7.0, 1e9, 3.4e38, np.inf], np.float32))  # saturation
    v = np.concatenate(parts)
    return np.concatenate([v, -v]).astype(np.float32)


def test_sr_converter_every_draw():
    v = sr_values()
    n = v.size
    log(f"[test_sr_converter_every_draw] {n} values x 65536 draws")
    vd = torch.from_numpy(v).cuda()
    out = torch.zeros(4 * n, dtype=torch.int32, device="cuda")
    assert P.probe_sr_thresholds(ctypes.c_void_p(vd.data_ptr()), n, ctypes.c_void_p(out.data_ptr()), stream()) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().view(np.uint32).reshape(n, 4)
    c0, c1, count, flags = o[:, 0], o[:, 1], o[:, 2].astype(np.int64), o[:, 3]
    bad = np.nonzero(flags != 7)[0]
    assert bad.size == 0, f"encoders disagree or codes are not a prefix at {v[bad[:8]]} (flags {flags[bad[:8]]})"
    sign = (np.signbit(v).astype(np.uint8) << 3)
    mag = np.abs(v)

    def want(h, idx=slice(None)):
        return oracle.e2m1_sr_array(mag[idx], np.asarray(h).astype(np.uint16)) | sign[idx]

    assert np.array_equal(c0.astype(np.uint8), want(np.zeros(n)))
    assert np.array_equal(c1.astype(np.uint8), want(np.full(n, 65535)))
    same = c0 == c1
    assert np.all(count[same] == 65536)
    split = ~same
    assert np.all((count[split] >= 1) & (count[split] <= 65535))
    # both sides of each threshold
    assert np.array_equal(want(count[split] - 1, split), c0[split].astype(np.uint8))
    assert np.array_equal(want(count[split], split), c1[split].astype(np.uint8))
    # not vacuous: most values in range split between two codes
    assert split.mean() > 0.8
