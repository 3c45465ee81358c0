#!/usr/bin/env python3
"""NVFP4 quantization benchmark on one MI355X.

Timed step (the workload the metric is quoted on): the 8192x4096 bf16
activation (tokens x hidden, N(0,1) with 8 outlier columns x100) goes
through the whole 1D path -- tensor amax, global scale, E4M3 block scales,
E2M1 round-to-nearest-even and packing -- emitting both the rowwise (fprop)
and the columnwise (wgrad) layouts, in one call (nvfp4_quantize_1d_fused: a single
pass over the tensor, which stays in registers between the amax and the
encoding). `value` is the step's algorithmic bytes
-- the input read once (2 B/element) plus the two outputs (2 x 0.5625
B/element) -- per second.

The other rows of the path are timed in the same run, each on its own
workload, and reported under "rows": the Hadamard + stochastic-rounding
gradient quantization (8192x14336 gradient and the activation), the 2D
weight quantization (14336x4096), the standalone transform, dequantization
and the dequantize-and-contract GEMM (8192x14336x4096, TFLOP/s).

Prints one JSON line. Inputs are synthetic (seeded), resident in HBM before
timing starts; the timed loop rotates over input copies whose total exceeds
the 256 MB Infinity Cache, so each step reads its input from HBM (the warm
figure, one copy served from that cache, is a separate row).

CPU figures, from the CPU oracle on the host: `cpu_baseline` (the step's
work on the activation, one thread), `cpu_baseline_all_cores` (the same
functions over row and column ranges on every core, checked byte-identical)
and `cpu_gemm_reference` (the fp64 product of 256 sampled GEMM rows).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
ALU_NOTE = ("vector-ALU bound, not HBM: Philox (two 32x32->64 multiplies per round, 10 rounds per "
            "8 elements), the 16-point butterfly and the SR encode; the HBM fraction is context")
F16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 (= bf16) matrix peak, TFLOP/s
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 (block-scaled) matrix peak, TFLOP/s
# Plain vector ALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one op per lane
# per clock, no packed math).
VALU_PEAK_GOPS = 256 * 4 * 16 * 2.4

METRIC = "NVFP4 quantize GB/s & % of HBM peak; NVFP4 dequant-GEMM TFLOP/s"
PROFILE_PMC = os.path.join(ROOT, "profiles", "quantize_rowcol_activation_8192x4096_traffic.md")
DOMINANT_SOURCES = [
    os.path.join(ROOT, "fp4_block_scaled_amax_amd", "csrc", "quantize.hip"),
    os.path.join(ROOT, "fp4_block_scaled_amax_amd", "csrc", "device.h"),
    os.path.join(ROOT, "fp4_block_scaled_amax_amd", "csrc", "encode.h"),
    os.path.join(ROOT, "fp4_block_scaled_amax_amd", "csrc", "quant_item.h"),
]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=5, help="input copies rotated in the timed loop")
    p.add_argument("--no-rows", action="store_true", help="skip the secondary per-row measurements")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--row-iters", type=int, default=10)
    p.add_argument("--calib-copy", action="store_true",
                   help="also run a plain 256 MiB device copy (counter calibration)")
    p.add_argument("--summarize-trace", metavar="DIR",
                   help="no GPU work: summarise a rocprofv3 --kernel-trace --marker-trace output directory of "
                        "a bench.py run per bench row (needs --bench-json)")
    p.add_argument("--bench-json", metavar="FILE", help="the JSON line that traced bench.py run printed")
    p.add_argument("--cpu-passes", type=int, default=3,
                   help="whole passes of the CPU oracle over its sample (about 10 s on one core)")
    p.add_argument("--cpu-rows", type=int, default=8192,
                   help="rows of the activation in the CPU baseline sample")
    p.add_argument("--no-cpu-gemm", action="store_true",
                   help="skip the CPU oracle's sampled GEMM reference")
    return p.parse_args()


def sources_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed
    counter summary, if it was taken on the current kernel source."""
    if not os.path.exists(PROFILE_PMC):
        return None
    text = open(PROFILE_PMC).read()
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sources_digest(DOMINANT_SOURCES):
        return None
    return float(m_b.group(1))


def host_threads() -> int:
    """Host threads for the all-cores oracle run: the CPUs this process may
    use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def split(n: int, parts: int, align: int):
    """[lo, hi) ranges covering 0..n, boundaries multiples of align."""
    step = -(-n // parts)
    step = -(-step // align) * align
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)]


def cpu_all_cores(oracle, sample, ref, args):
    """The same oracle functions on every host core: the amax over row
    ranges, then the rowwise layout over row ranges and the columnwise
    layout over column ranges, all with the one global scale; the result
    must equal the single-threaded call's byte for byte. The C functions
    release the interpreter lock, so threads run them in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    cores = host_threads()
    R_s, C_s = sample.shape
    rr, cr = split(R_s, cores, 16), split(C_s, cores, 1)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        a = max(ex.map(lambda r: oracle.amax(sample[r[0]:r[1]]), rr))
        sg = oracle.global_scale(a)
        rows = list(ex.map(lambda r: oracle.quantize_1d_rows(sample, sg, r0=r[0], r1=r[1]), rr))
        cols = list(ex.map(lambda c: oracle.quantize_1d_cols(sample, sg, c0=c[0], c1=c[1]), cr))
    t = time.perf_counter() - t0
    same = (np.float32(a) == np.float32(ref["amax"]) and
            np.array_equal(np.concatenate([r[0] for r in rows]), ref["codes_row"]) and
            np.array_equal(np.concatenate([r[1] for r in rows]), ref["scales_row"]) and
            np.array_equal(np.concatenate([c[0] for c in cols]), ref["codes_col"]) and
            np.array_equal(np.concatenate([c[1] for c in cols]), ref["scales_col"]))
    log(f"[bench] CPU oracle on {cores} threads: {t:.2f} s, identical={same}")
    return {"value": round(sample.size * 3.125 / t / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"same {R_s}x{C_s} sample; amax over {len(rr)} row ranges, rowwise over {len(rr)} row "
                      f"ranges, columnwise over {len(cr)} column ranges, one global scale",
            "seconds": round(t, 2), "identical_to_single_thread": bool(same)}


def cpu_gemm_reference(oracle, W):
    """The oracle's GEMM reference as the parity tests use it: the NVFP4
    operands of the 8192x14336x4096 product (quantized by the oracle), and
    the double-precision product of 256 sampled rows of A with all of B
    (B reconstructed once). The contraction runs in numpy's BLAS; its
    thread count is recorded."""
    from concurrent.futures import ThreadPoolExecutor

    a_bits, b_bits = W.gemm_operands()
    M, K = a_bits.shape
    N = b_bits.shape[0]
    rows = W.gemm_sample_rows()
    cores = host_threads()
    t0 = time.perf_counter()
    ag = oracle.global_scale(oracle.amax(a_bits))
    with ThreadPoolExecutor(cores) as ex:
        parts = list(ex.map(lambda r: oracle.quantize_1d_rows(a_bits, ag, r0=r[0], r1=r[1]),
                            split(M, cores, 16)))
    ac, as_ = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    bg = oracle.global_scale(oracle.amax(b_bits))
    bc, _, bs = oracle.quantize_2d(b_bits, bg)
    t_q = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gemm_rows(ac, as_, 1, ag, bc, bs, 2, bg, M, N, K, rows)
    t = time.perf_counter() - t0
    flop = 2.0 * rows.size * N * K
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                   default=1)
    except Exception:  # threadpoolctl missing or unreadable
        blas = None
    log(f"[bench] CPU oracle GEMM reference: {rows.size} rows in {t:.2f} s "
        f"({flop / t / 1e9:.1f} GFLOP/s, BLAS threads {blas})")
    return {"value": round(flop / t / 1e12, 5), "unit": "TFLOP/s", "cores": blas, "kind": "oracle",
            "sample": f"{rows.size} sampled rows of the {M}x{N}x{K} product in fp64 (A rows and all of B "
                      f"reconstructed exactly, then one BLAS product)",
            "seconds": round(t, 2), "operand_quantization_seconds": round(t_q, 2),
            "full_product_seconds_extrapolated": round(t * M / rows.size, 1)}


def error_study(F, tensors, mask, dev):
    """||x - x^||_F / ||x||_F of NVFP4 and MXFP4 (round-to-nearest-even) on
    each tensor: rowwise, columnwise, and columnwise after the 16-point
    Hadamard transform (measured against the transformed tensor, whose norm
    is the tensor's); the weight also with NVFP4's 16x16 tiles. Every step runs in the library's kernels; the
    norms are torch reductions in double precision."""
    torch = F._torch()
    out = {}

    def rel(ref, deq):
        ref = ref.double()
        return round(float(torch.linalg.vector_norm(deq.double() - ref) / torch.linalg.vector_norm(ref)), 5)

    for name, t in tensors.items():
        R, C = t.shape
        ref = t.view(torch.bfloat16).float()
        e = {}
        q = F.nvfp4_quantize_1d(t, F.nvfp4_amax(t), rowwise=True)
        e["nvfp4_1d_rowwise"] = rel(ref, F.nvfp4_dequantize(q["codes_row"], q["scales_row"], 1, q["global_scale"],
                                                             R, C))
        m = F.mxfp4_quantize(t)
        e["mxfp4_rowwise"] = rel(ref, F.mxfp4_dequantize(m["codes_row"], m["scales_row"], R, C))
        if name == "weight":
            q2 = F.nvfp4_quantize_2d(t, F.nvfp4_amax(t), colwise=False)
            e["nvfp4_2d"] = rel(ref, F.nvfp4_dequantize(q2["codes_row"], q2["scales"], 2, q2["global_scale"], R, C))
        # columnwise without the transform (blocks along the same axis as the
        # transformed layout), against the tensor itself
        tt = ref.t()
        q = F.nvfp4_quantize_1d(t, F.nvfp4_amax(t), rowwise=False, colwise=True)
        e["nvfp4_1d_colwise"] = rel(tt, F.nvfp4_dequantize(q["codes_col"], q["scales_col"], 1, q["global_scale"],
                                                           C, R))
        m = F.mxfp4_quantize(t, rowwise=False, colwise=True)
        e["mxfp4_colwise"] = rel(tt, F.mxfp4_dequantize(m["codes_col"], m["scales_col"], C, R))
        del ref, tt
        y = F.nvfp4_rht16(t, axis=0, rht_mask=mask).t()
        q = F.nvfp4_quantize_1d(t, F.nvfp4_amax(t, rht=True, rht_mask=mask), rowwise=False, colwise=True, rht=True,
                                rht_mask=mask)
        e["nvfp4_1d_colwise_rht"] = rel(y, F.nvfp4_dequantize(q["codes_col"], q["scales_col"], 1, q["global_scale"],
                                                               C, R))
        m = F.mxfp4_quantize(t, rowwise=False, colwise=True, rht=True, rht_mask=mask)
        e["mxfp4_colwise_rht"] = rel(y, F.mxfp4_dequantize(m["codes_col"], m["scales_col"], C, R))
        del y, q, m
        out[name] = e
        log(f"[bench] error {name}: " + ", ".join(f"{k} {v:.4f}" for k, v in e.items()))
    out["wgrad_product"] = wgrad_product_error(F, tensors["gradient"], tensors["activation"], mask)
    return out


def wgrad_product_error(F, dy, x, mask):
    """||dW - dY^T X||_F / ||dY^T X||_F for the weight gradient computed from
    columnwise operands (blocks along the tokens, round-to-nearest-even):
    NVFP4 and MXFP4, each without and with the shared Hadamard transform.
    The reference is a double-precision product on the GPU."""
    torch = F._torch()
    T, NO = dy.shape
    NI = x.shape[1]
    ref = torch.matmul(dy.view(torch.bfloat16).double().t().contiguous(),
                       x.view(torch.bfloat16).double().contiguous())
    nref = torch.linalg.vector_norm(ref)
    res = {}
    for rht in (False, True):
        tag = "rht" if rht else "no_rht"
        qs = []
        for t in (dy, x):
            a = F.nvfp4_amax(t, rht=rht, rht_mask=mask)
            qs.append(F.nvfp4_quantize_1d(t, a, rowwise=False, colwise=True, rht=rht, rht_mask=mask))
        c = F.nvfp4_gemm(qs[0]["codes_col"], qs[0]["scales_col"], 1, qs[0]["global_scale"], qs[1]["codes_col"],
                         qs[1]["scales_col"], 1, qs[1]["global_scale"], NO, NI, T)
        res[f"nvfp4_{tag}"] = round(float(torch.linalg.vector_norm(c.double() - ref) / nref), 5)
        ms = [F.mxfp4_quantize(t, rowwise=False, colwise=True, rht=rht, rht_mask=mask) for t in (dy, x)]
        c = F.mxfp4_gemm(ms[0]["codes_col"], ms[0]["scales_col"], ms[1]["codes_col"], ms[1]["scales_col"], NO, NI, T)
        res[f"mxfp4_{tag}"] = round(float(torch.linalg.vector_norm(c.double() - ref) / nref), 5)
        del qs, ms, c
    log("[bench] error wgrad product dY^T X: " + ", ".join(f"{k} {v:.4f}" for k, v in res.items()))
    return res


def summarize_trace(trace_dir, bench_json):
    """Per bench row: the kernels rocprofv3 traced inside the row's ROCTx
    range (its timed calls only), with launches and average duration, the
    kernel time per call (launch latency and the gaps between kernels left
    out) and the fraction of peak it gives, next to the row's own
    event-timed figure from the same run. Prints markdown."""
    import csv
    import glob

    def one(pattern):
        files = sorted(glob.glob(os.path.join(trace_dir, "**", pattern), recursive=True))
        if not files:
            raise SystemExit(f"no {pattern} under {trace_dir}")
        return list(csv.DictReader(open(files[0])))

    kernels = one("*kernel_trace.csv")
    markers = one("*marker_api_trace.csv")
    line = json.loads(open(bench_json).read().strip().splitlines()[-1])
    rows = dict(line.get("rows", {}))
    rows["step"] = {"us": line["roofline"]["avg_launch_us"], "calls": line["steps"],
                    "alg_bytes": line["roofline"]["alg_bytes_per_launch"], "peak": HBM_PEAK_GBS}
    ranges = {}
    for m in markers:
        label = next((v for v in m.values() if isinstance(v, str) and v.startswith("row:")), None)
        if label:
            ranges[label[4:]] = (int(m["Start_Timestamp"]), int(m["End_Timestamp"]))
    grid_key = next(k for k in kernels[0] if k.startswith("Grid_Size"))
    out = ["| row | kernel | grid | launches | avg µs | kernel µs per call | alg. work per call | "
           "kernel-only rate | frac | event-timed µs per call (same run) |", "|---|---|---|---:|---:|---:|---:|---:|"
           "---:|---:|"]
    for name, (t0, t1) in ranges.items():
        inside = [k for k in kernels if t0 <= int(k["Start_Timestamp"]) <= t1]
        groups = {}
        for k in inside:
            kname = k["Kernel_Name"].replace("(anonymous namespace)::", "")
            kname = re.sub(r"\([^()]*\)$", "", kname.strip())  # the parameter list
            key = (kname.replace("void ", "")[-80:], k[grid_key])
            groups.setdefault(key, []).append((int(k["End_Timestamp"]) - int(k["Start_Timestamp"])) / 1e3)
        row = rows.get(name, {})
        calls = row.get("calls") or 1
        per_call = sum(sum(v) for v in groups.values()) / calls
        work = row.get("alg_bytes") or row.get("flop")
        rate = frac = ""
        work_s = f"{work:.4g}" if work else ""
        if work and per_call > 0:
            if "flop" in row and "alg_bytes" not in row:
                r = work / (per_call * 1e-6) / 1e12
                rate = f"{r:.1f} TFLOP/s"
                frac = f"{r / row['peak']:.3f}" if row.get("peak") else ""
            else:
                r = work / (per_call * 1e-6) / 1e9
                rate = f"{r:.0f} GB/s"
                frac = f"{r / HBM_PEAK_GBS:.3f}"
        first = True
        for (kname, grid), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            out.append(f"| {name if first else ''} | `{kname}` | {grid} | {len(ds)} | {statistics.mean(ds):.2f} | "
                       + (f"{per_call:.2f} | {work_s} | {rate} | {frac} | {row.get('us', '')} |" if first
                          else "| | | | |"))
            first = False
    print("\n".join(out))


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.bench_json)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(there is no multi-GPU path: every block is independent, and only the tensor amax "
              "would need an all-reduce across GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import fp4_block_scaled_amax_amd as F
    import workloads as W

    F.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)

    # ---------------------------------------------------------- timed step
    R, C = 8192, 4096
    n = R * C
    log("[bench] generating the 8192x4096 activation")
    x_host = W.activation(R, C)
    xs = [to_dev(x_host) for _ in range(args.copies)]
    amax = torch.empty(1, dtype=torch.float32, device=dev)
    ws = F.nvfp4_workspace(dev)
    outs = []
    for _ in range(args.copies):
        outs.append({
            "codes_row": torch.empty((R, C // 2), dtype=torch.uint8, device=dev),
            "scales_row": torch.empty((R, C // 16), dtype=torch.uint8, device=dev),
            "codes_col": torch.empty((C, R // 2), dtype=torch.uint8, device=dev),
            "scales_col": torch.empty((C, R // 16), dtype=torch.uint8, device=dev),
            "global_scale": torch.empty(1, dtype=torch.float32, device=dev),
        })
    quant_bytes = n * (2 + 2 * (0.5 + 1 / 16))
    step_bytes = quant_bytes

    ev_q0 = torch.cuda.Event(enable_timing=True)
    ev_q1 = torch.cuda.Event(enable_timing=True)

    def step(k):
        x = xs[k % args.copies]
        o = outs[k % args.copies]
        F.nvfp4_quantize_1d_fused(x, ws, rowwise=True, colwise=True, out=o)

    if args.calib_copy:
        # A plain copy of known size: reads and writes 256 MiB each. Hardware
        # byte counters of the dominant kernel are scaled by what they read here.
        src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    log(f"[bench] warmup {args.warmup} steps")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # The K timed steps are captured once in a HIP graph (the launch-bound
    # loop then runs without the host's per-call overhead) and replayed once
    # as the timed region.
    step_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(step_graph):
        for k in range(args.steps):
            step(k)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.nvtx.range_push("row:step")
    t0 = time.perf_counter()
    ev_q0.record(stream)
    step_graph.replay()
    ev_q1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    torch.cuda.nvtx.range_pop()
    del step_graph
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes / (elapsed / args.steps) / 1e9
    # The dominant kernel's average launch duration: HIP events on its
    # stream around the timed region, which is K back-to-back launches of it
    # (one graph replay) and nothing else.
    q_avg_ms = ev_q0.elapsed_time(ev_q1) / args.steps
    achieved = quant_bytes / (q_avg_ms * 1e-3) / 1e9
    traffic = recorded_traffic()
    roofline = {
        "kernel": "quantize_fused_kernel<rowwise+colwise, RNE> (amax + quantize) on 8192x4096",
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "avg_launch_us": round(q_avg_ms * 1e3, 2),
        "alg_bytes_per_launch": quant_bytes,
    }
    log(f"[bench] step {ms_per_step * 1e3:.1f} us, {value:.0f} GB/s; quantize {q_avg_ms * 1e3:.1f} us "
        f"= {achieved:.0f} GB/s")

    # ------------------------------------------------------ secondary rows
    rows = {}
    gemm_tflops = None
    if not args.no_rows:
        flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)

        def timed(name, fn, iters=2 * args.row_iters, copies=1, graph=True):
            """Average time of one call of fn(k) over `iters` back-to-back
            calls (k = 0, 1, ...: the call rotates over `copies` inputs whose
            total exceeds the 256 MB Infinity Cache, so each call reads its
            input from HBM), between two events on the launch stream. With
            `graph` the calls are captured once in a HIP graph and the timed
            region is one replay of it, so the host's call overhead does not
            starve short kernels; the gaps between kernels stay in. The timed
            calls run inside a ROCTx range named after the row, which
            `--summarize-trace` uses to attribute rocprofv3 kernel durations
            to the row. The cache is flushed (a 512 MiB read, no dirty lines)
            before the timed region."""
            for k in range(min(copies, 3)):
                fn(k)
            torch.cuda.synchronize()
            gr = None
            if graph:
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    for k in range(iters):
                        fn(k)
                gr.replay()
                torch.cuda.synchronize()
            flush.max()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.nvtx.range_push(f"row:{name}")
            e0.record(stream)
            if gr is not None:
                gr.replay()
            else:
                for k in range(iters):
                    fn(k)
            e1.record(stream)
            torch.cuda.synchronize()
            torch.cuda.nvtx.range_pop()
            del gr
            return e0.elapsed_time(e1) * 1e3 / iters

        def row_hbm(name, fn, nbytes, shape, note=None, copies=1, iters=2 * args.row_iters):
            us = timed(name, fn, iters=iters, copies=copies)
            gbs = nbytes / (us * 1e-6) / 1e9
            rows[name] = {"shape": shape, "us": round(us, 2), "calls": iters, "alg_bytes": nbytes,
                          "GB/s": round(gbs, 1), "bound": "hbm", "peak": HBM_PEAK_GBS,
                          "frac": round(gbs / HBM_PEAK_GBS, 4)}
            if note:
                rows[name]["note"] = note
            log(f"[bench] {name}: {us:.1f} us {gbs:.0f} GB/s")

        src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        row_hbm("copy_256MiB_torch", lambda k: dst.copy_(src), 2 * src.numel() * 4, [src.numel()],
                note="device copy: practical streaming ceiling (read + write)")
        row_hbm("fill_256MiB_torch", lambda k: dst.fill_(2.0), src.numel() * 4, [src.numel()],
                note="device fill: practical ceiling for write-only streams")
        del src, dst
        # The step on one input copy, back to back: the 64 MiB tensor stays in
        # the 256 MB Infinity Cache between steps (warm), unlike the headline
        # loop, which rotates copies so every step reads HBM.
        row_hbm("step_warm_one_input_copy",
                lambda k: F.nvfp4_quantize_1d_fused(xs[0], ws, rowwise=True, colwise=True, out=outs[0]),
                step_bytes, [R, C], iters=50,
                note="the headline step on one input copy, 50 back-to-back launches: the input is "
                     "served from the Infinity Cache, so this is not an HBM figure")
        x = xs[0]
        n_x = R * C
        nc = len(xs)  # 5 activation copies: 320 MiB rotate past the Infinity Cache
        o = outs[0]
        row_hbm("amax_activation", lambda k: F.nvfp4_amax(xs[k % nc], out=amax), 2 * n_x, [R, C], copies=nc,
                note="two launches per call (a one-thread reset, then the reduction)")
        row_hbm("amax_then_quantize_row_and_col_two_calls",
                lambda k: (F.nvfp4_amax(xs[k % nc], out=amax),
                           F.nvfp4_quantize_1d(xs[k % nc], amax, rowwise=True, colwise=True, out=o)),
                n_x * 3.125, [R, C], copies=nc, note="nvfp4_amax + nvfp4_quantize_1d (the tensor is read twice)")
        F.nvfp4_amax(x, out=amax)
        row_hbm("quantize_1d_rowwise_rne_activation",
                lambda k: F.nvfp4_quantize_1d(xs[k % nc], amax, rowwise=True, colwise=False, out=o),
                n_x * 2.5625, [R, C], copies=nc)
        row_hbm("quantize_1d_colwise_rne_activation",
                lambda k: F.nvfp4_quantize_1d(xs[k % nc], amax, rowwise=False, colwise=True, out=o),
                n_x * 2.5625, [R, C], copies=nc)
        row_hbm("quantize_1d_row_and_col_rne_activation",
                lambda k: F.nvfp4_quantize_1d(xs[k % nc], amax, rowwise=True, colwise=True, out=o),
                n_x * 3.125, [R, C], copies=nc)
        mask = W.rht_sign_mask()
        a_rht = torch.empty(1, dtype=torch.float32, device=dev)
        row_hbm("amax_rht_activation", lambda k: F.nvfp4_amax(xs[k % nc], rht=True, rht_mask=mask, out=a_rht),
                2 * n_x, [R, C], copies=nc, note="two launches per call (a one-thread reset, then the reduction)")
        F.nvfp4_amax(x, rht=True, rht_mask=mask, out=a_rht)
        row_hbm("quantize_colwise_rht_sr_activation",
                lambda k: F.nvfp4_quantize_1d(xs[k % nc], a_rht, rowwise=False, colwise=True, sr=True, rht=True,
                                              rht_mask=mask, seed=W.SR_SEED, out=o),
                n_x * 2.5625, [R, C], copies=nc, note=ALU_NOTE)
        deq = torch.empty((R, C), dtype=torch.float32, device=dev)
        qo = [F.nvfp4_quantize_1d(xi, amax, rowwise=True, colwise=False) for xi in xs]
        row_hbm("dequantize_1d_fp32_activation",
                lambda k: F.nvfp4_dequantize(qo[k % nc]["codes_row"], qo[k % nc]["scales_row"], 1,
                                             qo[k % nc]["global_scale"], R, C, out=deq), n_x * 4.5625, [R, C],
                copies=nc, note="reads 18 MiB per call from 5 rotating copies (90 MiB, which the Infinity "
                                "Cache can hold); 88% of the row's bytes are the writes")
        deq16 = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
        row_hbm("dequantize_1d_bf16_activation",
                lambda k: F.nvfp4_dequantize(qo[k % nc]["codes_row"], qo[k % nc]["scales_row"], 1,
                                             qo[k % nc]["global_scale"], R, C, out_dtype=torch.bfloat16,
                                             out=deq16), n_x * 2.5625, [R, C], copies=nc)
        del xs[1:], outs[1:], deq, deq16, qo

        log("[bench] generating the 8192x14336 gradient")
        g_host = W.gradient()
        gs = [to_dev(g_host), to_dev(g_host)]  # 448 MiB rotate past the Infinity Cache
        g = gs[0]
        del g_host
        GR, GC = g.shape
        n_g = GR * GC
        row_hbm("amax_rht_gradient", lambda k: F.nvfp4_amax(gs[k % 2], rht=True, rht_mask=mask, out=a_rht),
                2 * n_g, [GR, GC], copies=2, note="two launches per call (a one-thread reset, then the reduction)")
        F.nvfp4_amax(g, rht=True, rht_mask=mask, out=a_rht)
        og = F.nvfp4_quantize_1d(g, a_rht, rowwise=False, colwise=True, sr=True, rht=True, rht_mask=mask,
                                 seed=W.SR_SEED)
        row_hbm("quantize_colwise_rht_sr_gradient",
                lambda k: F.nvfp4_quantize_1d(gs[k % 2], a_rht, rowwise=False, colwise=True, sr=True, rht=True,
                                              rht_mask=mask, seed=W.SR_SEED, out=og),
                n_g * 2.5625, [GR, GC], copies=2, note=ALU_NOTE)
        y = torch.empty((GR, GC), dtype=torch.float32, device=dev)
        row_hbm("rht16_axis0_gradient", lambda k: F.nvfp4_rht16(gs[k % 2], axis=0, rht_mask=mask, out=y),
                n_g * 6, [GR, GC], copies=2)
        del y
        # What the fused transform costs: the same calls without it, and both
        # amaxes of the gradient (plain for dgrad, transformed for wgrad)
        # from one read.
        a_g = torch.empty(1, dtype=torch.float32, device=dev)
        a_both = torch.empty(2, dtype=torch.float32, device=dev)
        row_hbm("amax_gradient", lambda k: F.nvfp4_amax(gs[k % 2], out=a_g), 2 * n_g, [GR, GC], copies=2,
                note="two launches per call (a one-thread reset, then the reduction)")
        row_hbm("amax_plain_and_rht_gradient_one_read",
                lambda k: F.nvfp4_amax(gs[k % 2], rht=True, rht_mask=mask, both=True, out=a_both), 2 * n_g,
                [GR, GC], copies=2,
                note="nvfp4_amax(NVFP4_RHT | NVFP4_AMAX_BOTH): replaces amax_gradient + amax_rht_gradient")
        F.nvfp4_amax(g, out=a_g)
        row_hbm("quantize_colwise_sr_gradient_no_rht",
                lambda k: F.nvfp4_quantize_1d(gs[k % 2], a_g, rowwise=False, colwise=True, sr=True,
                                              seed=W.SR_SEED, out=og),
                n_g * 2.5625, [GR, GC], copies=2, note="the RHT row's call without the transform")
        del og, gs[1:]

        log("[bench] generating the 14336x4096 weight")
        w_host = W.weight()
        wts = [to_dev(w_host) for _ in range(3)]  # 336 MiB rotate past the Infinity Cache
        w = wts[0]
        del w_host
        WR, WC = w.shape
        n_w = WR * WC
        a_w = F.nvfp4_amax(w)
        ow = F.nvfp4_quantize_2d(w, a_w)
        row_hbm("amax_weight", lambda k: F.nvfp4_amax(wts[k % 3], out=a_w), 2 * n_w, [WR, WC], copies=3,
                note="two launches per call (a one-thread reset, then the reduction)")
        F.nvfp4_amax(w, out=a_w)
        row_hbm("quantize_2d_weight", lambda k: F.nvfp4_quantize_2d(wts[k % 3], a_w, out=ow),
                n_w * (2 + 2 * 0.5 + 1 / 256), [WR, WC], copies=3)
        del wts[1:]

        log("[bench] GEMM 8192x14336x4096")
        a_host, b_host = W.gemm_operands()
        A = to_dev(a_host)
        Bm = to_dev(b_host)
        del a_host, b_host
        qa = F.nvfp4_quantize_1d(A, F.nvfp4_amax(A))
        qb = F.nvfp4_quantize_2d(Bm, F.nvfp4_amax(Bm), colwise=False)
        M, N, K = 8192, 14336, 4096
        c32 = torch.empty((M, N), dtype=torch.float32, device=dev)
        c16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        flop = 2.0 * M * N * K
        # sustained matrix work raises the clock over the first tens of ms:
        # time only after ~50 ms of it
        for _ in range(50):
            F.nvfp4_gemm(qa["codes_row"], qa["scales_row"], 1, qa["global_scale"], qb["codes_row"],
                         qb["scales"], 2, qb["global_scale"], M, N, K, out=c32)
        torch.cuda.synchronize()
        for name, cc, dt in (("gemm_fp32_out", c32, torch.float32), ("gemm_bf16_out", c16, torch.bfloat16)):
            us = timed(name, lambda k: F.nvfp4_gemm(qa["codes_row"], qa["scales_row"], 1, qa["global_scale"],
                                                    qb["codes_row"], qb["scales"], 2, qb["global_scale"], M, N, K,
                                                    out_dtype=dt, out=cc), iters=max(5, args.row_iters), graph=False)
            tf = flop / (us * 1e-6) / 1e12
            rows[name] = {"shape": [M, N, K], "us": round(us, 1), "calls": max(5, args.row_iters), "flop": flop,
                          "TFLOP/s": round(tf, 1), "bound": "mfma", "peak": F16_MFMA_PEAK_TFLOPS,
                          "frac": round(tf / F16_MFMA_PEAK_TFLOPS, 4)}
            log(f"[bench] {name}: {us:.0f} us {tf:.1f} TFLOP/s")
        gemm_tflops = rows["gemm_fp32_out"]["TFLOP/s"]
        # Reference only (not a path of this library): the vendor fp16 GEMM
        # (hipBLASLt through torch.matmul) on the same operand values, decoded
        # exactly to fp16 by nvfp4_dequantize with unit global scales.
        one = torch.ones(1, dtype=torch.float32, device=dev)
        da = F.nvfp4_dequantize(qa["codes_row"], qa["scales_row"], 1, one, M, K, out_dtype=torch.float32).half()
        db = F.nvfp4_dequantize(qb["codes_row"], qb["scales"], 2, one, N, K, out_dtype=torch.float32).half()
        ch = torch.empty((M, N), dtype=torch.float16, device=dev)
        dbt = db.t()
        for _ in range(50):
            torch.matmul(da, dbt, out=ch)
        torch.cuda.synchronize()
        us = timed("reference_hipblaslt_fp16_gemm_same_values", lambda k: torch.matmul(da, dbt, out=ch),
                   iters=max(5, args.row_iters), graph=False)
        tf = flop / (us * 1e-6) / 1e12
        rows["reference_hipblaslt_fp16_gemm_same_values"] = {
            "shape": [M, N, K], "us": round(us, 1), "calls": max(5, args.row_iters), "flop": flop,
            "TFLOP/s": round(tf, 1),
            "note": "vendor fp16 GEMM on the decoded operand values (reads 4x the operand bytes, no "
                    "decode); context for gemm_fp32_out, not part of this library"}
        log(f"[bench] reference hipBLASLt fp16 GEMM on the same values: {us:.0f} us {tf:.1f} TFLOP/s")
        del da, db, dbt, ch

        # A linear layer's three GEMMs with their quantizations, composed
        # from the library (fp4_block_scaled_amax_amd.linear): the activation
        # (8192 tokens x 4096), the weight (14336 x 4096), the gradient
        # (8192 x 14336).
        from fp4_block_scaled_amax_amd import linear as L
        log("[bench] NVFP4 linear layer 8192 tokens, 4096 -> 14336: fprop, dgrad, wgrad")
        ws_l = F.nvfp4_workspace(dev)
        wq = L.quantize_weight(w)
        lin_flop = 3 * 2.0 * R * C * WR
        parts = (("linear_weight_quantize_2d", lambda: L.quantize_weight(w), None),
                 ("linear_fprop", lambda: L.fprop(x, wq, ws=ws_l), 2.0 * R * C * WR),
                 ("linear_dgrad", lambda: L.dgrad(g, wq, W.SR_SEED, ws=ws_l), 2.0 * R * C * WR),
                 ("linear_wgrad", lambda: L.wgrad(g, x, mask, W.SR_SEED), 2.0 * R * C * WR),
                 ("linear_layer_step", lambda: L.training_step(x, w, g, mask, W.SR_SEED), lin_flop))
        def unfused_forward():
            yy = L.fprop(x, wq, ws=ws_l, out_dtype=torch.bfloat16)
            return F.nvfp4_quantize_1d(yy, F.nvfp4_amax(yy), rowwise=True, colwise=True)

        # the epilogue-quantized forward takes the amax of a previous
        # product of the same layer (here: the same inputs' own max |Y|)
        y0, _ = L.forward_quantized(x, wq, ws=ws_l)
        y_amax0 = F.nvfp4_amax(y0)
        del y0
        next_amax = torch.empty(1, dtype=torch.float32, device=dev)
        parts = parts + (
            ("linear_forward_quantized_output_fused", lambda: L.forward_quantized(x, wq, ws=ws_l),
             2.0 * R * C * WR),
            ("linear_forward_quantized_output_unfused", unfused_forward, 2.0 * R * C * WR),
            ("linear_forward_quantized_output_epilogue",
             lambda: L.forward_quantized_delayed(x, wq, y_amax0, ws=ws_l, out_amax=next_amax),
             2.0 * R * C * WR))
        for name, fn, fl in parts:
            us = timed(name, lambda k: fn(), iters=5, graph=False)
            rows[name] = {"shape": {"tokens": R, "in": C, "out": WR}, "us": round(us, 1), "calls": 5}
            if fl is not None:
                rows[name].update({"flop": fl, "TFLOP/s": round(fl / (us * 1e-6) / 1e12, 1),
                                   "note": "GEMM flop only; the time includes the operands' quantization"})
            log(f"[bench] {name}: {us:.0f} us" + (f" {fl / (us * 1e-6) / 1e12:.1f} TFLOP/s" if fl else ""))
        del wq

        # MXFP4, the comparator format (E8M0 scale per 32 elements, no tensor
        # scale): its quantizer on the same tensors, its GEMM on the gfx950
        # block-scaled matrix cores with operands from the same values, and
        # the representation error of both formats.
        log("[bench] MXFP4 comparator")
        # Like the NVFP4 rows, each call reads the next of the rotating input
        # copies (more than the Infinity Cache holds) and writes that copy's
        # own outputs.
        xm = [x] + [to_dev(x_host) for _ in range(nc - 1)]
        mos = [F.mxfp4_quantize(xm[k], rowwise=True, colwise=True) for k in range(nc)]
        row_hbm("mx_quantize_rowwise_activation", lambda k: F.mxfp4_quantize(xm[k % nc], out=mos[k % nc]),
                n_x * (2 + 0.5 + 1 / 32), [R, C], copies=nc)
        row_hbm("mx_quantize_row_and_col_activation",
                lambda k: F.mxfp4_quantize(xm[k % nc], rowwise=True, colwise=True, out=mos[k % nc]),
                n_x * (2 + 2 * (0.5 + 1 / 32)), [R, C], copies=nc)
        del xm[1:]
        gm = [g, g.clone()]  # 448 MiB rotate past the Infinity Cache
        mgs = [F.mxfp4_quantize(gm[k], rowwise=False, colwise=True, rht=True, rht_mask=mask) for k in range(2)]
        row_hbm("mx_quantize_colwise_rht_gradient",
                lambda k: F.mxfp4_quantize(gm[k % 2], rowwise=False, colwise=True, rht=True, rht_mask=mask,
                                           out=mgs[k % 2]),
                n_g * (2 + 0.5 + 1 / 32), [GR, GC], copies=2)
        del mgs, gm
        mdq = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
        row_hbm("mx_dequantize_bf16_activation",
                lambda k: F.mxfp4_dequantize(mos[k % nc]["codes_row"], mos[k % nc]["scales_row"], R, C,
                                             out_dtype=torch.bfloat16, out=mdq), n_x * (0.5 + 1 / 32 + 2), [R, C],
                copies=nc)
        del mdq
        ma = F.mxfp4_quantize(A)
        mb = F.mxfp4_quantize(Bm)
        for _ in range(50):
            F.mxfp4_gemm(ma["codes_row"], ma["scales_row"], mb["codes_row"], mb["scales_row"], M, N, K, out=c32)
        torch.cuda.synchronize()
        for name, cc, dt in (("mx_gemm_fp32_out", c32, torch.float32), ("mx_gemm_bf16_out", c16, torch.bfloat16)):
            us = timed(name, lambda k: F.mxfp4_gemm(ma["codes_row"], ma["scales_row"], mb["codes_row"],
                                                    mb["scales_row"], M, N, K, out_dtype=dt, out=cc),
                       iters=max(5, args.row_iters), graph=False)
            tf = flop / (us * 1e-6) / 1e12
            rows[name] = {"shape": [M, N, K], "us": round(us, 1), "calls": max(5, args.row_iters), "flop": flop,
                          "TFLOP/s": round(tf, 1), "bound": "mfma", "peak": FP4_MFMA_PEAK_TFLOPS,
                          "frac": round(tf / FP4_MFMA_PEAK_TFLOPS, 4)}
            log(f"[bench] {name}: {us:.0f} us {tf:.1f} TFLOP/s")
        del ma, mb, mos
        rows["error_study"] = error_study(F, {"activation": x, "weight": w, "gradient": g}, mask, dev)
        del g
        del flush

    # -------------------------------------------------- CPU oracle baseline
    cpu = cpu_all = cpu_gemm = None
    if not args.no_cpu:
        import oracle

        sample = np.ascontiguousarray(x_host[: args.cpu_rows])
        log(f"[bench] CPU oracle on the first {args.cpu_rows} rows, {args.cpu_passes} passes")
        # Whole passes over the sample until about 10 s of CPU work; the
        # median pass is the figure.
        passes = []
        for _ in range(max(1, args.cpu_passes)):
            t0 = time.perf_counter()
            ref = oracle.quantize_1d(sample, rowwise=True, colwise=True)
            passes.append(time.perf_counter() - t0)
        t_cpu = float(np.median(passes))
        ns = sample.size
        # the step's algorithmic bytes, as for the GPU value: the input once and both outputs
        cpu = {"value": round(ns * 3.125 / t_cpu / 1e9, 4), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"first {args.cpu_rows} rows of the activation ({args.cpu_rows}x{C}), amax + rowwise "
                         f"+ columnwise 1D RNE quantize as one tensor, {len(passes)} passes "
                         f"({sum(passes):.1f} s single-threaded); the median pass {t_cpu:.2f} s",
               "seconds": round(t_cpu, 2), "passes": len(passes)}
        cpu_all = cpu_all_cores(oracle, sample, ref, args)
        cpu_gemm = None if args.no_cpu_gemm else cpu_gemm_reference(oracle, W)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "activation 8192x4096 bf16, N(0,1) with 8 outlier columns x100 (seed 1): amax + "
                        "rowwise and columnwise 1D NVFP4 quantize, round-to-nearest-even",
            "rows": R, "cols": C, "block": 16, "layouts": ["rowwise", "colwise"],
            "input_copies": args.copies,
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "gemm_tflops": gemm_tflops,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "cpu_gemm_reference": cpu_gemm,
        "rows": rows,
        # The pages' own figures, with their hardware: context only, not
        # targets, and not comparable to any row above (they measure NVFP4
        # GEMM peak rates and end-to-end training on other parts).
        "pages_context": {
            "nvfp4_gemm_peak_vs_fp8": {"value": "2-3x", "hardware": "GB200, GB300",
                                       "source": "page 'Melatih model dalam 4 bit', section 'Presisi sebagai "
                                                 "tombol throughput'"},
            "training_tflops_per_gpu_nvfp4_vs_fp8": {
                "llama3_8b": {"GB200": "2017 vs 1497 (1.35x)", "GB300": "2301 vs 1759 (1.31x)"},
                "llama3.1_405b": {"GB200": "2241 vs 1557 (1.44x)", "GB300": "3633 vs 2103 (1.73x)"},
                "setup": "vendor JAX/MaxText measurement",
                "source": "page 'Melatih model dalam 4 bit', section 'Angka yang dilaporkan'"},
        },
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
