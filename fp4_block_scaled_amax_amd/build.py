"""Compile the gfx950 HIP library (libnvfp4.so) in-tree with hipcc.

Flags: -ffp-contract=off keeps every binary32 multiply and add a separate
IEEE operation (no fused multiply-add), IEEE division and denormals stay at
hipcc's defaults, and the packed-fp32 instructions are disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libnvfp4.so")

SOURCES = ["api.hip", "amax.hip", "quantize.hip", "rht_dequant.hip", "gemm.hip", "mx_quantize.hip",
           "mx_gemm.hip"]
HEADERS = ["device.h", "encode.h", "kernels.h", "quant_item.h"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    f"-I{os.path.join(ROOT, 'include')}",
    "-Wl,-rpath,/opt/rocm/lib",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the NVFP4 HIP library cannot be built")
    return path


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


OBJ_DIR = os.path.join(HERE, "_build")


def _run(cmd, verbose):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + proc.stdout + proc.stderr)
    if verbose:
        print(" ".join(cmd))


def build(verbose: bool = False) -> str:
    """Always recompiles (one hipcc per source, in parallel, then one link);
    writes the library atomically."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(OBJ_DIR, exist_ok=True)
    compile_flags = [f for f in FLAGS if f not in ("-shared",) and not f.startswith("-Wl,")]
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *compile_flags, "-c", "-o", obj, src])
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp,
          *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def is_stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    deps = sources() + [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(ROOT, "include", h) for h in ("nvfp4.h", "mxfp4.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
