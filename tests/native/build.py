"""Build the test probe library tests/native/libconverter_probe.so with
hipcc for gfx950, with the same code-generation flags as the library it
exercises."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "converter_probe.hip")
LIB_PATH = os.path.join(HERE, "libconverter_probe.so")


def build() -> str:
    sys.path.insert(0, ROOT)
    from fp4_block_scaled_amax_amd import build as B

    tmp = LIB_PATH + ".tmp"
    cmd = [B.hipcc(), *B.FLAGS, "-o", tmp, SRC]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + proc.stdout + proc.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def is_stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    deps = [SRC] + [os.path.join(ROOT, "fp4_block_scaled_amax_amd", "csrc", h) for h in ("device.h", "encode.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build())
