"""Builds libbsg.so (the C-ABI GEMM and quantisation library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbsg.so")
SOURCES = [os.path.join(HERE, "csrc", "api.hip"), os.path.join(HERE, "csrc", "quant.hip"),
           os.path.join(HERE, "csrc", "mqa.hip")]
HEADERS = [os.path.join(HERE, "csrc", h) for h in ("gemm_kernel.h", "configs.h", "internal.h",
                                                       "quant_math.h")] + \
    [os.path.join(ROOT, "include", "bsg.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops keeps the compiler from emitting v_pk_{add,mul,fma}_f32.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every HIP source into libbsg.so next to this file."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libbsg.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
