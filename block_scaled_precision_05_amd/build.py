"""Builds libbsg.so (the C-ABI GEMM and quantisation library) and libbsg_probe.so (the
sustained matrix-core rate probe, a measurement aid) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbsg.so")
SOURCES = [os.path.join(HERE, "csrc", "api.hip"), os.path.join(HERE, "csrc", "quant.hip"),
           os.path.join(HERE, "csrc", "mqa.hip")]
PROBE_LIB = os.path.join(HERE, "libbsg_probe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "probe.hip")]
HEADERS = [os.path.join(HERE, "csrc", h) for h in ("gemm_kernel.h", "configs.h", "internal.h",
                                                       "quant_math.h")] + \
    [os.path.join(ROOT, "include", "bsg.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops keeps the compiler from emitting v_pk_{add,mul,fma}_f32.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]
# Per-source code generation options.  The MQA logits kernel feeds its MFMA
# accumulators straight to vector arithmetic: kept in VGPRs (the MFMA's VGPR form)
# they need no accumulator-register reads, 32 instructions per key fragment.
SOURCE_FLAGS = {"mqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one object each) and link libbsg.so and
    libbsg_probe.so next to this file.  Returns the path of libbsg.so."""
    if not force and os.path.exists(LIB) and os.path.exists(PROBE_LIB):
        return LIB
    tag = ".tmp%d" % os.getpid()
    targets = [(LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)]
    objs, procs = {}, []
    for lib, sources in targets:
        for src in sources:
            obj = os.path.join(HERE, os.path.basename(src) + tag + ".o")
            cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(os.path.basename(src), []) + \
                ["-c", src, "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                text=True)))
            objs.setdefault(lib, []).append(obj)
    failed = []
    for src, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(out + err)
        elif verbose:
            sys.stderr.write(err)
    try:
        if failed:
            raise RuntimeError("hipcc failed on " + ", ".join(os.path.basename(f) for f in failed))
        for lib, _ in targets:
            tmp = lib + tag
            res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs[lib] +
                                 ["-o", tmp], capture_output=True, text=True)
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError("hipcc failed linking " + os.path.basename(lib))
            os.replace(tmp, lib)
    finally:
        for o in (o for os_ in objs.values() for o in os_):
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(force=True))
