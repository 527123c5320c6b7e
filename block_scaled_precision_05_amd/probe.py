"""ctypes binding of libbsg_probe.so (include/bsg_probe.h): the rate the matrix cores
sustain on MFMAs alone, a measurement aid beside the GEMM library."""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "libbsg_probe.so")
KINDS = {"bf16": 0, "fp8": 1, "fp4": 2}
# K of one MFMA and its flops (32 x 32 outputs, two per multiply-add)
MMA_K = {"bf16": 16, "fp8": 64, "fp4": 64}
MFMAS_PER_ROUND = 16   # per wave: two k-steps of 4 x 2 fragments
THREADS = 512

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded libbsg_probe.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(PROBE_LIB_PATH):
                raise RuntimeError(f"{PROBE_LIB_PATH} is missing: build it with "
                                   "`python -m block_scaled_precision_05_amd.build` (hipcc, gfx950)")
            l = ctypes.CDLL(PROBE_LIB_PATH)
            l.bsg_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
            l.bsg_probe_mfma.restype = ctypes.c_int
            _lib = l
        return _lib


def flops_per_call(kind: str, workgroups: int, iters: int) -> float:
    """Flops one call performs: 8 waves a workgroup, 16 MFMAs a round."""
    return float(workgroups) * 8 * MFMAS_PER_ROUND * iters * 2 * 32 * 32 * MMA_K[kind]


def mfma(kind: str, seed: int, workgroups: int, iters: int, out, stream=None) -> None:
    """Enqueues one probe call; `out` is a float32 device tensor of workgroups * 512
    elements (each thread's accumulator sum)."""
    import torch
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < workgroups * THREADS:
        raise ValueError("out must be a float32 device tensor of workgroups * 512 elements")
    if stream is None:
        stream = torch.cuda.current_stream(out.device)
    st = lib().bsg_probe_mfma(KINDS[kind], seed, workgroups, iters, out.data_ptr(),
                              ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise RuntimeError(f"bsg_probe_mfma({kind}) returned status {st}")
