"""Comparison of GPU outputs with the oracle, to the acceptance rule used here:

  err[i][j] = |D_gpu[i][j] - bf16(D_oracle[i][j])| / (||a_i|| * ||b_j||) <= 1e-3

with the norms taken over dequantised rows.  An element whose normalised error is
above the bound still passes when D_gpu is one of the two bf16 values that
bracket the exact fp64 result (a rounding-boundary flip caused by the fp32
accumulator); such elements are counted separately.  Rows whose norm is zero
must match exactly.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle

TOL = 1e-3


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits.astype(np.uint16)).view(np.int16)
    return torch.from_numpy(b).view(torch.bfloat16).to(torch.float64).numpy()


def gpu_bits(D: torch.Tensor) -> np.ndarray:
    return D.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class Report:
    max_err: float
    n: int
    n_bracket_only: int
    n_fail: int

    def __str__(self):
        return (f"max normalised error {self.max_err:.3e} over {self.n} outputs, "
                f"{self.n_bracket_only} pass only as bracketing bf16 neighbours, "
                f"{self.n_fail} fail")


def _neighbour(ref_bits: np.ndarray, ref_val: np.ndarray, exact: np.ndarray) -> np.ndarray:
    """The other bf16 value bracketing `exact` (ref_bits is its nearest)."""
    mag = ref_bits & 0x7FFF
    sign = ref_bits & 0x8000
    up = np.abs(ref_val) < np.abs(exact)        # exact lies further from zero
    other = np.where(up, mag + 1, np.maximum(mag, 1) - 1).astype(np.uint16) | sign
    # rounding to zero: the neighbour is the smallest subnormal with exact's sign
    zero = mag == 0
    other = np.where(zero, np.where(exact < 0, 0x8001, 0x0001), other).astype(np.uint16)
    return other


def compare(got_bits: np.ndarray, ref: np.ndarray, na: np.ndarray, nb: np.ndarray,
            tol: float = TOL) -> Report:
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    ref = np.asarray(ref, dtype=np.float64)
    assert got_bits.shape == ref.shape, (got_bits.shape, ref.shape)
    ref_bits = oracle.bf16_rne(ref)
    ref_val = bf16_bits_to_f64(ref_bits)
    got = bf16_bits_to_f64(got_bits)
    denom = na[:, None] * nb[None, :]
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.abs(got - ref_val) / denom
    zero_norm = denom == 0
    err = np.where(zero_norm, np.where(got == ref_val, 0.0, np.inf), err)
    err = np.where(np.isnan(got) & ~np.isnan(ref_val), np.inf, err)
    within = err <= tol
    other = _neighbour(ref_bits, ref_val, ref)
    bracket = ((got_bits == ref_bits) | (got_bits == other) |
               ((got_bits & 0x7FFF) == 0) & ((ref_bits & 0x7FFF) == 0))
    ok = within | (bracket & ~zero_norm)
    return Report(float(np.max(err)) if err.size else 0.0, int(err.size),
                  int(np.sum(~within & bracket & ~zero_norm)), int(np.sum(~ok)))


def assert_parity(got_bits, ref, na, nb, tol: float = TOL, what: str = ""):
    r = compare(got_bits, ref, na, nb, tol)
    print(f"[parity] {what}: {r}", flush=True)
    assert r.n_fail == 0, f"{what}: {r}"
    return r
