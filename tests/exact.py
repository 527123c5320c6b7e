"""Exact-rational brute force for tiny GEMMs, independent of the C oracle.

Element values come from library conversions (torch's bfloat16, float8_e4m3fn and
float8_e8m0fnu casts to float64, all exact) and, for e2m1, from the printed grid
in ``golden/e2m1_grid.txt``; scale bytes are read from the unpacked uint8 arrays
the test itself drew, never from a packed array.  Sums are exact Fractions and
the final rounding to bf16 is done on the exact value.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))


def e2m1_grid() -> list[float]:
    vals = [None] * 16
    with open(os.path.join(_HERE, "golden", "e2m1_grid.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return vals


def _frac_matrix(vals: np.ndarray) -> list[list[Fraction]]:
    return [[Fraction(float(x)) for x in row] for row in vals]


def dequant_bf16(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits.astype(np.uint16)).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def dequant_e4m3(codes: np.ndarray, sf: np.ndarray, gran_mn: int, gran_k: int) -> np.ndarray:
    v = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.ascontiguousarray(sf)).view(torch.float8_e8m0fnu).to(torch.float64)
    rows, K = codes.shape
    s = s.repeat_interleave(gran_mn, 0)[:rows].repeat_interleave(gran_k, 1)[:, :K]
    return (v * s).numpy()


def dequant_e2m1(packed: np.ndarray, sf: np.ndarray, K: int, gran_k: int = 32) -> np.ndarray:
    grid = np.array(e2m1_grid(), dtype=np.float64)
    lo = packed & 0xF
    hi = packed >> 4
    codes = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    v = grid[codes[:, :K]]
    s = torch.from_numpy(np.ascontiguousarray(sf)).view(torch.float8_e8m0fnu).to(torch.float64)
    s = s.repeat_interleave(gran_k, 1)[:, :K].numpy()
    return v * s


def exact_nt(a: np.ndarray, b: np.ndarray) -> list[list[Fraction]]:
    """Exact D = a @ b.T for float64 matrices holding dyadic values."""
    fa = _frac_matrix(a)
    fb = _frac_matrix(b)
    return [[sum((x * y for x, y in zip(ra, rb)), Fraction(0)) for rb in fb] for ra in fa]


def bf16_round_exact(x: Fraction) -> float:
    """Round an exact rational to bfloat16, nearest with ties to even."""
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    # 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 7, -133)
    r = a / (Fraction(2) ** q)
    n = r.numerator // r.denominator
    rem = r - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = Fraction(n) * Fraction(2) ** q
    if v >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * float(v)


def bf16_bits(x: float) -> int:
    """Bits of a float that is exactly representable in bfloat16."""
    t = torch.tensor([x], dtype=torch.float32).to(torch.bfloat16)
    assert float(t.to(torch.float64)) == x or x != x
    return int(t.view(torch.int16).item()) & 0xFFFF
