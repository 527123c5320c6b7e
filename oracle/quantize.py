"""Plain CPU oracle for per-token block quantisation of bf16 rows into FP8 e4m3
(1x128 blocks) or FP4 e2m1 (1x32 blocks) with UE8M0 power-of-two scales.

TEST INFRASTRUCTURE ONLY (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

The pages state that low-precision operands travel with UE8M0 scale factors and
that the scale helper emits them packed in pairs along K as int16, MN-major
("DeepGEMM-Ascend cobre quantas operacoes no Ascend 950?", section "Fatores de
escala FP8 e o formato UE8M0 no Ascend"); they do not say how a producer picks
the scale or rounds an element.  The readings taken here:

  * scale rule "ceil": the scale of a block is 2^e with e the smallest integer
    such that the block's largest magnitude fits the format's largest finite
    value (448 for e4m3, 6 for e2m1), so no element is clipped;
  * scale rule "ocp_mx": e = floor(log2(amax)) - emax, emax the exponent of the
    format's largest binade (8 for e4m3, 2 for e2m1), the OCP Microscaling rule;
    magnitudes beyond the largest finite value then saturate;
  * the UE8M0 byte is e + 127 clamped to [0, 254]; an all-zero block takes the
    lower clamp, byte 0;
  * each element x becomes the code nearest to x / 2^e on the format's finite
    grid, ties to the even code, saturating at the largest finite value; the
    code's sign bit is x's sign bit (so -0 and negative values that round to
    zero give the negative-zero code).

Every step below is done in fp64, where all of them are exact (bf16 values,
powers of two and their products are dyadic rationals well inside fp64's range)
except the rounding decision itself, which compares exact distances.

SwiGLU (for the MoE FFN core): y = silu(gate) * up with silu(g) = g / (1 + e^-g),
evaluated in fp64, then quantised as above.  The pages list SwiGLU between the two
grouped GEMMs of the fused MoE benchmark ("DeepGEMM-Ascend cobre quantas
operacoes no Ascend 950?" third page, "Kernels de computacao: DeepGEMM-Ascend
versus DeepGEMM", section "Execucao de MoE: MegaMoE e distribuicao de
especialistas") without defining it; the textbook SwiGLU, with the gate in the
first half of the up-projection's columns, is the reading taken here.

Parity status: pinned (tests/test_quantize_pins.py: hand-worked fixtures,
exhaustive-search brute force in exact rationals, torch's own e4m3 cast for
in-range values, exact reconstruction of representable blocks, scale shift
invariance; SwiGLU against torch's silu in fp64, the identity
silu(g) - silu(-g) = g, and its reduction to the quantiser where sigmoid is 1).
"""
from __future__ import annotations

import numpy as np

from . import e2m1_table, e4m3_table, pack_scales

FORMATS = {
    # name: (elements per block along K, largest finite magnitude, its binade's exponent)
    "e4m3": (128, 448.0, 8),
    "e2m1": (32, 6.0, 2),
}
RULES = ("ceil", "ocp_mx")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32; widen, then convert (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _positive_grid(fmt: str) -> np.ndarray:
    """Finite non-negative values of the format, indexed by code (they increase
    with the code for both formats)."""
    if fmt == "e4m3":
        g = e4m3_table()[:0x7F]          # 0x7F is NaN
    else:
        g = e2m1_table()[:8]
    assert np.all(np.diff(g) > 0)
    return g


def block_exponent(amax: np.ndarray, fmt: str, rule: str) -> np.ndarray:
    """Unclamped scale exponent e per block (float array; -inf for amax == 0)."""
    _, qmax, emax = FORMATS[fmt]
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    safe = np.where(pos, amax, 1.0)
    if rule == "ceil":
        # smallest integer e with amax <= qmax * 2^e: estimate, then correct with
        # exact comparisons (qmax * 2^e is exact in fp64)
        e = np.ceil(np.log2(safe / qmax))
        for _ in range(2):
            e = np.where(safe > np.ldexp(qmax, e.astype(np.int64)), e + 1, e)
            e = np.where(safe <= np.ldexp(qmax, (e - 1).astype(np.int64)), e - 1, e)
    elif rule == "ocp_mx":
        # p = floor(log2(amax)), i.e. 2^p <= amax < 2^(p+1), then e = p - emax
        p = np.floor(np.log2(safe))
        for _ in range(2):
            p = np.where(np.ldexp(1.0, p.astype(np.int64)) > safe, p - 1, p)
            p = np.where(np.ldexp(1.0, (p + 1).astype(np.int64)) <= safe, p + 1, p)
        e = p - emax
    else:
        raise ValueError(f"unknown scale rule {rule!r}")
    return np.where(pos, e, -np.inf)


def scale_bytes(amax: np.ndarray, fmt: str, rule: str) -> np.ndarray:
    e = block_exponent(amax, fmt, rule)
    return np.clip(e + 127, 0, 254).astype(np.uint8)


def round_to_grid(v: np.ndarray, fmt: str) -> np.ndarray:
    """Magnitude code of |v| on the format's finite grid: nearest value, ties to
    the even code, saturating at the largest finite value."""
    g = _positive_grid(fmt)
    a = np.abs(np.asarray(v, dtype=np.float64))
    top = len(g) - 1
    hi = np.clip(np.searchsorted(g, a, side="left"), 1, top)   # g[hi-1] < a <= g[hi] inside the grid
    lo = hi - 1
    d_lo = a - g[lo]
    d_hi = g[hi] - a
    code = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(a >= g[top], top, code)        # saturate
    code = np.where(a == 0, 0, code)
    return code.astype(np.uint8)


def quantize_values(x: np.ndarray, fmt: str, rule: str = "ceil"):
    """fp64 values [M][K] -> (codes, sf) with
         e4m3: codes uint8 [M][K];
         e2m1: codes uint8 [M][K/2], even k in the low nibble;
       sf: UE8M0 bytes uint8 [M][K / block], one per block of the row.
    A code's sign bit is the value's sign bit (np.signbit: -0.0 counts)."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    if rule not in RULES:
        raise ValueError(f"unknown scale rule {rule!r}")
    gk, _, _ = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    if K % gk:
        raise ValueError(f"K={K} is not a multiple of the block size {gk}")
    kb = K // gk
    amax = np.abs(x).reshape(M, kb, gk).max(axis=2) if K else np.zeros((M, 0))
    sf = scale_bytes(amax, fmt, rule)
    e = sf.astype(np.int64) - 127
    v = np.ldexp(x, -np.repeat(e, gk, axis=1))                # exact
    mag = round_to_grid(v, fmt)
    sign = np.signbit(x).astype(np.uint8)
    if fmt == "e4m3":
        codes = mag | (sign << 7)
    else:
        nib = mag | (sign << 3)
        codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return codes.astype(np.uint8), sf


def quantize_rows(x_bits: np.ndarray, fmt: str, rule: str = "ceil"):
    """bf16 bits uint16 [M][K] -> (codes, sf), as quantize_values on the decoded
    rows (bf16 -> fp64 is exact and keeps the sign of zero)."""
    return quantize_values(bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)), fmt, rule)


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU (swish) g * sigmoid(g) = g / (1 + e^-g), fp64.  For g below about -709
    e^-g overflows to inf and the quotient is a signed zero, the limit."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(h_bits: np.ndarray, inter: int) -> np.ndarray:
    """SwiGLU of an up-projection output: bf16 bits [M][2*inter] holding the gate
    in columns [0, inter) and the up projection in [inter, 2*inter); returns
    y = silu(gate) * up in fp64 [M][inter]."""
    h = bf16_bits_to_f64(np.asarray(h_bits, dtype=np.uint16))
    if h.shape[1] < 2 * inter:
        raise ValueError("h has fewer than 2*inter columns")
    return silu(h[:, :inter]) * h[:, inter:2 * inter]


def swiglu_quantize(h_bits: np.ndarray, inter: int, fmt: str = "e4m3", rule: str = "ceil"):
    """(codes, sf, y): the per-token quantisation of swiglu(h_bits, inter), and y."""
    y = swiglu(h_bits, inter)
    codes, sf = quantize_values(y, fmt, rule)
    return codes, sf, y


def quantize_rows_packed(x_bits: np.ndarray, fmt: str, rule: str = "ceil",
                         ld_packed: int | None = None):
    """As quantize_rows, with the scales packed two per int16 along K, MN-major:
    int16 [ceil(Kb/2)][ld_packed >= M]."""
    codes, sf = quantize_rows(x_bits, fmt, rule)
    return codes, pack_scales(sf, ld_packed)
