"""Pins of the per-token quantisation oracle (``oracle.quantize``) against things
other than itself: hand-worked fixtures, an exhaustive search in exact rationals,
torch's own e4m3 cast, exact reconstruction of representable blocks, and the
shift invariance of the scale."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import exact
import quant_fixture

QMAX = {"e4m3": 448, "e2m1": 6}
EMAX = {"e4m3": 8, "e2m1": 2}
GK = {"e4m3": 128, "e2m1": 32}


@pytest.fixture(scope="module")
def oq(orc):
    from oracle import quantize
    return quantize


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _random_bf16(rng, M, K, lo=-12, hi=12):
    """Finite bf16 values with random signs, mantissas and exponents in [lo, hi],
    a few exact zeros and negative zeros, and one block scaled far down."""
    sign = rng.integers(0, 2, (M, K))
    mant = rng.integers(0, 128, (M, K))
    ex = rng.integers(lo, hi + 1, (M, K))
    x = (-1.0) ** sign * (1 + mant / 128.0) * np.exp2(ex)
    x[rng.random((M, K)) < 0.03] = 0.0
    x[rng.random((M, K)) < 0.02] = -0.0
    bits = _bf16_bits(torch.from_numpy(x).to(torch.float32))
    return bits


def _values_e4m3():
    v = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
    return [Fraction(x) for x in v]


def _values_e2m1():
    return [Fraction(x) for x in exact.e2m1_grid()[:8]]


# ---------------------------------------------------------------------------
# hand-worked cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", quant_fixture.cases(), ids=lambda c: c.name)
def test_worked_examples(oq, orc, case):
    codes, sf = oq.quantize_rows(case.x_bits(), case.fmt, case.rule)
    assert sf[0].tolist() == case.sf
    assert np.array_equal(codes, case.expected_codes())
    if case.packed:
        _, packed = oq.quantize_rows_packed(case.x_bits(), case.fmt, case.rule)
        assert [int(w) & 0xFFFF for w in packed[:, 0]] == case.packed


# ---------------------------------------------------------------------------
# exhaustive search in exact rationals
# ---------------------------------------------------------------------------

def _brute_byte(amax: Fraction, fmt: str, rule: str) -> int:
    if amax == 0:
        return 0
    if rule == "ceil":
        best = None
        for e in range(300, -400, -1):      # smallest e with amax <= qmax * 2^e
            if amax <= QMAX[fmt] * Fraction(2) ** e:
                best = e
            else:
                break
    else:
        best = None
        for p in range(-400, 300):          # largest p with 2^p <= amax
            if Fraction(2) ** p <= amax:
                best = p
            else:
                break
        best -= EMAX[fmt]
    return min(max(best + 127, 0), 254)


def _brute_code(x: Fraction, neg: bool, e: int, grid, sign_bit: int) -> int:
    target = abs(x) / Fraction(2) ** e
    dist = [abs(g - target) for g in grid]
    m = min(dist)
    cands = [c for c, d in enumerate(dist) if d == m]
    code = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    return code | (sign_bit if neg else 0)


@pytest.mark.parametrize("fmt,rule,seed", [("e4m3", "ceil", 0), ("e4m3", "ocp_mx", 1),
                                           ("e2m1", "ceil", 2), ("e2m1", "ocp_mx", 3)])
def test_brute_force_exact(oq, fmt, rule, seed):
    rng = np.random.default_rng(seed)
    M, K = (2, 256) if fmt == "e4m3" else (3, 128)
    bits = _random_bf16(rng, M, K)
    bits[0, :GK[fmt]] = _bf16_bits(torch.tensor(
        np.ldexp(rng.standard_normal(GK[fmt]), -120), dtype=torch.float32))   # tiny block
    bits[1, GK[fmt]:2 * GK[fmt]] = 0                                            # zero block
    codes, sf = oq.quantize_rows(bits, fmt, rule)
    xs = exact.dequant_bf16(bits)
    grid = _values_e4m3() if fmt == "e4m3" else _values_e2m1()
    gk = GK[fmt]
    for i in range(M):
        for b in range(K // gk):
            blk = [Fraction(float(v)) for v in xs[i, b * gk:(b + 1) * gk]]
            byte = _brute_byte(max(abs(v) for v in blk), fmt, rule)
            assert sf[i, b] == byte, (i, b)
            for k in range(gk):
                kk = b * gk + k
                want = _brute_code(blk[k], bool(bits[i, kk] >> 15), byte - 127, grid,
                                   0x80 if fmt == "e4m3" else 0x8)
                if fmt == "e4m3":
                    got = int(codes[i, kk])
                else:
                    got = (int(codes[i, kk // 2]) >> (4 * (kk % 2))) & 0xF
                assert got == want, (i, kk, float(blk[k]), byte)


# ---------------------------------------------------------------------------
# library routine: torch's e4m3 cast of the scaled values
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("rule", ["ceil", "ocp_mx"])
def test_e4m3_codes_match_torch_cast(oq, rule):
    from block_scaled_precision_05_amd import workloads
    x = workloads.activations(64, 1024, seed=5, zero_rows=2)
    bits = _bf16_bits(x)
    codes, sf = oq.quantize_rows(bits, "e4m3", rule)
    e = torch.from_numpy(sf.astype(np.int32) - 127).repeat_interleave(128, dim=1)
    v = torch.ldexp(x.to(torch.float64), -e.to(torch.float64)).to(torch.float32)   # exact
    inrange = v.abs() <= 448
    if rule == "ceil":
        assert bool(inrange.all())
    ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    m = inrange.numpy()
    assert np.array_equal(codes[m], ref[m])
    # beyond 448 (ocp_mx only) the oracle saturates; torch's cast would give NaN
    assert np.all((codes[~m] & 0x7F) == 0x7E)


# ---------------------------------------------------------------------------
# exact reconstruction of representable blocks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("rule", ["ceil", "ocp_mx"])
def test_representable_blocks_come_back_exactly(oq, fmt, rule):
    """Blocks built as code * 2^e, with one element at +-qmax, quantise back to
    the same codes and byte (for both rules the largest magnitude qmax lies in
    [2^emax, 2^(emax+1)), so both pick e)."""
    rng = np.random.default_rng(11)
    M, gk = 6, GK[fmt]
    K = 4 * gk
    top = 0x7E if fmt == "e4m3" else 7
    mag = rng.integers(0, top + 1, (M, K))
    sign = rng.integers(0, 2, (M, K))
    blk_max = rng.integers(0, gk, (M, K // gk))
    for i in range(M):
        for b in range(K // gk):
            mag[i, b * gk + blk_max[i, b]] = top
    byte = rng.integers(100, 150, (M, K // gk))
    if fmt == "e4m3":
        code = (mag | (sign << 7)).astype(np.uint8)
        val = torch.from_numpy(code).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    else:
        code = (mag | (sign << 3)).astype(np.uint8)
        val = np.array(exact.e2m1_grid(), dtype=np.float64)[code]
    x = np.ldexp(val, np.repeat(byte - 127, gk, axis=1))
    bits = _bf16_bits(torch.from_numpy(x).to(torch.float32))
    assert np.array_equal(exact.dequant_bf16(bits), x)                # bf16-exact inputs
    codes, sf = oq.quantize_rows(bits, fmt, rule)
    assert np.array_equal(sf, byte.astype(np.uint8))
    if fmt == "e4m3":
        assert np.array_equal(codes, code)
    else:
        assert np.array_equal(codes, (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("rule", ["ceil", "ocp_mx"])
@pytest.mark.parametrize("s", [-5, 3])
def test_power_of_two_shift_moves_only_the_byte(oq, fmt, rule, s):
    from block_scaled_precision_05_amd import workloads
    x = workloads.activations(16, 512, seed=6)
    b0 = _bf16_bits(x)
    b1 = _bf16_bits(torch.ldexp(x.to(torch.float32), torch.tensor(float(s))))
    c0, s0 = oq.quantize_rows(b0, fmt, rule)
    c1, s1 = oq.quantize_rows(b1, fmt, rule)
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1.astype(np.int32), s0.astype(np.int32) + s)


def test_rounding_error_bound_ceil(oq):
    """With the ceil rule nothing saturates, so every element is within half a
    grid step: relative 2^-4 for normal e4m3 values, absolute 2^-10 * 2^e below."""
    from block_scaled_precision_05_amd import workloads
    x = workloads.activations(32, 1024, seed=7)
    bits = _bf16_bits(x)
    codes, sf = oq.quantize_rows(bits, "e4m3", "ceil")
    deq = exact.dequant_e4m3(codes, sf, 1, 128)
    xs = exact.dequant_bf16(bits)
    scale = np.repeat(np.exp2(sf.astype(np.float64) - 127), 128, axis=1)
    bound = np.maximum(np.abs(xs) * 2.0 ** -4, scale * 2.0 ** -10)
    assert np.all(np.abs(deq - xs) <= bound)


def test_rejects_ragged_k(oq):
    with pytest.raises(ValueError):
        oq.quantize_rows(np.zeros((2, 100), np.uint16), "e4m3", "ceil")
    with pytest.raises(ValueError):
        oq.quantize_rows(np.zeros((2, 48), np.uint16), "e2m1", "ceil")


# ---------------------------------------------------------------------------
# SwiGLU
# ---------------------------------------------------------------------------

def test_silu_matches_torch(oq):
    g = np.concatenate([np.linspace(-60, 60, 20001), [0.0, -0.0, 1e-30, -1e-30]])
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    got = oq.silu(g)
    assert np.allclose(got, ref, rtol=4 * 2.0 ** -52, atol=1e-300)
    assert oq.silu(np.array([-1000.0]))[0] == 0.0        # limit, no NaN


def test_silu_odd_part_identity(oq):
    g = np.random.default_rng(1).standard_normal(10000) * 8
    assert np.allclose(oq.silu(g) - oq.silu(-g), g, rtol=8 * 2.0 ** -52, atol=0)


def test_swiglu_reduces_to_quantiser_where_sigmoid_is_one(oq):
    """gate = 64 makes sigmoid exactly 1 in fp64, so y = 64 * up exactly, and the
    result must equal the (pinned) quantiser on 64 * up.  This also fixes which
    half of the row is the gate."""
    from block_scaled_precision_05_amd import workloads
    inter = 256
    up = workloads.activations(8, inter, seed=9)
    gate = torch.full((8, inter), 64.0, dtype=torch.bfloat16)
    h = _bf16_bits(torch.cat([gate, up], dim=1))
    codes, sf, y = oq.swiglu_quantize(h, inter, "e4m3", "ceil")
    assert np.array_equal(y, 64.0 * exact.dequant_bf16(_bf16_bits(up)))
    c2, s2 = oq.quantize_values(64.0 * exact.dequant_bf16(_bf16_bits(up)), "e4m3", "ceil")
    assert np.array_equal(codes, c2) and np.array_equal(sf, s2)
    hs = _bf16_bits(torch.cat([up, gate], dim=1))          # halves swapped: differs
    c3, _, _ = oq.swiglu_quantize(hs, inter, "e4m3", "ceil")
    assert not np.array_equal(c3, codes)


def test_quant_check_accepts_exact_and_rejects_planted_mistakes(oq):
    """The tolerant comparator used for fp32-computed inputs: it accepts the
    oracle's own codes, accepts a flip at an exact rounding midpoint, and
    rejects a wrong code, a wrong sign and a wrong scale away from boundaries."""
    import quant_check
    from block_scaled_precision_05_amd import workloads
    h = _bf16_bits(workloads.activations(16, 512, seed=3))
    codes, sf, y = oq.swiglu_quantize(h, 256, "e4m3", "ceil")
    quant_check.check_quantized(codes, sf, y, "e4m3")
    # a value exactly at a midpoint: both neighbours are acceptable
    y2 = y.copy()
    e = int(sf[0, 0]) - 127
    y2[0, 5] = np.ldexp(1.0625, e)            # midpoint of 1.0 and 1.125 at this scale
    c2, s2 = oq.quantize_values(y2, "e4m3", "ceil")
    c2b = c2.copy()
    c2b[0, 5] = (c2[0, 5] & 0x80) | 0x39      # the odd neighbour
    quant_check.check_quantized(c2b, s2, y2, "e4m3")
    # planted mistakes
    i, k = 3, 17
    far = codes.copy()
    far[i, k] = (far[i, k] & 0x80) | ((far[i, k] & 0x7F) + 2)
    with pytest.raises(AssertionError):
        quant_check.check_quantized(far, sf, y, "e4m3")
    flip = codes.copy()
    flip[i, k] ^= 0x80
    if y[i, k] != 0:
        with pytest.raises(AssertionError):
            quant_check.check_quantized(flip, sf, y, "e4m3")
    sfb = sf.copy()
    sfb[2, 1] += 1
    with pytest.raises(AssertionError):
        quant_check.check_quantized(codes, sfb, y, "e4m3")
