"""Acceptance of quantised codes whose input was computed in fp32 on the GPU
(SwiGLU) against the oracle's fp64 values.

The GPU evaluates y = silu(gate) * up in fp32 (a few ulps from the exact value),
so a code (or a block's scale) may legitimately differ from the oracle's where
the exact y sits within that error of a rounding boundary.  The rule: a block's
scale byte must be one that some amax' within relative `rel` of the oracle's
amax gives, and each code must be the rounding of some y' within relative `rel`
of the oracle's y (at the GPU's scale), with y's sign.  Everything else must
match exactly; the number of elements that needed the window is reported.
"""
from __future__ import annotations

import numpy as np

from oracle import quantize as oq

REL = 2.0 ** -18


def _nibbles(codes: np.ndarray, K: int) -> np.ndarray:
    out = np.empty((codes.shape[0], K), dtype=np.uint8)
    out[:, 0::2] = codes[:, : K // 2] & 0xF
    out[:, 1::2] = codes[:, : K // 2] >> 4
    return out


def check_quantized(codes_gpu: np.ndarray, sf_gpu: np.ndarray, y: np.ndarray, fmt: str,
                    rule: str = "ceil", rel: float = REL) -> dict:
    """codes_gpu: e4m3 [M][K] or e2m1 [M][K/2]; sf_gpu: UE8M0 bytes [M][K/gk];
    y: the oracle's fp64 values [M][K].  Raises AssertionError on a failure."""
    gk, qmax, _ = oq.FORMATS[fmt]
    M, K = y.shape
    kb = K // gk
    amax = np.abs(y).reshape(M, kb, gk).max(axis=2)
    b_o = oq.scale_bytes(amax, fmt, rule)
    b_lo = oq.scale_bytes(amax * (1 - rel), fmt, rule)
    b_hi = oq.scale_bytes(amax * (1 + rel), fmt, rule)
    sf_gpu = np.asarray(sf_gpu, dtype=np.uint8)
    bad_b = (sf_gpu < np.minimum(b_lo, b_hi)) | (sf_gpu > np.maximum(b_lo, b_hi))
    assert not bad_b.any(), f"{int(bad_b.sum())} scale bytes outside the window, first " \
        f"{np.argwhere(bad_b)[:3].tolist()}: gpu {sf_gpu[bad_b][:3]} oracle {b_o[bad_b][:3]}"
    e = np.repeat(sf_gpu.astype(np.int64) - 127, gk, axis=1)
    v = np.ldexp(y, -e)
    c_lo = oq.round_to_grid(v * (1 - rel), fmt)
    c_hi = oq.round_to_grid(v * (1 + rel), fmt)
    c_ex = oq.round_to_grid(v, fmt)
    sign_bit = 0x80 if fmt == "e4m3" else 0x8
    got = codes_gpu if fmt == "e4m3" else _nibbles(codes_gpu, K)
    got = np.asarray(got, dtype=np.uint8)
    mag = got & (sign_bit - 1)
    sgn = (got & sign_bit) != 0
    bad_sign = sgn != np.signbit(y)
    bad_mag = (mag < np.minimum(c_lo, c_hi)) | (mag > np.maximum(c_lo, c_hi))
    bad = bad_sign | bad_mag
    assert not bad.any(), f"{int(bad.sum())} codes outside the window, first " \
        f"{np.argwhere(bad)[:3].tolist()}: gpu {got[bad][:3]} exact {c_ex[bad][:3]} y {y[bad][:3]}"
    return {"elements": int(y.size), "blocks": int(sf_gpu.size),
            "bytes_off_exact": int((sf_gpu != b_o).sum()),
            "codes_off_exact": int(((mag != c_ex) & (sf_gpu.repeat(gk, axis=1) == b_o.repeat(gk, axis=1))).sum())}
