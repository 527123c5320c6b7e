"""Plain CPU oracle of the MoE FFN core on one GPU's share: grouped up-projection,
SwiGLU + FP8 1x128 requantisation, grouped down-projection.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages describe the fused MoE benchmark as dispatch, two grouped GEMMs,
SwiGLU and combine ("DeepGEMM-Ascend cobre quantas operacoes no Ascend 950?"
third page, "Kernels de computacao: DeepGEMM-Ascend versus DeepGEMM", section
"Execucao de MoE: MegaMoE e distribuicao de especialistas"); this is the part
between dispatch and combine, in the order the pages give, built from the
pinned oracle pieces:

  H  = bf16( grouped_fp8(A, W13) )        rows of expert g use W13[g]
  (Y, sfy) = per-token quantisation of silu(H[:, :I]) * H[:, I:2I]
  D  = Y x W2[g]^T, fp64                   with Y's own scales

The intermediate H is rounded to bf16 (RNE) because that is the stored type of
a grouped GEMM's output.

Parity status: pinned (tests/test_moe_pins.py: a closed form in which sigmoid
is exactly 1 and every step is exact, over two experts with different W2).
"""
from __future__ import annotations

import numpy as np

from . import bf16_rne, gemm_fp8, grouped_fp8, pack_scales
from . import quantize as _q


def expert_of_rows(offsets, rows) -> np.ndarray:
    """Expert index of each row (-1 outside [off[0], off[G]))."""
    off = np.asarray(offsets, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    g = np.searchsorted(off, rows, side="right") - 1
    inside = (rows >= off[0]) & (rows < off[-1])
    return np.where(inside, g, -1)


def moe_ffn(A, sfa, W13, sfw13, W2, sfw2, offsets, rows, rule: str = "ceil"):
    """A e4m3 [M_total][hidden], sfa packed [ceil(hidden/256)][>=M_total];
    W13 e4m3 [G][2I][hidden], sfw13 packed [G][..][>=ceil(2I/128)];
    W2 e4m3 [G][hidden][I], sfw2 packed [G][..][>=ceil(hidden/128)];
    offsets int32 [G+1]; rows: the rows to compute (inside the groups).
    Returns dict with H bits [r][2I], y fp64 [r][I], Y codes [r][I], sfy bytes
    [r][I/128] and D fp64 [r][hidden]."""
    rows = np.asarray(rows, dtype=np.int64)
    W13 = np.asarray(W13)
    W2 = np.asarray(W2)
    G, two_i, hidden = W13.shape
    inter = two_i // 2
    g_of = expert_of_rows(offsets, rows)
    if np.any(g_of < 0):
        raise ValueError("rows outside every group")
    H = grouped_fp8(A, sfa, W13, sfw13, offsets, rows=rows)
    h_bits = bf16_rne(H)
    codes, sf, y = _q.swiglu_quantize(h_bits, inter, "e4m3", rule)
    D = np.empty((rows.size, hidden), dtype=np.float64)
    for g in np.unique(g_of):
        sel = np.nonzero(g_of == g)[0]
        D[sel] = gemm_fp8(codes[sel], pack_scales(sf[sel]), W2[g], sfw2[g])
    return {"H": h_bits, "y": y, "Y": codes, "sfy": sf, "D": D, "expert": g_of}
