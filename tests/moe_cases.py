"""Structured MoE FFN inputs whose result is exact at every step (shared by the
oracle pin and the GPU test; input construction only).

Row i of A is the unit vector at column c_i (e4m3 1.0, scale 1).  Every gate row
of W13 holds 64.0, so H's gate half is 64 and sigmoid(64) is 1 (in fp64 and in
fp32): y = 64 * up.  The up rows of W13 hold e4m3 values v whose every 128-wide
block along the intermediate dimension contains +-448 (up row 0 holds 448 at
every column), so 64 * v quantises back to v's codes.  W2 of expert g is the 0/1
matrix W2[j][n] = [n == (j + g) mod inter].  Hence, for a row i of expert g,

    D[i][j] = 64 * v_g[(j + g) mod inter][c_i]      (a zero is +0, as in any sum)

exactly, and padding rows (zero A) give D = 0.
"""
from __future__ import annotations

import numpy as np
import torch


def e4m3_codes(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def structured(hidden: int, inter: int, counts, seed: int, align: int = 128):
    """Returns dict of numpy arrays: A, sfa (u8), W13, sfw13 (u8), W2, sfw2 (u8),
    offsets, counts, cols, up_values, and the closed-form D [M_total][hidden]."""
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts, dtype=np.int64)
    G = counts.size
    padded = (counts + align - 1) // align * align
    off = np.zeros(G + 1, dtype=np.int32)
    off[1:] = np.cumsum(padded)
    M = int(off[-1])
    one = e4m3_codes([1.0])[0]
    cols = rng.integers(0, hidden, M)
    A = np.zeros((M, hidden), np.uint8)
    valid = np.zeros(M, bool)
    for g in range(G):
        valid[off[g]:off[g] + counts[g]] = True
    A[np.nonzero(valid)[0], cols[valid]] = one
    sfa = np.full((M, hidden // 128), 127, np.uint8)
    W13 = np.zeros((G, 2 * inter, hidden), np.uint8)
    W13[:, :inter, :] = e4m3_codes([64.0])[0]
    up = rng.integers(0, 0x7E, (G, inter, hidden)).astype(np.uint8) | \
        (rng.integers(0, 2, (G, inter, hidden)).astype(np.uint8) << 7)
    for b in range(inter // 128):
        up[:, b * 128, :] = e4m3_codes([448.0])[0]
    W13[:, inter:, :] = up
    sfw13 = np.full((G, (2 * inter + 127) // 128, hidden // 128), 127, np.uint8)
    W2 = np.zeros((G, hidden, inter), np.uint8)
    j = np.arange(hidden)
    for g in range(G):
        W2[g, j, (j + g) % inter] = one
    sfw2 = np.full((G, (hidden + 127) // 128, inter // 128), 127, np.uint8)
    v = e4m3_values(up)
    D = np.zeros((M, hidden))
    for g in range(G):
        for i in range(off[g], off[g] + counts[g]):
            # "+ 0.0": D is a sum of products, so a zero result is +0 even where
            # v holds the e4m3 code of -0
            D[i] = 64.0 * v[g, (j + g) % inter, cols[i]] + 0.0
    return dict(A=A, sfa=sfa, W13=W13, sfw13=sfw13, W2=W2, sfw2=sfw2, offsets=off,
                counts=counts, cols=cols, D=D)
