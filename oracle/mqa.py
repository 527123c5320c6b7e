"""Plain CPU oracle of the MQA logits kernel (FP8 and FP4 operands).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages list "MQA logits" among the library's kernels: attention scores of
multi-query attention, part of the DeepSeek Lightning Indexer path, benchmarked
for prefill and decode in FP8 and FP4 (first page, "DeepGEMM-Ascend cobre quantas
operacoes no Ascend 950?", section "Cobertura de operacoes e a lacuna declarada
no repositorio"; third page, section "Kernels especificos de modelo: logits de MQA
e prenorm mHC").  They do not write the computation down.  The reading taken here
is the lightning indexer's index score as DeepSeek published it: every query
token t has H small query heads q[t][h] (head dimension D) and a weight w[t][h];
all heads share one key k[s] per token s (multi-query); the score of key s is

    L[t][s] = sum_h  w[t][h] * max(0, q[t][h] . k[s])

and keys outside the query's window [ks[t], ke[t]) get -inf.  Operands carry the
library's block scales: FP8 e4m3 codes with one UE8M0 scale per 128 elements of
a row, FP4 e2m1 codes (two per byte, even index in the low nibble) with one per
32, packed two per int16, MN-major, as for the GEMMs.  Keys come in groups (one
per sequence): query t reads group t // q_per_group, whose key s is row
(t // q_per_group) * group_rows + s of K.  w is fp32.

Every step is plain: elements decoded exactly to fp64 (the oracle's tables times
the scale), one fp64 matrix product per query (a library matmul), then the
max, the weighted sum over heads and the window, in that order.

Parity: pinned against the GEMM oracle, exact rationals, closed forms and
invariants (tests/test_mqa_pins.py).  Parity to the pages themselves is unpinned:
they print no value of this kernel and do not define it.
"""
from __future__ import annotations

import numpy as np

from . import e2m1_table, e4m3_table, ue8m0_table, unpack_scales

_E4M3 = None
_E2M1 = None
_UE8M0 = None


def _tables():
    global _E4M3, _E2M1, _UE8M0
    if _E4M3 is None:
        _E4M3, _E2M1, _UE8M0 = e4m3_table(), e2m1_table(), ue8m0_table()
    return _E4M3, _E2M1, _UE8M0


def dequant_rows(fmt: str, codes, packed_sf, rows, D: int) -> np.ndarray:
    """fp64 [len(rows)][D] of the given rows: fmt 'e4m3' (codes uint8 [..][>=D],
    one scale per 128) or 'e2m1' (uint8 [..][>=D/2], one scale per 32)."""
    e4m3, e2m1, ue8m0 = _tables()
    codes = np.asarray(codes, dtype=np.uint8)
    rows = np.asarray(rows, dtype=np.int64)
    gk = 128 if fmt == "e4m3" else 32
    kb = D // gk
    if rows.size == 0:
        return np.zeros((0, D))
    lo, hi = int(rows.min()), int(rows.max()) + 1
    packed = np.ascontiguousarray(np.asarray(packed_sf, dtype=np.int16)[:, lo:hi])
    sf = unpack_scales(packed, hi - lo, kb)[rows - lo]
    scale = np.repeat(ue8m0[sf], gk, axis=1)
    if fmt == "e4m3":
        v = e4m3[codes[rows, :D]]
    else:
        b = codes[rows, :D // 2]
        nib = np.empty((rows.size, D), dtype=np.uint8)
        nib[:, 0::2] = b & 0xF
        nib[:, 1::2] = b >> 4
        v = e2m1[nib]
    return v * scale


def mqa_logits(fmt: str, Q, sfq, K, sfk, W, ks, ke, S: int, H: int, q_per_group: int,
               group_rows: int, D: int = 128, queries=None) -> np.ndarray:
    """fp64 logits [len(queries)][S] (all T queries by default).

    Q: codes [T*H][..] (row t*H + h), sfq packed int16 over those rows;
    K: codes [rows][..], sfk packed over K's rows; W: float32 [T][>=H];
    ks, ke: int [T] with 0 <= ks <= ke <= S."""
    W = np.asarray(W, dtype=np.float32)
    T = W.shape[0]
    queries = np.arange(T) if queries is None else np.asarray(queries, dtype=np.int64)
    ks = np.asarray(ks, dtype=np.int64)
    ke = np.asarray(ke, dtype=np.int64)
    out = np.full((queries.size, S), -np.inf)
    keys_cache = {}
    for i, t in enumerate(queries):
        g = int(t) // q_per_group
        if g not in keys_cache:
            keys_cache = {g: dequant_rows(fmt, K, sfk, g * group_rows + np.arange(S), D)}
        k = keys_cache[g]
        q = dequant_rows(fmt, Q, sfq, int(t) * H + np.arange(H), D)
        scores = q @ k.T                                   # [H][S]
        w = W[t, :H].astype(np.float64)
        logits = w @ np.maximum(scores, 0.0)               # [S]
        lo, hi = int(ks[t]), int(ke[t])
        out[i, lo:hi] = logits[lo:hi]
    return out


def norm_denominator(fmt: str, Q, sfq, K, sfk, W, S: int, H: int, q_per_group: int,
                     group_rows: int, D: int = 128, queries=None) -> np.ndarray:
    """sum_h |w[t][h]| * |q[t][h]| * |k[s]| per (query, key): the scale against
    which the GPU's fp32 error is measured."""
    W = np.asarray(W, dtype=np.float32)
    T = W.shape[0]
    queries = np.arange(T) if queries is None else np.asarray(queries, dtype=np.int64)
    out = np.empty((queries.size, S))
    for i, t in enumerate(queries):
        g = int(t) // q_per_group
        k = dequant_rows(fmt, K, sfk, g * group_rows + np.arange(S), D)
        q = dequant_rows(fmt, Q, sfq, int(t) * H + np.arange(H), D)
        qn = np.linalg.norm(q, axis=1)
        kn = np.linalg.norm(k, axis=1)
        out[i] = (np.abs(W[t, :H].astype(np.float64)) * qn).sum() * kn
    return out
