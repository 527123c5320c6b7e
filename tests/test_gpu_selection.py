"""GPU parity, bit for bit, on selection matrices at long K.

Row i of A holds one unit element (BF16 1.0, e4m3 code 0x38 or e2m1 code 0x2,
scale byte 127) at column k_i and zeros elsewhere, so D[i][j] is one element of
the dequantised B, exact in fp32 and in bf16.  The k_i walk every 64-byte K stage
of the kernels' copy ring (row i sits in stage i mod nk at a random offset inside
it): a stage that is dropped, read twice, read from the wrong ring slot or paired
with the wrong scale word changes some output exactly, at any K, where the
normalised error bound alone cannot see it at K = 131072.  The cases cover the
dense shapes' K = 16384 and 131072, K = 2048 (whose launches start with dead
stages) and the grouped kinds at the MoE shapes' K = 7168 and 2048 (dead stages
too).  Expected values are the oracle's, computed in full.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_05_amd as bsg
import oracle
from parity import gpu_bits

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
ELEMS_PER_STAGE = {"bf16": 32, "fp8": 64, "fp4": 128}   # 64 bytes of K per row


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _selection_rows(kind, rows, K, rng):
    """Column k_i of each row: stage i mod nk, random offset inside the stage."""
    per = ELEMS_PER_STAGE[kind]
    nk = K // per
    i = np.arange(rows)
    return (i % nk) * per + rng.integers(0, per, rows)


def _a_selection(kind, k_sel, K):
    M = k_sel.size
    if kind == "bf16":
        A = np.zeros((M, K), dtype=np.uint16)
        A[np.arange(M), k_sel] = 0x3F80
        return A, None
    if kind == "fp8":
        A = np.zeros((M, K), dtype=np.uint8)
        A[np.arange(M), k_sel] = 0x38
        return A, np.full((M, K // 128), 127, dtype=np.uint8)
    codes = np.zeros((M, K), dtype=np.uint8)
    codes[np.arange(M), k_sel] = 0x2
    A = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return A, np.full((M, K // 32), 127, dtype=np.uint8)


def _b_random(kind, N, K, rng):
    if kind == "bf16":
        x = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32))
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16), None
    if kind == "fp8":
        B = rng.integers(0, 256, (N, K), dtype=np.uint8)
        B[(B & 0x7F) == 0x7F] = 0x38                   # no NaN codes
        return B, rng.integers(120, 135, ((N + 127) // 128, K // 128), dtype=np.uint8)
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    return B, rng.integers(118, 137, (N, K // 32), dtype=np.uint8)


def _assert_bits(got, ref, what):
    want = oracle.bf16_rne(ref)
    nz = (want & 0x7FFF) != 0
    bad = int(np.sum(got[nz] != want[nz])) + int(np.sum((got[~nz] & 0x7FFF) != 0))
    assert bad == 0, f"{what}: {bad} of {got.size} outputs differ from the oracle"
    _say(f"  {what}: {got.size} outputs bit-exact")


def _dense_gpu(kind, A, sfa, B, sfb, K):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if kind == "bf16":
        return bsg.gemm_bf16(t(A.view(np.int16)).view(torch.bfloat16),
                             t(B.view(np.int16)).view(torch.bfloat16))
    M, N = A.shape[0], B.shape[0]
    if kind == "fp8":
        return bsg.gemm_fp8_blockscaled(t(A), bsg.ensure_packed(t(sfa), M, K // 128), t(B),
                                        bsg.ensure_packed(t(sfb), (N + 127) // 128, K // 128))
    return bsg.gemm_fp4_blockscaled(t(A), bsg.ensure_packed(t(sfa), M, K // 32), t(B),
                                    bsg.ensure_packed(t(sfb), N, K // 32), K=K)


def _dense_oracle(kind, A, sfa, B, sfb, K):
    if kind == "bf16":
        return oracle.gemm_bf16(A, B)
    if kind == "fp8":
        return oracle.gemm_fp8(A, oracle.pack_scales(sfa), B, oracle.pack_scales(sfb))
    return oracle.gemm_fp4(A, oracle.pack_scales(sfa), B, oracle.pack_scales(sfb), K)


@pytest.mark.parametrize("kind,K", [("bf16", 2048), ("fp8", 2048), ("fp4", 2048),
                                    ("bf16", 16384), ("fp8", 16384), ("fp4", 16384),
                                    ("bf16", 131072), ("fp8", 131072), ("fp4", 131072)])
def test_dense_selection_bit_exact(kind, K):
    N = 200
    rng = np.random.default_rng(K + len(kind))
    nk = K // ELEMS_PER_STAGE[kind]
    M = max(nk, 300)        # every stage at least once, and more than one row tile
    _say(f"selection {kind} M={M} N={N} K={K} ({nk} stages of 64 bytes)")
    k_sel = _selection_rows(kind, M, K, rng)
    A, sfa = _a_selection(kind, k_sel, K)
    B, sfb = _b_random(kind, N, K, rng)
    D = _dense_gpu(kind, A, sfa, B, sfb, K)
    torch.cuda.synchronize()
    ref = _dense_oracle(kind, A, sfa, B, sfb, K)
    _assert_bits(gpu_bits(D), ref, f"{kind} {M}x{N}x{K}")


@pytest.mark.parametrize("kind,K", [("fp8", 7168), ("fp8", 2048), ("bf16", 7168),
                                    ("fp4", 7168)])
def test_grouped_selection_bit_exact(kind, K):
    """Three experts (one empty, one ragged) at the MoE shapes' K: every expert's
    rows walk every stage, including the launch's leading dead stages."""
    N, G = 200, 3
    rng = np.random.default_rng(7 * K + len(kind))
    nk = K // ELEMS_PER_STAGE[kind]
    counts = [nk, 0, nk + 37]
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    _say(f"grouped selection {kind} counts={counts} N={N} K={K} ({nk} stages)")
    k_sel = np.concatenate([_selection_rows(kind, c, K, rng) for c in counts])
    A, sfa = _a_selection(kind, k_sel, K)
    Bs = [_b_random(kind, N, K, rng) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    offd = t(off)
    if kind == "bf16":
        D = bsg.m_grouped_gemm_bf16(t(A.view(np.int16)).view(torch.bfloat16),
                                    t(B.view(np.int16)).view(torch.bfloat16), offd)
        ref = oracle.grouped_bf16(A, B, off)
    elif kind == "fp8":
        sfb = np.stack([s for _, s in Bs])
        sfbp = np.stack([oracle.pack_scales(s) for s in sfb])
        D = bsg.m_grouped_gemm_fp8(t(A), bsg.ensure_packed(t(sfa), M, K // 128), t(B),
                                   t(sfbp), offd)
        ref = oracle.grouped_fp8(A, oracle.pack_scales(sfa), B, sfbp, off)
    else:
        sfb = np.stack([s for _, s in Bs])
        sfbp = np.stack([oracle.pack_scales(s) for s in sfb])
        D = bsg.m_grouped_gemm_fp4(t(A), bsg.ensure_packed(t(sfa), M, K // 32), t(B),
                                   t(sfbp), offd, K=K)
        ref = oracle.grouped_fp4(A, oracle.pack_scales(sfa), B, sfbp, off, K)
    torch.cuda.synchronize()
    _assert_bits(gpu_bits(D), ref, f"grouped {kind} {M}x{N}x{K}")
