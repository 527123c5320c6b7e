"""GPU parity of the masked M-grouped FP8 GEMM against the oracle: valid rows of
every expert to the GEMM acceptance bound, rows past each expert's count left
untouched, counts clamped to [0, capacity]; the benchmark's decode workload on
sampled rows; and the quantiser's output used as the masked GEMM's A."""
import numpy as np
import pytest
import torch

import block_scaled_precision_05_amd as bsg
from block_scaled_precision_05_amd import workloads
import oracle
from oracle import quantize as oq
from parity import assert_parity, gpu_bits

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SENTINEL = 0x7FC1          # a bf16 NaN pattern no GEMM writes


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _run(w, masked_m=None):
    t = w.tensors
    A, B = t["A"], t["B"]
    G, cap, K = A.shape
    N = B.shape[1]
    sfa = bsg.ensure_packed(t["sfa"], G * cap, K // 128)
    sfb = torch.stack([bsg.ensure_packed(x, (N + 127) // 128, K // 128) for x in t["sfb"]])
    m = t["masked_m"] if masked_m is None else masked_m
    D = torch.full((G, cap, N), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    bsg.m_grouped_gemm_fp8_masked(A, sfa, B, sfb, m, out=D)
    torch.cuda.synchronize()
    return D


def _check(w, D, rows_per_expert=None, masked_m=None, what=""):
    t = {k: v.cpu() for k, v in w.tensors.items()}
    G, cap, K = t["A"].shape
    N = t["B"].shape[1]
    m = (t["masked_m"] if masked_m is None else masked_m.cpu()).numpy()
    mc = np.clip(m, 0, cap)
    A = t["A"].reshape(G * cap, K).numpy()
    sfa = oracle.pack_scales(t["sfa"].numpy())
    B = t["B"].numpy()
    sfb = np.stack([oracle.pack_scales(x) for x in t["sfb"].numpy()])
    got = gpu_bits(D.view(G * cap, N))
    for g in range(G):
        if rows_per_expert is None:
            valid = np.arange(mc[g])
        else:
            valid = np.unique(np.array([0, mc[g] // 2, mc[g] - 1])) if mc[g] else np.array([], int)
        rows = g * cap + valid
        if rows.size:
            ref = oracle.masked_fp8(A, sfa, B, sfb, m, cap, rows=rows)
            na = oracle.row_norms("e4m3", A, sfa, rows=rows)
            nb = oracle.row_norms("e4m3", B[g], sfb[g], gran_mn=128)
            assert_parity(got[rows], ref, na, nb, what=f"{what} expert {g}")
        # rows past the count: untouched
        rest = g * cap + np.arange(mc[g], cap)
        if rows_per_expert is not None:
            rest = rest[:: max(1, rest.size // 8)]
        assert np.all(got[rest] == SENTINEL), f"{what}: expert {g} wrote past its count"


def test_masked_small_with_clamps():
    _say("masked small: G=4 cap=192 N=320 K=512, counts -3, 1, 130, 197")
    w = workloads.masked(41, device=DEV, G=4, cap=192, N=320, K=512, counts=[0, 1, 130, 192])
    m = torch.tensor([-3, 1, 130, 197], dtype=torch.int32, device=DEV)
    D = _run(w, m)
    _check(w, D, masked_m=m, what="masked small")


def test_masked_single_expert_full():
    _say("masked G=1, full capacity")
    w = workloads.masked(42, device=DEV, G=1, cap=256, N=256, K=1024, counts=[256])
    D = _run(w)
    _check(w, D, what="masked G=1")


def test_masked_all_empty():
    _say("masked: every count zero")
    w = workloads.masked(43, device=DEV, G=3, cap=128, N=128, K=256, counts=[0, 0, 0])
    D = _run(w)
    assert np.all(gpu_bits(D.view(-1, 128)) == SENTINEL)


def test_masked_decode_workload_sampled_rows():
    """The benchmark's decode case (48 experts, capacity 512, N=4096, K=7168) in
    the launch the benchmark times; 3 rows of every non-empty expert."""
    _say("masked decode workload, sampled rows")
    w = workloads.make("masked_fp8", device=DEV)
    D = _run(w)
    _check(w, D, rows_per_expert=3, what="masked decode")


def test_quantiser_output_feeds_the_masked_gemm():
    """quantize_fp8_per_token on the [G*cap, K] view writes exactly the sfa the
    masked GEMM reads."""
    _say("quantize -> masked GEMM")
    G, cap, N, K = 3, 128, 256, 512
    X = workloads.activations(G * cap, K, seed=44)
    Q, S = bsg.quantize_fp8_per_token(X.to(DEV))
    wb = workloads.masked(45, device=DEV, G=G, cap=cap, N=N, K=K, counts=[5, 128, 77])
    sfb = torch.stack([bsg.ensure_packed(x, (N + 127) // 128, K // 128) for x in wb.tensors["sfb"]])
    m = wb.tensors["masked_m"]
    D = bsg.m_grouped_gemm_fp8_masked(Q.view(G, cap, K), S, wb.tensors["B"], sfb, m)
    torch.cuda.synchronize()
    codes, sf = oq.quantize_rows(X.view(torch.int16).numpy().view(np.uint16), "e4m3", "ceil")
    sfa = oracle.pack_scales(sf)
    B = wb.tensors["B"].cpu().numpy()
    sfb_h = np.stack([oracle.pack_scales(x) for x in wb.tensors["sfb"].cpu().numpy()])
    got = gpu_bits(D.view(G * cap, N))
    for g, c in enumerate([5, 128, 77]):
        rows = g * cap + np.arange(c)
        ref = oracle.masked_fp8(codes, sfa, B, sfb_h, [5, 128, 77], cap, rows=rows)
        na = oracle.row_norms("e4m3", codes, sfa, rows=rows)
        nb = oracle.row_norms("e4m3", B[g], sfb_h[g], gran_mn=128)
        assert_parity(got[rows], ref, na, nb, what=f"quantised A, masked expert {g}")
