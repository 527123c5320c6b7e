"""GPU parity of the M-grouped BF16 and FP4 GEMMs against the oracle: full small
cases (empty experts, 128-aligned and unaligned row ranges, untouched rows
outside the groups) and the MoE workload shape (256 experts, N=2048, K=7168) on
sampled rows of every expert class."""
import numpy as np
import pytest
import torch

import block_scaled_precision_05_amd as bsg
from block_scaled_precision_05_amd import workloads
import oracle
from parity import assert_parity, gpu_bits

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
SENTINEL = 0x7FC1


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _run(kind, w, pad_rows=0):
    t = w.tensors
    G, N = t["B"].shape[0], t["B"].shape[1]
    K = w.K
    M = t["A"].shape[0]
    D = torch.full((M + pad_rows, N), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    if kind == "bf16":
        bsg.m_grouped_gemm_bf16(t["A"], t["B"], t["offsets"], out=D)
    else:
        sfa = bsg.ensure_packed(t["sfa"], M, K // 32)
        sfb = torch.stack([bsg.ensure_packed(x, N, K // 32) for x in t["sfb"]])
        bsg.m_grouped_gemm_fp4(t["A"], sfa, t["B"], sfb, t["offsets"], K=K, out=D)
    torch.cuda.synchronize()
    return gpu_bits(D)


def _check(kind, w, got, rows, what):
    t = {k: v.cpu() for k, v in w.tensors.items()}
    off = t["offsets"].numpy()
    K = w.K
    g_of = np.searchsorted(off, rows, side="right") - 1
    if kind == "bf16":
        A, B = _u16(t["A"]), np.stack([_u16(b) for b in t["B"]])
        ref = oracle.grouped_bf16(A, B, off, rows=rows)
        na = oracle.row_norms("bf16", A, rows=rows)
        nbs = {g: oracle.row_norms("bf16", B[g]) for g in np.unique(g_of)}
    else:
        A, B = t["A"].numpy(), t["B"].numpy()
        sfa = oracle.pack_scales(t["sfa"].numpy())
        sfb = np.stack([oracle.pack_scales(x) for x in t["sfb"].numpy()])
        ref = oracle.grouped_fp4(A, sfa, B, sfb, off, K, rows=rows)
        na = oracle.row_norms("e2m1", A, sfa, K=K, rows=rows)
        nbs = {g: oracle.row_norms("e2m1", B[g], sfb[g], K=K) for g in np.unique(g_of)}
    for g in np.unique(g_of):
        sel = np.nonzero(g_of == g)[0]
        assert_parity(got[rows[sel]], ref[sel], na[sel], nbs[g], what=f"{what} expert {g}")


@pytest.mark.parametrize("kind", ["bf16", "fp4"])
@pytest.mark.parametrize("align", [128, 1])
def test_grouped_small_full(kind, align):
    _say(f"grouped {kind} small, align {align}")
    K = 512
    w = workloads.grouped(4, 320, K, seed=61, device=DEV, counts=[130, 0, 256, 77], align=align,
                          kind=kind)
    got = _run(kind, w, pad_rows=5)
    off = w.tensors["offsets"].cpu().numpy()
    rows = np.arange(off[0], off[-1])
    _check(kind, w, got, rows, f"grouped {kind} small align {align}")
    assert np.all(got[off[-1]:] == SENTINEL)


@pytest.mark.parametrize("kind", ["bf16", "fp4"])
def test_grouped_half_and_full_row_tiles(kind):
    """Last row tiles of at most half a tile's rows (128, 1, and 257 = a full
    tile then one row) beside full ones, ragged last column tile (N = 320)."""
    _say(f"grouped {kind} half and full row tiles")
    K = 512
    w = workloads.grouped(8, 320, K, seed=62, device=DEV, counts=[129, 128, 257, 1, 384, 255, 0, 64],
                          align=1, kind=kind)
    got = _run(kind, w, pad_rows=3)
    off = w.tensors["offsets"].cpu().numpy()
    _check(kind, w, got, np.arange(off[0], off[-1]), f"grouped {kind} half/full tiles")
    assert np.all(got[off[-1]:] == SENTINEL)


@pytest.mark.parametrize("kind", ["bf16", "fp4"])
def test_grouped_moe_workload_sampled(kind):
    """256 experts, N=2048, K=7168, Zipf routing, in the launch the benchmark
    times; the oracle checks the first, middle and last row of 12 experts."""
    _say(f"grouped {kind} MoE workload, sampled rows")
    w = workloads.make("moe_" + kind, device=DEV)
    got = _run(kind, w)
    off = w.tensors["offsets"].cpu().numpy()
    counts = w.tensors["counts"].cpu().numpy()
    rng = np.random.default_rng(6)
    live = [g for g in range(len(counts)) if counts[g] > 0]
    order = np.argsort(counts)
    pick = sorted(set([int(order[-1]), int(order[-2])] + list(rng.choice(live, 10, replace=False))))
    rows = []
    for g in pick:
        s0, c = int(off[g]), int(counts[g])
        rows += sorted(set([s0, s0 + (c - 1) // 2, s0 + c - 1]))
    _check(kind, w, got, np.array(rows), f"grouped {kind} MoE")


@pytest.mark.parametrize("kind", ["bf16", "fp4"])
def test_grouped_moe_workload_every_expert(kind):
    """Every routed expert of the MoE workload: its first and last routed rows, all
    2048 columns."""
    _say(f"grouped {kind} MoE workload, every expert")
    w = workloads.make("moe_" + kind, device=DEV)
    got = _run(kind, w)
    off = w.tensors["offsets"].cpu().numpy()
    counts = w.tensors["counts"].cpu().numpy()
    rows = []
    for g in range(len(counts)):
        if counts[g] > 0:
            rows += sorted({int(off[g]), int(off[g] + counts[g] - 1)})
    _check(kind, w, got, np.array(rows), f"grouped {kind} MoE, every expert")
