"""GPU parity: every entry point of the C ABI against the CPU oracle on the same
seeded bytes.  Small shapes are compared in full; the 4096x7168x16384 and MoE
workloads are compared on sampled rows and columns (every N tile, every expert
class) in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import block_scaled_precision_05_amd as bsg
from block_scaled_precision_05_amd import workloads
import oracle
from parity import assert_parity, gpu_bits, bf16_bits_to_f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


SENTINEL_BITS = 0x7FC1   # a bf16 NaN pattern no GEMM output has


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _u8(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


# ---------------------------------------------------------------------------
# runners
# ---------------------------------------------------------------------------

def run_gpu(kind, t, K=None, out=None):
    """t: device tensors with unpacked uint8 scales; packs them on the GPU."""
    if kind == "bf16":
        return bsg.gemm_bf16(t["A"], t["B"], out=out)
    M, N = t["A"].shape[0], t["B"].shape[0]
    if kind == "fp8":
        K = t["A"].shape[1]
        sfa = bsg.ensure_packed(t["sfa"], M, K // 128)
        sfb = bsg.ensure_packed(t["sfb"], (N + 127) // 128, K // 128)
        return bsg.gemm_fp8_blockscaled(t["A"], sfa, t["B"], sfb, out=out)
    if kind == "fp8_rowb":
        K = t["A"].shape[1]
        sfa = bsg.ensure_packed(t["sfa"], M, K // 128)
        sfb = bsg.ensure_packed(t["sfb"], N, K // 128)
        return bsg.gemm_fp8_blockscaled(t["A"], sfa, t["B"], sfb, out=out, sfb_gran_mn=1)
    K = K if K is not None else 2 * t["A"].shape[1]
    sfa = bsg.ensure_packed(t["sfa"], M, K // 32)
    sfb = bsg.ensure_packed(t["sfb"], N, K // 32)
    return bsg.gemm_fp4_blockscaled(t["A"], sfa, t["B"], sfb, K=K, out=out)


def run_oracle(kind, h, K, rows=None, cols=None):
    """h: host numpy arrays (A, sfa u8, B, sfb u8).  Returns (ref, na, nb)."""
    if kind == "bf16":
        A, B = h["A"].view(np.uint16), h["B"].view(np.uint16)
        ref = oracle.gemm_bf16(A, B, rows=rows, cols=cols)
        na = oracle.row_norms("bf16", A, rows=rows)
        nb = oracle.row_norms("bf16", B, rows=cols)
        return ref, na, nb
    sfa = oracle.pack_scales(h["sfa"])
    sfb = oracle.pack_scales(h["sfb"])
    if kind in ("fp8", "fp8_rowb"):
        gb = 128 if kind == "fp8" else 1
        ref = oracle.gemm_fp8(h["A"], sfa, h["B"], sfb, rows=rows, cols=cols, sfb_gran_mn=gb)
        na = oracle.row_norms("e4m3", h["A"], sfa, rows=rows)
        nb = oracle.row_norms("e4m3", h["B"], sfb, rows=cols, gran_mn=gb)
    else:
        ref = oracle.gemm_fp4(h["A"], sfa, h["B"], sfb, K, rows=rows, cols=cols)
        na = oracle.row_norms("e2m1", h["A"], sfa, K=K, rows=rows)
        nb = oracle.row_norms("e2m1", h["B"], sfb, K=K, rows=cols)
    return ref, na, nb


def host(t):
    out = {}
    for k, v in t.items():
        if v.dtype == torch.bfloat16:
            out[k] = v.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            out[k] = v.contiguous().view(torch.uint8).cpu().numpy() if v.element_size() == 1 \
                else v.cpu().numpy()
    return out


def dense_full(kind, M, N, K, seed):
    w = workloads.dense(kind, M, N, K, seed, device="cpu")
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    D = run_gpu(kind, t, K=K)
    torch.cuda.synchronize()
    ref, na, nb = run_oracle(kind, host(w.tensors), K)
    return assert_parity(gpu_bits(D), ref, na, nb, what=f"{kind} {M}x{N}x{K} seed {seed}")


# ---------------------------------------------------------------------------
# scale packing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mn,kb,ldp", [(1, 1, 1), (5, 3, 5), (1024, 32, 1024), (300, 57, 320),
                                       (7168, 512, 7168)])
def test_pack_unpack_bit_exact(mn, kb, ldp):
    _say(f"pack mn={mn} kb={kb} ld={ldp}")
    g = torch.Generator().manual_seed(mn * 7 + kb)
    sf = torch.randint(0, 256, (mn, kb), generator=g, dtype=torch.int32).to(torch.uint8)
    p = bsg.pack_ue8m0_scales(sf.to(DEV), ld_packed=ldp)
    torch.cuda.synchronize()
    want = oracle.pack_scales(sf.numpy(), ld_packed=ldp)
    got = p.cpu().numpy()
    assert np.array_equal(got[:, :mn], want[:, :mn])
    back = bsg.unpack_ue8m0_scales(p, mn, kb)
    assert np.array_equal(back.cpu().numpy(), sf.numpy())


def test_ensure_packed_reuses_or_converts():
    sf = torch.randint(0, 256, (64, 6), dtype=torch.int32).to(torch.uint8).to(DEV)
    p = bsg.ensure_packed(sf, 64, 6)
    assert p.dtype == torch.int16 and tuple(p.shape) == (3, 64)
    assert bsg.ensure_packed(p, 64, 6) is p
    e8 = sf.view(torch.float8_e8m0fnu)
    assert torch.equal(bsg.ensure_packed(e8, 64, 6), p)
    # fp32 scale factors: the powers of two those bytes stand for convert exactly
    # (byte 255, NaN in UE8M0, stays out: it has no fp32 power of two)
    ok = sf.clamp(max=254)
    f32 = torch.ldexp(torch.ones(64, 6, dtype=torch.float64, device=DEV),
                      ok.to(torch.int64) - 127).to(torch.float32)
    assert torch.equal(bsg.ensure_packed(f32, 64, 6), bsg.ensure_packed(ok, 64, 6))
    with pytest.raises(ValueError):         # byte values read as fp32: not powers of two
        bsg.ensure_packed(sf.float() + 3.0, 64, 6)
    with pytest.raises(TypeError):
        bsg.ensure_packed(sf.to(torch.int64), 64, 6)


def test_fp32_scales_feed_the_gemm_like_their_bytes():
    """FP8 GEMM with scales given as fp32 powers of two (converted on the GPU by the
    library) gives the bits of the same scales given as UE8M0 bytes."""
    w = workloads.dense("fp8", 300, 260, 640, 7777, device=DEV)
    t = w.tensors
    M, N, K = 300, 260, 640
    fa = torch.ldexp(torch.ones(t["sfa"].shape, dtype=torch.float64, device=DEV),
                     t["sfa"].to(torch.int64) - 127).to(torch.float32)
    fb = torch.ldexp(torch.ones(t["sfb"].shape, dtype=torch.float64, device=DEV),
                     t["sfb"].to(torch.int64) - 127).to(torch.float32)
    D1 = bsg.gemm_fp8_blockscaled(t["A"], bsg.ensure_packed(fa, M, K // 128), t["B"],
                                  bsg.ensure_packed(fb, (N + 127) // 128, K // 128))
    D2 = run_gpu("fp8", t)
    torch.cuda.synchronize()
    assert np.array_equal(gpu_bits(D1), gpu_bits(D2))


# ---------------------------------------------------------------------------
# dense parity
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp4", "fp8_rowb"])
def test_dense_small(kind):
    _say(f"dense small {kind}")
    dense_full(kind, 256, 256, 512, 1001)


@pytest.mark.parametrize("kind,M,N,K", [
    ("bf16", 300, 520, 200), ("bf16", 1, 1, 8), ("bf16", 513, 257, 1032),
    ("fp8", 300, 520, 384), ("fp8", 1, 129, 128), ("fp8", 777, 300, 1152),
    ("fp4", 300, 520, 224), ("fp4", 3, 5, 32), ("fp4", 600, 270, 1056),
    ("fp8_rowb", 300, 520, 384), ("fp8_rowb", 1, 129, 128), ("fp8_rowb", 777, 300, 1152),
])
def test_dense_ragged(kind, M, N, K):
    _say(f"dense ragged {kind} {M}x{N}x{K}")
    dense_full(kind, M, N, K, 2000 + M)


# The stage loop runs whole rounds of ten 64-byte stages; when the number of stages
# nk is not a multiple of ten, the first round starts with an even number of stages
# that hold no data (and an odd nk leaves one at the end).  These K values give every
# remainder for every kind: nk = ceil(bytes of K per row / 64).
@pytest.mark.parametrize("kind,K", [
    ("fp8", 128), ("fp8", 256), ("fp8", 384), ("fp8", 512), ("fp8", 640), ("fp8", 6528),
    ("fp8_rowb", 256), ("fp8_rowb", 640), ("fp8_rowb", 6528),
    ("fp4", 32), ("fp4", 160), ("fp4", 288), ("fp4", 544), ("fp4", 800), ("fp4", 1184),
    ("fp4", 3264),
    ("bf16", 8), ("bf16", 40), ("bf16", 104), ("bf16", 168), ("bf16", 232), ("bf16", 296),
    ("bf16", 3272),
])
def test_every_stage_remainder(kind, K):
    _say(f"stage remainder {kind} 300x260x{K}")
    dense_full(kind, 300, 260, K, 3000 + K)


# The dense grid gives every workgroup the same number of tiles where it can: 300
# tiles run as 152 workgroups (two tiles each, the last four with one), 520 tiles as
# 176 (three each, the last eight with two); every output tile must still be
# computed exactly once.
@pytest.mark.parametrize("M,N", [(20 * 256, 15 * 256), (26 * 256 - 37, 20 * 256 - 5)])
def test_dense_grid_with_uneven_tiles_per_workgroup(M, N):
    _say(f"dense grid fp8 {M}x{N}x256")
    dense_full("fp8", M, N, 256, 4000 + M)


def test_fp8_mid_workload():
    """FP8 1024x2048x4096 with 1x128 / 128x128 scales, compared in full."""
    _say("fp8 1024x2048x4096")
    w = workloads.make("fp8_mid", device="cpu")
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    D = run_gpu("fp8", t)
    torch.cuda.synchronize()
    ref, na, nb = run_oracle("fp8", host(w.tensors), w.K)
    assert_parity(gpu_bits(D), ref, na, nb, what="fp8_mid full")


def test_bf16_small_workload():
    _say("bf16 256x256x512")
    w = workloads.make("bf16_small", device="cpu")
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    D = run_gpu("bf16", t)
    torch.cuda.synchronize()
    ref, na, nb = run_oracle("bf16", host(w.tensors), w.K)
    assert_parity(gpu_bits(D), ref, na, nb, what="bf16_small full")


LARGE = {"bf16": "bf16_large", "fp8": "fp8_large", "fp4": "fp4_large", "fp8_rowb": "fp8_rowb_large"}


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp4", "fp8_rowb"])
def test_large_workload_sampled(kind):
    """4096x7168x16384: sampled rows x all columns and sampled columns x all rows."""
    name = LARGE[kind]
    _say(f"large {name}: generating on the GPU")
    w = workloads.make(name, device=DEV)
    D = run_gpu(kind, w.tensors, K=w.K)
    torch.cuda.synchronize()
    _say(f"large {name}: GPU done, oracle on samples")
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 2047, 4095],
                                     g.integers(0, w.M, 4)]))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, 223, 224, 255, 256, 3583, 7167],
                                     g.integers(0, w.N, 2)]))
    h = host(w.tensors)
    ref, na, nb = run_oracle(kind, h, w.K, rows=rows)
    Dh = gpu_bits(D)
    assert_parity(Dh[rows], ref, na, nb, what=f"{name} rows {len(rows)} x all cols")
    ref, na, nb = run_oracle(kind, h, w.K, cols=cols)
    assert_parity(Dh[:, cols], ref, na, nb, what=f"{name} all rows x cols {len(cols)}")


# ---------------------------------------------------------------------------
# structured cases with exactly known results (bit-exact)
# ---------------------------------------------------------------------------

def test_fp8_identity_gives_dequant_b_bit_exact():
    K = 512
    g = torch.Generator().manual_seed(11)
    B = torch.randint(0, 256, (300, K), generator=g, dtype=torch.int32).to(torch.uint8)
    B[(B & 0x7F) == 0x7F] = 0x38
    sfb = torch.randint(120, 135, (3, K // 128), generator=g, dtype=torch.int32).to(torch.uint8)
    A = torch.zeros(K, K, dtype=torch.uint8)
    A[torch.arange(K), torch.arange(K)] = 0x38
    sfa = torch.full((K, K // 128), 127, dtype=torch.uint8)
    t = {"A": A.to(DEV), "sfa": sfa.to(DEV), "B": B.to(DEV), "sfb": sfb.to(DEV)}
    D = run_gpu("fp8", t)
    ref = oracle.gemm_fp8(A.numpy(), oracle.pack_scales(sfa.numpy()), B.numpy(),
                          oracle.pack_scales(sfb.numpy()))
    got, want = gpu_bits(D), oracle.bf16_rne(ref)
    nz = (want & 0x7FFF) != 0
    assert np.array_equal(got[nz], want[nz]) and np.all((got[~nz] & 0x7FFF) == 0)


def test_fp4_identity_gives_dequant_b_bit_exact():
    K = 256
    g = torch.Generator().manual_seed(12)
    B = torch.randint(0, 256, (200, K // 2), generator=g, dtype=torch.int32).to(torch.uint8)
    sfb = torch.randint(118, 136, (200, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
    codes = torch.zeros(K, K, dtype=torch.uint8)
    codes[torch.arange(K), torch.arange(K)] = 0x2
    A = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
    sfa = torch.full((K, K // 32), 127, dtype=torch.uint8)
    t = {"A": A.to(DEV), "sfa": sfa.to(DEV), "B": B.to(DEV), "sfb": sfb.to(DEV)}
    D = run_gpu("fp4", t, K=K)
    ref = oracle.gemm_fp4(A.numpy(), oracle.pack_scales(sfa.numpy()), B.numpy(),
                          oracle.pack_scales(sfb.numpy()), K)
    got, want = gpu_bits(D), oracle.bf16_rne(ref)
    nz = (want & 0x7FFF) != 0
    assert np.array_equal(got[nz], want[nz]) and np.all((got[~nz] & 0x7FFF) == 0)


@pytest.mark.parametrize("kind", ["fp8", "fp4", "fp8_rowb"])
def test_scale_only_closed_form_bit_exact(kind):
    """Unit codes everywhere: D depends on the scales alone.  Scale exponents lie in
    [-4, 3], so every partial sum of the accumulation fits fp32's 24-bit significand
    in any order and the result is exact.  (With exponents in [-7, 5] and one B scale
    per row, a few sums need 25 bits: the GPU's fp32 result then differs from the
    exact one by a rounding, which is right but not bit-exact.)"""
    M, N = 200, 300
    K = 32 * 14 if kind == "fp4" else 128 * 6
    g = torch.Generator().manual_seed(13)
    if kind != "fp4":
        A = torch.full((M, K), 0x38, dtype=torch.uint8)
        B = torch.full((N, K), 0x38, dtype=torch.uint8)
        sfa = torch.randint(123, 131, (M, K // 128), generator=g, dtype=torch.int32).to(torch.uint8)
        sb_rows = N if kind == "fp8_rowb" else (N + 127) // 128
        sfb = torch.randint(123, 131, (sb_rows, K // 128), generator=g,
                            dtype=torch.int32).to(torch.uint8)
    else:
        A = torch.full((M, K // 2), 0x22, dtype=torch.uint8)
        B = torch.full((N, K // 2), 0x22, dtype=torch.uint8)
        sfa = torch.randint(123, 131, (M, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
        sfb = torch.randint(123, 131, (N, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
    t = {"A": A.to(DEV), "sfa": sfa.to(DEV), "B": B.to(DEV), "sfb": sfb.to(DEV)}
    D = run_gpu(kind, t, K=K)
    ref, _, _ = run_oracle(kind, host({"A": A, "sfa": sfa, "B": B, "sfb": sfb}), K)
    assert np.array_equal(gpu_bits(D), oracle.bf16_rne(ref))


@pytest.mark.parametrize("wide", [True, False])
def test_fp8_per_row_b_scales_repeating_blocks_equal_block_scales(wide):
    """Per-row B scales that repeat every 128-row block's byte must give the bits of
    the 128x128 call (ragged last block), with the A scale words loaded wide (8-byte
    aligned, leading dimension a multiple of 4) or two bytes at a time."""
    M, N, K = 336, 300, 1152                    # ld_sfa = M, a multiple of 4
    w = workloads.dense("fp8", M, N, K, 4242, device=DEV)
    t = w.tensors
    sfa = bsg.ensure_packed(t["sfa"], M, K // 128)
    if not wide:
        wider = torch.zeros(sfa.shape[0], M + 1, dtype=torch.int16, device=DEV)
        wider[:, :M] = sfa
        sfa = wider[:, :M]                       # leading dimension M + 1: not a multiple of 4
    blk = bsg.ensure_packed(t["sfb"], (N + 127) // 128, K // 128)
    rows = bsg.ensure_packed(t["sfb"].repeat_interleave(128, 0)[:N].contiguous(), N, K // 128)
    D128 = bsg.gemm_fp8_blockscaled(t["A"], sfa, t["B"], blk)
    D1 = bsg.gemm_fp8_blockscaled(t["A"], sfa, t["B"], rows, sfb_gran_mn=1)
    torch.cuda.synchronize()
    assert np.array_equal(gpu_bits(D1), gpu_bits(D128))


def test_all_ones_gives_K():
    K = 4096
    A = torch.ones(130, K, dtype=torch.bfloat16, device=DEV)
    D = bsg.gemm_bf16(A, A[:70])
    assert torch.all(D.float() == K)


def test_k_zero_writes_zeros_and_empty_is_noop():
    A = torch.zeros(10, 0, dtype=torch.bfloat16, device=DEV)
    B = torch.zeros(20, 0, dtype=torch.bfloat16, device=DEV)
    out = torch.full((10, 24), 3.0, dtype=torch.bfloat16, device=DEV)
    bsg.gemm_bf16(A, B, out=out)
    assert torch.all(out[:, :20] == 0) and torch.all(out[:, 20:] == 3.0)
    E = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    assert bsg.gemm_bf16(E, torch.zeros(8, 64, dtype=torch.bfloat16, device=DEV)).shape == (0, 8)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("col0,pad", [(0, 0), (0, 4), (4, 4), (2, 6), (1, 3)])
def test_output_alignment_and_stride(kind, col0, pad):
    """D written into a wider buffer at column col0 with leading dimension N + pad:
    16-byte, 8-byte and 2-byte stores of the staged rows give the same bits as a
    contiguous D, and nothing outside the window is written."""
    _say(f"output window {kind} col0={col0} pad={pad}")
    M, N, K = 300, 264, 512
    w = workloads.dense(kind, M, N, K, 77, device=DEV)
    ref = run_gpu(kind, w.tensors, K=K)
    buf = torch.full((M, N + pad), SENTINEL_BITS, dtype=torch.int16, device=DEV)
    out = buf.view(torch.bfloat16)[:, col0:col0 + N]
    run_gpu(kind, w.tensors, K=K, out=out)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got[:, col0:col0 + N], ref.view(torch.int16).cpu().numpy())
    assert np.all(got[:, :col0] == SENTINEL_BITS) and np.all(got[:, col0 + N:] == SENTINEL_BITS)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp4"])
def test_run_to_run_bitwise_deterministic(kind):
    w = workloads.dense(kind, 1024, 1536, 2048, 99, device=DEV)
    D1 = run_gpu(kind, w.tensors, K=w.K)
    D2 = run_gpu(kind, w.tensors, K=w.K)
    torch.cuda.synchronize()
    assert torch.equal(D1.view(torch.int16), D2.view(torch.int16))


# ---------------------------------------------------------------------------
# grouped
# ---------------------------------------------------------------------------

def run_grouped(w, out=None):
    t = w.tensors
    K = w.K
    sfa = bsg.ensure_packed(t["sfa"], t["A"].shape[0], K // 128)
    sfb = torch.stack([bsg.ensure_packed(s, (w.N + 127) // 128, K // 128) for s in t["sfb"]])
    return bsg.m_grouped_gemm_fp8(t["A"], sfa, t["B"], sfb, t["offsets"], out=out)


def grouped_oracle(w, rows, experts_needed=None):
    t = w.tensors
    off = t["offsets"].cpu().numpy()
    A = _u8(t["A"])
    sfa = oracle.pack_scales(t["sfa"].cpu().numpy())
    G = off.size - 1
    # decode only the experts that own a sampled row (the rest are not read)
    need = sorted({int(np.searchsorted(off, r, side="right") - 1) for r in rows
                   if off[0] <= r < off[-1]})
    Bsub = np.stack([_u8(t["B"][g]) for g in need]) if need else np.zeros((0, w.N, w.K), np.uint8)
    sfbsub = np.stack([oracle.pack_scales(t["sfb"][g].cpu().numpy()) for g in need]) if need else \
        np.zeros((0, 1, 1), np.int16)
    sub_off = []
    # remap rows of the needed experts onto a compact offset table
    ref = np.full((len(rows), w.N), np.nan)
    na = np.zeros(len(rows))
    nb_by_g = {}
    for i, r in enumerate(rows):
        if not (off[0] <= r < off[-1]):
            continue
        g = int(np.searchsorted(off, r, side="right") - 1)
        j = need.index(g)
        one_off = np.array([0, 1], np.int32)
        ref[i] = oracle.grouped_fp8(A[r:r + 1], oracle.pack_scales(t["sfa"][r:r + 1].cpu().numpy()),
                                    Bsub[j:j + 1], sfbsub[j:j + 1], one_off)[0]
        na[i] = oracle.row_norms("e4m3", A[r:r + 1],
                                 oracle.pack_scales(t["sfa"][r:r + 1].cpu().numpy()))[0]
        if g not in nb_by_g:
            nb_by_g[g] = oracle.row_norms("e4m3", Bsub[j], sfbsub[j], gran_mn=128)
    return ref, na, nb_by_g, off


def check_grouped(w, D, rows, what):
    ref, na, nb_by_g, off = grouped_oracle(w, rows)
    Dh = gpu_bits(D)
    for i, r in enumerate(rows):
        if not (off[0] <= r < off[-1]):
            continue
        g = int(np.searchsorted(off, r, side="right") - 1)
        assert_parity(Dh[r:r + 1], ref[i:i + 1], na[i:i + 1], nb_by_g[g],
                      what=f"{what} row {r} expert {g}")


def test_grouped_small_full():
    w = workloads.grouped(5, 640, 512, seed=21, device=DEV, counts=[128, 0, 256, 128, 0])
    D = run_grouped(w)
    torch.cuda.synchronize()
    rows = np.arange(w.tensors["A"].shape[0])
    # full comparison through the oracle's own grouped path
    t = w.tensors
    ref = oracle.grouped_fp8(_u8(t["A"]), oracle.pack_scales(t["sfa"].cpu().numpy()),
                             np.stack([_u8(b) for b in t["B"]]),
                             np.stack([oracle.pack_scales(s.cpu().numpy()) for s in t["sfb"]]),
                             t["offsets"].cpu().numpy(), rows=rows)
    na = oracle.row_norms("e4m3", _u8(t["A"]), oracle.pack_scales(t["sfa"].cpu().numpy()))
    off = t["offsets"].cpu().numpy()
    Dh = gpu_bits(D)
    for g in range(5):
        lo, hi = off[g], off[g + 1]
        if hi > lo:
            nb = oracle.row_norms("e4m3", _u8(t["B"][g]), oracle.pack_scales(t["sfb"][g].cpu().numpy()),
                                  gran_mn=128)
            assert_parity(Dh[lo:hi], ref[lo:hi], na[lo:hi], nb, what=f"grouped small expert {g}")


# Every remainder of the grouped stage loop: K = 128, 256, 640 and 2048 give 2, 4,
# 10 and 32 stages of 64 bytes, i.e. 8, 6, 0 and 8 leading dead stages.
@pytest.mark.parametrize("K", [128, 256, 640, 2048])
def test_grouped_every_stage_remainder(K):
    _say(f"grouped stage remainder K={K}")
    w = workloads.grouped(5, 384, K, seed=30 + K, device=DEV, counts=[256, 0, 384, 128, 0])
    D = run_grouped(w)
    torch.cuda.synchronize()
    t = w.tensors
    off = t["offsets"].cpu().numpy()
    A8, sfa = _u8(t["A"]), oracle.pack_scales(t["sfa"].cpu().numpy())
    ref = oracle.grouped_fp8(A8, sfa, np.stack([_u8(b) for b in t["B"]]),
                             np.stack([oracle.pack_scales(x.cpu().numpy()) for x in t["sfb"]]),
                             off, rows=np.arange(off[-1]))
    na = oracle.row_norms("e4m3", A8, sfa)
    Dh = gpu_bits(D)
    for g in range(5):
        lo, hi = off[g], off[g + 1]
        if hi > lo:
            nb = oracle.row_norms("e4m3", _u8(t["B"][g]), oracle.pack_scales(t["sfb"][g].cpu().numpy()),
                                  gran_mn=128)
            assert_parity(Dh[lo:hi], ref[lo:hi], na[lo:hi], nb, what=f"grouped K={K} expert {g}")


def test_grouped_half_and_full_row_tiles():
    """Experts whose last row tile holds at most half a tile's rows (129 = one
    full-height tile, 128 and 1 = half tiles, 257 = a full tile then one row)
    next to multi-tile experts, with a ragged last column tile (N = 320)."""
    counts = [129, 128, 257, 1, 384, 255, 0, 64]
    G, N, K = len(counts), 320, 1024
    w = workloads.grouped(G, N, K, seed=24, device=DEV, counts=counts, align=1)
    D = run_grouped(w)
    torch.cuda.synchronize()
    t = w.tensors
    off = t["offsets"].cpu().numpy()
    rows = np.arange(off[-1])
    A8, sfa = _u8(t["A"]), oracle.pack_scales(t["sfa"].cpu().numpy())
    ref = oracle.grouped_fp8(A8, sfa, np.stack([_u8(b) for b in t["B"]]),
                             np.stack([oracle.pack_scales(s.cpu().numpy()) for s in t["sfb"]]),
                             off, rows=rows)
    na = oracle.row_norms("e4m3", A8, sfa)
    Dh = gpu_bits(D)
    for g in range(G):
        lo, hi = off[g], off[g + 1]
        if hi > lo:
            nb = oracle.row_norms("e4m3", _u8(t["B"][g]), oracle.pack_scales(t["sfb"][g].cpu().numpy()),
                                  gran_mn=128)
            assert_parity(Dh[lo:hi], ref[lo:hi], na[lo:hi], nb, what=f"half/full tiles expert {g}")


def test_grouped_many_experts_mostly_empty():
    """1024 experts (the most the library takes), all but four empty and the
    non-empty ones far apart: the expert search walks sixteen 64-expert chunks."""
    G, N, K = 1024, 256, 256
    counts = [0] * G
    counts[3], counts[200], counts[700], counts[1023] = 5, 130, 1, 64
    w = workloads.grouped(G, N, K, seed=25, device=DEV, counts=counts, align=1)
    D = run_grouped(w)
    torch.cuda.synchronize()
    t = w.tensors
    off = t["offsets"].cpu().numpy()
    rows = np.arange(off[-1])
    A8, sfa = _u8(t["A"]), oracle.pack_scales(t["sfa"].cpu().numpy())
    live = [g for g in range(G) if counts[g]]
    Bh = np.zeros((G,) + tuple(t["B"].shape[1:]), dtype=np.uint8)
    Sh = np.zeros((G,) + tuple(oracle.pack_scales(t["sfb"][0].cpu().numpy()).shape), dtype=np.int16)
    for g in live:
        Bh[g] = _u8(t["B"][g])
        Sh[g] = oracle.pack_scales(t["sfb"][g].cpu().numpy())
    ref = oracle.grouped_fp8(A8, sfa, Bh, Sh, off, rows=rows)
    na = oracle.row_norms("e4m3", A8, sfa)
    Dh = gpu_bits(D)
    for g in live:
        lo, hi = off[g], off[g + 1]
        nb = oracle.row_norms("e4m3", Bh[g], Sh[g], gran_mn=128)
        assert_parity(Dh[lo:hi], ref[lo:hi], na[lo:hi], nb, what=f"1024 experts, expert {g}")


def test_grouped_unaligned_offsets_and_untouched_rows():
    """Offsets need no alignment; rows outside [off[0], off[G]) are not written."""
    G, N, K = 5, 256, 256
    w = workloads.grouped(G, N, K, seed=22, device=DEV, counts=[100, 0, 37, 300, 1], align=1)
    t = w.tensors
    # shift every expert by 5 rows: rows 0..4 and the tail belong to no expert
    Mt = t["A"].shape[0] + 9
    A = torch.zeros(Mt, K, dtype=torch.uint8, device=DEV)
    A[5:5 + t["A"].shape[0]] = t["A"]
    sfa = torch.full((Mt, K // 128), 127, dtype=torch.uint8, device=DEV)
    sfa[5:5 + t["A"].shape[0]] = t["sfa"]
    off = (t["offsets"] + 5).to(torch.int32)
    w.tensors.update(A=A, sfa=sfa, offsets=off)
    out = torch.full((Mt, N), -7.0, dtype=torch.bfloat16, device=DEV)
    run_grouped(w, out=out)
    torch.cuda.synchronize()
    o = off.cpu().numpy()
    assert torch.all(out[:o[0]] == -7.0) and torch.all(out[o[-1]:] == -7.0)
    rows = list(range(o[0], o[-1]))
    check_grouped(w, out, rows[:: max(1, len(rows) // 60)] + [o[-1] - 1], "grouped unaligned")


def test_grouped_single_expert_equals_dense():
    K, N = 512, 384
    w = workloads.grouped(1, N, K, seed=23, device=DEV, counts=[384])
    D = run_grouped(w)
    t = w.tensors
    sfa = bsg.ensure_packed(t["sfa"], 384, K // 128)
    sfb = bsg.ensure_packed(t["sfb"][0], 3, K // 128)
    Dd = bsg.gemm_fp8_blockscaled(t["A"], sfa, t["B"][0], sfb)
    torch.cuda.synchronize()
    assert torch.equal(D.view(torch.int16), Dd.view(torch.int16))


def test_grouped_offsets_outside_the_precondition_stay_in_bounds():
    """Device offsets that break the documented precondition (a negative first
    offset, a decreasing pair, a last offset past M_total) are clamped into
    [0, M_total] by the kernel: every row it writes lies inside D, the rows past
    M_total of the output buffer keep their sentinel, and the rows only one expert
    covers hold that expert's result."""
    _say("grouped FP8 with out-of-range offsets")
    M, N, K, G = 256, 256, 512, 3
    w = workloads.grouped(G, N, K, 4343, device=DEV, counts=[128, 0, 128])
    t = w.tensors
    A = t["A"][:M].contiguous()
    sfa_u8 = t["sfa"][:M].contiguous()
    sfa = bsg.ensure_packed(sfa_u8, M, K // 128)
    sfb = torch.stack([bsg.ensure_packed(x, (N + 127) // 128, K // 128) for x in t["sfb"]])
    off = torch.tensor([-5, 100, 50, 10 ** 6], dtype=torch.int32, device=DEV)
    buf = torch.full((M + 64, N), 0, dtype=torch.int16, device=DEV)
    buf.fill_(SENTINEL_BITS)
    D = buf.view(torch.bfloat16)
    bsg.m_grouped_gemm_fp8(A, sfa, t["B"], sfb, off, out=D[:M])
    torch.cuda.synchronize()
    got = gpu_bits(D)
    assert np.all(got[M:] == SENTINEL_BITS), "rows past M_total were written"
    Ah, sfah = _u8(A), oracle.pack_scales(sfa_u8.cpu().numpy())
    na = oracle.row_norms("e4m3", Ah, sfah)
    ref, nb = {}, {}
    for g in (0, 2):
        Bg = _u8(t["B"][g])
        sfbg = oracle.pack_scales(t["sfb"][g].cpu().numpy())
        ref[g] = oracle.gemm_fp8(Ah, sfah, Bg, sfbg)
        nb[g] = oracle.row_norms("e4m3", Bg, sfbg, gran_mn=128)
    # expert 0: rows [0, 100); expert 1: empty; expert 2: rows [50, 256)
    assert_parity(got[:50], ref[0][:50], na[:50], nb[0], what="rows of expert 0 only")
    assert_parity(got[100:M], ref[2][100:M], na[100:M], nb[2], what="rows of expert 2 only")
    # rows both ranges cover: every element is one of the two experts' results
    mid = bf16_bits_to_f64(got[50:100])
    err = [np.abs(mid - ref[g][50:100]) / (na[50:100, None] * nb[g][None, :]) for g in (0, 2)]
    assert np.all(np.minimum(err[0], err[1]) <= 4e-3)


def test_grouped_moe_workload_sampled():
    """256 experts, N=2048, K=7168, Zipf(1.1) routing padded to 128 rows."""
    _say("moe_fp8: generating on the GPU")
    w = workloads.make("moe_fp8", device=DEV)
    D = run_grouped(w)
    torch.cuda.synchronize()
    _say("moe_fp8: GPU done, oracle on samples")
    off = w.tensors["offsets"].cpu().numpy()
    counts = w.tensors["counts"].cpu().numpy()
    big = int(np.argmax(counts))
    nz = np.nonzero(counts)[0]
    small = int(nz[np.argmin(counts[nz])])
    rows = [off[big], off[big] + 1, off[big + 1] - 1, off[small], off[small] + counts[small] - 1,
            off[small + 1] - 1, off[0], off[-1] - 1]
    g = np.random.default_rng(7)
    rows += list(g.integers(off[0], off[-1], 6))
    check_grouped(w, D, sorted(set(int(r) for r in rows)), "moe_fp8")


def test_grouped_moe_workload_every_expert():
    """Every routed expert of the MoE workload: its first row, its last routed row and
    its last padded row, all 2048 columns, against one oracle call over the whole
    expert tensor (copied to the host)."""
    _say("moe_fp8: every expert, GPU")
    w = workloads.make("moe_fp8", device=DEV)
    D = run_grouped(w)
    torch.cuda.synchronize()
    t = w.tensors
    off = t["offsets"].cpu().numpy()
    counts = t["counts"].cpu().numpy()
    rows = []
    for g in range(len(counts)):
        if off[g + 1] > off[g]:
            rows += sorted({int(off[g]), int(off[g] + max(counts[g], 1) - 1), int(off[g + 1] - 1)})
    rows = np.array(rows)
    _say(f"moe_fp8: oracle on {rows.size} rows of {int((off[1:] > off[:-1]).sum())} experts")
    A = _u8(t["A"])
    sfa = oracle.pack_scales(t["sfa"].cpu().numpy())
    B = _u8(t["B"])
    sfb = np.stack([oracle.pack_scales(x) for x in t["sfb"].cpu().numpy()])
    ref = oracle.grouped_fp8(A, sfa, B, sfb, off, rows=rows)
    na = oracle.row_norms("e4m3", A, sfa, rows=rows)
    Dh = gpu_bits(D)
    g_of = np.searchsorted(off, rows, side="right") - 1
    for g in np.unique(g_of):
        sel = np.nonzero(g_of == g)[0]
        nb = oracle.row_norms("e4m3", B[g], sfb[g], gran_mn=128)
        assert_parity(Dh[rows[sel]], ref[sel], na[sel], nb, what=f"moe_fp8 expert {g}")


def test_fp4_scale_load_variants_agree():
    """FP4 fetches a lane's four scale words with one 8-byte load when the packed
    arrays allow it (8-byte aligned, leading dimension a multiple of 4) and with
    2-byte loads otherwise; both must give the same bits, and match the oracle."""
    _say("fp4 scale load variants")
    M, N, K = 512, 384, 1024
    w = workloads.dense("fp4", M, N, K, 77, device="cpu")
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    outs = []
    for pad in (0, 2):
        sfa = bsg.pack_ue8m0_scales(t["sfa"], ld_packed=M + pad)
        sfb = bsg.pack_ue8m0_scales(t["sfb"], ld_packed=N + pad)
        outs.append(gpu_bits(bsg.gemm_fp4_blockscaled(t["A"], sfa[:, :M], t["B"], sfb[:, :N], K=K)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])
    ref, na, nb = run_oracle("fp4", host(w.tensors), K)
    assert_parity(outs[0], ref, na, nb, what="fp4 512x384x1024 (8-byte scale loads)")


@pytest.mark.parametrize("kind,M,N", [("fp8", 423, 300), ("fp8", 421, 256),
                                      ("fp4", 423, 301), ("fp4", 512, 302), ("fp4", 257, 255)])
def test_wide_scale_loads_with_rows_not_a_multiple_of_four(kind, M, N):
    """Packed scale arrays whose leading dimension is a multiple of 4 (so the wide
    8- and 4-byte scale loads are taken) while the scale rows are not: the last
    row group's load must still deliver the words of the rows that exist, in every
    packed row including the last one."""
    K = 1024 if kind == "fp8" else 448
    _say(f"{kind} {M}x{N}x{K} with wide scale loads over ragged scale rows")
    w = workloads.dense(kind, M, N, K, 81 + M + N, device="cpu")
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    pad = lambda n: (n + 3) // 4 * 4
    if kind == "fp8":
        sfa = bsg.pack_ue8m0_scales(t["sfa"], ld_packed=pad(M))[:, :M]
        sfb = bsg.ensure_packed(t["sfb"], (N + 127) // 128, K // 128)
        D = bsg.gemm_fp8_blockscaled(t["A"], sfa, t["B"], sfb)
    else:
        sfa = bsg.pack_ue8m0_scales(t["sfa"], ld_packed=pad(M))[:, :M]
        sfb = bsg.pack_ue8m0_scales(t["sfb"], ld_packed=pad(N))[:, :N]
        D = bsg.gemm_fp4_blockscaled(t["A"], sfa, t["B"], sfb, K=K)
    torch.cuda.synchronize()
    ref, na, nb = run_oracle(kind, host(w.tensors), K)
    assert_parity(gpu_bits(D), ref, na, nb, what=f"{kind} {M}x{N}x{K}, scale rows padded to 4")


def test_fp8_scale_load_variants_agree():
    """FP8 fetches a lane's four A scale words with one 8-byte load when sfa
    allows it and with 2-byte loads otherwise: same bits, dense and grouped."""
    _say("fp8 scale load variants (dense and grouped)")
    M, N, K = 512, 384, 1024
    w = workloads.dense("fp8", M, N, K, 78, device="cpu")
    t = {k: v.to(DEV) for k, v in w.tensors.items()}
    sfb = bsg.ensure_packed(t["sfb"], (N + 127) // 128, K // 128)
    outs = []
    for pad in (0, 2):
        sfa = bsg.pack_ue8m0_scales(t["sfa"], ld_packed=M + pad)[:, :M]
        outs.append(gpu_bits(bsg.gemm_fp8_blockscaled(t["A"], sfa, t["B"], sfb)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])
    ref, na, nb = run_oracle("fp8", host(w.tensors), K)
    assert_parity(outs[0], ref, na, nb, what="fp8 512x384x1024 (8-byte A scale loads)")
    g = workloads.grouped(4, 256, 512, seed=79, counts=[130, 0, 256, 77], device=DEV)
    tg = g.tensors
    Mt = tg["A"].shape[0]
    sfbg = torch.stack([bsg.ensure_packed(x, 2, 4) for x in tg["sfb"]])
    outs = []
    for pad in (0, 2):
        sfa = bsg.pack_ue8m0_scales(tg["sfa"], ld_packed=Mt + pad)[:, :Mt]
        D = torch.zeros(Mt, 256, dtype=torch.bfloat16, device=DEV)
        bsg.m_grouped_gemm_fp8(tg["A"], sfa, tg["B"], sfbg, tg["offsets"], out=D)
        outs.append(gpu_bits(D))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])


def test_bf16_largest_row_stride():
    """Row strides at the library's limit (256 rows of offsets inside 31 bits):
    lda = ldb = 4194296 bf16 elements (8 MiB rows, 2 GiB per operand), only the
    first K of each row used."""
    _say("bf16 largest row stride (2 GiB operands)")
    M, N, K, ld = 256, 256, 1024, 4194296
    w = workloads.dense("bf16", M, N, K, 91, device="cpu")
    Ab = torch.empty(M, ld, dtype=torch.bfloat16, device=DEV)
    Bb = torch.empty(N, ld, dtype=torch.bfloat16, device=DEV)
    Ab[:, :K] = w.tensors["A"].to(DEV)
    Bb[:, :K] = w.tensors["B"].to(DEV)
    Ab[:, K:K + 64] = float("nan")          # must never be read
    Bb[:, K:K + 64] = float("nan")
    D = bsg.gemm_bf16(Ab[:, :K], Bb[:, :K])
    torch.cuda.synchronize()
    del Ab, Bb
    torch.cuda.empty_cache()
    ref, na, nb = run_oracle("bf16", host(w.tensors), K)
    assert_parity(gpu_bits(D), ref, na, nb, what="bf16 256x256x1024, lda = ldb = 4194296")


@pytest.mark.parametrize("kind", ["fp8", "fp4"])
def test_long_k(kind):
    """K = 131072 (1024 FP8 K-blocks, 4096 FP4 K-blocks): long scale arrays and
    offsets far into each row."""
    _say(f"{kind} 64x96x131072")
    M, N, K = 64, 96, 131072
    dense_full(kind, M, N, K, 92)
