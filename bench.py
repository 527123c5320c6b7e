"""Benchmark of the block-scaled GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--dtypes bf16,fp8,fp4,grouped,grouped_bf16,grouped_fp4,quant_fp8,
                              quant_fp4,quant_fp8_moe,moe_ffn,masked,mqa_prefill_fp8,
                              mqa_prefill_fp4,mqa_decode_fp8,mqa_decode_fp4]

Workload: D = A * B^T at M=4096, N=7168, K=16384, the dense shape the pages time
(431 TFLOPS BF16 on the other accelerator: "DeepSeek lanza kernels de DeepGEMM
para Huawei Ascend 950", section "Que alcance tienen las pruebas de
rendimiento"), in BF16, in FP8 e4m3 with 1x128 / 128x128 UE8M0 scales and in FP4
e2m1 with 1x32 scales, plus the M-grouped MoE GEMM (256 experts, N=2048,
K=7168, 16384 tokens routed top-6 with Zipf(1.1) popularity) in FP8, BF16 and FP4.  All inputs are
seeded synthetic data generated straight into HBM before timing starts.

One JSON line is printed.  `value` is the BF16 GEMM's throughput in TFLOPS
(2*M*N*K per call, the pages' convention) at the median of exactly `--steps`
timed calls, each preceded by a 512 MiB scratch write on the same stream (more
than the 256 MB MALL plus every XCD's 4 MB L2: the cold-L2 protocol of the
pages' own benchmark) and bracketed by HIP events on the stream it is launched
on; `ms_per_step` is that median.  The same calls back to back give the warm
rate beside it (`warm`).  Every other case is timed the same way in the same run
and reported under `per_dtype` with its fraction of the dtype's dense MFMA peak;
the mean event-timed launch of the cold calls is the duration behind each
`roofline`.  Before the timed calls, the warm-up calls are followed by 0.2 s of
untimed calls: under sustained load the clocks take tens of milliseconds to
settle.  A third loop, with the scratch write followed by a 512 MiB read, gives
`cold_clean`: caches just as cold, without the scratch's dirty lines being
written back during the call.  `vs_baseline` is null: the pages' 431 TFLOPS at this shape was
measured on another accelerator and is reported under `context`.

The per-token quantisers (bf16 activations -> FP8 1x128 or FP4 1x32 codes with
packed UE8M0 scales) are timed the same way on the dense shape's A (4096x16384)
and on the MoE tokens (16384x7168), reported in GB/s of algorithmic traffic
against the 8 TB/s HBM peak.

The MoE FFN core (grouped up-projection with SwiGLU + FP8 requantisation in its
epilogue, grouped down-projection) runs on one GPU's share of the pages' fused MoE case: 48 of 384
experts (EP8) plus the shared expert, 16384 tokens top-6, hidden 7168,
intermediate 2048; TFLOPS count useful (unpadded) rows.

The masked M-grouped FP8 GEMM runs a decode-sized case: 48 local experts of
384, capacity 512 rows, N=4096, K=7168, counts from 4096 tokens top-6; it is
bound by reading the experts' weights, so GB/s is reported beside TFLOPS.

The MQA logits kernels (64 heads of 128, FP8 and FP4) run a prefill of one
4096-token sequence with causal windows (its roofline: the vector ALU's max and
multiply-add per window pair and head; TFLOPS of the scores' dot products beside
it) and a decode of 128 requests over 32768-token contexts (GB/s against HBM:
each request streams its own keys).

`cpu_baseline` times the CPU oracle (plain C, fp64, every host thread) on a
bounded row sample of the BF16 case's own inputs; `per_config` adds the FP8, FP4
and grouped FP8 cases, and `host` the core count and CPU model.  The oracle's
rows are also compared with the GPU output of the timed calls (`parity`).

`--operands zeros` runs the dense cases on all-zero codes instead of the random
draws: the same instruction stream at a lower power draw, an experiment on the
clock, never the benchmark.

`mfma_only` (and each dense case's `per_dtype[...]["mfma_only"]`) is the rate the
matrix cores sustain when every SIMD runs nothing but MFMAs on random operands, in
the GEMM kernels' register tile and occupancy (libbsg_probe.so, include/bsg_probe.h):
under sustained load the chip runs at the clock its power limit allows for the
data, below the clock the published peaks assume, and `gemm_warm_frac` is the
GEMM's warm rate against that ceiling.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOPS and % of MI355X dense MFMA peak, GEMM 4096×7168×16384 per dtype"

# MI355X published dense MFMA peaks (TFLOP/s).
PEAK = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 10100.0, "grouped": 5000.0, "moe_ffn": 5000.0,
        "masked": 5000.0, "grouped_bf16": 2500.0, "grouped_fp4": 10100.0,
        "mqa_prefill_fp8": 5000.0, "mqa_prefill_fp4": 10100.0, "mqa_decode_fp8": 5000.0,
        "mqa_decode_fp4": 10100.0}
# Vector-ALU lane operations per second of the chip: 256 CUs x 4 SIMDs x 16 lanes x
# 2.4 GHz (one fp32 max or fused multiply-add per lane per clock; the packed
# two-wide fp32 forms, which the 157.3 TFLOP/s vector figure counts, are not used
# by this library).  Bound of the MQA prefill: per (query, window key) pair it
# takes one max and one fused multiply-add per head on the vector units.
ALU_PEAK_GOPS = 256 * 4 * 16 * 2.4
ALU_KINDS = ("mqa_prefill_fp8", "mqa_prefill_fp4")
# Cases bound by HBM (their weights or keys stream once): roofline in GB/s.
HBM_KINDS = ("masked", "mqa_decode_fp8", "mqa_decode_fp4")
MQA_KINDS = ("mqa_prefill_fp8", "mqa_prefill_fp4", "mqa_decode_fp8", "mqa_decode_fp4")
# MI355X published HBM3E bandwidth (GB/s): the bound of the quantisers.
HBM_PEAK_GBS = 8000.0
QUANT_KINDS = ("quant_fp8", "quant_fp4", "quant_fp8_moe")
# Operand values of the dense cases: "random" (the workloads' own draws, the
# benchmark) or "zeros" (an experiment on power: see --operands).
OPERANDS = "random"
# Cases whose inputs the CPU oracle is also timed on (cpu_baseline).
CPU_KINDS = ("bf16", "fp8", "fp4", "grouped")
# The pages' own figure at this shape (other accelerator; context only).
PAGES_BF16_TFLOPS = 431.0

KERNEL_NAME = {
    "bf16": "gemm_kernel<0, 256, 256, 2, 4, 64, 5, 1, false, 0, 8, 0>",
    "fp8": "gemm_kernel<1, 256, 256, 2, 4, 64, 5, 1, false, 1, 0, 0>",
    "fp4": "gemm_kernel<2, 256, 256, 2, 4, 64, 5, 1, false, 1, 2, 0>",
    "grouped": "gemm_kernel<1, 256, 256, 2, 4, 64, 5, 1, true, 1, 8, 0>",
    "quant_fp8": "quant_kernel<0, 0, 32, 2, 0>",
    "quant_fp4": "quant_kernel<1, 0, 32, 2, 0>",
    "quant_fp8_moe": "quant_kernel<0, 0, 32, 2, 0>",
    "moe_ffn": "gemm_kernel<1, 256, 256, 2, 4, 64, 5, 1, true, 1, 8, 1> (up, SwiGLU epilogue) + gemm_kernel<1, 256, 256, 2, 4, 64, 5, 1, true, 1, 8, 0> (down)",
    "masked": "gemm_kernel<1, 128, 256, 1, 4, 64, 6, 1, true, 1, 0, 0>",
    "grouped_bf16": "gemm_kernel<0, 256, 256, 2, 4, 64, 5, 1, true, 0, 6, 0>",
    "grouped_fp4": "gemm_kernel<2, 256, 256, 2, 4, 64, 5, 1, true, 1, 4, 0>",
    "mqa_prefill_fp8": "mqa_logits_kernel<0, 2, true>",
    "mqa_prefill_fp4": "mqa_logits_kernel<4, 2, true>",
    "mqa_decode_fp8": "mqa_logits_kernel<0, 2, false>",
    "mqa_decode_fp4": "mqa_logits_kernel<4, 2, false>",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Kernel sources behind each measured kind: a change to any of them detaches the
# committed rocprofv3 counters from the kernel.
SOURCES = {
    "gemm": ("gemm_kernel.h", "configs.h", "quant_math.h"),
    "quant": ("quant.hip", "quant_math.h"),
    "mqa": ("mqa.hip",),
}


def kernel_sources_sha(group: str = "gemm") -> str:
    """Hash of one group's kernel sources with comments and blank space removed,
    so that counters stay attached to the code they were taken on across comment
    edits."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_precision_05_amd", "csrc")
    for name in SOURCES[group]:
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = " ".join(text.split())
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


def load_traffic(kind: str, sha: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(kind)
    if not ent or ent.get("src_sha") != sha:
        return None
    return ent.get("bytes_per_launch")


def make_case(kind, dev):
    """Returns (call, flops, min_bytes, meta) with every input resident on `dev`."""
    import torch
    import block_scaled_precision_05_amd as bsg
    from block_scaled_precision_05_amd import workloads

    name = {"bf16": "bf16_large", "fp8": "fp8_large", "fp4": "fp4_large",
            "grouped": "moe_fp8", "quant_fp8": "act_large", "quant_fp4": "act_large",
            "quant_fp8_moe": "act_moe", "moe_ffn": "moe_ffn", "masked": "masked_fp8",
            "grouped_bf16": "moe_bf16", "grouped_fp4": "moe_fp4"}.get(kind, kind)
    w = workloads.make(name, device=dev)
    t = w.tensors
    M, N, K = w.M, w.N, w.K
    if OPERANDS == "zeros" and kind in ("bf16", "fp8", "fp4"):
        # the same instruction stream on all-zero codes (scales unchanged): what the
        # operand values cost in power, hence in clock
        t["A"].zero_()
        t["B"].zero_()
    if kind in QUANT_KINDS:
        X = t["X"]
        fp4 = kind == "quant_fp4"
        gk = 32 if fp4 else 128
        Q = torch.empty(M, K // 2 if fp4 else K, dtype=torch.uint8, device=dev)
        S = torch.empty((K // gk + 1) // 2, M, dtype=torch.int16, device=dev)
        # The kernel runs for tens of microseconds, about as long as the Python
        # binding's checks: time the C entry point itself (checked once through
        # the binding first), so that the CPU stays ahead of the GPU.
        fn = bsg.quantize_fp4_per_token if fp4 else bsg.quantize_fp8_per_token
        fn(X, rule="ceil", out=Q, sf_out=S)
        entry = getattr(bsg.lib(), "quantize_fp4_per_token" if fp4 else "quantize_fp8_per_token")
        args = (X.data_ptr(), X.stride(0), Q.data_ptr(), Q.stride(0), S.data_ptr(), S.stride(0),
                M, K, bsg.SCALE_RULES["ceil"], torch.cuda.current_stream().cuda_stream)
        held = (X, Q, S)   # the raw pointers above stay valid while the call lives

        def call(held=held):
            st = entry(*args)
            if st:
                raise RuntimeError(f"quantiser failed: {bsg.status_string(st)}")
        nbytes = 2 * M * K + Q.numel() + 2 * S.numel()
        meta = {"scales": f"1x{gk} UE8M0, rule ceil, packed int16 MN-major",
                "bytes_per_call": nbytes}
        meta.update({"M": M, "K": K})
        return call, 0.0, nbytes, meta, None
    if kind in MQA_KINDS:
        fmt = kind.rsplit("_", 1)[1]
        m = w.meta
        T, S, H = t["W"].shape[0], m["S"], m["H"]
        sfq = bsg.ensure_packed(t["sfq"], t["sfq"].shape[0], t["sfq"].shape[1])
        sfk = bsg.ensure_packed(t["sfk"], t["sfk"].shape[0], t["sfk"].shape[1])
        L = torch.empty(T, S, dtype=torch.float32, device=dev)
        # checked once through the binding, then timed at the C entry point (the
        # decode kernel runs for tens of microseconds)
        bsg.mqa_logits(fmt, t["Q"], sfq, t["K"], sfk, t["W"], t["ks"], t["ke"], S,
                       q_per_group=m["q_per_group"], group_rows=m["group_rows"], out=L)
        entry = getattr(bsg.lib(), "mqa_logits_" + fmt)
        Qb, Kb = t["Q"].view(torch.uint8), t["K"].view(torch.uint8)
        cargs = (Qb.data_ptr(), Qb.stride(0), sfq.data_ptr(), sfq.stride(0), Kb.data_ptr(),
                 Kb.stride(0), sfk.data_ptr(), sfk.stride(0), t["W"].data_ptr(), t["W"].stride(0),
                 t["ks"].data_ptr(), t["ke"].data_ptr(), L.data_ptr(), L.stride(0), T, S, H,
                 m["q_per_group"], m["group_rows"], torch.cuda.current_stream().cuda_stream)
        held = (Qb, Kb, sfq, sfk, t["W"], t["ks"], t["ke"], L)   # owners of the raw pointers

        def call(held=held):
            st = entry(*cargs)
            if st:
                raise RuntimeError(f"mqa_logits_{fmt} failed: {bsg.status_string(st)}")
        row = t["Q"].shape[1]
        # queries, their weights and all logits once; keys once per group for
        # prefill (one sequence, shared by every query), once per window key for
        # decode (each request reads its own context)
        keys = S if m["mode"] == "prefill" else m["valid_pairs"]
        nbytes = (T * H * row + 2 * sfq.numel() + 4 * T * H + 4 * T * S
                  + keys * (row + 2 * sfk.shape[0]))
        meta = {"mode": m["mode"], "queries": T, "keys": S, "heads": H, "head_dim": m["D"],
                "windows": m["windows"], "window_pairs": m["valid_pairs"], "bytes_per_call": nbytes,
                "flops_note": "2*H*D per (query, window key): the scores' dot products; the "
                              "weighted max-sum adds 2*H more on the vector units"}
        return call, w.flops, nbytes, meta, None
    if kind in ("grouped_bf16", "grouped_fp4"):
        A, B, off = t["A"], t["B"], t["offsets"]
        G = B.shape[0]
        D = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        if kind == "grouped_bf16":
            call = lambda: bsg.m_grouped_gemm_bf16(A, B, off, out=D)
            nbytes = 2 * (A.numel() + B.numel()) + 2 * M * N
        else:
            sfa = bsg.ensure_packed(t["sfa"], M, K // 32)
            sfb = torch.stack([bsg.ensure_packed(x, N, K // 32) for x in t["sfb"]])
            call = lambda: bsg.m_grouped_gemm_fp4(A, sfa, B, sfb, off, K=K, out=D)
            nbytes = A.numel() + B.numel() + 2 * M * N + 2 * (sfa.numel() + sfb.numel())
        meta = {"experts": G, "m_total": M, "useful_rows": w.meta["useful_rows"],
                "routing": w.meta["routing"], "executed_tflop": 2.0 * M * N * K / 1e12}
        meta.update({"M": M, "N": N, "K": K})
        return call, w.flops, nbytes, meta, None
    if kind == "masked":
        A, B, m = t["A"], t["B"], t["masked_m"]
        G, cap, _ = A.shape
        sfa = bsg.ensure_packed(t["sfa"], G * cap, K // 128)
        sfb = torch.stack([bsg.ensure_packed(x, (N + 127) // 128, K // 128) for x in t["sfb"]])
        D = torch.empty(G, cap, N, dtype=torch.bfloat16, device=dev)
        call = lambda: bsg.m_grouped_gemm_fp8_masked(A, sfa, B, sfb, m, out=D)
        useful = w.meta["useful_rows"]
        nbytes = B.numel() + useful * K + 2 * useful * N + 2 * sfb.numel()
        meta = {"experts": G, "capacity": cap, "useful_rows": useful, "routing": w.meta["routing"],
                "bytes_per_call": nbytes,
                "note": "decode-sized: the weights dominate, so HBM bounds it (see gb_per_s)"}
        meta.update({"M": G * cap, "N": N, "K": K})
        return call, w.flops, nbytes, meta, None
    if kind == "moe_ffn":
        G, two_i, hidden = t["W13"].shape
        inter = two_i // 2
        sfa = bsg.ensure_packed(t["sfa"], M, hidden // 128)
        sfw13 = torch.stack([bsg.ensure_packed(x, (two_i + 127) // 128, hidden // 128)
                             for x in t["sfw13"]])
        sfw2 = torch.stack([bsg.ensure_packed(x, (hidden + 127) // 128, inter // 128)
                            for x in t["sfw2"]])
        ws = (torch.empty(M, inter, dtype=torch.uint8, device=dev),
              torch.empty((inter // 128 + 1) // 2, M, dtype=torch.int16, device=dev))
        D = torch.empty(M, hidden, dtype=torch.bfloat16, device=dev)
        A, W13, W2, off = t["A"], t["W13"], t["W2"], t["offsets"]
        call = lambda: bsg.moe_ffn_fp8(A, sfa, W13, sfw13, W2, sfw2, off, out=D, workspace=ws)
        # tokens, both weight sets and D, plus Y written by the up-projection and
        # read back by the down-projection (H is never formed)
        nbytes = (A.numel() + W13.numel() + W2.numel() + 2 * M * hidden + M * inter * 2)
        meta = {"experts": G, "hidden": hidden, "inter": inter, "m_total": M,
                "useful_rows": w.meta["useful_rows"], "routing": w.meta["routing"],
                "executed_tflop": 2.0 * M * (two_i * hidden + hidden * inter) / 1e12,
                "steps": "grouped up-projection, SwiGLU + FP8 1x128 requantisation, "
                         "grouped down-projection"}
        meta.update({"M": M, "N": hidden, "K": hidden})
        return call, w.flops, nbytes, meta, None
    if kind == "bf16":
        A, B = t["A"], t["B"]
        D = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        call = lambda: bsg.gemm_bf16(A, B, out=D)
        nbytes = 2 * (M * K + N * K + M * N)
        meta = {}
    elif kind == "fp8":
        A, B, sfa_u8, sfb_u8 = t["A"], t["B"], t["sfa"], t["sfb"]
        D = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        sfa = bsg.ensure_packed(sfa_u8, M, K // 128)
        sfb = bsg.ensure_packed(sfb_u8, (N + 127) // 128, K // 128)

        def call():
            # reuse-or-convert on every call, as the pages' scale helper does
            a = bsg.ensure_packed(sfa, M, K // 128)
            b = bsg.ensure_packed(sfb, (N + 127) // 128, K // 128)
            return bsg.gemm_fp8_blockscaled(A, a, B, b, out=D)
        nbytes = M * K + N * K + 2 * M * N + 2 * (sfa.numel() + sfb.numel())
        meta = {"scales": "sfa 1x128, sfb 128x128, UE8M0 e~U{-8..4}, packed int16 MN-major"}
    elif kind == "fp4":
        A, B, sfa_u8, sfb_u8 = t["A"], t["B"], t["sfa"], t["sfb"]
        D = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        sfa = bsg.ensure_packed(sfa_u8, M, K // 32)
        sfb = bsg.ensure_packed(sfb_u8, N, K // 32)

        def call():
            a = bsg.ensure_packed(sfa, M, K // 32)
            b = bsg.ensure_packed(sfb, N, K // 32)
            return bsg.gemm_fp4_blockscaled(A, a, B, b, K=K, out=D)
        nbytes = (M * K + N * K) // 2 + 2 * M * N + 2 * (sfa.numel() + sfb.numel())
        meta = {"scales": "1x32 UE8M0, OCP MX rule floor(log2 amax)-2"}
    else:
        A, sfa_u8, B, sfb_u8, off = t["A"], t["sfa"], t["B"], t["sfb"], t["offsets"]
        G = B.shape[0]
        D = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        sfa = bsg.ensure_packed(sfa_u8, M, K // 128)
        sfb = torch.stack([bsg.ensure_packed(s, (N + 127) // 128, K // 128) for s in sfb_u8])
        call = lambda: bsg.m_grouped_gemm_fp8(A, sfa, B, sfb, off, out=D)
        nbytes = M * K + B.numel() + 2 * M * N + 2 * (sfa.numel() + sfb.numel())
        meta = {"experts": G, "m_total": M, "useful_rows": w.meta["useful_rows"],
                "routing": w.meta["routing"],
                "executed_tflop": 2.0 * M * N * K / 1e12}
    flops = w.flops
    meta.update({"M": M, "N": N, "K": K})
    return call, flops, nbytes, meta, lambda budget: cpu_sample(kind, w, budget, D)


def cpu_sample(kind, w, budget_s, D=None):
    """The CPU oracle (plain C, fp64, all host threads) on leading rows of the case's
    own inputs, copied to host memory: the dense shapes' first rows x all N columns;
    for the grouped GEMM the first rows of its largest expert x all N columns.  With
    the GPU's output D of the same inputs (after the timed calls), the rows the oracle
    computed, and the last 128x128 tile of the dense shapes, are also compared with
    it: the normalised error |D - bf16(oracle)| / (|a_i| |b_j|) against 1e-3."""
    import numpy as np
    import torch
    import oracle
    t = w.tensors
    M, N, K = w.M, w.N, w.K

    def u8(x):
        return x.contiguous().view(torch.uint8).cpu().numpy()

    r0 = 0
    if kind == "bf16":
        B = t["B"].view(torch.int16).cpu().numpy().view(np.uint16)
        A = t["A"].view(torch.int16).cpu().numpy().view(np.uint16)
        fn = lambda rows, cols=None: oracle.gemm_bf16(A, B, rows=rows, cols=cols)
        norms = lambda rows, cols: (oracle.row_norms("bf16", A, rows=rows),
                                    oracle.row_norms("bf16", B, rows=cols))
        n_rows, what = M, f"BF16 {M}x{N}x{K}"
    elif kind == "fp8":
        A, B = u8(t["A"]), u8(t["B"])
        sfa, sfb = oracle.pack_scales(u8(t["sfa"])), oracle.pack_scales(u8(t["sfb"]))
        fn = lambda rows, cols=None: oracle.gemm_fp8(A, sfa, B, sfb, rows=rows, cols=cols)
        norms = lambda rows, cols: (oracle.row_norms("e4m3", A, sfa, rows=rows),
                                    oracle.row_norms("e4m3", B, sfb, rows=cols, gran_mn=128))
        n_rows, what = M, f"FP8 {M}x{N}x{K}"
    elif kind == "fp4":
        A, B = u8(t["A"]), u8(t["B"])
        sfa, sfb = oracle.pack_scales(u8(t["sfa"])), oracle.pack_scales(u8(t["sfb"]))
        fn = lambda rows, cols=None: oracle.gemm_fp4(A, sfa, B, sfb, K, rows=rows, cols=cols)
        norms = lambda rows, cols: (oracle.row_norms("e2m1", A, sfa, K=K, rows=rows),
                                    oracle.row_norms("e2m1", B, sfb, K=K, rows=cols))
        n_rows, what = M, f"FP4 {M}x{N}x{K}"
    else:
        counts = t["counts"].cpu().numpy()
        off = t["offsets"].cpu().numpy()
        g = int(np.argmax(counts))
        r0, n_rows = int(off[g]), int(counts[g])
        A = u8(t["A"][r0:r0 + n_rows])
        sfa = oracle.pack_scales(u8(t["sfa"][r0:r0 + n_rows]))
        Bg, sfbg = u8(t["B"][g:g + 1]), np.stack([oracle.pack_scales(u8(t["sfb"][g]))])
        one = np.array([0, n_rows], dtype=np.int32)
        fn = lambda rows, cols=None: oracle.grouped_fp8(A, sfa, Bg, sfbg, one, rows=rows, cols=cols)
        norms = lambda rows, cols: (oracle.row_norms("e4m3", A, sfa, rows=rows),
                                    oracle.row_norms("e4m3", Bg[0], sfbg[0], rows=cols, gran_mn=128))
        what = f"M-grouped FP8, expert {g} ({n_rows} rows) of {w.meta['G']}, N={N}, K={K}"
    kept = []

    def timed_fn(rows):
        kept.append((rows, fn(rows)))
    out = oracle_rows(timed_fn, n_rows, 2.0 * N * K, budget_s, what)
    if D is not None:
        out["parity"] = _sample_parity(D, kept, fn, norms, r0, n_rows, N, kind != "grouped")
    return out


def _sample_parity(D, kept, fn, norms, r0, n_rows, N, corner):
    """Normalised error of the GPU output against the oracle rows already computed
    (and, for the dense shapes, the last 128x128 tile)."""
    import numpy as np
    import oracle
    import torch
    Dh = D.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    blocks = [(rows, None, vals) for rows, vals in kept]
    if corner:
        rows = np.arange(max(0, n_rows - 128), n_rows)
        cols = np.arange(max(0, N - 128), N)
        blocks.append((rows, cols, fn(rows, cols)))
    worst, n_over, n_out = 0.0, 0, 0
    for rows, cols, vals in blocks:
        cols_i = np.arange(N) if cols is None else cols
        na, nb = norms(rows, cols_i)
        got = Dh[np.ix_(r0 + np.asarray(rows), cols_i)]
        got = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        want = (oracle.bf16_rne(vals).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        den = na[:, None] * nb[None, :]
        err = np.abs(got - want) / np.where(den > 0, den, 1.0)
        err = np.where(den > 0, err, np.where(got == want, 0.0, np.inf))
        worst = max(worst, float(err.max()) if err.size else 0.0)
        n_over += int((err > 1e-3).sum())
        n_out += err.size
    return {"outputs": n_out, "max_normalised_error": worst, "over_1e-3": n_over,
            "tolerance": 1e-3, "what": "the oracle's sampled rows x all columns" +
            (", and the last 128x128 tile" if corner else "")}


def _stats(us):
    us = sorted(us)
    return {"us_median": statistics.median(us), "us_mean": statistics.fmean(us), "us_min": us[0],
            "us_p90": us[min(len(us) - 1, int(0.9 * len(us)))]}


def time_case(kind, steps, warmup, dev, cpu_budget=0.0, settle_s=0.2):
    """Warm-up: `warmup` calls, then untimed calls for `settle_s` seconds (under
    sustained load the chip's clocks take tens of milliseconds to settle; timed
    right after a short warm-up, the first loop reads 5-12% slow).  Then the timed
    region: exactly `steps` calls, each preceded on the same stream by a 512 MiB
    scratch write (more than the 256 MB MALL plus the eight 4 MB L2s), each
    bracketed by HIP events on that stream, with device synchronisation before and
    after the region.  Two more loops of `steps` calls give the warm rate (back to
    back) and a clean cold rate (the scratch write followed by a 512 MiB read, so
    no dirty line of the scratch is left to write back during the call).  With
    `cpu_budget` > 0 the oracle is then timed on a sample of the same inputs."""
    import torch
    call, flops, nbytes, meta, cpu_sample = make_case(kind, dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    settle = 0
    while time.perf_counter() - t0 < settle_s:
        for _ in range(4):
            call()
        settle += 4
        torch.cuda.synchronize()
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    rscratch = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def timed(mode):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s, e in ev:
            if mode != "warm":
                scratch.fill_(1)
            if mode == "clean":
                torch.sum(rscratch, dim=(0,), out=sink)
            s.record(stream)
            call()
            e.record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, [s.elapsed_time(e) * 1e3 for s, e in ev]

    wall_cold, cold = timed("cold")
    wall_warm, warm = timed("warm")
    _, clean = timed("clean")
    del scratch, rscratch
    res = {"per_launch_us": cold, "wall_s": wall_cold, "warm_us": warm, "warm_wall_s": wall_warm,
           "clean_us": clean, "settle_calls": settle, "flops": flops, "min_bytes": nbytes,
           "meta": meta}
    if cpu_budget > 0 and cpu_sample is not None:
        log(f"{kind}: oracle on a sample of the same inputs for ~{cpu_budget:.0f} s")
        res["cpu"] = cpu_sample(cpu_budget)
    return res


# rounds of MFMAs per probe call: about half a millisecond each at the rates measured
PROBE_ITERS = {"bf16": 800, "fp8": 400, "fp4": 800}
PROBE_SEED = 20240607


def mfma_only(kind, dev, calls=20, settle_s=0.2):
    """The rate the matrix cores sustain on MFMAs alone (libbsg_probe.so): the GEMM
    kernels' register tile and occupancy (one workgroup of eight waves per CU), random
    operand codes and UE8M0 scales, no memory traffic.  Calls back to back after a
    settle phase like the GEMMs' warm loop, each bracketed by HIP events on the launch
    stream; the median.  Under sustained load the chip holds the clock its power limit
    allows for the data, so this is the ceiling the GEMMs' warm rates compare with,
    beside the published peak."""
    import torch
    from block_scaled_precision_05_amd import probe
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    iters = PROBE_ITERS[kind]
    out = torch.empty(cus * probe.THREADS, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call():
        probe.mfma(kind, PROBE_SEED, cus, iters, out, stream)

    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(4):
            call()
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for s, e in ev:
        s.record(stream)
        call()
        e.record(stream)
    torch.cuda.synchronize()
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("mfma probe: non-finite accumulator sums")
    us = statistics.median(s.elapsed_time(e) * 1e3 for s, e in ev)
    tflops = probe.flops_per_call(kind, cus, iters) / (us * 1e-6) / 1e12
    return {"tflops": tflops, "frac_of_peak": tflops / PEAK[kind], "us_median": us,
            "calls": calls, "workgroups": cus, "rounds": iters,
            "kernel": f"mfma_probe_kernel<{probe.KINDS[kind]}>",
            "what": "MFMAs alone in the GEMM's register tile and occupancy, random codes and "
                    "scales, back to back"}


def summarize(kind, r, steps):
    """Per-case record.  The headline figures are the cold-L2 samples (the timed
    region); `warm` holds the back-to-back rate of the same calls."""
    cold = _stats(r["per_launch_us"])
    med, mean_us = cold["us_median"], cold["us_mean"]
    warm = _stats(r["warm_us"]) if r.get("warm_us") else None
    clean = statistics.median(r["clean_us"]) if r.get("clean_us") else None
    cold["settle_calls"] = r.get("settle_calls", 0)
    if kind in QUANT_KINDS:
        gbs = r["min_bytes"] / (med * 1e-6) / 1e9
        out = {
            "gb_per_s": gbs,
            "us_per_call": med,
            "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
            "hbm_peak_gb_per_s": HBM_PEAK_GBS,
            "cold_l2": dict(cold, wall_us_per_call=r["wall_s"] * 1e6 / steps),
            "kernel": KERNEL_NAME[kind],
        }
        if warm:
            out["warm"] = dict(warm, gb_per_s=r["min_bytes"] / (warm["us_median"] * 1e-6) / 1e9,
                               wall_us_per_call=r["warm_wall_s"] * 1e6 / steps)
        if clean:
            out["cold_clean"] = {"us_median": clean,
                                 "gb_per_s": r["min_bytes"] / (clean * 1e-6) / 1e9,
                                 "flush": "512 MiB write then 512 MiB read"}
        achieved = r["min_bytes"] / (mean_us * 1e-6) / 1e9
        out["roofline"] = {"kernel": KERNEL_NAME[kind], "bound": "hbm", "achieved": achieved,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                           "traffic": load_traffic(kind, kernel_sources_sha("quant")),
                           "src_sha": kernel_sources_sha("quant")}
        out.update(r["meta"])
        return out
    tflops = r["flops"] / (med * 1e-6) / 1e12
    out = {
        "tflops": tflops,
        "ms_per_call": med / 1e3,
        "frac_of_peak": tflops / PEAK[kind],
        "peak_tflops": PEAK[kind],
        "cold_l2": dict(cold, wall_ms_per_call=r["wall_s"] * 1e3 / steps),
        "tflop_per_call": r["flops"] / 1e12,
        "min_hbm_mb": r["min_bytes"] / 1e6,
    }
    if warm:
        out["warm"] = dict(warm, tflops=r["flops"] / (warm["us_median"] * 1e-6) / 1e12,
                           frac_of_peak=r["flops"] / (warm["us_median"] * 1e-6) / 1e12 / PEAK[kind],
                           wall_ms_per_call=r["warm_wall_s"] * 1e3 / steps)
    if clean:
        out["cold_clean"] = {"us_median": clean, "tflops": r["flops"] / (clean * 1e-6) / 1e12,
                             "flush": "512 MiB write then 512 MiB read"}
    if kind in HBM_KINDS:
        out["gb_per_s"] = r["min_bytes"] / (med * 1e-6) / 1e9
        out["frac_of_hbm_peak"] = out["gb_per_s"] / HBM_PEAK_GBS
    # per-launch roofline of the case's GEMM kernel over the timed region (the FFN
    # core: its two kernels together, against the FP8 peak)
    sha = kernel_sources_sha("mqa" if kind in MQA_KINDS else "gemm")
    if kind in HBM_KINDS:
        ach = r["min_bytes"] / (mean_us * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    elif kind in ALU_KINDS:
        ops = 2.0 * r["meta"]["window_pairs"] * r["meta"]["heads"]
        ach = ops / (mean_us * 1e-6) / 1e9
        out["roofline"] = {"bound": "alu", "achieved": ach, "peak": ALU_PEAK_GOPS,
                           "unit": "Gop/s (vector lane operations)",
                           "mfma_frac": r["flops"] / (mean_us * 1e-6) / 1e12 / PEAK[kind]}
    else:
        # The bound is whichever takes longer at peak: the flops on the matrix cores or
        # the algorithmic bytes through HBM.  The dense GEMMs are far on the flop side;
        # the MoE-shaped grouped GEMMs sit just past the ridge on the byte side (most
        # experts own one or two row tiles, so each weight byte meets few rows), and
        # report the other fraction beside it.
        ach = r["flops"] / (mean_us * 1e-6) / 1e12
        ach_b = r["min_bytes"] / (mean_us * 1e-6) / 1e9
        t_flops = r["flops"] / (PEAK[kind] * 1e12)
        t_bytes = r["min_bytes"] / (HBM_PEAK_GBS * 1e9)
        if t_bytes > t_flops:
            out["roofline"] = {"bound": "hbm", "achieved": ach_b, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "mfma_frac": ach / PEAK[kind]}
            ach = ach_b
        else:
            out["roofline"] = {"bound": "mfma", "achieved": ach, "peak": PEAK[kind], "unit": "TFLOP/s",
                               "hbm_frac": ach_b / HBM_PEAK_GBS}
    if kind == "moe_ffn":
        # the call's two kernels: the up-projection (with its SwiGLU epilogue) and the
        # down-projection
        parts = [load_traffic(k, sha) for k in ("moe_ffn_up", "moe_ffn_down")]
        traffic = None if None in parts else sum(parts)
    else:
        traffic = load_traffic(kind, sha)
    out["roofline"].update(kernel=KERNEL_NAME[kind], frac=ach / out["roofline"]["peak"],
                           traffic=traffic, src_sha=sha)
    if "cpu" in r:
        out["cpu_oracle"] = r["cpu"]
        out["cpu_oracle"]["gpu_over_cpu"] = tflops / r["cpu"]["value"]
    out.update(r["meta"])
    return out


def host_info():
    """Host cores and CPU model of the machine the oracle ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def oracle_rows(fn, n_rows, flops_per_row, budget_s, what):
    """Runs the oracle call fn(rows) on successive chunks of rows until about
    `budget_s` seconds are spent: a probe chunk, a second chunk four times as large
    (the two separate a call's fixed cost, the decode of B, from its cost per row),
    then one chunk sized to the rest of the budget.  Returns the oracle's rate over
    all rows and time, in TFLOPS."""
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    done, calls, times = 0, 0, []
    for size in (16, 64):
        size = min(size, n_rows - done)
        if size <= 0:
            break
        t = time.perf_counter()
        fn(np.arange(done, done + size))
        times.append((size, time.perf_counter() - t))
        done += size
        calls += 1
    if len(times) == 2 and n_rows > done:
        (n1, d1), (n2, d2) = times
        per_row = max((d2 - d1) / (n2 - n1), 1e-9) if d2 > d1 else d2 / n2
        fixed = max(d1 - n1 * per_row, 0.0)
        left = budget_s - (time.perf_counter() - t0) - fixed
        more = int(min(n_rows - done, max(0.0, left) / per_row))
        if more > 0:
            fn(np.arange(done, done + more))
            done += more
            calls += 1
    dt = time.perf_counter() - t0
    return {"value": done * flops_per_row / dt / 1e12, "unit": "TFLOPS",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{what}: rows 0..{done - 1} x all columns ({done} of {n_rows} rows, "
                      f"{dt:.1f} s, {calls} calls)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--dtypes",
                    default="bf16,fp8,fp4,grouped,grouped_bf16,grouped_fp4,quant_fp8,quant_fp4,"
                            "quant_fp8_moe,moe_ffn,masked,mqa_prefill_fp8,mqa_prefill_fp4,"
                            "mqa_decode_fp8,mqa_decode_fp4")
    ap.add_argument("--cpu-budget", type=float, default=24.0,
                    help="seconds of oracle time for cpu_baseline, shared by the BF16, FP8, FP4 "
                         "and grouped cases (0 disables it)")
    ap.add_argument("--operands", choices=("random", "zeros"), default="random",
                    help="operand codes of the dense BF16/FP8/FP4 cases: the workloads' random "
                         "draws (the benchmark), or all zeros, an experiment that runs the same "
                         "instruction stream at a lower power draw")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 512 MiB device copy three times (the reference "
                         "dispatch that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_precision_05_amd as bsg
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bsg.lib()   # fails loudly if the HIP library is missing
    global OPERANDS
    OPERANDS = args.operands
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    kinds = [k.strip() for k in args.dtypes.split(",") if k.strip()]
    if "bf16" not in kinds:
        kinds = ["bf16"] + kinds
    sha = kernel_sources_sha()
    cpu_kinds = [k for k in kinds if k in CPU_KINDS]

    per = {}
    for kind in kinds:
        log(f"{kind}: generating inputs and timing {args.warmup}+{args.steps} calls (cold L2), "
            f"then {args.steps} back to back")
        budget = args.cpu_budget / len(cpu_kinds) if kind in cpu_kinds else 0.0
        r = time_case(kind, args.steps, args.warmup, dev, budget)
        per[kind] = summarize(kind, r, args.steps)
        q = per[kind]
        if kind in QUANT_KINDS:
            log(f"{kind}: {q['gb_per_s']:.0f} GB/s ({100 * q['frac_of_hbm_peak']:.1f}% of HBM "
                f"peak) cold, {q['cold_l2']['us_mean']:.1f} us mean launch")
        else:
            log(f"{kind}: {q['tflops']:.1f} TFLOPS ({100 * q['frac_of_peak']:.1f}% of peak) cold, "
                f"{q['warm']['tflops']:.1f} warm, {q['cold_l2']['us_mean']:.1f} us mean launch")
        torch.cuda.empty_cache()

    # the matrix cores' sustained rate on MFMAs alone, for the dense cases' warm rates
    for kind in [k for k in ("bf16", "fp8", "fp4") if k in kinds]:
        m = mfma_only(kind, dev)
        m["gemm_warm_frac"] = per[kind]["warm"]["tflops"] / m["tflops"]
        per[kind]["mfma_only"] = m
        log(f"{kind}: MFMAs alone {m['tflops']:.1f} TFLOPS ({100 * m['frac_of_peak']:.1f}% of "
            f"peak); the GEMM's warm rate is {100 * m['gemm_warm_frac']:.1f}% of it")

    b = per["bf16"]
    roof = dict(b["roofline"])
    roof["traffic"] = load_traffic("bf16", sha)

    cpu = None
    if cpu_kinds and args.cpu_budget > 0:
        base = per["bf16"]["cpu_oracle"]
        cpu = {k: base[k] for k in ("value", "unit", "cores", "kind", "sample", "parity")
               if k in base}
        cpu["host"] = host_info()
        cpu["per_config"] = {k: per[k]["cpu_oracle"] for k in cpu_kinds}

    steps = args.steps
    line = {
        "metric": METRIC,
        "value": b["tflops"],
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": b["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic" if args.operands == "random" else
                "synthetic, dense cases on all-zero operand codes (power experiment)",
        "config": {"workload": "gemm_bf16 D=A*B^T M=4096 N=7168 K=16384, bf16 N(0,1) inputs, "
                               "fp32 accumulate, bf16 out",
                   "M": 4096, "N": 7168, "K": 16384, "parallelism": "single GPU"},
        "timing": "value and ms_per_step: median of the timed calls, each after a 512 MiB "
                  "scratch write (cold L2 and MALL), HIP events on the launch stream, after "
                  "the warm-up calls and a 0.2 s settle phase of untimed calls; warm: the same "
                  "calls back to back; cold_clean: after the scratch write and a 512 MiB read",
        "frac_of_peak": b["frac_of_peak"],
        "warm": b["warm"],
        "cold_clean": b.get("cold_clean"),
        "roofline": roof,
        "mfma_only": b["mfma_only"],
        "cpu_baseline": cpu,
        "context": {"pages_bf16_tflops": PAGES_BF16_TFLOPS,
                    "note": "the pages' figure at this shape on another accelerator (Ascend "
                            "950DT, 99.8% of its own stated limit); context, not a baseline"},
        "per_dtype": per,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
