"""Seeded synthetic inputs for the block-scaled GEMM workloads.

This module only draws random operands and encodes them into the storage formats
(bf16, e4m3 codes, e2m1 nibbles, UE8M0 exponent bytes).  It holds none of the
GEMM's arithmetic; the GPU library and the CPU oracle both take its bytes as
they are.  Every draw uses an explicit ``torch.Generator`` so a (workload, seed,
device) triple always yields the same bytes.

Workloads (the shapes follow the dense 4096x7168x16384 case and the MoE routing
shape of 16384 tokens, hidden 7168, top-6 of 256 experts that the pages report
on: "DeepSeek lanza kernels de DeepGEMM para Huawei Ascend 950", section "Que
alcance tienen las pruebas de rendimiento"; "DeepSeek publica bibliotecas Ascend
para calculo e comunicacao de IA", section "Resultados de kernel e comunicacao"):

  bf16_small    BF16 256x256x512, N(0,1) rounded to bf16
  fp8_mid       FP8 1024x2048x4096, 1x128 (A) and 128x128 (B) UE8M0 scales
  bf16_large    BF16 4096x7168x16384
  fp8_large     FP8 4096x7168x16384, scales as fp8_mid
  fp8_rowb_large  FP8 4096x7168x16384 with one B scale per row (1x128 on B too)
  moe_fp8       M-grouped FP8: 256 experts, N=2048, K=7168, Zipf(1.1) routing
  moe_bf16      the same routing and shape in BF16
  moe_fp4       the same routing and shape in FP4 (1x32 scales)
  fp4_large     FP4 4096x7168x16384, 1x32 UE8M0 scales on both operands
  act_large     bf16 activations 4096x16384 (A of the dense shape), to be quantised
  act_moe       bf16 activations 16384x7168 (the MoE tokens), to be quantised
  masked_fp8    masked M-grouped FP8 (decode): 48 local experts of 384 (EP8),
                capacity 512 rows each, N=4096, K=7168, 4096 tokens top-6
  mqa_*         MQA logits (64 heads of 128): prefill of one 4096-token sequence
                (causal) and decode of 128 requests over 32768-token contexts, FP8
                and FP4
  moe_ffn       MoE FFN core on one GPU's share of the pages' fused MoE case:
                384 experts over EP8 -> 48 local experts plus the shared expert,
                16384 tokens top-6, hidden 7168, intermediate 2048

Value recipes:
  * FP8: for every scale entry an exponent e ~ U{-8..4}; a value is
    e4m3(clip(x / 2^e, -448, 448)) with x ~ N(0,1); torch's cast rounds to
    nearest even.  The scale byte is e + 127.
  * FP4: per 32-wide K-block, e = floor(log2(amax)) - 2 (the OCP MX rule, e2m1's
    largest exponent is 2); x / 2^e is rounded to nearest (ties to the even code)
    onto the e2m1 grid, saturating at 6.  An all-zero block gets e = 0.
  * Expert weights are drawn a few experts at a time (one operand of c*N rows per
    batch, cut into experts), so a workload costs a handful of device dispatches
    rather than several per expert.
  * MoE routing: 16384 tokens x top-6 = 98304 assignments drawn multinomially
    over 256 experts with popularity p_r ~ r^-1.1 (rank r = 1..256), ranks mapped
    to expert ids by a seeded permutation; every count is padded up to a multiple
    of 128.  Padding rows hold zero codes and scale byte 127.
  * MoE FFN share: 98304 assignments drawn as for moe_fp8 but over 384 experts;
    the local experts are those the seeded permutation puts on rank 0 of 8
    (48 of them), plus one shared expert that every token visits; counts padded
    to multiples of 128.  W13 [G][2*inter][hidden] (gate rows first) and W2
    [G][hidden][inter] follow the FP8 recipe with 128x128 scales.
  * Masked layout: expert g owns rows [g*cap, (g+1)*cap) of A; its valid count is
    the rank-0 share of a Zipf(1.1) top-6 routing of the decode tokens, capped at
    cap; rows past the count hold random codes too (the GEMM must ignore them).
  * Activations (bf16, input of the per-token quantiser): x ~ N(0,1) times a
    per-row power of two 2^U{-6..6}; one column in 64 (a seeded choice) is an
    outlier channel scaled by 32; the last ``zero_rows`` rows are zero.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# e2m1 magnitude codes 0..7 are 0, .5, 1, 1.5, 2, 3, 4, 6.  Rounding to nearest
# with ties to the even code means the decision points below (a tie at a point
# that excludes it goes down, one that includes it goes up).
_E2M1_UP_STRICT = (0.25, 1.25, 2.5, 5.0)      # at the tie, stay on the even code below
_E2M1_UP_INCL = (0.75, 1.75, 3.5)             # at the tie, move up to the even code above


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def bf16_normal(rows: int, cols: int, g: torch.Generator, device) -> torch.Tensor:
    """N(0,1) rounded to bf16 (round to nearest even), shape [rows][cols]."""
    x = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def fp8_operand(rows: int, K: int, gran_mn: int, g: torch.Generator, device,
                exp_lo: int = -8, exp_hi: int = 4):
    """e4m3 codes uint8 [rows][K] and UE8M0 bytes uint8 [ceil(rows/gran_mn)][K/128]."""
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    srows = (rows + gran_mn - 1) // gran_mn
    kb = K // 128
    e = torch.randint(exp_lo, exp_hi + 1, (srows, kb), generator=g, device=device,
                      dtype=torch.int32)
    x = torch.randn(rows, K, generator=g, device=device, dtype=torch.float32)
    inv = torch.exp2(-e.to(torch.float32))                        # exact powers of two
    inv = inv.repeat_interleave(gran_mn, dim=0)[:rows].repeat_interleave(128, dim=1)
    q = (x * inv).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    sf = (e + 127).to(torch.uint8)
    return q, sf


def e2m1_encode(v: torch.Tensor) -> torch.Tensor:
    """Round fp32 values onto the e2m1 grid (nearest, ties to the even code,
    saturating at +-6) and return 4-bit codes (uint8, 0..15)."""
    a = v.abs()
    code = torch.zeros_like(a, dtype=torch.uint8)
    for t in _E2M1_UP_STRICT:
        code += (a > t).to(torch.uint8)
    for t in _E2M1_UP_INCL:
        code += (a >= t).to(torch.uint8)
    sign = (torch.signbit(v)).to(torch.uint8) << 3
    return code | sign


def fp4_operand(rows: int, K: int, g: torch.Generator, device):
    """e2m1 values packed two per byte (even k in the low nibble) uint8
    [rows][K/2] and UE8M0 bytes uint8 [rows][K/32]."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    x = torch.randn(rows, K, generator=g, device=device, dtype=torch.float32)
    blocks = x.view(rows, K // 32, 32)
    amax = blocks.abs().amax(dim=2)
    e = torch.floor(torch.log2(amax)).to(torch.int32) - 2
    e = torch.where(amax > 0, e, torch.zeros_like(e)).clamp_(-127, 127)
    v = blocks * torch.exp2(-e.to(torch.float32)).unsqueeze(2)
    codes = e2m1_encode(v).view(rows, K)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    sf = (e + 127).to(torch.uint8)
    return packed.contiguous(), sf


def activations(rows: int, K: int, seed: int, device="cpu", zero_rows: int = 0) -> torch.Tensor:
    """bf16 [rows][K] activations (recipe in the module docstring)."""
    g = _gen(device, seed)
    x = torch.randn(rows, K, generator=g, device=device, dtype=torch.float32)
    e = torch.randint(-6, 7, (rows, 1), generator=g, device=device, dtype=torch.int32)
    x = x * torch.exp2(e.to(torch.float32))
    hot = torch.rand(K, generator=g, device=device) < (1.0 / 64)
    x[:, hot] *= 32.0
    if zero_rows:
        x[rows - zero_rows:] = 0
    return x.to(torch.bfloat16)


def moe_counts(g: torch.Generator, device, tokens: int = 16384, topk: int = 6,
               experts: int = 256, zipf: float = 1.1):
    """Per-expert routed row counts (int64 [experts])."""
    ranks = torch.arange(1, experts + 1, dtype=torch.float64)
    p = ranks.pow(-zipf)
    p = (p / p.sum()).to(torch.float32).to(device)
    draws = torch.multinomial(p, tokens * topk, replacement=True, generator=g)
    by_rank = torch.bincount(draws, minlength=experts).to(torch.int64)
    perm = torch.randperm(experts, generator=g, device=device)
    counts = torch.empty_like(by_rank)
    counts[perm] = by_rank
    return counts


def pad_offsets(counts: torch.Tensor, align: int = 128) -> torch.Tensor:
    """int32 [G+1] start rows of every expert after padding each count up to
    a multiple of ``align``."""
    padded = (counts + align - 1) // align * align
    off = torch.zeros(counts.numel() + 1, dtype=torch.int64, device=counts.device)
    off[1:] = torch.cumsum(padded, 0)
    return off.to(torch.int32)


def expert_weights(kind: str, G: int, N: int, K: int, g: torch.Generator, device,
                   gran_mn: int = 128, max_elems: int = 1 << 31):
    """G experts' operands [G][N][..] (and UE8M0 bytes [G][..][..]) drawn a few
    experts at a time: each batch is one operand of c*N rows, cut into experts.
    FP8 batches need N % gran_mn == 0 so that no scale block straddles two experts
    (otherwise experts are drawn one by one)."""
    per = max(1, min(G, max_elems // max(1, N * K)))
    if kind == "fp8" and N % gran_mn:
        per = 1
    qs, sfs = [], []
    for e0 in range(0, G, per):
        c = min(per, G - e0)
        if kind == "fp8":
            q, sf = fp8_operand(c * N, K, gran_mn, g, device)
            qs.append(q.view(c, N, K))
            sfs.append(sf.view(c, -1, K // 128))
        elif kind == "fp4":
            q, sf = fp4_operand(c * N, K, g, device)
            qs.append(q.view(c, N, K // 2))
            sfs.append(sf.view(c, N, K // 32))
        elif kind == "bf16":
            qs.append(bf16_normal(c * N, K, g, device).view(c, N, K))
        else:
            raise ValueError(kind)
    B = torch.cat(qs) if len(qs) > 1 else qs[0]
    return B, (torch.cat(sfs) if len(sfs) > 1 else sfs[0]) if sfs else None


def padded_rows_mask(offsets: torch.Tensor, counts: torch.Tensor, m_total: int) -> torch.Tensor:
    """bool [m_total]: True for the first counts[g] rows of every expert's range
    [off[g], off[g+1]), False for its padding rows."""
    r = torch.arange(m_total, device=offsets.device, dtype=torch.int64)
    off = offsets.to(torch.int64)
    e = torch.searchsorted(off, r, right=True) - 1
    e = e.clamp(0, counts.numel() - 1)
    return (r - off[e]) < counts.to(off.device)[e]


@dataclass
class Workload:
    name: str
    kind: str                # 'bf16' | 'fp8' | 'fp4' | 'grouped_fp8'
    M: int
    N: int
    K: int
    tensors: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)

    @property
    def flops(self) -> float:
        """Algorithmic flops, 2*M*N*K (useful rows only for the grouped case)."""
        if self.kind.startswith("grouped_"):
            return 2.0 * float(self.meta["useful_rows"]) * self.N * self.K
        if self.kind == "masked_fp8":
            return 2.0 * float(self.meta["useful_rows"]) * self.N * self.K
        if self.kind == "moe_ffn":
            return float(self.meta["useful_flops"])
        if self.kind.startswith("mqa_"):
            # the scores' dot products over the window pairs (the weighted max-sum
            # adds 2 flops per head and pair on top: counted separately)
            return 2.0 * float(self.meta["valid_pairs"]) * self.meta["H"] * self.meta["D"]
        return 2.0 * self.M * self.N * self.K


SHAPES = {
    "bf16_small": ("bf16", 256, 256, 512, 1001),
    "fp8_mid": ("fp8", 1024, 2048, 4096, 1002),
    "bf16_large": ("bf16", 4096, 7168, 16384, 1003),
    "moe_fp8": ("grouped_fp8", None, 2048, 7168, 1004),
    "moe_bf16": ("grouped_bf16", None, 2048, 7168, 1011),
    "moe_fp4": ("grouped_fp4", None, 2048, 7168, 1012),
    "fp4_large": ("fp4", 4096, 7168, 16384, 1005),
    "fp8_large": ("fp8", 4096, 7168, 16384, 1006),
    "fp8_rowb_large": ("fp8_rowb", 4096, 7168, 16384, 1017),
    "act_large": ("act", 4096, None, 16384, 1007),
    "act_moe": ("act", 16384, None, 7168, 1008),
    "moe_ffn": ("moe_ffn", None, None, None, 1009),
    "masked_fp8": ("masked_fp8", None, 4096, 7168, 1010),
    # MQA logits (H = 64 heads of 128): prefill of one 4096-token sequence, causal;
    # decode of 128 requests with 32768-token contexts
    "mqa_prefill_fp8": ("mqa_fp8_prefill", 4096, 4096, 128, 1013),
    "mqa_prefill_fp4": ("mqa_fp4_prefill", 4096, 4096, 128, 1014),
    "mqa_decode_fp8": ("mqa_fp8_decode", 128, 32768, 128, 1015),
    "mqa_decode_fp4": ("mqa_fp4_decode", 128, 32768, 128, 1016),
}


def dense(kind: str, M: int, N: int, K: int, seed: int, device="cpu", name: str = "custom"):
    g = _gen(device, seed)
    w = Workload(name, kind, M, N, K)
    if kind == "bf16":
        w.tensors["A"] = bf16_normal(M, K, g, device)
        w.tensors["B"] = bf16_normal(N, K, g, device)
    elif kind == "fp8":
        w.tensors["A"], w.tensors["sfa"] = fp8_operand(M, K, 1, g, device)
        w.tensors["B"], w.tensors["sfb"] = fp8_operand(N, K, 128, g, device)
    elif kind == "fp8_rowb":
        # FP8 with one B scale per row and 128-wide K-block (sfb_gran_mn = 1)
        w.tensors["A"], w.tensors["sfa"] = fp8_operand(M, K, 1, g, device)
        w.tensors["B"], w.tensors["sfb"] = fp8_operand(N, K, 1, g, device)
    elif kind == "fp4":
        w.tensors["A"], w.tensors["sfa"] = fp4_operand(M, K, g, device)
        w.tensors["B"], w.tensors["sfb"] = fp4_operand(N, K, g, device)
        w.meta["fp4_scale_rule"] = "ocp_mx: floor(log2(amax32)) - 2"
    else:
        raise ValueError(kind)
    w.meta["seed"] = seed
    return w


def grouped(G: int, N: int, K: int, seed: int, device="cpu", counts=None, name="custom",
            align: int = 128, tokens: int = 16384, topk: int = 6, zipf: float = 1.1,
            kind: str = "fp8"):
    """M-grouped inputs (kind "fp8", "bf16" or "fp4").  ``counts`` (int sequence,
    length G) overrides the Zipf routing draw; counts are padded to multiples of
    ``align``.  Padding rows hold zero operands (scale byte 127)."""
    g = _gen(device, seed)
    if counts is None:
        counts = moe_counts(g, device, tokens=tokens, topk=topk, experts=G, zipf=zipf)
    else:
        counts = torch.as_tensor(list(counts), dtype=torch.int64, device=device)
    off = pad_offsets(counts, align)
    m_total = int(off[-1].item())
    rows = max(m_total, 1)
    sfa = None
    if kind == "fp8":
        A, sfa = fp8_operand(rows, K, 1, g, device)
    elif kind == "fp4":
        A, sfa = fp4_operand(rows, K, g, device)
    elif kind == "bf16":
        A = bf16_normal(rows, K, g, device)
    else:
        raise ValueError(kind)
    A = A[:m_total]
    # zero the padding rows of every expert
    valid = padded_rows_mask(off, counts, m_total)
    A[~valid] = 0
    if sfa is not None:
        sfa = sfa[:m_total]
        sfa[~valid] = 127
    B, sfb = expert_weights(kind, G, N, K, g, device)
    w = Workload(name, "grouped_" + kind, m_total, N, K)
    w.tensors.update(A=A.contiguous(), B=B, offsets=off, counts=counts)
    if sfa is not None:
        w.tensors.update(sfa=sfa.contiguous(), sfb=sfb)
    w.meta.update(seed=seed, G=G, useful_rows=int(counts.sum().item()), m_total=m_total,
                  routing=f"multinomial({tokens}x{topk}), zipf {zipf}, pad {align}")
    return w


def masked(seed: int, device="cpu", G: int = 48, cap: int = 512, N: int = 4096, K: int = 7168,
           experts: int = 384, tokens: int = 4096, topk: int = 6, zipf: float = 1.1, counts=None,
           name: str = "custom"):
    """Masked M-grouped FP8 inputs (recipe in the module docstring)."""
    g = _gen(device, seed)
    if counts is None:
        all_counts = moe_counts(g, device, tokens=tokens, topk=topk, experts=experts, zipf=zipf)
        counts = all_counts[:G].clamp(max=cap)
    else:
        counts = torch.as_tensor(list(counts), dtype=torch.int64, device=device)
    A, sfa = fp8_operand(G * cap, K, 1, g, device)
    B, sfb = expert_weights("fp8", G, N, K, g, device)
    w = Workload(name, "masked_fp8", G * cap, N, K)
    w.tensors.update(A=A.view(G, cap, K), sfa=sfa, B=B, sfb=sfb,
                     masked_m=counts.to(torch.int32))
    useful = int(counts.clamp(min=0, max=cap).sum().item())
    w.meta.update(seed=seed, G=G, cap=cap, useful_rows=useful,
                  routing=f"{G} of {experts} experts, multinomial({tokens}x{topk}), zipf {zipf}, "
                          f"capacity {cap}")
    return w


def moe_ffn(seed: int, device="cpu", hidden: int = 7168, inter: int = 2048, experts: int = 384,
            ranks: int = 8, rank: int = 0, shared: int = 1, tokens: int = 16384, topk: int = 6,
            zipf: float = 1.1, counts=None, name: str = "custom", align: int = 128):
    """Inputs of the MoE FFN core for one rank's experts (recipe in the module
    docstring).  ``counts`` (length G) overrides the routing draw."""
    g = _gen(device, seed)
    if counts is None:
        all_counts = moe_counts(g, device, tokens=tokens, topk=topk, experts=experts, zipf=zipf)
        per = experts // ranks
        local = all_counts[rank * per:(rank + 1) * per]
        counts = torch.cat([local, torch.full((shared,), tokens, dtype=torch.int64,
                                              device=local.device)])
    else:
        counts = torch.as_tensor(list(counts), dtype=torch.int64, device=device)
    G = counts.numel()
    off = pad_offsets(counts, align)
    m_total = int(off[-1].item())
    A, sfa = fp8_operand(max(m_total, 1), hidden, 1, g, device)
    A, sfa = A[:m_total], sfa[:m_total]
    valid = padded_rows_mask(off, counts, m_total)
    A[~valid] = 0
    sfa[~valid] = 127
    W13, s13 = expert_weights("fp8", G, 2 * inter, hidden, g, device)
    W2, s2 = expert_weights("fp8", G, hidden, inter, g, device)
    w = Workload(name, "moe_ffn", m_total, hidden, hidden)
    w.tensors.update(A=A.contiguous(), sfa=sfa.contiguous(), W13=W13, sfw13=s13, W2=W2,
                     sfw2=s2, offsets=off, counts=counts)
    useful = int(counts.sum().item())
    w.meta.update(seed=seed, G=G, hidden=hidden, inter=inter, useful_rows=useful,
                  m_total=m_total,
                  routing=f"rank {rank} of {ranks}: {experts // ranks} of {experts} experts "
                          f"+ {shared} shared, multinomial({tokens}x{topk}), zipf {zipf}, pad {align}",
                  useful_flops=2.0 * useful * (2 * inter * hidden + hidden * inter))
    return w


def mqa(fmt: str, mode: str, seed: int, device="cpu", T: int = 4096, S: int = 4096, H: int = 64,
        ctx=None, name: str = "custom"):
    """Inputs of the MQA logits kernel (head dimension 128).  fmt "fp8" or "fp4";
    mode "prefill": T query tokens of one sequence over its S = T keys, causal
    windows [0, t+1); mode "decode": T requests with one query each over their own
    S-key context (key group per request), windows [0, ctx_t) with ctx_t drawn
    uniformly in [S/2, S] unless ``ctx`` gives them.  q and k rows follow the GEMM
    operand recipes (FP8: one UE8M0 scale per 128-element row, e ~ U{-8..4}; FP4:
    the OCP MX rule per 32), w ~ N(0,1) in fp32."""
    g = _gen(device, seed)
    D = 128
    groups = 1 if mode == "prefill" else T
    k_rows = groups * S
    if fmt == "fp8":
        Q, sfq = fp8_operand(T * H, D, 1, g, device)
        K, sfk = fp8_operand(k_rows, D, 1, g, device)
    else:
        Q, sfq = fp4_operand(T * H, D, g, device)
        K, sfk = fp4_operand(k_rows, D, g, device)
    W = torch.randn(T, H, generator=g, device=device, dtype=torch.float32)
    t = torch.arange(T, device=device, dtype=torch.int64)
    if mode == "prefill":
        ks = torch.zeros(T, dtype=torch.int32, device=device)
        ke = (t + 1).clamp(max=S).to(torch.int32)
        per, grows = T, 0
    else:
        if ctx is None:
            ctx = torch.randint(S // 2, S + 1, (T,), generator=g, device=device)
        ks = torch.zeros(T, dtype=torch.int32, device=device)
        ke = torch.as_tensor(ctx, device=device).to(torch.int32)
        per, grows = 1, S
    w = Workload(name, "mqa_" + fmt, T, S, D)
    w.tensors.update(Q=Q, sfq=sfq, K=K, sfk=sfk, W=W, ks=ks, ke=ke)
    valid = int((ke.to(torch.int64) - ks.to(torch.int64)).clamp(min=0).sum().item())
    w.meta.update(seed=seed, mode=mode, H=H, D=D, S=S, q_per_group=per, group_rows=grows,
                  k_rows=k_rows, valid_pairs=valid,
                  windows="causal [0, t+1)" if mode == "prefill" else "[0, ctx), ctx ~ U[S/2, S]")
    return w


def make(name: str, device="cpu", seed: int | None = None) -> Workload:
    """One of the named workloads in ``SHAPES``."""
    kind, M, N, K, default_seed = SHAPES[name]
    seed = default_seed if seed is None else seed
    if kind.startswith("grouped_"):
        w = grouped(256, N, K, seed, device=device, name=name, kind=kind[len("grouped_"):])
    elif kind == "moe_ffn":
        w = moe_ffn(seed, device=device, name=name)
    elif kind == "masked_fp8":
        w = masked(seed, device=device, N=N, K=K, name=name)
    elif kind.startswith("mqa_"):
        _, fmt, mode = kind.split("_")
        w = mqa(fmt, mode, seed, device=device, T=M, S=N, name=name)
    elif kind == "act":
        w = Workload(name, "act", M, 0, K)
        w.tensors["X"] = activations(M, K, seed, device=device)
        w.meta["seed"] = seed
    else:
        w = dense(kind, M, N, K, seed, device=device, name=name)
    w.name = name
    return w


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)
