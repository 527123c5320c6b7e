"""Python binding of the block-scaled GEMM library for MI355X (gfx950).

Every function here only marshals torch tensors (device memory and streams) into
the C ABI declared in ``include/bsg.h`` and raises on a non-zero status; every
step of the computation runs in the library's HIP kernels.  There is no fallback:
if ``libbsg.so`` is missing or cannot be loaded, every call raises.

    D = gemm_bf16(A, B)                         # bf16 [M,K] x bf16 [N,K] -> bf16 [M,N]
    D = gemm_fp8_blockscaled(A, sfa, B, sfb)    # e4m3 with UE8M0 1x128 / 128x128 scales
    D = gemm_fp4_blockscaled(A, sfa, B, sfb)    # e2m1 (2 per byte) with UE8M0 1x32 scales
    D = m_grouped_gemm_fp8(A, sfa, B, sfb, offsets)
    D = m_grouped_gemm_bf16(A, B, offsets) / m_grouped_gemm_fp4(A, sfa, B, sfb, offsets, K=K)
    D = m_grouped_gemm_fp8_masked(A, sfa, B, sfb, masked_m)   # A [G, max_m, K], counts on the GPU
    P = pack_ue8m0_scales(sf)                   # uint8 [mn, kb] -> int16 [ceil(kb/2), mn]
    sf = unpack_ue8m0_scales(P, mn, kb)
    P = ensure_packed(sf, mn, kb)               # reuse if already packed, else pack
    Q, P = quantize_fp8_per_token(X)            # bf16 [M,K] -> e4m3 + packed 1x128 scales
    Q, P = quantize_fp4_per_token(X)            # bf16 [M,K] -> e2m1 (2/byte) + packed 1x32 scales
    Q, P = swiglu_quantize_fp8(H, inter)        # silu(H[:, :I]) * H[:, I:2I] -> e4m3 + scales
    D = moe_ffn_fp8(A, sfa, W13, sfw13, W2, sfw2, offsets)   # grouped up, SwiGLU, grouped down
    moe_ffn_fp8_noalloc(A, sfa, W13, sfw13, W2, sfw2, offsets, out=D)   # no workspace, no allocation
    L = mqa_logits(fmt, Q, sfq, K, sfk, W, ks, ke, S)  # sum_h w * max(0, q_h . k) in key windows
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsg.so")

BSG_OK = 0
BSG_ERR_INVALID_ARG = 1
BSG_ERR_UNSUPPORTED_SHAPE = 2
BSG_ERR_MISALIGNED = 3
BSG_ERR_HIP = 4

SCALE_RULES = {"ceil": 0, "ocp_mx": 1}

_lock = threading.Lock()
_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

EXPORTS = {
    "gemm_bf16": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _vp],
    "gemm_fp8_blockscaled": [_vp, _i64, _vp, _i64, _i32, _vp, _i64, _vp, _i64, _i32, _vp, _i64,
                             _i64, _i64, _i64, _vp],
    "gemm_fp4_blockscaled": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                             _i64, _i64, _i64, _vp],
    "m_grouped_gemm_fp8": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64,
                           _vp, _i32, _i64, _i64, _i64, _vp],
    "m_grouped_gemm_bf16": [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i32, _i64, _i64, _i64, _vp],
    "m_grouped_gemm_fp4": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64,
                           _vp, _i32, _i64, _i64, _i64, _vp],
    "m_grouped_gemm_fp8_masked": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp,
                                  _i64, _vp, _i32, _i64, _i64, _i64, _vp],
    "pack_ue8m0_scales": [_vp, _i64, _i64, _i64, _vp, _i64, _vp],
    "unpack_ue8m0_scales": [_vp, _i64, _i64, _i64, _vp, _i64, _vp],
    "pack_ue8m0_scales_f32": [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp],
    "quantize_fp8_per_token": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _vp],
    "quantize_fp4_per_token": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _vp],
    "swiglu_quantize_fp8": [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _vp],
    "moe_ffn_fp8": [_vp, _i64, _vp, _i64,
                    _vp, _i64, _i64, _vp, _i64, _i64,
                    _vp, _i64, _i64, _vp, _i64, _i64,
                    _vp, _i32, _i64, _i64, _i64,
                    _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i32, _vp],
    "mqa_logits_fp8": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64,
                       _i64, _i64, _i32, _i64, _i64, _vp],
    "mqa_logits_fp4": [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64,
                       _i64, _i64, _i32, _i64, _i64, _vp],
    "moe_ffn_fp8_noalloc": [_vp, _i64, _vp, _i64,
                            _vp, _i64, _i64, _vp, _i64, _i64,
                            _vp, _i64, _i64, _vp, _i64, _i64,
                            _vp, _i32, _i64, _i64, _i64,
                            _vp, _i64, _i32, _vp],
}


class BsgError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """The loaded libbsg.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m block_scaled_precision_05_amd.build` (hipcc, gfx950)")
            l = ctypes.CDLL(LIB_PATH)
            for name, argtypes in EXPORTS.items():
                f = getattr(l, name)
                f.argtypes = argtypes
                f.restype = ctypes.c_int
            l.bsg_status_string.argtypes = [ctypes.c_int]
            l.bsg_status_string.restype = ctypes.c_char_p
            _lib = l
        return _lib


def status_string(status: int) -> str:
    return lib().bsg_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != BSG_OK:
        raise BsgError(fn, status)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None) -> int:
    return 0 if t is None else t.data_ptr()


def _mat(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")


def _bytes_u8(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


def _out(out, M, N, device):
    if out is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device)
    if out.dtype != torch.bfloat16 or out.shape[0] < M or out.shape[1] < N:
        raise ValueError("out must be a bfloat16 tensor of at least [M, N]")
    return out


def gemm_bf16(A: torch.Tensor, B: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """D[M,N] = A[M,K] @ B[N,K]^T, bf16 in, fp32 accumulate, bf16 out."""
    _dev(A, B, out)
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("K mismatch")
    D = _out(out, M, N, A.device)
    _check("gemm_bf16", lib().gemm_bf16(_ptr(A), _mat(A, "A"), _ptr(B), _mat(B, "B"), _ptr(D),
                                        _mat(D, "out"), M, N, K, _stream(stream)))
    return D


def _packed(sf: torch.Tensor, name: str) -> int:
    if sf.dtype != torch.int16:
        raise TypeError(f"{name} must be packed int16 scales (see ensure_packed)")
    return _mat(sf, name)


def gemm_fp8_blockscaled(A, sfa, B, sfb, out=None, stream=None, sfb_gran_mn: int = 128):
    """FP8 e4m3 GEMM with UE8M0 scales: sfa packed int16 [ceil(K/256), >=M] (1x128
    per row of A); sfb packed int16 [ceil(K/256), >=ceil(N/128)] (128x128 blocks of
    B, sfb_gran_mn = 128) or [ceil(K/256), >=N] (one per row of B per 128-wide
    K-block, sfb_gran_mn = 1).  A and B are float8_e4m3fn or uint8 codes."""
    _dev(A, sfa, B, sfb, out)
    A, B = _bytes_u8(A), _bytes_u8(B)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("K mismatch")
    D = _out(out, M, N, A.device)
    _check("gemm_fp8_blockscaled", lib().gemm_fp8_blockscaled(
        _ptr(A), _mat(A, "A"), _ptr(sfa), _packed(sfa, "sfa"), 1, _ptr(B), _mat(B, "B"),
        _ptr(sfb), _packed(sfb, "sfb"), sfb_gran_mn, _ptr(D), _mat(D, "out"), M, N, K,
        _stream(stream)))
    return D


def gemm_fp4_blockscaled(A, sfa, B, sfb, K: int | None = None, out=None, stream=None):
    """FP4 e2m1 GEMM: A uint8 [M, K/2] and B uint8 [N, K/2] hold two values per
    byte (even K index in the low nibble); sfa / sfb packed int16 [ceil(K/64), >=M]
    / [.., >=N] (one UE8M0 byte per row per 32-wide K-block)."""
    _dev(A, sfa, B, sfb, out)
    A, B = _bytes_u8(A), _bytes_u8(B)
    M = A.shape[0]
    N = B.shape[0]
    if K is None:
        K = 2 * A.shape[1]
    if A.shape[1] * 2 < K or B.shape[1] * 2 < K:
        raise ValueError("K larger than the operands")
    D = _out(out, M, N, A.device)
    _check("gemm_fp4_blockscaled", lib().gemm_fp4_blockscaled(
        _ptr(A), _mat(A, "A"), _ptr(sfa), _packed(sfa, "sfa"), _ptr(B), _mat(B, "B"), _ptr(sfb),
        _packed(sfb, "sfb"), _ptr(D), _mat(D, "out"), M, N, K, _stream(stream)))
    return D


def m_grouped_gemm_fp8(A, sfa, B, sfb, offsets, out=None, stream=None):
    """M-grouped FP8 GEMM.  A e4m3 [M_total, K]; B e4m3 [G, N, K]; sfa packed int16
    [ceil(K/256), >=M_total]; sfb packed int16 [G, ceil(K/256), >=ceil(N/128)];
    offsets int32 [G+1] on the GPU (rows [off[g], off[g+1]) use expert g).  Rows
    outside [off[0], off[G]) of ``out`` are left untouched."""
    _dev(A, sfa, B, sfb, offsets, out)
    A, B = _bytes_u8(A), _bytes_u8(B)
    if B.dim() != 3 or sfb.dim() != 3:
        raise ValueError("B must be [G, N, K] and sfb [G, kp, ld]")
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise TypeError("offsets must be a contiguous int32 vector")
    G, N, K = B.shape
    if offsets.numel() != G + 1:
        raise ValueError("offsets must have G+1 entries")
    M = A.shape[0]
    if A.shape[1] != K:
        raise ValueError("K mismatch")
    if B.stride(2) != 1 or sfb.stride(2) != 1 or sfb.dtype != torch.int16:
        raise ValueError("B and sfb must be contiguous along their last dimension")
    D = _out(out, M, N, A.device)
    _check("m_grouped_gemm_fp8", lib().m_grouped_gemm_fp8(
        _ptr(A), _mat(A, "A"), _ptr(sfa), _packed(sfa, "sfa"), _ptr(B), B.stride(1), B.stride(0),
        _ptr(sfb), sfb.stride(1), sfb.stride(0), _ptr(D), _mat(D, "out"), _ptr(offsets), G, M, N,
        K, _stream(stream)))
    return D


def _offsets_check(offsets, G):
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise TypeError("offsets must be a contiguous int32 vector")
    if offsets.numel() != G + 1:
        raise ValueError("offsets must have G+1 entries")


def m_grouped_gemm_bf16(A, B, offsets, out=None, stream=None):
    """M-grouped BF16 GEMM.  A bf16 [M_total, K]; B bf16 [G, N, K]; offsets int32
    [G+1] on the GPU.  Rows outside [off[0], off[G]) of ``out`` are left untouched."""
    _dev(A, B, offsets, out)
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if B.dim() != 3 or B.stride(2) != 1:
        raise ValueError("B must be [G, N, K], contiguous along K")
    G, N, K = B.shape
    _offsets_check(offsets, G)
    M = A.shape[0]
    if A.shape[1] != K:
        raise ValueError("K mismatch")
    D = _out(out, M, N, A.device)
    _check("m_grouped_gemm_bf16", lib().m_grouped_gemm_bf16(
        _ptr(A), _mat(A, "A"), _ptr(B), B.stride(1), B.stride(0), _ptr(D), _mat(D, "out"),
        _ptr(offsets), G, M, N, K, _stream(stream)))
    return D


def m_grouped_gemm_fp4(A, sfa, B, sfb, offsets, K: int | None = None, out=None, stream=None):
    """M-grouped FP4 GEMM.  A uint8 [M_total, K/2]; B uint8 [G, N, K/2] (two e2m1
    values per byte, even K index in the low nibble); sfa packed int16
    [ceil(K/64), >=M_total]; sfb packed int16 [G, ceil(K/64), >=N]; offsets int32
    [G+1] on the GPU."""
    _dev(A, sfa, B, sfb, offsets, out)
    A, B = _bytes_u8(A), _bytes_u8(B)
    if B.dim() != 3 or sfb.dim() != 3:
        raise ValueError("B must be [G, N, K/2] and sfb [G, kp, ld]")
    G, N, kb = B.shape
    K = 2 * kb if K is None else K
    _offsets_check(offsets, G)
    M = A.shape[0]
    if A.shape[1] * 2 < K or kb * 2 < K:
        raise ValueError("K larger than the operands")
    if B.stride(2) != 1 or sfb.stride(2) != 1 or sfb.dtype != torch.int16:
        raise ValueError("B and sfb must be contiguous along their last dimension")
    D = _out(out, M, N, A.device)
    _check("m_grouped_gemm_fp4", lib().m_grouped_gemm_fp4(
        _ptr(A), _mat(A, "A"), _ptr(sfa), _packed(sfa, "sfa"), _ptr(B), B.stride(1), B.stride(0),
        _ptr(sfb), sfb.stride(1), sfb.stride(0), _ptr(D), _mat(D, "out"), _ptr(offsets), G, M, N,
        K, _stream(stream)))
    return D


def m_grouped_gemm_fp8_masked(A, sfa, B, sfb, masked_m, out=None, stream=None):
    """Masked M-grouped FP8 GEMM.  A e4m3 [G, max_m, K]; B e4m3 [G, N, K]; sfa packed
    int16 [ceil(K/256), >=G*max_m] over the G*max_m rows; sfb packed int16
    [G, ceil(K/256), >=ceil(N/128)]; masked_m int32 [G] on the GPU.  Returns D bf16
    [G, max_m, N]; rows r >= masked_m[g] of expert g are left untouched."""
    _dev(A, sfa, B, sfb, masked_m, out)
    A, B = _bytes_u8(A), _bytes_u8(B)
    if A.dim() != 3 or B.dim() != 3 or sfb.dim() != 3:
        raise ValueError("A must be [G, max_m, K], B [G, N, K] and sfb [G, kp, ld]")
    if masked_m.dtype != torch.int32 or masked_m.dim() != 1 or not masked_m.is_contiguous():
        raise TypeError("masked_m must be a contiguous int32 vector")
    G, max_m, K = A.shape
    N = B.shape[1]
    if B.shape[0] != G or B.shape[2] != K or masked_m.numel() != G:
        raise ValueError("A, B and masked_m disagree on G or K")
    if A.stride(2) != 1 or A.stride(0) != max_m * A.stride(1):
        raise ValueError("A's experts must be stacked rows of one [G*max_m, K] matrix")
    if B.stride(2) != 1 or sfb.stride(2) != 1 or sfb.dtype != torch.int16:
        raise ValueError("B and sfb must be contiguous along their last dimension")
    if out is None:
        out = torch.empty((G, max_m, N), dtype=torch.bfloat16, device=A.device)
    if out.dtype != torch.bfloat16 or out.dim() != 3 or out.stride(2) != 1 or \
            out.stride(0) != max_m * out.stride(1) or out.shape[1] != max_m or out.shape[2] < N:
        raise ValueError("out must be bfloat16 [G, max_m, >=N] stacked rows")
    _check("m_grouped_gemm_fp8_masked", lib().m_grouped_gemm_fp8_masked(
        _ptr(A), A.stride(1), _ptr(sfa), _packed(sfa, "sfa"), _ptr(B), B.stride(1), B.stride(0),
        _ptr(sfb), sfb.stride(1), sfb.stride(0), _ptr(out), out.stride(1), _ptr(masked_m), G,
        max_m, N, K, _stream(stream)))
    return out


# hipStreamLegacy: the legacy default stream as a non-NULL handle (the pack and
# unpack entry points read a NULL stream as "host pointers").
_HIP_STREAM_LEGACY = 1


def _pack_stream(tensors, stream) -> int:
    """NULL (host path) when every tensor lives in host memory; otherwise the
    device stream, with the default stream passed as hipStreamLegacy."""
    on_gpu = [t.is_cuda for t in tensors if t is not None]
    if not any(on_gpu):
        if stream is not None:
            raise ValueError("host tensors are packed synchronously: pass no stream")
        return 0
    if not all(on_gpu):
        raise ValueError("sf and the packed array must both live on the GPU or both on the host")
    s = _stream(stream)
    return s if s else _HIP_STREAM_LEGACY


def pack_ue8m0_scales(sf: torch.Tensor, ld_packed: int | None = None, out=None, stream=None):
    """uint8 (or float8_e8m0fnu) [mn, kb] -> packed int16 [ceil(kb/2), ld_packed].
    GPU tensors are packed by a kernel on ``stream``; host tensors on the calling
    thread (the C entry point's NULL-stream path)."""
    sf = _bytes_u8(sf)
    mn, kb = sf.shape
    ldp = mn if ld_packed is None else int(ld_packed)
    if out is None:
        out = torch.empty(((kb + 1) // 2, ldp), dtype=torch.int16, device=sf.device)
    st = _pack_stream((sf, out), stream)
    _check("pack_ue8m0_scales", lib().pack_ue8m0_scales(_ptr(sf), mn, kb, _mat(sf, "sf"),
                                                        _ptr(out), _mat(out, "out"), st))
    return out


def pack_ue8m0_scales_f32(sf: torch.Tensor, ld_packed: int | None = None, out=None, stream=None):
    """fp32 [mn, kb] holding powers of two 2^e (-127 <= e <= 127) -> packed int16
    [ceil(kb/2), ld_packed], exactly; raises ValueError if any value has no UE8M0
    code (the library counts them; for GPU tensors reading the count back
    synchronises the stream)."""
    if sf.dtype != torch.float32 or sf.dim() != 2:
        raise TypeError("sf must be a 2-D float32 tensor")
    mn, kb = sf.shape
    ldp = mn if ld_packed is None else int(ld_packed)
    if out is None:
        out = torch.empty(((kb + 1) // 2, ldp), dtype=torch.int16, device=sf.device)
    count = torch.zeros(1, dtype=torch.int32, device=sf.device)
    st = _pack_stream((sf, out, count), stream)
    _check("pack_ue8m0_scales_f32", lib().pack_ue8m0_scales_f32(
        _ptr(sf), mn, kb, _mat(sf, "sf"), _ptr(out), _mat(out, "out"), _ptr(count), st))
    bad = int(count.item())
    if bad:
        raise ValueError(f"{bad} scale factors are not powers of two in [2^-127, 2^127]: "
                         "UE8M0 cannot represent them (rounding scales is the quantiser's job)")
    return out


def unpack_ue8m0_scales(packed: torch.Tensor, mn: int, kb: int, out=None, stream=None):
    """packed int16 [ceil(kb/2), >=mn] -> uint8 [mn, kb] (on the GPU or, for host
    tensors, on the calling thread)."""
    if out is None:
        out = torch.empty((mn, kb), dtype=torch.uint8, device=packed.device)
    st = _pack_stream((packed, out), stream)
    _check("unpack_ue8m0_scales", lib().unpack_ue8m0_scales(_ptr(packed), mn, kb,
                                                            _packed(packed, "packed"), _ptr(out),
                                                            _mat(out, "out"), st))
    return out


def is_packed(sf: torch.Tensor, mn: int, kb: int) -> bool:
    """True if ``sf`` already has the packed layout: int16 [ceil(kb/2), >=mn] with
    unit stride along MN."""
    return (sf.dtype == torch.int16 and sf.dim() == 2 and sf.shape[0] == (kb + 1) // 2
            and sf.shape[1] >= mn and (sf.shape[1] <= 1 or sf.stride(1) == 1))


def ensure_packed(sf: torch.Tensor, mn: int, kb: int, stream=None) -> torch.Tensor:
    """Reuse-or-convert, decided on every call: an already packed tensor is
    returned as it is; UE8M0 bytes ([mn, kb] uint8 or float8_e8m0fnu) are packed,
    and fp32 powers of two ([mn, kb]) converted exactly and packed (anything else
    in fp32 raises: UE8M0 cannot hold it), on the GPU for GPU tensors.  The pages describe this helper and note the conversion costs
    time when it is needed ("DeepGEMM-Ascend cobre quantas operacoes no Ascend
    950?", section "Fatores de escala FP8 e o formato UE8M0 no Ascend")."""
    if is_packed(sf, mn, kb):
        return sf
    if sf.dtype in (torch.uint8, torch.float8_e8m0fnu) and sf.dim() == 2 and \
            tuple(sf.shape) == (mn, kb):
        return pack_ue8m0_scales(sf, stream=stream if sf.is_cuda else None)
    if sf.dtype == torch.float32 and sf.dim() == 2 and tuple(sf.shape) == (mn, kb):
        return pack_ue8m0_scales_f32(sf, stream=stream if sf.is_cuda else None)
    raise TypeError(
        f"scales must be packed int16 [{(kb + 1) // 2}, >={mn}], UE8M0 bytes [{mn}, {kb}] or "
        f"fp32 powers of two [{mn}, {kb}]; got {sf.dtype} {tuple(sf.shape)}")


def _quantize(fn: str, X, rule, q_cols, gk, out, sf_out, ld_sf, stream):
    _dev(X, out, sf_out)
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    if rule not in SCALE_RULES:
        raise ValueError(f"rule must be one of {sorted(SCALE_RULES)}")
    M, K = X.shape
    kp = (K // gk + 1) // 2
    ld = M if ld_sf is None else int(ld_sf)
    Q = torch.empty((M, q_cols(K)), dtype=torch.uint8, device=X.device) if out is None \
        else _bytes_u8(out)
    P = torch.empty((kp, ld), dtype=torch.int16, device=X.device) if sf_out is None else sf_out
    _check(fn, getattr(lib(), fn)(_ptr(X), _mat(X, "X"), _ptr(Q), _mat(Q, "out"), _ptr(P),
                                  _packed(P, "sf_out"), M, K, SCALE_RULES[rule], _stream(stream)))
    return Q, P


def quantize_fp8_per_token(X, rule: str = "ceil", out=None, sf_out=None, ld_sf=None, stream=None):
    """bf16 [M, K] -> (e4m3 codes uint8 [M, K], packed int16 scales [ceil(K/256), ld_sf])
    with one UE8M0 scale per row per 128-wide K-block; ``rule`` is "ceil" (no
    clipping) or "ocp_mx".  The scales are ready to pass as ``sfa``."""
    return _quantize("quantize_fp8_per_token", X, rule, lambda K: K, 128, out, sf_out, ld_sf,
                     stream)


def quantize_fp4_per_token(X, rule: str = "ceil", out=None, sf_out=None, ld_sf=None, stream=None):
    """bf16 [M, K] -> (e2m1 codes uint8 [M, K/2], even K index in the low nibble;
    packed int16 scales [ceil(K/64), ld_sf]), one UE8M0 scale per row per 32-wide
    K-block."""
    return _quantize("quantize_fp4_per_token", X, rule, lambda K: K // 2, 32, out, sf_out, ld_sf,
                     stream)


def swiglu_quantize_fp8(H, inter: int, rule: str = "ceil", out=None, sf_out=None, ld_sf=None,
                        stream=None):
    """bf16 H [M, >=2*inter] (gate in columns [0, inter), up in [inter, 2*inter)) ->
    (e4m3 codes uint8 [M, inter], packed int16 scales [ceil(inter/256), ld_sf]) of
    y = silu(gate) * up, one UE8M0 scale per row per 128 columns."""
    _dev(H, out, sf_out)
    if H.dtype != torch.bfloat16:
        raise TypeError("H must be bfloat16")
    if rule not in SCALE_RULES:
        raise ValueError(f"rule must be one of {sorted(SCALE_RULES)}")
    M = H.shape[0]
    kp = (inter // 128 + 1) // 2
    ld = M if ld_sf is None else int(ld_sf)
    Q = torch.empty((M, inter), dtype=torch.uint8, device=H.device) if out is None \
        else _bytes_u8(out)
    P = torch.empty((kp, ld), dtype=torch.int16, device=H.device) if sf_out is None else sf_out
    _check("swiglu_quantize_fp8", lib().swiglu_quantize_fp8(
        _ptr(H), _mat(H, "H"), _ptr(Q), _mat(Q, "out"), _ptr(P), _packed(P, "sf_out"), M, inter,
        SCALE_RULES[rule], _stream(stream)))
    return Q, P


def moe_ffn_fp8(A, sfa, W13, sfw13, W2, sfw2, offsets, rule: str = "ceil", out=None,
                workspace=None, stream=None):
    """MoE FFN core: grouped up-projection (W13 [G, 2*inter, hidden]), SwiGLU + FP8
    requantisation, grouped down-projection (W2 [G, hidden, inter]); A e4m3
    [M_total, hidden] with packed scales; offsets int32 [G+1] on the GPU.  Returns
    D bf16 [M_total, hidden].  ``workspace`` may pass the (Y, sfy) buffers (e4m3
    uint8 [M_total, >=inter] and packed int16 [ceil(inter/256), >=M_total]); they
    are allocated here otherwise.  The bf16 up-projection output H is never formed."""
    _dev(A, sfa, W13, sfw13, W2, sfw2, offsets, out)
    A, W13, W2 = _bytes_u8(A), _bytes_u8(W13), _bytes_u8(W2)
    if W13.dim() != 3 or W2.dim() != 3 or sfw13.dim() != 3 or sfw2.dim() != 3:
        raise ValueError("W13, W2 and their scales must be [G, rows, cols]")
    if offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise TypeError("offsets must be a contiguous int32 vector")
    G, two_i, hidden = W13.shape
    inter = two_i // 2
    if W2.shape[0] != G or W2.shape[1] != hidden or W2.shape[2] != inter or two_i != 2 * inter:
        raise ValueError("W2 must be [G, hidden, inter] for W13 [G, 2*inter, hidden]")
    M = A.shape[0]
    if workspace is None:
        Y = torch.empty((M, inter), dtype=torch.uint8, device=A.device)
        sfy = torch.empty(((inter // 128 + 1) // 2, M), dtype=torch.int16, device=A.device)
    else:
        Y, sfy = workspace
    D = _out(out, M, hidden, A.device)
    for t, n in ((W13, "W13"), (W2, "W2"), (sfw13, "sfw13"), (sfw2, "sfw2")):
        if t.stride(2) != 1:
            raise ValueError(f"{n} must be contiguous along its last dimension")
    _check("moe_ffn_fp8", lib().moe_ffn_fp8(
        _ptr(A), _mat(A, "A"), _ptr(sfa), _packed(sfa, "sfa"),
        _ptr(W13), W13.stride(1), W13.stride(0), _ptr(sfw13), sfw13.stride(1), sfw13.stride(0),
        _ptr(W2), W2.stride(1), W2.stride(0), _ptr(sfw2), sfw2.stride(1), sfw2.stride(0),
        _ptr(offsets), G, M, hidden, inter,
        0, 0, _ptr(Y), _mat(_bytes_u8(Y), "Y"), _ptr(sfy), _packed(sfy, "sfy"),
        _ptr(D), _mat(D, "out"), SCALE_RULES[rule], _stream(stream)))
    return D


def moe_ffn_fp8_noalloc(A, sfa, W13, sfw13, W2, sfw2, offsets, out, rule: str = "ceil",
                        stream=None):
    """moe_ffn_fp8 without a workspace: the library keeps Y and its scales in a fixed
    64 MiB device array (one per GPU), so the call allocates nothing; ``out`` (bf16
    [M_total, hidden]) must be given.  Calls that overlap on one GPU race on that
    array."""
    _dev(A, sfa, W13, sfw13, W2, sfw2, offsets, out)
    A, W13, W2 = _bytes_u8(A), _bytes_u8(W13), _bytes_u8(W2)
    if W13.dim() != 3 or W2.dim() != 3 or sfw13.dim() != 3 or sfw2.dim() != 3:
        raise ValueError("W13, W2 and their scales must be [G, rows, cols]")
    _offsets_check(offsets, W13.shape[0])
    G, two_i, hidden = W13.shape
    M = A.shape[0]
    if out.dtype != torch.bfloat16 or out.shape[0] < M or out.shape[1] < hidden:
        raise ValueError("out must be a bfloat16 tensor of at least [M_total, hidden]")
    for t, n in ((W13, "W13"), (W2, "W2"), (sfw13, "sfw13"), (sfw2, "sfw2")):
        if t.stride(2) != 1:
            raise ValueError(f"{n} must be contiguous along its last dimension")
    _check("moe_ffn_fp8_noalloc", lib().moe_ffn_fp8_noalloc(
        _ptr(A), _mat(A, "A"), _ptr(sfa), _packed(sfa, "sfa"),
        _ptr(W13), W13.stride(1), W13.stride(0), _ptr(sfw13), sfw13.stride(1), sfw13.stride(0),
        _ptr(W2), W2.stride(1), W2.stride(0), _ptr(sfw2), sfw2.stride(1), sfw2.stride(0),
        _ptr(offsets), G, M, hidden, two_i // 2, _ptr(out), _mat(out, "out"),
        SCALE_RULES[rule], _stream(stream)))
    return out


def mqa_logits(fmt: str, Q, sfq, K, sfk, W, ks, ke, S: int, q_per_group: int | None = None,
               group_rows: int = 0, out=None, stream=None):
    """MQA logits (fmt "fp8" or "fp4"): L[t][s] = sum_h W[t][h] * max(0, q[t][h] . k[s])
    for ks[t] <= s < ke[t], -inf for the other s < S.  Q: codes [T*H, 128] (fp8) or
    [T*H, 64] (fp4, two per byte) with packed scales sfq over its rows; K: codes over
    the key rows with packed scales sfk; W float32 [T, H]; ks, ke int32 [T] on the GPU.
    Query t reads key group t // q_per_group (default: one group), whose key s is
    row g * group_rows + s of K.  Returns float32 [T, S]."""
    _dev(Q, sfq, K, sfk, W, ks, ke, out)
    if fmt not in ("fp8", "fp4"):
        raise ValueError("fmt must be 'fp8' or 'fp4'")
    Q, K = _bytes_u8(Q), _bytes_u8(K)
    if W.dtype != torch.float32 or ks.dtype != torch.int32 or ke.dtype != torch.int32:
        raise TypeError("W must be float32 and ks, ke int32")
    T, H = W.shape
    if Q.shape[0] != T * H:
        raise ValueError("Q must hold T*H rows")
    per = T if q_per_group is None else int(q_per_group)
    if out is None:
        out = torch.empty((T, S), dtype=torch.float32, device=Q.device)
    fn = lib().mqa_logits_fp8 if fmt == "fp8" else lib().mqa_logits_fp4
    _check("mqa_logits_" + fmt, fn(
        _ptr(Q), _mat(Q, "Q"), _ptr(sfq), _packed(sfq, "sfq"), _ptr(K), _mat(K, "K"), _ptr(sfk),
        _packed(sfk, "sfk"), _ptr(W), _mat(W, "W"), _ptr(ks), _ptr(ke), _ptr(out), _mat(out, "out"),
        T, S, H, max(per, 1), int(group_rows), _stream(stream)))
    return out
