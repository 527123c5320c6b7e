"""Plain CPU oracle for the block-scaled GEMM D = A @ B.T (BF16, FP8 e4m3, FP4 e2m1).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the GPU library ``block_scaled_precision_05_amd`` and neither imports the
other; the only thing both sides see is the seeded input bytes.

The arithmetic lives in ``oracle.c`` (plain C, fp64, no fast-math): exact decode
of every element, exact scaling by powers of two, one fp64 dot product per output
in plain k order.  This module only marshals numpy arrays into it and builds it
with gcc.  An independent exact-rational brute force for tiny shapes lives with
the tests (``tests/exact.py``), which pin this package against it.

``oracle.quantize`` (numpy, fp64) holds the per-token quantiser: bf16 rows to
e4m3 or e2m1 codes with UE8M0 block scales.

Parity status of each function (what pins it is in ``tests/test_oracle_pins.py``
and ``tests/test_quantize_pins.py``):
  decoders, bf16 rounding, pack/unpack, dense BF16/FP8/FP4, grouped BF16/FP8/FP4,
  masked grouped FP8, per-token quantisation, row norms (bf16, e4m3, e2m1): pinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)
_vp = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_bf16_to_f64.restype = ctypes.c_double
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_e4m3_to_f64.restype = ctypes.c_double
        lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_e2m1_to_f64.restype = ctypes.c_double
        lib.orc_e2m1_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_ue8m0_to_f64.restype = ctypes.c_double
        lib.orc_ue8m0_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_f64_to_bf16_rne.restype = ctypes.c_uint16
        lib.orc_f64_to_bf16_rne.argtypes = [ctypes.c_double]
        lib.orc_f64_to_bf16_rne_array.restype = None
        lib.orc_f64_to_bf16_rne_array.argtypes = [_vp, _vp, ctypes.c_int64]
        lib.orc_scale_byte.restype = ctypes.c_uint8
        lib.orc_scale_byte.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        lib.orc_pack_scales.restype = None
        lib.orc_pack_scales.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        _vp, ctypes.c_int64]
        lib.orc_unpack_scales.restype = None
        lib.orc_unpack_scales.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          _vp, ctypes.c_int64]
        sel = [_i64p, ctypes.c_int64, _i64p, ctypes.c_int64, _f64p]
        lib.orc_gemm_bf16.restype = ctypes.c_int
        lib.orc_gemm_bf16.argtypes = [_vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                      ctypes.c_int64] + sel
        lib.orc_gemm_fp8.restype = ctypes.c_int
        lib.orc_gemm_fp8.argtypes = [_vp, ctypes.c_int64, _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                     _vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64] + sel
        lib.orc_gemm_fp4.restype = ctypes.c_int
        lib.orc_gemm_fp4.argtypes = [_vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                     _vp, ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int64] + sel
        lib.orc_grouped_fp8.restype = ctypes.c_int
        lib.orc_grouped_fp8.argtypes = [_vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                        _vp, ctypes.c_int64, ctypes.c_int64,
                                        _vp, ctypes.c_int64, ctypes.c_int64,
                                        _vp, ctypes.c_int32, ctypes.c_int64] + sel
        lib.orc_norms.restype = ctypes.c_int
        lib.orc_norms.argtypes = [ctypes.c_int, _vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                  _i64p, ctypes.c_int64, _f64p]
        lib.orc_num_threads.restype = ctypes.c_int
        lib.orc_num_threads.argtypes = []
        _lib = lib
        return lib


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _c2d(a: np.ndarray, dtype) -> np.ndarray:
    """A 2-D array whose rows may be padded (stride >= width) but whose elements
    are contiguous within a row."""
    a = np.asarray(a)
    if a.dtype != np.dtype(dtype):
        a = a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype)
    if a.ndim != 2:
        raise ValueError("expected a 2-D array")
    if a.strides[1] != a.itemsize or a.strides[0] % a.itemsize or a.strides[0] < a.shape[1] * a.itemsize:
        a = np.ascontiguousarray(a)
    return a


def _ld(a: np.ndarray) -> int:
    return a.strides[0] // a.itemsize


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _sel(idx, n):
    if idx is None:
        idx = np.arange(n, dtype=np.int64)
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int64))
    if idx.size and (idx.min() < 0 or idx.max() >= n):
        raise IndexError("row/column selection out of range")
    return idx


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS, else all cores)."""
    return int(_load().orc_num_threads())


# ---------------------------------------------------------------------------
# element formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.orc_bf16_to_f64(int(x)) for x in b], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_e4m3_to_f64(c) for c in range(256)], dtype=np.float64)


def e2m1_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_e2m1_to_f64(c) for c in range(16)], dtype=np.float64)


def ue8m0_table() -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_ue8m0_to_f64(c) for c in range(256)], dtype=np.float64)


def bf16_rne(x) -> np.ndarray:
    """fp64 -> bf16 bits (uint16), round to nearest even, one rounding."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f64_to_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


# ---------------------------------------------------------------------------
# packed UE8M0 scales
# ---------------------------------------------------------------------------

def pack_scales(sf, ld_packed: int | None = None) -> np.ndarray:
    """uint8 [mn][kb] -> int16 [ceil(kb/2)][ld_packed] (MN-major), padding columns
    beyond mn left at 0."""
    sf = _c2d(sf, np.uint8)
    mn, kb = sf.shape
    ldp = mn if ld_packed is None else int(ld_packed)
    out = np.zeros(((kb + 1) // 2, ldp), dtype=np.int16)
    _load().orc_pack_scales(_ptr(sf), mn, kb, _ld(sf), _ptr(out), ldp)
    return out


def unpack_scales(packed, mn: int, kb: int) -> np.ndarray:
    packed = _c2d(packed, np.int16)
    if packed.shape[0] < (kb + 1) // 2 or packed.shape[1] < mn:
        raise ValueError("packed array too small")
    out = np.zeros((mn, kb), dtype=np.uint8)
    _load().orc_unpack_scales(_ptr(packed), mn, kb, _ld(packed), _ptr(out), kb)
    return out


def scale_byte(packed, mn: int, kb: int) -> int:
    packed = _c2d(packed, np.int16)
    return int(_load().orc_scale_byte(_ptr(packed), _ld(packed), mn, kb))


# ---------------------------------------------------------------------------
# GEMMs: return fp64 D[rows][:, cols]
# ---------------------------------------------------------------------------

def _run(fn, args, rows, cols):
    out = np.empty((rows.size, cols.size), dtype=np.float64)
    rc = fn(*args, rows.ctypes.data_as(_i64p), rows.size, cols.ctypes.data_as(_i64p),
            cols.size, out.ctypes.data_as(_f64p))
    if rc != 0:
        raise MemoryError("oracle ran out of memory")
    return out


def gemm_bf16(A, B, rows=None, cols=None) -> np.ndarray:
    """A bf16 bits uint16 [M][K], B uint16 [N][K]."""
    A = _c2d(A, np.uint16)
    B = _c2d(B, np.uint16)
    if A.shape[1] != B.shape[1]:
        raise ValueError("K mismatch")
    K = A.shape[1]
    rows = _sel(rows, A.shape[0])
    cols = _sel(cols, B.shape[0])
    return _run(_load().orc_gemm_bf16, (_ptr(A), _ld(A), _ptr(B), _ld(B), K), rows, cols)


def gemm_fp8(A, sfa, B, sfb, rows=None, cols=None, sfb_gran_mn: int = 128) -> np.ndarray:
    """A e4m3 codes uint8 [M][K], sfa packed int16 [ceil(K/256)][>=M];
    B uint8 [N][K], sfb packed int16 [ceil(K/256)][>=ceil(N/sfb_gran_mn)]: one scale
    per 128x128 block of B (sfb_gran_mn = 128) or per row and 128-wide K-block (1)."""
    A = _c2d(A, np.uint8)
    B = _c2d(B, np.uint8)
    sfa = _c2d(sfa, np.int16)
    sfb = _c2d(sfb, np.int16)
    K = A.shape[1]
    if B.shape[1] != K or K % 128:
        raise ValueError("bad K")
    if sfb_gran_mn not in (1, 128):
        raise ValueError("sfb_gran_mn must be 1 or 128")
    kp = (K // 128 + 1) // 2
    if sfa.shape[0] < kp or sfa.shape[1] < A.shape[0] or sfb.shape[0] < kp or \
            sfb.shape[1] < (B.shape[0] + sfb_gran_mn - 1) // sfb_gran_mn:
        raise ValueError("scale array too small")
    rows = _sel(rows, A.shape[0])
    cols = _sel(cols, B.shape[0])
    return _run(_load().orc_gemm_fp8, (_ptr(A), _ld(A), _ptr(sfa), _ld(sfa), _ptr(B), _ld(B),
                                       _ptr(sfb), _ld(sfb), sfb_gran_mn, K), rows, cols)


def gemm_fp4(A, sfa, B, sfb, K: int, rows=None, cols=None) -> np.ndarray:
    """A uint8 [M][K/2] (even k in the low nibble), sfa packed int16
    [ceil(K/64)][>=M]; B uint8 [N][K/2], sfb packed int16 [ceil(K/64)][>=N]."""
    A = _c2d(A, np.uint8)
    B = _c2d(B, np.uint8)
    sfa = _c2d(sfa, np.int16)
    sfb = _c2d(sfb, np.int16)
    if K % 32 or A.shape[1] * 2 < K or B.shape[1] * 2 < K:
        raise ValueError("bad K")
    kp = (K // 32 + 1) // 2
    if sfa.shape[0] < kp or sfa.shape[1] < A.shape[0] or sfb.shape[0] < kp or \
            sfb.shape[1] < B.shape[0]:
        raise ValueError("scale array too small")
    rows = _sel(rows, A.shape[0])
    cols = _sel(cols, B.shape[0])
    return _run(_load().orc_gemm_fp4, (_ptr(A), _ld(A), _ptr(sfa), _ld(sfa), _ptr(B), _ld(B),
                                       _ptr(sfb), _ld(sfb), K), rows, cols)


def grouped_fp8(A, sfa, B, sfb, offsets, rows=None, cols=None) -> np.ndarray:
    """A uint8 [M_total][K], sfa packed int16 [ceil(K/256)][>=M_total];
    B uint8 [G][N][K], sfb packed int16 [G][ceil(K/256)][>=ceil(N/128)];
    offsets int32 [G+1].  Rows outside every group come back as NaN."""
    A = _c2d(A, np.uint8)
    sfa = _c2d(sfa, np.int16)
    B = np.asarray(B)
    sfb = np.asarray(sfb)
    if B.ndim != 3 or sfb.ndim != 3:
        raise ValueError("B and sfb must be [G][..][..]")
    B = np.ascontiguousarray(B.view(np.uint8))
    sfb = np.ascontiguousarray(sfb.view(np.int16))
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32))
    G, N, K = B.shape
    if off.size != G + 1 or A.shape[1] != K or K % 128:
        raise ValueError("bad shapes")
    rows = _sel(rows, A.shape[0])
    cols = _sel(cols, N)
    return _run(_load().orc_grouped_fp8,
                (_ptr(A), _ld(A), _ptr(sfa), _ld(sfa), _ptr(B), K, N * K,
                 _ptr(sfb), sfb.shape[2], sfb.shape[1] * sfb.shape[2], _ptr(off), G, K),
                rows, cols)


def _expert_rows(offsets, rows):
    off = np.asarray(offsets, dtype=np.int64)
    g = np.searchsorted(off, rows, side="right") - 1
    inside = (rows >= off[0]) & (rows < off[-1])
    return np.where(inside, g, -1)


def grouped_bf16(A, B, offsets, rows=None, cols=None) -> np.ndarray:
    """M-grouped BF16 GEMM: rows [off[g], off[g+1]) of A (bf16 bits uint16
    [M_total][K]) multiply B[g] (uint16 [G][N][K]).  Rows outside every group
    come back as NaN."""
    A = _c2d(A, np.uint16)
    B = np.asarray(B)
    rows = _sel(rows, A.shape[0])
    cols = _sel(cols, B.shape[1])
    out = np.full((rows.size, cols.size), np.nan)
    g_of = _expert_rows(offsets, rows)
    for g in np.unique(g_of[g_of >= 0]):
        sel = np.nonzero(g_of == g)[0]
        out[sel] = gemm_bf16(A, B[g], rows=rows[sel], cols=cols)
    return out


def grouped_fp4(A, sfa, B, sfb, offsets, K: int, rows=None, cols=None) -> np.ndarray:
    """M-grouped FP4 GEMM: rows [off[g], off[g+1]) of A (uint8 [M_total][K/2],
    sfa packed [ceil(K/64)][>=M_total]) multiply B[g] (uint8 [G][N][K/2], sfb
    packed [G][ceil(K/64)][>=N]).  Rows outside every group come back as NaN."""
    A = _c2d(A, np.uint8)
    B = np.asarray(B)
    sfb = np.asarray(sfb)
    rows = _sel(rows, A.shape[0])
    cols = _sel(cols, B.shape[1])
    out = np.full((rows.size, cols.size), np.nan)
    g_of = _expert_rows(offsets, rows)
    for g in np.unique(g_of[g_of >= 0]):
        sel = np.nonzero(g_of == g)[0]
        out[sel] = gemm_fp4(A, sfa, B[g], sfb[g], K, rows=rows[sel], cols=cols)
    return out


def masked_fp8(A, sfa, B, sfb, masked_m, max_m: int, rows=None, cols=None) -> np.ndarray:
    """Masked M-grouped FP8 GEMM.  Expert g owns rows [g*max_m, (g+1)*max_m) of A
    (uint8 [G*max_m][K]) and of D; the first m_g = min(max(masked_m[g], 0), max_m)
    of them are computed as A_row x B[g]^T (B uint8 [G][N][K], sfb packed
    [G][ceil(K/256)][>=ceil(N/128)]; sfa packed over all G*max_m rows).  Rows
    past m_g come back as NaN."""
    A = _c2d(A, np.uint8)
    B = np.asarray(B)
    sfb = np.asarray(sfb)
    G = B.shape[0]
    m = np.clip(np.asarray(masked_m, dtype=np.int64), 0, max_m)
    rows = _sel(rows, G * max_m)
    cols = _sel(cols, B.shape[1])
    out = np.full((rows.size, cols.size), np.nan)
    g_of = rows // max_m
    valid = (rows - g_of * max_m) < m[g_of]
    for g in np.unique(g_of[valid]):
        sel = np.nonzero(valid & (g_of == g))[0]
        out[sel] = gemm_fp8(A, sfa, B[g], sfb[g], rows=rows[sel], cols=cols)
    return out


def row_norms(fmt: str, data, sf=None, K: int | None = None, rows=None,
              gran_mn: int = 1) -> np.ndarray:
    """Euclidean norms of dequantised rows.  fmt in {'bf16', 'e4m3', 'e2m1'}."""
    code = {"bf16": 0, "e4m3": 1, "e2m1": 2}[fmt]
    dt = np.uint16 if fmt == "bf16" else np.uint8
    data = _c2d(data, dt)
    if K is None:
        K = data.shape[1] * (2 if fmt == "e2m1" else 1)
    gran_k = {"bf16": 1, "e4m3": 128, "e2m1": 32}[fmt]
    if sf is None:
        if fmt != "bf16":
            raise ValueError("scales required")
        sfp, ldsf = ctypes.c_void_p(0), 0
    else:
        sf = _c2d(sf, np.int16)
        sfp, ldsf = _ptr(sf), _ld(sf)
    rows = _sel(rows, data.shape[0])
    out = np.empty(rows.size, dtype=np.float64)
    rc = _load().orc_norms(code, _ptr(data), _ld(data), sfp, ldsf, gran_mn, gran_k, K,
                           rows.ctypes.data_as(_i64p), rows.size, out.ctypes.data_as(_f64p))
    if rc != 0:
        raise MemoryError("oracle ran out of memory")
    return out
