"""Python front of the CPU oracle (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It wraps ``liboracle.so`` (plain C, built by
``oracle/build.py`` with gcc) through ctypes and works on numpy arrays of raw
fp16/bf16 bit patterns (``uint16``) and E4M3/E5M2/E8M0 bytes (``uint8``), so
that the oracle consumes exactly the bits the GPU consumes.  Nothing here
imports the GPU library.

What each call computes is documented in ``gemm_oracle.c``; the sources are
the NineToothed GEMM primer (studypath task3 appendix, s3-s6, s8) for the
definition, index map, tail masks and accumulator precision, and the Croqtile
tutorial ch.4 ([N,K] right operand) for the TN form and for the FP8 operands
with per-tile scales.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

# The oracle's own format codes (see gemm_oracle.c).
FMT = {"f16": 0, "bf16": 1, "f32": 2, "f64": 3, "e4m3": 4, "e5m2": 5}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from oracle import build as _b  # compiled only when nothing is built
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.orc_decode.restype = ctypes.c_double
    lib.orc_decode.argtypes = [ctypes.c_int, ctypes.c_uint16]
    lib.orc_encode.restype = ctypes.c_uint16
    lib.orc_encode.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.orc_decode_array.restype = None
    lib.orc_decode_array.argtypes = [ctypes.c_int, p, p, i64]
    lib.orc_encode_array.restype = None
    lib.orc_encode_array.argtypes = [ctypes.c_int, p, p, i64]
    lib.orc_gemm.restype = ctypes.c_int
    lib.orc_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                             p, i64, i64, p, i64, i64, p, i64, i64, i64,
                             p, i64, ctypes.c_int]
    lib.orc_tiled_gemm.restype = ctypes.c_int
    lib.orc_tiled_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64,
                                   p, i64, p, i64, i64, i64, i64,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, p, i64]
    lib.orc_tile_geometry.restype = ctypes.c_int
    lib.orc_tile_geometry.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, i64, p]
    lib.orc_decode_f8.restype = ctypes.c_double
    lib.orc_decode_f8.argtypes = [ctypes.c_int, ctypes.c_uint8]
    lib.orc_decode_e8m0.restype = ctypes.c_double
    lib.orc_decode_e8m0.argtypes = [ctypes.c_uint8]
    lib.orc_decode_f8_array.restype = None
    lib.orc_decode_f8_array.argtypes = [ctypes.c_int, p, p, i64]
    lib.orc_decode_e8m0_array.restype = None
    lib.orc_decode_e8m0_array.argtypes = [p, p, i64]
    lib.orc_gemm_f8.restype = ctypes.c_int
    lib.orc_gemm_f8.argtypes = [i64, i64, i64, p, i64, ctypes.c_int, p, i64, ctypes.c_int,
                                p, i64, p, i64, i64, p, i64, p, i64, p, i64, ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bits(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are uint16 bit patterns, got %s" % a.dtype)
    return a


def decode(bits, fmt: str) -> np.ndarray:
    """fp16/bf16 bit patterns -> exact float64 values."""
    b = np.ascontiguousarray(_bits(bits))
    out = np.empty(b.shape, dtype=np.float64)
    _load().orc_decode_array(FMT[fmt], _ptr(b), _ptr(out), b.size)
    return out


def encode(x, fmt: str) -> np.ndarray:
    """float64 values -> fp16/bf16 bit patterns, round-to-nearest-even."""
    v = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_encode_array(FMT[fmt], _ptr(v), _ptr(out), v.size)
    return out


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def gemm(a_bits, b_bits, fmt: str, layout: str = "nn", rows=None, nthreads=None) -> np.ndarray:
    """Plain-definition product in float64.

    ``a_bits``: (M, K) or (batch, M, K) uint16.  ``b_bits``: (K, N) for
    ``layout='nn'`` or (N, K) for ``'tn'`` (C = A B^T), optionally batched.
    Row-major with any row stride (numpy strides in elements are honoured for
    the row dimension; the last dimension must be contiguous).  ``rows``
    restricts the output to the listed rows of every batch entry.
    Returns float64 (batch?, len(rows) or M, N).
    """
    a = _bits(a_bits)
    b = _bits(b_bits)
    batched = a.ndim == 3
    if not batched:
        a = a[None]
        b = b[None]
    if a.ndim != 3 or b.ndim != 3 or a.shape[0] != b.shape[0]:
        raise ValueError("shape mismatch")
    transb = {"nn": 0, "tn": 1}[layout]
    batch, M, K = a.shape
    if transb:
        N, K2 = b.shape[1], b.shape[2]
    else:
        K2, N = b.shape[1], b.shape[2]
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if rows is None:
        rows_arr = None
        nrows = M
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    c = np.zeros((batch, nrows, N), dtype=np.float64)
    nt = nthreads or default_threads()
    rc = _load().orc_gemm(transb, FMT[fmt], M, N, K,
                          _ptr(a), K, M * K, _ptr(b), b.shape[2], b.shape[1] * b.shape[2],
                          _ptr(c), N, nrows * N, batch,
                          _ptr(rows_arr) if rows_arr is not None else None, nrows, nt)
    if rc != 0:
        raise ValueError("orc_gemm failed with %d" % rc)
    return c if batched else c[0]


def gemm_raw(transb, fmt_code, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, batch,
             rows=None, nrows=0, nthreads=1) -> int:
    """Direct call with explicit strides (argument-checking tests)."""
    return _load().orc_gemm(transb, fmt_code, M, N, K, A, lda, sA, B, ldb, sB,
                            C, ldc, sC, batch, rows, nrows, nthreads)


def tiled_gemm(a_bits, b_bits, fmt: str, layout: str = "nn", BM=64, BN=64, BK=64,
               acc: str = "f64", out: str = "f64", drop_last_k: bool = False,
               c_init=None) -> np.ndarray:
    """The tiled algorithm (masked tile reads, per-program accumulator,
    masked store).  ``acc`` is the accumulator precision, ``out`` the
    rounding of the stored value.  ``c_init`` pre-fills C so that tests can
    see which elements the masked store leaves untouched."""
    a = np.ascontiguousarray(_bits(a_bits))
    b = np.ascontiguousarray(_bits(b_bits))
    transb = {"nn": 0, "tn": 1}[layout]
    M, K = a.shape
    N = b.shape[0] if transb else b.shape[1]
    c = np.zeros((M, N)) if c_init is None else np.array(c_init, dtype=np.float64, copy=True)
    rc = _load().orc_tiled_gemm(transb, FMT[fmt], M, N, K, _ptr(a), K, _ptr(b), b.shape[1],
                                BM, BN, BK, FMT[acc], FMT[out], int(drop_last_k), _ptr(c), N)
    if rc != 0:
        raise ValueError("orc_tiled_gemm failed with %d" % rc)
    return c


def tile_geometry(M, N, K, BM, BN, BK, i=0, j=0, p=0) -> dict:
    """Grid sizes and the tile ranges of program (i, j) at K step p."""
    g = np.zeros(27, dtype=np.int64)
    rc = _load().orc_tile_geometry(M, N, K, BM, BN, BK, i, j, p, _ptr(g))
    if rc != 0:
        raise ValueError("orc_tile_geometry failed with %d" % rc)
    r = [int(x) for x in g]
    return {
        "grid": (r[0], r[1]), "ksteps": r[2],
        "a_nominal": ((r[3], r[4]), (r[5], r[6])),
        "b_nominal": ((r[7], r[8]), (r[9], r[10])),
        "c_nominal": ((r[11], r[12]), (r[13], r[14])),
        "a_valid": ((r[15], r[16]), (r[17], r[18])),
        "b_valid": ((r[19], r[20]), (r[21], r[22])),
        "c_valid": ((r[23], r[24]), (r[25], r[26])),
    }


def _bytes(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint8:
        raise TypeError("8-bit oracle inputs are uint8 bit patterns, got %s" % a.dtype)
    return a


def decode_f8(bits, fmt: str) -> np.ndarray:
    """E4M3 / E5M2 bit patterns (uint8) -> exact float64 values."""
    b = np.ascontiguousarray(_bytes(bits))
    out = np.empty(b.shape, dtype=np.float64)
    _load().orc_decode_f8_array(FMT[fmt], _ptr(b), _ptr(out), b.size)
    return out


def decode_e8m0(bits) -> np.ndarray:
    """E8M0 scale bytes -> 2^(e - 127) (0xFF -> NaN)."""
    b = np.ascontiguousarray(_bytes(bits))
    out = np.empty(b.shape, dtype=np.float64)
    _load().orc_decode_e8m0_array(_ptr(b), _ptr(out), b.size)
    return out


def gemm_f8(a_bits, b_bits, a_fmt: str, b_fmt: str, xa=None, xb=None, sa=None, sb=None,
            block: int = 32, nthreads=None) -> np.ndarray:
    """Scaled 8-bit TN product in float64 (C = A B^T with scales).

    ``a_bits`` (M, K) and ``b_bits`` (N, K) uint8 patterns of ``a_fmt`` /
    ``b_fmt`` ("e4m3" | "e5m2").  ``xa`` (M, cdiv(K, block)) and ``xb``
    (N, cdiv(K, block)) are optional E8M0 block-scale bytes; ``sa`` (M,) or
    (1,) and ``sb`` (N,) or (1,) are optional float32 row scales (a length-1
    array is one scale for the whole operand).  Returns float64 (M, N).
    """
    a = np.ascontiguousarray(_bytes(a_bits))
    b = np.ascontiguousarray(_bytes(b_bits))
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("shape mismatch")
    M, K = a.shape
    N = b.shape[0]
    nb = (K + block - 1) // block

    def blk(x, rows):
        if x is None:
            return None, 0
        x = np.ascontiguousarray(_bytes(x))
        if x.shape != (rows, nb):
            raise ValueError("block scales must be (%d, %d), got %s" % (rows, nb, x.shape))
        return x, nb

    def row(x, rows):
        if x is None:
            return None, 0
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(-1))
        if x.size not in (1, rows):
            raise ValueError("row scales must have 1 or %d entries" % rows)
        return x, (0 if x.size == 1 else 1)

    xa_, ldxa = blk(xa, M)
    xb_, ldxb = blk(xb, N)
    sa_, inca = row(sa, M)
    sb_, incb = row(sb, N)
    c = np.zeros((M, N), dtype=np.float64)
    nt = nthreads or default_threads()
    keep = (xa_, xb_, sa_, sb_)  # noqa: F841  (alive across the call)
    rc = _load().orc_gemm_f8(M, N, K, _ptr(a), K, FMT[a_fmt], _ptr(b), K, FMT[b_fmt],
                             _ptr(xa_) if xa_ is not None else None, ldxa,
                             _ptr(xb_) if xb_ is not None else None, ldxb, block,
                             _ptr(sa_) if sa_ is not None else None, inca,
                             _ptr(sb_) if sb_ is not None else None, incb,
                             _ptr(c), N, nt)
    if rc != 0:
        raise ValueError("orc_gemm_f8 failed with %d" % rc)
    return c
