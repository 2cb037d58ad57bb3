"""CPU oracle for 2:4 structured-sparse compression and SpMM (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline leg may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64/int64 accumulation, see
its header for the passages of the pages it follows).  This module only
builds it with gcc, loads it with ctypes and marshals numpy arrays:

* fp16 / bf16 matrices are passed as ``numpy.uint16`` arrays of raw bits;
* int8 matrices as ``numpy.int8``; 8-bit floats as ``numpy.uint8`` bits;
* dtype names are ``"f16"``, ``"bf16"``, ``"i8"``, ``"e4m3"`` and ``"e5m2"``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the oracle at another build of oracle.c (a copy with a
# planted mistake) to show that the pins catch it.
_OVERRIDE = os.environ.get("SSG_ORACLE_LIB")

DTYPES = {"f16": 0, "bf16": 1, "i8": 2, "e4m3": 3, "e5m2": 4, "i4": 5}
ERRORS = {
    -1: "null pointer", -2: "bad shape", -3: "bad stride", -4: "bad dtype",
    -5: "non-finite input", -6: "bad format", -7: "out of memory", -8: "out of range",
}

_lock = threading.Lock()
_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP over rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(_HDR)
    ):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if _OVERRIDE:
                lib = ctypes.CDLL(_OVERRIDE)
            else:
                build()
                lib = ctypes.CDLL(_LIB)
            lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
            lib.orc_f16_to_f64.restype = ctypes.c_double
            lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
            lib.orc_bf16_to_f64.restype = ctypes.c_double
            lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
            lib.orc_e4m3_to_f64.restype = ctypes.c_double
            lib.orc_e5m2_to_f64.argtypes = [ctypes.c_uint8]
            lib.orc_e5m2_to_f64.restype = ctypes.c_double
            lib.orc_select_group.argtypes = [_vp, _vp]
            lib.orc_select_group.restype = None
            lib.orc_compress.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
            lib.orc_prune.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _i64]
            lib.orc_decompress.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64]
            lib.orc_decompress.restype = _i64
            lib.orc_split_count.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, _vp]
            lib.orc_split_fill.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                           _vp, _vp, _vp]
            lib.orc_spmm.argtypes = [ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                                     _vp, _vp, _vp, _i64]
            lib.orc_spmm_residual.argtypes = [ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                              _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _i64]
            lib.orc_spmm_entries.argtypes = [ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                             _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp, _vp]
            lib.orc_delta_count.argtypes = [_i64, _i64, _vp, _vp, _vp]
            lib.orc_delta_fill.argtypes = [ctypes.c_int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
            lib.orc_spmm_residual_delta.argtypes = lib.orc_spmm_residual.argtypes
            lib.orc_spmm_entries_delta.argtypes = lib.orc_spmm_entries.argtypes
            lib.orc_select_nm.argtypes = [ctypes.c_int, ctypes.c_int, _vp, _vp]
            lib.orc_select_nm.restype = None
            lib.orc_compress_nm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64, _vp, _i64, _vp,
                                            _i64, _vp, _i64]
            lib.orc_decompress_nm.argtypes = lib.orc_compress_nm.argtypes
            lib.orc_decompress_nm.restype = _i64
            lib.orc_spmm_nm.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp,
                                        _i64, _vp, _i64, _vp, _vp, _vp, _i64]
            lib.orc_spmm_nm_w4a16.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64,
                                              _vp, _i64, _vp, _vp, _i64]
            lib.orc_i4_to_f64.argtypes = [ctypes.c_uint8, ctypes.c_int]
            lib.orc_i4_to_f64.restype = ctypes.c_double
            lib.orc_spmm_csr.argtypes = [ctypes.c_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                                         _i64]
            lib.orc_num_threads.restype = ctypes.c_int
            lib.orc_cbm_sizes.argtypes = [ctypes.c_int, _i64, _i64, _vp, _vp]
            lib.orc_cbm_encode.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
            lib.orc_cbm_decode.argtypes = [ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
            lib.orc_set_num_threads.argtypes = [ctypes.c_int]
            lib.orc_set_num_threads.restype = None
            _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str) -> None:
    if rc < 0:
        raise OracleError("%s: %s (%d)" % (what, ERRORS.get(rc, "error"), rc))


def _p(a):
    return None if a is None else a.ctypes.data_as(_vp)


def _store_dtype(dt: str):
    if dt not in DTYPES:
        raise OracleError("unknown dtype %r" % (dt,))
    return np.int8 if dt == "i8" else (np.uint8 if dt in ("e4m3", "e5m2", "i4") else np.uint16)


def _mat(a, dt: str) -> np.ndarray:
    a = np.asarray(a)
    want = _store_dtype(dt)
    if a.dtype != want or a.ndim != 2:
        raise OracleError("expected a 2-D %s array for %s, got %s %s" % (want.__name__, dt, a.dtype, a.shape))
    # keep the caller's row stride when rows are contiguous; otherwise copy
    if a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        a = np.ascontiguousarray(a)
    return a


def _ld(a: np.ndarray) -> int:
    return a.strides[0] // a.itemsize if a.shape[0] > 1 else a.shape[1]


def meta_cols(K: int) -> int:
    return (K + 7) // 8


def f16_to_f64(bits: int) -> float:
    return _load().orc_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return _load().orc_bf16_to_f64(int(bits))


def e4m3_to_f64(bits: int) -> float:
    return _load().orc_e4m3_to_f64(int(bits))


def e5m2_to_f64(bits: int) -> float:
    return _load().orc_e5m2_to_f64(int(bits))


def select_group(mag) -> list:
    """keep flags (0/1) of the top-2 rule for four magnitudes."""
    m = np.ascontiguousarray(np.asarray(mag, dtype=np.float64).reshape(4))
    keep = np.zeros(4, dtype=np.int32)
    _load().orc_select_group(_p(m), _p(keep))
    return [int(x) for x in keep]


def compress(dt: str, A):
    A = _mat(A, dt)
    M, K = A.shape
    vals = np.zeros((M, K // 2), dtype=A.dtype)
    meta = np.zeros((M, meta_cols(K)), dtype=np.uint8)
    _check(_load().orc_compress(DTYPES[dt], M, K, _p(A), _ld(A), _p(vals), max(K // 2, 1), _p(meta),
                                max(meta_cols(K), 1)), "compress")
    return vals, meta


def prune(dt: str, A):
    A = _mat(A, dt)
    M, K = A.shape
    P = np.zeros((M, K), dtype=A.dtype)
    _check(_load().orc_prune(DTYPES[dt], M, K, _p(A), _ld(A), _p(P), max(K, 1)), "prune")
    return P


def decompress(dt: str, vals, meta, K: int):
    """Returns (D, number of groups with an invalid nibble)."""
    vals = _mat(vals, dt)
    meta = np.ascontiguousarray(np.asarray(meta, dtype=np.uint8))
    M = vals.shape[0]
    D = np.zeros((M, K), dtype=vals.dtype)
    bad = _load().orc_decompress(DTYPES[dt], M, K, _p(vals), max(vals.shape[1], 1), _p(meta),
                                 max(meta.shape[1], 1), _p(D), max(K, 1))
    _check(bad, "decompress")
    return D, int(bad)


def split(dt: str, A):
    """2:4 layer plus CSR residual of the dropped non-zeros: (vals, meta, row_ptr, col, rvals)."""
    A = _mat(A, dt)
    M, K = A.shape
    lib = _load()
    row_ptr = np.zeros(M + 1, dtype=np.int32)
    _check(lib.orc_split_count(DTYPES[dt], M, K, _p(A), _ld(A), _p(row_ptr)), "split_count")
    nnz = int(row_ptr[M])
    col = np.zeros(max(nnz, 1), dtype=np.int32)
    rvals = np.zeros(max(nnz, 1), dtype=A.dtype)
    vals = np.zeros((M, K // 2), dtype=A.dtype)
    meta = np.zeros((M, meta_cols(K)), dtype=np.uint8)
    _check(lib.orc_split_fill(DTYPES[dt], M, K, _p(A), _ld(A), _p(vals), max(K // 2, 1), _p(meta),
                              max(meta_cols(K), 1), _p(row_ptr), _p(col), _p(rvals)), "split_fill")
    return vals, meta, row_ptr, col[:nnz], rvals[:nnz]


def delta_encode(dt: str, row_ptr, col, rvals, K: int):
    """Delta-coded residual of a CSR (columns strictly ascending in [0, K)):
    (drow_ptr int32 [M+1], dcol uint8, dvals).  Entry j of a row stores its
    column as the byte col_j - col_(j-1), col_(-1) = -1; a gap above 255 is
    bridged by fillers (255, +0) in front of the entry."""
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    rvals = np.ascontiguousarray(rvals, dtype=_store_dtype(dt))
    M = row_ptr.shape[0] - 1
    lib = _load()
    drow_ptr = np.zeros(M + 1, dtype=np.int32)
    _check(lib.orc_delta_count(M, K, _p(row_ptr), _p(col) if col.size else None, _p(drow_ptr)), "delta_count")
    n = int(drow_ptr[M])
    dcol = np.zeros(max(n, 1), dtype=np.uint8)
    dvals = np.zeros(max(n, 1), dtype=_store_dtype(dt))
    _check(lib.orc_delta_fill(DTYPES[dt], M, K, _p(row_ptr), _p(col) if col.size else None,
                              _p(rvals) if rvals.size else None, _p(drow_ptr), _p(dcol), _p(dvals)), "delta_fill")
    return drow_ptr, dcol[:n], dvals[:n]


def _mm(dt, vals, meta, B, K, residual, delta=False):
    vals = _mat(vals, dt)
    B = _mat(B, dt)
    meta = np.ascontiguousarray(np.asarray(meta, dtype=np.uint8))
    M, N = vals.shape[0], B.shape[1]
    if B.shape[0] != K:
        raise OracleError("B has %d rows, K is %d" % (B.shape[0], K))
    lib = _load()
    if dt == "i8":
        C = np.zeros((M, N), dtype=np.int64)
        Cf, Ci, S = None, C, None
    else:
        C = np.zeros((M, N), dtype=np.float64)
        S = np.zeros((M, N), dtype=np.float64)
        Cf, Ci = C, None
    ldv, ldm, ldb = max(vals.shape[1], 1), max(meta.shape[1], 1), _ld(B) if K > 0 else max(N, 1)
    if residual is None:
        rc = lib.orc_spmm(DTYPES[dt], M, N, K, _p(vals), ldv, _p(meta), ldm, _p(B), ldb,
                          _p(Cf), _p(Ci), _p(S), max(N, 1))
    else:
        row_ptr, col, rvals = residual
        row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
        col = np.ascontiguousarray(col, dtype=np.uint8 if delta else np.int32)
        rvals = np.ascontiguousarray(rvals, dtype=_store_dtype(dt))
        fn = lib.orc_spmm_residual_delta if delta else lib.orc_spmm_residual
        rc = fn(DTYPES[dt], M, N, K, _p(vals), ldv, _p(meta), ldm, _p(row_ptr), _p(col), _p(rvals), _p(B), ldb,
                _p(Cf), _p(Ci), _p(S), max(N, 1))
    _check(rc, "spmm")
    return C, S


def spmm(dt: str, vals, meta, B, K: int):
    """C = decompress(vals, meta) @ B: (C fp64, S) for fp16/bf16, (C int64, None) for int8."""
    return _mm(dt, vals, meta, B, K, None)


def spmm_residual(dt: str, vals, meta, row_ptr, col, rvals, B, K: int):
    return _mm(dt, vals, meta, B, K, (row_ptr, col, rvals))


def spmm_csr(dt: str, row_ptr, col, vals, B, K: int):
    """C = S @ B for an unstructured sparse S given as CSR: (C fp64, S) or (C int64, None)."""
    B = _mat(B, dt)
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    vals = np.ascontiguousarray(vals, dtype=_store_dtype(dt))
    M, N = row_ptr.shape[0] - 1, B.shape[1]
    if B.shape[0] != K:
        raise OracleError("B has %d rows, K is %d" % (B.shape[0], K))
    if dt == "i8":
        C, S = np.zeros((M, N), dtype=np.int64), None
        Cf, Ci = None, C
    else:
        C, S = np.zeros((M, N), dtype=np.float64), np.zeros((M, N), dtype=np.float64)
        Cf, Ci = C, None
    _check(_load().orc_spmm_csr(DTYPES[dt], M, N, K, _p(row_ptr), _p(col) if col.size else None,
                                _p(vals) if vals.size else None, _p(B), _ld(B) if K > 0 else max(N, 1),
                                _p(Cf), _p(Ci), _p(S), max(N, 1)), "spmm_csr")
    return C, S


def spmm_residual_delta(dt: str, vals, meta, drow_ptr, dcol, dvals, B, K: int):
    """As spmm_residual with a delta-coded residual (see delta_encode)."""
    return _mm(dt, vals, meta, B, K, (drow_ptr, dcol, dvals), delta=True)


def cbm_sizes(dt: str, M: int, K: int):
    """(mask bytes, blocks) of the complement-bitmap residual layout; roff has blocks + 1 entries."""
    mb, nb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_load().orc_cbm_sizes(DTYPES[dt], M, K, ctypes.byref(mb), ctypes.byref(nb)), "cbm_sizes")
    return int(mb.value), int(nb.value)


def cbm_encode(dt: str, meta, row_ptr, col, rvals, M: int, K: int):
    """(rmask uint8, roff int32, cvals) of a CSR residual whose entries sit at
    the complement positions of the 2:4 layer (meta) -- see orc_cbm_encode."""
    mb, nb = cbm_sizes(dt, M, K)
    meta = np.ascontiguousarray(np.asarray(meta, dtype=np.uint8))
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    rvals = np.ascontiguousarray(rvals, dtype=_store_dtype(dt))
    nnz = int(row_ptr[M]) if M > 0 else 0
    rmask = np.zeros(max(mb, 1), dtype=np.uint8)
    roff = np.zeros(nb + 1, dtype=np.int32)
    cvals = np.zeros(max(nnz, 1), dtype=_store_dtype(dt))
    _check(_load().orc_cbm_encode(DTYPES[dt], M, K, _p(meta) if meta.size else None, max(meta.shape[-1], 1),
                                  _p(row_ptr), _p(col) if col.size else None, _p(rvals) if rvals.size else None,
                                  _p(rmask), _p(roff), _p(cvals)), "cbm_encode")
    return rmask[:mb], roff, cvals[:nnz]


def cbm_decode(dt: str, meta, rmask, roff, cvals, M: int, K: int):
    """The CSR (row_ptr, col, rvals) of a complement-bitmap residual."""
    meta = np.ascontiguousarray(np.asarray(meta, dtype=np.uint8))
    rmask = np.ascontiguousarray(rmask, dtype=np.uint8)
    roff = np.ascontiguousarray(roff, dtype=np.int32)
    cvals = np.ascontiguousarray(cvals, dtype=_store_dtype(dt))
    nnz = int(roff[-1])
    row_ptr = np.zeros(M + 1, dtype=np.int32)
    col = np.zeros(max(nnz, 1), dtype=np.int32)
    rv = np.zeros(max(nnz, 1), dtype=_store_dtype(dt))
    _check(_load().orc_cbm_decode(DTYPES[dt], M, K, _p(meta) if meta.size else None, max(meta.shape[-1], 1),
                                  _p(rmask) if rmask.size else None, _p(roff), _p(cvals) if cvals.size else None,
                                  _p(row_ptr), _p(col), _p(rv)), "cbm_decode")
    return row_ptr, col[:nnz], rv[:nnz]


def spmm_entries(dt: str, vals, meta, B, K: int, ms, ns, residual=None, delta: bool = False):
    """Outputs C[ms[e], ns[e]] (and their bounds) one by one.  `residual` is a
    CSR (row_ptr, col, rvals), or with delta=True a delta-coded
    (drow_ptr, dcol, dvals)."""
    vals = _mat(vals, dt)
    B = _mat(B, dt)
    meta = np.ascontiguousarray(np.asarray(meta, dtype=np.uint8))
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    M, N, E = vals.shape[0], B.shape[1], ms.shape[0]
    if dt == "i8":
        C, S, Cf, Ci = np.zeros(E, dtype=np.int64), None, None, None
        Ci = C
    else:
        C, S = np.zeros(E, dtype=np.float64), np.zeros(E, dtype=np.float64)
        Cf, Ci = C, None
    rp = col = rv = None
    if residual is not None:
        rp = np.ascontiguousarray(residual[0], dtype=np.int32)
        col = np.ascontiguousarray(residual[1], dtype=np.uint8 if delta else np.int32)
        rv = np.ascontiguousarray(residual[2], dtype=_store_dtype(dt))
    fn = _load().orc_spmm_entries_delta if delta else _load().orc_spmm_entries
    rc = fn(DTYPES[dt], M, N, K, _p(vals), max(vals.shape[1], 1), _p(meta),
                                  max(meta.shape[1], 1), _p(rp), _p(col), _p(rv), _p(B),
                                  _ld(B) if K > 0 else max(N, 1), E, _p(ms), _p(ns), _p(Cf), _p(Ci), _p(S))
    _check(rc, "spmm_entries")
    return C, S


def select_nm(n: int, m: int, mag) -> list:
    """keep flags (0/1) of the top-n rule for m magnitudes."""
    g = np.ascontiguousarray(np.asarray(mag, dtype=np.float64).reshape(m))
    keep = np.zeros(m, dtype=np.int32)
    _load().orc_select_nm(n, m, _p(g), _p(keep))
    return [int(x) for x in keep]


def i4_to_f64(byte: int, high: bool) -> float:
    return _load().orc_i4_to_f64(int(byte), int(bool(high)))


def _per(dt: str) -> int:
    """Elements per storage unit: 2 for 4-bit integers (two per byte), else 1."""
    return 2 if dt == "i4" else 1


def compress_nm(dt: str, n: int, m: int, A):
    """N:M compressed form of A: (vals [M, K/m*n], mask uint8 [M, ceil(K/8)]);
    mask bit k % 8 of byte k / 8 is set iff element k is kept.  For "i4" the
    arrays hold two elements per byte (A [M, K/2], vals [M, K/m*n/2])."""
    A = _mat(A, dt)
    e = _per(dt)
    M, K = A.shape[0], A.shape[1] * e
    vc = K // m * n if m > 0 else 0
    vals = np.zeros((M, -(-vc // e)), dtype=A.dtype)
    mask = np.zeros((M, meta_cols(K)), dtype=np.uint8)
    _check(_load().orc_compress_nm(DTYPES[dt], n, m, M, K, _p(A), _ld(A) * e, _p(vals), max(vals.shape[1] * e, e),
                                   _p(mask), max(meta_cols(K), 1)), "compress_nm")
    return vals, mask


def decompress_nm(dt: str, n: int, m: int, vals, mask, K: int):
    """(D, number of groups whose mask does not hold exactly n bits)."""
    vals = _mat(vals, dt)
    e = _per(dt)
    mask = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))
    M = vals.shape[0]
    D = np.zeros((M, -(-K // e)), dtype=vals.dtype)
    bad = _load().orc_decompress_nm(DTYPES[dt], n, m, M, K, _p(vals), max(vals.shape[1] * e, e), _p(mask),
                                    max(mask.shape[1], 1), _p(D), max(D.shape[1] * e, e))
    _check(bad, "decompress_nm")
    return D, int(bad)


def spmm_nm(dt: str, n: int, m: int, vals, mask, B, K: int):
    """C = decompress_nm(vals, mask) @ B: (C fp64, S) for floats, (C int64, None) for int8.
    For "i4" weights B is fp16 (raw uint16 bits)."""
    vals = _mat(vals, dt)
    if dt == "i4":
        B = _mat(B, "f16")
        mask = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))
        M, N = vals.shape[0], B.shape[1]
        if B.shape[0] != K:
            raise OracleError("B has %d rows, K is %d" % (B.shape[0], K))
        C, S = np.zeros((M, N), dtype=np.float64), np.zeros((M, N), dtype=np.float64)
        _check(_load().orc_spmm_nm_w4a16(n, m, M, N, K, _p(vals), max(vals.shape[1] * 2, 2), _p(mask),
                                         max(mask.shape[1], 1), _p(B), _ld(B) if K > 0 else max(N, 1), _p(C), _p(S),
                                         max(N, 1)), "spmm_nm_w4a16")
        return C, S
    B = _mat(B, dt)
    mask = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8))
    M, N = vals.shape[0], B.shape[1]
    if B.shape[0] != K:
        raise OracleError("B has %d rows, K is %d" % (B.shape[0], K))
    if dt == "i8":
        C, S = np.zeros((M, N), dtype=np.int64), None
        Cf, Ci = None, C
    else:
        C, S = np.zeros((M, N), dtype=np.float64), np.zeros((M, N), dtype=np.float64)
        Cf, Ci = C, None
    _check(_load().orc_spmm_nm(DTYPES[dt], n, m, M, N, K, _p(vals), max(vals.shape[1], 1), _p(mask),
                               max(mask.shape[1], 1), _p(B), _ld(B) if K > 0 else max(N, 1), _p(Cf), _p(Ci),
                               _p(S), max(N, 1)), "spmm_nm")
    return C, S


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (timing only)."""
    _load().orc_set_num_threads(int(n))
