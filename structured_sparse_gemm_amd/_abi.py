"""ctypes binding of libssgemm.so (include/ssgemm.h).  Loading only: no
arithmetic, no fallback.  If the library is missing it is built once with
hipcc; if that fails the import of any binding raises."""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libssgemm.so")

SSG_OK, SSG_ERR_NULL, SSG_ERR_SHAPE, SSG_ERR_STRIDE, SSG_ERR_DTYPE = 0, 1, 2, 3, 4
SSG_ERR_FORMAT, SSG_ERR_WORKSPACE, SSG_ERR_HIP, SSG_ERR_ALGO = 5, 6, 7, 8
SSG_F16, SSG_BF16, SSG_I8, SSG_F32, SSG_I32, SSG_E4M3, SSG_E5M2, SSG_I4 = 0, 1, 2, 3, 4, 5, 6, 7
SSG_ALGO_AUTO, SSG_ALGO_GENERIC, SSG_ALGO_SMALL_N, SSG_ALGO_LARGE_N = 0, 1, 2, 3

_i = ctypes.c_int
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/ssgemm.h
SIGNATURES = {
    "ssg_abi_version": (_i, []),
    "ssg_status_str": (ctypes.c_char_p, [_i]),
    "ssg_last_error": (ctypes.c_char_p, []),
    "ssg_vals_cols": (_i64, [_i64]),
    "ssg_meta_cols": (_i64, [_i64]),
    "ssg_prune_2to4": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    "ssg_compress_2to4": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "ssg_decompress_2to4": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "ssg_split_count": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _vp]),
    "ssg_split_fill": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp]),
    "ssg_spmm_workspace_bytes": (_sz, [_i, _i64, _i64, _i64]),
    "ssg_spmm_2to4": (_i, [_i, _i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "ssg_spmm_2to4_residual": (_i, [_i, _i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64,
                                    _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "ssg_spmm_2to4_ex": (_i, [_i, _i, _i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64,
                              _vp, _sz, _vp]),
    "ssg_spmm_2to4_residual_ex": (_i, [_i, _i, _i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp,
                                       _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "ssg_residual_delta_count": (_i, [_i64, _i64, _vp, _vp, _i64, _vp, _vp]),
    "ssg_residual_delta_fill": (_i, [_i, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp]),
    "ssg_spmm_2to4_residual_delta": (_i, [_i, _i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64,
                                          _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "ssg_spmm_2to4_residual_delta_ex": (_i, [_i, _i, _i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp,
                                             _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "ssg_spmm_csr": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "ssg_spmm_csr_delta": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "ssg_packed_sizes": (_i, [_i, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "ssg_pack_2to4_decode": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp]),
    "ssg_spmm_2to4_packed": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "ssg_spmm_2to4_packed_bt": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "ssg_spmm_2to4_packed_residual": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                           _i64, _vp]),
    "ssg_spmm_2to4_packed_residual_delta": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64,
                                                 _vp, _i64, _vp]),
    "ssg_prefill_packed_sizes": (_i, [_i, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "ssg_compress_2to4_prefill": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
    "ssg_pack_2to4_prefill": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp]),
    "ssg_spmm_2to4_prefill": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "ssg_spmm_2to4_prefill_bt": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "ssg_nm_vals_cols": (_i64, [_i, _i, _i64]),
    "ssg_compress_nm": (_i, [_i, _i, _i, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "ssg_decompress_nm": (_i, [_i, _i, _i, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "ssg_spmm_nm": (_i, [_i, _i, _i, _i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "ssg_nm_packed_sizes": (_i, [_i, _i, _i, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "ssg_pack_nm_decode": (_i, [_i, _i, _i, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _vp]),
    "ssg_spmm_nm_packed": (_i, [_i, _i, _i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "ssg_noalloc_scratch_bytes": (_i64, []),
    "ssg_spmm_2to4_noalloc": (_i, [_i, _i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp]),
    "ssg_cbm_sizes": (_i, [_i, _i64, _i64, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "ssg_pack_residual_cbm": (_i, [_i, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp]),
    "ssg_spmm_2to4_packed_residual_cbm": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                               _i64, _vp]),
    "ssg_spmm_2to4_packed_residual_cbm_bt": (_i, [_i, _i, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64,
                                                  _vp, _i64, _vp]),
    "ssg_stream_read_sink_words": (_i64, [_i64]),
    "ssg_stream_read": (_i, [_vp, _i64, _vp, _vp]),
    "ssg_mfma_probe_forms": (_i, []),
    "ssg_mfma_probe_name": (ctypes.c_char_p, [_i]),
    "ssg_mfma_probe_ops": (_i64, [_i, _i64, _i64]),
    "ssg_mfma_probe": (_i, [_i, _i64, _i64, _vp, _vp]),
    "ssg_lds_read_probe": (_i, [_vp, _i64, _i64, _vp, _vp]),
    "ssg_spmm_select_algo": (_i, [_i, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64]),
}

_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH):
    """The loaded library (built once with hipcc if absent)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(path):
                from . import build as _build
                _build.build()
            lib = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            if lib.ssg_abi_version() != 1:
                raise RuntimeError("libssgemm ABI version %d, expected 1" % lib.ssg_abi_version())
            _lib = lib
    return _lib
