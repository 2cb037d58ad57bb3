"""structured_sparse_gemm_amd -- 2:4 structured-sparse weight x dense activation
matrix multiply for AMD Instinct MI355X (gfx950).

Every computation runs in the HIP kernels of libssgemm.so; this module only
marshals torch tensors (device memory and the current stream) into the C
ABI declared in include/ssgemm.h.  There is no CPU fallback: tensors must
live on a ROCm device and the library must load.

Same-named bindings of the C ABI (``ssg_compress_2to4`` ...) take
preallocated tensors; ``compress``, ``prune``, ``decompress``, ``split``,
``delta_encode``, ``spmm``, ``spmm_residual`` and ``spmm_residual_delta``
allocate their outputs.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _abi
from ._abi import (SSG_ALGO_AUTO, SSG_ALGO_GENERIC, SSG_ALGO_LARGE_N, SSG_ALGO_SMALL_N, SSG_BF16, SSG_F16,
                   SSG_F32, SSG_I8, SSG_I32)

__all__ = [
    "SsgError", "compress", "prune", "decompress", "split", "delta_encode", "spmm", "spmm_residual",
    "spmm_residual_delta", "vals_cols", "meta_cols",
    "ssg_prune_2to4", "ssg_compress_2to4", "ssg_decompress_2to4", "ssg_split_count", "ssg_split_fill",
    "ssg_residual_delta_count", "ssg_residual_delta_fill", "ssg_spmm_workspace_bytes", "ssg_spmm_2to4",
    "ssg_spmm_2to4_residual", "ssg_spmm_2to4_residual_delta", "ssg_spmm_select_algo", "ssg_spmm_csr",
    "ssg_spmm_csr_delta", "spmm_csr", "spmm_csr_delta", "ssg_packed_sizes", "ssg_pack_2to4_decode",
    "ssg_spmm_2to4_packed", "pack_decode", "spmm_packed",
    "ssg_spmm_2to4_packed_residual", "ssg_spmm_2to4_packed_residual_delta", "spmm_packed_residual",
    "spmm_packed_residual_delta",
    "ssg_prefill_packed_sizes", "ssg_compress_2to4_prefill", "ssg_pack_2to4_prefill", "ssg_spmm_2to4_prefill",
    "compress_prefill", "pack_prefill", "spmm_prefill",
    "ssg_compress_nm", "ssg_decompress_nm", "ssg_spmm_nm", "compress_nm", "decompress_nm", "spmm_nm",
    "ssg_nm_packed_sizes", "ssg_pack_nm_decode", "ssg_spmm_nm_packed", "pack_nm", "spmm_nm_packed",
    "ssg_noalloc_scratch_bytes", "ssg_spmm_2to4_noalloc",
    "ssg_cbm_sizes", "ssg_pack_residual_cbm", "ssg_spmm_2to4_packed_residual_cbm", "pack_residual_cbm",
    "spmm_packed_residual_cbm",
    "ssg_spmm_2to4_prefill_bt", "spmm_prefill_bt", "ssg_spmm_2to4_packed_bt", "spmm_packed_bt",
    "ssg_spmm_2to4_packed_residual_cbm_bt", "spmm_packed_residual_cbm_bt",
    "ssg_stream_read_sink_words", "ssg_stream_read",
    "ssg_mfma_probe_forms", "ssg_mfma_probe_name", "ssg_mfma_probe_ops", "ssg_mfma_probe", "ssg_lds_read_probe",
    "SSG_ALGO_AUTO", "SSG_ALGO_GENERIC", "SSG_ALGO_SMALL_N", "SSG_ALGO_LARGE_N", "library_path",
]

# torch.uint8 element tensors are 4-bit weights, two per byte (the N:M calls
# only; their element counts are twice the byte counts)
_DT = {torch.float16: SSG_F16, torch.bfloat16: SSG_BF16, torch.int8: SSG_I8,
       torch.float8_e4m3fn: _abi.SSG_E4M3, torch.float8_e5m2: _abi.SSG_E5M2, torch.uint8: _abi.SSG_I4}
_OUT = {SSG_F16: (SSG_F32, torch.float32), SSG_BF16: (SSG_F32, torch.float32), SSG_I8: (SSG_I32, torch.int32),
        _abi.SSG_E4M3: (SSG_F32, torch.float32), _abi.SSG_E5M2: (SSG_F32, torch.float32),
        _abi.SSG_I4: (SSG_F32, torch.float32)}


def _per(t: torch.Tensor) -> int:
    """Elements per storage unit of an element tensor: 2 for 4-bit weights."""
    return 2 if t.dtype == torch.uint8 else 1
ALGO_NAMES = {SSG_ALGO_AUTO: "auto", SSG_ALGO_GENERIC: "generic", SSG_ALGO_SMALL_N: "small_n",
              SSG_ALGO_LARGE_N: "large_n"}


class SsgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _abi.LIB_PATH


def _lib():
    return _abi.load()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        lib = _lib()
        raise SsgError(rc, "%s: %s (%s)" % (what, lib.ssg_status_str(rc).decode(), lib.ssg_last_error().decode()))


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise SsgError(_abi.SSG_ERR_DTYPE, "unsupported element type %s" % (t.dtype,))
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise SsgError(_abi.SSG_ERR_NULL, "%s must be a ROCm device tensor (got %s)" % (name, t.device))
    return t.data_ptr() if t.numel() > 0 else None


def _ld(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2:
        raise SsgError(_abi.SSG_ERR_SHAPE, "%s must be 2-D, got shape %s" % (name, tuple(t.shape)))
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise SsgError(_abi.SSG_ERR_STRIDE, "%s must have unit column stride" % name)
    return max(t.stride(0), t.shape[1]) if t.shape[0] > 1 else t.shape[1]


def _stream(t: torch.Tensor, stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return getattr(stream, "cuda_stream", stream) or None


def vals_cols(K: int) -> int:
    return int(_lib().ssg_vals_cols(K))


def meta_cols(K: int) -> int:
    return int(_lib().ssg_meta_cols(K))


# ---------------------------------------------------------------- same-named bindings

def ssg_prune_2to4(A: torch.Tensor, P: torch.Tensor, stream=None) -> None:
    M, K = A.shape
    _check(_lib().ssg_prune_2to4(_dtype(A), M, K, _ptr(A, "A"), _ld(A, "A"), _ptr(P, "P"), _ld(P, "P"),
                                 _stream(A, stream)), "ssg_prune_2to4")


def ssg_compress_2to4(A: torch.Tensor, vals: torch.Tensor, meta: torch.Tensor, stream=None) -> None:
    M, K = A.shape
    _check(_lib().ssg_compress_2to4(_dtype(A), M, K, _ptr(A, "A"), _ld(A, "A"), _ptr(vals, "vals"),
                                    _ld(vals, "vals"), _ptr(meta, "meta"), _ld(meta, "meta"), _stream(A, stream)),
           "ssg_compress_2to4")


def ssg_decompress_2to4(vals: torch.Tensor, meta: torch.Tensor, D: torch.Tensor,
                        bad_count: Optional[torch.Tensor] = None, stream=None) -> None:
    M, K = D.shape
    _check(_lib().ssg_decompress_2to4(_dtype(vals), M, K, _ptr(vals, "vals"), _ld(vals, "vals"),
                                      _ptr(meta, "meta"), _ld(meta, "meta"), _ptr(D, "D"), _ld(D, "D"),
                                      _ptr(bad_count, "bad_count"), _stream(D, stream)), "ssg_decompress_2to4")


def ssg_split_count(A: torch.Tensor, row_ptr: torch.Tensor, stream=None) -> None:
    M, K = A.shape
    _check(_lib().ssg_split_count(_dtype(A), M, K, _ptr(A, "A"), _ld(A, "A"), _ptr(row_ptr, "row_ptr"),
                                  _stream(A, stream)), "ssg_split_count")


def ssg_split_fill(A, vals, meta, row_ptr, col, rvals, stream=None) -> None:
    M, K = A.shape
    _check(_lib().ssg_split_fill(_dtype(A), M, K, _ptr(A, "A"), _ld(A, "A"), _ptr(vals, "vals"), _ld(vals, "vals"),
                                 _ptr(meta, "meta"), _ld(meta, "meta"), _ptr(row_ptr, "row_ptr"),
                                 _ptr(col, "col"), _ptr(rvals, "rvals"), _stream(A, stream)), "ssg_split_fill")


def ssg_residual_delta_count(row_ptr, col, K: int, drow_ptr, stream=None) -> None:
    M = row_ptr.numel() - 1
    nnz = int(col.numel()) if col is not None else 0
    _check(_lib().ssg_residual_delta_count(M, K, _ptr(row_ptr, "row_ptr"), _ptr(col, "col"), nnz,
                                           _ptr(drow_ptr, "drow_ptr"), _stream(row_ptr, stream)),
           "ssg_residual_delta_count")


def ssg_residual_delta_fill(row_ptr, col, rvals, K: int, drow_ptr, dcol, dvals, stream=None) -> None:
    M = row_ptr.numel() - 1
    nnz = int(col.numel()) if col is not None else 0
    _check(_lib().ssg_residual_delta_fill(_dtype(rvals), M, K, _ptr(row_ptr, "row_ptr"), _ptr(col, "col"),
                                          _ptr(rvals, "rvals"), nnz, _ptr(drow_ptr, "drow_ptr"), _ptr(dcol, "dcol"),
                                          _ptr(dvals, "dvals"), _stream(row_ptr, stream)), "ssg_residual_delta_fill")


def ssg_spmm_workspace_bytes(dtype: torch.dtype, M: int, N: int, K: int) -> int:
    return int(_lib().ssg_spmm_workspace_bytes(_DT[dtype], M, N, K))


def _torch_stream(t: torch.Tensor, stream):
    """The torch stream object of a `stream` argument (None: the current stream;
    a raw hipStream_t handle is wrapped)."""
    if stream is None:
        return torch.cuda.current_stream(t.device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=t.device)


def _workspace(dt_t: torch.dtype, M, N, K, device, ws, stream=None):
    """The caller's workspace, or a new one allocated on the stream the
    kernels run on, so the caching allocator does not hand its memory to
    another stream while they may still use it."""
    need = ssg_spmm_workspace_bytes(dt_t, M, N, K)
    if ws is None and need > 0 and torch.device(device).type == "cuda":   # host tensors fail in _ptr
        probe = torch.empty(0, device=device)
        with torch.cuda.stream(_torch_stream(probe, stream)):
            ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, (ws.numel() * ws.element_size() if ws is not None else 0)


def ssg_spmm_2to4(vals, meta, B, C, ws=None, algo: int = SSG_ALGO_AUTO, stream=None) -> None:
    ab = _dtype(vals)
    M, N, K = vals.shape[0], B.shape[1], B.shape[0]
    ws, wsb = _workspace(vals.dtype, M, N, K, vals.device, ws, stream)
    _check(_lib().ssg_spmm_2to4_ex(algo, ab, _OUT[ab][0], M, N, K, _ptr(vals, "vals"), _ld(vals, "vals"),
                                   _ptr(meta, "meta"), _ld(meta, "meta"), _ptr(B, "B"), _ld(B, "B"), _ptr(C, "C"),
                                   _ld(C, "C"), _ptr(ws, "ws"), wsb, _stream(C, stream)), "ssg_spmm_2to4")


def ssg_spmm_2to4_residual(vals, meta, row_ptr, col, rvals, B, C, ws=None, algo: int = SSG_ALGO_AUTO,
                           stream=None) -> None:
    ab = _dtype(vals)
    M, N, K = vals.shape[0], B.shape[1], B.shape[0]
    nnz = int(col.numel()) if col is not None else 0
    ws, wsb = _workspace(vals.dtype, M, N, K, vals.device, ws, stream)
    _check(_lib().ssg_spmm_2to4_residual_ex(algo, ab, _OUT[ab][0], M, N, K, _ptr(vals, "vals"), _ld(vals, "vals"),
                                            _ptr(meta, "meta"), _ld(meta, "meta"), _ptr(row_ptr, "row_ptr"),
                                            _ptr(col, "col"), _ptr(rvals, "rvals"), nnz, _ptr(B, "B"), _ld(B, "B"),
                                            _ptr(C, "C"), _ld(C, "C"), _ptr(ws, "ws"), wsb, _stream(C, stream)),
           "ssg_spmm_2to4_residual")


def ssg_spmm_2to4_residual_delta(vals, meta, drow_ptr, dcol, dvals, B, C, ws=None, algo: int = SSG_ALGO_AUTO,
                                 stream=None) -> None:
    ab = _dtype(vals)
    M, N, K = vals.shape[0], B.shape[1], B.shape[0]
    nnz = int(dcol.numel()) if dcol is not None else 0
    ws, wsb = _workspace(vals.dtype, M, N, K, vals.device, ws, stream)
    _check(_lib().ssg_spmm_2to4_residual_delta_ex(algo, ab, _OUT[ab][0], M, N, K, _ptr(vals, "vals"),
                                                  _ld(vals, "vals"), _ptr(meta, "meta"), _ld(meta, "meta"),
                                                  _ptr(drow_ptr, "drow_ptr"), _ptr(dcol, "dcol"),
                                                  _ptr(dvals, "dvals"), nnz, _ptr(B, "B"), _ld(B, "B"),
                                                  _ptr(C, "C"), _ld(C, "C"), _ptr(ws, "ws"), wsb,
                                                  _stream(C, stream)), "ssg_spmm_2to4_residual_delta")


def ssg_spmm_csr(row_ptr, col, vals, B, C, stream=None) -> None:
    ab = _dtype(vals)
    M, N, K = row_ptr.numel() - 1, B.shape[1], B.shape[0]
    nnz = int(col.numel()) if col is not None else 0
    _check(_lib().ssg_spmm_csr(ab, _OUT[ab][0], M, N, K, _ptr(row_ptr, "row_ptr"), _ptr(col, "col"),
                               _ptr(vals, "vals"), nnz, _ptr(B, "B"), _ld(B, "B"), _ptr(C, "C"), _ld(C, "C"),
                               _stream(C, stream)), "ssg_spmm_csr")


def ssg_spmm_csr_delta(drow_ptr, dcol, dvals, B, C, stream=None) -> None:
    ab = _dtype(dvals)
    M, N, K = drow_ptr.numel() - 1, B.shape[1], B.shape[0]
    nnz = int(dcol.numel()) if dcol is not None else 0
    _check(_lib().ssg_spmm_csr_delta(ab, _OUT[ab][0], M, N, K, _ptr(drow_ptr, "drow_ptr"), _ptr(dcol, "dcol"),
                                     _ptr(dvals, "dvals"), nnz, _ptr(B, "B"), _ld(B, "B"), _ptr(C, "C"),
                                     _ld(C, "C"), _stream(C, stream)), "ssg_spmm_csr_delta")


def ssg_packed_sizes(dtype: torch.dtype, M: int, K: int) -> Tuple[int, int]:
    import ctypes
    vb, mb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib().ssg_packed_sizes(_DT[dtype], M, K, ctypes.byref(vb), ctypes.byref(mb)), "ssg_packed_sizes")
    return int(vb.value), int(mb.value)


def ssg_pack_2to4_decode(vals, meta, K: int, pvals, pmeta, stream=None) -> None:
    M = vals.shape[0]
    _check(_lib().ssg_pack_2to4_decode(_dtype(vals), M, K, _ptr(vals, "vals"), _ld(vals, "vals"), _ptr(meta, "meta"),
                                       _ld(meta, "meta"), _ptr(pvals, "pvals"), _ptr(pmeta, "pmeta"),
                                       _stream(vals, stream)), "ssg_pack_2to4_decode")


def ssg_spmm_2to4_packed(pvals, pmeta, M: int, B, C, stream=None) -> None:
    ab = _dtype(B)
    N, K = B.shape[1], B.shape[0]
    _check(_lib().ssg_spmm_2to4_packed(ab, _OUT[ab][0], M, N, K, _ptr(pvals, "pvals"), _ptr(pmeta, "pmeta"),
                                       _ptr(B, "B"), _ld(B, "B"), _ptr(C, "C"), _ld(C, "C"), _stream(C, stream)),
           "ssg_spmm_2to4_packed")


def ssg_spmm_2to4_packed_bt(pvals, pmeta, M: int, Bt, C, stream=None) -> None:
    ab = _dtype(Bt)
    N, K = Bt.shape[0], Bt.shape[1]
    _check(_lib().ssg_spmm_2to4_packed_bt(ab, _OUT[ab][0], M, N, K, _ptr(pvals, "pvals"), _ptr(pmeta, "pmeta"),
                                          _ptr(Bt, "Bt"), _ld(Bt, "Bt"), _ptr(C, "C"), _ld(C, "C"),
                                          _stream(C, stream)), "ssg_spmm_2to4_packed_bt")


def ssg_prefill_packed_sizes(dtype: torch.dtype, M: int, K: int) -> Tuple[int, int]:
    import ctypes
    vb, mb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib().ssg_prefill_packed_sizes(_DT[dtype], M, K, ctypes.byref(vb), ctypes.byref(mb)),
           "ssg_prefill_packed_sizes")
    return int(vb.value), int(mb.value)


def ssg_compress_2to4_prefill(A: torch.Tensor, pvals, pmeta, stream=None) -> None:
    M, K = A.shape
    _check(_lib().ssg_compress_2to4_prefill(_dtype(A), M, K, _ptr(A, "A"), _ld(A, "A"), _ptr(pvals, "pvals"),
                                            _ptr(pmeta, "pmeta"), _stream(A, stream)), "ssg_compress_2to4_prefill")


def ssg_pack_2to4_prefill(vals, meta, K: int, pvals, pmeta, stream=None) -> None:
    M = vals.shape[0]
    _check(_lib().ssg_pack_2to4_prefill(_dtype(vals), M, K, _ptr(vals, "vals"), _ld(vals, "vals"),
                                        _ptr(meta, "meta"), _ld(meta, "meta"), _ptr(pvals, "pvals"),
                                        _ptr(pmeta, "pmeta"), _stream(vals, stream)), "ssg_pack_2to4_prefill")


def ssg_spmm_2to4_prefill(pvals, pmeta, M: int, B, C, stream=None) -> None:
    ab = _dtype(B)
    N, K = B.shape[1], B.shape[0]
    _check(_lib().ssg_spmm_2to4_prefill(ab, _OUT[ab][0], M, N, K, _ptr(pvals, "pvals"), _ptr(pmeta, "pmeta"),
                                        _ptr(B, "B"), _ld(B, "B"), _ptr(C, "C"), _ld(C, "C"), _stream(C, stream)),
           "ssg_spmm_2to4_prefill")


def ssg_spmm_2to4_prefill_bt(pvals, pmeta, M: int, Bt, C, stream=None) -> None:
    ab = _dtype(Bt)
    N, K = Bt.shape[0], Bt.shape[1]
    _check(_lib().ssg_spmm_2to4_prefill_bt(ab, _OUT[ab][0], M, N, K, _ptr(pvals, "pvals"), _ptr(pmeta, "pmeta"),
                                           _ptr(Bt, "Bt"), _ld(Bt, "Bt"), _ptr(C, "C"), _ld(C, "C"),
                                           _stream(C, stream)), "ssg_spmm_2to4_prefill_bt")


def ssg_spmm_2to4_packed_residual(pvals, pmeta, M: int, row_ptr, col, rvals, B, C, stream=None) -> None:
    ab = _dtype(B)
    N, K = B.shape[1], B.shape[0]
    nnz = int(col.numel()) if col is not None else 0
    _check(_lib().ssg_spmm_2to4_packed_residual(ab, _OUT[ab][0], M, N, K, _ptr(pvals, "pvals"), _ptr(pmeta, "pmeta"),
                                                _ptr(row_ptr, "row_ptr"), _ptr(col, "col"), _ptr(rvals, "rvals"), nnz,
                                                _ptr(B, "B"), _ld(B, "B"), _ptr(C, "C"), _ld(C, "C"),
                                                _stream(C, stream)), "ssg_spmm_2to4_packed_residual")


def ssg_spmm_2to4_packed_residual_delta(pvals, pmeta, M: int, drow_ptr, dcol, dvals, B, C, stream=None) -> None:
    ab = _dtype(B)
    N, K = B.shape[1], B.shape[0]
    nnz = int(dcol.numel()) if dcol is not None else 0
    _check(_lib().ssg_spmm_2to4_packed_residual_delta(ab, _OUT[ab][0], M, N, K, _ptr(pvals, "pvals"),
                                                      _ptr(pmeta, "pmeta"), _ptr(drow_ptr, "drow_ptr"),
                                                      _ptr(dcol, "dcol"), _ptr(dvals, "dvals"), nnz, _ptr(B, "B"),
                                                      _ld(B, "B"), _ptr(C, "C"), _ld(C, "C"), _stream(C, stream)),
           "ssg_spmm_2to4_packed_residual_delta")


def ssg_spmm_select_algo(vals, meta, B, C) -> int:
    return int(_lib().ssg_spmm_select_algo(_dtype(vals), vals.shape[0], B.shape[1], B.shape[0], _ptr(vals, "vals"),
                                           _ld(vals, "vals"), _ptr(meta, "meta"), _ld(meta, "meta"), _ptr(B, "B"),
                                           _ld(B, "B"), _ptr(C, "C"), _ld(C, "C")))


def ssg_noalloc_scratch_bytes() -> int:
    return int(_lib().ssg_noalloc_scratch_bytes())


def ssg_spmm_2to4_noalloc(vals, meta, B, C, stream=None) -> None:
    """ssg_spmm_2to4 without a workspace: nothing is allocated (the library's
    own scratch array holds a padded narrow B)."""
    ab = _dtype(vals)
    M, N, K = vals.shape[0], B.shape[1], B.shape[0]
    _check(_lib().ssg_spmm_2to4_noalloc(ab, _OUT[ab][0], M, N, K, _ptr(vals, "vals"), _ld(vals, "vals"),
                                        _ptr(meta, "meta"), _ld(meta, "meta"), _ptr(B, "B"), _ld(B, "B"),
                                        _ptr(C, "C"), _ld(C, "C"), _stream(C, stream)), "ssg_spmm_2to4_noalloc")


def ssg_cbm_sizes(dtype: torch.dtype, M: int, K: int) -> Tuple[int, int]:
    """(mask bytes, blocks) of the complement-bitmap residual; roff has blocks + 1 entries."""
    import ctypes
    mb, nb = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib().ssg_cbm_sizes(_DT[dtype], M, K, ctypes.byref(mb), ctypes.byref(nb)), "ssg_cbm_sizes")
    return int(mb.value), int(nb.value)


def ssg_pack_residual_cbm(meta, row_ptr, col, rvals, K: int, rmask, roff, cvals, bad_count=None,
                          stream=None) -> None:
    M = row_ptr.numel() - 1
    nnz = int(col.numel()) if col is not None else 0
    _check(_lib().ssg_pack_residual_cbm(_dtype(rvals), M, K, _ptr(meta, "meta"), _ld(meta, "meta"),
                                        _ptr(row_ptr, "row_ptr"), _ptr(col, "col"), _ptr(rvals, "rvals"), nnz,
                                        _ptr(rmask, "rmask"), _ptr(roff, "roff"), _ptr(cvals, "cvals"),
                                        _ptr(bad_count, "bad_count"), _stream(row_ptr, stream)),
           "ssg_pack_residual_cbm")


def ssg_spmm_2to4_packed_residual_cbm(pvals, pmeta, M: int, rmask, roff, cvals, B, C, stream=None) -> None:
    ab = _dtype(B)
    N, K = B.shape[1], B.shape[0]
    _check(_lib().ssg_spmm_2to4_packed_residual_cbm(ab, _OUT[ab][0], M, N, K, _ptr(pvals, "pvals"),
                                                    _ptr(pmeta, "pmeta"), _ptr(rmask, "rmask"), _ptr(roff, "roff"),
                                                    _ptr(cvals, "cvals"), int(cvals.numel()), _ptr(B, "B"),
                                                    _ld(B, "B"), _ptr(C, "C"), _ld(C, "C"), _stream(C, stream)),
           "ssg_spmm_2to4_packed_residual_cbm")


def ssg_spmm_2to4_packed_residual_cbm_bt(pvals, pmeta, M: int, rmask, roff, cvals, Bt, C, stream=None) -> None:
    ab = _dtype(Bt)
    N, K = Bt.shape[0], Bt.shape[1]
    _check(_lib().ssg_spmm_2to4_packed_residual_cbm_bt(ab, _OUT[ab][0], M, N, K, _ptr(pvals, "pvals"),
                                                       _ptr(pmeta, "pmeta"), _ptr(rmask, "rmask"), _ptr(roff, "roff"),
                                                       _ptr(cvals, "cvals"), int(cvals.numel()), _ptr(Bt, "Bt"),
                                                       _ld(Bt, "Bt"), _ptr(C, "C"), _ld(C, "C"), _stream(C, stream)),
           "ssg_spmm_2to4_packed_residual_cbm_bt")


def ssg_stream_read_sink_words(nbytes: int) -> int:
    return int(_lib().ssg_stream_read_sink_words(nbytes))


def ssg_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement helper: one streaming read of every byte of src."""
    nbytes = src.numel() * src.element_size()
    _check(_lib().ssg_stream_read(_ptr(src, "src"), nbytes, _ptr(sink, "sink"), _stream(src, stream)),
           "ssg_stream_read")


def ssg_mfma_probe_forms() -> int:
    return int(_lib().ssg_mfma_probe_forms())


def ssg_mfma_probe_name(form: int) -> Optional[str]:
    name = _lib().ssg_mfma_probe_name(form)
    return name.decode() if name is not None else None


def ssg_mfma_probe_ops(form: int, workgroups: int, iters: int) -> int:
    return int(_lib().ssg_mfma_probe_ops(form, workgroups, iters))


def ssg_mfma_probe(form: int, workgroups: int, iters: int, sink: torch.Tensor, stream=None) -> None:
    """Measurement helper: one launch of the issue-rate probe of a matrix-core
    instruction form (sink: at least `workgroups` int32 words on the device)."""
    if sink.numel() * sink.element_size() < 4 * workgroups:
        raise ValueError("sink holds fewer than %d words" % workgroups)
    _check(_lib().ssg_mfma_probe(form, workgroups, iters, _ptr(sink, "sink"), _stream(sink, stream)),
           "ssg_mfma_probe")


def ssg_lds_read_probe(offsets, workgroups: int, iters: int, sink: torch.Tensor, stream=None) -> None:
    """Measurement helper: one launch of the LDS read probe (offsets: 64 byte
    offsets, one per lane; sink: at least `workgroups` int32 words on the
    device)."""
    offs = (ctypes.c_uint32 * 64)(*[int(o) for o in offsets]) if len(offsets) == 64 else None
    if offs is None:
        raise ValueError("offsets must hold 64 entries, one per lane")
    if sink.numel() * sink.element_size() < 4 * workgroups:
        raise ValueError("sink holds fewer than %d words" % workgroups)
    _check(_lib().ssg_lds_read_probe(ctypes.cast(offs, ctypes.c_void_p), workgroups, iters, _ptr(sink, "sink"),
                                     _stream(sink, stream)), "ssg_lds_read_probe")


def ssg_compress_nm(A: torch.Tensor, n: int, m: int, vals: torch.Tensor, mask: torch.Tensor, stream=None) -> None:
    e = _per(A)
    _check(_lib().ssg_compress_nm(_dtype(A), n, m, A.shape[0], A.shape[1] * e, _ptr(A, "A"), _ld(A, "A") * e,
                                  _ptr(vals, "vals"), _ld(vals, "vals") * e, _ptr(mask, "mask"), _ld(mask, "mask"),
                                  _stream(A, stream)), "ssg_compress_nm")


def ssg_decompress_nm(vals: torch.Tensor, mask: torch.Tensor, n: int, m: int, D: torch.Tensor,
                      bad_count: Optional[torch.Tensor] = None, stream=None) -> None:
    e = _per(vals)
    _check(_lib().ssg_decompress_nm(_dtype(vals), n, m, D.shape[0], D.shape[1] * e, _ptr(vals, "vals"),
                                    _ld(vals, "vals") * e, _ptr(mask, "mask"), _ld(mask, "mask"), _ptr(D, "D"),
                                    _ld(D, "D") * e, _ptr(bad_count, "bad_count"), _stream(D, stream)),
           "ssg_decompress_nm")


def ssg_spmm_nm(vals: torch.Tensor, mask: torch.Tensor, n: int, m: int, K: int, B: torch.Tensor, C: torch.Tensor,
                stream=None) -> None:
    ab = _dtype(vals)
    _check(_lib().ssg_spmm_nm(ab, _OUT[ab][0], n, m, vals.shape[0], B.shape[1], K, _ptr(vals, "vals"),
                              _ld(vals, "vals") * _per(vals), _ptr(mask, "mask"), _ld(mask, "mask"), _ptr(B, "B"),
                              _ld(B, "B"),
                              _ptr(C, "C"), _ld(C, "C"), _stream(C, stream)), "ssg_spmm_nm")


def ssg_nm_packed_sizes(dtype: torch.dtype, n: int, m: int, M: int, K: int) -> Tuple[int, int]:
    import ctypes
    vb, mb = ctypes.c_int64(0), ctypes.c_int64(0)
    dt = _DT.get(dtype)
    if dt is None:
        raise SsgError(_abi.SSG_ERR_DTYPE, "unsupported element type %s" % (dtype,))
    _check(_lib().ssg_nm_packed_sizes(dt, n, m, M, K, ctypes.byref(vb), ctypes.byref(mb)), "ssg_nm_packed_sizes")
    return vb.value, mb.value


def ssg_pack_nm_decode(vals, mask, n: int, m: int, K: int, pvals, pmask, stream=None) -> None:
    _check(_lib().ssg_pack_nm_decode(_dtype(vals), n, m, vals.shape[0], K, _ptr(vals, "vals"),
                                     _ld(vals, "vals") * _per(vals),
                                     _ptr(mask, "mask"), _ld(mask, "mask"), _ptr(pvals, "pvals"),
                                     _ptr(pmask, "pmask"), _stream(vals, stream)), "ssg_pack_nm_decode")


def ssg_spmm_nm_packed(pvals, pmask, n: int, m: int, M: int, B, C, stream=None, i4: bool = False) -> None:
    """i4: the packed weights are 4-bit (B is then fp16)."""
    ab = _abi.SSG_I4 if i4 else _dtype(B)
    _check(_lib().ssg_spmm_nm_packed(ab, _OUT[ab][0], n, m, M, B.shape[1], B.shape[0], _ptr(pvals, "pvals"),
                                     _ptr(pmask, "pmask"), _ptr(B, "B"), _ld(B, "B"), _ptr(C, "C"), _ld(C, "C"),
                                     _stream(C, stream)), "ssg_spmm_nm_packed")


# ---------------------------------------------------------------- allocating helpers

def prune(A: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    P = torch.empty_like(A) if out is None else out
    ssg_prune_2to4(A, P)
    return P


def compress(A: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """(vals [M, K/2], meta [M, ceil(K/8)] uint8) of a dense [M, K] weight."""
    M, K = A.shape
    vals = torch.empty((M, K // 2), dtype=A.dtype, device=A.device)
    meta = torch.empty((M, (K + 7) // 8), dtype=torch.uint8, device=A.device)
    ssg_compress_2to4(A, vals, meta)
    return vals, meta


def decompress(vals: torch.Tensor, meta: torch.Tensor, K: Optional[int] = None, count_bad: bool = False):
    M = vals.shape[0]
    K = 2 * vals.shape[1] if K is None else K
    D = torch.empty((M, K), dtype=vals.dtype, device=vals.device)
    bad = torch.zeros(1, dtype=torch.int32, device=vals.device) if count_bad else None
    ssg_decompress_2to4(vals, meta, D, bad)
    return (D, int(bad.item())) if count_bad else D


def split(A: torch.Tensor):
    """2:4 layer plus CSR residual: (vals, meta, row_ptr, col, rvals).  Reads the
    residual size back to the host between the two passes (one sync)."""
    M, K = A.shape
    row_ptr = torch.empty(M + 1, dtype=torch.int32, device=A.device)
    ssg_split_count(A, row_ptr)
    nnz = int(row_ptr[M].item())
    vals = torch.empty((M, K // 2), dtype=A.dtype, device=A.device)
    meta = torch.empty((M, (K + 7) // 8), dtype=torch.uint8, device=A.device)
    col = torch.empty(nnz, dtype=torch.int32, device=A.device)
    rvals = torch.empty(nnz, dtype=A.dtype, device=A.device)
    ssg_split_fill(A, vals, meta, row_ptr, col if nnz else None, rvals if nnz else None)
    return vals, meta, row_ptr, col, rvals


def spmm(vals: torch.Tensor, meta: torch.Tensor, B: torch.Tensor, algo: int = SSG_ALGO_AUTO,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand(vals, meta) @ B: fp32 for fp16/bf16, int32 for int8."""
    ab = _dtype(vals)
    C = torch.empty((vals.shape[0], B.shape[1]), dtype=_OUT[ab][1], device=vals.device) if out is None else out
    ssg_spmm_2to4(vals, meta, B, C, algo=algo)
    return C


def spmm_residual(vals, meta, row_ptr, col, rvals, B, algo: int = SSG_ALGO_AUTO,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    ab = _dtype(vals)
    C = torch.empty((vals.shape[0], B.shape[1]), dtype=_OUT[ab][1], device=vals.device) if out is None else out
    ssg_spmm_2to4_residual(vals, meta, row_ptr, col, rvals, B, C, algo=algo)
    return C


def delta_encode(row_ptr: torch.Tensor, col: torch.Tensor, rvals: torch.Tensor, K: int):
    """Delta-coded form (drow_ptr, dcol uint8, dvals) of a CSR residual (columns
    ascending in every row).  Reads the coded size back to the host between
    the two passes (one sync)."""
    M = row_ptr.numel() - 1
    drow_ptr = torch.empty(M + 1, dtype=torch.int32, device=row_ptr.device)
    ssg_residual_delta_count(row_ptr, col, K, drow_ptr)
    n = int(drow_ptr[M].item())
    dcol = torch.empty(n, dtype=torch.uint8, device=row_ptr.device)
    dvals = torch.empty(n, dtype=rvals.dtype, device=row_ptr.device)
    ssg_residual_delta_fill(row_ptr, col, rvals, K, drow_ptr, dcol, dvals)
    return drow_ptr, dcol, dvals


def spmm_residual_delta(vals, meta, drow_ptr, dcol, dvals, B, algo: int = SSG_ALGO_AUTO,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    ab = _dtype(vals)
    C = torch.empty((vals.shape[0], B.shape[1]), dtype=_OUT[ab][1], device=vals.device) if out is None else out
    ssg_spmm_2to4_residual_delta(vals, meta, drow_ptr, dcol, dvals, B, C, algo=algo)
    return C


def spmm_csr(row_ptr, col, vals, B, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = S @ B for an unstructured sparse S given as CSR (no 2:4 layer)."""
    ab = _dtype(vals)
    C = torch.empty((row_ptr.numel() - 1, B.shape[1]), dtype=_OUT[ab][1], device=B.device) if out is None else out
    ssg_spmm_csr(row_ptr, col, vals, B, C)
    return C


def spmm_csr_delta(drow_ptr, dcol, dvals, B, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = S @ B for an unstructured sparse S in the delta-coded form (no 2:4 layer)."""
    ab = _dtype(dvals)
    C = torch.empty((drow_ptr.numel() - 1, B.shape[1]), dtype=_OUT[ab][1], device=B.device) if out is None else out
    ssg_spmm_csr_delta(drow_ptr, dcol, dvals, B, C)
    return C


def _padded(rows: int, cols: int, dtype: torch.dtype, align: int, device) -> torch.Tensor:
    """[rows, cols] view of a buffer whose rows start every `align` bytes."""
    es = torch.empty((), dtype=dtype).element_size()
    ld = max(1, -(-cols * es // align) * align // es)
    return torch.empty((rows, ld), dtype=dtype, device=device)[:, :cols]


def compress_nm(A: torch.Tensor, n: int, m: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """(vals [M, K/m*n], mask [M, ceil(K/8)] uint8) of a dense [M, K] weight under
    the n:m rule; rows padded to 16 (vals) and 8 (mask) bytes as the product
    wants them."""
    e = _per(A)
    M, K = A.shape[0], A.shape[1] * e
    vals = _padded(M, K // m * n // e, A.dtype, 16, A.device)
    mask = _padded(M, (K + 7) // 8, torch.uint8, 8, A.device)
    ssg_compress_nm(A, n, m, vals, mask)
    return vals, mask


def decompress_nm(vals: torch.Tensor, mask: torch.Tensor, n: int, m: int, K: int, count_bad: bool = False):
    D = torch.empty((vals.shape[0], K // _per(vals)), dtype=vals.dtype, device=vals.device)
    bad = torch.zeros(1, dtype=torch.int32, device=vals.device) if count_bad else None
    ssg_decompress_nm(vals, mask, n, m, D, bad)
    return (D, int(bad.item())) if count_bad else D


def spmm_nm(vals: torch.Tensor, mask: torch.Tensor, n: int, m: int, B: torch.Tensor,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand_nm(vals, mask) @ B, K = B.shape[0]: fp32 for float inputs, int32 for int8."""
    ab = _dtype(vals)
    C = torch.empty((vals.shape[0], B.shape[1]), dtype=_OUT[ab][1], device=vals.device) if out is None else out
    ssg_spmm_nm(vals, mask, n, m, B.shape[0], B, C)
    return C


def pack_nm(vals: torch.Tensor, mask: torch.Tensor, n: int, m: int, K: int):
    """(pvals, pmask) byte tensors of the packed decode layout of an n:m operand."""
    vb, mb = ssg_nm_packed_sizes(vals.dtype, n, m, vals.shape[0], K)
    pvals = torch.empty(vb, dtype=torch.uint8, device=vals.device)
    pmask = torch.empty(mb, dtype=torch.uint8, device=vals.device)
    ssg_pack_nm_decode(vals, mask, n, m, K, pvals, pmask)
    return pvals, pmask


def spmm_nm_packed(pvals: torch.Tensor, pmask: torch.Tensor, n: int, m: int, M: int, B: torch.Tensor,
                   out: Optional[torch.Tensor] = None, i4: bool = False) -> torch.Tensor:
    ab = _abi.SSG_I4 if i4 else _dtype(B)
    C = torch.empty((M, B.shape[1]), dtype=_OUT[ab][1], device=B.device) if out is None else out
    ssg_spmm_nm_packed(pvals, pmask, n, m, M, B, C, i4=i4)
    return C


def pack_decode(vals: torch.Tensor, meta: torch.Tensor, K: Optional[int] = None):
    """(pvals, pmeta) byte tensors of the packed decode layout of (vals, meta)."""
    K = 2 * vals.shape[1] if K is None else K
    vb, mb = ssg_packed_sizes(vals.dtype, vals.shape[0], K)
    pvals = torch.empty(vb, dtype=torch.uint8, device=vals.device)
    pmeta = torch.empty(mb, dtype=torch.uint8, device=vals.device)
    ssg_pack_2to4_decode(vals, meta, K, pvals, pmeta)
    return pvals, pmeta


def _prefill_buffers(dtype: torch.dtype, M: int, K: int, device):
    vb, mb = ssg_prefill_packed_sizes(dtype, M, K)
    return (torch.empty(vb, dtype=torch.uint8, device=device), torch.empty(mb, dtype=torch.uint8, device=device))


def compress_prefill(A: torch.Tensor):
    """(pvals, pmeta) byte tensors of the packed prefill layout of a dense [M, K]
    weight, compressed straight into it."""
    M, K = A.shape
    pvals, pmeta = _prefill_buffers(A.dtype, M, K, A.device)
    ssg_compress_2to4_prefill(A, pvals, pmeta)
    return pvals, pmeta


def pack_prefill(vals: torch.Tensor, meta: torch.Tensor, K: Optional[int] = None):
    """(pvals, pmeta) byte tensors of the packed prefill layout of (vals, meta)."""
    K = 2 * vals.shape[1] if K is None else K
    pvals, pmeta = _prefill_buffers(vals.dtype, vals.shape[0], K, vals.device)
    ssg_pack_2to4_prefill(vals, meta, K, pvals, pmeta)
    return pvals, pmeta


def spmm_prefill(pvals: torch.Tensor, pmeta: torch.Tensor, M: int, B: torch.Tensor,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand(packed prefill) @ B on the large-N kernel: fp32 for float
    inputs, int32 for int8."""
    ab = _dtype(B)
    C = torch.empty((M, B.shape[1]), dtype=_OUT[ab][1], device=B.device) if out is None else out
    ssg_spmm_2to4_prefill(pvals, pmeta, M, B, C)
    return C


def spmm_prefill_bt(pvals: torch.Tensor, pmeta: torch.Tensor, M: int, Bt: torch.Tensor,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand(packed prefill) @ Bt.T on the large-N kernel, Bt [N, K]
    row-major (token-major activations): fp32 for float inputs, int32 for
    int8."""
    ab = _dtype(Bt)
    C = torch.empty((M, Bt.shape[0]), dtype=_OUT[ab][1], device=Bt.device) if out is None else out
    ssg_spmm_2to4_prefill_bt(pvals, pmeta, M, Bt, C)
    return C


def spmm_packed_residual(pvals, pmeta, M: int, row_ptr, col, rvals, B: torch.Tensor,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand(packed) @ B + residual(CSR) @ B, B [K, 16]."""
    ab = _dtype(B)
    C = torch.empty((M, B.shape[1]), dtype=_OUT[ab][1], device=B.device) if out is None else out
    ssg_spmm_2to4_packed_residual(pvals, pmeta, M, row_ptr, col, rvals, B, C)
    return C


def spmm_packed_residual_delta(pvals, pmeta, M: int, drow_ptr, dcol, dvals, B: torch.Tensor,
                               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand(packed) @ B + residual(delta-coded) @ B, B [K, 16]."""
    ab = _dtype(B)
    C = torch.empty((M, B.shape[1]), dtype=_OUT[ab][1], device=B.device) if out is None else out
    ssg_spmm_2to4_packed_residual_delta(pvals, pmeta, M, drow_ptr, dcol, dvals, B, C)
    return C


def pack_residual_cbm(meta: torch.Tensor, row_ptr: torch.Tensor, col: torch.Tensor, rvals: torch.Tensor, K: int):
    """(rmask, roff, cvals) of the complement-bitmap layout of a CSR residual
    (from split) against its 2:4 layer's metadata; cvals is 16-byte aligned."""
    M = row_ptr.numel() - 1
    mb, nb = ssg_cbm_sizes(rvals.dtype, M, K)
    dev = row_ptr.device
    rmask = torch.empty(mb, dtype=torch.uint8, device=dev)
    roff = torch.empty(nb + 1, dtype=torch.int32, device=dev)
    nnz = int(col.numel())
    es = rvals.element_size()
    cvals = torch.empty(-(-max(nnz, 1) * es // 16) * 16 // es, dtype=rvals.dtype, device=dev)[:nnz]
    ssg_pack_residual_cbm(meta, row_ptr, col, rvals, K, rmask, roff, cvals)
    return rmask, roff, cvals


def spmm_packed_residual_cbm(pvals, pmeta, M: int, rmask, roff, cvals, B: torch.Tensor,
                             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand(packed) @ B + residual(complement bitmap) @ B, B [K, 16]."""
    ab = _dtype(B)
    C = torch.empty((M, B.shape[1]), dtype=_OUT[ab][1], device=B.device) if out is None else out
    ssg_spmm_2to4_packed_residual_cbm(pvals, pmeta, M, rmask, roff, cvals, B, C)
    return C


def spmm_packed_residual_cbm_bt(pvals, pmeta, M: int, rmask, roff, cvals, Bt: torch.Tensor,
                                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """As spmm_packed_residual_cbm with B given as Bt [N, K] row-major, N <= 16."""
    ab = _dtype(Bt)
    C = torch.empty((M, Bt.shape[0]), dtype=_OUT[ab][1], device=Bt.device) if out is None else out
    ssg_spmm_2to4_packed_residual_cbm_bt(pvals, pmeta, M, rmask, roff, cvals, Bt, C)
    return C


def spmm_packed_bt(pvals: torch.Tensor, pmeta: torch.Tensor, M: int, Bt: torch.Tensor,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand(packed) @ Bt.T, Bt [N, K] row-major with N <= 16
    (token-major activations of a decode step)."""
    ab = _dtype(Bt)
    C = torch.empty((M, Bt.shape[0]), dtype=_OUT[ab][1], device=Bt.device) if out is None else out
    ssg_spmm_2to4_packed_bt(pvals, pmeta, M, Bt, C)
    return C


def spmm_packed(pvals: torch.Tensor, pmeta: torch.Tensor, M: int, B: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = expand(packed) @ B, B [K, 16]: fp32 for fp16/bf16, int32 for int8."""
    ab = _dtype(B)
    C = torch.empty((M, B.shape[1]), dtype=_OUT[ab][1], device=B.device) if out is None else out
    ssg_spmm_2to4_packed(pvals, pmeta, M, B, C)
    return C
