"""The C ABI library on the CPU: it loads, exports every function the header
declares, and rejects invalid arguments on the host before any HIP call
(so these run without a GPU).  No compute call is made here."""
import ctypes
import os
import re

import pytest
import torch

import structured_sparse_gemm_amd as ssg
from structured_sparse_gemm_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssgemm.h")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first
F16, BF16, I8, F32, I32 = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssg_\w+)\s*\(", text)))


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for required in ("ssg_compress_2to4", "ssg_prune_2to4", "ssg_decompress_2to4", "ssg_split_count",
                     "ssg_split_fill", "ssg_spmm_2to4", "ssg_spmm_2to4_residual", "ssg_spmm_workspace_bytes",
                     "ssg_status_str", "ssg_last_error", "ssg_vals_cols", "ssg_meta_cols", "ssg_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing
    # and the ctypes signature table covers them all
    assert set(declared_functions()) == set(_abi.SIGNATURES)


def test_version_and_sizes(lib):
    assert lib.ssg_abi_version() == 1
    for K, v, m in [(0, 0, 0), (4, 2, 1), (8, 4, 1), (12, 6, 2), (4096, 2048, 512), (8196, 4098, 1025)]:
        assert lib.ssg_vals_cols(K) == v and lib.ssg_meta_cols(K) == m
    for s in range(9):
        assert lib.ssg_status_str(s).decode().startswith("SSG_")
    assert lib.ssg_spmm_workspace_bytes(F16, 11008, 16, 4096) == 0


def test_noalloc_rejects_a_padded_b_beyond_its_scratch(lib):
    # checked on the host before anything is enqueued
    cap = lib.ssg_noalloc_scratch_bytes()
    assert cap == 2 << 20
    K = cap // 32 + 64
    assert lib.ssg_spmm_2to4_noalloc(F16, F32, 8, 5, K, FAKE, K // 2, FAKE, K // 8, FAKE, 5, FAKE, 5,
                                     None) == _abi.SSG_ERR_WORKSPACE
    assert "scratch" in lib.ssg_last_error().decode()
    assert lib.ssg_spmm_2to4_noalloc(F16, I32, 8, 5, 64, FAKE, 32, FAKE, 8, FAKE, 5, FAKE, 5,
                                     None) == _abi.SSG_ERR_DTYPE
    assert lib.ssg_spmm_2to4_noalloc(F16, F32, 0, 5, 64, FAKE, 32, FAKE, 8, FAKE, 5, FAKE, 5, None) == 0


def test_workspace_size_and_requirement(lib):
    ws = lib.ssg_spmm_workspace_bytes
    # B padded to K x 16 elements, rounded up to 256 bytes, for 0 < N < 16 only
    assert ws(F16, 11008, 1, 4096) == 4096 * 16 * 2
    assert ws(BF16, 5, 15, 100) == (100 * 16 * 2 + 255) // 256 * 256
    assert ws(I8, 300, 8, 1024) == 1024 * 16
    assert ws(_abi.SSG_E4M3, 300, 8, 1028) == (1028 * 16 + 255) // 256 * 256
    for args in [(F16, 8, 16, 64), (F16, 8, 17, 64), (F16, 8, 0, 64), (F16, 8, 5, 0), (F16, 0, 5, 64),
                 (F16, 8, 5, 62), (F32, 8, 5, 64),
                 (F16, 8, 5, 1 << 26),             # the padded copy would need 2^31 bytes: never padded
                 (I8, 8, 5, 1 << 27)]:
        assert ws(*args) == 0, args
    assert ws(F16, 8, 5, (1 << 26) - 4) > 0
    # a product that takes the padded decode path fails without its workspace
    # (checked on the host: nothing is enqueued)
    f = lib.ssg_spmm_2to4
    need = ws(F16, 8, 5, 64)
    assert f(F16, F32, 8, 5, 64, FAKE, 32, FAKE, 8, FAKE, 5, FAKE, 5, None, 0, None) == _abi.SSG_ERR_WORKSPACE
    assert "workspace" in lib.ssg_last_error().decode()
    assert f(F16, F32, 8, 5, 64, FAKE, 32, FAKE, 8, FAKE, 5, FAKE, 5, FAKE, need - 1, None) == _abi.SSG_ERR_WORKSPACE
    assert f(F16, F32, 8, 5, 64, FAKE, 32, FAKE, 8, FAKE, 5, FAKE, 5, ctypes.c_void_p(0x1008), need,
             None) == _abi.SSG_ERR_WORKSPACE                  # misaligned
    r = lib.ssg_spmm_2to4_residual
    assert r(F16, F32, 8, 5, 64, FAKE, 32, FAKE, 8, FAKE, FAKE, FAKE, 4, FAKE, 5, FAKE, 5, None, 0,
             None) == _abi.SSG_ERR_WORKSPACE


def _status(rc):
    return rc


def test_dense_argument_errors(lib):
    # bad dtype / shape / stride / null, all caught on the host
    assert lib.ssg_compress_2to4(F32, 4, 8, FAKE, 8, FAKE, 4, FAKE, 1, None) == _abi.SSG_ERR_DTYPE
    assert lib.ssg_compress_2to4(F16, 4, 6, FAKE, 8, FAKE, 4, FAKE, 1, None) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_compress_2to4(F16, -1, 8, FAKE, 8, FAKE, 4, FAKE, 1, None) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_compress_2to4(F16, 4, 8, FAKE, 7, FAKE, 4, FAKE, 1, None) == _abi.SSG_ERR_STRIDE
    assert lib.ssg_compress_2to4(F16, 4, 8, FAKE, 8, FAKE, 3, FAKE, 1, None) == _abi.SSG_ERR_STRIDE
    assert lib.ssg_compress_2to4(F16, 4, 16, FAKE, 16, FAKE, 8, FAKE, 1, None) == _abi.SSG_ERR_STRIDE
    assert lib.ssg_compress_2to4(I8, 4, 8, None, 8, FAKE, 4, FAKE, 1, None) == _abi.SSG_ERR_NULL
    assert lib.ssg_compress_2to4(I8, 4, 8, FAKE, 8, FAKE, 4, None, 1, None) == _abi.SSG_ERR_NULL
    assert "meta" in lib.ssg_last_error().decode()
    assert lib.ssg_prune_2to4(BF16, 2, 8, FAKE, 8, None, 8, None) == _abi.SSG_ERR_NULL
    assert lib.ssg_prune_2to4(BF16, 2, 8, FAKE, 16, FAKE, 8, None) == _abi.SSG_ERR_STRIDE   # in place needs lda == ldp
    assert lib.ssg_decompress_2to4(F16, 2, 8, FAKE, 4, FAKE, 1, FAKE, 4, None, None) == _abi.SSG_ERR_STRIDE
    assert lib.ssg_split_count(F16, 2, 8, FAKE, 8, None, None) == _abi.SSG_ERR_NULL
    assert lib.ssg_split_fill(F16, 2, 8, FAKE, 8, FAKE, 4, FAKE, 1, FAKE, FAKE, None, None) == _abi.SSG_ERR_NULL
    # int32 row_ptr cannot count the residual of a huge matrix
    assert lib.ssg_split_count(F16, 1 << 20, 1 << 14, FAKE, 1 << 14, FAKE, None) == _abi.SSG_ERR_SHAPE


def test_delta_code_argument_errors(lib):
    assert lib.ssg_residual_delta_count(4, 64, FAKE, FAKE, 3, None, None) == _abi.SSG_ERR_NULL
    assert lib.ssg_residual_delta_count(4, 64, None, FAKE, 3, FAKE, None) == _abi.SSG_ERR_NULL
    assert lib.ssg_residual_delta_count(4, 64, FAKE, None, 3, FAKE, None) == _abi.SSG_ERR_NULL
    assert lib.ssg_residual_delta_count(-1, 64, FAKE, FAKE, 3, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_residual_delta_count(4, 64, FAKE, FAKE, -1, FAKE, None) == _abi.SSG_ERR_FORMAT
    # worst-case coded length beyond int32
    assert lib.ssg_residual_delta_count(1 << 20, 1 << 20, FAKE, FAKE, 3, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_residual_delta_fill(F32, 4, 64, FAKE, FAKE, FAKE, 3, FAKE, FAKE, FAKE, None) == _abi.SSG_ERR_DTYPE
    assert lib.ssg_residual_delta_fill(F16, 4, 64, FAKE, FAKE, FAKE, 3, FAKE, None, FAKE, None) == _abi.SSG_ERR_NULL
    assert lib.ssg_residual_delta_fill(F16, 4, 64, FAKE, FAKE, FAKE, 3, None, FAKE, FAKE, None) == _abi.SSG_ERR_NULL
    # the product: the same host checks as the CSR form, plus its own pointers
    args = (F16, F32, 16, 16, 64, FAKE, 32, FAKE, 8)
    tail = (FAKE, 16, FAKE, 16, None, 0, None)
    assert lib.ssg_spmm_2to4_residual_delta(*args, None, FAKE, FAKE, 5, *tail) == _abi.SSG_ERR_NULL
    assert lib.ssg_spmm_2to4_residual_delta(*args, FAKE, None, FAKE, 5, *tail) == _abi.SSG_ERR_NULL
    assert lib.ssg_spmm_2to4_residual_delta(*args, FAKE, FAKE, FAKE, -2, *tail) == _abi.SSG_ERR_FORMAT
    assert lib.ssg_spmm_2to4_residual_delta(I8, F32, 16, 16, 64, FAKE, 32, FAKE, 8, FAKE, FAKE, FAKE, 5,
                                            *tail) == _abi.SSG_ERR_DTYPE
    assert lib.ssg_spmm_2to4_residual_delta_ex(9, *args, FAKE, FAKE, FAKE, 5, *tail) == _abi.SSG_ERR_ALGO


def test_nm_argument_errors(lib):
    assert [lib.ssg_nm_vals_cols(n, m, 4096) for n, m in [(1, 4), (2, 4), (2, 8), (4, 8)]] == [1024, 2048, 1024, 2048]
    c = lib.ssg_compress_nm
    # patterns without kernels, K not a multiple of m, strides, nulls, dtype
    for n, m in [(3, 8), (1, 8), (4, 4), (0, 4), (2, 16)]:
        assert c(F16, n, m, 4, 64, FAKE, 64, FAKE, 64, FAKE, 8, None) == _abi.SSG_ERR_SHAPE
    assert c(F16, 2, 8, 4, 60, FAKE, 60, FAKE, 16, FAKE, 8, None) == _abi.SSG_ERR_SHAPE
    assert c(F16, 2, 8, 4, 64, FAKE, 63, FAKE, 16, FAKE, 8, None) == _abi.SSG_ERR_STRIDE
    assert c(F16, 2, 8, 4, 64, FAKE, 64, FAKE, 15, FAKE, 8, None) == _abi.SSG_ERR_STRIDE
    assert c(F16, 2, 8, 4, 64, FAKE, 64, FAKE, 16, FAKE, 7, None) == _abi.SSG_ERR_STRIDE
    assert c(F16, 2, 8, 4, 64, None, 64, FAKE, 16, FAKE, 8, None) == _abi.SSG_ERR_NULL
    assert c(F16, 2, 8, 4, 64, FAKE, 64, FAKE, 16, None, 8, None) == _abi.SSG_ERR_NULL
    assert c(F32, 2, 8, 4, 64, FAKE, 64, FAKE, 16, FAKE, 8, None) == _abi.SSG_ERR_DTYPE
    assert c(I8, 1, 4, 0, 64, FAKE, 64, FAKE, 16, FAKE, 8, None) == 0          # nothing to do
    assert lib.ssg_decompress_nm(F16, 2, 8, 4, 64, FAKE, 16, FAKE, 8, FAKE, 63, None, None) == _abi.SSG_ERR_STRIDE
    p = lib.ssg_spmm_nm
    ok = (FAKE, 16, FAKE, 8, FAKE, 16, FAKE, 16, None)
    assert p(F16, I32, 2, 8, 8, 16, 64, *ok) == _abi.SSG_ERR_DTYPE
    assert p(F16, F32, 3, 8, 8, 16, 64, *ok) == _abi.SSG_ERR_SHAPE
    assert p(F16, F32, 2, 8, 8, 16, 64, FAKE, 20, FAKE, 8, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_STRIDE  # 40-byte vals rows
    assert p(F16, F32, 2, 8, 8, 16, 64, FAKE, 16, FAKE, 12, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_STRIDE  # mask rows
    assert p(F16, F32, 2, 8, 8, 12, 64, FAKE, 16, FAKE, 8, FAKE, 12, FAKE, 12, None) == _abi.SSG_ERR_STRIDE  # 24-byte B rows
    assert p(F16, F32, 2, 8, 8, 16, 64, ctypes.c_void_p(0x1008), 16, FAKE, 8, FAKE, 16, FAKE, 16,
             None) == _abi.SSG_ERR_STRIDE
    assert p(F16, F32, 2, 8, 8, 16, 64, FAKE, 16, FAKE, 8, None, 16, FAKE, 16, None) == _abi.SSG_ERR_NULL
    assert p(F16, F32, 2, 8, 8, 16, 64, FAKE, 16, FAKE, 8, FAKE, 16, None, 16, None) == _abi.SSG_ERR_NULL
    assert p(F16, F32, 2, 8, 8, 16 * 65536, 64, FAKE, 16, FAKE, 8, FAKE, 16 * 65536, FAKE, 16 * 65536,
             None) == _abi.SSG_ERR_SHAPE
    assert p(F16, F32, 2, 8, 0, 16, 64, *ok) == 0                           # M == 0: nothing to do
    # packed layout: sizes by their closed form, argument errors
    vb, mb = ctypes.c_int64(0), ctypes.c_int64(0)
    for dt, n, m, M, K, want in [(F16, 1, 4, 11008, 4096, (688 * 32 * 1024, 688 * 32 * 64 * 4)),
                                 (F16, 2, 4, 20, 100, (2 * 2 * 1024, 2 * 2 * 64 * 2)),
                                 (I8, 2, 8, 16, 4096, (1 * 16 * 1024, 1 * 16 * 64 * 8)),
                                 (I8, 4, 8, 17, 128, (2 * 1 * 1024, 2 * 1 * 64 * 4))]:
        assert lib.ssg_nm_packed_sizes(dt, n, m, M, K, ctypes.byref(vb), ctypes.byref(mb)) == 0
        assert (vb.value, mb.value) == want
    assert lib.ssg_nm_packed_sizes(F16, 3, 8, 16, 64, ctypes.byref(vb), ctypes.byref(mb)) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_nm_packed_sizes(F16, 2, 8, 16, 64, None, ctypes.byref(mb)) == _abi.SSG_ERR_NULL
    q = lib.ssg_spmm_nm_packed
    assert q(F16, F32, 2, 8, 8, 16, 0, FAKE, FAKE, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_SHAPE
    assert q(F16, F32, 2, 8, 8, 16, 64, ctypes.c_void_p(0x1004), FAKE, FAKE, 16, FAKE, 16,
             None) == _abi.SSG_ERR_STRIDE
    assert q(F16, F32, 2, 8, 8, 16, 64, FAKE, FAKE, FAKE, 12, FAKE, 16, None) == _abi.SSG_ERR_STRIDE
    assert q(F16, F32, 2, 8, 8, 16, 64, None, FAKE, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_NULL
    assert lib.ssg_pack_nm_decode(F16, 2, 8, 8, 64, FAKE, 16, FAKE, 8, None, FAKE, None) == _abi.SSG_ERR_NULL


def test_last_error_names_the_problem(lib):
    assert lib.ssg_compress_2to4(F16, 4, 8, FAKE, 7, FAKE, 4, FAKE, 1, None) == _abi.SSG_ERR_STRIDE
    assert "lda=7" in lib.ssg_last_error().decode()


def test_zero_size_is_a_no_op(lib):
    # M == 0 or K == 0: nothing is enqueued, so this succeeds without a GPU
    assert lib.ssg_compress_2to4(F16, 0, 8, FAKE, 8, FAKE, 4, FAKE, 1, None) == 0
    assert lib.ssg_compress_2to4(F16, 5, 0, None, 0, None, 0, None, 0, None) == 0
    assert lib.ssg_prune_2to4(I8, 0, 8, FAKE, 8, FAKE, 8, None) == 0
    assert lib.ssg_spmm_2to4(F16, F32, 0, 16, 64, FAKE, 32, FAKE, 8, FAKE, 16, FAKE, 16, None, 0, None) == 0
    assert lib.ssg_spmm_2to4(F16, F32, 8, 0, 64, FAKE, 32, FAKE, 8, FAKE, 0, FAKE, 0, None, 0, None) == 0


def test_spmm_argument_errors(lib):
    f = lib.ssg_spmm_2to4
    ok = dict(M=8, N=16, K=64)
    # (input, output) type pairs
    for ab, c in [(F16, I32), (I8, F32), (F32, F32), (BF16, 5)]:
        assert f(ab, c, 8, 16, 64, FAKE, 32, FAKE, 8, FAKE, 16, FAKE, 16, None, 0, None) == _abi.SSG_ERR_DTYPE
    assert f(F16, F32, 8, 16, 62, FAKE, 31, FAKE, 8, FAKE, 16, FAKE, 16, None, 0, None) == _abi.SSG_ERR_SHAPE
    assert f(F16, F32, 8, 16, 64, FAKE, 31, FAKE, 8, FAKE, 16, FAKE, 16, None, 0, None) == _abi.SSG_ERR_STRIDE
    assert f(F16, F32, 8, 16, 64, FAKE, 32, FAKE, 7, FAKE, 16, FAKE, 16, None, 0, None) == _abi.SSG_ERR_STRIDE
    assert f(F16, F32, 8, 16, 64, FAKE, 32, FAKE, 8, FAKE, 15, FAKE, 16, None, 0, None) == _abi.SSG_ERR_STRIDE
    assert f(F16, F32, 8, 16, 64, FAKE, 32, FAKE, 8, FAKE, 16, FAKE, 15, None, 0, None) == _abi.SSG_ERR_STRIDE
    assert f(F16, F32, 8, 16, 64, None, 32, FAKE, 8, FAKE, 16, FAKE, 16, None, 0, None) == _abi.SSG_ERR_NULL
    assert f(F16, F32, 8, 16, 64, FAKE, 32, FAKE, 8, None, 16, FAKE, 16, None, 0, None) == _abi.SSG_ERR_NULL
    assert f(F16, F32, 8, 16, 64, FAKE, 32, FAKE, 8, FAKE, 16, None, 16, None, 0, None) == _abi.SSG_ERR_NULL
    r = lib.ssg_spmm_2to4_residual
    assert r(F16, F32, 8, 16, 64, FAKE, 32, FAKE, 8, FAKE, FAKE, FAKE, -1, FAKE, 16, FAKE, 16, None, 0,
             None) == _abi.SSG_ERR_FORMAT
    assert r(F16, F32, 8, 16, 64, FAKE, 32, FAKE, 8, None, FAKE, FAKE, 4, FAKE, 16, FAKE, 16, None, 0,
             None) == _abi.SSG_ERR_NULL
    assert r(F16, F32, 8, 16, 64, FAKE, 32, FAKE, 8, FAKE, None, FAKE, 4, FAKE, 16, FAKE, 16, None, 0,
             None) == _abi.SSG_ERR_NULL
    e = lib.ssg_spmm_2to4_ex
    assert e(99, F16, F32, 8, 16, 64, FAKE, 32, FAKE, 8, FAKE, 16, FAKE, 16, None, 0, None) == _abi.SSG_ERR_ALGO
    del ok


def test_python_binding_has_no_cpu_fallback():
    A = torch.zeros((4, 8), dtype=torch.float16)
    with pytest.raises(ssg.SsgError):
        ssg.compress(A)
    with pytest.raises(ssg.SsgError):
        ssg.spmm(torch.zeros((4, 4), dtype=torch.float16), torch.zeros((4, 1), dtype=torch.uint8),
                 torch.zeros((8, 2), dtype=torch.float16))


def test_python_binding_names_match_the_abi():
    for name in declared_functions():
        if name in ("ssg_abi_version", "ssg_status_str", "ssg_last_error", "ssg_vals_cols", "ssg_meta_cols",
                    "ssg_nm_vals_cols",
                    "ssg_spmm_2to4_ex", "ssg_spmm_2to4_residual_ex", "ssg_spmm_2to4_residual_delta_ex"):
            continue
        assert hasattr(ssg, name), name


def test_prefill_argument_errors(lib):
    E4M3 = _abi.SSG_E4M3
    vb, mb = ctypes.c_int64(-1), ctypes.c_int64(-1)
    # sizes: 256-row tiles x K/2*s bytes of values; 8 KiB per tile and 256 dense k of metadata
    for dt, M, K, v, m in [(F16, 300, 192, 2 * 256 * 192, 2 * 8192), (I8, 256, 4096, 256 * 2048, 16 * 8192),
                           (E4M3, 1, 384, 256 * 192, 2 * 8192), (BF16, 0, 64, 0, 0)]:
        assert lib.ssg_prefill_packed_sizes(dt, M, K, ctypes.byref(vb), ctypes.byref(mb)) == 0
        assert (vb.value, mb.value) == (v, m)
    # K not a multiple of the stage (64 dense k for 16-bit, 128 for 8-bit)
    assert lib.ssg_prefill_packed_sizes(F16, 8, 96, ctypes.byref(vb), ctypes.byref(mb)) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_prefill_packed_sizes(I8, 8, 64, ctypes.byref(vb), ctypes.byref(mb)) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_prefill_packed_sizes(F32, 8, 64, ctypes.byref(vb), ctypes.byref(mb)) == _abi.SSG_ERR_DTYPE
    assert lib.ssg_prefill_packed_sizes(F16, 8, 64, None, None) == _abi.SSG_ERR_NULL
    c = lib.ssg_compress_2to4_prefill
    assert c(F16, 8, 96, FAKE, 96, FAKE, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert c(F16, 8, 64, FAKE, 63, FAKE, FAKE, None) == _abi.SSG_ERR_STRIDE
    assert c(F16, 8, 64, FAKE, 64, None, FAKE, None) == _abi.SSG_ERR_NULL
    assert c(F16, 8, 64, FAKE, 64, ctypes.c_void_p(0x1008), FAKE, None) == _abi.SSG_ERR_STRIDE
    assert c(F16, 0, 64, FAKE, 64, None, None, None) == 0          # nothing to write
    p = lib.ssg_pack_2to4_prefill
    assert p(I8, 8, 128, FAKE, 63, FAKE, 16, FAKE, FAKE, None) == _abi.SSG_ERR_STRIDE
    assert p(I8, 8, 128, FAKE, 64, FAKE, 15, FAKE, FAKE, None) == _abi.SSG_ERR_STRIDE
    assert p(I8, 8, 128, ctypes.c_void_p(0x1004), 64, FAKE, 16, FAKE, FAKE, None) == _abi.SSG_ERR_STRIDE
    s = lib.ssg_spmm_2to4_prefill
    assert s(F16, I32, 8, 16, 64, FAKE, FAKE, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_DTYPE
    assert s(F16, F32, 8, 16, 96, FAKE, FAKE, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_SHAPE
    assert s(F16, F32, 8, 16, 64, FAKE, FAKE, FAKE, 15, FAKE, 16, None) == _abi.SSG_ERR_STRIDE
    assert s(F16, F32, 8, 16, 64, FAKE, FAKE, FAKE, 16, FAKE, 15, None) == _abi.SSG_ERR_STRIDE
    assert s(F16, F32, 8, 16, 64, None, FAKE, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_NULL
    assert s(I8, I32, 8, 8, 128, FAKE, FAKE, FAKE, 8, FAKE, 8, None) == _abi.SSG_ERR_ALGO   # N % 16
    assert s(F16, F32, 8, 12, 64, FAKE, FAKE, FAKE, 12, FAKE, 12, None) == _abi.SSG_ERR_ALGO   # N % 8
    assert s(F16, F32, 0, 16, 64, None, None, None, 16, None, 16, None) == 0


def test_packed_residual_argument_errors(lib):
    r = lib.ssg_spmm_2to4_packed_residual
    d = lib.ssg_spmm_2to4_packed_residual_delta
    assert r(F16, F32, 32, 16, 128, FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_FORMAT
    assert r(F16, F32, 32, 16, 128, FAKE, FAKE, None, FAKE, FAKE, 4, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_NULL
    assert r(F16, F32, 32, 16, 128, FAKE, FAKE, FAKE, None, FAKE, 4, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_NULL
    assert r(F16, I32, 32, 16, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_DTYPE
    assert r(F16, F32, 32, 16, 96, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_SHAPE
    assert r(F16, F32, 32, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 8, FAKE, 8, None) == _abi.SSG_ERR_ALGO
    # column indices not aligned to 4 entries (16 bytes)
    assert r(F16, F32, 32, 16, 128, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1004), FAKE, 4, FAKE, 16, FAKE, 16,
             None) == _abi.SSG_ERR_ALGO
    assert d(F16, F32, 32, 16, 128, FAKE, FAKE, FAKE, FAKE, None, 4, FAKE, 16, FAKE, 16, None) == _abi.SSG_ERR_NULL
    assert d(F16, F32, 32, 16, 128, FAKE, FAKE, FAKE, ctypes.c_void_p(0x1002), FAKE, 4, FAKE, 16, FAKE, 16,
             None) == _abi.SSG_ERR_ALGO
    assert r(F16, F32, 0, 16, 128, None, None, None, None, None, 0, FAKE, 16, None, 16, None) == 0


def test_mfma_probe_description_and_argument_errors(lib):
    # ten forms: sparse / dense pairs; the dense-equivalent operation count of
    # a launch is 2 * rows * columns * dense k per instruction, times the
    # accumulators per round (8 at 32x32, 16 at 16x16), rounds, waves
    forms = lib.ssg_mfma_probe_forms()
    assert forms == 10
    names = [lib.ssg_mfma_probe_name(f).decode() for f in range(forms)]
    assert names[0] == "v_smfmac_f32_32x32x32_bf16" and names[1] == "v_mfma_f32_32x32x16_bf16"
    assert all(n.startswith("v_smfmac_") for n in names[0::2]) and all(n.startswith("v_mfma_") for n in names[1::2])
    assert lib.ssg_mfma_probe_name(-1) is None and lib.ssg_mfma_probe_name(forms) is None
    assert lib.ssg_mfma_probe_ops(0, 256, 2000) == 2 * 32 * 32 * 32 * 8 * 2000 * 256 * 4
    assert lib.ssg_mfma_probe_ops(1, 256, 2000) == 2 * 32 * 32 * 16 * 8 * 2000 * 256 * 4
    assert lib.ssg_mfma_probe_ops(6, 3, 5) == 2 * 16 * 16 * 128 * 16 * 5 * 3 * 4
    # a sparse form covers twice the dense k of its dense partner (fp8: the
    # dense 32x32x64 form covers the same k)
    for f in (0, 2, 4, 6):
        assert lib.ssg_mfma_probe_ops(f, 1, 1) == 2 * lib.ssg_mfma_probe_ops(f + 1, 1, 1)
    assert lib.ssg_mfma_probe_ops(8, 1, 1) == lib.ssg_mfma_probe_ops(9, 1, 1)
    assert lib.ssg_mfma_probe_ops(forms, 1, 1) == 0 and lib.ssg_mfma_probe_ops(0, 0, 1) == 0
    assert lib.ssg_mfma_probe(forms, 1, 1, FAKE, None) == _abi.SSG_ERR_ALGO
    assert lib.ssg_mfma_probe(0, 0, 1, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_mfma_probe(0, 1, 0, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert lib.ssg_mfma_probe(0, 1, 1, None, None) == _abi.SSG_ERR_NULL


def test_lds_read_probe_argument_errors(lib):
    good = (ctypes.c_uint32 * 64)(*[16 * l for l in range(64)])
    bad_align = (ctypes.c_uint32 * 64)(*([16 * l for l in range(63)] + [8]))
    too_far = (ctypes.c_uint32 * 64)(*([16 * l for l in range(63)] + [65536 - 7 * 4096]))
    last_ok = (ctypes.c_uint32 * 64)(*([16 * l for l in range(63)] + [65536 - 7 * 4096 - 16]))
    f = lib.ssg_lds_read_probe
    cast = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert f(None, 1, 1, FAKE, None) == _abi.SSG_ERR_NULL
    assert f(cast(good), 1, 1, None, None) == _abi.SSG_ERR_NULL
    assert f(cast(good), 0, 1, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert f(cast(good), 1, 0, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert f(cast(bad_align), 1, 1, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert f(cast(too_far), 1, 1, FAKE, None) == _abi.SSG_ERR_SHAPE
    assert f(cast(last_ok), 0, 1, FAKE, None) == _abi.SSG_ERR_SHAPE      # only the count is wrong
    assert b"workgroups" in lib.ssg_last_error()


def test_prefill_bt_argument_errors(lib):
    f = lib.ssg_spmm_2to4_prefill_bt
    assert f(BF16, F32, 64, 16, 128, FAKE, FAKE, FAKE, 100, FAKE, 16, None) == _abi.SSG_ERR_STRIDE   # ldbt < K
    assert f(BF16, F32, 64, 16, 128, FAKE, FAKE, FAKE, 128, FAKE, 8, None) == _abi.SSG_ERR_STRIDE    # ldc < N
    assert f(BF16, F32, 64, 16, 96, FAKE, FAKE, FAKE, 128, FAKE, 16, None) == _abi.SSG_ERR_SHAPE     # K % 64
    assert f(BF16, I32, 64, 16, 128, FAKE, FAKE, FAKE, 128, FAKE, 16, None) == _abi.SSG_ERR_DTYPE
    assert f(BF16, F32, 64, 16, 128, FAKE, FAKE, None, 128, FAKE, 16, None) == _abi.SSG_ERR_NULL
    # rows of Bt 8 bytes apart from a multiple of 16; Bt misaligned
    assert f(BF16, F32, 64, 16, 128, FAKE, FAKE, FAKE, 132, FAKE, 16, None) == _abi.SSG_ERR_ALGO
    assert f(BF16, F32, 64, 16, 128, FAKE, FAKE, ctypes.c_void_p(0x1008), 128, FAKE, 16, None) == _abi.SSG_ERR_ALGO
    assert f(BF16, F32, 64, 0, 128, None, None, None, 128, None, 0, None) == 0                       # N = 0


def test_decode_bt_argument_errors(lib):
    f = lib.ssg_spmm_2to4_packed_bt
    g = lib.ssg_spmm_2to4_packed_residual_cbm_bt
    assert f(F16, F32, 32, 17, 128, FAKE, FAKE, FAKE, 128, FAKE, 17, None) == _abi.SSG_ERR_ALGO     # N > 16
    assert f(F16, F32, 32, 8, 128, FAKE, FAKE, FAKE, 100, FAKE, 8, None) == _abi.SSG_ERR_STRIDE     # ldbt < K
    assert f(F16, F32, 32, 8, 128, FAKE, FAKE, FAKE, 132, FAKE, 8, None) == _abi.SSG_ERR_STRIDE     # rows 264 B apart
    assert f(F16, F32, 32, 8, 128, FAKE, FAKE, ctypes.c_void_p(0x1008), 128, FAKE, 8, None) == _abi.SSG_ERR_STRIDE
    assert f(F16, F32, 32, 8, 96, FAKE, FAKE, FAKE, 128, FAKE, 8, None) == _abi.SSG_ERR_SHAPE       # K % 64
    assert f(F16, F32, 32, 8, 128, FAKE, FAKE, None, 128, FAKE, 8, None) == _abi.SSG_ERR_NULL
    assert f(F16, F32, 32, 0, 128, None, None, None, 128, None, 0, None) == 0                       # N = 0
    assert g(F16, F32, 32, 17, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 128, FAKE, 17, None) == _abi.SSG_ERR_ALGO
    assert g(F16, F32, 32, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, 100, FAKE, 8, None) == _abi.SSG_ERR_STRIDE
    assert g(F16, F32, 32, 8, 128, FAKE, FAKE, None, FAKE, FAKE, 4, FAKE, 128, FAKE, 8, None) == _abi.SSG_ERR_NULL
