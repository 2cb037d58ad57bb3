"""The product that allocates nothing (ssg_spmm_2to4_noalloc), through the C
ABI: it must give the same bits as ssg_spmm_2to4 with a caller workspace,
call after call on the same device (its scratch keeps the previous call's
contents), and reject a padded B larger than its scratch.  Named to run
last: it must pass after the other GPU tests as well as alone."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from structured_sparse_gemm_amd import _abi
import structured_sparse_gemm_amd as ssg
from tests import _util as U
import workloads as W

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    torch.cuda.init()
    return _abi.load()


OUT = {"f16": (_abi.SSG_F32, torch.float32), "bf16": (_abi.SSG_F32, torch.float32),
       "i8": (_abi.SSG_I32, torch.int32), "e4m3": (_abi.SSG_F32, torch.float32)}
AB = {"f16": _abi.SSG_F16, "bf16": _abi.SSG_BF16, "i8": _abi.SSG_I8, "e4m3": _abi.SSG_E4M3}


def operands(dt, M, K, N, seed):
    a = U.random_matrix(dt, M, K, "normal", seed=seed)
    b = U.random_matrix(dt, K, N, "normal", seed=seed + 1)
    vals, meta = oracle.compress(dt, a)
    V = W.from_bits(vals, dt).cuda()
    Mt = torch.from_numpy(np.ascontiguousarray(meta)).cuda()
    # a strided B (row stride N + 3), so the padded copy is what the kernel reads
    Bbuf = torch.zeros((K, N + 3), dtype=W.TORCH_DTYPE[dt], device="cuda")
    Bbuf[:, :N] = W.from_bits(b, dt).cuda()
    return V, Mt, Bbuf[:, :N], (vals, meta, b)


def noalloc(lib, dt, V, Mt, B, C):
    M, N, K = V.shape[0], B.shape[1], B.shape[0]
    s = torch.cuda.current_stream().cuda_stream
    return lib.ssg_spmm_2to4_noalloc(AB[dt], OUT[dt][0], M, N, K, V.data_ptr(), V.stride(0), Mt.data_ptr(),
                                     Mt.stride(0), B.data_ptr(), B.stride(0), C.data_ptr(), C.stride(0), s)


@pytest.mark.parametrize("dt", ["f16", "i8", "bf16", "e4m3"])
def test_noalloc_matches_the_workspace_product(lib, dt):
    # two calls in a row, the second smaller, then the first shape again
    for M, K, N, seed in [(1000, 2048, 5, 11), (300, 1024, 3, 17), (1000, 2048, 5, 23)]:
        V, Mt, B, (vals, meta, b) = operands(dt, M, K, N, seed)
        C_ref = torch.empty((M, N), dtype=OUT[dt][1], device="cuda")
        ssg.ssg_spmm_2to4(V, Mt, B, C_ref)                      # caller workspace, from torch
        C = torch.full((M, N), -7, dtype=OUT[dt][1], device="cuda")
        assert noalloc(lib, dt, V, Mt, B, C) == 0, lib.ssg_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(C, C_ref), (dt, M, K, N)
        # and both within the bar against the oracle
        cref, sref = oracle.spmm(dt, vals, meta, b, K)
        c = C.cpu().numpy().astype(np.float64)
        if dt == "i8":
            assert np.array_equal(c.astype(np.int64), cref)
        else:
            assert np.linalg.norm(c - cref) <= 1e-3 * np.linalg.norm(cref)
            assert (np.abs(c - cref) <= 1e-2 * sref).all()


def test_noalloc_without_padding_uses_no_scratch(lib):
    # N == 16: nothing is padded; the call is the plain product
    V, Mt, B, _ = operands("f16", 64, 512, 16, 31)
    B = B.contiguous()
    C_ref = torch.empty((64, 16), dtype=torch.float32, device="cuda")
    ssg.ssg_spmm_2to4(V, Mt, B, C_ref)
    C = torch.empty_like(C_ref)
    assert noalloc(lib, "f16", V, Mt, B, C) == 0
    torch.cuda.synchronize()
    assert torch.equal(C, C_ref)


def test_noalloc_rejects_a_padded_b_beyond_its_scratch(lib):
    cap = lib.ssg_noalloc_scratch_bytes()
    assert cap == 2 << 20
    K = cap // (16 * 2) + 64                                    # 16-bit B of K x 16 past the scratch
    FAKE = ctypes.c_void_p(0x1000)
    rc = lib.ssg_spmm_2to4_noalloc(_abi.SSG_F16, _abi.SSG_F32, 8, 5, K, FAKE, K // 2, FAKE, K // 8, FAKE, 5, FAKE,
                                   5, None)
    assert rc == _abi.SSG_ERR_WORKSPACE
    assert "scratch" in lib.ssg_last_error().decode()
