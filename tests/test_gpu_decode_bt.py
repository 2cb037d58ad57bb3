"""The decode-shape products on activation-major B (Bt [N, K] row-major, the
token-major activations of a decode step) through the C ABI: the packed
decode product and the one with the complement-bitmap residual fused, each
against the oracle of C = A B with B = Bt^T, at any N from 1 to 16, and with
the same bits as the row-major-B products where those take the shape."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_amd as ssg
import workloads as W
from tests import _util as U
from tests.test_gpu_cbm import gpu_pack, ks_of
from tests.test_gpu_parity import check_product, dev_or_empty, to_dev

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "i8", "e4m3", "e5m2"]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    torch.cuda.init()
    return torch.device("cuda:0")


def shapes_for(dt):
    # (M, k-steps, N): one tile and one k-step; ragged tiles; 1..4 tiles per
    # workgroup; more workgroups than CUs; N from 1 to 16
    return [(16, 1, 16), (40, 4, 1), (33, 8, 5), (300, 16, 16), (1000, 2, 8), (4100, 4, 15), (16400, 1, 16)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("which", range(7))
def test_spmm_packed_bt_matches_oracle(dt, which):
    M, steps, N = shapes_for(dt)[which]
    K = steps * ks_of(dt)
    a = U.random_matrix(dt, M, K, "normal", seed=M + 3 * K + which)
    bt = U.random_matrix(dt, N, K, "normal", seed=N + K)
    b = np.ascontiguousarray(np.asarray(bt).T)
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    C = ssg.spmm_packed_bt(pv, pm, M, to_dev(bt, dt))
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "packed Bt %s %s" % (dt, (M, K, N)))
    if N == 16:
        # the same MFMAs on the same operands as the row-major-B product
        C_rm = ssg.spmm_packed(pv, pm, M, to_dev(b, dt))
        assert torch.equal(C.view(torch.int32), C_rm.view(torch.int32))


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_spmm_packed_bt_strided_rows(dt):
    # Bt a column slice of a wider activation matrix (rows ldbt > K apart)
    M, K, N = 700, 8 * ks_of(dt), 12
    a = U.random_matrix(dt, M, K, "normal", seed=51)
    wide = U.random_matrix(dt, N, K + 2 * ks_of(dt), "normal", seed=53)
    off = ks_of(dt)
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    C = ssg.spmm_packed_bt(pv, pm, M, to_dev(wide, dt)[:, off:off + K])
    b = np.ascontiguousarray(np.asarray(wide)[:, off:off + K].T)
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "packed Bt strided %s" % dt)


def test_spmm_packed_bt_exact_small_integers():
    M, K, N = 300, 1024, 7
    rng = np.random.default_rng(29)
    a = rng.integers(-3, 4, size=(M, K)).astype(np.float16).view(np.uint16)
    bt = rng.integers(-3, 4, size=(N, K)).astype(np.float16).view(np.uint16)
    vals, meta = oracle.compress("f16", a)
    pv, pm = ssg.pack_decode(to_dev(vals, "f16"), dev_or_empty(meta), K)
    C = ssg.spmm_packed_bt(pv, pm, M, to_dev(bt, "f16")).cpu().numpy().astype(np.float64)
    cref, _ = oracle.spmm("f16", vals, meta, np.ascontiguousarray(bt.T), K)
    assert np.array_equal(C, cref)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("which", range(7))
def test_spmm_packed_residual_cbm_bt_matches_oracle(dt, which):
    M, steps, N = shapes_for(dt)[which]
    K = steps * ks_of(dt)
    a = U.random_matrix(dt, M, K, "sparse", seed=M + 7 * K + which)
    bt = U.random_matrix(dt, N, K, "normal", seed=N + 2 * K)
    b = np.ascontiguousarray(np.asarray(bt).T)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    rmask, roff, cv = gpu_pack(dt, meta, row_ptr, col, rvals, M, K)
    C = ssg.spmm_packed_residual_cbm_bt(pv, pm, M, rmask, roff, cv, to_dev(bt, dt))
    cref, sref = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "cbm Bt %s %s" % (dt, (M, K, N)))
    if N == 16:
        C_rm = ssg.spmm_packed_residual_cbm(pv, pm, M, rmask, roff, cv, to_dev(b, dt))
        assert torch.equal(C.view(torch.int32), C_rm.view(torch.int32))


def test_full_size_decode_bt():
    # the decode workload and the moderately-unstructured one with
    # token-major activations: every output against the oracle
    w = W.WORKLOADS["c3"]
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    vals, meta = ssg.compress(a_cpu.cuda())
    pv, pm = ssg.pack_decode(vals, meta, w.K)
    C = ssg.spmm_packed_bt(pv, pm, w.M, b_cpu.cuda().t().contiguous()).cpu().numpy()
    r = oracle.compress(w.dtype, W.bits(a_cpu))
    cref, sref = oracle.spmm(w.dtype, r[0], r[1], W.bits(b_cpu), w.K)
    check_product(w.dtype, C, cref, sref, "c3 packed, Bt (all outputs)")

    w = W.WORKLOADS["c5"]
    print("full-size complement-bitmap residual, Bt: %s" % w.title, flush=True)
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    vals, meta, row_ptr, col, rvals = ssg.split(a_cpu.cuda())
    pv, pm = ssg.pack_decode(vals, meta, w.K)
    rmask, roff, cv = ssg.pack_residual_cbm(meta, row_ptr, col, rvals, w.K)
    C = ssg.spmm_packed_residual_cbm_bt(pv, pm, w.M, rmask, roff, cv, b_cpu.cuda().t().contiguous()).cpu().numpy()
    r = oracle.split(w.dtype, W.bits(a_cpu))
    cref, sref = oracle.spmm_residual(w.dtype, *r, W.bits(b_cpu), w.K)
    check_product(w.dtype, C, cref, sref, "c5 complement-bitmap residual, Bt (all outputs)")


def test_decode_bt_argument_errors():
    a = U.random_matrix("f16", 32, 128, "normal", 1)
    vals, meta = oracle.compress("f16", a)
    pv, pm = ssg.pack_decode(to_dev(vals, "f16"), dev_or_empty(meta), 128)
    with pytest.raises(ssg.SsgError) as e:                  # more than 16 columns
        ssg.spmm_packed_bt(pv, pm, 32, to_dev(U.random_matrix("f16", 17, 128, "normal", 2), "f16"))
    assert e.value.status == 8
    wide = to_dev(U.random_matrix("f16", 8, 132, "normal", 3), "f16")
    with pytest.raises(ssg.SsgError) as e:                  # rows 264 bytes apart
        ssg.spmm_packed_bt(pv, pm, 32, wide[:, :128])
    assert e.value.status == 3
