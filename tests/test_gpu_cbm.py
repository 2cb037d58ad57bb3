"""The complement-bitmap residual through the C ABI: the GPU encoder against
the oracle's (bit-exact), and the packed decode product with the residual
fused into its k-steps against the oracle's product of the same split
(int8 exact; floats within the stated tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_amd as ssg
import workloads as W
from tests import _util as U
from tests.test_gpu_parity import check_product, dev_or_empty, to_dev, to_host

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "i8", "e4m3", "e5m2"]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    torch.cuda.init()
    return torch.device("cuda:0")


def ks_of(dt):
    return 64 if dt in ("f16", "bf16") else 128


def shapes_for(dt):
    ks = ks_of(dt)
    # one k-step; ragged tiles; one and two tiles per workgroup; more
    # workgroups than CUs
    return [(16, ks), (40, 4 * ks), (33, 8 * ks), (300, 16 * ks), (1000, 2 * ks), (4100, 4 * ks), (16400, ks)]


def gpu_pack(dt, meta, row_ptr, col, rvals, M, K, bad=None):
    rp = torch.from_numpy(np.ascontiguousarray(row_ptr)).cuda()
    cl = torch.from_numpy(np.ascontiguousarray(col)).cuda()
    rv = to_dev(rvals, dt) if len(rvals) else torch.empty(0, dtype=W.TORCH_DTYPE[dt], device="cuda")
    mt = torch.from_numpy(np.ascontiguousarray(meta)).cuda()
    mb, nb = ssg.ssg_cbm_sizes(W.TORCH_DTYPE[dt], M, K)
    rmask = torch.full((mb,), 0xA5, dtype=torch.uint8, device="cuda")      # unwritten bytes would show
    roff = torch.full((nb + 1,), -7, dtype=torch.int32, device="cuda")
    es = torch.empty((), dtype=W.TORCH_DTYPE[dt]).element_size()
    nnz = len(col)
    cv = torch.full((-(-max(nnz, 1) * es // 16) * 16 // es,), 0, dtype=W.TORCH_DTYPE[dt], device="cuda")
    cv.view(torch.uint8).fill_(0xA5)
    cv = cv[:nnz]
    ssg.ssg_pack_residual_cbm(mt, rp, cl, rv, K, rmask, roff, cv, bad_count=bad)
    return rmask, roff, cv


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("fam", ["sparse", "normal", "ties"])
@pytest.mark.parametrize("which", range(7))
def test_cbm_pack_bitexact(dt, fam, which):
    M, K = shapes_for(dt)[which]
    a = U.random_matrix(dt, M, K, fam, seed=M + 3 * K + which)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    want = oracle.cbm_encode(dt, meta, row_ptr, col, rvals, M, K)
    rmask, roff, cv = gpu_pack(dt, meta, row_ptr, col, rvals, M, K)
    assert np.array_equal(rmask.cpu().numpy(), want[0]), "rmask"
    assert np.array_equal(roff.cpu().numpy(), want[1]), "roff"
    assert np.array_equal(np.asarray(to_host(cv)).view(np.uint8), np.asarray(want[2]).view(np.uint8)), "cvals"


def test_cbm_pack_counts_entries_at_kept_positions():
    dt, M, K = "f16", 16, 64
    a = np.zeros((M, K))
    a[0, :4] = [1, 2, 3, 4]                                 # keeps positions 2 and 3
    a[3, 8:12] = [0, 5, 0, 6]
    vals, meta, row_ptr, col, rvals = oracle.split(dt, U.encode(dt, a))
    # a CSR with one more entry, at kept position 3 of row 0
    row_ptr2 = row_ptr.copy()
    row_ptr2[1:] += 1
    col2 = np.concatenate([col[:row_ptr[1]], [3], col[row_ptr[1]:]]).astype(np.int32)
    rv2 = np.concatenate([rvals[:row_ptr[1]], U.encode(dt, [9.0]), rvals[row_ptr[1]:]])
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    rmask, roff, cv = gpu_pack(dt, meta, row_ptr2, col2, rv2, M, K, bad=bad)
    assert int(bad.item()) == 1
    want = oracle.cbm_encode(dt, meta, row_ptr, col, rvals, M, K)
    assert np.array_equal(rmask.cpu().numpy(), want[0]) and np.array_equal(roff.cpu().numpy(), want[1])
    assert np.array_equal(np.asarray(to_host(cv[:int(roff[-1])])).view(np.uint8), np.asarray(want[2]).view(np.uint8))


def product(dt, a, M, K, b):
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    rmask, roff, cv = gpu_pack(dt, meta, row_ptr, col, rvals, M, K)
    C = ssg.spmm_packed_residual_cbm(pv, pm, M, rmask, roff, cv, to_dev(b, dt))
    cref, sref = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, b, K)
    return C, cref, sref, (vals, meta, row_ptr, col, rvals)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("fam", ["sparse", "normal"])
@pytest.mark.parametrize("which", range(7))
def test_spmm_packed_residual_cbm_matches_oracle(dt, fam, which):
    # "normal" has no zeros: every group holds two residual values, the
    # largest value windows (512 values per block for 16-bit types)
    M, K = shapes_for(dt)[which]
    a = U.random_matrix(dt, M, K, fam, seed=M + 5 * K + which)
    b = U.random_matrix(dt, K, 16, "normal", seed=K + which)
    C, cref, sref, _ = product(dt, a, M, K, b)
    check_product(dt, C.cpu().numpy(), cref, sref, "cbm %s %s %s" % (dt, fam, (M, K)))


@pytest.mark.parametrize("dt", ["f16", "bf16", "i8"])
def test_spmm_packed_residual_cbm_exact_small_integers(dt):
    # small integers: every product and partial sum exact in fp32, so the
    # fused product equals the oracle's exactly, residual included
    ks = ks_of(dt)
    M, K = 300, 16 * ks
    rng = np.random.default_rng(13)
    dense = rng.integers(-3, 4, size=(M, K)) * (rng.random((M, K)) < 0.5)
    a = U.encode(dt, dense.astype(np.float64))
    b = U.encode(dt, rng.integers(-3, 4, size=(K, 16)).astype(np.float64))
    C, cref, _, _ = product(dt, a, M, K, b)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), np.asarray(cref, dtype=np.float64))


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_spmm_packed_residual_cbm_empty_residual(dt):
    # a matrix already 2:4: no residual values; the product is the plain one
    ks = ks_of(dt)
    M, K = 100, 4 * ks
    a = U.random_matrix(dt, M, K, "normal", seed=17)
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    row_ptr = np.zeros(M + 1, np.int32)
    rmask, roff, cv = gpu_pack(dt, meta, row_ptr, np.zeros(0, np.int32), np.zeros(0, U.store_dtype(dt)), M, K)
    assert int(roff[-1]) == 0 and int(rmask.sum()) == 0
    b = U.random_matrix(dt, K, 16, "normal", seed=19)
    C = ssg.spmm_packed_residual_cbm(pv, pm, M, rmask, roff, cv, to_dev(b, dt))
    C_plain = ssg.spmm_packed(pv, pm, M, to_dev(b, dt))
    assert torch.equal(C, C_plain)


def test_spmm_packed_residual_cbm_int8_equals_csr_products():
    # integer sums: the fused product, the CSR residual epilogue and the
    # row-major ring kernel all give the same bits
    dt, M, K = "i8", 1000, 1024
    a = U.random_matrix(dt, M, K, "sparse", seed=23)
    b = U.random_matrix(dt, K, 16, "normal", seed=29)
    C, cref, _, (vals, meta, row_ptr, col, rvals) = product(dt, a, M, K, b)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    C_csr = ssg.spmm_packed_residual(pv, pm, M, dev_or_empty(row_ptr), dev_or_empty(col), dev_or_empty(rvals, dt),
                                     to_dev(b, dt))
    assert torch.equal(C, C_csr)
    assert np.array_equal(C.cpu().numpy().astype(np.int64), cref)


def test_full_size_residual_cbm():
    # the moderately-unstructured workload end to end on the GPU (split,
    # pack, encode, fused product), every output against the oracle
    w = W.WORKLOADS["c5"]
    print("full-size complement-bitmap residual: %s" % w.title, flush=True)
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    a, b = W.bits(a_cpu), W.bits(b_cpu)
    vals, meta, row_ptr, col, rvals = ssg.split(a_cpu.cuda())
    pv, pm = ssg.pack_decode(vals, meta, w.K)
    rmask, roff, cv = ssg.pack_residual_cbm(meta, row_ptr, col, rvals, w.K)
    C = ssg.spmm_packed_residual_cbm(pv, pm, w.M, rmask, roff, cv, b_cpu.cuda()).cpu().numpy()
    r = oracle.split(w.dtype, a)
    enc = oracle.cbm_encode(w.dtype, r[1], r[2], r[3], r[4], w.M, w.K)
    assert np.array_equal(rmask.cpu().numpy(), enc[0]) and np.array_equal(roff.cpu().numpy(), enc[1])
    assert np.array_equal(np.asarray(to_host(cv)).view(np.uint8), np.asarray(enc[2]).view(np.uint8))
    cref, sref = oracle.spmm_residual(w.dtype, *r, b, w.K)
    check_product(w.dtype, C, cref, sref, "c5 complement-bitmap residual (all outputs)")


def test_cbm_argument_errors():
    f16 = torch.float16
    with pytest.raises(ssg.SsgError) as e:                  # K not a multiple of the k-step
        ssg.ssg_cbm_sizes(f16, 16, 96)
    assert e.value.status == 2
    a = U.random_matrix("f16", 32, 128, "sparse", 1)
    vals, meta, row_ptr, col, rvals = oracle.split("f16", a)
    pv, pm = ssg.pack_decode(to_dev(vals, "f16"), dev_or_empty(meta), 128)
    rmask, roff, cv = gpu_pack("f16", meta, row_ptr, col, rvals, 32, 128)
    b8 = to_dev(U.random_matrix("f16", 128, 8, "normal", 2), "f16")
    with pytest.raises(ssg.SsgError) as e:                  # the packed product takes N == 16
        ssg.spmm_packed_residual_cbm(pv, pm, 32, rmask, roff, cv, b8)
    assert e.value.status == 8
    if cv.numel() > 1:
        with pytest.raises(ssg.SsgError) as e:              # values not 16-byte aligned
            ssg.spmm_packed_residual_cbm(pv, pm, 32, rmask, roff, cv[1:],
                                         to_dev(U.random_matrix("f16", 128, 16, "normal", 3), "f16"))
        assert e.value.status == 3
