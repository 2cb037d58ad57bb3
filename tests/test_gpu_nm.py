"""Parity of the N:M path (1:4, 2:4, 2:8, 4:8; kept values plus a keep mask)
with the CPU oracle, through the C ABI.

* compression and expansion: bit-exact;
* int8 products: bit-exact (int32 vs int64);
* float products: relative Frobenius error <= 1e-3 and, element by element,
  |C_gpu - C_ref| <= 1e-2 * sum_k |a_mk b_kn|.
"""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_amd as ssg
import workloads as W
from tests import _util as U
from tests.test_gpu_parity import check_product, to_dev, to_host

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "i8", "e4m3", "e5m2"]
PATS = U.NM_PATTERNS
PAT_IDS = ["%d:%d" % p for p in PATS]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    torch.cuda.init()
    return torch.device("cuda:0")


def b_dev(b: np.ndarray, dt: str) -> torch.Tensor:
    """B on the device with rows padded to 16 bytes, as the N:M product takes it."""
    t = to_dev(b, dt)
    es = t.element_size()
    ld = -(-t.shape[1] * es // 16) * 16 // es
    buf = torch.zeros((t.shape[0], max(ld, 1)), dtype=t.dtype, device=t.device)
    buf[:, :t.shape[1]] = t
    return buf[:, :t.shape[1]]


def _ref_product(dt, n, m, a, b, K):
    rv, rmask = oracle.compress_nm(dt, n, m, a)
    return oracle.spmm_nm(dt, n, m, rv, rmask, b, K)


# ------------------------------------------------------------------ compression

@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("pat", PATS, ids=PAT_IDS)
@pytest.mark.parametrize("fam", ["normal", "ties", "sparse", "extreme"])
@pytest.mark.parametrize("shape", [(1, 8), (3, 40), (37, 200), (128, 4096), (33, 8200)])
def test_compress_and_expand_bitexact(dt, pat, fam, shape):
    n, m = pat
    M, K = shape
    a = U.random_matrix(dt, M, K, fam, seed=M * 7 + K + n * 3 + m)
    vals, mask = ssg.compress_nm(to_dev(a, dt), n, m)
    rv, rmask = oracle.compress_nm(dt, n, m, a)
    assert np.array_equal(to_host(vals.contiguous()), rv)
    assert np.array_equal(to_host(mask.contiguous()), rmask)
    D, bad = ssg.decompress_nm(vals, mask, n, m, K, count_bad=True)
    rd, rbad = oracle.decompress_nm(dt, n, m, rv, rmask, K)
    assert bad == rbad == 0
    assert np.array_equal(to_host(D), rd)


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_compress_unaligned_operands_and_bad_masks(dt):
    n, m, M, K = 2, 8, 9, 96
    a = U.random_matrix(dt, M, K, "normal", seed=5)
    base = torch.zeros((M, K + 3), dtype=W.TORCH_DTYPE[dt], device="cuda")
    base[:, 1:1 + K] = to_dev(a, dt)
    A = base[:, 1:1 + K]                                  # unaligned rows: element-wise path
    vb = torch.zeros((M, K // m * n + 5), dtype=A.dtype, device="cuda")
    mb = torch.zeros((M, K // 8 + 3), dtype=torch.uint8, device="cuda")
    vals, mask = vb[:, 1:1 + K // m * n], mb[:, 1:1 + K // 8]
    ssg.ssg_compress_nm(A, n, m, vals, mask)
    rv, rmask = oracle.compress_nm(dt, n, m, a)
    assert np.array_equal(to_host(vals.contiguous()), rv)
    assert np.array_equal(to_host(mask.contiguous()), rmask)
    bits = vb.view(torch.uint8) if vb.element_size() == 1 else vb.view(torch.int16)
    assert not bits[:, :1].any() and not bits[:, 1 + K // m * n:].any() and not mb[:, :1].any()
    # groups with the wrong number of mask bits expand to zeros and are counted
    badmask = rmask.copy()
    badmask[2, 0] = 0xFF
    badmask[4, 3] = 0x01
    D, bad = ssg.decompress_nm(vals, torch.from_numpy(badmask).cuda(), n, m, K, count_bad=True)
    rd, rbad = oracle.decompress_nm(dt, n, m, rv, badmask, K)
    assert bad == rbad == 2 and np.array_equal(to_host(D), rd)


# ------------------------------------------------------------------ products

PRODUCT_SHAPES = [
    (1, 64, 16),        # one row
    (37, 264, 5),       # ragged rows, ragged K (not a multiple of a super-step), narrow B
    (100, 1000, 16),
    (300, 2048, 40),    # three column slices of B
    (8200, 512, 16),    # more tiles than workgroups: several tiles per workgroup, ragged last tile
    (2048, 4096, 16),
]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("pat", PATS, ids=PAT_IDS)
@pytest.mark.parametrize("shape", PRODUCT_SHAPES, ids=["x".join(map(str, s)) for s in PRODUCT_SHAPES])
def test_spmm_nm_matches_oracle(dt, pat, shape):
    n, m = pat
    M, K, N = shape
    if K % m:
        K += m - K % m
    a = U.random_matrix(dt, M, K, "normal", seed=M + K + N)
    b = U.random_matrix(dt, K, N, "normal", seed=M * 3 + N)
    vals, mask = ssg.compress_nm(to_dev(a, dt), n, m)
    C = ssg.spmm_nm(vals, mask, n, m, b_dev(b, dt))
    torch.cuda.synchronize()
    c_ref, s_ref = _ref_product(dt, n, m, a, b, K)
    check_product(dt, to_host(C), c_ref, s_ref, "%s %d:%d %s" % (dt, n, m, shape))


@pytest.mark.parametrize("dt", ["f16", "bf16", "e4m3", "e5m2"])
@pytest.mark.parametrize("pat", PATS, ids=PAT_IDS)
def test_spmm_nm_exact_small_integers(dt, pat):
    """Small-integer operands: every product and partial sum is exact in fp32,
    so the float path must match the oracle exactly (a misplaced element or
    B row shows as a hard mismatch, not as rounding)."""
    n, m = pat
    M, K, N = 160, 2304, 16
    rng = np.random.default_rng(11 * n + m)
    a = U.encode(dt, rng.integers(-3, 4, size=(M, K)))
    b = U.encode(dt, rng.integers(-3, 4, size=(K, N)))
    vals, mask = ssg.compress_nm(to_dev(a, dt), n, m)
    C = ssg.spmm_nm(vals, mask, n, m, to_dev(b, dt))
    c_ref, _ = _ref_product(dt, n, m, a, b, K)
    assert np.array_equal(to_host(C).astype(np.float64), c_ref)


@pytest.mark.parametrize("dt", DTS)
def test_spmm_nm_2_of_4_agrees_with_the_2to4_product(dt):
    M, K, N = 512, 2048, 16
    a = U.random_matrix(dt, M, K, "normal", seed=77)
    b = U.random_matrix(dt, K, N, "normal", seed=78)
    A, B = to_dev(a, dt), to_dev(b, dt)
    vals, mask = ssg.compress_nm(A, 2, 4)
    v24, meta = ssg.compress(A)
    assert np.array_equal(to_host(vals.contiguous()), to_host(v24))
    C = ssg.spmm_nm(vals, mask, 2, 4, B)
    C24 = ssg.spmm(v24, meta, B)
    c_ref, s_ref = oracle.spmm(dt, to_host(v24), to_host(meta), b, K)
    check_product(dt, to_host(C), c_ref, s_ref, "nm 2:4")
    check_product(dt, to_host(C24), c_ref, s_ref, "2to4")


@pytest.mark.parametrize("pat", PATS, ids=PAT_IDS)
@pytest.mark.parametrize("dt", ["f16", "i8", "e4m3"])
def test_decode_workload_full_size(dt, pat):
    """The decode workload (11008 x 4096, N = 16) at full size, in the launch
    configuration the benchmark times, compared in full."""
    n, m = pat
    w = W.WORKLOADS["c3nm"]
    w = W.Workload(w.key, w.title, dt, w.M, w.K, w.N, w.index, a_sigma=w.a_sigma, klass=w.klass)
    a_t, b_t = W.gen_a(w), W.gen_b(w)
    a, b = W.bits(a_t), W.bits(b_t)
    vals, mask = ssg.compress_nm(a_t.cuda(), n, m)
    rv, rmask = oracle.compress_nm(dt, n, m, a)
    assert np.array_equal(to_host(vals.contiguous()), rv)
    assert np.array_equal(to_host(mask.contiguous()), rmask)
    C = ssg.spmm_nm(vals, mask, n, m, b_t.cuda())
    c_ref, s_ref = oracle.spmm_nm(dt, n, m, rv, rmask, b, w.K)
    check_product(dt, to_host(C), c_ref, s_ref, "c3nm %s %d:%d" % (dt, n, m))


def test_spmm_nm_k_zero_and_empty():
    B = torch.zeros((0, 16), dtype=torch.float16, device="cuda")
    vals = torch.zeros((8, 0), dtype=torch.float16, device="cuda")
    mask = torch.zeros((8, 0), dtype=torch.uint8, device="cuda")
    C = torch.full((8, 16), 7.0, device="cuda")
    ssg.ssg_spmm_nm(vals, mask, 1, 4, 0, B, C)
    assert (C.cpu() == 0).all()
    vals = torch.zeros((0, 16), dtype=torch.float16, device="cuda")
    mask = torch.zeros((0, 8), dtype=torch.uint8, device="cuda")
    C = torch.empty((0, 16), device="cuda")
    ssg.ssg_spmm_nm(vals, mask, 1, 4, 64, torch.zeros((64, 16), dtype=torch.float16, device="cuda"), C)


def test_spmm_nm_argument_errors():
    a = U.random_matrix("f16", 32, 256, "normal", seed=1)
    A = to_dev(a, "f16")
    vals, mask = ssg.compress_nm(A, 2, 8)
    B = torch.zeros((256, 16), dtype=torch.float16, device="cuda")
    C = torch.empty((32, 16), device="cuda")
    with pytest.raises(ssg.SsgError) as e:
        ssg.ssg_spmm_nm(vals, mask, 3, 8, 256, B, C)            # pattern without kernels
    assert e.value.status == ssg._abi.SSG_ERR_SHAPE
    with pytest.raises(ssg.SsgError) as e:
        ssg.ssg_spmm_nm(vals, mask, 2, 8, 252, B[:252], C)       # K not a multiple of m
    assert e.value.status == ssg._abi.SSG_ERR_SHAPE
    Bw = torch.zeros((256, 17), dtype=torch.float16, device="cuda")
    with pytest.raises(ssg.SsgError) as e:
        ssg.ssg_spmm_nm(vals, mask, 2, 8, 256, Bw, torch.empty((32, 17), device="cuda"))   # 34-byte B rows
    assert e.value.status == ssg._abi.SSG_ERR_STRIDE
    with pytest.raises(ssg.SsgError) as e:
        vb = torch.zeros((32, 65), dtype=torch.float16, device="cuda")
        vb[:, :64] = vals
        ssg.ssg_spmm_nm(vb[:, :64], mask, 2, 8, 256, B, C)      # 130-byte rows of vals
    assert e.value.status == ssg._abi.SSG_ERR_STRIDE


# ------------------------------------------------------------------ packed decode layout

def expected_packed_nm(dt, n, m, vals, mask, M, K):
    """The packed layout written out from its definition with numpy: per tile
    and super-step, lane l = 16q + r carries row r's value bytes
    [64g + 16q, +16) and mask bytes [g*D/2 + q*D/8, +D/8)."""
    es = 2 if dt in ("f16", "bf16") else 1
    D = 32 if dt == "i4" else (16 // es) * m // n
    VB = D * n // m // 2 if dt == "i4" else 16        # value bytes per lane per super-step
    SK, MB = 4 * D, D // 8
    nsteps, tiles = -(-K // SK), -(-M // 16)
    vb = np.ascontiguousarray(vals).view(np.uint8).reshape(M, -1)
    Vp = np.zeros((tiles * 16, nsteps * 4 * VB), dtype=np.uint8)
    Vp[:M, :vb.shape[1]] = vb
    Mp = np.zeros((tiles * 16, nsteps * 4 * MB), dtype=np.uint8)
    Mp[:M, :mask.shape[1]] = mask
    pv = Vp.reshape(tiles, 16, nsteps, 4, VB).transpose(0, 2, 3, 1, 4).reshape(-1)
    pm = Mp.reshape(tiles, 16, nsteps, 4, MB).transpose(0, 2, 3, 1, 4).reshape(-1)
    return pv, pm


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("pat", PATS, ids=PAT_IDS)
@pytest.mark.parametrize("shape", [(1, 64, 16), (37, 264, 5), (300, 2048, 40), (8200, 512, 16)],
                         ids=["1x64x16", "37x264x5", "300x2048x40", "8200x512x16"])
def test_packed_layout_and_product(dt, pat, shape):
    n, m = pat
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "normal", seed=M + 2 * K + N)
    b = U.random_matrix(dt, K, N, "normal", seed=M * 5 + N)
    vals, mask = ssg.compress_nm(to_dev(a, dt), n, m)
    pvals, pmask = ssg.pack_nm(vals, mask, n, m, K)
    rv, rmask = oracle.compress_nm(dt, n, m, a)
    ev, em = expected_packed_nm(dt, n, m, rv, rmask, M, K)
    assert np.array_equal(pvals.cpu().numpy(), ev)
    assert np.array_equal(pmask.cpu().numpy(), em)
    C = ssg.spmm_nm_packed(pvals, pmask, n, m, M, b_dev(b, dt))
    c_ref, s_ref = oracle.spmm_nm(dt, n, m, rv, rmask, b, K)
    check_product(dt, to_host(C), c_ref, s_ref, "packed %s %d:%d %s" % (dt, n, m, shape))


@pytest.mark.parametrize("pat", PATS, ids=PAT_IDS)
@pytest.mark.parametrize("dt", ["f16", "i8", "e4m3"])
def test_packed_decode_workload_full_size(dt, pat):
    n, m = pat
    w = W.WORKLOADS["c3nm"]
    w = W.Workload(w.key, w.title, dt, w.M, w.K, w.N, w.index, a_sigma=w.a_sigma, klass=w.klass)
    a_t, b_t = W.gen_a(w), W.gen_b(w)
    a, b = W.bits(a_t), W.bits(b_t)
    vals, mask = ssg.compress_nm(a_t.cuda(), n, m)
    pvals, pmask = ssg.pack_nm(vals, mask, n, m, w.K)
    C = ssg.spmm_nm_packed(pvals, pmask, n, m, w.M, b_t.cuda())
    rv, rmask = oracle.compress_nm(dt, n, m, a)
    c_ref, s_ref = oracle.spmm_nm(dt, n, m, rv, rmask, b, w.K)
    check_product(dt, to_host(C), c_ref, s_ref, "c3nm packed %s %d:%d" % (dt, n, m))


@pytest.mark.parametrize("dt", ["f16", "i8", "e4m3"])
@pytest.mark.parametrize("pat", [(1, 4), (2, 8)], ids=["1:4", "2:8"])
def test_patterns_within_2to4_run_on_the_sparse_mfma(dt, pat):
    """1:4 and 2:8 never keep more than two values in an aligned group of
    four, so the 2:4 form of their expansion is the same matrix and the
    2:4 prefill kernel computes the same product."""
    n, m = pat
    M, K, N = 512, 1024, 512
    a = U.random_matrix(dt, M, K, "normal", seed=3 + n + m)
    b = U.random_matrix(dt, K, N, "normal", seed=4 + n + m)
    vals, mask = ssg.compress_nm(to_dev(a, dt), n, m)
    D = ssg.decompress_nm(vals, mask, n, m, K)
    v24, meta = ssg.compress(D)
    assert np.array_equal(to_host(ssg.decompress(v24, meta, K)), to_host(D))
    C = ssg.spmm(v24, meta, to_dev(b, dt), algo=ssg.SSG_ALGO_LARGE_N)
    rv, rmask = oracle.compress_nm(dt, n, m, a)
    c_ref, s_ref = oracle.spmm_nm(dt, n, m, rv, rmask, b, K)
    check_product(dt, to_host(C), c_ref, s_ref, "%d:%d via 2:4 large-N" % pat)


# ------------------------------------------------------------------ 4-bit weights, fp16 activations

I4_PATS = [(2, 4), (2, 8), (4, 8)]
I4_IDS = ["%d:%d" % p for p in I4_PATS]


@pytest.mark.parametrize("pat", I4_PATS, ids=I4_IDS)
@pytest.mark.parametrize("fam", ["normal", "ties", "sparse", "extreme"])
@pytest.mark.parametrize("shape", [(1, 8), (3, 40), (37, 200), (128, 4096), (33, 8200)])
def test_i4_compress_and_expand_bitexact(pat, fam, shape):
    n, m = pat
    M, K = shape
    if K % m:
        K += m - K % m
    a = U.random_matrix("i4", M, K, fam, seed=M + K + n + 7 * m)
    vals, mask = ssg.compress_nm(to_dev(a, "i4"), n, m)
    rv, rmask = oracle.compress_nm("i4", n, m, a)
    assert np.array_equal(to_host(vals.contiguous()), rv)
    assert np.array_equal(to_host(mask.contiguous()), rmask)
    D, bad = ssg.decompress_nm(vals, mask, n, m, K, count_bad=True)
    rd, rbad = oracle.decompress_nm("i4", n, m, rv, rmask, K)
    assert bad == rbad == 0
    assert np.array_equal(to_host(D), rd)


@pytest.mark.parametrize("pat", I4_PATS, ids=I4_IDS)
@pytest.mark.parametrize("shape", PRODUCT_SHAPES, ids=["x".join(map(str, s)) for s in PRODUCT_SHAPES])
def test_i4_w4a16_product_matches_oracle(pat, shape):
    n, m = pat
    M, K, N = shape
    if K % m:
        K += m - K % m
    a = U.random_matrix("i4", M, K, "normal", seed=M + K + N + 1)
    b = U.random_matrix("f16", K, N, "normal", seed=M * 3 + N + 1)
    vals, mask = ssg.compress_nm(to_dev(a, "i4"), n, m)
    B = b_dev(b, "f16")
    C = ssg.spmm_nm(vals, mask, n, m, B)
    rv, rmask = oracle.compress_nm("i4", n, m, a)
    c_ref, s_ref = oracle.spmm_nm("i4", n, m, rv, rmask, b, K)
    check_product("f16", to_host(C), c_ref, s_ref, "i4 %d:%d %s" % (n, m, shape))
    pvals, pmask = ssg.pack_nm(vals, mask, n, m, K)
    ev, em = expected_packed_nm("i4", n, m, rv, rmask, M, K)
    assert np.array_equal(pvals.cpu().numpy(), ev)
    assert np.array_equal(pmask.cpu().numpy(), em)
    Cp = ssg.spmm_nm_packed(pvals, pmask, n, m, M, B, i4=True)
    check_product("f16", to_host(Cp), c_ref, s_ref, "i4 packed %d:%d %s" % (n, m, shape))


@pytest.mark.parametrize("pat", I4_PATS, ids=I4_IDS)
def test_i4_w4a16_exact_small_integers(pat):
    """Every 4-bit value times a small integer, and every partial sum, is exact
    in fp32: a misplaced element, a wrong nibble or a sign error shows as a
    hard mismatch."""
    n, m = pat
    M, K, N = 160, 2304, 16
    a = U.random_matrix("i4", M, K, "normal", seed=5 * n + m)
    b = U.encode("f16", np.random.default_rng(2 * n + m).integers(-3, 4, size=(K, N)))
    vals, mask = ssg.compress_nm(to_dev(a, "i4"), n, m)
    B = to_dev(b, "f16")
    rv, rmask = oracle.compress_nm("i4", n, m, a)
    c_ref, _ = oracle.spmm_nm("i4", n, m, rv, rmask, b, K)
    assert np.array_equal(to_host(ssg.spmm_nm(vals, mask, n, m, B)).astype(np.float64), c_ref)
    pv, pm = ssg.pack_nm(vals, mask, n, m, K)
    assert np.array_equal(to_host(ssg.spmm_nm_packed(pv, pm, n, m, M, B, i4=True)).astype(np.float64), c_ref)


@pytest.mark.parametrize("pat", I4_PATS, ids=I4_IDS)
def test_i4_decode_workload_full_size(pat):
    """The fp16 decode shape 11008 x 4096 x 16 with 4-bit weights, in full."""
    n, m = pat
    w = W.Workload("c3w4", "4-bit weights", "i4", 11008, 4096, 16, 9, klass="small_n", b_dtype="f16")
    a_t, b_t = W.gen_a(w), W.gen_b(w)
    a, b = W.bits(a_t), W.bits(b_t)
    vals, mask = ssg.compress_nm(a_t.cuda(), n, m)
    rv, rmask = oracle.compress_nm("i4", n, m, a)
    assert np.array_equal(to_host(vals.contiguous()), rv)
    assert np.array_equal(to_host(mask.contiguous()), rmask)
    c_ref, s_ref = oracle.spmm_nm("i4", n, m, rv, rmask, b, w.K)
    C = ssg.spmm_nm(vals, mask, n, m, b_t.cuda())
    check_product("f16", to_host(C), c_ref, s_ref, "c3w4 %d:%d" % pat)
    pv, pm = ssg.pack_nm(vals, mask, n, m, w.K)
    Cp = ssg.spmm_nm_packed(pv, pm, n, m, w.M, b_t.cuda(), i4=True)
    check_product("f16", to_host(Cp), c_ref, s_ref, "c3w4 packed %d:%d" % pat)


def test_i4_argument_errors():
    a = U.random_matrix("i4", 16, 256, "normal", seed=1)
    A = to_dev(a, "i4")
    with pytest.raises(ssg.SsgError) as e:
        ssg.compress_nm(A, 1, 4)                                    # half a byte per group
    assert e.value.status == ssg._abi.SSG_ERR_SHAPE
    vals, mask = ssg.compress_nm(A, 2, 4)
    B = torch.zeros((256, 16), dtype=torch.float16, device="cuda")
    C = torch.empty((16, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(ssg.SsgError) as e:
        ssg._check(ssg._lib().ssg_spmm_nm(ssg._abi.SSG_I4, ssg.SSG_I32, 2, 4, 16, 16, 256, vals.data_ptr(), 256,
                                          mask.data_ptr(), 32, B.data_ptr(), 16, C.data_ptr(), 16, None), "w4")
    assert e.value.status == ssg._abi.SSG_ERR_DTYPE
