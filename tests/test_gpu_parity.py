"""Parity of the HIP path (through the C ABI) with the CPU oracle.

* compression, pruning, expansion and the residual split: bit-exact;
* int8 SpMM: bit-exact (int32 vs int64);
* fp16/bf16 SpMM: relative Frobenius error <= 1e-3 and, element by element,
  |C_gpu - C_ref| <= 1e-2 * sum_k |a_mk b_kn|.

Small cases are compared in full; the full-size workloads compare the whole
compressed operand and a sample of outputs the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_amd as ssg
import workloads as W
from tests import _util as U

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "i8", "e4m3", "e5m2"]
FLOATS = ["f16", "bf16", "e4m3", "e5m2"]
FRO_TOL = 1e-3
ELEM_TOL = 1e-2
ALGOS = [ssg.SSG_ALGO_GENERIC, ssg.SSG_ALGO_SMALL_N, ssg.SSG_ALGO_LARGE_N]
ALGO_IDS = ["generic", "small_n", "large_n"]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    torch.cuda.init()
    return torch.device("cuda:0")


def to_dev(a_bits: np.ndarray, dt: str) -> torch.Tensor:
    return W.from_bits(a_bits, dt).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype in (torch.float16, torch.bfloat16, torch.int8, torch.float8_e4m3fn, torch.float8_e5m2):
        return W.bits(t)
    return t.numpy()


def check_fp(c_gpu, c_ref, s_ref, what=""):
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    err = np.abs(c_gpu - c_ref)
    ref_norm = np.linalg.norm(c_ref)
    fro = np.linalg.norm(c_gpu - c_ref) / ref_norm if ref_norm > 0 else np.linalg.norm(c_gpu - c_ref)
    assert fro <= FRO_TOL, "%s: relative Frobenius error %.3g" % (what, fro)
    bad = err > ELEM_TOL * s_ref
    assert not bad.any(), "%s: %d elements beyond 1e-2*sum|ab| (worst at %s)" % (
        what, int(bad.sum()), np.unravel_index(np.argmax(err - ELEM_TOL * s_ref), err.shape))


def check_product(dt, c_gpu, c_ref, s_ref, what=""):
    if dt == "i8":
        assert np.array_equal(np.asarray(c_gpu, dtype=np.int64), c_ref), what
    else:
        check_fp(c_gpu, c_ref, s_ref, what)


def strided(t: torch.Tensor, extra: int) -> torch.Tensor:
    """The same values inside a wider buffer (leading dimension > row length)."""
    if extra == 0:
        return t
    buf = torch.zeros((t.shape[0], t.shape[1] + extra), dtype=t.dtype, device=t.device)
    buf[:, :t.shape[1]] = t
    return buf[:, :t.shape[1]]


# ------------------------------------------------------------------ compression

SHAPES = [(1, 4), (3, 36), (5, 12), (64, 256), (77, 1000), (128, 4096), (33, 8196)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("fam", ["normal", "ties", "sparse", "extreme"])
@pytest.mark.parametrize("shape", SHAPES)
def test_compress_prune_decompress_bitexact(dt, fam, shape):
    M, K = shape
    a = U.random_matrix(dt, M, K, fam, seed=M * 131 + K)
    A = to_dev(a, dt)
    vals, meta = ssg.compress(A)
    rv, rm = oracle.compress(dt, a)
    assert np.array_equal(to_host(vals), rv)
    assert np.array_equal(to_host(meta), rm)
    P = ssg.prune(A)
    assert np.array_equal(to_host(P), oracle.prune(dt, a))
    D, bad = ssg.decompress(vals, meta, K, count_bad=True)
    assert bad == 0 and np.array_equal(to_host(D), oracle.prune(dt, a))


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("extra,offset", [(1, 0), (8, 0), (0, 1), (5, 3)])
def test_compress_strided_and_unaligned(dt, extra, offset):
    M, K = 19, 200
    a = U.random_matrix(dt, M, K, "normal", seed=extra * 7 + offset)
    base = torch.zeros((M, K + extra + offset), dtype=W.TORCH_DTYPE[dt], device="cuda")
    base[:, offset:offset + K] = to_dev(a, dt)
    A = base[:, offset:offset + K]
    vb = torch.zeros((M, K // 2 + extra + offset), dtype=A.dtype, device="cuda")
    mb = torch.zeros((M, (K + 7) // 8 + extra + offset), dtype=torch.uint8, device="cuda")
    vals, meta = vb[:, offset:offset + K // 2], mb[:, offset:offset + (K + 7) // 8]
    ssg.ssg_compress_2to4(A, vals, meta)
    rv, rm = oracle.compress(dt, a)
    assert np.array_equal(to_host(vals.contiguous()), rv)
    assert np.array_equal(to_host(meta.contiguous()), rm)
    P = torch.zeros_like(base)[:, offset:offset + K]
    ssg.ssg_prune_2to4(A, P)
    assert np.array_equal(to_host(P.contiguous()), oracle.prune(dt, a))
    # neighbours of the strided outputs were not touched
    bits = vb.view(torch.uint8) if vb.element_size() == 1 else vb.view(torch.int16)   # torch has no any() on fp8
    assert not bits[:, :offset].any() and not bits[:, offset + K // 2:].any()
    assert not mb[:, :offset].any() and not mb[:, offset + (K + 7) // 8:].any()


@pytest.mark.parametrize("dt", DTS)
def test_prune_in_place(dt):
    a = U.random_matrix(dt, 40, 128, "ties", seed=3)
    A = to_dev(a, dt)
    ssg.ssg_prune_2to4(A, A)
    assert np.array_equal(to_host(A), oracle.prune(dt, a))


@pytest.mark.parametrize("dt", DTS)
def test_decompress_counts_bad_nibbles(dt):
    a = U.random_matrix(dt, 6, 64, "normal", seed=5)
    rv, rm = oracle.compress(dt, a)
    rm = rm.copy()
    rm[1, 0] = (rm[1, 0] & 0xF0) | 0x5
    rm[4, 7] = (rm[4, 7] & 0x0F) | 0x30
    rm[5, 2] = 0x00                                   # two bad groups
    D, bad = ssg.decompress(to_dev(rv, dt), torch.from_numpy(rm).cuda(), 64, count_bad=True)
    ref, rbad = oracle.decompress(dt, rv, rm, 64)
    assert bad == rbad == 4
    assert np.array_equal(to_host(D), ref)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("fam", ["normal", "ties", "sparse"])
@pytest.mark.parametrize("shape", [(1, 4), (7, 44), (64, 256), (50, 1100), (9, 8192)])
def test_split_bitexact(dt, fam, shape):
    M, K = shape
    a = U.random_matrix(dt, M, K, fam, seed=M + 3 * K)
    vals, meta, row_ptr, col, rvals = ssg.split(to_dev(a, dt))
    r = oracle.split(dt, a)
    assert np.array_equal(to_host(vals), r[0]) and np.array_equal(to_host(meta), r[1])
    assert np.array_equal(row_ptr.cpu().numpy(), r[2])
    assert np.array_equal(col.cpu().numpy(), r[3])
    assert np.array_equal(to_host(rvals), r[4])


# ------------------------------------------------------------------ products

def run_algo(algo, fn):
    try:
        return fn()
    except ssg.SsgError as e:
        if e.status == 8:          # SSG_ERR_ALGO: this family does not take the problem
            pytest.skip("algorithm %s does not take this problem" % ssg.ALGO_NAMES[algo])
        raise


PRODUCT_SHAPES = [(1, 4, 1), (16, 64, 16), (37, 64, 9), (256, 256, 64), (48, 512, 16), (100, 1024, 13),
                  (130, 4096, 16), (64, 192, 48), (256, 512, 256), (300, 1024, 200)]


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", PRODUCT_SHAPES)
def test_spmm_matches_oracle(algo, dt, shape):
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "normal", seed=M + K)
    b = U.random_matrix(dt, K, N, "normal", seed=N + 17)
    vals, meta = oracle.compress(dt, a)
    C = run_algo(algo, lambda: ssg.spmm(to_dev(vals, dt), torch.from_numpy(meta).cuda(), to_dev(b, dt), algo=algo))
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "spmm %s %s" % (dt, shape))


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", [(16, 64, 16), (40, 256, 16), (130, 2048, 16), (64, 128, 40), (200, 512, 256)])
def test_spmm_residual_matches_oracle(algo, dt, shape):
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "sparse", seed=M * K)
    b = U.random_matrix(dt, K, N, "normal", seed=N)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    dev = lambda x: torch.from_numpy(x).cuda()
    C = run_algo(algo, lambda: ssg.spmm_residual(to_dev(vals, dt), dev(meta), dev(row_ptr), dev(col),
                                                 to_dev(rvals, dt) if len(rvals) else torch.empty(0, dtype=W.TORCH_DTYPE[dt], device="cuda"),
                                                 to_dev(b, dt), algo=algo))
    cref, sref = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "residual %s %s" % (dt, shape))


# ------------------------------------------------------------------ delta-coded residual

def far_csr(M, K, seed, per_row=6):
    """CSR rows with a few columns spread over K, so gaps above 255 (fillers)
    are common, plus empty rows."""
    rng = np.random.default_rng(seed)
    cols = [np.sort(rng.choice(K, size=int(rng.integers(0, per_row + 1)), replace=False)) for _ in range(M)]
    row_ptr = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    col = np.concatenate(cols).astype(np.int32)
    return row_ptr, col


def dev_or_empty(x: np.ndarray, dt: str = None) -> torch.Tensor:
    if dt is None:
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if len(x) == 0:
        return torch.empty(0, dtype=W.TORCH_DTYPE[dt], device="cuda")
    return to_dev(x, dt)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("case", ["split", "far", "empty_rows", "one_row"])
def test_delta_encode_bitexact(dt, case):
    if case == "split":
        K = 1100
        a = U.random_matrix(dt, 70, K, "sparse", seed=71)
        _, _, row_ptr, col, rvals = oracle.split(dt, a)
    elif case == "far":
        K = 5000
        row_ptr, col = far_csr(300, K, 5)
        rvals = U.random_matrix(dt, 1, max(len(col), 1), "normal", 6)[0, :len(col)]
    elif case == "empty_rows":
        K = 64
        row_ptr, col = np.zeros(9, np.int32), np.zeros(0, np.int32)
        rvals = np.zeros(0, U.store_dtype(dt))
    else:   # one long row: several 256-entry blocks of the encoder, gaps of 1 to 600
        K = 200000
        rng = np.random.default_rng(9)
        col = np.cumsum(rng.integers(1, 601, size=700)).astype(np.int32)
        col = col[col < K]
        row_ptr = np.array([0, len(col)], np.int32)
        rvals = U.random_matrix(dt, 1, len(col), "normal", 10)[0]
    want = oracle.delta_encode(dt, row_ptr, col, rvals, K)
    got = ssg.delta_encode(dev_or_empty(row_ptr), dev_or_empty(col), dev_or_empty(rvals, dt), K)
    assert np.array_equal(got[0].cpu().numpy(), want[0])
    assert np.array_equal(got[1].cpu().numpy(), want[1])
    assert np.array_equal(to_host(got[2]) if len(want[2]) else np.zeros(0, U.store_dtype(dt)), want[2])


DELTA_SHAPES = [(16, 64, 16), (40, 256, 16), (130, 2048, 16), (40, 8192, 16), (64, 128, 40), (200, 512, 256)]


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", DELTA_SHAPES)
def test_spmm_residual_delta_matches_oracle(algo, dt, shape):
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "sparse", seed=M * K + 1)
    b = U.random_matrix(dt, K, N, "normal", seed=N + 1)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    drow_ptr, dcol, dvals = oracle.delta_encode(dt, row_ptr, col, rvals, K)
    C = run_algo(algo, lambda: ssg.spmm_residual_delta(to_dev(vals, dt), dev_or_empty(meta), dev_or_empty(drow_ptr),
                                                       dev_or_empty(dcol), dev_or_empty(dvals, dt), to_dev(b, dt),
                                                       algo=algo))
    cref, sref = oracle.spmm_residual_delta(dt, vals, meta, drow_ptr, dcol, dvals, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "residual delta %s %s" % (dt, shape))


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", [(48, 4096, 16), (33, 16384, 16)])
def test_spmm_residual_delta_with_fillers(algo, dt, shape):
    # a 2:4 layer plus a residual whose entries lie far apart (many fillers),
    # across several LDS chunks of K for the small-N kernel
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "normal", seed=K + 5)
    b = U.random_matrix(dt, K, N, "normal", seed=K + 6)
    vals, meta = oracle.compress(dt, a)
    row_ptr, col = far_csr(M, K, K, per_row=12)
    rvals = U.random_matrix(dt, 1, max(len(col), 1), "normal", 7)[0, :len(col)]
    drow_ptr, dcol, dvals = oracle.delta_encode(dt, row_ptr, col, rvals, K)
    assert (dcol == 255).sum() > len(col) // 2
    C = run_algo(algo, lambda: ssg.spmm_residual_delta(to_dev(vals, dt), dev_or_empty(meta), dev_or_empty(drow_ptr),
                                                       dev_or_empty(dcol), dev_or_empty(dvals, dt), to_dev(b, dt),
                                                       algo=algo))
    cref, sref = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "residual delta fillers %s %s" % (dt, shape))


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", [(40, 8192, 16), (20, 12288, 8), (100, 10240, 16)])
def test_spmm_residual_small_n_long_k(dt, shape):
    # narrow slabs whose K needs several LDS chunks run as wider slabs
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "sparse", seed=K + M)
    b = U.random_matrix(dt, K, N, "normal", seed=K + N)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    C = ssg.spmm_residual(to_dev(vals, dt), dev_or_empty(meta), dev_or_empty(row_ptr), dev_or_empty(col),
                          dev_or_empty(rvals, dt), to_dev(b, dt), algo=ssg.SSG_ALGO_SMALL_N)
    cref, sref = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "residual long K %s %s" % (dt, shape))


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("dt", FLOATS)
@pytest.mark.parametrize("delta", [False, True])
@pytest.mark.parametrize("shape", [(40, 256, 16), (33, 512, 16), (70, 1024, 8), (17, 8192, 16),
                                   (8200, 512, 16), (8192, 4992 + 64, 16)])
def test_spmm_residual_exact_small_integers(algo, dt, delta, shape):
    # small integers: every product and partial sum is exact in fp32, so the
    # fp16/bf16 result must equal the oracle's exactly -- a dropped or
    # doubled residual entry cannot hide inside the rounding tolerance
    M, K, N = shape
    rng = np.random.default_rng(M * K + N)
    x = rng.integers(-3, 4, size=(M, K)) * (rng.random((M, K)) < 0.5)
    a = U.encode(dt, x)
    b = U.encode(dt, rng.integers(-3, 4, size=(K, N)))
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    if delta:
        row_ptr, col, rvals = oracle.delta_encode(dt, row_ptr, col, rvals, K)
    fn = ssg.spmm_residual_delta if delta else ssg.spmm_residual
    C = run_algo(algo, lambda: fn(to_dev(vals, dt), dev_or_empty(meta), dev_or_empty(row_ptr), dev_or_empty(col),
                                  dev_or_empty(rvals, dt), to_dev(b, dt), algo=algo))
    want = x.astype(np.int64) @ U.to_f64(dt, b).astype(np.int64)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), want.astype(np.float64))


# ------------------------------------------------------------------ packed decode layout

def expected_packed(dt, vals_bits, meta, M, K):
    """The packed layout written out from its definition (a reordering)."""
    es = 2 if dt in ("f16", "bf16") else 1
    ks = 64 if es == 2 else 128
    ib = 2 if es == 2 else 4
    vb = np.ascontiguousarray(vals_bits).view(np.uint8).reshape(M, -1)
    tiles, nk = (M + 15) // 16, K // ks
    pv = np.zeros((tiles, nk, 64, 16), np.uint8)
    pm = np.zeros((tiles, nk, 64, ib), np.uint8)
    for lane in range(64):
        r, q = lane % 16, lane // 16
        for t in range(tiles):
            row = 16 * t + r
            if row >= M:
                continue
            for g in range(nk):
                pv[t, g, lane] = vb[row, g * (ks // 2) * es + 16 * q: g * (ks // 2) * es + 16 * q + 16]
                pm[t, g, lane] = meta[row, g * (ks // 8) + ib * q: g * (ks // 8) + ib * q + ib]
    return pv.reshape(-1), pm.reshape(-1)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", [(16, 128), (40, 256), (33, 512)])
def test_pack_decode_layout(dt, shape):
    M, K = shape
    a = U.random_matrix(dt, M, K, "normal", seed=M + K)
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    ev, em = expected_packed(dt, vals, meta, M, K)
    assert np.array_equal(pv.cpu().numpy(), ev) and np.array_equal(pm.cpu().numpy(), em)


PACKED_SHAPES = [(16, 128, 16), (40, 256, 16), (130, 2048, 16), (1000, 1024, 16), (4100, 512, 16), (16400, 256, 16)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", PACKED_SHAPES)
def test_spmm_packed_matches_oracle(dt, shape):
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "normal", seed=M + 2 * K)
    b = U.random_matrix(dt, K, N, "normal", seed=N + 3)
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    C = ssg.spmm_packed(pv, pm, M, to_dev(b, dt))
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "packed %s %s" % (dt, shape))


def test_spmm_packed_takes_only_16_columns():
    vals, meta = oracle.compress("f16", U.random_matrix("f16", 32, 128, "normal", 1))
    pv, pm = ssg.pack_decode(to_dev(vals, "f16"), dev_or_empty(meta), 128)
    with pytest.raises(ssg.SsgError) as e:
        ssg.spmm_packed(pv, pm, 32, to_dev(U.random_matrix("f16", 128, 8, "normal", 2), "f16"))
    assert e.value.status == 8


NARROW_SHAPES = [(11008, 4096, 1), (1000, 2048, 5), (300, 1024, 8), (4100, 512, 15)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", NARROW_SHAPES)
def test_spmm_narrow_b(dt, shape):
    # N < 16 with a strided B: the product pads B to 16 columns in its
    # workspace and runs the decode kernel that takes a contiguous K x 16 B
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "normal", seed=M + 3 * K)
    b = U.random_matrix(dt, K, N, "normal", seed=N + 29)
    vals, meta = oracle.compress(dt, a)
    assert ssg.ssg_spmm_workspace_bytes(W.TORCH_DTYPE[dt], M, N, K) >= K * 16 * (2 if dt in ("f16", "bf16") else 1)
    B = strided(to_dev(b, dt), 3)
    C = ssg.spmm(to_dev(vals, dt), dev_or_empty(meta), B)
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "narrow %s %s" % (dt, shape))


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_spmm_narrow_b_with_row_stride_16(dt):
    # N < 16 inside rows of 16 elements: the product still pads B (it reads
    # nothing past the last row's N-th element) and the result is exact/within tolerance
    M, K, N = 300, 1024, 5
    a = U.random_matrix(dt, M, K, "normal", seed=71)
    b = U.random_matrix(dt, K, N, "normal", seed=73)
    vals, meta = oracle.compress(dt, a)
    B = strided(to_dev(b, dt), 16 - N)
    assert B.stride(0) == 16
    C = ssg.spmm(to_dev(vals, dt), dev_or_empty(meta), B)
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "narrow B, ldb 16, %s" % dt)


def test_spmm_narrow_b_on_a_side_stream():
    # the workspace is allocated on the stream the kernels run on
    M, K, N = 1000, 2048, 3
    a = U.random_matrix("f16", M, K, "normal", seed=75)
    b = U.random_matrix("f16", K, N, "normal", seed=77)
    vals, meta = oracle.compress("f16", a)
    V, Mt, B = to_dev(vals, "f16"), dev_or_empty(meta), to_dev(b, "f16")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(side):
        C.record_stream(side)
    ssg.ssg_spmm_2to4(V, Mt, B, C, stream=side)
    side.synchronize()
    cref, sref = oracle.spmm("f16", vals, meta, b, K)
    check_product("f16", C.cpu().numpy(), cref, sref, "narrow B on a side stream")


def test_forced_kernels_need_no_workspace():
    # only the padded decode path uses the workspace: forced generic and
    # large-N products of a narrow B run without one
    M, K, N = 64, 256, 5
    a = U.random_matrix("i8", M, K, "normal", seed=79)
    b = U.random_matrix("i8", K, N, "normal", seed=81)
    vals, meta = oracle.compress("i8", a)
    cref, _ = oracle.spmm("i8", vals, meta, b, K)
    for algo in (ssg.SSG_ALGO_GENERIC,):
        C = torch.empty((M, N), dtype=torch.int32, device="cuda")
        ssg.ssg_spmm_2to4(to_dev(vals, "i8"), dev_or_empty(meta), to_dev(b, "i8"), C, ws=None, algo=algo)
        assert np.array_equal(C.cpu().numpy().astype(np.int64), cref)


@pytest.mark.parametrize("dt", DTS)
def test_spmm_residual_narrow_b(dt):
    M, K, N = 300, 1024, 8
    a = U.random_matrix(dt, M, K, "sparse", seed=41)
    b = U.random_matrix(dt, K, N, "normal", seed=43)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    B = strided(to_dev(b, dt), 5)
    C = ssg.spmm_residual(to_dev(vals, dt), dev_or_empty(meta), dev_or_empty(row_ptr), dev_or_empty(col),
                          dev_or_empty(rvals, dt), B)
    cref, sref = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "narrow residual %s" % dt)


PACKED_RES_SHAPES = [(16, 128), (40, 256), (300, 1024), (1000, 2048), (4100, 512)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("code", ["csr", "delta"])
@pytest.mark.parametrize("shape", PACKED_RES_SHAPES)
def test_spmm_packed_residual_matches_oracle(dt, code, shape):
    M, K = shape
    a = U.random_matrix(dt, M, K, "sparse", seed=M + 5 * K)
    b = U.random_matrix(dt, K, 16, "normal", seed=K + 9)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    pv, pm = ssg.pack_decode(to_dev(vals, dt), dev_or_empty(meta), K)
    B = to_dev(b, dt)
    V, Mt = to_dev(vals, dt), dev_or_empty(meta)
    if code == "csr":
        rp, cl, rv = dev_or_empty(row_ptr), dev_or_empty(col), dev_or_empty(rvals, dt)
        C = ssg.spmm_packed_residual(pv, pm, M, rp, cl, rv, B)
        C_ring = ssg.spmm_residual(V, Mt, rp, cl, rv, B)
    else:
        d = oracle.delta_encode(dt, row_ptr, col, rvals, K)
        dr, dc, dv = dev_or_empty(d[0]), dev_or_empty(d[1]), dev_or_empty(d[2], dt)
        C = ssg.spmm_packed_residual_delta(pv, pm, M, dr, dc, dv, B)
        C_ring = ssg.spmm_residual_delta(V, Mt, dr, dc, dv, B)
    cref, sref = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "packed residual %s %s %s" % (dt, code, shape))
    if dt == "i8":      # integer sums: the same bits as the row-major kernel
        assert torch.equal(C, C_ring)


def test_spmm_packed_residual_exact_small_integers():
    # fp16 small integers: every partial sum exact in fp32, so the product
    # equals the oracle's exactly, residual included
    M, K = 300, 1024
    rng = np.random.default_rng(11)
    dense = rng.integers(-3, 4, size=(M, K)) * (rng.random((M, K)) < 0.5)
    a = dense.astype(np.float16).view(np.uint16)
    b = rng.integers(-3, 4, size=(K, 16)).astype(np.float16).view(np.uint16)
    vals, meta, row_ptr, col, rvals = oracle.split("f16", a)
    pv, pm = ssg.pack_decode(to_dev(vals, "f16"), dev_or_empty(meta), K)
    C = ssg.spmm_packed_residual(pv, pm, M, dev_or_empty(row_ptr), dev_or_empty(col), dev_or_empty(rvals, "f16"),
                                 to_dev(b, "f16")).cpu().numpy().astype(np.float64)
    cref, _ = oracle.spmm_residual("f16", vals, meta, row_ptr, col, rvals, b, K)
    assert np.array_equal(C, cref)


def test_full_size_residual_packed():
    w = W.WORKLOADS["c5"]
    print("full-size packed residual: %s" % w.title, flush=True)
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    a, b = W.bits(a_cpu), W.bits(b_cpu)
    vals, meta, row_ptr, col, rvals = ssg.split(a_cpu.cuda())
    pv, pm = ssg.pack_decode(vals, meta, w.K)
    B = b_cpu.cuda()
    C = ssg.spmm_packed_residual(pv, pm, w.M, row_ptr, col, rvals, B).cpu().numpy()
    drow_ptr, dcol, dvals = ssg.delta_encode(row_ptr, col, rvals, w.K)
    Cd = ssg.spmm_packed_residual_delta(pv, pm, w.M, drow_ptr, dcol, dvals, B).cpu().numpy()
    r = oracle.split(w.dtype, a)
    cref, sref = oracle.spmm_residual(w.dtype, *r, b, w.K)
    check_product(w.dtype, C, cref, sref, "c5 packed residual (all outputs)")
    check_product(w.dtype, Cd, cref, sref, "c5 packed residual, delta-coded (all outputs)")


def test_full_size_decode_packed():
    w = W.WORKLOADS["c3"]
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    a, b = W.bits(a_cpu), W.bits(b_cpu)
    vals, meta = ssg.compress(a_cpu.cuda())
    pv, pm = ssg.pack_decode(vals, meta, w.K)
    C = ssg.spmm_packed(pv, pm, w.M, b_cpu.cuda()).cpu().numpy()
    r = oracle.compress(w.dtype, a)
    cref, sref = oracle.spmm(w.dtype, r[0], r[1], b, w.K)
    check_product(w.dtype, C, cref, sref, "c3 packed (all outputs)")


# ------------------------------------------------------------------ unstructured products

def random_csr(M, K, density, seed):
    rng = np.random.default_rng(seed)
    cols = [np.nonzero(rng.random(K) < density)[0] for _ in range(M)]
    row_ptr = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    col = np.concatenate(cols).astype(np.int32) if row_ptr[-1] else np.zeros(0, np.int32)
    return row_ptr, col


CSR_SHAPES = [(40, 256, 16), (130, 2048, 16), (64, 512, 8), (33, 300, 5), (100, 1024, 40), (8192, 5056, 16)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("delta", [False, True])
@pytest.mark.parametrize("shape", CSR_SHAPES)
def test_spmm_csr_matches_oracle(dt, delta, shape):
    # small integers in fp16/bf16 keep every sum exact: compared bit for bit
    M, K, N = shape
    row_ptr, col = random_csr(M, K, 0.1 if M < 8192 else 0.02, M + K)
    rng = np.random.default_rng(K)
    vals = U.encode(dt, rng.integers(1, 4, size=len(col)) * rng.choice([-1, 1], size=len(col)))
    b = U.encode(dt, rng.integers(-3, 4, size=(K, N)))
    cref, _ = oracle.spmm_csr(dt, row_ptr, col, vals, b, K)
    if delta:
        d = oracle.delta_encode(dt, row_ptr, col, vals, K)
        C = ssg.spmm_csr_delta(dev_or_empty(d[0]), dev_or_empty(d[1]), dev_or_empty(d[2], dt), to_dev(b, dt))
    else:
        C = ssg.spmm_csr(dev_or_empty(row_ptr), dev_or_empty(col), dev_or_empty(vals, dt), to_dev(b, dt))
    assert np.array_equal(C.cpu().numpy().astype(np.float64), np.asarray(cref, dtype=np.float64))


@pytest.mark.parametrize("dt", FLOATS)
def test_spmm_csr_random_values_within_tolerance(dt):
    M, K, N = 300, 4096, 16
    row_ptr, col = random_csr(M, K, 0.05, 5)
    vals = U.random_matrix(dt, 1, len(col), "normal", 6)[0]
    b = U.random_matrix(dt, K, N, "normal", 7)
    cref, sref = oracle.spmm_csr(dt, row_ptr, col, vals, b, K)
    C = ssg.spmm_csr(dev_or_empty(row_ptr), dev_or_empty(col), dev_or_empty(vals, dt), to_dev(b, dt))
    check_fp(C.cpu().numpy(), cref, sref, "csr %s" % dt)


def test_spmm_csr_empty_is_zero():
    row_ptr = np.zeros(65, np.int32)
    b = U.encode("f16", np.ones((256, 16)))
    C = ssg.spmm_csr(dev_or_empty(row_ptr), None, dev_or_empty(np.zeros(0, np.uint16), "f16"), to_dev(b, "f16"),
                     out=torch.full((64, 16), 7.0, device="cuda"))
    assert not C.cpu().numpy().any()


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("delta", [False, True])
def test_spmm_residual_unaligned_arrays(dt, delta):
    # residual arrays at odd element offsets: the tiled kernels do not take
    # them (SSG_ERR_ALGO when forced), AUTO runs them on the generic kernel
    M, K, N = 48, 512, 16
    a = U.random_matrix(dt, M, K, "sparse", seed=77)
    b = U.random_matrix(dt, K, N, "normal", seed=78)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, a)
    if delta:
        row_ptr, col, rvals = oracle.delta_encode(dt, row_ptr, col, rvals, K)
    cbuf = dev_or_empty(np.concatenate([col[:1], col]))[1:]
    vbuf = dev_or_empty(np.concatenate([rvals[:1], rvals]), dt)[1:]
    args = (to_dev(vals, dt), dev_or_empty(meta), dev_or_empty(row_ptr), cbuf, vbuf, to_dev(b, dt))
    fn = ssg.spmm_residual_delta if delta else ssg.spmm_residual
    with pytest.raises(ssg.SsgError):
        fn(*args, algo=ssg.SSG_ALGO_SMALL_N)
    C = fn(*args)
    cref, sref = (oracle.spmm_residual_delta if delta else oracle.spmm_residual)(dt, vals, meta, row_ptr, col, rvals,
                                                                                 b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "unaligned residual %s" % dt)


@pytest.mark.parametrize("dt", FLOATS)
def test_identity_B_gives_the_pruned_matrix_exactly(dt):
    K = 256
    a = U.random_matrix(dt, 64, K, "normal", seed=9)
    vals, meta = oracle.compress(dt, a)
    eye = U.encode(dt, np.eye(K))
    for algo in ALGOS:
        try:
            C = ssg.spmm(to_dev(vals, dt), torch.from_numpy(meta).cuda(), to_dev(eye, dt), algo=algo)
        except ssg.SsgError as e:
            assert e.status == 8
            continue
        assert np.array_equal(C.cpu().numpy().astype(np.float64), U.to_f64(dt, oracle.prune(dt, a)))


@pytest.mark.parametrize("dt", DTS)
def test_spmm_strided_operands(dt):
    M, K, N = 50, 512, 24
    a = U.random_matrix(dt, M, K, "normal", seed=1)
    b = U.random_matrix(dt, K, N, "normal", seed=2)
    vals, meta = oracle.compress(dt, a)
    V = strided(to_dev(vals, dt), 8)
    Mt = strided(torch.from_numpy(meta).cuda(), 4)
    B = strided(to_dev(b, dt), 16)
    cbuf = torch.full((M, N + 8), 7, dtype=torch.int32 if dt == "i8" else torch.float32, device="cuda")
    C = cbuf[:, :N]
    ssg.ssg_spmm_2to4(V, Mt, B, C)
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref)
    assert (cbuf[:, N:] == 7).all()


def test_k_zero_fills_C():
    vals = torch.empty((5, 0), dtype=torch.float16, device="cuda")
    meta = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    B = torch.empty((0, 3), dtype=torch.float16, device="cuda")
    C = torch.full((5, 3), 1.5, dtype=torch.float32, device="cuda")
    ssg.ssg_spmm_2to4(vals, meta, B, C)
    assert (C == 0).all()


def test_int8_extremes_exact():
    M, K, N = 64, 2048, 64
    rng = np.random.default_rng(0)
    a = rng.choice([-128, 127, -127], size=(M, K)).astype(np.int8)
    b = rng.choice([-128, 127], size=(K, N)).astype(np.int8)
    vals, meta = oracle.compress("i8", a)
    for algo in ALGOS:
        try:
            C = ssg.spmm(to_dev(vals, "i8"), torch.from_numpy(meta).cuda(), to_dev(b, "i8"), algo=algo)
        except ssg.SsgError as e:
            assert e.status == 8
            continue
        cref, _ = oracle.spmm("i8", vals, meta, b, K)
        assert np.array_equal(C.cpu().numpy().astype(np.int64), cref)


@pytest.mark.parametrize("dt", DTS)
def test_results_are_reproducible(dt):
    M, K, N = 512, 2048, 16
    a = U.random_matrix(dt, M, K, "normal", seed=4)
    b = U.random_matrix(dt, K, N, "normal", seed=5)
    vals, meta = oracle.compress(dt, a)
    V, Mt, B = to_dev(vals, dt), torch.from_numpy(meta).cuda(), to_dev(b, dt)
    c1 = ssg.spmm(V, Mt, B)
    c2 = ssg.spmm(V, Mt, B)
    assert torch.equal(c1, c2)


# ------------------------------------------------------------------ full-size workloads

def sample_entries(M, N, count, seed):
    """Sampled (m, n): the four corners, tile edges and a random spread."""
    rng = np.random.default_rng(seed)
    ms = [0, M - 1, 0, M - 1] + [min(M - 1, x) for x in (15, 16, 31, 32, 127, 128, 255, 256)]
    ns = [0, 0, N - 1, N - 1] + [min(N - 1, x) for x in (15, 16, 31, 32, 127, 128, 255, 256)]
    ms += list(rng.integers(0, M, count))
    ns += list(rng.integers(0, N, count))
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)


MAX_GENERIC_MACS = 1 << 32


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4", "c5"])
def test_full_size_workload(key):
    w = W.WORKLOADS[key]
    print("full-size workload %s: %s" % (key, w.title), flush=True)
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    a, b = W.bits(a_cpu), W.bits(b_cpu)
    A, B = a_cpu.cuda(), b_cpu.cuda()
    if w.residual:
        vals, meta, row_ptr, col, rvals = ssg.split(A)
        r = oracle.split(w.dtype, a)
        assert np.array_equal(to_host(vals), r[0]) and np.array_equal(to_host(meta), r[1])
        assert np.array_equal(row_ptr.cpu().numpy(), r[2]) and np.array_equal(col.cpu().numpy(), r[3])
        assert np.array_equal(to_host(rvals), r[4])
        residual = (r[2], r[3], r[4])
    else:
        vals, meta = ssg.compress(A)
        r = oracle.compress(w.dtype, a)
        assert np.array_equal(to_host(vals), r[0]) and np.array_equal(to_host(meta), r[1])
        residual = None
    del A
    algo = ssg.ssg_spmm_select_algo(vals, meta, B, torch.empty((1, 1), dtype=torch.float32, device="cuda"))
    if algo == ssg.SSG_ALGO_GENERIC and w.M * w.N * w.K > MAX_GENERIC_MACS:
        pytest.skip("no fast kernel selected for %s yet" % key)
    if residual is None:
        C = ssg.spmm(vals, meta, B)
    else:
        C = ssg.spmm_residual(vals, meta, row_ptr, col, rvals, B)
        # the delta-coded form of the same residual, encoded on the GPU from
        # the GPU's split: bit-exact with the oracle's code, same product
        drow_ptr, dcol, dvals = ssg.delta_encode(row_ptr, col, rvals, w.K)
        d = oracle.delta_encode(w.dtype, *residual, w.K)
        assert np.array_equal(drow_ptr.cpu().numpy(), d[0]) and np.array_equal(dcol.cpu().numpy(), d[1])
        assert np.array_equal(to_host(dvals), d[2])
        Cd = ssg.spmm_residual_delta(vals, meta, drow_ptr, dcol, dvals, B).cpu().numpy()
    C = C.cpu().numpy()
    if key != "c4":
        # every output (the largest, int8 4096^3, is 6.9e10 exact int64 MACs:
        # a few seconds of the oracle on the host's threads)
        cref, sref = (oracle.spmm(w.dtype, r[0], r[1], b, w.K) if residual is None
                      else oracle.spmm_residual(w.dtype, r[0], r[1], *residual, b, w.K))
        check_product(w.dtype, C, cref, sref, key + " (all outputs)")
        if residual is not None:
            dref, dsref = oracle.spmm_residual_delta(w.dtype, r[0], r[1], *d, b, w.K)
            check_product(w.dtype, Cd, dref, dsref, key + " delta (all outputs)")
    else:
        # bf16 28672 x 8192 x 2048: whole rows at every row-tile position and
        # all eight column tiles, plus a random sample
        rows = np.unique(np.concatenate([np.arange(0, w.M, 997), [255, 256, 24575, 24576, w.M - 1]]))
        cref, sref = oracle.spmm(w.dtype, r[0][rows], r[1][rows], b, w.K)
        check_product(w.dtype, C[rows], cref, sref, key + " (whole rows)")
        ms, ns = sample_entries(w.M, w.N, 3000, seed=w.index)
        cref, sref = oracle.spmm_entries(w.dtype, r[0], r[1], b, w.K, ms, ns, residual=residual)
        check_product(w.dtype, C[ms, ns], cref, sref, key)
        if residual is not None:
            dref, dsref = oracle.spmm_entries(w.dtype, r[0], r[1], b, w.K, ms, ns, residual=d, delta=True)
            check_product(w.dtype, Cd[ms, ns], dref, dsref, key + " delta")
