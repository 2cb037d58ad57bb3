"""The packed prefill layout (the large-N kernel's LDS image of each 256-row
tile) and the product on it, through the C ABI.

* layout: bit-exact with the layout written out below from its definition
  in include/ssgemm.h, both from the pack of (vals, meta) and from the
  compressor that writes it directly;
* product: against the oracle (int8 exact, floats within the stated
  tolerance), and bit for bit equal to the large-N kernel on the row-major
  operand, which feeds the same operands to the same MFMA sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_amd as ssg
import workloads as W
from tests import _util as U
from tests.test_gpu_parity import check_product, dev_or_empty, sample_entries, to_dev

pytestmark = pytest.mark.gpu

DTS = ["f16", "bf16", "i8", "e4m3", "e5m2"]


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    torch.cuda.init()
    return torch.device("cuda:0")


def expected_prefill(dt, vals_bits, meta, M, K):
    """The packed prefill layout written out from its definition."""
    es = 2 if dt in ("f16", "bf16") else 1
    stages, mblocks, tiles = K * es // 128, (K + 255) // 256, (M + 255) // 256
    vb = np.zeros((tiles * 256, K // 2 * es), np.uint8)
    vb[:M] = np.ascontiguousarray(vals_bits).view(np.uint8).reshape(M, -1)
    mb = np.zeros((tiles * 256, mblocks * 32), np.uint8)
    mb[:M, :K // 8] = meta[:, :K // 8]
    # values in lane order: row r = 32 rt + rl of the tile, stage st, chunk
    # c = 2 s2 + q of the stage's 64 bytes; order [tile][stage][rt][s2][q][rl]
    pv = vb.reshape(tiles, 8, 32, stages, 2, 2, 16).transpose(0, 3, 1, 4, 5, 2, 6)
    # metadata blocks in 16-byte lane chunks: row r = 128 wm + 32 i + rl, block
    # byte j = ((hq * kpc + hs) * 2 + q) * iw + e (k-step h = hq * kpc + hs,
    # lane half q, index-word byte e); order [tile][block][hq][wm][q][rl][hs][i][e]
    iw = 4 if es == 1 else 2
    kpc = 4 // iw
    pm = mb.reshape(tiles, 2, 4, 32, mblocks, 4, kpc, 2, iw).transpose(0, 4, 5, 1, 7, 3, 6, 2, 8)
    return np.ascontiguousarray(pv).reshape(-1), np.ascontiguousarray(pm).reshape(-1)


def shapes_for(dt):
    # (M, K): one row; ragged tiles; K whose last metadata block is partial
    if dt in ("f16", "bf16"):
        return [(1, 64), (300, 192), (256, 512), (513, 1024)]
    return [(1, 128), (300, 384), (256, 512), (513, 1152)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("which", [0, 1, 2, 3])
def test_prefill_layout(dt, which):
    M, K = shapes_for(dt)[which]
    a = U.random_matrix(dt, M, K, "normal", seed=M + 5 * K)
    vals, meta = oracle.compress(dt, a)
    ev, em = expected_prefill(dt, vals, meta, M, K)
    vb, mb = ssg.ssg_prefill_packed_sizes(W.TORCH_DTYPE[dt], M, K)
    assert (vb, mb) == (ev.size, em.size)
    pv, pm = ssg.pack_prefill(to_dev(vals, dt), dev_or_empty(meta), K)
    assert np.array_equal(pv.cpu().numpy(), ev), "pack: values"
    assert np.array_equal(pm.cpu().numpy(), em), "pack: metadata"
    # the compressor writing the layout directly; the buffers start as 0xA5
    # so that a byte it fails to write shows
    pv2 = torch.full((vb,), 0xA5, dtype=torch.uint8, device="cuda")
    pm2 = torch.full((mb,), 0xA5, dtype=torch.uint8, device="cuda")
    ssg.ssg_compress_2to4_prefill(to_dev(a, dt), pv2, pm2)
    assert np.array_equal(pv2.cpu().numpy(), ev), "compress: values"
    assert np.array_equal(pm2.cpu().numpy(), em), "compress: metadata"


PRODUCT_SHAPES = [(64, 128, 16), (300, 384, 272), (256, 512, 256), (520, 1152, 528)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", PRODUCT_SHAPES)
def test_spmm_prefill_matches_oracle(dt, shape):
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "normal", seed=M + 7 * K)
    b = U.random_matrix(dt, K, N, "normal", seed=N + 11)
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.compress_prefill(to_dev(a, dt))
    B = to_dev(b, dt)
    C = ssg.spmm_prefill(pv, pm, M, B)
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "prefill %s %s" % (dt, shape))
    # same LDS bytes, same MFMA order as the row-major large-N kernel
    C_rm = ssg.spmm(to_dev(vals, dt), dev_or_empty(meta), B, algo=ssg.SSG_ALGO_LARGE_N)
    assert torch.equal(C.view(torch.int32), C_rm.view(torch.int32))


def test_spmm_prefill_exact_small_integers():
    # fp16 values that are small integers: every product and partial sum is
    # exact in fp32, so the product must equal the oracle's exactly
    M, K, N = 300, 640, 264
    rng = np.random.default_rng(3)
    a = rng.integers(-3, 4, size=(M, K)).astype(np.float16).view(np.uint16)
    b = rng.integers(-3, 4, size=(K, N)).astype(np.float16).view(np.uint16)
    vals, meta = oracle.compress("f16", a)
    pv, pm = ssg.compress_prefill(to_dev(a, "f16"))
    C = ssg.spmm_prefill(pv, pm, M, to_dev(b, "f16")).cpu().numpy().astype(np.float64)
    cref, _ = oracle.spmm("f16", vals, meta, b, K)
    assert np.array_equal(C, cref)


def test_spmm_prefill_argument_errors():
    a = U.random_matrix("i8", 64, 128, "normal", 1)
    pv, pm = ssg.compress_prefill(to_dev(a, "i8"))
    b = to_dev(U.random_matrix("i8", 128, 8, "normal", 2), "i8")
    with pytest.raises(ssg.SsgError) as e:      # N not a multiple of 16 for 8-bit inputs
        ssg.spmm_prefill(pv, pm, 64, b)
    assert e.value.status == 8
    with pytest.raises(ssg.SsgError) as e:      # K not a multiple of the stage
        ssg.compress_prefill(to_dev(U.random_matrix("i8", 64, 64, "normal", 3), "i8"))
    assert e.value.status == 2


@pytest.mark.parametrize("dt", ["bf16", "i8"])
def test_spmm_prefill_mixed_widths(dt):
    # 20 x 13 = 260 tiles: the last wave of 256 CUs would hold 4 tiles, so
    # the last row of 13 tiles runs as 26 half-width tiles in the same
    # launch; every output against the oracle, and the same bits as the
    # row-major operand (which takes the same split)
    K = 128 if dt == "bf16" else 256
    M, N = 256 * 20 - 37, 256 * 13 - 48
    a = U.random_matrix(dt, M, K, "normal", seed=31)
    b = U.random_matrix(dt, K, N, "normal", seed=37)
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.compress_prefill(to_dev(a, dt))
    B = to_dev(b, dt)
    C = ssg.spmm_prefill(pv, pm, M, B)
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "prefill mixed widths %s" % dt)
    C_rm = ssg.spmm(to_dev(vals, dt), dev_or_empty(meta), B, algo=ssg.SSG_ALGO_LARGE_N)
    assert torch.equal(C.view(torch.int32), C_rm.view(torch.int32))


@pytest.mark.parametrize("key", ["c2", "c4"])
def test_full_size_prefill(key):
    w = W.WORKLOADS[key]
    print("full-size packed prefill %s: %s" % (key, w.title), flush=True)
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    a, b = W.bits(a_cpu), W.bits(b_cpu)
    A, B = a_cpu.cuda(), b_cpu.cuda()
    pv, pm = ssg.compress_prefill(A)
    vals, meta = ssg.compress(A)
    del A
    pv2, pm2 = ssg.pack_prefill(vals, meta, w.K)
    assert torch.equal(pv, pv2) and torch.equal(pm, pm2)
    del pv2, pm2
    C = ssg.spmm_prefill(pv, pm, w.M, B)
    C_rm = ssg.spmm(vals, meta, B, algo=ssg.SSG_ALGO_LARGE_N)
    assert torch.equal(C.view(torch.int32), C_rm.view(torch.int32))
    del C_rm
    r = oracle.compress(w.dtype, a)
    Ch = C.cpu().numpy()
    if key == "c2":
        # int8 4096^3: every output (the oracle's int64 sums, exact)
        cref, _ = oracle.spmm(w.dtype, r[0], r[1], b, w.K)
        assert np.array_equal(Ch.astype(np.int64), cref), "c2 packed prefill (all outputs)"
    else:
        # bf16 28672 x 8192 x 2048: whole rows spanning every row-tile
        # position and all eight column tiles (both the full-width tiles and
        # the half-width ones of the last rows), plus a random sample
        rows = np.unique(np.concatenate([np.arange(0, w.M, 997), [255, 256, 24575, 24576, w.M - 1]]))
        cref, sref = oracle.spmm(w.dtype, r[0][rows], r[1][rows], b, w.K)
        check_product(w.dtype, Ch[rows], cref, sref, key + " packed prefill (whole rows)")
        ms, ns = sample_entries(w.M, w.N, 3000, seed=w.index + 70)
        cref, sref = oracle.spmm_entries(w.dtype, r[0], r[1], b, w.K, ms, ns)
        check_product(w.dtype, Ch[ms, ns], cref, sref, key + " packed prefill")


# ---- activation-major B (Bt [N, K] row-major) ------------------------------

BT_SHAPES = [(64, 128, 16), (300, 384, 272), (256, 512, 256), (520, 1152, 528), (77, 256, 5), (600, 384, 1)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", BT_SHAPES)
def test_spmm_prefill_bt_matches_oracle(dt, shape):
    # any N (ragged column tiles, fewer columns than one 16-byte chunk of a
    # B row); against the oracle of C = A B with B = Bt^T, and the same bits
    # as the row-major operand where that one takes the shape
    M, K, N = shape
    a = U.random_matrix(dt, M, K, "normal", seed=M + 13 * K)
    bt = U.random_matrix(dt, N, K, "normal", seed=N + 17)
    b = np.ascontiguousarray(np.asarray(bt).T)
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.compress_prefill(to_dev(a, dt))
    C = ssg.spmm_prefill_bt(pv, pm, M, to_dev(bt, dt))
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "prefill Bt %s %s" % (dt, shape))
    if N % (16 // np.dtype(U.store_dtype(dt)).itemsize) == 0:
        C_rm = ssg.spmm_prefill(pv, pm, M, to_dev(b, dt))
        assert torch.equal(C.view(torch.int32), C_rm.view(torch.int32))


@pytest.mark.parametrize("dt", ["bf16", "i8"])
def test_spmm_prefill_bt_strided_and_mixed_widths(dt):
    # Bt rows longer than K (a column slice of a wider activation matrix)
    # and 260 tiles, so the last row tiles run as half-width tiles
    K = 128 if dt == "bf16" else 256
    M, N = 256 * 20 - 37, 256 * 13 - 48
    a = U.random_matrix(dt, M, K, "normal", seed=41)
    wide = U.random_matrix(dt, N, K + 64, "normal", seed=43)
    bt = np.asarray(wide)[:, 32:32 + K]
    vals, meta = oracle.compress(dt, a)
    pv, pm = ssg.compress_prefill(to_dev(a, dt))
    Bw = to_dev(wide, dt)
    C = ssg.spmm_prefill_bt(pv, pm, M, Bw[:, 32:32 + K])
    b = np.ascontiguousarray(bt.T)
    cref, sref = oracle.spmm(dt, vals, meta, b, K)
    check_product(dt, C.cpu().numpy(), cref, sref, "prefill Bt strided %s" % dt)
    C_rm = ssg.spmm_prefill(pv, pm, M, to_dev(b, dt))
    assert torch.equal(C.view(torch.int32), C_rm.view(torch.int32))


def test_spmm_prefill_bt_exact_small_integers():
    M, K, N = 300, 640, 264
    rng = np.random.default_rng(5)
    a = rng.integers(-3, 4, size=(M, K)).astype(np.float16).view(np.uint16)
    bt = rng.integers(-3, 4, size=(N, K)).astype(np.float16).view(np.uint16)
    vals, meta = oracle.compress("f16", a)
    pv, pm = ssg.compress_prefill(to_dev(a, "f16"))
    C = ssg.spmm_prefill_bt(pv, pm, M, to_dev(bt, "f16")).cpu().numpy().astype(np.float64)
    cref, _ = oracle.spmm("f16", vals, meta, np.ascontiguousarray(bt.T), K)
    assert np.array_equal(C, cref)


def test_spmm_prefill_bt_argument_errors():
    a = U.random_matrix("bf16", 64, 128, "normal", 1)
    pv, pm = ssg.compress_prefill(to_dev(a, "bf16"))
    wide = to_dev(U.random_matrix("bf16", 16, 136, "normal", 2), "bf16")
    with pytest.raises(ssg.SsgError) as e:      # rows of Bt not a multiple of 16 bytes apart
        ssg.spmm_prefill_bt(pv, pm, 64, torch.empty((16, 132), dtype=torch.bfloat16, device="cuda")[:, :128])
    assert e.value.status == 8
    with pytest.raises(ssg.SsgError) as e:      # Bt not 16-byte aligned
        ssg.spmm_prefill_bt(pv, pm, 64, wide[:, 4:132])
    assert e.value.status == 8


def test_full_size_prefill_bt():
    # the headline shape with token-major activations: the same bits as the
    # row-major B product, whose full-size parity is checked above, and
    # whole rows against the oracle
    w = W.WORKLOADS["c4"]
    print("full-size packed prefill, Bt: %s" % w.title, flush=True)
    a_cpu, b_cpu = W.gen_a(w), W.gen_b(w)
    A, B = a_cpu.cuda(), b_cpu.cuda()
    pv, pm = ssg.compress_prefill(A)
    vals, meta = ssg.compress(A)
    del A
    Bt = B.t().contiguous()
    C = ssg.spmm_prefill_bt(pv, pm, w.M, Bt)
    C_rm = ssg.spmm_prefill(pv, pm, w.M, B)
    assert torch.equal(C.view(torch.int32), C_rm.view(torch.int32))
    del C_rm, Bt
    rows = np.array([0, 255, 256, 13001, 24575, 24576, w.M - 1])
    r = oracle.compress(w.dtype, W.bits(a_cpu))
    cref, sref = oracle.spmm(w.dtype, r[0][rows], r[1][rows], W.bits(b_cpu), w.K)
    check_product(w.dtype, C.cpu().numpy()[rows], cref, sref, "c4 packed prefill, Bt (whole rows)")
