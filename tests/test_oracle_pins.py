"""Pins of the CPU oracle against facts fixed outside it: values the pages
print, closed forms, invariants, brute force on tiny inputs and independent
library routines (numpy / torch).  CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import _util as U

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DTS = ["f16", "bf16", "i8", "e4m3", "e5m2"]
FAMILIES = ["normal", "ties", "sparse", "extreme"]


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- decoders

def test_f16_decoder_matches_numpy_on_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero survives
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_bf16_decoder_matches_torch_on_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("dt,fn", [("e4m3", "e4m3_to_f64"), ("e5m2", "e5m2_to_f64")])
def test_fp8_decoders_match_torch_on_every_bit_pattern(dt, fn):
    bits = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(bits.copy()).view(U.TORCH_DTYPE[dt]).to(torch.float64).numpy()
    got = np.array([getattr(oracle, fn)(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.signbit(got[0x80]) and not np.signbit(got[0])
    # the format's own landmarks
    top = {"e4m3": 448.0, "e5m2": 57344.0}[dt]
    tiny = {"e4m3": 2.0 ** -9, "e5m2": 2.0 ** -16}[dt]
    assert np.nanmax(got[np.isfinite(got)]) == top and got[1] == tiny


# ---------------------------------------------------------------- selection

@pytest.mark.parametrize("mags", [
    [5, 3, 3, 1], [3, 3, 3, 3], [2, 5, 5, 5], [5, 3, 5, 3], [0, 0, 0, 5], [1, 2, 3, 4], [4, 3, 2, 1],
    [0, 0, 0, 0], [1, 0, 0, 1], [0, 7, 0, 7],
])
def test_select_group_equals_pair_enumeration(mags):
    keep = oracle.select_group(mags)
    p, q = U.brute_pair(mags)
    assert keep == [int(i in (p, q)) for i in range(4)]


def test_worked_example_from_the_pages():
    g = _golden("worked_example.json")
    for dt, case in g["cases"].items():
        row = U.encode(dt, case["row"]).reshape(1, -1)
        vals, meta = oracle.compress(dt, row)
        assert np.array_equal(U.to_f64(dt, vals)[0], case["vals"])
        assert list(meta[0]) == case["meta"]
        nibs = [meta[0, 0] & 0xF, meta[0, 0] >> 4]
        assert [[n & 3, n >> 2] for n in nibs] == case["indices"]
        P = oracle.prune(dt, row)
        assert np.array_equal(U.to_f64(dt, P)[0], case["pruned"])


def test_hand_cases():
    # all equal -> the two lowest positions
    v, m = oracle.compress("f16", U.encode("f16", [1, 1, 1, 1]).reshape(1, 4))
    assert m[0, 0] == 0x4 and list(U.to_f64("f16", v)[0]) == [1, 1]
    # one non-zero: a zero is stored beside it, positions ascending
    v, m = oracle.compress("f16", U.encode("f16", [0, 0, 0, 5]).reshape(1, 4))
    assert m[0, 0] == 0xC and list(U.to_f64("f16", v)[0]) == [0, 5]
    # -0 and +0 tie; kept bits are copied (the -0 stays -0)
    a = np.array([[0x8000, 0x0000, 0x0000, 0x0000]], dtype=np.uint16)
    v, m = oracle.compress("f16", a)
    assert m[0, 0] == 0x4 and list(v[0]) == [0x8000, 0x0000]
    # int8: |-128| = 128 outranks 127
    v, m = oracle.compress("i8", np.array([[127, 3, -128, 5]], dtype=np.int8))
    assert m[0, 0] == (0 | (2 << 2)) and list(v[0]) == [127, -128]
    # bf16: magnitude, not sign, decides
    v, m = oracle.compress("bf16", U.encode("bf16", [-8, 1, 7, -2]).reshape(1, 4))
    assert m[0, 0] == (0 | (2 << 2)) and list(U.to_f64("bf16", v)[0]) == [-8, 7]


@pytest.mark.parametrize("dt", DTS)
def test_selection_matches_pair_enumeration_on_8x8(dt):
    for seed in range(40):
        for fam in FAMILIES:
            A = U.random_matrix(dt, 8, 8, fam, seed)
            keep = U.brute_keep_mask(dt, A)
            vals, meta = oracle.compress(dt, A)
            for m in range(8):
                for g in range(2):
                    kept = [p for p in range(4) if keep[m, 4 * g + p]]
                    nib = (meta[m, g // 2] >> (4 * (g % 2))) & 0xF
                    assert [nib & 3, nib >> 2] == kept
                    assert list(vals[m, 2 * g:2 * g + 2]) == [A[m, 4 * g + kept[0]], A[m, 4 * g + kept[1]]]


# ---------------------------------------------------------------- the pages' printed numbers

def test_printed_byte_accounting_of_the_listing():
    g = _golden("byte_accounting.json")
    torch.manual_seed(0)
    W = torch.randn(g["M"], g["K"])                    # the listing's own input
    A = W.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    vals, meta = oracle.compress("f16", A)
    P = oracle.prune("f16", A)
    zero = U.is_zero("f16", P)
    assert "%.1f%%" % (100 * zero.mean()) == g["printed"]["sparsity"]
    per_group = (~zero).reshape(g["M"], g["K"] // 4, 4).sum(-1)
    assert bool((per_group == 2).all()) is g["printed"]["all_groups_have_exactly_2_nonzeros"]
    dense = A.size * g["bytes_per_value"]
    sparse = vals.nbytes + meta.nbytes                 # values + 2 bits per kept value
    assert "%.1f" % (dense / 1024) == g["printed"]["dense_KB"]
    assert "%.1f" % (sparse / 1024) == g["printed"]["sparse_KB"]
    assert "%.1f%%" % (100 * sparse / dense) == g["printed"]["sparse_fraction_of_dense"]


def test_storage_closed_form():
    g = _golden("storage_closed_form.json")
    M, K = 16, 64
    for dt, b in (("f16", 16), ("i8", 8)):
        A = U.random_matrix(dt, M, K, "normal", 7)
        vals, meta = oracle.compress(dt, A)
        assert vals.size * 2 == A.size                  # half of the values are stored
        assert meta.size * 8 == A.size                  # one metadata bit per dense element
        frac = (vals.nbytes + meta.nbytes) / A.nbytes
        assert frac == pytest.approx(0.5 + 1.0 / b)
    p = g["printed"]
    assert "%d%%" % round(100 * (0.5 + 1 / 16)) == p["fp16_fraction_of_dense"]
    assert "%d%%" % round(100 * (1 / 16)) == p["metadata_overhead_16bit"]
    assert "%d%%" % round(100 * (1 / 4)) == p["metadata_overhead_4bit"]
    assert "%.1fx" % (1 / (0.5 + 1 / 16)) == p["decode_bandwidth_gain_fp16"]


# ---------------------------------------------------------------- invariants and round trips

@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("fam", FAMILIES)
def test_invariants(dt, fam):
    A = U.random_matrix(dt, 24, 64, fam, 11)
    P = oracle.prune(dt, A)
    mag_a = np.abs(U.to_f64(dt, A)).reshape(24, 16, 4)
    keep = U.brute_keep_mask(dt, A).reshape(24, 16, 4)
    # (i) every kept magnitude >= every dropped magnitude in its group
    kept_min = np.where(keep, mag_a, np.inf).min(-1)
    drop_max = np.where(~keep, mag_a, -np.inf).max(-1)
    assert (kept_min >= drop_max).all()
    # (ii)/(iii) at most two non-zeros per group, exactly min(nnz_g(A), 2)
    nz_a = (~U.is_zero(dt, A)).reshape(24, 16, 4).sum(-1)
    nz_p = (~U.is_zero(dt, P)).reshape(24, 16, 4).sum(-1)
    assert (nz_p <= 2).all()
    assert np.array_equal(nz_p, np.minimum(nz_a, 2))
    # dropped positions are +0 bits; kept positions are bit copies
    Pg = P.reshape(24, 16, 4)
    Ag = A.reshape(24, 16, 4)
    assert np.array_equal(Pg[keep], Ag[keep])
    assert (Pg[~keep] == 0).all()


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("fam", FAMILIES)
def test_roundtrip_and_idempotence(dt, fam):
    A = U.random_matrix(dt, 16, 72, fam, 3)           # K=72: odd number of groups per meta byte
    vals, meta = oracle.compress(dt, A)
    D, bad = oracle.decompress(dt, vals, meta, 72)
    assert bad == 0
    assert np.array_equal(D, oracle.prune(dt, A))
    v2, m2 = oracle.compress(dt, oracle.prune(dt, A))
    assert np.array_equal(v2, vals) and np.array_equal(m2, meta)
    groups = np.stack([meta & 0xF, meta >> 4], axis=-1).reshape(16, -1)[:, :18]
    assert set(np.unique(groups)) <= U.VALID_NIBBLES
    # the unused high nibble of the last byte (18 groups -> 9 bytes exactly) is absent;
    # K=20 leaves one: it must be 0
    A5 = U.random_matrix(dt, 3, 20, fam, 4)
    _, m5 = oracle.compress(dt, A5)
    assert m5.shape == (3, 3) and (m5[:, 2] >> 4 == 0).all()


@pytest.mark.parametrize("dt", DTS)
def test_decompress_counts_invalid_nibbles_and_zero_fills(dt):
    A = U.random_matrix(dt, 4, 16, "normal", 5)
    vals, meta = oracle.compress(dt, A)
    meta = meta.copy()
    meta[1, 0] = (meta[1, 0] & 0xF0) | 0x5            # (1,1): repeated position
    meta[2, 1] = (meta[2, 1] & 0x0F) | (0x7 << 4)     # (3,1): descending
    D, bad = oracle.decompress(dt, vals, meta, 16)
    assert bad == 2
    assert (D[1, 0:4] == 0).all() and (D[2, 12:16] == 0).all()
    ref = oracle.prune(dt, A)
    assert np.array_equal(D[0], ref[0]) and np.array_equal(D[3], ref[3])
    with pytest.raises(oracle.OracleError):
        oracle.spmm(dt, vals, meta, U.random_matrix(dt, 16, 4, "normal", 6), 16)


# ---------------------------------------------------------------- residual split

@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("fam", ["normal", "ties", "sparse"])
def test_split(dt, fam):
    M, K = 20, 48
    A = U.random_matrix(dt, M, K, fam, 9)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, A)
    v0, m0 = oracle.compress(dt, A)
    assert np.array_equal(vals, v0) and np.array_equal(meta, m0)
    keep = U.brute_keep_mask(dt, A)
    nz = ~U.is_zero(dt, A)
    want = nz & ~keep                                  # dropped non-zeros
    assert row_ptr[0] == 0 and np.array_equal(np.diff(row_ptr), want.sum(1))
    for m in range(M):
        cols = col[row_ptr[m]:row_ptr[m + 1]]
        assert list(cols) == list(np.nonzero(want[m])[0])            # ascending
        assert np.array_equal(rvals[row_ptr[m]:row_ptr[m + 1]], A[m, cols])
    # nnz(L) + nnz(R) = nnz(A); residual only in groups with > 2 non-zeros, at most 2 per group
    P = oracle.prune(dt, A)
    assert (~U.is_zero(dt, P)).sum() + len(col) == nz.sum()
    per_group_r = want.reshape(M, K // 4, 4).sum(-1)
    per_group_a = nz.reshape(M, K // 4, 4).sum(-1)
    assert (per_group_r <= 2).all() and (per_group_r[per_group_a <= 2] == 0).all()
    # decompress(L) + scatter(R) reproduces A's values
    D, _ = oracle.decompress(dt, vals, meta, K)
    Dv = U.to_f64(dt, D)
    Dv[np.repeat(np.arange(M), np.diff(row_ptr)), col] += U.to_f64(dt, rvals)
    assert np.array_equal(Dv, U.to_f64(dt, A))


# ---------------------------------------------------------------- delta-coded residual

def _golden_delta(dt):
    g = _golden("delta_code.json")
    rows = g["rows"]
    row_ptr = np.concatenate([[0], np.cumsum([len(r["col"]) for r in rows])]).astype(np.int32)
    col = np.array([c for r in rows for c in r["col"]], dtype=np.int32)
    rvals = U.encode(dt, np.array([v for r in rows for v in r["val"]], dtype=np.float64))
    return g, row_ptr, col, rvals


@pytest.mark.parametrize("dt", DTS)
def test_delta_code_hand_worked_rows(dt):
    g, row_ptr, col, rvals = _golden_delta(dt)
    drow_ptr, dcol, dvals = oracle.delta_encode(dt, row_ptr, col, rvals, g["K"])
    assert list(drow_ptr) == g["drow_ptr"]
    assert list(dcol) == [d for r in g["rows"] for d in r["dcol"]]
    want = U.encode(dt, np.array([v for r in g["rows"] for v in r["dval"]], dtype=np.float64))
    assert np.array_equal(dvals, want)                  # fillers are +0 (all bits clear)


def _random_csr(M, K, density, seed, far=False):
    """Random CSR rows (ascending columns); `far` spreads a few entries over
    long gaps so that fillers appear."""
    rng = np.random.default_rng(seed)
    cols = []
    for m in range(M):
        if far:
            c = np.sort(rng.choice(K, size=rng.integers(0, 6), replace=False))
        else:
            c = np.nonzero(rng.random(K) < density)[0]
        cols.append(c)
    row_ptr = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    col = np.concatenate(cols).astype(np.int32) if row_ptr[-1] else np.zeros(0, np.int32)
    return row_ptr, col


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("far", [False, True])
def test_delta_code_invariants(dt, far):
    M, K = 40, 3000
    row_ptr, col = _random_csr(M, K, 0.09, 7 + far, far)
    rvals = U.random_matrix(dt, 1, max(len(col), 1), "normal", 8)[0, :len(col)]
    rvals = np.where(U.is_zero(dt, rvals), U.encode(dt, np.ones(len(col))), rvals)   # no explicit zeros
    drow_ptr, dcol, dvals = oracle.delta_encode(dt, row_ptr, col, rvals, K)
    assert drow_ptr[0] == 0 and (np.diff(drow_ptr) >= 0).all()
    assert ((dcol >= 1) & (dcol <= 255)).all()
    nz = ~U.is_zero(dt, dvals)
    for m in range(M):
        lo, hi, dlo, dhi = row_ptr[m], row_ptr[m + 1], drow_ptr[m], drow_ptr[m + 1]
        c = col[lo:hi].astype(np.int64)
        gaps = np.diff(np.concatenate([[-1], c]))
        assert dhi - dlo == len(c) + ((gaps - 1) // 255).sum()          # closed-form length
        dec = np.cumsum(dcol[dlo:dhi].astype(np.int64)) - 1             # running sum decodes the columns
        real = nz[dlo:dhi]
        assert np.array_equal(dec[real], c)
        assert np.array_equal(dvals[dlo:dhi][real], rvals[lo:hi])
        assert (dcol[dlo:dhi][~real] == 255).all()                      # fillers: full steps, value +0
        if len(c):
            assert dec[-1] == c[-1] and real[-1]
    if far:
        assert (~nz).sum() > 0                                           # the case exercises fillers


@pytest.mark.parametrize("dt", DTS)
def test_spmm_residual_delta_equals_csr_product(dt):
    M, K, N = 24, 1024, 10
    A = U.random_matrix(dt, M, K, "sparse", 61)
    B = U.random_matrix(dt, K, N, "normal", 62)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, A)
    drow_ptr, dcol, dvals = oracle.delta_encode(dt, row_ptr, col, rvals, K)
    C0, S0 = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, B, K)
    C1, S1 = oracle.spmm_residual_delta(dt, vals, meta, drow_ptr, dcol, dvals, B, K)
    assert np.array_equal(C0, C1)
    if S0 is not None:
        assert np.array_equal(S0, S1)
    # against the dense product of A itself
    if dt == "i8":
        assert np.array_equal(C1, U.to_i64(A) @ U.to_i64(B))
    else:
        ref = U.to_f64(dt, A) @ U.to_f64(dt, B)
        assert np.allclose(C1, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    rng = np.random.default_rng(3)
    ms, ns = rng.integers(0, M, 40), rng.integers(0, N, 40)
    e, _ = oracle.spmm_entries(dt, vals, meta, B, K, ms, ns, residual=(drow_ptr, dcol, dvals), delta=True)
    assert np.array_equal(e, C1[ms, ns])


def test_spmm_residual_delta_with_fillers_bruteforce():
    # residual entries far apart (fillers), int8 so every sum is exact
    M, K, N = 6, 1200, 3
    row_ptr, col = _random_csr(M, K, 0.0, 5, far=True)
    rng = np.random.default_rng(4)
    rv = rng.integers(1, 9, size=len(col)) * rng.choice([-1, 1], size=len(col))
    rvals = U.encode("i8", rv)
    B = U.encode("i8", rng.integers(-5, 6, size=(K, N)))
    vals = np.zeros((M, K // 2), dtype=np.int8)
    meta = np.full((M, K // 8), 0x44, dtype=np.uint8)                     # keep positions 0, 1 (values 0)
    drow_ptr, dcol, dvals = oracle.delta_encode("i8", row_ptr, col, rvals, K)
    C, _ = oracle.spmm_residual_delta("i8", vals, meta, drow_ptr, dcol, dvals, B, K)
    want = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        for j in range(row_ptr[m], row_ptr[m + 1]):
            for n in range(N):
                want[m, n] += int(rv[j]) * int(B[col[j], n])
    assert np.array_equal(C, want)


@pytest.mark.parametrize("dt", DTS)
def test_spmm_csr_equals_dense_product_of_the_scattered_matrix(dt):
    M, K, N = 30, 200, 7
    row_ptr, col = _random_csr(M, K, 0.15, 21)
    vals = U.random_matrix(dt, 1, max(len(col), 1), "normal", 22)[0, :len(col)]
    B = U.random_matrix(dt, K, N, "normal", 23)
    C, S = oracle.spmm_csr(dt, row_ptr, col, vals, B, K)
    D = np.zeros((M, K))
    D[np.repeat(np.arange(M), np.diff(row_ptr)), col] = U.to_f64(dt, vals)   # independent scatter
    if dt == "i8":
        assert np.array_equal(C, D.astype(np.int64) @ U.to_i64(B))
    else:
        ref = D @ U.to_f64(dt, B)
        assert np.allclose(C, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        assert np.allclose(S, np.abs(D) @ np.abs(U.to_f64(dt, B)), rtol=1e-12)
    # and the same matrix as a residual on an all-zero 2:4 layer
    if K % 4 == 0:
        vz = np.zeros((M, K // 2), dtype=U.store_dtype(dt))
        mz = np.full((M, (K + 7) // 8), 0x44, dtype=np.uint8)
        C2, _ = oracle.spmm_residual(dt, vz, mz, row_ptr, col, vals, B, K)
        assert np.array_equal(C, C2)


def test_delta_code_rejects_bad_csr():
    K = 100
    for row_ptr, col in [([0, 2], [5, 5]), ([0, 2], [7, 3]), ([0, 1], [100]), ([0, 1], [-1]), ([0, 2, 1], [1, 2])]:
        with pytest.raises(oracle.OracleError, match="bad format"):
            oracle.delta_encode("i8", np.array(row_ptr), np.array(col), np.ones(len(col), np.int8), K)


# ---------------------------------------------------------------- products

def _exact_small(dt, shape, seed, lo=-3, hi=3):
    rng = np.random.default_rng(seed)
    return U.encode(dt, rng.integers(lo, hi + 1, size=shape))


@pytest.mark.parametrize("dt", DTS)
def test_spmm_bruteforce_exact_8x8(dt):
    for seed in range(30):
        A = _exact_small(dt, (8, 8), seed)
        B = _exact_small(dt, (8, 8), seed + 1000)
        keep = U.brute_keep_mask(dt, A)
        a = [[int(x) for x in row] for row in U.to_f64(dt, A)]
        b = [[int(x) for x in row] for row in U.to_f64(dt, B)]
        want = [[sum(a[m][k] * b[k][n] for k in range(8) if keep[m, k]) for n in range(8)] for m in range(8)]
        vals, meta = oracle.compress(dt, A)
        C, S = oracle.spmm(dt, vals, meta, B, 8)
        assert np.array_equal(np.asarray(C, dtype=np.float64), np.array(want, dtype=np.float64))
        if S is not None:
            sw = [[sum(abs(a[m][k] * b[k][n]) for k in range(8) if keep[m, k]) for n in range(8)] for m in range(8)]
            assert np.array_equal(S, np.array(sw, dtype=np.float64))


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("shape", [(37, 64, 9), (16, 256, 33), (1, 4, 1), (5, 12, 64)])
def test_spmm_matches_numpy_matmul(dt, shape):
    M, K, N = shape
    A = U.random_matrix(dt, M, K, "normal", M + K)
    B = U.random_matrix(dt, K, N, "normal", N + 17)
    vals, meta = oracle.compress(dt, A)
    C, S = oracle.spmm(dt, vals, meta, B, K)
    P = np.where(U.brute_keep_mask(dt, A), U.to_f64(dt, A), 0.0)   # independent pruned dense
    if dt == "i8":
        ref = P.astype(np.int64) @ U.to_i64(B)
        assert np.array_equal(C, ref)
    else:
        Bf = U.to_f64(dt, B)
        ref = P @ Bf
        assert np.allclose(C, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        assert np.allclose(S, np.abs(P) @ np.abs(Bf), rtol=1e-12, atol=0)
        assert (S >= np.abs(C) - 1e-12).all()


@pytest.mark.parametrize("dt", DTS)
def test_spmm_identity_B_returns_the_pruned_matrix(dt):
    K = 32
    A = U.random_matrix(dt, 12, K, "normal", 21)
    I = U.encode(dt, np.eye(K))
    vals, meta = oracle.compress(dt, A)
    C, _ = oracle.spmm(dt, vals, meta, I, K)
    assert np.array_equal(np.asarray(C, dtype=np.float64), U.to_f64(dt, oracle.prune(dt, A)))


@pytest.mark.parametrize("dt", DTS)
def test_spmm_residual_equals_dense_product(dt):
    M, K, N = 24, 64, 10
    A = U.random_matrix(dt, M, K, "sparse", 31)
    B = U.random_matrix(dt, K, N, "normal", 32)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, A)
    C, S = oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, B, K)
    if dt == "i8":
        assert np.array_equal(C, U.to_i64(A) @ U.to_i64(B))
    else:
        ref = U.to_f64(dt, A) @ U.to_f64(dt, B)
        assert np.allclose(C, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        assert np.allclose(S, np.abs(U.to_f64(dt, A)) @ np.abs(U.to_f64(dt, B)), rtol=1e-12)


@pytest.mark.parametrize("dt", DTS)
def test_spmm_entries_match_the_full_product(dt):
    M, K, N = 20, 40, 12
    A = U.random_matrix(dt, M, K, "sparse", 41)
    B = U.random_matrix(dt, K, N, "normal", 42)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, A)
    rng = np.random.default_rng(0)
    ms, ns = rng.integers(0, M, 50), rng.integers(0, N, 50)
    for residual in (None, (row_ptr, col, rvals)):
        full, fs = (oracle.spmm(dt, vals, meta, B, K) if residual is None
                    else oracle.spmm_residual(dt, vals, meta, row_ptr, col, rvals, B, K))
        e, es = oracle.spmm_entries(dt, vals, meta, B, K, ms, ns, residual=residual)
        assert np.array_equal(e, full[ms, ns])
        if fs is not None:
            assert np.array_equal(es, fs[ms, ns])


def test_int8_linearity_in_B():
    A = U.random_matrix("i8", 9, 32, "normal", 51)
    B1 = U.encode("i8", np.random.default_rng(1).integers(-60, 61, size=(32, 7)))
    B2 = U.encode("i8", np.random.default_rng(2).integers(-60, 61, size=(32, 7)))
    vals, meta = oracle.compress("i8", A)
    c1, _ = oracle.spmm("i8", vals, meta, B1, 32)
    c2, _ = oracle.spmm("i8", vals, meta, B2, 32)
    c12, _ = oracle.spmm("i8", vals, meta, (B1.astype(np.int16) + B2).astype(np.int8), 32)
    assert np.array_equal(c12, c1 + c2)


# ---------------------------------------------------------------- argument errors

def test_errors():
    A = U.random_matrix("f16", 2, 6, "normal", 0)
    with pytest.raises(oracle.OracleError, match="bad shape"):
        oracle.compress("f16", A)                      # K % 4 != 0
    nan = U.encode("f16", [1.0, np.nan, 0.0, 2.0]).reshape(1, 4)
    with pytest.raises(oracle.OracleError, match="non-finite"):
        oracle.compress("f16", nan)
    inf = U.encode("bf16", [1.0, np.inf, 0.0, 2.0]).reshape(1, 4)
    with pytest.raises(oracle.OracleError, match="non-finite"):
        oracle.prune("bf16", inf)
    with pytest.raises(oracle.OracleError):
        oracle.compress("f32", A)
    for dt, bad in (("e4m3", 0x7F), ("e5m2", 0x7C), ("e5m2", 0xFE)):   # NaN, +Inf, NaN
        a8 = np.array([[0x38, bad, 0, 0x38]], dtype=np.uint8)
        with pytest.raises(oracle.OracleError, match="non-finite"):
            oracle.compress(dt, a8)


def test_empty_inputs():
    for dt in DTS:
        A = np.zeros((0, 8), dtype=U.store_dtype(dt))
        v, m = oracle.compress(dt, A)
        assert v.shape == (0, 4) and m.shape == (0, 1)
        A = np.zeros((3, 0), dtype=U.store_dtype(dt))
        v, m = oracle.compress(dt, A)
        assert v.shape == (3, 0) and m.shape == (3, 0)


# ---------------------------------------------------------------- N:M generalization

@pytest.mark.parametrize("pat", ["1:4", "2:4", "2:8", "4:8"])
def test_nm_hand_worked_rows(pat):
    n, m = map(int, pat.split(":"))
    for case in _golden("nm_select.json")["cases"]:
        if case["dt"] == "i4":
            row = np.array([case["row_bytes"]], dtype=np.uint8)
            assert np.array_equal(W.pack_i4(np.array([case["row"]])), row)      # the packing itself
            assert list(U.to_f64("i4", row)[0]) == case["row"]
            want = case["expect_bytes"][pat]
        elif case["dt"] == "i8":
            row = np.array([case["row"]], dtype=np.int8)
            want = case["expect"][pat]
        else:
            row = np.array([case["row_bits"]], dtype=np.uint16)
            want = case["expect_bits"][pat]
        vals, mask = oracle.compress_nm(case["dt"], n, m, row)
        assert [int(v) for v in vals[0]] == want["vals"], case["why"]
        assert [int(b) for b in mask[0]] == want["mask"], case["why"]


@pytest.mark.parametrize("n,m", [(1, 4), (2, 4), (3, 4), (1, 8), (2, 8), (3, 8), (4, 8), (5, 8), (2, 16)])
def test_select_nm_equals_subset_enumeration(n, m):
    rng = np.random.default_rng(100 * n + m)
    for trial in range(300):
        hi = 1 + trial % 4                              # few distinct magnitudes: many ties
        mags = [float(x) for x in rng.integers(0, hi + 1, size=m)]
        keep = oracle.select_nm(n, m, mags)
        sub = U.brute_subset(mags, n)
        assert keep == [int(p in sub) for p in range(m)], mags


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", U.NM_PATTERNS)
def test_compress_nm_matches_subset_enumeration(dt, n, m):
    for seed in range(12):
        for fam in FAMILIES:
            A = U.random_matrix(dt, 6, 16, fam, seed)
            keep = U.brute_keep_mask_nm(dt, A, n, m)
            vals, mask = oracle.compress_nm(dt, n, m, A)
            assert np.array_equal(U.mask_bits(mask, 16), keep)
            # values: the kept elements, row by row in ascending k
            assert np.array_equal(vals, A[keep].reshape(6, 16 * n // m))


@pytest.mark.parametrize("dt", DTS)
def test_nm_2_of_4_is_the_2to4_format(dt):
    A = U.random_matrix(dt, 20, 72, "ties", 5)
    v24, meta = oracle.compress(dt, A)
    vnm, mask = oracle.compress_nm(dt, 2, 4, A)
    assert np.array_equal(v24, vnm)
    nib = np.stack([meta & 0xF, meta >> 4], axis=-1).reshape(20, -1)[:, :18]
    pos = np.zeros((20, 72), dtype=bool)
    for g in range(18):
        pos[np.arange(20), 4 * g + (nib[:, g] & 3)] = True
        pos[np.arange(20), 4 * g + (nib[:, g] >> 2)] = True
    assert np.array_equal(U.mask_bits(mask, 72), pos)
    B = U.random_matrix(dt, 72, 9, "normal", 6)
    C24, S24 = oracle.spmm(dt, v24, meta, B, 72)
    Cnm, Snm = oracle.spmm_nm(dt, 2, 4, vnm, mask, B, 72)
    assert np.array_equal(C24, Cnm)
    if S24 is not None:
        assert np.array_equal(S24, Snm)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", U.NM_PATTERNS)
def test_nm_invariants_and_roundtrip(dt, n, m):
    M, K = 12, 64
    for fam in FAMILIES:
        A = U.random_matrix(dt, M, K, fam, 13)
        vals, mask = oracle.compress_nm(dt, n, m, A)
        keep = U.mask_bits(mask, K)
        assert vals.shape == (M, K * n // m) and mask.shape == (M, K // 8)
        assert (keep.reshape(M, K // m, m).sum(-1) == n).all()
        mag = np.abs(U.to_f64(dt, A)).reshape(M, K // m, m)
        kg = keep.reshape(M, K // m, m)
        assert (np.where(kg, mag, np.inf).min(-1) >= np.where(~kg, mag, -np.inf).max(-1)).all()
        D, bad = oracle.decompress_nm(dt, n, m, vals, mask, K)
        assert bad == 0
        assert np.array_equal(D[keep], A[keep]) and (D[~keep] == 0).all()
        v2, m2 = oracle.compress_nm(dt, n, m, D)        # re-selecting the expansion keeps the same set
        assert np.array_equal(v2, vals) and np.array_equal(m2, mask)
    # n:m keeps a subset of what a larger n keeps for the same m
    if n < m // 2:
        A = U.random_matrix(dt, M, K, "normal", 14)
        small = U.mask_bits(oracle.compress_nm(dt, n, m, A)[1], K)
        big = U.mask_bits(oracle.compress_nm(dt, m // 2, m, A)[1], K)
        assert (big | ~small).all()


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", U.NM_PATTERNS)
def test_spmm_nm_bruteforce_exact(dt, n, m):
    for seed in range(8):
        A = _exact_small(dt, (8, 16), seed)
        B = _exact_small(dt, (16, 5), seed + 500)
        keep = U.brute_keep_mask_nm(dt, A, n, m)
        a = [[int(x) for x in row] for row in U.to_f64(dt, A)]
        b = [[int(x) for x in row] for row in U.to_f64(dt, B)]
        want = [[sum(a[r][k] * b[k][c] for k in range(16) if keep[r, k]) for c in range(5)] for r in range(8)]
        vals, mask = oracle.compress_nm(dt, n, m, A)
        C, S = oracle.spmm_nm(dt, n, m, vals, mask, B, 16)
        assert np.array_equal(np.asarray(C, dtype=np.float64), np.array(want, dtype=np.float64))
        if S is not None:
            sw = [[sum(abs(a[r][k] * b[k][c]) for k in range(16) if keep[r, k]) for c in range(5)] for r in range(8)]
            assert np.array_equal(S, np.array(sw, dtype=np.float64))


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("n,m", U.NM_PATTERNS)
def test_spmm_nm_matches_numpy_matmul(dt, n, m):
    M, K, N = 33, 200, 17
    A = U.random_matrix(dt, M, K, "normal", 41)
    B = U.random_matrix(dt, K, N, "normal", 42)
    vals, mask = oracle.compress_nm(dt, n, m, A)
    C, S = oracle.spmm_nm(dt, n, m, vals, mask, B, K)
    P = np.where(U.brute_keep_mask_nm(dt, A, n, m), U.to_f64(dt, A), 0.0)
    if dt == "i8":
        assert np.array_equal(C, P.astype(np.int64) @ U.to_i64(B))
    else:
        Bf = U.to_f64(dt, B)
        ref = P @ Bf
        assert np.allclose(C, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
        assert np.allclose(S, np.abs(P) @ np.abs(Bf), rtol=1e-12, atol=0)


def test_nm_bad_masks_and_errors():
    A = U.random_matrix("i8", 3, 16, "normal", 1)
    vals, mask = oracle.compress_nm("i8", 2, 8, A)
    bad = mask.copy()
    bad[1, 0] |= 0xFF                                   # row 1, group 0: eight bits set
    bad[2, 1] = 0x01                                    # row 2, group 1: one bit set
    D, nbad = oracle.decompress_nm("i8", 2, 8, vals, bad, 16)
    assert nbad == 2
    assert (D[1, :8] == 0).all() and (D[2, 8:] == 0).all()
    D0, _ = oracle.decompress_nm("i8", 2, 8, vals, mask, 16)
    assert np.array_equal(D[0], D0[0]) and np.array_equal(D[1, 8:], D0[1, 8:])
    B = U.random_matrix("i8", 16, 4, "normal", 2)
    with pytest.raises(oracle.OracleError, match="bad format"):
        oracle.spmm_nm("i8", 2, 8, vals, bad, B, 16)
    for n, m, K in [(4, 4, 16), (0, 4, 16), (2, 8, 12), (1, 1, 16)]:
        with pytest.raises(oracle.OracleError, match="shape"):
            oracle.compress_nm("i8", n, m, U.random_matrix("i8", 2, K, "normal", 3))
    nan = U.encode("f16", [1.0, float("nan"), 0.0, 2.0]).reshape(1, 4)
    with pytest.raises(oracle.OracleError):
        oracle.compress_nm("f16", 1, 4, nan)


# ---------------------------------------------------------------- 4-bit weights (N:M family)

def test_i4_decoder_on_every_byte():
    for b in range(256):
        lo, hi = b & 0xF, b >> 4
        assert oracle.i4_to_f64(b, False) == (lo - 16 if lo >= 8 else lo)
        assert oracle.i4_to_f64(b, True) == (hi - 16 if hi >= 8 else hi)
        assert list(U.to_f64("i4", np.array([[b]], dtype=np.uint8))[0]) == [oracle.i4_to_f64(b, False),
                                                                         oracle.i4_to_f64(b, True)]


@pytest.mark.parametrize("n,m", [(1, 4), (2, 4), (2, 8), (4, 8), (3, 8)])
def test_i4_compress_matches_subset_enumeration(n, m):
    for seed in range(10):
        for fam in FAMILIES:
            A = U.random_matrix("i4", 6, 32, fam, seed)
            keep = U.brute_keep_mask_nm("i4", A, n, m)
            vals, mask = oracle.compress_nm("i4", n, m, A)
            assert np.array_equal(U.mask_bits(mask, 32), keep)
            assert np.array_equal(U.to_f64("i4", vals), U.to_f64("i4", A)[keep].reshape(6, 32 * n // m))
            D, bad = oracle.decompress_nm("i4", n, m, vals, mask, 32)
            assert bad == 0
            assert np.array_equal(U.to_f64("i4", D), np.where(keep, U.to_f64("i4", A), 0.0))


def test_i4_2_of_4_selects_as_int8_does():
    """The same integers stored as int8 go through the independent 2:4
    compressor: the kept values and positions agree."""
    rng = np.random.default_rng(9)
    v = rng.choice([-8, -7, -2, -1, 0, 1, 2, 7], size=(16, 64))
    v24, meta = oracle.compress("i8", v.astype(np.int8))
    vi4, mask = oracle.compress_nm("i4", 2, 4, W.pack_i4(v))
    assert np.array_equal(U.to_f64("i4", vi4), v24.astype(np.float64))
    nib = np.stack([meta & 0xF, meta >> 4], axis=-1).reshape(16, -1)
    pos = np.zeros((16, 64), dtype=bool)
    for g in range(16):
        pos[np.arange(16), 4 * g + (nib[:, g] & 3)] = True
        pos[np.arange(16), 4 * g + (nib[:, g] >> 2)] = True
    assert np.array_equal(U.mask_bits(mask, 64), pos)


@pytest.mark.parametrize("n,m", [(2, 4), (2, 8), (4, 8)])
def test_i4_w4a16_product_exact(n, m):
    for seed in range(6):
        A = U.random_matrix("i4", 8, 32, "normal", seed)
        b = np.random.default_rng(seed + 50).integers(-3, 4, size=(32, 5))
        B = U.encode("f16", b)
        keep = U.brute_keep_mask_nm("i4", A, n, m)
        a = U.to_f64("i4", A).astype(np.int64)
        want = np.array([[sum(int(a[r, k]) * int(b[k, c]) for k in range(32) if keep[r, k]) for c in range(5)]
                         for r in range(8)], dtype=np.float64)
        vals, mask = oracle.compress_nm("i4", n, m, A)
        C, S = oracle.spmm_nm("i4", n, m, vals, mask, B, 32)
        assert np.array_equal(C, want)
        sw = np.array([[sum(abs(int(a[r, k]) * int(b[k, c])) for k in range(32) if keep[r, k]) for c in range(5)]
                       for r in range(8)], dtype=np.float64)
        assert np.array_equal(S, sw)


def test_i4_w4a16_product_matches_numpy():
    A = U.random_matrix("i4", 33, 256, "normal", 3)
    B = U.random_matrix("f16", 256, 17, "normal", 4)
    vals, mask = oracle.compress_nm("i4", 2, 4, A)
    C, S = oracle.spmm_nm("i4", 2, 4, vals, mask, B, 256)
    P = np.where(U.brute_keep_mask_nm("i4", A, 2, 4), U.to_f64("i4", A), 0.0)
    Bf = U.to_f64("f16", B)
    assert np.allclose(C, P @ Bf, rtol=1e-12, atol=1e-12 * np.abs(P @ Bf).max())
    assert np.allclose(S, np.abs(P) @ np.abs(Bf), rtol=1e-12, atol=0)


@pytest.mark.parametrize("dt", ["i4", "i8", "f16"])
def test_nm_outputs_overwrite_whatever_the_buffers_held(dt):
    """Compression and expansion write every byte of their outputs: buffers
    filled with 0xFF beforehand end up as they do when they start zeroed."""
    import ctypes
    A = U.random_matrix(dt, 5, 32, "sparse", 21)
    e = 2 if dt == "i4" else 1
    vals, mask = oracle.compress_nm(dt, 2, 8, A)
    D0, _ = oracle.decompress_nm(dt, 2, 8, vals, mask, 32)
    lib = oracle._load()
    dirty_v = np.full_like(vals, 0xFF if vals.dtype != np.int8 else -1)
    dirty_m = np.full_like(mask, 0xFF)
    rc = lib.orc_compress_nm(oracle.DTYPES[dt], 2, 8, 5, 32, A.ctypes.data_as(ctypes.c_void_p), 32,
                             dirty_v.ctypes.data_as(ctypes.c_void_p), vals.shape[1] * e,
                             dirty_m.ctypes.data_as(ctypes.c_void_p), mask.shape[1])
    assert rc == 0 and np.array_equal(dirty_v, vals) and np.array_equal(dirty_m, mask)
    dirty_d = np.full_like(D0, 0xFF if D0.dtype != np.int8 else -1)
    bad = lib.orc_decompress_nm(oracle.DTYPES[dt], 2, 8, 5, 32, vals.ctypes.data_as(ctypes.c_void_p),
                                vals.shape[1] * e, mask.ctypes.data_as(ctypes.c_void_p), mask.shape[1],
                                dirty_d.ctypes.data_as(ctypes.c_void_p), D0.shape[1] * e)
    assert bad == 0 and np.array_equal(dirty_d, D0)


# ---------------------------------------------------------------- complement-bitmap residual

def _cbm_golden_matrix(dt, K):
    g = _golden("cbm_example.json")
    dense = np.zeros((g["M"], K))
    for e in g["dense_nonzeros"]:
        dense[e["row"], e["k"]] = e["v"]
    return g, U.encode(dt, dense)


@pytest.mark.parametrize("dt", DTS)
def test_cbm_hand_worked_example(dt):
    key = "16-bit" if dt in ("f16", "bf16") else "8-bit"
    g = _golden("cbm_example.json")
    lay = g["layouts"][key]
    _, A = _cbm_golden_matrix(dt, lay["K"])
    M, K = g["M"], lay["K"]
    vals, meta, row_ptr, col, rvals = oracle.split(dt, A)
    # the split's residual is the hand-worked CSR
    assert list(row_ptr) == g["csr"]["row_ptr"] and list(col) == g["csr"]["col"]
    assert np.array_equal(U.to_f64(dt, rvals), np.array(g["csr"]["val"], dtype=np.float64))
    rmask, roff, cvals = oracle.cbm_encode(dt, meta, row_ptr, col, rvals, M, K)
    assert oracle.cbm_sizes(dt, M, K) == (lay["mask_bytes"], lay["blocks"])
    want = np.zeros(lay["mask_bytes"], dtype=np.uint8)
    for i, v in lay["rmask_nonzero"].items():
        want[int(i)] = v
    assert np.array_equal(rmask, want)
    assert list(roff) == lay["roff"]
    assert np.array_equal(U.to_f64(dt, cvals), np.array(lay["cvals"], dtype=np.float64))


def _cbm_shapes(dt):
    ks = 64 if dt in ("f16", "bf16") else 128
    return [(1, ks), (16, 2 * ks), (40, 4 * ks), (33, ks), (0, ks), (17, 0)]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("fam", FAMILIES)
def test_cbm_round_trip_and_invariants(dt, fam):
    ks = 64 if dt in ("f16", "bf16") else 128
    for M, K in _cbm_shapes(dt):
        A = U.random_matrix(dt, M, K, fam, seed=M * 7 + K) if M * K else np.zeros((M, K), U.store_dtype(dt))
        vals, meta, row_ptr, col, rvals = oracle.split(dt, A)
        rmask, roff, cvals = oracle.cbm_encode(dt, meta, row_ptr, col, rvals, M, K)
        nnz = int(row_ptr[-1]) if M else 0
        # closed-form sizes: ceil(M/16) * K/KS blocks of 64 lanes x (1 or 2) mask bytes
        blocks = (M + 15) // 16 * (K // ks)
        assert rmask.size == blocks * 64 * (1 if ks == 64 else 2) and roff.size == blocks + 1
        # one mask bit per residual entry; offsets an exclusive scan of the blocks' bits
        per_block = np.unpackbits(rmask).reshape(blocks, -1).sum(1) if blocks else np.zeros(0, np.int64)
        assert int(per_block.sum()) == nnz == int(roff[-1]) == cvals.size
        assert list(roff) == list(np.concatenate([[0], np.cumsum(per_block)]).astype(int))
        # decoding gives the split's CSR back, and with the 2:4 layer reproduces A's values
        rp2, col2, rv2 = oracle.cbm_decode(dt, meta, rmask, roff, cvals, M, K)
        assert np.array_equal(rp2, row_ptr) and np.array_equal(col2, col)
        assert np.array_equal(np.asarray(rv2).view(np.uint8), np.asarray(rvals).view(np.uint8))
        if M * K:
            D, _ = oracle.decompress(dt, vals, meta, K)
            Dv = U.to_f64(dt, D)
            Dv[np.repeat(np.arange(M), np.diff(rp2)), col2] += U.to_f64(dt, rv2)
            assert np.array_equal(Dv, U.to_f64(dt, A))


def test_cbm_bits_only_at_complement_positions():
    # brute force over every lane: a set bit names a non-kept position whose
    # dense value is non-zero, and every such position has its bit
    dt, M, K = "f16", 33, 128
    A = U.random_matrix(dt, M, K, "sparse", seed=5)
    vals, meta, row_ptr, col, rvals = oracle.split(dt, A)
    rmask, roff, cvals = oracle.cbm_encode(dt, meta, row_ptr, col, rvals, M, K)
    keep = U.brute_keep_mask(dt, A)
    nz = ~U.is_zero(dt, A)
    S = K // 64
    for b in range(rmask.size // 64):
        t, g = divmod(b, S)
        for lane in range(64):
            q, r = divmod(lane, 16)
            m = 16 * t + r
            word = int(rmask[b * 64 + lane])
            for gi in range(4):
                k0 = g * 64 + q * 16 + 4 * gi
                comp = [p for p in range(4) if m < M and not keep[m, k0 + p]] if m < M else [0, 1]
                for j in range(2):
                    bit = word >> (2 * gi + j) & 1
                    expect = m < M and bool(nz[m, k0 + comp[j]])
                    assert bit == expect, (b, lane, gi, j)


def test_cbm_rejects_an_entry_at_a_kept_position():
    dt, M, K = "f16", 2, 64
    A = np.zeros((M, K))
    A[0, :4] = [1, 2, 3, 4]                       # keeps positions 2 and 3
    vals, meta, row_ptr, col, rvals = oracle.split(dt, U.encode(dt, A))
    assert row_ptr[-1] == 2                        # the dropped 1 and 2 at columns 0 and 1
    one = U.encode(dt, [1.0])
    for kept in (2, 3):
        with pytest.raises(oracle.OracleError):
            oracle.cbm_encode(dt, meta, np.array([0, 1, 1], np.int32), np.array([kept], np.int32), one, M, K)
    # a complement position is accepted
    rmask, roff, cvals = oracle.cbm_encode(dt, meta, np.array([0, 1, 1], np.int32), np.array([1], np.int32), one,
                                           M, K)
    assert rmask[0] == 2 and list(roff) == [0, 1]
