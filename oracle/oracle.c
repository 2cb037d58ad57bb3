/*
 * oracle.c -- plain CPU reference for 2:4 compression and sparse x dense
 * matrix multiply.  TEST INFRASTRUCTURE ONLY (see oracle.h): the product
 * path never includes, links or calls this file.
 *
 * Every function is the plain definition written out: per-group top-2
 * selection by magnitude ([P3] "2:4 Fine-Grained Structured Sparsity" and the
 * first listing of "Python: Build a 2:4 Mask, Compress It ..."), bit-copied
 * values with 2-bit positions ([P3] worked example; [P2] "How Tensor Cores
 * Leverage This Pattern"), a residual that keeps what the selection dropped
 * ([P4] "How the three-layer format makes moderate sparsity fast"), and a
 * product computed by expanding to dense and summing over k in ascending
 * order in fp64 (int64 for int8).  No blocking, no reordering.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- element decoding, from the IEEE-754 binary16 and bfloat16 definitions ---- */

double orc_f16_to_f64(uint16_t bits) {
    /* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
    int sign = bits >> 15, e = (bits >> 10) & 0x1F, f = bits & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

double orc_bf16_to_f64(uint16_t bits) {
    /* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
    int sign = bits >> 15, e = (bits >> 7) & 0xFF, f = bits & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* subnormal: f * 2^-126 * 2^-7 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/2^7) * 2^(e-127) */
    return sign ? -v : v;
}

double orc_e4m3_to_f64(uint8_t bits) {
    /* E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; the
     * all-ones exponent is a normal binade except S.1111.111 = NaN. */
    int sign = bits >> 7, e = (bits >> 3) & 0xF, f = bits & 0x7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);                  /* subnormal: f * 2^-6 * 2^-3 */
    else
        v = ldexp((double)(8 + f), e - 10);        /* (1 + f/2^3) * 2^(e-7) */
    return sign ? -v : v;
}

double orc_e5m2_to_f64(uint8_t bits) {
    /* E5M2: 1 sign bit, 5 exponent bits (bias 15), 2 fraction bits, with
     * infinities and NaNs in the all-ones exponent as in IEEE-754. */
    int sign = bits >> 7, e = (bits >> 2) & 0x1F, f = bits & 0x3;
    double v;
    if (e == 31)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)f, -16);                 /* subnormal: f * 2^-14 * 2^-2 */
    else
        v = ldexp((double)(4 + f), e - 17);        /* (1 + f/2^2) * 2^(e-15) */
    return sign ? -v : v;
}

static int valid_dtype(int dt) {
    return dt == ORC_F16 || dt == ORC_BF16 || dt == ORC_I8 || dt == ORC_E4M3 || dt == ORC_E5M2;
}
static size_t esize(int dt) { return dt == ORC_F16 || dt == ORC_BF16 ? 2 : 1; }

/* 4-bit two's-complement integers, two per byte: element i is the low
 * nibble of byte i/2 for even i, the high nibble for odd i. */
static int i4_get(const void* base, int64_t i) {
    int nib = (((const uint8_t*)base)[i / 2] >> (4 * (i % 2))) & 0xF;
    return nib >= 8 ? nib - 16 : nib;
}
static void i4_set(void* base, int64_t i, int v) {
    uint8_t* b = (uint8_t*)base + i / 2;
    int sh = 4 * (int)(i % 2);
    *b = (uint8_t)((*b & ~(0xF << sh)) | ((v & 0xF) << sh));
}

double orc_i4_to_f64(uint8_t byte, int high) { return (double)i4_get(&byte, high ? 1 : 0); }

static double elem_f64(int dt, const void* base, int64_t i) {
    if (dt == ORC_I4) return (double)i4_get(base, i);
    if (dt == ORC_I8) return (double)((const int8_t*)base)[i];
    if (dt == ORC_E4M3) return orc_e4m3_to_f64(((const uint8_t*)base)[i]);
    if (dt == ORC_E5M2) return orc_e5m2_to_f64(((const uint8_t*)base)[i]);
    uint16_t u = ((const uint16_t*)base)[i];
    return dt == ORC_F16 ? orc_f16_to_f64(u) : orc_bf16_to_f64(u);
}

static int64_t elem_i64(const void* base, int64_t i) { return (int64_t)((const int8_t*)base)[i]; }

static void elem_copy(int dt, void* dst, int64_t di, const void* src, int64_t si) {
    if (dt == ORC_I4) { i4_set(dst, di, i4_get(src, si)); return; }
    size_t s = esize(dt);
    memcpy((char*)dst + (size_t)di * s, (const char*)src + (size_t)si * s, s);
}

static void elem_zero(int dt, void* dst, int64_t di) {
    if (dt == ORC_I4) { i4_set(dst, di, 0); return; }
    memset((char*)dst + (size_t)di * esize(dt), 0, esize(dt));
}

/* ---- selection ---- */

void orc_select_group(const double mag[4], int keep[4]) {
    for (int p = 0; p < 4; ++p) {
        int rank = 0;
        for (int q = 0; q < 4; ++q) {
            if (q == p) continue;
            if (mag[q] > mag[p] || (mag[q] == mag[p] && q < p)) ++rank;
        }
        keep[p] = rank < 2;
    }
}

/* Selection for group g of row m of A.  Returns 0, or ORC_ENONFINITE. */
static int group_keep(int dt, const void* A, int64_t lda, int64_t m, int64_t g, int keep[4]) {
    double mag[4];
    for (int p = 0; p < 4; ++p) {
        double x = elem_f64(dt, A, m * lda + 4 * g + p);
        if (!isfinite(x)) return ORC_ENONFINITE;
        mag[p] = fabs(x);                          /* int8: |-128| = 128 */
    }
    orc_select_group(mag, keep);
    return ORC_OK;
}

static int64_t meta_cols(int64_t K) { return (K + 7) / 8; }

static int check_a(int dt, int64_t M, int64_t K, const void* A, int64_t lda) {
    if (!valid_dtype(dt)) return ORC_EDTYPE;
    if (M < 0 || K < 0 || K % 4 != 0) return ORC_ESHAPE;
    if (M > 0 && K > 0 && !A) return ORC_ENULL;
    if (lda < K) return ORC_ESTRIDE;
    return ORC_OK;
}

/* Writes the 2:4 layer of row m. */
static int compress_row(int dt, int64_t K, const void* A, int64_t lda, int64_t m,
                        void* vals, int64_t ldv, uint8_t* meta, int64_t ldm) {
    for (int64_t j = 0; j < meta_cols(K); ++j) meta[m * ldm + j] = 0;
    for (int64_t g = 0; g < K / 4; ++g) {
        int keep[4], t = 0, pos[2] = {0, 0};
        int rc = group_keep(dt, A, lda, m, g, keep);
        if (rc) return rc;
        for (int p = 0; p < 4; ++p)
            if (keep[p]) pos[t++] = p;             /* ascending: pos[0] < pos[1] */
        elem_copy(dt, vals, m * ldv + 2 * g, A, m * lda + 4 * g + pos[0]);
        elem_copy(dt, vals, m * ldv + 2 * g + 1, A, m * lda + 4 * g + pos[1]);
        uint8_t nib = (uint8_t)(pos[0] | (pos[1] << 2));
        meta[m * ldm + g / 2] |= (uint8_t)(nib << (4 * (g % 2)));
    }
    return ORC_OK;
}

int orc_compress(int dt, int64_t M, int64_t K, const void* A, int64_t lda,
                 void* vals, int64_t ldv, uint8_t* meta, int64_t ldm) {
    int rc = check_a(dt, M, K, A, lda);
    if (rc) return rc;
    if (M > 0 && K > 0 && (!vals || !meta)) return ORC_ENULL;
    if (ldv < K / 2 || ldm < meta_cols(K)) return ORC_ESTRIDE;
    for (int64_t m = 0; m < M; ++m) {
        rc = compress_row(dt, K, A, lda, m, vals, ldv, meta, ldm);
        if (rc) return rc;
    }
    return ORC_OK;
}

int orc_prune(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* P, int64_t ldp) {
    int rc = check_a(dt, M, K, A, lda);
    if (rc) return rc;
    if (M > 0 && K > 0 && !P) return ORC_ENULL;
    if (ldp < K) return ORC_ESTRIDE;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < K / 4; ++g) {
            int keep[4];
            rc = group_keep(dt, A, lda, m, g, keep);
            if (rc) return rc;
            for (int p = 0; p < 4; ++p) {
                if (keep[p]) elem_copy(dt, P, m * ldp + 4 * g + p, A, m * lda + 4 * g + p);
                else elem_zero(dt, P, m * ldp + 4 * g + p);
            }
        }
    return ORC_OK;
}

/* Nibble of group g of row m; positions decoded into i0, i1.  Returns 1 if
 * the nibble names two distinct positions in ascending order. */
static int decode_nibble(const uint8_t* meta, int64_t ldm, int64_t m, int64_t g, int* i0, int* i1) {
    int nib = (meta[m * ldm + g / 2] >> (4 * (g % 2))) & 0xF;
    *i0 = nib & 3;
    *i1 = nib >> 2;
    return *i0 < *i1;
}

int64_t orc_decompress(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv,
                       const uint8_t* meta, int64_t ldm, void* D, int64_t ldd) {
    if (!valid_dtype(dt)) return ORC_EDTYPE;
    if (M < 0 || K < 0 || K % 4 != 0) return ORC_ESHAPE;
    if (M > 0 && K > 0 && (!vals || !meta || !D)) return ORC_ENULL;
    if (ldv < K / 2 || ldm < meta_cols(K) || ldd < K) return ORC_ESTRIDE;
    int64_t bad = 0;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < K / 4; ++g) {
            int i0, i1;
            for (int p = 0; p < 4; ++p) elem_zero(dt, D, m * ldd + 4 * g + p);
            if (!decode_nibble(meta, ldm, m, g, &i0, &i1)) { ++bad; continue; }
            elem_copy(dt, D, m * ldd + 4 * g + i0, vals, m * ldv + 2 * g);
            elem_copy(dt, D, m * ldd + 4 * g + i1, vals, m * ldv + 2 * g + 1);
        }
    return bad;
}

/* ---- residual split ---- */

/* Count (and optionally emit) the dropped non-zeros of row m, k ascending. */
static int row_overflow(int dt, int64_t K, const void* A, int64_t lda, int64_t m,
                        int64_t* count, int32_t* col, void* rvals, int64_t base) {
    int64_t c = 0;
    for (int64_t g = 0; g < K / 4; ++g) {
        int keep[4];
        int rc = group_keep(dt, A, lda, m, g, keep);
        if (rc) return rc;
        for (int p = 0; p < 4; ++p) {
            int64_t k = 4 * g + p;
            if (keep[p] || elem_f64(dt, A, m * lda + k) == 0.0) continue;   /* -0 counts as zero */
            if (col) {
                col[base + c] = (int32_t)k;
                elem_copy(dt, rvals, base + c, A, m * lda + k);
            }
            ++c;
        }
    }
    *count = c;
    return ORC_OK;
}

int orc_split_count(int dt, int64_t M, int64_t K, const void* A, int64_t lda, int32_t* row_ptr) {
    int rc = check_a(dt, M, K, A, lda);
    if (rc) return rc;
    if (!row_ptr) return ORC_ENULL;
    int64_t total = 0;
    row_ptr[0] = 0;
    for (int64_t m = 0; m < M; ++m) {
        int64_t c;
        rc = row_overflow(dt, K, A, lda, m, &c, NULL, NULL, 0);
        if (rc) return rc;
        total += c;
        if (total > INT32_MAX) return ORC_ERANGE;
        row_ptr[m + 1] = (int32_t)total;
    }
    return ORC_OK;
}

int orc_split_fill(int dt, int64_t M, int64_t K, const void* A, int64_t lda,
                   void* vals, int64_t ldv, uint8_t* meta, int64_t ldm,
                   const int32_t* row_ptr, int32_t* col, void* rvals) {
    int rc = orc_compress(dt, M, K, A, lda, vals, ldv, meta, ldm);
    if (rc) return rc;
    if (!row_ptr) return ORC_ENULL;
    if (M > 0 && row_ptr[M] > 0 && (!col || !rvals)) return ORC_ENULL;
    for (int64_t m = 0; m < M; ++m) {
        int64_t c;
        rc = row_overflow(dt, K, A, lda, m, &c, col, rvals, row_ptr[m]);
        if (rc) return rc;
        if (c != (int64_t)row_ptr[m + 1] - row_ptr[m]) return ORC_EFORMAT;
    }
    return ORC_OK;
}

/* ---- delta-coded residual ----
 * [P4] section "How the three-layer format makes moderate sparsity fast"
 * names a compact differential position code for the sparse layers, decoded
 * in parallel on chip, and gives no layout.  The layout here is this
 * library's own.  Per row, in CSR order, entry j stores its column as the
 * gap d_j = col_j - col_(j-1) in one byte, with col_(-1) = -1 (so the first
 * entry stores col_0 + 1).  A gap above 255 is bridged by filler entries,
 * d = 255 and value +0, placed before the entry, as many as leave its own d
 * in [1, 255].  Decoding is a running sum; a filler adds zero. */

/* Fillers in front of an entry whose gap from the previous column is gap >= 1. */
static int64_t fillers_for_gap(int64_t gap) { return (gap - 1) / 255; }

/* Columns of a CSR row must ascend strictly within [0, K). */
static int check_csr_row(int64_t K, const int32_t* col, int64_t lo, int64_t hi) {
    int64_t prev = -1;
    for (int64_t j = lo; j < hi; ++j) {
        if (col[j] <= prev || col[j] >= K) return ORC_EFORMAT;
        prev = col[j];
    }
    return ORC_OK;
}

static int check_csr(int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col) {
    if (M < 0 || K < 0) return ORC_ESHAPE;
    if (!row_ptr) return ORC_ENULL;
    if (row_ptr[0] != 0) return ORC_EFORMAT;
    for (int64_t m = 0; m < M; ++m)
        if (row_ptr[m + 1] < row_ptr[m]) return ORC_EFORMAT;
    if (M > 0 && row_ptr[M] > 0 && !col) return ORC_ENULL;
    for (int64_t m = 0; m < M; ++m) {
        int rc = check_csr_row(K, col, row_ptr[m], row_ptr[m + 1]);
        if (rc) return rc;
    }
    return ORC_OK;
}

int orc_delta_count(int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col, int32_t* drow_ptr) {
    int rc = check_csr(M, K, row_ptr, col);
    if (rc) return rc;
    if (!drow_ptr) return ORC_ENULL;
    int64_t total = 0;
    drow_ptr[0] = 0;
    for (int64_t m = 0; m < M; ++m) {
        int64_t prev = -1;
        for (int64_t j = row_ptr[m]; j < row_ptr[m + 1]; ++j) {
            total += 1 + fillers_for_gap((int64_t)col[j] - prev);
            prev = col[j];
        }
        if (total > INT32_MAX) return ORC_ERANGE;
        drow_ptr[m + 1] = (int32_t)total;
    }
    return ORC_OK;
}

int orc_delta_fill(int dt, int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col, const void* rvals,
                   const int32_t* drow_ptr, uint8_t* dcol, void* dvals) {
    if (!valid_dtype(dt)) return ORC_EDTYPE;
    int rc = check_csr(M, K, row_ptr, col);
    if (rc) return rc;
    if (!drow_ptr) return ORC_ENULL;
    if (M > 0 && row_ptr[M] > 0 && !rvals) return ORC_ENULL;
    if (M > 0 && drow_ptr[M] > 0 && (!dcol || !dvals)) return ORC_ENULL;
    for (int64_t m = 0; m < M; ++m) {
        int64_t pos = drow_ptr[m], prev = -1;
        for (int64_t j = row_ptr[m]; j < row_ptr[m + 1]; ++j) {
            int64_t gap = (int64_t)col[j] - prev;
            for (; gap > 255; gap -= 255) {
                if (pos >= drow_ptr[m + 1]) return ORC_EFORMAT;
                dcol[pos] = 255;
                elem_zero(dt, dvals, pos);
                ++pos;
            }
            if (pos >= drow_ptr[m + 1]) return ORC_EFORMAT;
            dcol[pos] = (uint8_t)gap;
            elem_copy(dt, dvals, pos, rvals, j);
            ++pos;
            prev = col[j];
        }
        if (pos != drow_ptr[m + 1]) return ORC_EFORMAT;
    }
    return ORC_OK;
}

/* ---- complement-bitmap residual, in the decode product's block order ----
 * [P4] section "How the three-layer format makes moderate sparsity fast"
 * keeps what the 2:4 layer drops in a residual layer, decoded in parallel on
 * chip, and gives no layout.  This layout is the library's own.  It rests
 * on one fact of the split: in a group where the 2:4 layer kept positions
 * i0 < i1, a residual entry can only sit at one of the other two positions,
 * c0 < c1 (the group's complement positions).  So one bit per complement
 * position says whether the residual holds a value there.
 *
 * Geometry: a k-step is KS dense columns (64 for 16-bit element types, 128
 * for 8-bit ones); tile t is rows [16t, 16t + 16); block b = t * S + g for
 * tile t and k-step g (T = ceil(M/16) tiles, S = K / KS k-steps).  Lane
 * l = 16q + r of block (t, g) is row 16t + r and dense columns
 * [g*KS + q*EB, g*KS + (q+1)*EB), EB = KS / 4: GL = EB / 4 groups (4 or 8).
 *   rmask: per block, 64 lanes x MB bytes (MB = GL / 4: 1 or 2), lane-major;
 *          a lane's MB bytes are one little-endian word whose bit 2*gi + j
 *          is set iff the residual has an entry at complement position c_j
 *          of the lane's group gi (groups in ascending column order).
 *          Rows past M have no bits.
 *   roff:  int32 [T*S + 1]; roff[b] = entries in blocks before b, roff[T*S]
 *          = all entries (an exclusive scan of the blocks' counts).
 *   cvals: the entries' values, bit-copied, in block order, then lane order,
 *          then bit order within the lane word.
 * The bytes: GL/4 mask bytes per 64 lanes of a block plus 4 per block plus
 * one value per entry, against the CSR's 4 + s per entry. */

static int cbm_geom(int dt, int64_t M, int64_t K, int64_t* T, int64_t* S, int* GL) {
    const int64_t KS = esize(dt) == 2 ? 64 : 128;
    if (M < 0 || K < 0 || K % KS != 0) return ORC_ESHAPE;
    *T = (M + 15) / 16;
    *S = K / KS;
    *GL = (int)(KS / 4 / 4);
    return ORC_OK;
}

int orc_cbm_sizes(int dt, int64_t M, int64_t K, int64_t* mask_bytes, int64_t* blocks) {
    if (!valid_dtype(dt) || dt == ORC_I4) return ORC_EDTYPE;
    if (!mask_bytes || !blocks) return ORC_ENULL;
    int64_t T, S;
    int GL;
    int rc = cbm_geom(dt, M, K, &T, &S, &GL);
    if (rc) return rc;
    *blocks = T * S;
    *mask_bytes = T * S * 64 * (GL / 4);
    return ORC_OK;
}

/* The complement positions c0 < c1 of a group whose kept pair is (i0, i1). */
static void complement_pair(int i0, int i1, int* c0, int* c1) {
    int n = 0, c[2] = {0, 0};
    for (int p = 0; p < 4; ++p)
        if (p != i0 && p != i1) c[n++] = p;
    *c0 = c[0];
    *c1 = c[1];
}

int orc_cbm_encode(int dt, int64_t M, int64_t K, const uint8_t* meta, int64_t ldm, const int32_t* row_ptr,
                   const int32_t* col, const void* rvals, uint8_t* rmask, int32_t* roff, void* cvals) {
    if (!valid_dtype(dt) || dt == ORC_I4) return ORC_EDTYPE;
    int64_t T, S;
    int GL;
    int rc = cbm_geom(dt, M, K, &T, &S, &GL);
    if (rc) return rc;
    rc = check_csr(M, K, row_ptr, col);
    if (rc) return rc;
    if (!roff || (T * S > 0 && !rmask)) return ORC_ENULL;
    if (M > 0 && K > 0 && (!meta || ldm < meta_cols(K))) return ORC_ENULL;
    const int64_t nnz = M > 0 ? row_ptr[M] : 0;
    if (nnz > 0 && (!rvals || !cvals)) return ORC_ENULL;
    const int MB = GL / 4, EB = 4 * GL;
    /* entry index of each column of the tile's 16 rows (-1: none) */
    int64_t* at = (int64_t*)malloc(sizeof(int64_t) * 16 * (size_t)(K > 0 ? K : 1));
    if (!at) return ORC_ENOMEM;
    int64_t out = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t i = 0; i < 16 * K; ++i) at[i] = -1;
        for (int r = 0; r < 16 && 16 * t + r < M; ++r)
            for (int64_t j = row_ptr[16 * t + r]; j < row_ptr[16 * t + r + 1]; ++j) at[r * K + col[j]] = j;
        for (int64_t g = 0; g < S; ++g) {
            const int64_t b = t * S + g;
            roff[b] = (int32_t)out;
            for (int l = 0; l < 64; ++l) {
                const int q = l / 16, r = l % 16;   /* lane l = 16q + r */
                const int64_t m = 16 * t + r, kb = g * 4 * EB + (int64_t)q * EB;
                uint32_t word = 0;
                if (m < M) {
                    for (int gi = 0; gi < GL; ++gi) {
                        int i0, i1, c[2];
                        if (!decode_nibble(meta, ldm, m, kb / 4 + gi, &i0, &i1)) { free(at); return ORC_EFORMAT; }
                        complement_pair(i0, i1, &c[0], &c[1]);
                        for (int j = 0; j < 2; ++j) {
                            const int64_t e = at[r * K + kb + 4 * gi + c[j]];
                            if (e < 0) continue;
                            word |= 1u << (2 * gi + j);
                            elem_copy(dt, cvals, out, rvals, e);
                            ++out;
                        }
                    }
                }
                for (int y = 0; y < MB; ++y) rmask[(b * 64 + l) * MB + y] = (uint8_t)(word >> (8 * y));
            }
        }
    }
    free(at);
    /* every entry must sit at a complement position (the split's residual does) */
    if (out != nnz) return ORC_EFORMAT;
    roff[T * S] = (int32_t)out;
    return ORC_OK;
}

int orc_cbm_decode(int dt, int64_t M, int64_t K, const uint8_t* meta, int64_t ldm, const uint8_t* rmask,
                   const int32_t* roff, const void* cvals, int32_t* row_ptr, int32_t* col, void* rvals) {
    if (!valid_dtype(dt) || dt == ORC_I4) return ORC_EDTYPE;
    int64_t T, S;
    int GL;
    int rc = cbm_geom(dt, M, K, &T, &S, &GL);
    if (rc) return rc;
    if (!roff || !row_ptr || (T * S > 0 && !rmask)) return ORC_ENULL;
    if (M > 0 && K > 0 && (!meta || ldm < meta_cols(K))) return ORC_ENULL;
    const int MB = GL / 4, EB = 4 * GL;
    /* pass 1: entries per row, and the block offsets checked against the bits */
    for (int64_t m = 0; m <= M; ++m) row_ptr[m] = 0;
    if (roff[0] != 0) return ORC_EFORMAT;
    for (int64_t b = 0; b < T * S; ++b) {
        int64_t n = 0;
        for (int l = 0; l < 64; ++l) {
            uint32_t word = 0;
            for (int y = 0; y < MB; ++y) word |= (uint32_t)rmask[(b * 64 + l) * MB + y] << (8 * y);
            const int64_t m = 16 * (b / S) + l % 16;
            for (int bit = 0; bit < 2 * GL; ++bit)
                if (word >> bit & 1u) {
                    if (m >= M) return ORC_EFORMAT;
                    ++row_ptr[m + 1];
                    ++n;
                }
        }
        if ((int64_t)roff[b + 1] - roff[b] != n) return ORC_EFORMAT;
    }
    for (int64_t m = 0; m < M; ++m) row_ptr[m + 1] += row_ptr[m];
    const int64_t nnz = M > 0 ? row_ptr[M] : 0;
    if (nnz > 0 && (!col || !rvals || !cvals)) return ORC_ENULL;
    /* pass 2: for a fixed row the block, lane and bit order visits columns in
     * ascending order, so each row is filled front to back */
    int64_t* cur = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    if (!cur) return ORC_ENOMEM;
    for (int64_t m = 0; m < M; ++m) cur[m] = row_ptr[m];
    int64_t in = 0;
    for (int64_t b = 0; b < T * S; ++b) {
        const int64_t t = b / S, g = b % S;
        for (int l = 0; l < 64; ++l) {
            const int q = l / 16, r = l % 16;
            const int64_t m = 16 * t + r, kb = g * 4 * EB + (int64_t)q * EB;
            uint32_t word = 0;
            for (int y = 0; y < MB; ++y) word |= (uint32_t)rmask[(b * 64 + l) * MB + y] << (8 * y);
            if (!word) continue;
            for (int gi = 0; gi < GL; ++gi) {
                int i0, i1, c[2];
                if (!decode_nibble(meta, ldm, m, kb / 4 + gi, &i0, &i1)) { free(cur); return ORC_EFORMAT; }
                complement_pair(i0, i1, &c[0], &c[1]);
                for (int j = 0; j < 2; ++j)
                    if (word >> (2 * gi + j) & 1u) {
                        col[cur[m]] = (int32_t)(kb + 4 * gi + c[j]);
                        elem_copy(dt, rvals, cur[m], cvals, in);
                        ++cur[m];
                        ++in;
                    }
            }
        }
    }
    free(cur);
    return ORC_OK;
}

/* ---- sparse x dense product ---- */

static int check_mm(int dt, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                    const uint8_t* meta, int64_t ldm, const void* B, int64_t ldb, int64_t ldc,
                    const double* Cf, const int64_t* Ci) {
    if (!valid_dtype(dt)) return ORC_EDTYPE;
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0) return ORC_ESHAPE;
    if (M > 0 && K > 0 && (!vals || !meta)) return ORC_ENULL;
    if (K > 0 && N > 0 && !B) return ORC_ENULL;
    if (M > 0 && N > 0 && (dt == ORC_I8 ? !Ci : !Cf)) return ORC_ENULL;
    if (ldv < K / 2 || ldm < meta_cols(K) || ldb < N || ldc < N) return ORC_ESTRIDE;
    return ORC_OK;
}

/* Dense row m of decompress(vals, meta) [+ residual], as fp64 and int64.
 * Returns ORC_EFORMAT on a bad nibble. */
static int dense_row(int dt, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                     const int32_t* row_ptr, const int32_t* col, const uint8_t* dcol, const void* rvals,
                     int64_t m, double* rowf, int64_t* rowi) {
    for (int64_t k = 0; k < K; ++k) { rowf[k] = 0.0; rowi[k] = 0; }
    for (int64_t g = 0; g < K / 4; ++g) {
        int i0, i1;
        if (!decode_nibble(meta, ldm, m, g, &i0, &i1)) return ORC_EFORMAT;
        int64_t v0 = m * ldv + 2 * g, v1 = v0 + 1;
        rowf[4 * g + i0] = elem_f64(dt, vals, v0);
        rowf[4 * g + i1] = elem_f64(dt, vals, v1);
        if (dt == ORC_I8) { rowi[4 * g + i0] = elem_i64(vals, v0); rowi[4 * g + i1] = elem_i64(vals, v1); }
    }
    if (row_ptr) {
        int64_t k = -1;                            /* delta-coded: column before the row's first entry */
        for (int64_t j = row_ptr[m]; j < row_ptr[m + 1]; ++j) {
            if (dcol) k += dcol[j];
            else k = col[j];
            if (k < 0 || k >= K) return ORC_EFORMAT;
            rowf[k] += elem_f64(dt, rvals, j);
            if (dt == ORC_I8) rowi[k] += elem_i64(rvals, j);
        }
    }
    return ORC_OK;
}

static int spmm_impl(int dt, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                     const uint8_t* meta, int64_t ldm, const int32_t* row_ptr, const int32_t* col,
                     const uint8_t* dcol, const void* rvals, const void* B, int64_t ldb, double* Cf,
                     int64_t* Ci, double* S, int64_t ldc) {
    int rc = check_mm(dt, M, N, K, vals, ldv, meta, ldm, B, ldb, ldc, Cf, Ci);
    if (rc) return rc;
    if (row_ptr && M > 0 && row_ptr[M] > 0 && ((!col && !dcol) || !rvals)) return ORC_ENULL;
    if (M == 0 || N == 0) return ORC_OK;
    /* B converted once, stored column by column so each output walks one
     * contiguous column; the sum order over k is unchanged. */
    double* bt = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (size_t)N);
    int64_t* bti = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1) * (size_t)N);
    if (!bt || !bti) { free(bt); free(bti); return ORC_ENOMEM; }
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) {
            bt[n * K + k] = elem_f64(dt, B, k * ldb + n);
            bti[n * K + k] = dt == ORC_I8 ? elem_i64(B, k * ldb + n) : 0;
        }
    int err = ORC_OK;
#pragma omp parallel
    {
        double* rowf = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        int64_t* rowi = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
        if (!rowf || !rowi) {
#pragma omp critical
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            if (!rowf || !rowi) continue;
            int r = dense_row(dt, K, vals, ldv, meta, ldm, row_ptr, col, dcol, rvals, m, rowf, rowi);
            if (r) {
#pragma omp critical
                err = r;
                continue;
            }
            for (int64_t n = 0; n < N; ++n) {
                if (dt == ORC_I8) {
                    int64_t acc = 0;
                    for (int64_t k = 0; k < K; ++k) acc += rowi[k] * bti[n * K + k];
                    Ci[m * ldc + n] = acc;
                } else {
                    double acc = 0.0, s = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        double t = rowf[k] * bt[n * K + k];
                        acc += t;
                        s += fabs(t);
                    }
                    Cf[m * ldc + n] = acc;
                    if (S) S[m * ldc + n] = s;
                }
            }
        }
        free(rowf);
        free(rowi);
    }
    free(bt);
    free(bti);
    return err;
}

int orc_spmm(int dt, int64_t M, int64_t N, int64_t K,
             const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
             const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S, int64_t ldc) {
    return spmm_impl(dt, M, N, K, vals, ldv, meta, ldm, NULL, NULL, NULL, NULL, B, ldb, Cf, Ci, S, ldc);
}

int orc_spmm_residual(int dt, int64_t M, int64_t N, int64_t K,
                      const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                      const int32_t* row_ptr, const int32_t* col, const void* rvals,
                      const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S, int64_t ldc) {
    if (!row_ptr) return ORC_ENULL;
    return spmm_impl(dt, M, N, K, vals, ldv, meta, ldm, row_ptr, col, NULL, rvals, B, ldb, Cf, Ci, S, ldc);
}

int orc_spmm_residual_delta(int dt, int64_t M, int64_t N, int64_t K,
                            const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                            const int32_t* drow_ptr, const uint8_t* dcol, const void* dvals,
                            const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S, int64_t ldc) {
    if (!drow_ptr) return ORC_ENULL;
    return spmm_impl(dt, M, N, K, vals, ldv, meta, ldm, drow_ptr, NULL, dcol, dvals, B, ldb, Cf, Ci, S, ldc);
}

static int entries_impl(int dt, int64_t M, int64_t N, int64_t K,
                        const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                        const int32_t* row_ptr, const int32_t* col, const uint8_t* dcol, const void* rvals,
                        const void* B, int64_t ldb, int64_t n_entries,
                        const int64_t* ms, const int64_t* ns, double* Cf, int64_t* Ci, double* S) {
    int rc = check_mm(dt, M, N, K, vals, ldv, meta, ldm, B, ldb, N, Cf, Ci);
    if (rc) return rc;
    if (n_entries < 0) return ORC_ESHAPE;
    if (n_entries > 0 && (!ms || !ns || (dt == ORC_I8 ? !Ci : !Cf))) return ORC_ENULL;
    double* rowf = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    int64_t* rowi = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
    if (!rowf || !rowi) { free(rowf); free(rowi); return ORC_ENOMEM; }
    for (int64_t e = 0; e < n_entries && rc == ORC_OK; ++e) {
        int64_t m = ms[e], n = ns[e];
        if (m < 0 || m >= M || n < 0 || n >= N) { rc = ORC_ERANGE; break; }
        rc = dense_row(dt, K, vals, ldv, meta, ldm, row_ptr, col, dcol, rvals, m, rowf, rowi);
        if (rc) break;
        if (dt == ORC_I8) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) acc += rowi[k] * elem_i64(B, k * ldb + n);
            Ci[e] = acc;
        } else {
            double acc = 0.0, s = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = rowf[k] * elem_f64(dt, B, k * ldb + n);
                acc += t;
                s += fabs(t);
            }
            Cf[e] = acc;
            if (S) S[e] = s;
        }
    }
    free(rowf);
    free(rowi);
    return rc;
}

/* ---- unstructured sparse x dense product ----
 * [P3] sections "Why Hardware Wants Dense, Regular Data" and "The Honest
 * Numbers on Unstructured Sparsity" set the unstructured baseline the 2:4
 * format is weighed against: a sparse matrix stored as its non-zeros with
 * their column indices.  C[m,n] = sum over the row's entries j, in CSR
 * order, of vals[j] * B[col[j], n] (fp64 / int64), with the bound S. */
int orc_spmm_csr(int dt, int64_t M, int64_t N, int64_t K, const int32_t* row_ptr, const int32_t* col,
                 const void* vals, const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S, int64_t ldc) {
    if (!valid_dtype(dt)) return ORC_EDTYPE;
    if (M < 0 || N < 0 || K < 0) return ORC_ESHAPE;
    if (!row_ptr) return ORC_ENULL;
    if (M > 0 && row_ptr[M] > 0 && (!col || !vals)) return ORC_ENULL;
    if (K > 0 && N > 0 && !B) return ORC_ENULL;
    if (M > 0 && N > 0 && (dt == ORC_I8 ? !Ci : !Cf)) return ORC_ENULL;
    if (ldb < N || ldc < N) return ORC_ESTRIDE;
    for (int64_t m = 0; m < M; ++m)
        if (row_ptr[m + 1] < row_ptr[m]) return ORC_EFORMAT;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, s = 0.0;
            int64_t acci = 0;
            for (int64_t j = row_ptr[m]; j < row_ptr[m + 1]; ++j) {
                int64_t k = col[j];
                if (k < 0 || k >= K) return ORC_EFORMAT;
                if (dt == ORC_I8) {
                    acci += elem_i64(vals, j) * elem_i64(B, k * ldb + n);
                } else {
                    double t = elem_f64(dt, vals, j) * elem_f64(dt, B, k * ldb + n);
                    acc += t;
                    s += fabs(t);
                }
            }
            if (dt == ORC_I8) Ci[m * ldc + n] = acci;
            else {
                Cf[m * ldc + n] = acc;
                if (S) S[m * ldc + n] = s;
            }
        }
    }
    return ORC_OK;
}

int orc_spmm_entries(int dt, int64_t M, int64_t N, int64_t K,
                     const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                     const int32_t* row_ptr, const int32_t* col, const void* rvals,
                     const void* B, int64_t ldb, int64_t n_entries,
                     const int64_t* ms, const int64_t* ns, double* Cf, int64_t* Ci, double* S) {
    return entries_impl(dt, M, N, K, vals, ldv, meta, ldm, row_ptr, col, NULL, rvals, B, ldb, n_entries, ms, ns,
                        Cf, Ci, S);
}

int orc_spmm_entries_delta(int dt, int64_t M, int64_t N, int64_t K,
                           const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                           const int32_t* drow_ptr, const uint8_t* dcol, const void* dvals,
                           const void* B, int64_t ldb, int64_t n_entries,
                           const int64_t* ms, const int64_t* ns, double* Cf, int64_t* Ci, double* S) {
    return entries_impl(dt, M, N, K, vals, ldv, meta, ldm, drow_ptr, NULL, dcol, dvals, B, ldb, n_entries, ms, ns,
                        Cf, Ci, S);
}

/* ---- N:M generalization ----
 * [P3] section "Block Sparsity, N:M Generalizations, and Channel Pruning"
 * lists N:M patterns other than 2:4 (1:4, 2:8, 4:8) and gives no selection
 * rule or storage.  Reading taken here: the 2:4 rule widened, i.e. each group
 * of nm_m consecutive elements along K keeps its nm_n largest magnitudes
 * (ties to the lower position); the kept values are stored in ascending
 * position order, nm_n per group, and the kept positions as one bit per
 * dense element (bit k % 8 of byte k / 8 of the row's mask, set iff element k
 * is kept).  The product expands a row to dense and sums over k ascending,
 * as for 2:4. */

static int nm_ok(int nm_n, int nm_m) { return nm_m >= 2 && nm_m <= 16 && nm_n >= 1 && nm_n < nm_m; }

void orc_select_nm(int nm_n, int nm_m, const double* mag, int* keep) {
    for (int p = 0; p < nm_m; ++p) {
        int rank = 0;
        for (int q = 0; q < nm_m; ++q) {
            if (q == p) continue;
            if (mag[q] > mag[p] || (mag[q] == mag[p] && q < p)) ++rank;
        }
        keep[p] = rank < nm_n;
    }
}

static int check_nm_shape(int dt, int nm_n, int nm_m, int64_t M, int64_t K) {
    if (!valid_dtype(dt) && dt != ORC_I4) return ORC_EDTYPE;
    if (dt == ORC_I4 && K % 2 != 0) return ORC_ESHAPE;
    if (!nm_ok(nm_n, nm_m) || M < 0 || K < 0 || K % nm_m != 0) return ORC_ESHAPE;
    return ORC_OK;
}

int orc_compress_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* A, int64_t lda,
                    void* vals, int64_t ldv, uint8_t* mask, int64_t ldmask) {
    int rc = check_nm_shape(dt, nm_n, nm_m, M, K);
    if (rc) return rc;
    if (M > 0 && K > 0 && (!A || !vals || !mask)) return ORC_ENULL;
    if (lda < K || ldv < K / nm_m * nm_n || ldmask < meta_cols(K)) return ORC_ESTRIDE;
    if (dt == ORC_I4 && (lda % 2 || ldv % 2)) return ORC_ESTRIDE;   /* rows start on whole bytes */
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < meta_cols(K); ++j) mask[m * ldmask + j] = 0;
        for (int64_t g = 0; g < K / nm_m; ++g) {
            double mag[16];
            int keep[16], t = 0;
            for (int p = 0; p < nm_m; ++p) {
                double x = elem_f64(dt, A, m * lda + g * nm_m + p);
                if (!isfinite(x)) return ORC_ENONFINITE;
                mag[p] = fabs(x);
            }
            orc_select_nm(nm_n, nm_m, mag, keep);
            for (int p = 0; p < nm_m; ++p) {
                if (!keep[p]) continue;
                int64_t k = g * nm_m + p;
                elem_copy(dt, vals, m * ldv + g * nm_n + t++, A, m * lda + k);
                mask[m * ldmask + k / 8] |= (uint8_t)(1u << (k % 8));
            }
        }
    }
    return ORC_OK;
}

static int mask_bit(const uint8_t* mask, int64_t ldmask, int64_t m, int64_t k) {
    return (mask[m * ldmask + k / 8] >> (k % 8)) & 1;
}

/* Dense row m of the N:M operand.  Returns 1 if every group has exactly
 * nm_n mask bits; a group that has not is left zero. */
static int64_t nm_row(int dt, int nm_n, int nm_m, int64_t K, const void* vals, int64_t ldv,
                      const uint8_t* mask, int64_t ldmask, int64_t m, double* rowf, int64_t* rowi,
                      void* D, int64_t ldd) {
    int64_t bad = 0;
    for (int64_t k = 0; k < K; ++k) {
        if (rowf) { rowf[k] = 0.0; rowi[k] = 0; }
        if (D) elem_zero(dt, D, m * ldd + k);
    }
    for (int64_t g = 0; g < K / nm_m; ++g) {
        int cnt = 0;
        for (int p = 0; p < nm_m; ++p) cnt += mask_bit(mask, ldmask, m, g * nm_m + p);
        if (cnt != nm_n) { ++bad; continue; }
        int t = 0;
        for (int p = 0; p < nm_m; ++p) {
            int64_t k = g * nm_m + p;
            if (!mask_bit(mask, ldmask, m, k)) continue;
            int64_t v = m * ldv + g * nm_n + t++;
            if (rowf) {
                rowf[k] = elem_f64(dt, vals, v);
                if (dt == ORC_I8) rowi[k] = elem_i64(vals, v);
            }
            if (D) elem_copy(dt, D, m * ldd + k, vals, v);
        }
    }
    return bad;
}

int64_t orc_decompress_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                          const uint8_t* mask, int64_t ldmask, void* D, int64_t ldd) {
    int rc = check_nm_shape(dt, nm_n, nm_m, M, K);
    if (rc) return rc;
    if (M > 0 && K > 0 && (!vals || !mask || !D)) return ORC_ENULL;
    if (ldv < K / nm_m * nm_n || ldmask < meta_cols(K) || ldd < K) return ORC_ESTRIDE;
    if (dt == ORC_I4 && (ldv % 2 || ldd % 2)) return ORC_ESTRIDE;
    int64_t bad = 0;
    for (int64_t m = 0; m < M; ++m) bad += nm_row(dt, nm_n, nm_m, K, vals, ldv, mask, ldmask, m, NULL, NULL, D, ldd);
    return bad;
}

/* adt: element type of the N:M operand; bdt: that of B (the same, or fp16
 * for 4-bit weights).  int8 x int8 sums in int64, everything else in fp64. */
static int spmm_nm_impl(int dt, int bdt, int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* vals,
                        int64_t ldv, const uint8_t* mask, int64_t ldmask, const void* B, int64_t ldb, double* Cf,
                        int64_t* Ci, double* S, int64_t ldc) {
    int rc = check_nm_shape(dt, nm_n, nm_m, M, K);
    if (rc) return rc;
    if (dt == ORC_I4 && ldv % 2) return ORC_ESTRIDE;
    if (N < 0) return ORC_ESHAPE;
    if (M > 0 && K > 0 && (!vals || !mask)) return ORC_ENULL;
    if (K > 0 && N > 0 && !B) return ORC_ENULL;
    if (M > 0 && N > 0 && (dt == ORC_I8 ? !Ci : !Cf)) return ORC_ENULL;
    if (ldv < K / nm_m * nm_n || ldmask < meta_cols(K) || ldb < N || ldc < N) return ORC_ESTRIDE;
    if (M == 0 || N == 0) return ORC_OK;
    int err = ORC_OK;
#pragma omp parallel
    {
        double* rowf = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        int64_t* rowi = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
        if (!rowf || !rowi) {
#pragma omp critical
            err = ORC_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t m = 0; m < M; ++m) {
            if (!rowf || !rowi) continue;
            if (nm_row(dt, nm_n, nm_m, K, vals, ldv, mask, ldmask, m, rowf, rowi, NULL, 0)) {
#pragma omp critical
                err = ORC_EFORMAT;
                continue;
            }
            for (int64_t n = 0; n < N; ++n) {
                if (dt == ORC_I8) {
                    int64_t acc = 0;
                    for (int64_t k = 0; k < K; ++k) acc += rowi[k] * elem_i64(B, k * ldb + n);
                    Ci[m * ldc + n] = acc;
                } else {
                    double acc = 0.0, s = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        double t = rowf[k] * elem_f64(bdt, B, k * ldb + n);
                        acc += t;
                        s += fabs(t);
                    }
                    Cf[m * ldc + n] = acc;
                    if (S) S[m * ldc + n] = s;
                }
            }
        }
        free(rowf);
        free(rowi);
    }
    return err;
}

int orc_spmm_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                const uint8_t* mask, int64_t ldmask, const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S,
                int64_t ldc) {
    if (dt == ORC_I4) return ORC_EDTYPE;                  /* 4-bit weights take fp16 B: orc_spmm_nm_w4a16 */
    return spmm_nm_impl(dt, dt, nm_n, nm_m, M, N, K, vals, ldv, mask, ldmask, B, ldb, Cf, Ci, S, ldc);
}

int orc_spmm_nm_w4a16(int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                      const uint8_t* mask, int64_t ldmask, const void* B, int64_t ldb, double* Cf, double* S,
                      int64_t ldc) {
    return spmm_nm_impl(ORC_I4, ORC_F16, nm_n, nm_m, M, N, K, vals, ldv, mask, ldmask, B, ldb, Cf, NULL, S, ldc);
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops use from now on (n >= 1); for timing the
 * oracle on one core as well as on all of them. */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
