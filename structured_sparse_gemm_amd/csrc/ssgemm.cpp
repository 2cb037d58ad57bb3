// ssgemm.cpp -- the C ABI of libssgemm (include/ssgemm.h): host-side
// argument validation, alignment checks and kernel dispatch.  Nothing here
// allocates device memory.  The mutable state is the per-thread text of the
// last error and, for the entry point that allocates nothing, the device
// address of its file-scope scratch array on each device it has run on.
#include "ssgemm.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "ssg_kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SSG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool in_dtype(int dt) {
    return dt == SSG_F16 || dt == SSG_BF16 || dt == SSG_I8 || dt == SSG_E4M3 || dt == SSG_E5M2;
}
int64_t esize(int dt) { return dt == SSG_F16 || dt == SSG_BF16 ? 2 : 1; }

// The (input, output) type pairs of the products: 16-bit and 8-bit floats
// accumulate into fp32, int8 into int32.
bool pair_ok(int ab, int c) {
    return (ab == SSG_I8 && c == SSG_I32) || (ab != SSG_I8 && in_dtype(ab) && c == SSG_F32);
}
bool al(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A row chunk of 32 elements is 16-byte aligned when the base is and the
// row stride is a multiple of 16 bytes.
bool rows_aligned16(const void* p, int64_t ld, int dt) { return al(p, 16) && (ld * esize(dt)) % 16 == 0; }

int check_dense(int dt, int64_t M, int64_t K, const void* A, int64_t lda) {
    if (!in_dtype(dt)) return fail(SSG_ERR_DTYPE, "element type %d is not SSG_F16, SSG_BF16, SSG_I8, SSG_E4M3 or SSG_E5M2", dt);
    if (M < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (K % 4 != 0) return fail(SSG_ERR_SHAPE, "K=%lld is not a multiple of 4", (long long)K);
    // thread count of the chunked kernels must fit a 1-D grid
    if ((M * ((K + 31) / 32)) / 256 >= (int64_t)1 << 31)
        return fail(SSG_ERR_SHAPE, "M*K too large (%lld x %lld)", (long long)M, (long long)K);
    if (M > 0 && K > 0 && !A) return fail(SSG_ERR_NULL, "A is NULL");
    if (lda < K) return fail(SSG_ERR_STRIDE, "lda=%lld < K=%lld", (long long)lda, (long long)K);
    return SSG_OK;
}

int check_compressed(int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                     bool need) {
    if (need && M > 0 && K > 0 && (!vals || !meta)) return fail(SSG_ERR_NULL, "vals or meta is NULL");
    if (ldv < K / 2) return fail(SSG_ERR_STRIDE, "ldv=%lld < K/2=%lld", (long long)ldv, (long long)(K / 2));
    if (ldm < (K + 7) / 8) return fail(SSG_ERR_STRIDE, "ldm=%lld < ceil(K/8)=%lld", (long long)ldm, (long long)((K + 7) / 8));
    return SSG_OK;
}

bool vec_compressed(int dt, const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm) {
    return rows_aligned16(vals, ldv, dt) && al(meta, 4) && ldm % 4 == 0;
}

int to_dt(int dt) {
    switch (dt) {
        case SSG_F16: return ssg::DT_F16;
        case SSG_BF16: return ssg::DT_BF16;
        case SSG_E4M3: return ssg::DT_E4M3;
        case SSG_E5M2: return ssg::DT_E5M2;
        case SSG_I4: return ssg::DT_I4;
        default: return ssg::DT_I8;
    }
}

int check_spmm(int ab, int c, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
               int64_t ldm, const void* B, int64_t ldb, const void* C, int64_t ldc) {
    if (!pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    if (M < 0 || N < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size");
    if (K % 4 != 0) return fail(SSG_ERR_SHAPE, "K=%lld is not a multiple of 4", (long long)K);
    if (N > ((int64_t)1 << 31) || M > ((int64_t)1 << 40)) return fail(SSG_ERR_SHAPE, "size too large");
    int rc = check_compressed(M, K, vals, ldv, meta, ldm, true);
    if (rc) return rc;
    if (K > 0 && N > 0 && !B) return fail(SSG_ERR_NULL, "B is NULL");
    if (M > 0 && N > 0 && !C) return fail(SSG_ERR_NULL, "C is NULL");
    if (ldb < N) return fail(SSG_ERR_STRIDE, "ldb=%lld < N=%lld", (long long)ldb, (long long)N);
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    return SSG_OK;
}

int pick_algo(const ssg::SpmmArgs& a) {
    if (a.K > 0 && ssg::supported_small_n(a)) return SSG_ALGO_SMALL_N;
    if (a.K > 0 && ssg::supported_large_n(a)) return SSG_ALGO_LARGE_N;
    return SSG_ALGO_GENERIC;
}

// Workspace of a product with 0 < N < 16: B padded to 16 columns, which lets
// the decode kernels that take B as one contiguous K x 16 block run.  Zero
// where that copy could not be addressed with 31-bit offsets.
int64_t padded_b_bytes(int ab, int64_t N, int64_t K) {
    if (!(N > 0 && N < 16 && K > 0) || K * 16 * esize(ab) >= 0x7fffffff) return 0;
    return (K * 16 * esize(ab) + 255) / 256 * 256;
}

// Workspace bytes this call will use: the padded copy of B, when algorithm
// `algo` takes the padded decode path for this problem (AUTO or SMALL_N, and
// the small-N kernel accepts the problem with a padded B); else 0.
int64_t pad_need(int algo, const ssg::SpmmArgs& a) {
    if (algo != SSG_ALGO_AUTO && algo != SSG_ALGO_SMALL_N) return 0;
    const int64_t bytes = padded_b_bytes(a.dt == ssg::DT_F16 || a.dt == ssg::DT_BF16 ? SSG_F16 : SSG_I8, a.N, a.K);
    if (bytes == 0 || a.M <= 0) return 0;
    ssg::SpmmArgs p = a;
    p.B = reinterpret_cast<const void*>(uintptr_t(256));   // stands for any 16-byte aligned workspace (not read)
    p.ldb = 16;
    p.b_pad16 = 1;
    return ssg::supported_small_n(p) ? bytes : 0;
}

int check_workspace(int64_t need, const void* ws, size_t ws_bytes) {
    if (need == 0) return SSG_OK;
    if (!ws || (int64_t)ws_bytes < need)
        return fail(SSG_ERR_WORKSPACE, "workspace %zu < %lld bytes", ws ? ws_bytes : (size_t)0, (long long)need);
    if (!al(ws, 16)) return fail(SSG_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    return SSG_OK;
}

// Runs the product; the caller has validated the arguments and the workspace
// against pad_need(algo, a).
int run_spmm(int algo, ssg::SpmmArgs a, hipStream_t s, void* ws) {
    if (a.M == 0 || a.N == 0) return SSG_OK;
    // B narrower than 16 columns: padded into the workspace for the decode kernels
    if (pad_need(algo, a) > 0) {
        hipError_t e = ssg::launch_pad_b(a.dt, a.K, a.N, a.B, a.ldb, ws, s);
        if (e != hipSuccess) return hip_fail(e, "B padding launch");
        a.B = ws;
        a.ldb = 16;
        a.b_pad16 = 1;
    }
    if (algo == SSG_ALGO_AUTO) algo = pick_algo(a);
    hipError_t e = hipSuccess;
    switch (algo) {
        case SSG_ALGO_GENERIC:
            e = ssg::launch_spmm_generic(a, s);
            break;
        case SSG_ALGO_SMALL_N:
            if (a.K == 0 || !ssg::supported_small_n(a))
                return fail(SSG_ERR_ALGO, "the small-N kernel does not take this problem (N=%lld, alignment)",
                            (long long)a.N);
            e = ssg::launch_spmm_small_n(a, s);
            break;
        case SSG_ALGO_LARGE_N:
            if (a.K == 0 || !ssg::supported_large_n(a))
                return fail(SSG_ERR_ALGO, "the large-N kernel does not take this problem (shape, alignment)");
            e = ssg::launch_spmm_large_n(a, s);
            // the large-N tiles cover the 2:4 layer; the residual is a second pass
            if (e == hipSuccess && a.row_ptr) e = ssg::launch_residual_add(a, s);
            break;
        default:
            return fail(SSG_ERR_ALGO, "unknown algorithm %d", algo);
    }
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return SSG_OK;
}

ssg::SpmmArgs make_args(int ab, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                        const uint8_t* meta, int64_t ldm, const void* B, int64_t ldb, void* C, int64_t ldc) {
    ssg::SpmmArgs a{};
    a.dt = to_dt(ab);
    a.M = M; a.N = N; a.K = K;
    a.vals = vals; a.ldv = ldv; a.meta = meta; a.ldm = ldm;
    a.row_ptr = nullptr; a.col = nullptr; a.dcol = nullptr; a.rvals = nullptr; a.nnz_r = 0;
    a.B = B; a.ldb = ldb; a.C = C; a.ldc = ldc;
    return a;
}

}  // namespace

extern "C" {

int ssg_abi_version(void) { return SSG_ABI_VERSION; }

const char* ssg_status_str(int status) {
    switch (status) {
        case SSG_OK: return "SSG_OK";
        case SSG_ERR_NULL: return "SSG_ERR_NULL: a required pointer is NULL";
        case SSG_ERR_SHAPE: return "SSG_ERR_SHAPE: invalid or unsupported size";
        case SSG_ERR_STRIDE: return "SSG_ERR_STRIDE: leading dimension smaller than the row";
        case SSG_ERR_DTYPE: return "SSG_ERR_DTYPE: unsupported element type";
        case SSG_ERR_FORMAT: return "SSG_ERR_FORMAT: inconsistent sparse operand";
        case SSG_ERR_WORKSPACE: return "SSG_ERR_WORKSPACE: workspace too small";
        case SSG_ERR_HIP: return "SSG_ERR_HIP: HIP runtime error";
        case SSG_ERR_ALGO: return "SSG_ERR_ALGO: algorithm cannot run this problem";
        default: return "unknown ssg_status";
    }
}

const char* ssg_last_error(void) { return g_last_error.c_str(); }

int64_t ssg_vals_cols(int64_t K) { return K / 2; }
int64_t ssg_meta_cols(int64_t K) { return (K + 7) / 8; }

int ssg_prune_2to4(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* P, int64_t ldp, void* stream) {
    int rc = check_dense(dt, M, K, A, lda);
    if (rc) return rc;
    if (M > 0 && K > 0 && !P) return fail(SSG_ERR_NULL, "P is NULL");
    if (ldp < K) return fail(SSG_ERR_STRIDE, "ldp=%lld < K=%lld", (long long)ldp, (long long)K);
    if (P == A && ldp != lda) return fail(SSG_ERR_STRIDE, "in-place prune needs ldp == lda");
    const bool vec = rows_aligned16(A, lda, dt) && rows_aligned16(P, ldp, dt);
    hipError_t e = ssg::launch_prune(to_dt(dt), M, K, A, lda, P, ldp, vec, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "prune launch");
}

int ssg_compress_2to4(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* vals, int64_t ldv,
                      uint8_t* meta, int64_t ldm, void* stream) {
    int rc = check_dense(dt, M, K, A, lda);
    if (rc) return rc;
    rc = check_compressed(M, K, vals, ldv, meta, ldm, true);
    if (rc) return rc;
    const bool vec = rows_aligned16(A, lda, dt) && vec_compressed(dt, vals, ldv, meta, ldm);
    hipError_t e = ssg::launch_compress(to_dt(dt), M, K, A, lda, vals, ldv, meta, ldm, vec, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "compress launch");
}

int ssg_decompress_2to4(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                        int64_t ldm, void* D, int64_t ldd, int32_t* bad_count, void* stream) {
    int rc = check_dense(dt, M, K, D, ldd);
    if (rc) return rc;
    rc = check_compressed(M, K, vals, ldv, meta, ldm, true);
    if (rc) return rc;
    const bool vec = rows_aligned16(D, ldd, dt) && vec_compressed(dt, vals, ldv, meta, ldm);
    hipError_t e = ssg::launch_decompress(to_dt(dt), M, K, vals, ldv, meta, ldm, D, ldd, bad_count, vec,
                                          (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "decompress launch");
}

int ssg_split_count(int dt, int64_t M, int64_t K, const void* A, int64_t lda, int32_t* row_ptr, void* stream) {
    int rc = check_dense(dt, M, K, A, lda);
    if (rc) return rc;
    if (!row_ptr) return fail(SSG_ERR_NULL, "row_ptr is NULL");
    if (M > 0 && K / 2 > 0 && M > INT32_MAX / (K / 2))
        return fail(SSG_ERR_SHAPE, "residual of a %lld x %lld matrix may not fit int32 row_ptr", (long long)M,
                    (long long)K);
    hipError_t e = ssg::launch_split_count(to_dt(dt), M, K, A, lda, row_ptr, rows_aligned16(A, lda, dt),
                                           (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "split_count launch");
}

int ssg_split_fill(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* vals, int64_t ldv,
                   uint8_t* meta, int64_t ldm, const int32_t* row_ptr, int32_t* col, void* rvals, void* stream) {
    int rc = check_dense(dt, M, K, A, lda);
    if (rc) return rc;
    rc = check_compressed(M, K, vals, ldv, meta, ldm, true);
    if (rc) return rc;
    if (!row_ptr) return fail(SSG_ERR_NULL, "row_ptr is NULL");
    if ((col == nullptr) != (rvals == nullptr)) return fail(SSG_ERR_NULL, "col and rvals must both be set or both NULL");
    if (M > 0 && K / 2 > 0 && M > INT32_MAX / (K / 2))
        return fail(SSG_ERR_SHAPE, "residual may not fit int32 indices");
    const bool vec = rows_aligned16(A, lda, dt) && vec_compressed(dt, vals, ldv, meta, ldm);
    hipError_t e = ssg::launch_split_fill(to_dt(dt), M, K, A, lda, vals, ldv, meta, ldm, row_ptr, col, rvals, vec,
                                          (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "split_fill launch");
}

size_t ssg_spmm_workspace_bytes(int ab, int64_t M, int64_t N, int64_t K) {
    if (!in_dtype(ab) || M <= 0 || N < 0 || K < 0 || K % 4) return 0;
    return (size_t)padded_b_bytes(ab, N, K);
}

int ssg_spmm_2to4_ex(int algo, int ab, int c, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                     const uint8_t* meta, int64_t ldm, const void* B, int64_t ldb, void* C, int64_t ldc, void* ws,
                     size_t ws_bytes, void* stream) {
    int rc = check_spmm(ab, c, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc);
    if (rc) return rc;
    const ssg::SpmmArgs a = make_args(ab, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc);
    rc = check_workspace(pad_need(algo, a), ws, ws_bytes);
    if (rc) return rc;
    return run_spmm(algo, a, (hipStream_t)stream, ws);
}

int ssg_spmm_2to4(int ab, int c, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                  int64_t ldm, const void* B, int64_t ldb, void* C, int64_t ldc, void* ws, size_t ws_bytes,
                  void* stream) {
    return ssg_spmm_2to4_ex(SSG_ALGO_AUTO, ab, c, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc, ws, ws_bytes,
                            stream);
}

int ssg_spmm_2to4_residual_ex(int algo, int ab, int c, int64_t M, int64_t N, int64_t K, const void* vals,
                              int64_t ldv, const uint8_t* meta, int64_t ldm, const int32_t* row_ptr,
                              const int32_t* col, const void* rvals, int64_t nnz_r, const void* B, int64_t ldb,
                              void* C, int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_spmm(ab, c, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc);
    if (rc) return rc;
    if (nnz_r < 0 || nnz_r > INT32_MAX) return fail(SSG_ERR_FORMAT, "nnz_r=%lld out of range", (long long)nnz_r);
    if (M > 0 && !row_ptr) return fail(SSG_ERR_NULL, "row_ptr is NULL");
    if (nnz_r > 0 && (!col || !rvals)) return fail(SSG_ERR_NULL, "col or rvals is NULL with nnz_r > 0");
    ssg::SpmmArgs a = make_args(ab, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc);
    // an empty residual adds nothing: the plain 2:4 product (the residual
    // kernels may read entry 0 of a non-empty residual unconditionally)
    if (nnz_r > 0) { a.row_ptr = row_ptr; a.col = col; a.rvals = rvals; a.nnz_r = nnz_r; }
    rc = check_workspace(pad_need(algo, a), ws, ws_bytes);
    if (rc) return rc;
    return run_spmm(algo, a, (hipStream_t)stream, ws);
}

int ssg_residual_delta_count(int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col, int64_t nnz_r,
                             int32_t* drow_ptr, void* stream) {
    if (M < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (nnz_r < 0 || nnz_r > INT32_MAX) return fail(SSG_ERR_FORMAT, "nnz_r=%lld out of range", (long long)nnz_r);
    if (!drow_ptr) return fail(SSG_ERR_NULL, "drow_ptr is NULL");
    if (M > 0 && !row_ptr) return fail(SSG_ERR_NULL, "row_ptr is NULL");
    if (nnz_r > 0 && !col) return fail(SSG_ERR_NULL, "col is NULL with nnz_r > 0");
    // every entry plus at most one filler per 255 columns of each row
    if (M > 0 && nnz_r + M * (K / 255 + 1) > INT32_MAX)
        return fail(SSG_ERR_SHAPE, "delta-coded residual of %lld rows x %lld columns may not fit int32 indices",
                    (long long)M, (long long)K);
    hipError_t e = ssg::launch_delta_count(M, K, row_ptr, col, nnz_r, drow_ptr, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "delta_count launch");
}

int ssg_residual_delta_fill(int dt, int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col,
                            const void* rvals, int64_t nnz_r, const int32_t* drow_ptr, uint8_t* dcol, void* dvals,
                            void* stream) {
    if (!in_dtype(dt)) return fail(SSG_ERR_DTYPE, "element type %d is not SSG_F16, SSG_BF16, SSG_I8, SSG_E4M3 or SSG_E5M2", dt);
    if (M < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (nnz_r < 0 || nnz_r > INT32_MAX) return fail(SSG_ERR_FORMAT, "nnz_r=%lld out of range", (long long)nnz_r);
    if (M > 0 && (!row_ptr || !drow_ptr)) return fail(SSG_ERR_NULL, "row_ptr or drow_ptr is NULL");
    if (nnz_r > 0 && (!col || !rvals || !dcol || !dvals))
        return fail(SSG_ERR_NULL, "col, rvals, dcol or dvals is NULL with nnz_r > 0");
    hipError_t e = ssg::launch_delta_fill(to_dt(dt), M, K, row_ptr, col, rvals, nnz_r, drow_ptr, dcol, dvals,
                                          (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "delta_fill launch");
}

int ssg_spmm_2to4_residual_delta_ex(int algo, int ab, int c, int64_t M, int64_t N, int64_t K, const void* vals,
                                    int64_t ldv, const uint8_t* meta, int64_t ldm, const int32_t* drow_ptr,
                                    const uint8_t* dcol, const void* dvals, int64_t nnz_d, const void* B,
                                    int64_t ldb, void* C, int64_t ldc, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_spmm(ab, c, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc);
    if (rc) return rc;
    if (nnz_d < 0 || nnz_d > INT32_MAX) return fail(SSG_ERR_FORMAT, "nnz_d=%lld out of range", (long long)nnz_d);
    if (M > 0 && !drow_ptr) return fail(SSG_ERR_NULL, "drow_ptr is NULL");
    if (nnz_d > 0 && (!dcol || !dvals)) return fail(SSG_ERR_NULL, "dcol or dvals is NULL with nnz_d > 0");
    ssg::SpmmArgs a = make_args(ab, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc);
    // an empty residual adds nothing: the plain 2:4 product (the residual
    // kernels may read entry 0 of a non-empty residual unconditionally)
    if (nnz_d > 0) { a.row_ptr = drow_ptr; a.dcol = dcol; a.rvals = dvals; a.nnz_r = nnz_d; }
    rc = check_workspace(pad_need(algo, a), ws, ws_bytes);
    if (rc) return rc;
    return run_spmm(algo, a, (hipStream_t)stream, ws);
}

int ssg_spmm_2to4_residual_delta(int ab, int c, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                                 const uint8_t* meta, int64_t ldm, const int32_t* drow_ptr, const uint8_t* dcol,
                                 const void* dvals, int64_t nnz_d, const void* B, int64_t ldb, void* C, int64_t ldc,
                                 void* ws, size_t ws_bytes, void* stream) {
    return ssg_spmm_2to4_residual_delta_ex(SSG_ALGO_AUTO, ab, c, M, N, K, vals, ldv, meta, ldm, drow_ptr, dcol, dvals,
                                           nnz_d, B, ldb, C, ldc, ws, ws_bytes, stream);
}

namespace {

// C = residual x B with no 2:4 layer: the small-N kernel (its weight stream
// empty) where it takes the problem, else the generic one.
int run_unstructured(int ab, int c, int64_t M, int64_t N, int64_t K, const int32_t* row_ptr, const int32_t* col,
                     const uint8_t* dcol, const void* vals, int64_t nnz, const void* B, int64_t ldb, void* C,
                     int64_t ldc, void* stream) {
    if (!pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    if (M < 0 || N < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size");
    if (N > ((int64_t)1 << 31) || M > ((int64_t)1 << 40)) return fail(SSG_ERR_SHAPE, "size too large");
    if (nnz < 0 || nnz > INT32_MAX) return fail(SSG_ERR_FORMAT, "nnz=%lld out of range", (long long)nnz);
    if (M > 0 && !row_ptr) return fail(SSG_ERR_NULL, "row_ptr is NULL");
    if (nnz > 0 && ((!col && !dcol) || !vals)) return fail(SSG_ERR_NULL, "column indices or values are NULL");
    if (K > 0 && N > 0 && !B) return fail(SSG_ERR_NULL, "B is NULL");
    if (M > 0 && N > 0 && !C) return fail(SSG_ERR_NULL, "C is NULL");
    if (ldb < N) return fail(SSG_ERR_STRIDE, "ldb=%lld < N=%lld", (long long)ldb, (long long)N);
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    if (M == 0 || N == 0) return SSG_OK;
    ssg::SpmmArgs a{};
    a.dt = to_dt(ab);
    a.M = M; a.N = N; a.K = K;
    a.vals = nullptr; a.ldv = 0; a.meta = nullptr; a.ldm = 0;
    a.row_ptr = row_ptr; a.col = dcol ? nullptr : col; a.dcol = dcol; a.rvals = vals; a.nnz_r = nnz;
    a.B = B; a.ldb = ldb; a.C = C; a.ldc = ldc;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (nnz == 0 || K == 0) {
        // the product is zero: the generic kernel writes it (no entries to read)
        a.row_ptr = nullptr;
        e = ssg::launch_spmm_generic(a, s);
    } else if (ssg::supported_small_n(a)) {
        e = ssg::launch_spmm_small_n(a, s);
    } else {
        e = ssg::launch_spmm_generic(a, s);
    }
    return e == hipSuccess ? SSG_OK : hip_fail(e, "unstructured spmm launch");
}

}  // namespace

int ssg_spmm_csr(int ab, int c, int64_t M, int64_t N, int64_t K, const int32_t* row_ptr, const int32_t* col,
                 const void* vals, int64_t nnz, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    return run_unstructured(ab, c, M, N, K, row_ptr, col, nullptr, vals, nnz, B, ldb, C, ldc, stream);
}

int ssg_spmm_csr_delta(int ab, int c, int64_t M, int64_t N, int64_t K, const int32_t* drow_ptr, const uint8_t* dcol,
                       const void* dvals, int64_t nnz_d, const void* B, int64_t ldb, void* C, int64_t ldc,
                       void* stream) {
    if (nnz_d > 0 && !dcol) return fail(SSG_ERR_NULL, "dcol is NULL with nnz_d > 0");
    return run_unstructured(ab, c, M, N, K, drow_ptr, nullptr, dcol, dvals, nnz_d, B, ldb, C, ldc, stream);
}

namespace {

int64_t kstep_of(int dt) { return esize(dt) == 1 ? 128 : 64; }
int64_t idx_bytes_of(int dt) { return esize(dt) == 1 ? 4 : 2; }

// Sizes of the packed decode layout; fails on K not a multiple of the k-step
// or a layout beyond the kernels' 31-bit offsets.
int packed_sizes(int dt, int64_t M, int64_t K, int64_t* vb, int64_t* mb) {
    if (!in_dtype(dt)) return fail(SSG_ERR_DTYPE, "element type %d is not SSG_F16, SSG_BF16, SSG_I8, SSG_E4M3 or SSG_E5M2", dt);
    if (M < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (K % kstep_of(dt) != 0)
        return fail(SSG_ERR_SHAPE, "K=%lld is not a multiple of %lld", (long long)K, (long long)kstep_of(dt));
    const int64_t blocks = ((M + 15) / 16) * (K / kstep_of(dt));
    if (blocks > (int64_t)0x7fffffff / 1024) return fail(SSG_ERR_SHAPE, "packed layout too large");
    *vb = blocks * 1024;
    *mb = blocks * 64 * idx_bytes_of(dt);
    return SSG_OK;
}

}  // namespace

int ssg_packed_sizes(int dt, int64_t M, int64_t K, int64_t* vals_bytes, int64_t* meta_bytes) {
    if (!vals_bytes || !meta_bytes) return fail(SSG_ERR_NULL, "size pointers are NULL");
    return packed_sizes(dt, M, K, vals_bytes, meta_bytes);
}

int ssg_pack_2to4_decode(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                         int64_t ldm, void* pvals, void* pmeta, void* stream) {
    int64_t vb, mb;
    int rc = packed_sizes(dt, M, K, &vb, &mb);
    if (rc) return rc;
    rc = check_compressed(M, K, vals, ldv, meta, ldm, true);
    if (rc) return rc;
    if (vb > 0 && (!pvals || !pmeta)) return fail(SSG_ERR_NULL, "pvals or pmeta is NULL");
    if (!rows_aligned16(vals, ldv, dt)) return fail(SSG_ERR_STRIDE, "vals rows must be 16-byte aligned");
    hipError_t e = ssg::launch_pack_decode(to_dt(dt), M, K, vals, ldv, meta, ldm, pvals, pmeta, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "pack launch");
}

namespace {

// The packed decode product, with an optional residual (CSR: col != NULL,
// delta-coded: dcol != NULL; nnz == 0: none).
int run_packed(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
               const int32_t* row_ptr, const int32_t* col, const uint8_t* dcol, const void* rvals, int64_t nnz,
               const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    if (!pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    int64_t vb, mb;
    int rc = packed_sizes(ab, M, K, &vb, &mb);
    if (rc) return rc;
    if (M == 0) return SSG_OK;
    if (N != 16 || ldb != 16)
        return fail(SSG_ERR_ALGO, "the packed product takes N == 16 with ldb == 16 (got N=%lld, ldb=%lld)",
                    (long long)N, (long long)ldb);
    if (K == 0) return fail(SSG_ERR_SHAPE, "K must be positive");
    if (!pvals || !pmeta || !B || !C) return fail(SSG_ERR_NULL, "a required pointer is NULL");
    if (!al(pvals, 16) || !al(pmeta, (uintptr_t)idx_bytes_of(ab)) || !al(B, 16))
        return fail(SSG_ERR_STRIDE, "pvals and B must be 16-byte aligned, pmeta aligned to its index words");
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    if (K * 16 * esize(ab) >= 0x7fffffff) return fail(SSG_ERR_SHAPE, "B too large for 31-bit offsets");
    ssg::SpmmArgs a = make_args(ab, M, N, K, nullptr, 0, nullptr, 0, B, ldb, C, ldc);
    if (nnz > 0) {
        // the residual epilogue reads up to 4 entries per lane with one load
        // per array, at 31-bit byte offsets
        const int64_t ib = dcol ? 1 : 4;
        const void* idx = dcol ? static_cast<const void*>(dcol) : static_cast<const void*>(col);
        if (!al(idx, (uintptr_t)(4 * ib)) || !al(rvals, (uintptr_t)(4 * esize(ab))) || nnz * ib >= 0x7fff0000 ||
            nnz * esize(ab) >= 0x7fff0000)
            return fail(SSG_ERR_ALGO, "residual arrays must be aligned to 4 entries and under 2^31 bytes");
        a.row_ptr = row_ptr; a.col = col; a.dcol = dcol; a.rvals = rvals; a.nnz_r = nnz;
    }
    hipError_t e = ssg::launch_spmm_packed(a, pvals, pmeta, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "packed spmm launch");
}

}  // namespace

int ssg_spmm_2to4_packed(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                         const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    return run_packed(ab, c, M, N, K, pvals, pmeta, nullptr, nullptr, nullptr, nullptr, 0, B, ldb, C, ldc, stream);
}

namespace {

// Validation shared by the activation-major decode products: Bt [N, K]
// row-major, 1 <= N <= 16, rows 16-byte multiples apart, 16-byte aligned,
// 16 rows within 31-bit offsets.
int check_bt_decode(int ab, int64_t N, int64_t K, const void* Bt, int64_t ldbt, int64_t ldc) {
    if (N < 1 || N > 16) return fail(SSG_ERR_ALGO, "the activation-major decode product takes 1 <= N <= 16 (got %lld)",
                                     (long long)N);
    if (ldbt < K) return fail(SSG_ERR_STRIDE, "ldbt=%lld < K=%lld", (long long)ldbt, (long long)K);
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    if (!al(Bt, 16) || (ldbt * esize(ab)) % 16 != 0)
        return fail(SSG_ERR_STRIDE, "Bt must be 16-byte aligned with rows a multiple of 16 bytes apart");
    if (16 * ldbt * esize(ab) >= 0x7fffffff) return fail(SSG_ERR_SHAPE, "Bt rows too long for 31-bit offsets");
    return SSG_OK;
}

}  // namespace

int ssg_spmm_2to4_packed_bt(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                            const void* Bt, int64_t ldbt, void* C, int64_t ldc, void* stream) {
    if (!pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    int64_t vb, mb;
    int rc = packed_sizes(ab, M, K, &vb, &mb);
    if (rc) return rc;
    if (M == 0 || N == 0) return SSG_OK;
    if (K == 0) return fail(SSG_ERR_SHAPE, "K must be positive");
    rc = check_bt_decode(ab, N, K, Bt, ldbt, ldc);
    if (rc) return rc;
    if (!pvals || !pmeta || !Bt || !C) return fail(SSG_ERR_NULL, "a required pointer is NULL");
    if (!al(pvals, 16) || !al(pmeta, (uintptr_t)idx_bytes_of(ab)))
        return fail(SSG_ERR_STRIDE, "pvals must be 16-byte aligned, pmeta aligned to its index words");
    ssg::SpmmArgs a = make_args(ab, M, N, K, nullptr, 0, nullptr, 0, Bt, ldbt, C, ldc);
    hipError_t e = ssg::launch_spmm_packed_bt(a, pvals, pmeta, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "packed spmm (Bt) launch");
}

int ssg_spmm_2to4_packed_residual(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals,
                                  const void* pmeta, const int32_t* row_ptr, const int32_t* col, const void* rvals,
                                  int64_t nnz_r, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    if (nnz_r < 0 || nnz_r > INT32_MAX) return fail(SSG_ERR_FORMAT, "nnz_r=%lld out of range", (long long)nnz_r);
    if (M > 0 && !row_ptr) return fail(SSG_ERR_NULL, "row_ptr is NULL");
    if (nnz_r > 0 && (!col || !rvals)) return fail(SSG_ERR_NULL, "col or rvals is NULL with nnz_r > 0");
    return run_packed(ab, c, M, N, K, pvals, pmeta, row_ptr, col, nullptr, rvals, nnz_r, B, ldb, C, ldc, stream);
}

int ssg_spmm_2to4_packed_residual_delta(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals,
                                        const void* pmeta, const int32_t* drow_ptr, const uint8_t* dcol,
                                        const void* dvals, int64_t nnz_d, const void* B, int64_t ldb, void* C,
                                        int64_t ldc, void* stream) {
    if (nnz_d < 0 || nnz_d > INT32_MAX) return fail(SSG_ERR_FORMAT, "nnz_d=%lld out of range", (long long)nnz_d);
    if (M > 0 && !drow_ptr) return fail(SSG_ERR_NULL, "drow_ptr is NULL");
    if (nnz_d > 0 && (!dcol || !dvals)) return fail(SSG_ERR_NULL, "dcol or dvals is NULL with nnz_d > 0");
    return run_packed(ab, c, M, N, K, pvals, pmeta, drow_ptr, nullptr, dcol, dvals, nnz_d, B, ldb, C, ldc, stream);
}

namespace {

// Geometry of the complement-bitmap residual: K a multiple of the k-step,
// every buffer within 31-bit offsets.
int cbm_sizes(int dt, int64_t M, int64_t K, int64_t* mask_bytes, int64_t* blocks) {
    if (!in_dtype(dt)) return fail(SSG_ERR_DTYPE, "element type %d is not SSG_F16, SSG_BF16, SSG_I8, SSG_E4M3 or SSG_E5M2", dt);
    if (M < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (K % kstep_of(dt) != 0)
        return fail(SSG_ERR_SHAPE, "K=%lld is not a multiple of %lld", (long long)K, (long long)kstep_of(dt));
    ssg::cbm_geometry(to_dt(dt), M, K, blocks, mask_bytes);
    if (*mask_bytes >= 0x7fffffff || (*blocks + 1) * 4 >= 0x7fffffff)
        return fail(SSG_ERR_SHAPE, "complement-bitmap residual too large (M=%lld, K=%lld)", (long long)M, (long long)K);
    return SSG_OK;
}

}  // namespace

int ssg_cbm_sizes(int dt, int64_t M, int64_t K, int64_t* mask_bytes, int64_t* blocks) {
    if (!mask_bytes || !blocks) return fail(SSG_ERR_NULL, "size pointers are NULL");
    return cbm_sizes(dt, M, K, mask_bytes, blocks);
}

int ssg_pack_residual_cbm(int dt, int64_t M, int64_t K, const uint8_t* meta, int64_t ldm, const int32_t* row_ptr,
                          const int32_t* col, const void* rvals, int64_t nnz_r, uint8_t* rmask, int32_t* roff,
                          void* cvals, int32_t* bad_count, void* stream) {
    int64_t mbytes, blocks;
    int rc = cbm_sizes(dt, M, K, &mbytes, &blocks);
    if (rc) return rc;
    if (nnz_r < 0 || nnz_r > INT32_MAX || nnz_r * esize(dt) >= 0x7fff0000)
        return fail(SSG_ERR_FORMAT, "nnz_r=%lld out of range", (long long)nnz_r);
    if (M > 0 && K > 0 && !meta) return fail(SSG_ERR_NULL, "meta is NULL");
    if (ldm < (K + 7) / 8) return fail(SSG_ERR_STRIDE, "ldm=%lld < ceil(K/8)=%lld", (long long)ldm, (long long)((K + 7) / 8));
    if (M > 0 && !row_ptr) return fail(SSG_ERR_NULL, "row_ptr is NULL");
    if (nnz_r > 0 && (!col || !rvals || !cvals)) return fail(SSG_ERR_NULL, "col, rvals or cvals is NULL with nnz_r > 0");
    if (!roff || (blocks > 0 && !rmask)) return fail(SSG_ERR_NULL, "rmask or roff is NULL");
    hipError_t e = ssg::launch_pack_cbm(to_dt(dt), M, K, meta, ldm, row_ptr, col, rvals, nnz_r, rmask, roff, cvals,
                                        bad_count, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "complement-bitmap pack launch");
}

namespace {

int run_packed_cbm(bool bt, int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                   const uint8_t* rmask, const int32_t* roff, const void* cvals, int64_t nvals, const void* B,
                   int64_t ldb, void* C, int64_t ldc, void* stream) {
    if (!pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    int64_t vb, mb, mbytes, blocks;
    int rc = packed_sizes(ab, M, K, &vb, &mb);
    if (rc) return rc;
    rc = cbm_sizes(ab, M, K, &mbytes, &blocks);
    if (rc) return rc;
    if (M == 0 || (bt && N == 0)) return SSG_OK;
    if (bt) {
        if (K == 0) return fail(SSG_ERR_SHAPE, "K must be positive");
        rc = check_bt_decode(ab, N, K, B, ldb, ldc);
        if (rc) return rc;
    } else if (N != 16 || ldb != 16) {
        return fail(SSG_ERR_ALGO, "the packed product takes N == 16 with ldb == 16 (got N=%lld, ldb=%lld)",
                    (long long)N, (long long)ldb);
    }
    if (K == 0) return fail(SSG_ERR_SHAPE, "K must be positive");
    if (!pvals || !pmeta || !B || !C || !rmask || !roff) return fail(SSG_ERR_NULL, "a required pointer is NULL");
    if (nvals < 0 || nvals * esize(ab) >= 0x7fff0000) return fail(SSG_ERR_FORMAT, "nvals=%lld out of range", (long long)nvals);
    if (nvals > 0 && !cvals) return fail(SSG_ERR_NULL, "cvals is NULL with nvals > 0");
    if (!al(pvals, 16) || !al(pmeta, (uintptr_t)idx_bytes_of(ab)) || !al(B, 16) || !al(rmask, (uintptr_t)(esize(ab) == 1 ? 2 : 1)) ||
        !al(roff, 4) || !al(cvals, 16))
        return fail(SSG_ERR_STRIDE, "pvals, B and cvals must be 16-byte aligned, pmeta and rmask aligned to their words, "
                                    "roff to 4 bytes");
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    if (K * 16 * esize(ab) >= 0x7fffffff) return fail(SSG_ERR_SHAPE, "B too large for 31-bit offsets");
    ssg::SpmmArgs a = make_args(ab, M, N, K, nullptr, 0, nullptr, 0, B, ldb, C, ldc);
    hipError_t e = bt ? ssg::launch_spmm_packed_cbm_bt(a, pvals, pmeta, rmask, roff, cvals, nvals, (hipStream_t)stream)
                      : ssg::launch_spmm_packed_cbm(a, pvals, pmeta, rmask, roff, cvals, nvals, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "packed spmm (complement-bitmap residual) launch");
}

}  // namespace

int ssg_spmm_2to4_packed_residual_cbm(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals,
                                      const void* pmeta, const uint8_t* rmask, const int32_t* roff, const void* cvals,
                                      int64_t nvals, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    return run_packed_cbm(false, ab, c, M, N, K, pvals, pmeta, rmask, roff, cvals, nvals, B, ldb, C, ldc, stream);
}

int ssg_spmm_2to4_packed_residual_cbm_bt(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals,
                                         const void* pmeta, const uint8_t* rmask, const int32_t* roff,
                                         const void* cvals, int64_t nvals, const void* Bt, int64_t ldbt, void* C,
                                         int64_t ldc, void* stream) {
    return run_packed_cbm(true, ab, c, M, N, K, pvals, pmeta, rmask, roff, cvals, nvals, Bt, ldbt, C, ldc, stream);
}

namespace {

// Sizes of the packed prefill layout; fails on K not a multiple of the stage
// (64 dense k for 16-bit types, 128 for 8-bit) or a tile's blocks beyond the
// kernel's 31-bit offsets.
int prefill_sizes(int dt, int64_t M, int64_t K, int64_t* vb, int64_t* mb) {
    if (!in_dtype(dt)) return fail(SSG_ERR_DTYPE, "element type %d is not SSG_F16, SSG_BF16, SSG_I8, SSG_E4M3 or SSG_E5M2", dt);
    if (M < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    const int64_t bk = esize(dt) == 1 ? 128 : 64;
    if (K % bk != 0) return fail(SSG_ERR_SHAPE, "K=%lld is not a multiple of %lld", (long long)K, (long long)bk);
    if (K / 2 * esize(dt) * 256 >= 0x7fffffff || M > ((int64_t)1 << 40))
        return fail(SSG_ERR_SHAPE, "packed prefill layout too large (M=%lld, K=%lld)", (long long)M, (long long)K);
    int64_t tiles, stages, mblocks;
    ssg::prefill_geometry(to_dt(dt), M, K, &tiles, &stages, &mblocks);
    *vb = tiles * stages * 16384;
    *mb = tiles * mblocks * 8192;
    return SSG_OK;
}

int check_prefill_out(int64_t vb, const void* pvals, const void* pmeta) {
    if (vb > 0 && (!pvals || !pmeta)) return fail(SSG_ERR_NULL, "pvals or pmeta is NULL");
    if (!al(pvals, 16) || !al(pmeta, 4)) return fail(SSG_ERR_STRIDE, "pvals must be 16-byte and pmeta 4-byte aligned");
    return SSG_OK;
}

}  // namespace

int ssg_prefill_packed_sizes(int dt, int64_t M, int64_t K, int64_t* vals_bytes, int64_t* meta_bytes) {
    if (!vals_bytes || !meta_bytes) return fail(SSG_ERR_NULL, "size pointers are NULL");
    return prefill_sizes(dt, M, K, vals_bytes, meta_bytes);
}

int ssg_compress_2to4_prefill(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* pvals, void* pmeta,
                              void* stream) {
    int64_t vb, mb;
    int rc = prefill_sizes(dt, M, K, &vb, &mb);
    if (rc) return rc;
    rc = check_dense(dt, M, K, A, lda);
    if (rc) return rc;
    rc = check_prefill_out(vb, pvals, pmeta);
    if (rc) return rc;
    if (vb == 0) return SSG_OK;
    hipError_t e = ssg::launch_compress_prefill(to_dt(dt), M, K, A, lda, pvals, pmeta, rows_aligned16(A, lda, dt),
                                                (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "compress (packed prefill) launch");
}

int ssg_pack_2to4_prefill(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                          int64_t ldm, void* pvals, void* pmeta, void* stream) {
    int64_t vb, mb;
    int rc = prefill_sizes(dt, M, K, &vb, &mb);
    if (rc) return rc;
    rc = check_compressed(M, K, vals, ldv, meta, ldm, true);
    if (rc) return rc;
    rc = check_prefill_out(vb, pvals, pmeta);
    if (rc) return rc;
    if (vb == 0) return SSG_OK;
    if (!rows_aligned16(vals, ldv, dt)) return fail(SSG_ERR_STRIDE, "vals rows must be 16-byte aligned");
    hipError_t e = ssg::launch_pack_prefill(to_dt(dt), M, K, vals, ldv, meta, ldm, pvals, pmeta, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "pack (prefill) launch");
}

int ssg_spmm_2to4_prefill(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                          const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    if (!pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    if (N < 0 || N > ((int64_t)1 << 31)) return fail(SSG_ERR_SHAPE, "N=%lld out of range", (long long)N);
    int64_t vb, mb;
    int rc = prefill_sizes(ab, M, K, &vb, &mb);
    if (rc) return rc;
    if (ldb < N) return fail(SSG_ERR_STRIDE, "ldb=%lld < N=%lld", (long long)ldb, (long long)N);
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    if (M == 0 || N == 0) return SSG_OK;
    if (K == 0) return fail(SSG_ERR_SHAPE, "K must be positive");
    if (!pvals || !pmeta || !B || !C) return fail(SSG_ERR_NULL, "a required pointer is NULL");
    ssg::SpmmArgs a = make_args(ab, M, N, K, pvals, 0, static_cast<const uint8_t*>(pmeta), 0, B, ldb, C, ldc);
    if (!ssg::supported_prefill_packed(a))
        return fail(SSG_ERR_ALGO,
                    "the packed prefill product needs N a multiple of %d, pvals and B rows 16-byte aligned, pmeta "
                    "4-byte aligned and B within 31-bit offsets",
                    (int)(16 / esize(ab)));
    hipError_t e = ssg::launch_spmm_prefill_packed(a, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "packed prefill spmm launch");
}

int ssg_spmm_2to4_prefill_bt(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                             const void* Bt, int64_t ldbt, void* C, int64_t ldc, void* stream) {
    if (!pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    if (N < 0 || N > ((int64_t)1 << 31)) return fail(SSG_ERR_SHAPE, "N=%lld out of range", (long long)N);
    int64_t vb, mb;
    int rc = prefill_sizes(ab, M, K, &vb, &mb);
    if (rc) return rc;
    if (ldbt < K) return fail(SSG_ERR_STRIDE, "ldbt=%lld < K=%lld", (long long)ldbt, (long long)K);
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    if (M == 0 || N == 0) return SSG_OK;
    if (K == 0) return fail(SSG_ERR_SHAPE, "K must be positive");
    if (!pvals || !pmeta || !Bt || !C) return fail(SSG_ERR_NULL, "a required pointer is NULL");
    ssg::SpmmArgs a = make_args(ab, M, N, K, pvals, 0, static_cast<const uint8_t*>(pmeta), 0, Bt, ldbt, C, ldc);
    if (!ssg::supported_prefill_packed_bt(a))
        return fail(SSG_ERR_ALGO,
                    "the packed prefill product with Bt needs pvals and Bt rows 16-byte aligned, pmeta 4-byte "
                    "aligned and 256 rows of Bt within 31-bit offsets");
    hipError_t e = ssg::launch_spmm_prefill_packed_bt(a, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "packed prefill spmm (Bt) launch");
}

int64_t ssg_stream_read_sink_words(int64_t bytes) { return bytes > 0 ? ssg::stream_read_grid(bytes) : 0; }

int ssg_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    if (bytes < 0 || bytes % 16) return fail(SSG_ERR_SHAPE, "bytes=%lld is not a non-negative multiple of 16",
                                             (long long)bytes);
    if (bytes == 0) return SSG_OK;
    if (!src || !sink) return fail(SSG_ERR_NULL, "src or sink is NULL");
    if (!al(src, 16)) return fail(SSG_ERR_STRIDE, "src must be 16-byte aligned");
    hipError_t e = ssg::launch_stream_read(src, bytes, sink, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "stream read launch");
}

int ssg_mfma_probe_forms(void) { return ssg::mfma_probe_forms(); }

const char* ssg_mfma_probe_name(int form) { return ssg::mfma_probe_name(form); }

int64_t ssg_mfma_probe_ops(int form, int64_t workgroups, int64_t iters) {
    return ssg::mfma_probe_ops(form, workgroups, iters);
}

int ssg_mfma_probe(int form, int64_t workgroups, int64_t iters, uint32_t* sink, void* stream) {
    if (!ssg::mfma_probe_name(form))
        return fail(SSG_ERR_ALGO, "form %d is not in [0, %d)", form, ssg::mfma_probe_forms());
    if (workgroups <= 0 || workgroups > 0x7fffffff || iters <= 0)
        return fail(SSG_ERR_SHAPE, "workgroups=%lld and iters=%lld must be positive (workgroups below 2^31)",
                    (long long)workgroups, (long long)iters);
    if (!sink) return fail(SSG_ERR_NULL, "sink is NULL");
    hipError_t e = ssg::launch_mfma_probe(form, workgroups, iters, sink, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "matrix-instruction probe launch");
}

int ssg_lds_read_probe(const uint32_t* offsets, int64_t workgroups, int64_t iters, uint32_t* sink, void* stream) {
    if (!offsets || !sink) return fail(SSG_ERR_NULL, "offsets or sink is NULL");
    ssg::LdsPattern pat;
    for (int l = 0; l < 64; ++l) {
        if (offsets[l] % 16 || offsets[l] > ssg::kLdsProbeMaxOffset)
            return fail(SSG_ERR_SHAPE, "offsets[%d]=%u is not a multiple of 16 in [0, %u]", l, offsets[l],
                        ssg::kLdsProbeMaxOffset);
        pat.off[l] = offsets[l];
    }
    if (workgroups <= 0 || workgroups > 0x7fffffff || iters <= 0)
        return fail(SSG_ERR_SHAPE, "workgroups=%lld and iters=%lld must be positive (workgroups below 2^31)",
                    (long long)workgroups, (long long)iters);
    hipError_t e = ssg::launch_lds_read_probe(pat, workgroups, iters, sink, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "LDS read probe launch");
}

int64_t ssg_nm_vals_cols(int nm_n, int nm_m, int64_t K) {
    return nm_m > 0 && nm_n >= 0 ? K / nm_m * nm_n : 0;
}

}  // extern "C"

namespace {

// Bytes of a row of ld elements (4-bit weights: two per byte).
int64_t row_bytes(int dt, int64_t ld) { return dt == SSG_I4 ? ld / 2 : ld * esize(dt); }

// N:M products: the 2:4 pairs, and 4-bit weights with fp16 B into fp32.
bool nm_pair_ok(int ab, int c) { return pair_ok(ab, c) || (ab == SSG_I4 && c == SSG_F32); }

int check_nm_shape(int dt, int nm_n, int nm_m, int64_t M, int64_t K) {
    if (!in_dtype(dt) && dt != SSG_I4)
        return fail(SSG_ERR_DTYPE, "element type %d is not SSG_F16, SSG_BF16, SSG_I8, SSG_E4M3, SSG_E5M2 or SSG_I4", dt);
    if (!ssg::nm_pattern_supported(nm_n, nm_m))
        return fail(SSG_ERR_SHAPE, "pattern %d:%d is not one of 1:4, 2:4, 2:8, 4:8", nm_n, nm_m);
    if (dt == SSG_I4 && nm_n % 2)
        return fail(SSG_ERR_SHAPE, "4-bit weights take 2:4, 2:8 or 4:8 (whole bytes per group), not %d:%d", nm_n, nm_m);
    if (M < 0 || K < 0) return fail(SSG_ERR_SHAPE, "negative size M=%lld K=%lld", (long long)M, (long long)K);
    if (K % nm_m != 0) return fail(SSG_ERR_SHAPE, "K=%lld is not a multiple of %d", (long long)K, nm_m);
    if ((M * ((K + 31) / 32)) / 256 >= (int64_t)1 << 31)
        return fail(SSG_ERR_SHAPE, "M*K too large (%lld x %lld)", (long long)M, (long long)K);
    return SSG_OK;
}

int check_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* mask,
             int64_t ldm) {
    int rc = check_nm_shape(dt, nm_n, nm_m, M, K);
    if (rc) return rc;
    if (M > 0 && K > 0 && (!vals || !mask)) return fail(SSG_ERR_NULL, "vals or mask is NULL");
    if (ldv < K / nm_m * nm_n)
        return fail(SSG_ERR_STRIDE, "ldv=%lld < K/%d*%d=%lld", (long long)ldv, nm_m, nm_n, (long long)(K / nm_m * nm_n));
    if (ldm < (K + 7) / 8) return fail(SSG_ERR_STRIDE, "ldmask=%lld < ceil(K/8)=%lld", (long long)ldm, (long long)((K + 7) / 8));
    if (dt == SSG_I4 && ldv % 2) return fail(SSG_ERR_STRIDE, "4-bit rows start on whole bytes: ldv=%lld is odd", (long long)ldv);
    return SSG_OK;
}

// The compress / expand kernels' 32-element chunks: A or D rows 16-byte
// aligned, value rows 8-byte aligned, mask rows 4-byte aligned.
bool vec_nm(int dt, const void* dense, int64_t ldd, const void* vals, int64_t ldv, const uint8_t* mask, int64_t ldm) {
    return al(dense, 16) && row_bytes(dt, ldd) % 16 == 0 && al(vals, 8) && row_bytes(dt, ldv) % 8 == 0 &&
           al(mask, 4) && ldm % 4 == 0;
}

}  // namespace

extern "C" {

int ssg_compress_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* A, int64_t lda, void* vals,
                    int64_t ldv, uint8_t* mask, int64_t ldmask, void* stream) {
    int rc = check_nm(dt, nm_n, nm_m, M, K, vals, ldv, mask, ldmask);
    if (rc) return rc;
    if (M > 0 && K > 0 && !A) return fail(SSG_ERR_NULL, "A is NULL");
    if (lda < K) return fail(SSG_ERR_STRIDE, "lda=%lld < K=%lld", (long long)lda, (long long)K);
    if (dt == SSG_I4 && lda % 2) return fail(SSG_ERR_STRIDE, "4-bit rows start on whole bytes: lda=%lld is odd", (long long)lda);
    hipError_t e = ssg::launch_compress_nm(to_dt(dt), nm_n, nm_m, M, K, A, lda, vals, ldv, mask, ldmask,
                                           vec_nm(dt, A, lda, vals, ldv, mask, ldmask), (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "compress_nm launch");
}

int ssg_decompress_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                      const uint8_t* mask, int64_t ldmask, void* D, int64_t ldd, int32_t* bad_count, void* stream) {
    int rc = check_nm(dt, nm_n, nm_m, M, K, vals, ldv, mask, ldmask);
    if (rc) return rc;
    if (M > 0 && K > 0 && !D) return fail(SSG_ERR_NULL, "D is NULL");
    if (ldd < K) return fail(SSG_ERR_STRIDE, "ldd=%lld < K=%lld", (long long)ldd, (long long)K);
    if (dt == SSG_I4 && ldd % 2) return fail(SSG_ERR_STRIDE, "4-bit rows start on whole bytes: ldd=%lld is odd", (long long)ldd);
    hipError_t e = ssg::launch_decompress_nm(to_dt(dt), nm_n, nm_m, M, K, vals, ldv, mask, ldmask, D, ldd, bad_count,
                                             (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "decompress_nm launch");
}

int ssg_spmm_nm(int ab, int c, int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                const uint8_t* mask, int64_t ldmask, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    if (!nm_pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    int rc = check_nm(ab, nm_n, nm_m, M, K, vals, ldv, mask, ldmask);
    if (rc) return rc;
    // one grid row per 16 columns of B
    if (N < 0 || (N + 15) / 16 > 65535) return fail(SSG_ERR_SHAPE, "N=%lld out of range", (long long)N);
    if (K > 0 && N > 0 && !B) return fail(SSG_ERR_NULL, "B is NULL");
    if (M > 0 && N > 0 && !C) return fail(SSG_ERR_NULL, "C is NULL");
    if (ldb < N) return fail(SSG_ERR_STRIDE, "ldb=%lld < N=%lld", (long long)ldb, (long long)N);
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    if (M == 0 || N == 0) return SSG_OK;
    const int bt = ab == SSG_I4 ? SSG_F16 : ab;          // B's element type
    const int64_t es = esize(bt);
    if (K == 0) {
        // an empty sum: the generic kernel writes the zeros and reads nothing
        hipError_t e = ssg::launch_spmm_generic(make_args(bt, M, N, 0, nullptr, 0, nullptr, 0, B, ldb, C, ldc),
                                                (hipStream_t)stream);
        return e == hipSuccess ? SSG_OK : hip_fail(e, "zero fill");
    }
    // row strides matter only where there is more than one row
    if (!al(vals, 16) || (M > 1 && row_bytes(ab, ldv) % 16 != 0))
        return fail(SSG_ERR_STRIDE, "vals rows must be 16-byte aligned (base and row bytes)");
    if (!al(mask, 8) || (M > 1 && ldmask % 8 != 0))
        return fail(SSG_ERR_STRIDE, "mask rows must be 8-byte aligned (base and ldmask)");
    if (!al(B, 16) || (K > 1 && (ldb * es) % 16 != 0))
        return fail(SSG_ERR_STRIDE, "B rows must be 16-byte aligned (base and ldb * element size)");
    // 32-bit buffer offsets: a workgroup's 64 rows of vals / mask, all of B
    if (64 * row_bytes(ab, ldv) >= 0x7fffffff || 64 * ldmask >= 0x7fffffff || K * ldb * es >= 0x7fffffff)
        return fail(SSG_ERR_SHAPE, "operands too large for 31-bit buffer offsets");
    ssg::SpmmArgs a = make_args(ab, M, N, K, vals, ldv, mask, ldmask, B, ldb, C, ldc);
    hipError_t e = ssg::launch_spmm_nm(nm_n, nm_m, a, false, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "spmm_nm launch");
}

int ssg_nm_packed_sizes(int dt, int nm_n, int nm_m, int64_t M, int64_t K, int64_t* vals_bytes,
                        int64_t* mask_bytes) {
    int rc = check_nm_shape(dt, nm_n, nm_m, M, K);
    if (rc) return rc;
    if (!vals_bytes || !mask_bytes) return fail(SSG_ERR_NULL, "vals_bytes or mask_bytes is NULL");
    int64_t tiles, nsteps;
    int vb, mb;
    ssg::nm_packed_geometry(to_dt(dt), nm_n, nm_m, M, K, &tiles, &nsteps, &vb, &mb);
    *vals_bytes = tiles * nsteps * 64 * vb;
    *mask_bytes = tiles * nsteps * 64 * mb;
    return SSG_OK;
}

int ssg_pack_nm_decode(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                       const uint8_t* mask, int64_t ldmask, void* pvals, void* pmask, void* stream) {
    int rc = check_nm(dt, nm_n, nm_m, M, K, vals, ldv, mask, ldmask);
    if (rc) return rc;
    int64_t vb, mb;
    rc = ssg_nm_packed_sizes(dt, nm_n, nm_m, M, K, &vb, &mb);
    if (rc) return rc;
    if (vb > 0 && (!pvals || !pmask)) return fail(SSG_ERR_NULL, "pvals or pmask is NULL");
    if (!al(pvals, 16) || !al(pmask, 8)) return fail(SSG_ERR_STRIDE, "pvals must be 16-byte and pmask 8-byte aligned");
    hipError_t e = ssg::launch_pack_nm(to_dt(dt), nm_n, nm_m, M, K, vals, ldv, mask, ldmask, pvals, pmask,
                                       (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "pack_nm launch");
}

int ssg_spmm_nm_packed(int ab, int c, int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* pvals,
                       const void* pmask, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    if (!nm_pair_ok(ab, c)) return fail(SSG_ERR_DTYPE, "unsupported (input, output) types (%d, %d)", ab, c);
    int64_t vb, mb;
    int rc = ssg_nm_packed_sizes(ab, nm_n, nm_m, M, K, &vb, &mb);
    if (rc) return rc;
    if (N < 0 || (N + 15) / 16 > 65535) return fail(SSG_ERR_SHAPE, "N=%lld out of range", (long long)N);
    if (M == 0 || N == 0) return SSG_OK;
    if (K == 0) return fail(SSG_ERR_SHAPE, "K must be positive");
    if (!pvals || !pmask || !B || !C) return fail(SSG_ERR_NULL, "a required pointer is NULL");
    if (ldb < N) return fail(SSG_ERR_STRIDE, "ldb=%lld < N=%lld", (long long)ldb, (long long)N);
    if (ldc < N) return fail(SSG_ERR_STRIDE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
    const int64_t es = esize(ab == SSG_I4 ? SSG_F16 : ab);   // B's element size
    if (!al(pvals, 16) || !al(pmask, 8)) return fail(SSG_ERR_STRIDE, "pvals must be 16-byte and pmask 8-byte aligned");
    if (!al(B, 16) || (K > 1 && (ldb * es) % 16 != 0))
        return fail(SSG_ERR_STRIDE, "B rows must be 16-byte aligned (base and ldb * element size)");
    // 32-bit buffer offsets: a workgroup's 4 tiles of blocks, all of B
    if (4 * (vb / ((M + 15) / 16)) >= 0x7fffffff || K * ldb * es >= 0x7fffffff)
        return fail(SSG_ERR_SHAPE, "operands too large for 31-bit buffer offsets");
    ssg::SpmmArgs a = make_args(ab, M, N, K, pvals, 0, static_cast<const uint8_t*>(pmask), 0, B, ldb, C, ldc);
    hipError_t e = ssg::launch_spmm_nm(nm_n, nm_m, a, true, (hipStream_t)stream);
    return e == hipSuccess ? SSG_OK : hip_fail(e, "spmm_nm_packed launch");
}

int ssg_spmm_2to4_residual(int ab, int c, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                           const uint8_t* meta, int64_t ldm, const int32_t* row_ptr, const int32_t* col,
                           const void* rvals, int64_t nnz_r, const void* B, int64_t ldb, void* C, int64_t ldc,
                           void* ws, size_t ws_bytes, void* stream) {
    return ssg_spmm_2to4_residual_ex(SSG_ALGO_AUTO, ab, c, M, N, K, vals, ldv, meta, ldm, row_ptr, col, rvals, nnz_r,
                                     B, ldb, C, ldc, ws, ws_bytes, stream);
}

int ssg_spmm_select_algo(int ab, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                         const uint8_t* meta, int64_t ldm, const void* B, int64_t ldb, const void* C, int64_t ldc) {
    if (!in_dtype(ab) || M <= 0 || N <= 0 || K <= 0 || K % 4) return SSG_ALGO_GENERIC;
    return pick_algo(make_args(ab, M, N, K, vals, ldv, meta, ldm, B, ldb, const_cast<void*>(C), ldc));
}

}  // extern "C"

// ---- the product that allocates nothing --------------------------------------
//
// For callers that cannot allocate (code under stream capture, tight serving
// loops): ssg_spmm_2to4_noalloc takes its padded copy of a narrow B from a
// file-scope device array instead of a caller workspace.  Each device holds
// its own copy of the array until the process ends; its address on a device
// is looked up once, with that device current, and kept.  In host code the
// array's name is not a device address: only the looked-up pointer is ever
// passed to a kernel.

namespace {

constexpr int64_t kScratchBytes = (int64_t)2 << 20;   // B padded to K x 16: K <= 65536 (16-bit), 131072 (8-bit)
constexpr int kScratchDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there).
int scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(SSG_ERR_HIP, "device %d is beyond the %d devices the scratch table holds", dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SSG_OK;
}

}  // namespace

extern "C" {

int64_t ssg_noalloc_scratch_bytes(void) { return kScratchBytes; }

int ssg_spmm_2to4_noalloc(int ab, int c, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                          const uint8_t* meta, int64_t ldm, const void* B, int64_t ldb, void* C, int64_t ldc,
                          void* stream) {
    int rc = check_spmm(ab, c, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc);
    if (rc) return rc;
    const ssg::SpmmArgs a = make_args(ab, M, N, K, vals, ldv, meta, ldm, B, ldb, C, ldc);
    const int64_t need = pad_need(SSG_ALGO_AUTO, a);
    if (need > kScratchBytes)
        return fail(SSG_ERR_WORKSPACE,
                    "the padded B (K=%lld x 16 columns, %lld bytes) exceeds the %lld-byte scratch of the no-alloc "
                    "product; call ssg_spmm_2to4 with a workspace",
                    (long long)K, (long long)need, (long long)kScratchBytes);
    void* ws = nullptr;
    if (need > 0) {
        rc = scratch_for_current_device(&ws);
        if (rc) return rc;
    }
    return run_spmm(SSG_ALGO_AUTO, a, (hipStream_t)stream, ws);
}

}  // extern "C"
