/*
 * ssgemm.h -- C ABI of libssgemm.so: 2:4 structured-sparse weight times dense
 * activation matrix multiply (SpMM) on AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages this follows):
 *   - 2:4 structure: in every group of 4 consecutive elements along the
 *     reduction dimension at most two are non-zero; the two kept values are
 *     stored with a 2-bit position each, 4 bits per group
 *     ["Chapter 26 -- Sparsity: The Hardware View", section "2:4 Fine-Grained
 *      Structured Sparsity", worked example; "10.4g Structured Sparsity (2:4)",
 *      sections "What is 2:4 Structured Sparsity?" and "How Tensor Cores
 *      Leverage This Pattern"].
 *   - Pruning keeps the two largest magnitudes of each group and the kept
 *     positions are stored in ascending order ["Chapter 26", first listing of
 *     section "Python: Build a 2:4 Mask, Compress It, ..."].
 *   - The product is C = A x B with the sparse weight on the left ["Chapter 26",
 *     second listing of the same section].
 *   - Moderately unstructured weights are split into a 2:4 layer plus a
 *     residual layer holding what the 2:4 layer dropped, so the product stays
 *     exact ["How sparse LLM weights cut GPU inference cost without
 *     quantization", section "How the three-layer format makes moderate
 *     sparsity fast"].
 *
 * Layout (all row-major, leading dimensions counted in elements):
 *   A     [M, K]  dense weight, K % 4 == 0, groups of 4 along K (lda >= K)
 *   vals  [M, K/2] kept values, group g at columns 2g, 2g+1 (ldv >= K/2)
 *   meta  [M, ceil(K/8)] uint8: nibble of group g is i0 | (i1 << 2), with
 *         i0 < i1 the kept positions inside the group; group 2j is the low
 *         nibble of byte j, group 2j+1 the high nibble; an unused high nibble
 *         of the last byte is 0 (ldm >= ceil(K/8)).  Valid nibbles are
 *         0x4, 0x8, 0xC, 0x9, 0xD, 0xE.
 *   B     [K, N]  dense activation (ldb >= N)
 *   C     [M, N]  fp32 for fp16/bf16/fp8 inputs, int32 for int8 inputs (ldc >= N)
 *   residual: CSR, row_ptr int32 [M+1] (row_ptr[0] = 0), col int32 [nnz]
 *         ascending within a row, rvals [nnz] in the element type of A; or
 *         delta-coded (one-byte column gaps, described before
 *         ssg_residual_delta_count).
 *
 * Selection rule: for a group with magnitudes a0..a3 (|x| of the value; int8
 * -128 has magnitude 128; -0 and +0 are equal), position p is kept iff fewer
 * than two positions q != p have |a_q| > |a_p|, or |a_q| == |a_p| and q < p.
 * Exactly two slots are stored per group; a kept slot may hold a zero.
 * Inputs must be finite; NaN/Inf inputs give unspecified selections.
 *
 * Ownership and execution: every pointer is device memory owned by the
 * caller; the library allocates no device memory and keeps no mutable global
 * state (calls are re-entrant).  Every call validates its arguments on the
 * host, enqueues its kernels on `stream` (a hipStream_t; NULL = the null
 * stream) and returns without synchronising.  Asynchronous device faults show
 * at the caller's next synchronisation.  No C++ exception crosses the ABI.
 *
 * Errors: a non-zero return is an ssg_status; nothing was enqueued when
 * validation fails.  Zero-size problems return SSG_OK and enqueue nothing,
 * except spmm with K == 0, which zero-fills C.  ssg_last_error() gives a
 * thread-local description of the last failure.
 */
#ifndef SSGEMM_H
#define SSGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSG_ABI_VERSION 1

typedef enum {
    SSG_OK = 0,
    SSG_ERR_NULL = 1,       /* a required pointer is NULL */
    SSG_ERR_SHAPE = 2,      /* negative size, K % 4 != 0, or a size too large for the kernels */
    SSG_ERR_STRIDE = 3,     /* a leading dimension smaller than its row */
    SSG_ERR_DTYPE = 4,      /* unsupported element type or (input, output) pair */
    SSG_ERR_FORMAT = 5,     /* inconsistent sparse operand arguments (nnz_r < 0 or above 2^31 - 1) */
    SSG_ERR_WORKSPACE = 6,  /* a needed workspace is missing, too small or misaligned */
    SSG_ERR_HIP = 7,        /* a HIP runtime call failed; see ssg_last_error() */
    SSG_ERR_ALGO = 8        /* the requested algorithm cannot run this problem */
} ssg_status;

/* Element types.  SSG_E4M3 / SSG_E5M2 are the OCP 8-bit floats (sign, 4 / 5
 * exponent bits with bias 7 / 15, 3 / 2 fraction bits; E4M3 has no
 * infinities and S.1111.111 is NaN), which the pages stack with 2:4
 * ("Chapter 26 -- Sparsity: The Hardware View", section "Sparsity +
 * Quantization Combine"); they take the int8 layouts (1 byte per value,
 * 4 metadata bytes per 16 stored values of a sparse-MFMA lane) and
 * accumulate into fp32. */
typedef enum {
    SSG_F16 = 0, SSG_BF16 = 1, SSG_I8 = 2, SSG_F32 = 3, SSG_I32 = 4, SSG_E4M3 = 5, SSG_E5M2 = 6, SSG_I4 = 7
} ssg_dtype;

/* SpMM algorithms.  AUTO picks by shape; the others force one kernel family
 * (for A/B comparison and tests) and return SSG_ERR_ALGO when the problem is
 * outside what that family handles. */
typedef enum {
    SSG_ALGO_AUTO = 0,
    SSG_ALGO_GENERIC = 1,   /* one thread per output, any shape/stride/alignment */
    SSG_ALGO_SMALL_N = 2,   /* bandwidth-bound decode shapes (N <= 16) on sparse MFMA */
    SSG_ALGO_LARGE_N = 3    /* compute-bound tiles on sparse MFMA */
} ssg_algo;

int ssg_abi_version(void);
const char* ssg_status_str(int status);
const char* ssg_last_error(void);

/* Row lengths of the compressed operands for a reduction length K. */
int64_t ssg_vals_cols(int64_t K);   /* K / 2 */
int64_t ssg_meta_cols(int64_t K);   /* ceil(K / 8) bytes */

/* P = A with the two dropped elements of every group set to +0 (kept ones
 * bit-copied).  dt: SSG_F16, SSG_BF16 or SSG_I8.  P may alias A exactly
 * (in place, lda == ldp); other overlaps are undefined. */
int ssg_prune_2to4(int dt, int64_t M, int64_t K, const void* A, int64_t lda,
                   void* P, int64_t ldp, void* stream);

/* (vals, meta) = the 2:4 compressed form of A (values bit-copied). */
int ssg_compress_2to4(int dt, int64_t M, int64_t K, const void* A, int64_t lda,
                      void* vals, int64_t ldv, uint8_t* meta, int64_t ldm, void* stream);

/* D = dense expansion of (vals, meta): the two stored values at their
 * positions, +0 elsewhere.  A group whose nibble is not a valid pair is
 * written as four zeros and, if bad_count is not NULL, counted into the
 * device int32 *bad_count (added atomically; the caller zeroes it). */
int ssg_decompress_2to4(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv,
                        const uint8_t* meta, int64_t ldm, void* D, int64_t ldd,
                        int32_t* bad_count, void* stream);

/* Residual split, pass 1: row_ptr[0] = 0 and row_ptr[m+1] = row_ptr[m] + the
 * number of numerically non-zero elements of row m (-0 counts as zero) that
 * the 2:4 selection drops.  The caller then reads row_ptr[M] (nnz of the
 * residual) to size col and rvals.  Fails with SSG_ERR_SHAPE if M * K exceeds
 * what int32 row_ptr can count (2^31 - 1). */
int ssg_split_count(int dt, int64_t M, int64_t K, const void* A, int64_t lda,
                    int32_t* row_ptr, void* stream);

/* Residual split, pass 2: writes the 2:4 layer (as ssg_compress_2to4) and the
 * CSR residual (col ascending, rvals bit-copied) using row_ptr from pass 1.
 * col and rvals may be NULL only if row_ptr[M] == 0. */
int ssg_split_fill(int dt, int64_t M, int64_t K, const void* A, int64_t lda,
                   void* vals, int64_t ldv, uint8_t* meta, int64_t ldm,
                   const int32_t* row_ptr, int32_t* col, void* rvals, void* stream);

/* Workspace the SpMM calls may need for this problem (bytes; may be 0).  It
 * is 0 except for 0 < N < 16 (and M > 0, K % 4 == 0, K * 16 elements under
 * 2^31 bytes), where it holds B padded to 16 zero-extended columns (K * 16
 * elements, rounded up to 256 bytes): the decode kernels then take B as one
 * contiguous K x 16 block.  A product requires it (16-byte aligned, at least
 * this size; else SSG_ERR_WORKSPACE) only when it takes that padded path:
 * algorithm AUTO or SMALL_N, and an operand the small-N kernel accepts
 * (vals rows 16-byte aligned, K a multiple of its k-step, residual arrays
 * aligned).  Forced GENERIC or LARGE_N calls never touch it and may pass
 * ws = NULL.  The workspace is used on `stream` only. */
size_t ssg_spmm_workspace_bytes(int ab, int64_t M, int64_t N, int64_t K);

/* C = expand(vals, meta) x B.  (ab, c) must be (SSG_F16, SSG_F32),
 * (SSG_BF16, SSG_F32), (SSG_E4M3, SSG_F32), (SSG_E5M2, SSG_F32) or
 * (SSG_I8, SSG_I32).  fp16/bf16 products are
 * accumulated in fp32 in an order that is fixed for a given shape and
 * algorithm (results are reproducible run to run); int8 accumulates exactly
 * in int32 (the caller keeps |C| < 2^31).  Metadata nibbles must be valid
 * (as produced by ssg_compress_2to4); invalid ones give unspecified values
 * in the affected outputs, never out-of-bounds accesses. */
int ssg_spmm_2to4(int ab, int c, int64_t M, int64_t N, int64_t K,
                  const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                  const void* B, int64_t ldb, void* C, int64_t ldc,
                  void* ws, size_t ws_bytes, void* stream);

/* C = (expand(vals, meta) + residual) x B.  nnz_r must equal row_ptr[M]
 * (it sizes nothing on the device; it selects the launch shape and is
 * trusted).  Column indices must lie in [0, K). */
int ssg_spmm_2to4_residual(int ab, int c, int64_t M, int64_t N, int64_t K,
                           const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                           const int32_t* row_ptr, const int32_t* col, const void* rvals,
                           int64_t nnz_r, const void* B, int64_t ldb, void* C, int64_t ldc,
                           void* ws, size_t ws_bytes, void* stream);

/* Delta-coded residual: the residual CSR with each column index replaced by
 * a one-byte gap, decoded on the GPU by a running sum.  "How sparse LLM
 * weights cut GPU inference cost without quantization", section "How the
 * three-layer format makes moderate sparsity fast", names a differential
 * position code for the sparse layers that is decoded in parallel on chip;
 * it gives no layout, and this one is the library's own:
 *   drow_ptr int32 [M+1], drow_ptr[0] = 0, row m = entries
 *            [drow_ptr[m], drow_ptr[m+1]);
 *   dcol     uint8 [n]: entry j of a row stores col_j - col_(j-1), with
 *            col_(-1) = -1, a value in [1, 255];
 *   dvals    [n] in the element type of A.
 * A gap above 255 is bridged by filler entries (dcol 255, dvals +0) placed in
 * front of the entry, floor((gap - 1) / 255) of them.  An entry costs 1 + s
 * bytes (s = element size) instead of the CSR's 4 + s; fillers appear only
 * where a row's residual columns lie more than 255 apart.
 *
 * Encoding, pass 1: drow_ptr from a CSR whose columns ascend strictly
 * within [0, K) in every row; nnz_r = row_ptr[M] (trusted, as for the
 * products).  A CSR outside that contract gives an unspecified code but no
 * out-of-bounds access: entries are clamped to [0, nnz_r), columns to
 * [0, K - 1], and a gap below 1 counts as 1.  The caller reads drow_ptr[M]
 * to size dcol and dvals.  Fails with SSG_ERR_SHAPE when the worst case,
 * nnz_r + M * (K / 255 + 1) entries, exceeds 2^31 - 1. */
int ssg_residual_delta_count(int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col, int64_t nnz_r,
                             int32_t* drow_ptr, void* stream);

/* Encoding, pass 2: dcol and dvals (values bit-copied, fillers +0) at the
 * positions drow_ptr (from pass 1 on the same CSR) gives.  Writes stay
 * inside each row's [drow_ptr[m], drow_ptr[m+1]). */
int ssg_residual_delta_fill(int dt, int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col,
                            const void* rvals, int64_t nnz_r, const int32_t* drow_ptr, uint8_t* dcol, void* dvals,
                            void* stream);

/* C = (expand(vals, meta) + delta-coded residual) x B, as
 * ssg_spmm_2to4_residual.  nnz_d must equal drow_ptr[M] (trusted; it selects
 * the launch shape).  Decoded columns at or beyond K are skipped. */
int ssg_spmm_2to4_residual_delta(int ab, int c, int64_t M, int64_t N, int64_t K,
                                 const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                                 const int32_t* drow_ptr, const uint8_t* dcol, const void* dvals,
                                 int64_t nnz_d, const void* B, int64_t ldb, void* C, int64_t ldc,
                                 void* ws, size_t ws_bytes, void* stream);

/* Unstructured sparse x dense, the baseline the 2:4 format is weighed
 * against ("Chapter 26 -- Sparsity: The Hardware View", sections "Why
 * Hardware Wants Dense, Regular Data" and "The Honest Numbers on
 * Unstructured Sparsity"): C = S x B for a sparse S [M, K] given as a CSR
 * (row_ptr, col ascending within each row, vals) or delta-coded (as
 * above), with no 2:4 layer.  Same (input, output) pairs and accumulation
 * as ssg_spmm_2to4; nnz / nnz_d must equal the last row pointer (trusted).
 * N <= 16 with B a contiguous K x 16 block runs on the small-N kernel,
 * anything else on the generic one. */
int ssg_spmm_csr(int ab, int c, int64_t M, int64_t N, int64_t K, const int32_t* row_ptr, const int32_t* col,
                 const void* vals, int64_t nnz, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);
int ssg_spmm_csr_delta(int ab, int c, int64_t M, int64_t N, int64_t K, const int32_t* drow_ptr, const uint8_t* dcol,
                       const void* dvals, int64_t nnz_d, const void* B, int64_t ldb, void* C, int64_t ldc,
                       void* stream);

/* Packed decode layout: the 2:4 operand rearranged, offline like the
 * compression, into the order the small-N kernel consumes it, for
 * bandwidth-bound decode products ("Chapter 26 -- Sparsity: The Hardware
 * View", section "2:4 in the Memory-Bound Regime": there the bytes streamed
 * set the time).  For each 16-row tile and k-step (64 dense k for
 * fp16/bf16, 128 for int8): pvals holds one 1 KiB block, lane l = 16q + r
 * of the sparse MFMA carrying row r's 16 stored-value bytes
 * [16q, 16q + 16) of the k-step; pmeta holds one block of 64 index words,
 * lane l's being row r's metadata bytes [2q, 2q + 2) (fp16/bf16) or
 * [4q, 4q + 4) (int8) of the k-step.  Tiles follow each other, a tile's
 * blocks are consecutive in k, rows past M are zero.  The same bytes as
 * (vals, meta), only reordered.
 *
 * ssg_packed_sizes: bytes of pvals and pmeta.  K must be a multiple of the
 * k-step (SSG_ERR_SHAPE otherwise). */
int ssg_packed_sizes(int dt, int64_t M, int64_t K, int64_t* vals_bytes, int64_t* meta_bytes);

/* Pack (vals, meta) (rows 16-byte aligned) into caller-allocated pvals and
 * pmeta of ssg_packed_sizes() bytes. */
int ssg_pack_2to4_decode(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                         int64_t ldm, void* pvals, void* pmeta, void* stream);

/* C = expand(packed) x B for N == 16 with B one contiguous K x 16 block
 * (ldb == 16, 16-byte aligned); pvals 16-byte aligned, pmeta aligned to
 * its index words.  Other N give SSG_ERR_ALGO.  Accumulation as
 * ssg_spmm_2to4. */
int ssg_spmm_2to4_packed(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                         const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);

/* The same product with B given as its transpose: Bt [N, K] row-major (row
 * stride ldbt >= K elements), the token-major layout in which a decode
 * step's activations arrive, for any 1 <= N <= 16 (no padding).  Each lane
 * of the kernel loads its B operand straight into registers as two 16-byte
 * pieces of one row of Bt, instead of staging B through LDS.  The result has
 * the same bits as ssg_spmm_2to4_packed on B = Bt^T (N == 16).  Needs Bt
 * 16-byte aligned, rows a multiple of 16 bytes apart (SSG_ERR_STRIDE
 * otherwise) and 16 * ldbt elements within 31-bit byte offsets
 * (SSG_ERR_SHAPE); N outside [1, 16] gives SSG_ERR_ALGO, N == 0 is a
 * no-op. */
int ssg_spmm_2to4_packed_bt(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                            const void* Bt, int64_t ldbt, void* C, int64_t ldc, void* stream);

/* The same product plus a residual layer ("How sparse LLM weights cut GPU
 * inference cost without quantization", section "How the three-layer
 * format makes moderate sparsity fast"): C = expand(packed) x B + R x B,
 * with R as in ssg_spmm_2to4_residual (CSR, int32 columns) or
 * ssg_spmm_2to4_residual_delta (one-byte gaps).  The residual arrays
 * (col or dcol, and the values) must be aligned to 4 entries and under 2^31
 * bytes (SSG_ERR_ALGO otherwise); row pointers are trusted as there. */
int ssg_spmm_2to4_packed_residual(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals,
                                  const void* pmeta, const int32_t* row_ptr, const int32_t* col, const void* rvals,
                                  int64_t nnz_r, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);
int ssg_spmm_2to4_packed_residual_delta(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals,
                                        const void* pmeta, const int32_t* drow_ptr, const uint8_t* dcol,
                                        const void* dvals, int64_t nnz_d, const void* B, int64_t ldb, void* C,
                                        int64_t ldc, void* stream);

/* Packed prefill layout: the 2:4 operand rearranged, offline like the
 * compression, into the order the large-N (compute-bound) kernel stages it
 * in LDS, so that every load of stored values or metadata is one contiguous
 * piece ("Chapter 26 -- Sparsity: The Hardware View", section "2:4: ~2x on
 * the Matmul, Less End-to-End": in the compute-bound regime the doubled
 * sparse matrix rate pays only if the operands keep up).  Rows are grouped in tiles of 256; a stage is
 * 64 stored-value bytes of a row (64 dense k for fp16/bf16, 128 for the
 * 8-bit types); a metadata block is 32 metadata bytes of a row (256 dense k).
 *   pvals: tile t, stage s -> 16 KiB block (t * stages + s) of 1024
 *          16-byte lane chunks.  The 16-byte chunk c < 4 of row
 *          r = 32 rt + rl of the tile (stored-value bytes [64 s + 16 c, +16)
 *          of the row; rt < 8, rl < 32) sits at chunk
 *          (2 rt + c / 2) * 64 + 32 (c % 2) + rl.
 *   pmeta: tile t, block g -> 8 KiB block (t * mblocks + g) of 512
 *          16-byte lane chunks.  With IW = 2 (fp16/bf16) or 4 (8-bit types)
 *          and KPC = 4 / IW, metadata byte 32 g + j of row r of the tile
 *          (j < 32: k-step h = j / (2 IW), half q = (j / IW) % 2, byte
 *          e = j % IW of its index word; r = 128 wm + 32 i + rl with
 *          i < 4, rl < 32) sits in chunk ((h / KPC) * 2 + wm) * 64 + 32 q + rl
 *          at byte ((h % KPC) * 4 + i) * IW + e.
 * stages = K / 64 (fp16/bf16) or K / 128 (8-bit); mblocks = ceil(K / 256).
 * Rows past M and metadata bytes past K / 8 hold zeros.  The same bytes as
 * (vals, meta), only reordered.
 *
 * ssg_prefill_packed_sizes: bytes of pvals and pmeta.  K must be a multiple
 * of the stage (SSG_ERR_SHAPE otherwise). */
int ssg_prefill_packed_sizes(int dt, int64_t M, int64_t K, int64_t* vals_bytes, int64_t* meta_bytes);

/* Prune and compress A (as ssg_compress_2to4) straight into the packed
 * prefill layout: caller-allocated pvals (16-byte aligned) and pmeta (4-byte
 * aligned) of ssg_prefill_packed_sizes() bytes, every byte written. */
int ssg_compress_2to4_prefill(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* pvals, void* pmeta,
                              void* stream);

/* Pack (vals, meta) (vals rows 16-byte aligned) into the packed prefill
 * layout; the result equals ssg_compress_2to4_prefill of the dense matrix. */
int ssg_pack_2to4_prefill(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                          int64_t ldm, void* pvals, void* pmeta, void* stream);

/* C = expand(packed prefill) x B on the large-N kernel, with the pairs and
 * accumulation of ssg_spmm_2to4.  Needs N a multiple of 8 (16-bit) or 16
 * (8-bit), B rows 16-byte aligned (SSG_ERR_ALGO otherwise), K > 0. */
int ssg_spmm_2to4_prefill(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                          const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);

/* The same product with B given as its transpose: Bt [N, K] row-major
 * (row stride ldbt >= K elements), the token-major layout in which a
 * linear layer's activations arrive (C = W X^T for activations X = Bt).
 * Each column of B is then a contiguous row, which the large-N kernel reads
 * in 16-byte pieces (half the LDS reads per B operand of the row-major
 * form); the result has the same bits as ssg_spmm_2to4_prefill with
 * B = Bt^T.  Needs Bt 16-byte aligned with rows a multiple of 16 bytes, and
 * 256 * ldbt elements within 31-bit byte offsets (SSG_ERR_ALGO otherwise);
 * any N >= 0. */
int ssg_spmm_2to4_prefill_bt(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals, const void* pmeta,
                             const void* Bt, int64_t ldbt, void* C, int64_t ldc, void* stream);

/* N:M patterns other than 2:4 ("Chapter 26 -- Sparsity: The Hardware View",
 * section "Block Sparsity, N:M Generalizations, and Channel Pruning", which
 * lists 1:4, 2:8 and 4:8 and gives no selection rule or storage; what
 * follows is this library's reading).  (nm_n, nm_m) is one of (1, 4),
 * (2, 4), (2, 8), (4, 8) (else SSG_ERR_SHAPE); K % nm_m == 0.
 *
 * Selection: in each group of nm_m consecutive elements along K, position
 * p is kept iff fewer than nm_n other positions outrank it (the 2:4 rule
 * above with nm_n in place of two).
 * Layout:
 *   vals  [M, K/nm_m*nm_n] kept values, group g at columns
 *         g*nm_n .. g*nm_n+nm_n-1 in ascending position order
 *         (ldv >= K/nm_m*nm_n);
 *   mask  [M, ceil(K/8)] uint8, bit k%8 of byte k/8 set iff element k is
 *         kept; bits past K are 0 (ldmask >= ceil(K/8)).
 * For 2:4 this holds the same values as ssg_compress_2to4 with the
 * positions as bits instead of nibbles.
 *
 * 4-bit weights (SSG_I4; "Chapter 26", section "Sparsity + Quantization
 * Combine", stacks 2:4 with 4-bit values): two's-complement integers in
 * [-8, 7], two per byte, element k of a row in the low nibble of byte k/2
 * for even k and the high nibble for odd k; A, vals and D are byte arrays
 * whose leading dimensions stay counted in elements and must be even.
 * Patterns 2:4, 2:8, 4:8 (whole bytes per group).  The products take them
 * as weight-only quantized weights: B is fp16, C fp32 ((ab, c) =
 * (SSG_I4, SSG_F32)); the values enter the fp16 MFMA exactly.
 *
 * ssg_nm_vals_cols: K / nm_m * nm_n. */
int64_t ssg_nm_vals_cols(int nm_n, int nm_m, int64_t K);

/* (vals, mask) = the N:M form of A (values bit-copied). */
int ssg_compress_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* A, int64_t lda,
                    void* vals, int64_t ldv, uint8_t* mask, int64_t ldmask, void* stream);

/* D = dense expansion of (vals, mask): each group's stored values at its
 * mask bits in ascending order, +0 elsewhere.  A group whose mask does not
 * hold exactly nm_n bits is written as zeros and, if bad_count is not NULL,
 * counted into the device int32 *bad_count (added atomically). */
int ssg_decompress_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                      const uint8_t* mask, int64_t ldmask, void* D, int64_t ldd, int32_t* bad_count,
                      void* stream);

/* C = expand_nm(vals, mask) x B on the dense MFMA (gfx950 has no sparse form
 * for these patterns; the stored operand is expanded in registers, so the
 * gain is the bytes streamed, which set the time of decode shapes).  (ab, c)
 * as ssg_spmm_2to4.  Alignment: vals 16-byte aligned and ldv * element size
 * a multiple of 16; mask 8-byte aligned and ldmask a multiple of 8; B
 * 16-byte aligned and ldb * element size a multiple of 16 (strides are only
 * checked where there is more than one row), else SSG_ERR_STRIDE.  Any N
 * (one workgroup column per 16 columns of B, at most 65535 of them).
 * K == 0 zero-fills C.  Accumulation as ssg_spmm_2to4.  A mask group with
 * the wrong number of bits gives unspecified values in its row's outputs,
 * never out-of-bounds accesses. */
int ssg_spmm_nm(int ab, int c, int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                const uint8_t* mask, int64_t ldmask, const void* B, int64_t ldb, void* C, int64_t ldc,
                void* stream);

/* Packed decode layout of the N:M operand, made offline like the
 * compression: for each 16-row tile and super-step (4*D dense k, with
 * D = 16 / element size * nm_m / nm_n: the k one 16-byte load of stored
 * values covers), pvals holds one 1 KiB block in which lane l = 16q + r
 * carries row r's stored bytes [64g + 16q, 64g + 16q + 16) of super-step g,
 * and pmask one block of 64 * D/8 bytes, lane l's being row r's mask bytes
 * [g*D/2 + q*D/8, +D/8).  Tiles follow each other, a tile's blocks are
 * consecutive in g; bytes past a row's end and rows past M are zero.  The
 * same bytes as (vals, mask), reordered, so every load of the product is
 * one coalesced block.
 *
 * ssg_nm_packed_sizes: bytes of pvals and pmask. */
int ssg_nm_packed_sizes(int dt, int nm_n, int nm_m, int64_t M, int64_t K, int64_t* vals_bytes,
                        int64_t* mask_bytes);

/* Pack (vals, mask) into caller-allocated pvals (16-byte aligned) and pmask
 * (8-byte aligned) of ssg_nm_packed_sizes() bytes. */
int ssg_pack_nm_decode(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                       const uint8_t* mask, int64_t ldmask, void* pvals, void* pmask, void* stream);

/* C = expand_nm(packed) x B, as ssg_spmm_nm (B alignment, any N, same
 * accumulation) with K > 0. */
int ssg_spmm_nm_packed(int ab, int c, int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* pvals,
                       const void* pmask, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);

/* As the SpMM calls above with an explicit algorithm (ssg_algo). */
int ssg_spmm_2to4_ex(int algo, int ab, int c, int64_t M, int64_t N, int64_t K,
                     const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                     const void* B, int64_t ldb, void* C, int64_t ldc,
                     void* ws, size_t ws_bytes, void* stream);
int ssg_spmm_2to4_residual_ex(int algo, int ab, int c, int64_t M, int64_t N, int64_t K,
                              const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                              const int32_t* row_ptr, const int32_t* col, const void* rvals,
                              int64_t nnz_r, const void* B, int64_t ldb, void* C, int64_t ldc,
                              void* ws, size_t ws_bytes, void* stream);
int ssg_spmm_2to4_residual_delta_ex(int algo, int ab, int c, int64_t M, int64_t N, int64_t K,
                                    const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                                    const int32_t* drow_ptr, const uint8_t* dcol, const void* dvals,
                                    int64_t nnz_d, const void* B, int64_t ldb, void* C, int64_t ldc,
                                    void* ws, size_t ws_bytes, void* stream);

/* The algorithm SSG_ALGO_AUTO would run for this problem and these pointers
 * and leading dimensions (alignment decides between fast and generic paths). */
int ssg_spmm_select_algo(int ab, int64_t M, int64_t N, int64_t K,
                         const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                         const void* B, int64_t ldb, const void* C, int64_t ldc);

/* For callers that cannot allocate device memory (code under HIP stream
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product as ssg_spmm_2to4 with algorithm AUTO, without a workspace
 * argument.  The one buffer the product may need -- B padded to 16 columns
 * when 0 < N < 16 -- comes from a file-scope device array of the library of
 * ssg_noalloc_scratch_bytes() = 2 MiB (K * 16 elements: K <= 65536 for
 * 16-bit types, 131072 for 8-bit ones); a larger padded B fails with
 * SSG_ERR_WORKSPACE and nothing is enqueued.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine).  Each device the
 * library runs on holds its own copy of the array until the process ends;
 * its address on a device is looked up on the first call there, with that
 * device current (the stream must belong to the current device).  Every
 * call on a device shares that device's array and overwrites what the
 * previous call left in it, so calls that may overlap on one device (on
 * different streams, or from different host threads) race. */
int64_t ssg_noalloc_scratch_bytes(void);
int ssg_spmm_2to4_noalloc(int ab, int c, int64_t M, int64_t N, int64_t K,
                          const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                          const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);

/* Complement-bitmap residual: the residual layer in the packed decode
 * product's block order, fused into its k-steps.  "How sparse LLM weights cut
 * GPU inference cost without quantization", section "How the three-layer
 * format makes moderate sparsity fast", keeps what the 2:4 layer drops in a
 * residual layer decoded on chip in the same pipeline, and gives no layout;
 * this one is the library's own.  It rests on one fact of the split: in a
 * group where the 2:4 layer kept positions i0 < i1, a residual entry can
 * only sit at one of the two other positions c0 < c1 (the complement
 * positions).  With the packed decode geometry (16-row tiles, k-steps of KS
 * = 64 dense columns for 16-bit types and 128 for 8-bit ones; block
 * b = t * (K / KS) + g; lane l = 16q + r of block (t, g) = row 16t + r and
 * dense columns [g*KS + q*KS/4, g*KS + (q+1)*KS/4), i.e. KS/16 groups):
 *   rmask  per block, 64 lanes x MB bytes (MB = 1 for 16-bit types, 2 for
 *          8-bit), lane-major; a lane's MB bytes are one little-endian word
 *          whose bit 2*gi + j is set iff the residual holds a value at
 *          complement position c_j of the lane's group gi (groups in
 *          ascending column order); rows past M have no bits;
 *   roff   int32 [blocks + 1]: roff[b] = values in the blocks before b,
 *          roff[blocks] = all of them;
 *   cvals  the values, bit-copied, in block, then lane, then bit order.
 * Bytes: MB*64 + 4 per block plus s per entry, against 4 + s per entry for
 * the CSR.  For a lane the residual is itself a 2:4 operand (its values at
 * the complement positions, zeros elsewhere) whose index word is the
 * complement of the 2:4 layer's, so the product adds one sparse MFMA per
 * tile and k-step on the same B operand.
 *
 * Sizes: mask bytes and blocks (roff holds blocks + 1 entries).  K must be a
 * multiple of KS. */
int ssg_cbm_sizes(int dt, int64_t M, int64_t K, int64_t* mask_bytes, int64_t* blocks);

/* Encoding from the CSR residual of ssg_split_fill (columns strictly
 * ascending within [0, K) in every row) and the row-major metadata of the
 * same 2:4 layer.  cvals holds nnz_r values (16-byte aligned for the
 * product).  An entry at a kept position of its group, in a group with an
 * invalid nibble, or repeating a column is left out and, if bad_count is
 * not NULL, counted into the device int32 *bad_count (added atomically; the
 * caller zeroes it); roff[blocks] then falls short of nnz_r.  Other
 * violations of the CSR contract give an unspecified code but no
 * out-of-bounds access. */
int ssg_pack_residual_cbm(int dt, int64_t M, int64_t K, const uint8_t* meta, int64_t ldm,
                          const int32_t* row_ptr, const int32_t* col, const void* rvals, int64_t nnz_r,
                          uint8_t* rmask, int32_t* roff, void* cvals, int32_t* bad_count, void* stream);

/* C = (expand(packed decode layout) + residual) x B, the residual in the
 * complement-bitmap layout above, fused into every k-step.  Shapes, types
 * and the packed operand as for ssg_spmm_2to4_packed (N == 16, ldb == 16).
 * nvals is the number of values cvals holds (at least roff[blocks]; it bounds
 * the loads).  Alignment: pvals, B and cvals 16 bytes; pmeta and rmask to
 * their words; roff 4 bytes. */
int ssg_spmm_2to4_packed_residual_cbm(int ab, int c, int64_t M, int64_t N, int64_t K,
                                      const void* pvals, const void* pmeta, const uint8_t* rmask,
                                      const int32_t* roff, const void* cvals, int64_t nvals,
                                      const void* B, int64_t ldb, void* C, int64_t ldc, void* stream);

/* The same with B given as Bt [N, K] row-major, 1 <= N <= 16, under the
 * conditions of ssg_spmm_2to4_packed_bt. */
int ssg_spmm_2to4_packed_residual_cbm_bt(int ab, int c, int64_t M, int64_t N, int64_t K, const void* pvals,
                                         const void* pmeta, const uint8_t* rmask, const int32_t* roff,
                                         const void* cvals, int64_t nvals, const void* Bt, int64_t ldbt, void* C,
                                         int64_t ldc, void* stream);

/* Measurement helper (not part of the product): one streaming read of
 * `bytes` bytes of device memory at src (16-byte aligned, bytes a multiple
 * of 16), 16 bytes per lane per load, non-temporal, every byte once.  Its
 * rate is the achievable read bandwidth the bandwidth-bound products ("2:4 in
 * the Memory-Bound Regime" of "Chapter 26 -- Sparsity: The Hardware View":
 * the bytes streamed set the time) are compared against.  sink is device
 * memory of ssg_stream_read_sink_words(bytes) uint32 words; it is written
 * only when a workgroup's fold of the data hits one fixed value, which keeps
 * the loads from being optimised away. */
int64_t ssg_stream_read_sink_words(int64_t bytes);
int ssg_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/* Measurement helper (not part of the product): the issue rate of one
 * matrix-core instruction form, the ceiling of the compute-bound products
 * and the measure for the choice between the sparse MFMA and a decode of
 * the compressed operand to dense followed by the dense MFMA ("Chapter 26
 * -- Sparsity: The Hardware View", section "2:4: ~2x on the Matmul, Less
 * End-to-End": the sparse unit doubles the math rate of the matmul).
 * Forms 0 .. ssg_mfma_probe_forms()-1, named by ssg_mfma_probe_name (NULL
 * outside that range): sparse and dense bf16 at 32x32 and 16x16, the same
 * for int8, then sparse and dense fp8 (E4M3) at 32x32.  One launch is
 * `workgroups` workgroups of four 64-lane waves; every wave runs `iters`
 * rounds of independent accumulators through the one instruction, with
 * operands from a hash of its lane.  ssg_mfma_probe_ops gives the launch's
 * dense-equivalent operation count (2 * rows * columns * dense k per
 * instruction; 0 for an invalid form or a non-positive count), so that
 * count over the launch's time is the rate.  sink is device memory of
 * `workgroups` uint32 words, written only when a workgroup's fold of its
 * accumulators hits one fixed value.  Errors: SSG_ERR_ALGO for an invalid
 * form, SSG_ERR_SHAPE for non-positive counts, SSG_ERR_NULL for no sink. */
int ssg_mfma_probe_forms(void);
const char* ssg_mfma_probe_name(int form);
int64_t ssg_mfma_probe_ops(int form, int64_t workgroups, int64_t iters);
int ssg_mfma_probe(int form, int64_t workgroups, int64_t iters, uint32_t* sink, void* stream);

/* Measurement helper (not part of the product): the rate of 16-byte LDS
 * reads (ds_read_b128) for one pattern of per-lane addresses, the measure
 * behind the LDS images of the large-N kernel, whose operand reads must
 * keep up with the sparse matrix unit ("Chapter 26 -- Sparsity: The
 * Hardware View", section "2:4: ~2x on the Matmul, Less End-to-End").
 * offsets: host array of 64 byte offsets, each a multiple of 16 and at most
 * 65536 - 7 * 4096 - 16 = 36848.  One launch is `workgroups` workgroups of
 * four 64-lane waves, each with 64 KiB of LDS; lane l of every wave reads
 * the 16 bytes at offsets[l] + 4096 j for j < 8, `iters` times (8 * iters
 * reads per wave).  sink is device memory of `workgroups` uint32 words,
 * written only when a workgroup's fold of the data hits one fixed value.
 * Errors: SSG_ERR_NULL for no offsets or sink, SSG_ERR_SHAPE for
 * non-positive counts or an offset that is misaligned or too large. */
int ssg_lds_read_probe(const uint32_t* offsets, int64_t workgroups, int64_t iters, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSGEMM_H */
