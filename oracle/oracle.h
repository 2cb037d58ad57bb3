/*
 * oracle.h -- plain, slow, obviously-correct CPU reference for 2:4
 * structured-sparse compression and sparse x dense matrix multiply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no source, header, table or
 * helper with the GPU library.
 *
 * Sources (the pages this follows):
 *   [P3] "Chapter 26 -- Sparsity: The Hardware View" (karam-nus.github.io),
 *        section "2:4 Fine-Grained Structured Sparsity" (worked example of an
 *        8-weight row, its compressed values and 2-bit indices) and the first
 *        Python listing of section "Python: Build a 2:4 Mask, Compress It ..."
 *        (keep the two largest magnitudes of every group of 4 along the last
 *        dimension; kept positions sorted ascending; values gathered).
 *   [P2] "10.4g Structured Sparsity (2:4)" (aikaboom.com), sections
 *        "What is 2:4 Structured Sparsity?" and "How Tensor Cores Leverage
 *        This Pattern" (compressed = non-zero values plus their indices).
 *   [P4] "How sparse LLM weights cut GPU inference cost without quantization"
 *        (groundy.com), section "How the three-layer format makes moderate
 *        sparsity fast" (a residual layer carries what the structured layer
 *        dropped, so the product stays exact).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes):
 *   - exactly two slots are stored per group; a stored slot may hold a zero;
 *   - magnitude ties go to the lower position;
 *   - nibble of a group = i0 | (i1 << 2) with i0 < i1; group 2j sits in the
 *     low nibble of metadata byte j; a row has ceil(K/8) metadata bytes;
 *   - the residual is the set of numerically non-zero elements the top-2
 *     selection dropped, stored as CSR (int32 row_ptr/col, col ascending);
 *   - fp16/bf16 products are accumulated in fp64, int8 in int64;
 *   - the compact residual position code ([P4], same section, names one and
 *     gives no layout) is this library's own delta code, defined at
 *     orc_delta_count below.
 *
 * Element types: ORC_F16 (IEEE-754 binary16), ORC_BF16 (bfloat16),
 * ORC_I8 (two's-complement int8), ORC_E4M3 / ORC_E5M2 (OCP 8-bit floats;
 * [P3] section "Sparsity + Quantization Combine" stacks 2:4 with
 * 8-bit formats).  All matrices are row-major with an
 * explicit leading dimension in elements.  Return value 0 = success,
 * negative = invalid argument (see ORC_E* below); nothing is ever allocated
 * on behalf of the caller except internal scratch freed before return.
 */
#ifndef SSG_ORACLE_H
#define SSG_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_I8 = 2, ORC_E4M3 = 3, ORC_E5M2 = 4, ORC_I4 = 5 };
enum { ORC_OK = 0, ORC_ENULL = -1, ORC_ESHAPE = -2, ORC_ESTRIDE = -3, ORC_EDTYPE = -4,
       ORC_ENONFINITE = -5, ORC_EFORMAT = -6, ORC_ENOMEM = -7, ORC_ERANGE = -8 };

/* Exact value of a binary16 / bfloat16 bit pattern (NaN -> NaN, Inf -> Inf). */
double orc_f16_to_f64(uint16_t bits);
double orc_bf16_to_f64(uint16_t bits);
/* Exact value of an 8-bit float (OCP FP8): E4M3 (bias 7, no infinities,
 * S.1111.111 is NaN) and E5M2 (bias 15, IEEE-style infinities and NaNs). */
double orc_e4m3_to_f64(uint8_t bits);
double orc_e5m2_to_f64(uint8_t bits);
/* ORC_I4: 4-bit two's-complement integers (-8..7), two per byte, element i
 * in the low nibble of byte i/2 for even i and the high nibble for odd i
 * ([P3] "Sparsity + Quantization Combine" stacks 2:4 with 4-bit weights).
 * Only the N:M functions below take it, as the weight; leading dimensions
 * stay counted in elements and must be even.  orc_i4_to_f64: the value of
 * the low (high = 0) or high nibble of a byte. */
double orc_i4_to_f64(uint8_t byte, int high);

/* Top-2 of a group of 4 magnitudes, ties to the lower position:
 * keep[p] = 1 iff fewer than two other positions q outrank p, where q outranks
 * p when mag[q] > mag[p], or mag[q] == mag[p] and q < p. */
void orc_select_group(const double mag[4], int keep[4]);

/* Compress A[M,K] (K % 4 == 0) into vals[M, K/2] and meta[M, ceil(K/8)]. */
int orc_compress(int dt, int64_t M, int64_t K, const void* A, int64_t lda,
                 void* vals, int64_t ldv, uint8_t* meta, int64_t ldm);

/* Dense pruned copy: P = A where kept (bit copy), +0 elsewhere. */
int orc_prune(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* P, int64_t ldp);

/* Expand vals/meta back to dense D.  Groups whose nibble is not one of
 * {0x4,0x8,0xC,0x9,0xD,0xE} are written as zeros and counted.  Returns the
 * count (>= 0) or a negative error. */
int64_t orc_decompress(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv,
                       const uint8_t* meta, int64_t ldm, void* D, int64_t ldd);

/* Residual split, pass 1: row_ptr[0] = 0, row_ptr[m+1] = row_ptr[m] + number of
 * non-zero elements of row m that the top-2 selection dropped. */
int orc_split_count(int dt, int64_t M, int64_t K, const void* A, int64_t lda, int32_t* row_ptr);

/* Residual split, pass 2: writes the 2:4 layer (as orc_compress) and the CSR
 * residual (col ascending within a row, rvals bit copies of A). */
int orc_split_fill(int dt, int64_t M, int64_t K, const void* A, int64_t lda,
                   void* vals, int64_t ldv, uint8_t* meta, int64_t ldm,
                   const int32_t* row_ptr, int32_t* col, void* rvals);

/* Delta-coded residual, pass 1.  Input: a CSR with columns strictly
 * ascending within [0, K) in every row (else ORC_EFORMAT).  Per row, in CSR
 * order, entry j is stored as the byte d_j = col_j - col_(j-1), col_(-1) = -1;
 * a gap above 255 is bridged by filler entries (d = 255, value +0) placed
 * before the entry, floor((gap - 1) / 255) of them, which leaves d_j in
 * [1, 255].  drow_ptr[0] = 0, drow_ptr[m+1] = drow_ptr[m] + entries of row m
 * including fillers. */
int orc_delta_count(int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col, int32_t* drow_ptr);

/* Delta-coded residual, pass 2: dcol[] (bytes) and dvals[] (bit copies of
 * rvals, +0 for fillers) at the positions drow_ptr gives. */
int orc_delta_fill(int dt, int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col, const void* rvals,
                   const int32_t* drow_ptr, uint8_t* dcol, void* dvals);

/* C[m,n] = sum_k D[m,k] * B[k,n] over k ascending, D = decompress(vals, meta),
 * B[K,N] row-major.  fp16/bf16: Cf (fp64) and the bound S[m,n] = sum_k
 * |D[m,k] B[k,n]| (S may be NULL).  int8: Ci (int64).  Rows run in parallel
 * when built with OpenMP.  A bad nibble is an error (ORC_EFORMAT). */
int orc_spmm(int dt, int64_t M, int64_t N, int64_t K,
             const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
             const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S, int64_t ldc);

/* As orc_spmm on D = decompress(vals, meta) + scatter(residual CSR). */
int orc_spmm_residual(int dt, int64_t M, int64_t N, int64_t K,
                      const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                      const int32_t* row_ptr, const int32_t* col, const void* rvals,
                      const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S, int64_t ldc);

/* As orc_spmm_residual with the residual delta-coded: entry j of row m adds
 * dvals[j] at column -1 + the sum of dcol over the row's entries up to j. */
int orc_spmm_residual_delta(int dt, int64_t M, int64_t N, int64_t K,
                            const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                            const int32_t* drow_ptr, const uint8_t* dcol, const void* dvals,
                            const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S, int64_t ldc);

/* Unstructured sparse x dense: C[m,n] = sum over row m's CSR entries j of
 * vals[j] * B[col[j], n], in CSR order (fp64 with the bound S; int64 for
 * int8).  Columns must lie in [0, K) (else ORC_EFORMAT). */
int orc_spmm_csr(int dt, int64_t M, int64_t N, int64_t K, const int32_t* row_ptr, const int32_t* col,
                 const void* vals, const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S, int64_t ldc);

/* Selected outputs only: for e < n_entries, (m, n) = (ms[e], ns[e]); writes
 * Cf[e]/Ci[e] and S[e].  row_ptr may be NULL (no residual). */
int orc_spmm_entries(int dt, int64_t M, int64_t N, int64_t K,
                     const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                     const int32_t* row_ptr, const int32_t* col, const void* rvals,
                     const void* B, int64_t ldb, int64_t n_entries,
                     const int64_t* ms, const int64_t* ns, double* Cf, int64_t* Ci, double* S);

/* As orc_spmm_entries with a delta-coded residual (drow_ptr not NULL). */
int orc_spmm_entries_delta(int dt, int64_t M, int64_t N, int64_t K,
                           const void* vals, int64_t ldv, const uint8_t* meta, int64_t ldm,
                           const int32_t* drow_ptr, const uint8_t* dcol, const void* dvals,
                           const void* B, int64_t ldb, int64_t n_entries,
                           const int64_t* ms, const int64_t* ns, double* Cf, int64_t* Ci, double* S);

/* N:M generalization ([P3] section "Block Sparsity, N:M Generalizations,
 * and Channel Pruning"; selection and storage are this library's reading).
 * 1 <= nm_n < nm_m <= 16, K % nm_m == 0.
 *
 * orc_select_nm: keep[p] = 1 iff fewer than nm_n other positions q outrank
 * p (mag[q] > mag[p], or equal and q < p).
 * orc_compress_nm: vals[M, K/nm_m*nm_n] holds the kept values of group g at
 * columns g*nm_n .. g*nm_n+nm_n-1 in ascending position order;
 * mask[M, ceil(K/8)] has bit k%8 of byte k/8 set iff element k is kept.
 * orc_decompress_nm: dense expansion; groups whose mask does not hold exactly
 * nm_n bits are written as zeros and counted (the count is returned).
 * orc_spmm_nm: as orc_spmm on the expansion (ORC_EFORMAT on a bad group). */
void orc_select_nm(int nm_n, int nm_m, const double* mag, int* keep);
int orc_compress_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* A, int64_t lda,
                    void* vals, int64_t ldv, uint8_t* mask, int64_t ldmask);
int64_t orc_decompress_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                          const uint8_t* mask, int64_t ldmask, void* D, int64_t ldd);
int orc_spmm_nm(int dt, int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                const uint8_t* mask, int64_t ldmask, const void* B, int64_t ldb, double* Cf, int64_t* Ci, double* S,
                int64_t ldc);
/* Weight-only 4-bit: the N:M operand holds ORC_I4 values, B is fp16; the
 * product is summed in fp64 with the bound S, as orc_spmm_nm for floats. */
int orc_spmm_nm_w4a16(int nm_n, int nm_m, int64_t M, int64_t N, int64_t K, const void* vals, int64_t ldv,
                      const uint8_t* mask, int64_t ldmask, const void* B, int64_t ldb, double* Cf, double* S,
                      int64_t ldc);

/* Number of threads an OpenMP parallel region would use (1 without OpenMP). */
/* Complement-bitmap residual in the decode product's block order (layout
 * at orc_cbm_encode in oracle.c): sizes (mask bytes and blocks; roff holds
 * blocks + 1 entries), the encoding of a CSR residual whose entries sit at
 * the complement positions of the 2:4 layer's groups (any other entry:
 * ORC_EFORMAT), and the decoding back to CSR (columns ascending). */
int orc_cbm_sizes(int dt, int64_t M, int64_t K, int64_t* mask_bytes, int64_t* blocks);
int orc_cbm_encode(int dt, int64_t M, int64_t K, const uint8_t* meta, int64_t ldm, const int32_t* row_ptr,
                   const int32_t* col, const void* rvals, uint8_t* rmask, int32_t* roff, void* cvals);
int orc_cbm_decode(int dt, int64_t M, int64_t K, const uint8_t* meta, int64_t ldm, const uint8_t* rmask,
                   const int32_t* roff, const void* cvals, int32_t* row_ptr, int32_t* col, void* rvals);

int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
