// ssg_kernels.hpp -- host-side launchers of the HIP kernels (internal to
// libssgemm; the public surface is include/ssgemm.h).  Every launcher
// enqueues on stream `s` and returns the launch status; the caller has
// validated sizes, strides and pointers.  `vec` = operands are aligned for
// 16-byte vector accesses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssg {

// DT_E4M3 / DT_E5M2: OCP 8-bit floats (sign, 4/5 exponent bits with bias
// 7/15, 3/2 fraction bits), products accumulated in fp32.
// DT_I4: 4-bit two's-complement weights, two per byte (low nibble first),
// taken by the N:M kernels only, against fp16 activations.
enum Dtype { DT_F16 = 0, DT_BF16 = 1, DT_I8 = 2, DT_E4M3 = 3, DT_E5M2 = 4, DT_I4 = 5 };

constexpr bool dt_is_fp8(int dt) { return dt == DT_E4M3 || dt == DT_E5M2; }
constexpr int dt_bytes(int dt) { return dt == DT_F16 || dt == DT_BF16 ? 2 : 1; }

hipError_t launch_compress(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* vals, int64_t ldv,
                           uint8_t* meta, int64_t ldm, bool vec, hipStream_t s);
hipError_t launch_prune(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* P, int64_t ldp, bool vec,
                        hipStream_t s);
hipError_t launch_decompress(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                             int64_t ldm, void* D, int64_t ldd, int32_t* bad, bool vec, hipStream_t s);
hipError_t launch_split_count(int dt, int64_t M, int64_t K, const void* A, int64_t lda, int32_t* row_ptr, bool vec,
                              hipStream_t s);
hipError_t launch_split_fill(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* vals, int64_t ldv,
                             uint8_t* meta, int64_t ldm, const int32_t* row_ptr, int32_t* col, void* rvals, bool vec,
                             hipStream_t s);
// Delta-coded residual from a CSR: pass 1 writes the scanned entry counts
// (fillers included) into drow_ptr, pass 2 the gap bytes and values.
hipError_t launch_delta_count(int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col, int64_t nnz,
                              int32_t* drow_ptr, hipStream_t s);
hipError_t launch_delta_fill(int dt, int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col,
                             const void* rvals, int64_t nnz, const int32_t* drow_ptr, uint8_t* dcol, void* dvals,
                             hipStream_t s);

// Sparse operand of one SpMM call.
struct SpmmArgs {
    int dt;                     // DT_F16 / DT_BF16 / DT_I8
    int64_t M, N, K;
    const void* vals; int64_t ldv;     // 2:4 layer (vals == nullptr: none, an
    const uint8_t* meta; int64_t ldm;  // unstructured product of the residual)
    const int32_t* row_ptr;     // residual (nullptr: none)
    const int32_t* col;         // CSR column indices, or nullptr when
    const uint8_t* dcol;        // the residual is delta-coded (gap bytes)
    const void* rvals;
    int64_t nnz_r;
    const void* B; int64_t ldb;
    void* C; int64_t ldc;       // fp32 or int32
    int b_pad16;                // B is the library's copy padded to 16 columns
                                // (readable past column N up to 16)
};

hipError_t launch_spmm_generic(const SpmmArgs& a, hipStream_t s);
// Residual-only pass: C += residual x B (C already holds the 2:4 product).
hipError_t launch_residual_add(const SpmmArgs& a, hipStream_t s);

// Fast paths.  `supported_*` say whether a problem fits the kernel family
// (shape, alignment); the launchers assume it does.
bool supported_small_n(const SpmmArgs& a);
hipError_t launch_spmm_small_n(const SpmmArgs& a, hipStream_t s);
// B [K, N] with N < 16 copied to out [K, 16] (zero columns past N).
hipError_t launch_pad_b(int dt, int64_t K, int64_t N, const void* B, int64_t ldb, void* out, hipStream_t s);
// Packed decode layout (see spmm_small_n.hip): pack from (vals, meta), and
// the product on it (B one contiguous K x 16 block, K a multiple of the
// k-step; a.vals / a.meta unused).
hipError_t launch_pack_decode(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                              int64_t ldm, void* pvals, void* pmeta, hipStream_t s);
hipError_t launch_spmm_packed(const SpmmArgs& a, const void* pvals, const void* pmeta, hipStream_t s);
// The same product with B given as Bt [N, K] row-major (a.B, a.ldb), N <= 16:
// each lane loads its B operand straight into registers.
hipError_t launch_spmm_packed_bt(const SpmmArgs& a, const void* pvals, const void* pmeta, hipStream_t s);
// Complement-bitmap residual (residual_cbm.hip): blocks and mask bytes of
// the layout, its encoder from a CSR residual and the 2:4 layer's row-major
// metadata, and the packed decode product with it fused into every k-step
// (B one contiguous K x 16 block; nvals = roff[blocks] values in cvals).
void cbm_geometry(int dt, int64_t M, int64_t K, int64_t* blocks, int64_t* mask_bytes);
hipError_t launch_pack_cbm(int dt, int64_t M, int64_t K, const uint8_t* meta, int64_t ldm, const int32_t* row_ptr,
                           const int32_t* col, const void* rvals, int64_t nnz, void* rmask, int32_t* roff,
                           void* cvals, int32_t* bad, hipStream_t s);
hipError_t launch_spmm_packed_cbm(const SpmmArgs& a, const void* pvals, const void* pmeta, const void* rmask,
                                  const int32_t* roff, const void* cvals, int64_t nvals, hipStream_t s);
// The same with B given as Bt [N, K] row-major (a.B, a.ldb), N <= 16.
hipError_t launch_spmm_packed_cbm_bt(const SpmmArgs& a, const void* pvals, const void* pmeta, const void* rmask,
                                  const int32_t* roff, const void* cvals, int64_t nvals, hipStream_t s);
// Inclusive scan of a[1..n] in place, a[0] = 0 (one workgroup).
hipError_t launch_scan_counts(int64_t n, int32_t* a, hipStream_t s);
bool supported_large_n(const SpmmArgs& a);          // pipelined kernel or the basic one
hipError_t launch_spmm_large_n(const SpmmArgs& a, hipStream_t s);
bool supported_large_n_basic(const SpmmArgs& a);
hipError_t launch_spmm_large_n_basic(const SpmmArgs& a, hipStream_t s);
// Packed prefill layout (see ssg_device.hpp): geometry, the compress pass
// that writes it directly, the pack from (vals, meta), and the large-N
// product on it (a.vals / a.meta are pvals / pmeta).
void prefill_geometry(int dt, int64_t M, int64_t K, int64_t* tiles, int64_t* stages, int64_t* mblocks);
hipError_t launch_compress_prefill(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* pvals,
                                   void* pmeta, bool vec, hipStream_t s);
hipError_t launch_pack_prefill(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                               int64_t ldm, void* pvals, void* pmeta, hipStream_t s);
bool supported_prefill_packed(const SpmmArgs& a);
hipError_t launch_spmm_prefill_packed(const SpmmArgs& a, hipStream_t s);
// The same product with B given as Bt [N, K] row-major (a.B, a.ldb).
bool supported_prefill_packed_bt(const SpmmArgs& a);
hipError_t launch_spmm_prefill_packed_bt(const SpmmArgs& a, hipStream_t s);

// N:M patterns other than 2:4 (spmm_nm.hip): kept values plus a keep mask
// (bit k%8 of byte k/8 of a row).  (n, m) in {(1,4), (2,4), (2,8), (4,8)}.
bool nm_pattern_supported(int n, int m);
hipError_t launch_compress_nm(int dt, int n, int m, int64_t M, int64_t K, const void* A, int64_t lda, void* vals,
                              int64_t ldv, uint8_t* mask, int64_t ldm, bool vec, hipStream_t s);
hipError_t launch_decompress_nm(int dt, int n, int m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                                const uint8_t* mask, int64_t ldm, void* D, int64_t ldd, int32_t* bad, hipStream_t s);
// Product; a.vals / a.meta are the stored values and the mask, rows 16- and
// 8-byte aligned, or (packed) their packed decode layout; B rows 16-byte
// aligned.
hipError_t launch_spmm_nm(int n, int m, const SpmmArgs& a, bool packed, hipStream_t s);
// Packed decode layout of the N:M operand: tiles of 16 rows, super-steps of
// 4*D dense k, vb value bytes and mb mask bytes per lane per super-step;
// pvals holds tiles*nsteps*64*vb bytes, pmask tiles*nsteps*64*mb.
void nm_packed_geometry(int dt, int n, int m, int64_t M, int64_t K, int64_t* tiles, int64_t* nsteps, int* vb,
                        int* mb);
hipError_t launch_pack_nm(int dt, int n, int m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                          const uint8_t* mask, int64_t ldm, void* pvals, void* pmask, hipStream_t s);

// Measurement: a streaming read of `bytes` (a multiple of 16) from src; the
// sink holds stream_read_grid(bytes) words and is written only by chance.
int64_t stream_read_grid(int64_t bytes);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);

// Issue-rate probe of one matrix-core instruction form (0 .. forms-1):
// workgroups of four waves, each wave `iters` rounds of its independent
// accumulators; ops = dense-equivalent operations of one launch; sink holds
// `workgroups` words and is written only by chance.
int mfma_probe_forms();
const char* mfma_probe_name(int form);
int64_t mfma_probe_ops(int form, int64_t workgroups, int64_t iters);
hipError_t launch_mfma_probe(int form, int64_t workgroups, int64_t iters, uint32_t* sink, hipStream_t s);

// The LDS read probe: lane l of every wave reads 16 bytes at LDS byte
// off[l] + 4096 j, j < 8 (off[l] a multiple of 16, at most
// kLdsProbeMaxOffset), `iters` times; 4 waves per workgroup.
constexpr uint32_t kLdsProbeMaxOffset = 65536 - 7 * 4096 - 16;
struct LdsPattern {
    uint32_t off[64];
};
hipError_t launch_lds_read_probe(const LdsPattern& pat, int64_t workgroups, int64_t iters, uint32_t* sink,
                                 hipStream_t s);

}  // namespace ssg
