// spmm_small_n.hip -- 2:4 SpMM for decode shapes (N <= 16): the weight
// stream from HBM is the whole cost, so the kernel is built to keep that
// stream wide and deep.
//
// What it computes: C[m, n] = sum over groups g of the two stored values of
// row m times the two rows of B their 2-bit positions select (the mux of
// "Chapter 26 -- Sparsity: The Hardware View", section "2:4 Fine-Grained
// Structured Sparsity"), plus, when a residual CSR is given, the dropped
// non-zeros ("How sparse LLM weights cut GPU inference cost without
// quantization", section "How the three-layer format makes moderate sparsity
// fast").  In the memory-bound regime the bytes streamed set the time
// ("Chapter 26", section "2:4 in the Memory-Bound Regime").
//
// Mapping on gfx950 (wave64, sparse MFMA):
// * One sparse MFMA (16 rows x 16 columns, 64 dense k for fp16/bf16, 128 for
//   int8) per (16-row tile, k-step).  Its sparse operand is exactly a slice
//   of the stored layout: lane l holds row l%16's 8 (16-bit) or 16 (int8)
//   stored values for dense k in [q*EB, (q+1)*EB), q = l/16, which is one
//   16-byte load from `vals`, and the matching 16 / 32 metadata bits, which
//   are 2 / 4 consecutive bytes of `meta` in the stored nibble order.  No
//   repacking and no decode instructions: the hardware takes the nibbles.
// * A workgroup owns a slab of <= 64 consecutive rows (<= 4 tiles) and all
//   of K; its waves split the k-steps in batches of 4.  Each wave issues the
//   loads of its first batch before B is staged, so every CU has its whole
//   first batch of weight bytes in flight from the start.
// * B (K x N, N <= 16, zero-padded to 16 columns) is staged in LDS in chunks
//   of up to 128 KiB, row-major; the MFMA operand (16 consecutive k of one
//   column per lane) comes from transposing LDS reads (ds_read_b64_tr_b16 /
//   _b8), 4 per k-step, shared by the slab's tiles.
// * The residual CSR rows of the slab are processed by the same workgroup
//   while the matching B chunk is in LDS: one entry per lane, 16 columns per
//   lane, a wave reduction per row.
// * Partial tiles of the waves are summed through LDS in wave order, so the
//   fp32 result is the same on every run.
#include "ssg_device.hpp"
#include "ssg_kernels.hpp"

namespace ssg {

namespace {

constexpr int kUnits = 12;                // (tile, k-step) weight fragments per wave per batch
constexpr int kTMax = 4;                  // 16-row tiles per workgroup
constexpr int kMaxWaves = 16;
constexpr int kLdsB = 128 * 1024;         // B chunk
constexpr int kLdsM = 24 * 1024;         // the slab's metadata rows for one chunk
constexpr int kLdsRes = kTMax * 16 * 16 * 4;   // residual row sums (fp32/int32)

template <int DT> struct SN;
template <> struct SN<DT_F16> {
    static constexpr int KS = 64;          // dense k per MFMA
    static constexpr int VALS = 32;        // stored values per row per k-step
    static constexpr int ES = 2;           // element bytes
    static constexpr int META = 8;         // metadata bytes per row per k-step
};
template <> struct SN<DT_BF16> : SN<DT_F16> {};
template <> struct SN<DT_I8> {
    static constexpr int KS = 128;
    static constexpr int VALS = 64;
    static constexpr int ES = 1;
    static constexpr int META = 16;
};

template <int DT> using AccT = typename std::conditional<DT == DT_I8, i32x4, f32x4>::type;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// B operand of one k-step from the LDS chunk (row-major, 16 columns).
// Element e of lane l (column l%16, block bb=l/16) is dense
// k = (e / H) * (KS / 2) + H * bb + e % H with H = 8 (16-bit) or 16 (int8).
template <int DT>
__device__ __forceinline__ void load_b_operand(const uint8_t* ldsb, int kstep, int lane, uint4 (&b)[2]) {
    const int bb = lane >> 4, i = lane & 15;
    if constexpr (DT == DT_I8) {
        // rows of 16 bytes; tr8: source lane 2q+r names row q, bytes [8r, 8r+8)
        const int q = i >> 1, r = i & 1;
        const uint8_t* base = ldsb + (kstep * 128 + 16 * bb + q) * 16 + 8 * r;
        i32x2 v0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base));
        i32x2 v1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 8 * 16));
        i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 64 * 16));
        i32x2 v3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 72 * 16));
        b[0] = make_uint4(v0[0], v0[1], v1[0], v1[1]);
        b[1] = make_uint4(v2[0], v2[1], v3[0], v3[1]);
    } else {
        // rows of 32 bytes; tr16: source lane 4q+r names row q, columns [4r, 4r+4)
        const int q = i >> 2, r = i & 3;
        const uint8_t* base = ldsb + (kstep * 64 + 8 * bb + q) * 32 + 8 * r;
        i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
        i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * 32));
        i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 32 * 32));
        i16x4 v3 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 36 * 32));
        uint2 w0, w1, w2, w3;
        __builtin_memcpy(&w0, &v0, 8);
        __builtin_memcpy(&w1, &v1, 8);
        __builtin_memcpy(&w2, &v2, 8);
        __builtin_memcpy(&w3, &v3, 8);
        b[0] = make_uint4(w0.x, w0.y, w1.x, w1.y);
        b[1] = make_uint4(w2.x, w2.y, w3.x, w3.y);
    }
}

template <int DT>
__device__ __forceinline__ AccT<DT> smfmac(uint4 a, const uint4 (&b)[2], AccT<DT> c, uint32_t idx) {
    if constexpr (DT == DT_I8) {
        i32x4 av;
        i32x8 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_i32_16x16x128_i8(av, bv, c, (int)idx, 0, 0);
    } else if constexpr (DT == DT_F16) {
        f16x8 av;
        f16x16 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_f32_16x16x64_f16(av, bv, c, (int)idx, 0, 0);
    } else {
        bf16x8 av;
        bf16x16 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(av, bv, c, (int)idx, 0, 0);
    }
}

// Stage rows [k0, k0 + rows) of B into LDS as 16-column rows, zero-padded.
template <int DT>
__device__ __forceinline__ void stage_b(const SpmmArgs& a, uint8_t* ldsb, int64_t k0, int rows, bool vecb) {
    constexpr int ES = SN<DT>::ES, ROWB = 16 * ES;
    if (vecb) {
        constexpr int PIECES = ROWB / 16;
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.B) + k0 * a.ldb * ES;
        for (int i = threadIdx.x; i < rows * PIECES; i += blockDim.x) {
            const int r = i / PIECES, p = i - r * PIECES;
            *reinterpret_cast<uint4*>(ldsb + r * ROWB + 16 * p) =
                *reinterpret_cast<const uint4*>(src + (int64_t)r * a.ldb * ES + 16 * p);
        }
    } else {
        for (int i = threadIdx.x; i < rows * 16; i += blockDim.x) {
            const int r = i >> 4, n = i & 15;
            if constexpr (ES == 2) {
                const uint16_t* src = reinterpret_cast<const uint16_t*>(a.B);
                reinterpret_cast<uint16_t*>(ldsb)[i] = n < a.N ? src[(k0 + r) * a.ldb + n] : (uint16_t)0;
            } else {
                const int8_t* src = reinterpret_cast<const int8_t*>(a.B);
                reinterpret_cast<int8_t*>(ldsb)[i] = n < a.N ? src[(k0 + r) * a.ldb + n] : (int8_t)0;
            }
        }
    }
}

template <int DT>
__device__ __forceinline__ float res_value(const void* rvals, int64_t j) {
    return elem_to_f32<DT>(reinterpret_cast<const uint16_t*>(rvals)[j]);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}

// Direct-to-LDS load of BYTES (4 or 16) per lane: lane l's bytes from buffer
// offset `voff` land at the LDS address of `dst` + l * BYTES; an offset past
// the buffer reads as zero.  Inline assembly, so the compiler does not track
// it: the kernel waits for these loads itself (vmcnt) before its barrier.
template <int BYTES>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, const uint8_t* dst, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)dst);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
                     : "memory");
    else
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
                     : "memory");
}

constexpr uint32_t kOob = 0x80000000u;   // buffer offset that reads as zero

// Residual rows of the slab owned by this wave, restricted to columns of the
// current B chunk [kc0, kc1).  Columns ascend within a row, so each row keeps
// a cursor (first entry not yet consumed) across chunks.  Entries are taken
// 128 at a time (2 per lane, loads in flight together); row sums accumulate
// into res[row][16] in chunk order.
template <int DT>
__device__ __forceinline__ void residual_chunk(const SpmmArgs& a, const uint8_t* ldsb, void* res, int32_t* cursor,
                                               int64_t r0, int nrows, int64_t kc0, int64_t kc1, bool first_chunk,
                                               int wave, int waves, int lane) {
    constexpr int ES = SN<DT>::ES;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    for (int rl = wave; rl < nrows; rl += waves) {
        const int64_t m = r0 + rl;
        const int64_t hi = min<int64_t>(a.row_ptr[m + 1], a.nnz_r);
        int64_t lo = first_chunk ? max<int64_t>(a.row_ptr[m], 0) : (int64_t)cursor[rl];
        S acc[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[n] = S(0);
        while (lo < hi) {
            int32_t c[2];
            S v[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t j = lo + 64 * u + lane;
                c[u] = j < hi ? a.col[j] : (int32_t)kc1;
                if constexpr (DT == DT_I8) v[u] = j < hi ? (int32_t)reinterpret_cast<const int8_t*>(a.rvals)[j] : 0;
                else v[u] = j < hi ? res_value<DT>(a.rvals, j) : 0.0f;
            }
            int taken = 0;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bool in = c[u] >= kc0 && c[u] < kc1;
                taken += __popcll(__ballot(c[u] < kc1 && lo + 64 * u + lane < hi));
                if (in) {
                    const uint8_t* brow = ldsb + (c[u] - kc0) * 16 * ES;
                    if constexpr (DT == DT_I8) {
                        const uint4 w = *reinterpret_cast<const uint4*>(brow);
                        int8_t bv[16];
                        __builtin_memcpy(bv, &w, 16);
#pragma unroll
                        for (int n = 0; n < 16; ++n) acc[n] += v[u] * (int32_t)bv[n];
                    } else {
                        const uint4 w0 = *reinterpret_cast<const uint4*>(brow);
                        const uint4 w1 = *reinterpret_cast<const uint4*>(brow + 16);
                        uint16_t bv[16];
                        __builtin_memcpy(bv, &w0, 16);
                        __builtin_memcpy(bv + 8, &w1, 16);
#pragma unroll
                        for (int n = 0; n < 16; ++n) acc[n] = fmaf(v[u], elem_to_f32<DT>(bv[n]), acc[n]);
                    }
                }
            }
            lo += taken;
            if (taken < 128) break;     // reached an entry of a later chunk, or the row's end
        }
        if (lane == 0) cursor[rl] = (int32_t)lo;
        S mine = S(0);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            S x = acc[n];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
            if (lane == n) mine = x;
        }
        if (lane < 16) reinterpret_cast<S*>(res)[rl * 16 + lane] += mine;
    }
}

// TM = 16-row tiles of the slab; each wave takes batches of KB = 12/TM
// k-steps for all TM tiles (12 fragments in flight per wave).
template <int DT, int TM>
__global__ void __launch_bounds__(kMaxWaves * 64) k_spmm_small_n(SpmmArgs a, int rows_per_wg, int chunk_steps,
                                                                 int dma_b) {
    constexpr int kBatch = kUnits / TM;
    using T = SN<DT>;
    using Acc = AccT<DT>;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsB + kLdsM + kLdsRes + 256];
    uint8_t* ldsb = lds;
    uint8_t* ldsm = lds + kLdsB;
    void* res = lds + kLdsB + kLdsM;
    int32_t* cursor = reinterpret_cast<int32_t*>(lds + kLdsB + kLdsM + kLdsRes);

    const int lane = threadIdx.x & 63, waves = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)min<int64_t>(rows_per_wg, a.M - r0);
    const int tiles = (nrows + 15) >> 4;
    const int64_t ksteps = a.K / T::KS;
    const bool residual = a.row_ptr != nullptr;

    if (residual)
        for (int i = threadIdx.x; i < kTMax * 16 * 16; i += blockDim.x) reinterpret_cast<S*>(res)[i] = S(0);

    Acc acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = Acc{0, 0, 0, 0};

    // sparse operand of lane l: row r0 + 16t + l%16, stored values
    // [q*VALS/4, (q+1)*VALS/4) of each k-step, q = l/16
    const int q = lane >> 4, rl = lane & 15;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vals) + (r0 + rl) * a.ldv * T::ES + q * 16;
    const int64_t vstep = (int64_t)T::VALS * T::ES;
    const int64_t vtile = 16 * a.ldv * T::ES;

    for (int64_t c0 = 0; c0 < ksteps; c0 += chunk_steps) {
        const int csteps = (int)min<int64_t>(chunk_steps, ksteps - c0);
        const int mpitch = csteps * T::META;             // metadata bytes per row in this chunk
        if (c0 > 0) __syncthreads();                      // previous chunk consumed

        // 1. direct-to-LDS: this chunk of B (when it copies in 16-byte
        //    pieces) and the slab's metadata rows for the chunk
        if (dma_b) {
            constexpr int ROWB = 16 * T::ES, PIECES = ROWB / 16;
            const int rows = csteps * T::KS;
            const __amdgpu_buffer_rsrc_t rb =
                rsrc(reinterpret_cast<const uint8_t*>(a.B) + c0 * T::KS * a.ldb * T::ES,
                     ((a.K - c0 * T::KS - 1) * a.ldb + a.N) * T::ES);
            for (int ins = wave; ins * 64 < rows * PIECES; ins += waves) {
                const int p = ins * 64 + lane, row = p / PIECES, piece = p - row * PIECES;
                const uint32_t off = row < rows ? (uint32_t)(row * a.ldb * T::ES + 16 * piece) : kOob;
                dma<16>(rb, ldsb + ins * 1024, off);
            }
        }
        {
            const int words = mpitch / 4;                 // dwords per metadata row
            const __amdgpu_buffer_rsrc_t rm =
                rsrc(a.meta + r0 * a.ldm + c0 * T::META, (a.M - r0 - 1) * a.ldm + (a.K + 7) / 8 - c0 * T::META);
            for (int ins = wave; ins * 64 < nrows * words; ins += waves) {
                const int p = ins * 64 + lane, row = p / words, w = p - row * words;
                const uint32_t off = row < nrows ? (uint32_t)(row * a.ldm + 4 * w) : kOob;
                dma<4>(rm, ldsm + ins * 256, off);
            }
        }
        // 2. B chunks that are not 16 full columns: element-wise staging
        if (!dma_b) stage_b<DT>(a, ldsb, c0 * T::KS, csteps * T::KS, false);

        // 3. weight batches; the first batch's loads are issued before the
        //    wait so they stream while B and the metadata land
        bool first = true;
        for (int kb = wave * kBatch;; kb += waves * kBatch) {
            const bool have = kb < csteps;
            uint4 av[kBatch][TM];
            if (have) {
#pragma unroll
                for (int s = 0; s < kBatch; ++s) {
#pragma unroll
                    for (int t = 0; t < TM; ++t) {
                        const bool ok = 16 * t + rl < nrows && kb + s < csteps;
                        av[s][t] = ok ? *reinterpret_cast<const uint4*>(vbase + t * vtile + (c0 + kb + s) * vstep)
                                      : make_uint4(0, 0, 0, 0);
                    }
                }
            }
            if (first) {
                // this wave's direct-to-LDS loads are done once its vector
                // memory counter drains; the barrier covers the other waves'
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                __syncthreads();
                first = false;
            }
            if (!have) break;
#pragma unroll
            for (int s = 0; s < kBatch; ++s) {
                if (kb + s >= csteps) break;
                uint4 b[2];
                load_b_operand<DT>(ldsb, kb + s, lane, b);
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    {
                        const uint8_t* mp = ldsm + (16 * t + rl) * mpitch + (kb + s) * T::META + q * (T::META / 4);
                        uint32_t ix;
                        if constexpr (DT == DT_I8) ix = *reinterpret_cast<const uint32_t*>(mp);
                        else ix = *reinterpret_cast<const uint16_t*>(mp);
                        acc[t] = smfmac<DT>(av[s][t], b, acc[t], ix);
                    }
                }
            }
        }
        if (residual)
            residual_chunk<DT>(a, ldsb, res, cursor, r0, nrows, c0 * T::KS, (c0 + csteps) * T::KS, c0 == 0, wave,
                               waves, lane);
    }
    __syncthreads();

    // fixed-order reduction of the waves' partial tiles
    Acc* red = reinterpret_cast<Acc*>(ldsb);
#pragma unroll
    for (int t = 0; t < TM; ++t) red[(wave * kTMax + t) * 64 + lane] = acc[t];
    __syncthreads();
    for (int i = threadIdx.x; i < tiles * 256; i += blockDim.x) {
        const int t = i >> 8, ln = (i >> 2) & 63, r = i & 3;
        S sum = S(0);
        for (int w = 0; w < waves; ++w) sum += reinterpret_cast<const S*>(red)[((w * kTMax + t) * 64 + ln) * 4 + r];
        const int row = 16 * t + 4 * (ln >> 4) + r, col = ln & 15;
        if (row < nrows && col < a.N) {
            if (residual) sum += reinterpret_cast<const S*>(res)[row * 16 + col];
            reinterpret_cast<S*>(a.C)[(r0 + row) * a.ldc + col] = sum;
        }
    }
}

template <int DT>
bool supported_t(const SpmmArgs& a) {
    using T = SN<DT>;
    const uintptr_t v = reinterpret_cast<uintptr_t>(a.vals), m = reinterpret_cast<uintptr_t>(a.meta);
    // vals rows 16-byte aligned; metadata rows 4-byte aligned (dword copies);
    // every buffer addressed with 31-bit offsets
    return a.N >= 1 && a.N <= 16 && a.K > 0 && a.K % T::KS == 0 && v % 16 == 0 && (a.ldv * T::ES) % 16 == 0 &&
           m % 4 == 0 && a.ldm % 4 == 0 && a.M > 0 && (a.M - 1) * a.ldm + a.K / 8 < 0x7fffffff &&
           ((a.K - 1) * a.ldb + a.N) * T::ES < 0x7fffffff;
}

template <int DT>
hipError_t launch_t(const SpmmArgs& a, hipStream_t s) {
    using T = SN<DT>;
    const int64_t tiles = (a.M + 15) / 16;
    int64_t G = tiles < 256 ? tiles : 256;
    const int64_t min_g = (tiles + kTMax - 1) / kTMax;
    if (G < min_g) G = min_g;
    const int64_t rows_per_wg = (a.M + G - 1) / G;
    G = (a.M + rows_per_wg - 1) / rows_per_wg;
    const int64_t ksteps = a.K / T::KS;
    // chunks of K: B rows (16 columns) and the slab's metadata rows must fit
    // their LDS regions; chunks are made equal
    int64_t max_steps = kLdsB / (16 * T::ES * T::KS);
    const int64_t msteps = kLdsM / (rows_per_wg * T::META);
    if (msteps < max_steps) max_steps = msteps;
    const int64_t nchunks = (ksteps + max_steps - 1) / max_steps;
    const int chunk_steps = (int)((ksteps + nchunks - 1) / nchunks);
    const int tm = (int)((rows_per_wg + 15) / 16);
    const int kbatch = kUnits / tm;
    int waves = (chunk_steps + kbatch - 1) / kbatch;
    if (waves > kMaxWaves) waves = kMaxWaves;
    const uintptr_t bp = reinterpret_cast<uintptr_t>(a.B);
    const bool dma_b = a.N == 16 && bp % 16 == 0 && (a.ldb * T::ES) % 16 == 0;
    const dim3 grid((unsigned)G), block(64 * waves);
    switch (tm) {
        case 1: hipLaunchKernelGGL((k_spmm_small_n<DT, 1>), grid, block, 0, s, a, (int)rows_per_wg, chunk_steps, (int)dma_b); break;
        case 2: hipLaunchKernelGGL((k_spmm_small_n<DT, 2>), grid, block, 0, s, a, (int)rows_per_wg, chunk_steps, (int)dma_b); break;
        case 3: hipLaunchKernelGGL((k_spmm_small_n<DT, 3>), grid, block, 0, s, a, (int)rows_per_wg, chunk_steps, (int)dma_b); break;
        default: hipLaunchKernelGGL((k_spmm_small_n<DT, 4>), grid, block, 0, s, a, (int)rows_per_wg, chunk_steps, (int)dma_b); break;
    }
    return hipGetLastError();
}

}  // namespace

bool supported_small_n(const SpmmArgs& a) {
    switch (a.dt) {
        case DT_F16: return supported_t<DT_F16>(a);
        case DT_BF16: return supported_t<DT_BF16>(a);
        case DT_I8: return supported_t<DT_I8>(a);
        default: return false;
    }
}

hipError_t launch_spmm_small_n(const SpmmArgs& a, hipStream_t s) {
    switch (a.dt) {
        case DT_F16: return launch_t<DT_F16>(a, s);
        case DT_BF16: return launch_t<DT_BF16>(a, s);
        case DT_I8: return launch_t<DT_I8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssg
