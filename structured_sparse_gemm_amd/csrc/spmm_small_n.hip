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

constexpr int kBatch = 4;                 // k-steps per wave per batch
constexpr int kTMax = 4;                  // 16-row tiles per workgroup
constexpr int kMaxWaves = 16;
constexpr int kLdsB = 128 * 1024;         // B chunk
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

// First index in [lo, hi) whose column is >= k (columns ascending).
__device__ __forceinline__ int64_t lower_bound_col(const int32_t* col, int64_t lo, int64_t hi, int64_t k) {
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (col[mid] < k) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Residual rows of the slab owned by this wave, for the columns of the
// current B chunk [kc0, kc1); row sums accumulate into res[row][16].
template <int DT>
__device__ __forceinline__ void residual_chunk(const SpmmArgs& a, const uint8_t* ldsb, void* res, int64_t r0,
                                               int nrows, int64_t kc0, int64_t kc1, bool multi_chunk, int wave,
                                               int waves, int lane) {
    constexpr int ES = SN<DT>::ES;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    for (int rl = wave; rl < nrows; rl += waves) {
        const int64_t m = r0 + rl;
        int64_t lo = max<int64_t>(a.row_ptr[m], 0), hi = min<int64_t>(a.row_ptr[m + 1], a.nnz_r);
        if (multi_chunk && lo < hi) {
            const int64_t l2 = lower_bound_col(a.col, lo, hi, kc0);
            hi = lower_bound_col(a.col, l2, hi, kc1);
            lo = l2;
        }
        S acc[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[n] = S(0);
        for (int64_t j = lo + lane; j < hi; j += 64) {
            const int64_t c = a.col[j];
            if (c < kc0 || c >= kc1) continue;
            const uint8_t* brow = ldsb + (c - kc0) * 16 * ES;
            if constexpr (DT == DT_I8) {
                const int32_t rv = reinterpret_cast<const int8_t*>(a.rvals)[j];
                const uint4 w = *reinterpret_cast<const uint4*>(brow);
                int8_t bv[16];
                __builtin_memcpy(bv, &w, 16);
#pragma unroll
                for (int n = 0; n < 16; ++n) acc[n] += rv * (int32_t)bv[n];
            } else {
                const float rv = res_value<DT>(a.rvals, j);
                const uint4 w0 = *reinterpret_cast<const uint4*>(brow);
                const uint4 w1 = *reinterpret_cast<const uint4*>(brow + 16);
                uint16_t bv[16];
                __builtin_memcpy(bv, &w0, 16);
                __builtin_memcpy(bv + 8, &w1, 16);
#pragma unroll
                for (int n = 0; n < 16; ++n) acc[n] = fmaf(rv, elem_to_f32<DT>(bv[n]), acc[n]);
            }
        }
        S mine = S(0);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            S v = acc[n];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
            if (lane == n) mine = v;
        }
        if (lane < 16) reinterpret_cast<S*>(res)[rl * 16 + lane] += mine;
    }
}

template <int DT>
__global__ void __launch_bounds__(kMaxWaves * 64) k_spmm_small_n(SpmmArgs a, int rows_per_wg, int chunk_steps,
                                                                 int vecb) {
    using T = SN<DT>;
    using Acc = AccT<DT>;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsB + kLdsRes];
    uint8_t* ldsb = lds;
    void* res = lds + kLdsB;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)min<int64_t>(rows_per_wg, a.M - r0);
    const int tiles = (nrows + 15) >> 4;
    const int64_t ksteps = a.K / T::KS;
    const bool residual = a.row_ptr != nullptr;
    const bool multi_chunk = ksteps > chunk_steps;

    if (residual)
        for (int i = threadIdx.x; i < kTMax * 16 * 16; i += blockDim.x) reinterpret_cast<S*>(res)[i] = S(0);

    Acc acc[kTMax];
#pragma unroll
    for (int t = 0; t < kTMax; ++t) acc[t] = Acc{0, 0, 0, 0};

    // per-lane operand addresses: row r0 + 16t + lane%16, stored values
    // [q*VALS/4, (q+1)*VALS/4) of each k-step, q = lane/16
    const int q = lane >> 4, rl = lane & 15;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vals) + (r0 + rl) * a.ldv * T::ES + q * 16;
    const uint8_t* mbase = a.meta + (r0 + rl) * a.ldm + q * (T::META / 4);
    const int64_t vstep = (int64_t)T::VALS * T::ES;     // bytes of vals per row per k-step
    const int64_t vtile = 16 * a.ldv * T::ES, mtile = 16 * a.ldm;

    for (int64_t c0 = 0; c0 < ksteps; c0 += chunk_steps) {
        const int csteps = (int)min<int64_t>(chunk_steps, ksteps - c0);
        bool first = true;
        for (int kb = wave * kBatch; kb < csteps; kb += waves * kBatch) {
            uint4 av[kBatch][kTMax];
            uint32_t ix[kBatch][kTMax];
#pragma unroll
            for (int s = 0; s < kBatch; ++s) {
#pragma unroll
                for (int t = 0; t < kTMax; ++t) {
                    const bool ok = t < tiles && 16 * t + rl < nrows && kb + s < csteps;
                    const int64_t ks = c0 + kb + s;
                    if (ok) {
                        av[s][t] = *reinterpret_cast<const uint4*>(vbase + t * vtile + ks * vstep);
                        if constexpr (DT == DT_I8)
                            ix[s][t] = *reinterpret_cast<const uint32_t*>(mbase + t * mtile + ks * T::META);
                        else
                            ix[s][t] = *reinterpret_cast<const uint16_t*>(mbase + t * mtile + ks * T::META);
                    } else {
                        av[s][t] = make_uint4(0, 0, 0, 0);
                        ix[s][t] = 0x44444444u;     // any valid pairs: the values are zero
                    }
                }
            }
            if (first) {
                // the first batch's loads are in flight; now stage this chunk of B
                __syncthreads();
                stage_b<DT>(a, ldsb, c0 * T::KS, csteps * T::KS, vecb != 0);
                __syncthreads();
                first = false;
            }
#pragma unroll
            for (int s = 0; s < kBatch; ++s) {
                if (kb + s >= csteps) break;
                uint4 b[2];
                load_b_operand<DT>(ldsb, kb + s, lane, b);
#pragma unroll
                for (int t = 0; t < kTMax; ++t)
                    if (t < tiles) acc[t] = smfmac<DT>(av[s][t], b, acc[t], ix[s][t]);
            }
        }
        if (first) {
            // this wave had no k-steps in the chunk: it still joins the barriers
            __syncthreads();
            stage_b<DT>(a, ldsb, c0 * T::KS, csteps * T::KS, vecb != 0);
            __syncthreads();
        }
        if (residual)
            residual_chunk<DT>(a, ldsb, res, r0, nrows, c0 * T::KS, (c0 + csteps) * T::KS, multi_chunk, wave, waves,
                               lane);
        __syncthreads();   // the chunk is consumed before the next one is staged
    }

    // fixed-order reduction of the waves' partial tiles
    Acc* red = reinterpret_cast<Acc*>(ldsb);
#pragma unroll
    for (int t = 0; t < kTMax; ++t)
        if (t < tiles) red[(wave * kTMax + t) * 64 + lane] = acc[t];
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
    const int malign = T::META / 4;   // 2 or 4 bytes per lane
    return a.N >= 1 && a.N <= 16 && a.K > 0 && a.K % T::KS == 0 && v % 16 == 0 && (a.ldv * T::ES) % 16 == 0 &&
           m % malign == 0 && a.ldm % malign == 0 && a.M > 0;
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
    const int64_t max_chunk = kLdsB / (16 * T::ES) / T::KS;
    const int chunk_steps = (int)(ksteps < max_chunk ? ksteps : max_chunk);
    int waves = (chunk_steps + kBatch - 1) / kBatch;
    if (waves > kMaxWaves) waves = kMaxWaves;
    const uintptr_t bp = reinterpret_cast<uintptr_t>(a.B);
    const bool vecb = a.N == 16 && bp % 16 == 0 && (a.ldb * T::ES) % 16 == 0;
    hipLaunchKernelGGL(k_spmm_small_n<DT>, dim3((unsigned)G), dim3(64 * waves), 0, s, a, (int)rows_per_wg,
                       chunk_steps, (int)vecb);
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
