// spmm_large_n_basic.hip -- 2:4 SpMM on gfx950's sparse MFMA for large-N
// operands the pipelined kernel (spmm_large_n.hip) does not take: any N,
// any B leading dimension and alignment (element-wise B staging at edges).
//
// What it computes: C = expand(vals, meta) x B, where each stored pair of a
// group meets the two rows of B its 2-bit positions select ("Chapter 26 --
// Sparsity: The Hardware View", section "2:4 Fine-Grained Structured
// Sparsity"); in the compute-bound regime the sparse matrix units' doubled
// rate is what pays ("Chapter 26", sections "2:4: ~2x on the Matmul, Less
// End-to-End" and "2:4 in the Memory-Bound Regime").
//
// Mapping:
// * Workgroup tile BM x BN (256 x 256 by default), 4 waves in a 2 x 2
//   layout, each wave a (BM/2) x (BN/2) block of 32 x 32 sparse MFMA tiles
//   (v_smfmac_f32_32x32x32_{f16,bf16}: 32 dense k per step;
//   v_smfmac_i32_32x32x64_i8: 64 dense k per step).
// * Sparse operand straight from global memory into registers: lane l holds
//   row l%32's stored values for dense k in [q*EB, (q+1)*EB), q = l/32, which
//   is one 16-byte load of `vals` plus 2 (16-bit) / 4 (int8) bytes of `meta`
//   in the stored nibble order.  Prefetched one k-step ahead.
// * B tile (one k-step x BN) staged through LDS, double-buffered, rows padded
//   so the transposing reads (ds_read_b64_tr_b16 / _b8) that build the MFMA
//   operand (consecutive k of one column per lane) hit distinct banks:
//   pitch = 2*BN + 64 bytes (16-bit), BN + 32 bytes (int8).
// * One barrier per k-step.  Edges in M and N are masked (zero operands,
//   masked stores); K must be a multiple of the k-step.
#include "ssg_device.hpp"
#include "ssg_kernels.hpp"

namespace ssg {

namespace {

template <int DT> struct LN;
template <> struct LN<DT_F16> {
    static constexpr int KSTEP = 32;       // dense k per MFMA
    static constexpr int ES = 2;
    static constexpr int VALS = 16;        // stored values per row per k-step
    static constexpr int META = 4;         // metadata bytes per row per k-step
    static constexpr int IDXB = 2;         // metadata bytes per lane
    static constexpr int PAD = 64;         // LDS row padding (bytes)
};
template <> struct LN<DT_BF16> : LN<DT_F16> {};
template <> struct LN<DT_I8> {
    static constexpr int KSTEP = 64;
    static constexpr int ES = 1;
    static constexpr int VALS = 32;
    static constexpr int META = 8;
    static constexpr int IDXB = 4;
    static constexpr int PAD = 32;
};
template <> struct LN<DT_E4M3> : LN<DT_I8> {};   // 8-bit floats: the int8 shapes
template <> struct LN<DT_E5M2> : LN<DT_I8> {};

template <int DT> using Acc16 = typename std::conditional<DT == DT_I8, i32x16, f32x16>::type;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int DT>
__device__ __forceinline__ Acc16<DT> smfmac32(uint4 a, const uint4 (&b)[2], Acc16<DT> c, uint32_t idx) {
    if constexpr (DT == DT_I8) {
        i32x4 av;
        i32x8 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_i32_32x32x64_i8(av, bv, c, (int)idx, 0, 0);
    } else if constexpr (dt_is_fp8(DT)) {
        i32x4 av;
        i32x8 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        if constexpr (DT == DT_E4M3) return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(av, bv, c, (int)idx, 0, 0);
        else return __builtin_amdgcn_smfmac_f32_32x32x64_bf8_bf8(av, bv, c, (int)idx, 0, 0);
    } else if constexpr (DT == DT_F16) {
        f16x8 av;
        f16x16 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_f32_32x32x32_f16(av, bv, c, (int)idx, 0, 0);
    } else {
        bf16x8 av;
        bf16x16 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(av, bv, c, (int)idx, 0, 0);
    }
}

// MFMA B operand of the 32-column block starting at tile column `cb`
// (an element index; byte offsets are formed here).
// Lane l: column cb + l%32, block bb = l/32; element e is dense
// k = (e / H) * (KSTEP / 2) + H * bb + e % H, H = 8 (16-bit) / 16 (int8).
// Transposing reads work on 16-lane groups: source lane 4q+r (tr16) or 2q+r
// (tr8) names a row and 4 / 8 consecutive columns; output lane i receives
// column i of 4 / 8 consecutive rows.
template <int DT, int PITCH>
__device__ __forceinline__ void b_operand(const uint8_t* buf, int cb, int lane, uint4 (&b)[2]) {
    const int bb = lane >> 5, h = (lane >> 4) & 1, i = lane & 15;
    if constexpr (dt_bytes(DT) == 1) {
        const int q = i >> 1, r = i & 1;
        const uint8_t* p = buf + (16 * bb + q) * PITCH + cb + 16 * h + 8 * r;
        i32x2 v0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
        i32x2 v1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 8 * PITCH));
        i32x2 v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 32 * PITCH));
        i32x2 v3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 40 * PITCH));
        b[0] = make_uint4(v0[0], v0[1], v1[0], v1[1]);
        b[1] = make_uint4(v2[0], v2[1], v3[0], v3[1]);
    } else {
        const int q = i >> 2, r = i & 3;
        const uint8_t* p = buf + (8 * bb + q) * PITCH + 2 * (cb + 16 * h + 4 * r);
        i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
        i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * PITCH));
        i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * PITCH));
        i16x4 v3 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 20 * PITCH));
        uint2 w0, w1, w2, w3;
        __builtin_memcpy(&w0, &v0, 8);
        __builtin_memcpy(&w1, &v1, 8);
        __builtin_memcpy(&w2, &v2, 8);
        __builtin_memcpy(&w3, &v3, 8);
        b[0] = make_uint4(w0.x, w0.y, w1.x, w1.y);
        b[1] = make_uint4(w2.x, w2.y, w3.x, w3.y);
    }
}

template <int DT, int BM, int BN>
struct Cfg {
    using T = LN<DT>;
    static constexpr int THREADS = 256;
    static constexpr int TM = BM / 64, TN = BN / 64;          // 32x32 tiles per wave (2x2 waves)
    static constexpr int ROWB = BN * T::ES;                   // B tile row bytes
    static constexpr int PITCH = ROWB + T::PAD;
    static constexpr int BUF = T::KSTEP * PITCH;              // one LDS buffer
    static constexpr int CHUNKS = T::KSTEP * ROWB / 16;       // 16-byte pieces per B tile
    static constexpr int CPT = CHUNKS / THREADS;              // per thread
    static_assert(CHUNKS % THREADS == 0, "B tile must split evenly");
};

// Global -> registers: this thread's pieces of the B tile of k-step ks.
template <int DT, int BM, int BN>
__device__ __forceinline__ void load_b_tile(const SpmmArgs& a, int64_t n0, int64_t ks, bool vecb,
                                            uint4 (&r)[Cfg<DT, BM, BN>::CPT]) {
    using C = Cfg<DT, BM, BN>;
    using T = LN<DT>;
    constexpr int PER_ROW = C::ROWB / 16, EPV = 16 / T::ES;
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
        const int c = threadIdx.x + j * C::THREADS;
        const int row = c / PER_ROW, col = (c % PER_ROW) * EPV;
        const int64_t k = ks * T::KSTEP + row, n = n0 + col;
        const uint8_t* src = reinterpret_cast<const uint8_t*>(a.B) + (k * a.ldb + n) * T::ES;
        if (vecb && n + EPV <= a.N) {
            r[j] = *reinterpret_cast<const uint4*>(src);
        } else {
            uint8_t tmp[16];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                if constexpr (T::ES == 2) {
                    const uint16_t v = (n + e < a.N) ? reinterpret_cast<const uint16_t*>(src)[e] : (uint16_t)0;
                    __builtin_memcpy(tmp + 2 * e, &v, 2);
                } else {
                    tmp[e] = (n + e < a.N) ? src[e] : (uint8_t)0;
                }
            }
            __builtin_memcpy(&r[j], tmp, 16);
        }
    }
}

template <int DT, int BM, int BN>
__device__ __forceinline__ void store_b_tile(uint8_t* buf, const uint4 (&r)[Cfg<DT, BM, BN>::CPT]) {
    using C = Cfg<DT, BM, BN>;
    constexpr int PER_ROW = C::ROWB / 16;
#pragma unroll
    for (int j = 0; j < C::CPT; ++j) {
        const int c = threadIdx.x + j * C::THREADS;
        const int row = c / PER_ROW, colb = (c % PER_ROW) * 16;
        *reinterpret_cast<uint4*>(buf + row * C::PITCH + colb) = r[j];
    }
}

// Sparse operand of this wave's TM row tiles for k-step ks.
template <int DT, int TM>
__device__ __forceinline__ void load_a(const SpmmArgs& a, int64_t row0, int64_t ks, int lane, uint4 (&av)[TM],
                                       uint32_t (&ix)[TM]) {
    using T = LN<DT>;
    const int q = lane >> 5, rl = lane & 31;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t row = row0 + 32 * i + rl;
        if (row < a.M) {
            const uint8_t* vp = reinterpret_cast<const uint8_t*>(a.vals) +
                                (row * a.ldv + ks * T::VALS + q * (T::VALS / 2)) * T::ES;
            const uint8_t* mp = a.meta + row * a.ldm + ks * T::META + q * T::IDXB;
            av[i] = *reinterpret_cast<const uint4*>(vp);
            if constexpr (T::IDXB == 4) ix[i] = *reinterpret_cast<const uint32_t*>(mp);
            else ix[i] = *reinterpret_cast<const uint16_t*>(mp);
        } else {
            av[i] = make_uint4(0, 0, 0, 0);
            ix[i] = 0x44444444u;
        }
    }
}

template <int DT, int BM, int BN>
__global__ void __launch_bounds__(256) k_spmm_large_n(SpmmArgs a, int vecb) {
    using C = Cfg<DT, BM, BN>;
    using T = LN<DT>;
    using Acc = Acc16<DT>;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    constexpr int TM = C::TM, TN = C::TN;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::BUF];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int64_t wrow0 = m0 + wm * (BM / 2);
    const int wcol0 = wn * (BN / 2);            // column offset inside the tile
    const int64_t nk = a.K / T::KSTEP;

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = S(0);

    uint4 av[TM], av_next[TM];
    uint32_t ix[TM], ix_next[TM];
    uint4 breg[C::CPT];

    load_a<DT, TM>(a, wrow0, 0, lane, av, ix);
    load_b_tile<DT, BM, BN>(a, n0, 0, vecb != 0, breg);
    store_b_tile<DT, BM, BN>(lds, breg);
    __syncthreads();

    for (int64_t ks = 0; ks < nk; ++ks) {
        const uint8_t* cur = lds + (ks & 1) * C::BUF;
        uint8_t* nxt = lds + ((ks + 1) & 1) * C::BUF;
        const bool more = ks + 1 < nk;
        if (more) {
            load_a<DT, TM>(a, wrow0, ks + 1, lane, av_next, ix_next);
            load_b_tile<DT, BM, BN>(a, n0, ks + 1, vecb != 0, breg);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            uint4 b[2];
            b_operand<DT, C::PITCH>(cur, wcol0 + 32 * j, lane, b);   // column index (elements)
#pragma unroll
            for (int i = 0; i < TM; ++i) acc[i][j] = smfmac32<DT>(av[i], b, acc[i][j], ix[i]);
        }
        if (more) store_b_tile<DT, BM, BN>(nxt, breg);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            av[i] = av_next[i];
            ix[i] = ix_next[i];
        }
    }

    // epilogue: D element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wcol0 + 32 * j + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = wrow0 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row < a.M && col < a.N) reinterpret_cast<S*>(a.C)[row * a.ldc + col] = acc[i][j][e];
            }
        }
    }
}

template <int DT>
bool supported_t(const SpmmArgs& a) {
    using T = LN<DT>;
    const uintptr_t v = reinterpret_cast<uintptr_t>(a.vals), m = reinterpret_cast<uintptr_t>(a.meta);
    return a.M > 0 && a.N > 0 && a.K > 0 && a.K % T::KSTEP == 0 && v % 16 == 0 && (a.ldv * T::ES) % 16 == 0 &&
           m % T::IDXB == 0 && a.ldm % T::IDXB == 0 && (a.M + 255) / 256 <= 65535;
}

template <int DT>
hipError_t launch_t(const SpmmArgs& a, hipStream_t s) {
    using T = LN<DT>;
    constexpr int BM = 256, BN = 256;
    const uintptr_t bp = reinterpret_cast<uintptr_t>(a.B);
    const bool vecb = bp % 16 == 0 && (a.ldb * T::ES) % 16 == 0;
    const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL((k_spmm_large_n<DT, BM, BN>), grid, dim3(256), 0, s, a, (int)vecb);
    return hipGetLastError();
}

}  // namespace

bool supported_large_n_basic(const SpmmArgs& a) {
    switch (a.dt) {
        case DT_F16: return supported_t<DT_F16>(a);
        case DT_BF16: return supported_t<DT_BF16>(a);
        case DT_I8: return supported_t<DT_I8>(a);
        case DT_E4M3: return supported_t<DT_E4M3>(a);
        case DT_E5M2: return supported_t<DT_E5M2>(a);
        default: return false;
    }
}

hipError_t launch_spmm_large_n_basic(const SpmmArgs& a, hipStream_t s) {
    switch (a.dt) {
        case DT_F16: return launch_t<DT_F16>(a, s);
        case DT_BF16: return launch_t<DT_BF16>(a, s);
        case DT_I8: return launch_t<DT_I8>(a, s);
        case DT_E4M3: return launch_t<DT_E4M3>(a, s);
        case DT_E5M2: return launch_t<DT_E5M2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssg
