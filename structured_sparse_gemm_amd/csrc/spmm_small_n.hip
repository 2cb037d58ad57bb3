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
// * The residual rows of the slab (CSR, or delta-coded gap bytes decoded by
//   a wave prefix sum) are processed by the same workgroup while the
//   matching B chunk is in LDS: one entry per lane, 16 columns per lane, a
//   wave reduction per row.
// * Partial tiles of the waves are summed through LDS in wave order, so the
//   fp32 result is the same on every run.
#include <algorithm>

#include "ssg_device.hpp"
#include "ssg_kernels.hpp"
#include "ssg_stream.hpp"

namespace ssg {

namespace {

constexpr int kTMax = 4;                  // 16-row tiles per workgroup
constexpr int kWaves = 8;
constexpr int kLdsRes = kTMax * 16 * 16 * 4;   // residual row sums (fp32/int32)
constexpr int kLdsCursor = 512;                // residual row cursors (entry, column before it)
// B chunk followed by the slab's padded metadata rows for the chunk
constexpr int kLdsData = 160 * 1024 - kLdsRes - kLdsCursor;
constexpr int kRingResOff = 160 * 1024 - kLdsRes;       // ring kernel: residual row sums at the top of LDS

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
template <> struct SN<DT_E4M3> : SN<DT_I8> {};   // 8-bit floats: the int8 shapes
template <> struct SN<DT_E5M2> : SN<DT_I8> {};

template <int DT> using AccT = typename std::conditional<DT == DT_I8, i32x4, f32x4>::type;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// B operand of one k-step from the LDS chunk (row-major, 16 columns).
// Element e of lane l (column l%16, block bb=l/16) is dense
// k = (e / H) * (KS / 2) + H * bb + e % H with H = 8 (16-bit) or 16 (int8).
template <int DT>
__device__ __forceinline__ void load_b_operand(const uint8_t* ldsb, int kstep, int lane, uint4 (&b)[2]) {
    const int bb = lane >> 4, i = lane & 15;
    if constexpr (SN<DT>::ES == 1) {
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
    } else if constexpr (dt_is_fp8(DT)) {
        i32x4 av;
        i32x8 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        if constexpr (DT == DT_E4M3) return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(av, bv, c, (int)idx, 0, 0);
        else return __builtin_amdgcn_smfmac_f32_16x16x128_bf8_bf8(av, bv, c, (int)idx, 0, 0);
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

template <int CTRL, typename S>
__device__ __forceinline__ S dpp_xor(S x) {
    int v;
    __builtin_memcpy(&v, &x, 4);
    const int r = __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
    S y;
    __builtin_memcpy(&y, &r, 4);
    return y;
}

// ds_swizzle in bit-mask mode: lane i reads lane i ^ X within its 32 lanes
template <int X, typename S>
__device__ __forceinline__ S swz_xor(S x) {
    int v;
    __builtin_memcpy(&v, &x, 4);
    const int r = __builtin_amdgcn_ds_swizzle(v, 0x1F | (X << 10));
    S y;
    __builtin_memcpy(&y, &r, 4);
    return y;
}

// Transposing reduction of 16 per-lane column sums over the 64 lanes: at
// each exchange a lane keeps half of its columns and adds its partner's
// copy of them, so after 4 exchanges within a row of 16 lanes lane i holds
// one column, bitrev4(i % 16), and two more fold the four rows.  About 60
// instructions instead of 16 full-wave reductions; the order of the adds is
// fixed, so the sum is the same on every run.
template <typename S>
__device__ __forceinline__ S transpose_sum16(S (&x)[16], int lane) {
    const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4, b3 = lane & 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const S send = b0 ? x[i] : x[i + 8], keep = b0 ? x[i + 8] : x[i];
        x[i] = keep + dpp_xor<0xB1>(send);   // quad_perm [1,0,3,2]
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const S send = b1 ? x[i] : x[i + 4], keep = b1 ? x[i + 4] : x[i];
        x[i] = keep + dpp_xor<0x4E>(send);   // quad_perm [2,3,0,1]
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const S send = b2 ? x[i] : x[i + 2], keep = b2 ? x[i + 2] : x[i];
        x[i] = keep + swz_xor<4>(send);
    }
    {
        const S send = b3 ? x[0] : x[1], keep = b3 ? x[1] : x[0];
        x[0] = keep + swz_xor<8>(send);
    }
    S t = x[0];
    t += swz_xor<16>(t);
    t += __shfl_xor(t, 32, 64);
    return t;
}

__device__ __forceinline__ int transpose_col(int lane) {
    return ((lane & 1) << 3) | ((lane & 2) << 1) | ((lane & 4) >> 1) | ((lane & 8) >> 3);
}

// Inclusive prefix sum over the wave's 64 lanes: four row_shr steps inside
// each row of 16 lanes, then every lane adds the totals of the rows below.
__device__ __forceinline__ int wave_incl_sum(int x, int lane) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
              r2 = __builtin_amdgcn_readlane(x, 47);
    return x + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// The chunk's B rows (16 columns, contiguous in memory when ldb == 16) as
// 1 KiB direct-to-LDS loads, dealt round-robin to the waves.
template <int DT>
__device__ __forceinline__ void dma_b(const SpmmArgs& a, uint32_t ldsb, int64_t k0, int rows, int wave) {
    constexpr int ES = SN<DT>::ES;
    const int bytes = rows * 16 * ES;
    const int64_t avail = (a.K - k0) * 16 * ES;
    const __amdgpu_buffer_rsrc_t r = rsrc(reinterpret_cast<const uint8_t*>(a.B) + k0 * 16 * ES, avail);
    const int lane = threadIdx.x & 63;
    for (int ins = wave; ins * 1024 < bytes; ins += kWaves) dma<16>(r, ldsb + ins * 1024, (uint32_t)(ins * 1024 + lane * 16));
}

// The slab's metadata for the chunk as 256-byte direct-to-LDS loads, one row
// segment each (rows padded to `pitch` in LDS); lanes past a row's end are
// masked off so they write nothing.
template <int DT>
__device__ __forceinline__ void dma_meta(const SpmmArgs& a, uint32_t ldsm, int64_t r0, int nrows, int64_t c0,
                                         int csteps, int pitch, int wave) {
    constexpr int META = SN<DT>::META;
    const int rowb = csteps * META, segs = (rowb + 255) / 256;
    const __amdgpu_buffer_rsrc_t r = rsrc(a.meta + r0 * a.ldm, (a.M - r0 - 1) * a.ldm + (a.K + 7) / 8);
    const int lane = threadIdx.x & 63;
    for (int ins = wave; ins < nrows * segs; ins += kWaves) {
        const int row = ins / segs, seg = ins - row * segs;
        const int off = 256 * seg + 4 * lane;
        if (off < rowb) dma<4>(r, ldsm + row * pitch + 256 * seg, (uint32_t)(row * a.ldm + c0 * META + off));
    }
}

// Stage B rows [k0, k0 + rows) as 16-column rows into LDS.  The 16-byte
// path issues all of a thread's loads before its first LDS write, so the
// staging costs one memory latency, not one per piece.
template <int DT>
__device__ __forceinline__ void stage_b_batched(const SpmmArgs& a, uint8_t* ldsb, int64_t k0, int rows, bool vecb) {
    constexpr int ES = SN<DT>::ES, ROWB = 16 * ES, PIECES = ROWB / 16, J = 16;
    if (!vecb) {
        stage_b<DT>(a, ldsb, k0, rows, false);
        return;
    }
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.B) + k0 * a.ldb * ES;
    const int n = rows * PIECES;
    for (int base = threadIdx.x; base < n; base += J * blockDim.x) {
        uint4 v[J];
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int i = base + j * blockDim.x;
            const int r = i / PIECES, p = i - r * PIECES;
            v[j] = i < n ? *reinterpret_cast<const uint4*>(src + (int64_t)r * a.ldb * ES + 16 * p) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int i = base + j * blockDim.x;
            if (i < n) *reinterpret_cast<uint4*>(ldsb + 16 * i) = v[j];
        }
    }
}

// Stage the slab's metadata for k-steps [c0, c0 + csteps) into LDS rows of
// `pitch` bytes (the chunk's bytes plus 4 of padding, so the 16 lanes that
// read one column of 16 rows hit different banks).  Batched like B.
template <int DT>
__device__ __forceinline__ void stage_meta(const SpmmArgs& a, uint8_t* ldsm, int64_t r0, int nrows, int64_t c0,
                                           int csteps, int pitch, bool vec) {
    constexpr int META = SN<DT>::META, J = 16;
    const int rowb = csteps * META;
    if (vec) {
        const int pieces = rowb / 4, n = nrows * pieces;
        for (int base = threadIdx.x; base < n; base += J * blockDim.x) {
            uint32_t v[J];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int i = base + j * blockDim.x;
                const int r = i / pieces, p = i - r * pieces;
                v[j] = i < n ? *reinterpret_cast<const uint32_t*>(a.meta + (r0 + r) * a.ldm + c0 * META + 4 * p) : 0u;
            }
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int i = base + j * blockDim.x;
                const int r = i / pieces, p = i - r * pieces;
                if (i < n) *reinterpret_cast<uint32_t*>(ldsm + r * pitch + 4 * p) = v[j];
            }
        }
    } else {
        for (int i = threadIdx.x; i < nrows * rowb; i += blockDim.x) {
            const int r = i / rowb, p = i - r * rowb;
            ldsm[r * pitch + p] = a.meta[(r0 + r) * a.ldm + c0 * META + p];
        }
    }
}

// ---- residual pass ---------------------------------------------------------
//
// Residual rows of the slab owned by this wave (rl = wave + W*j), taken
// chunk by chunk of K (the columns whose B rows are in LDS).  Columns ascend
// within a row, so each row keeps a cursor (first entry not yet consumed)
// across chunks.  A pass covers 64*EPL consecutive entries of a row, EPL per
// lane (lane l: entries ld + 64*EPL*p + EPL*l + i), read with one buffer load
// per array: the column indices (CSR) or gap bytes (delta-coded), and the
// values.  Offsets past an array read zero, and entries outside
// [lo, hi) are masked when consumed, so no load sits in a branch.  NP passes
// per row are loaded before the chunk's 2:4 work, so they land during it.
//
// A delta-coded residual stores each column as its gap from the previous
// one: a lane sums its EPL gap bytes, a wave prefix sum places the lanes,
// and the row keeps the column of the entry before the cursor.
template <int DT, int NRW, int EPL, int NP, bool DELTA>
struct ResPass {
    static constexpr int PASS = 64 * EPL;                     // entries per pass
    static constexpr int CW = DELTA ? 1 : EPL;                // index words per lane per pass
    static constexpr int VW = (EPL * SN<DT>::ES + 3) / 4;     // value words per lane per pass
    int32_t lo[NRW], hi[NRW], ld[NRW];                        // entries (nnz < 2^31)
    bool open[NRW];
    int32_t base[NRW];                                        // DELTA: column of entry lo - 1 (-1 at row start)
    uint32_t cw[NRW][NP][CW];
    uint32_t vw[NRW][NP][VW];
};

template <int DT, int NRW, int EPL, int NP, bool DELTA>
__device__ __forceinline__ void residual_begin(ResPass<DT, NRW, EPL, NP, DELTA>& st, const SpmmArgs& a,
                                               const int32_t* cursor, int64_t r0, int nrows, bool first_chunk,
                                               int wave, int waves) {
    // all row bounds are read before any is used (rows past the slab read
    // its last row and are masked)
    int32_t p0[NRW], p1[NRW];
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
        const int64_t m = r0 + min(wave + waves * j, nrows - 1);
        p0[j] = a.row_ptr[m];
        p1[j] = a.row_ptr[m + 1];
    }
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
        const int rl = wave + waves * j;
        const bool valid = rl < nrows;
        st.hi[j] = valid ? (int32_t)min<int64_t>(p1[j], a.nnz_r) : 0;
        st.lo[j] = valid ? (first_chunk || cursor == nullptr ? max(p0[j], 0) : cursor[rl]) : 0;
        st.open[j] = st.lo[j] < st.hi[j];
        if constexpr (DELTA) st.base[j] = valid && !first_chunk && cursor != nullptr ? cursor[64 + rl] : -1;
    }
}

// Issue NP passes of every open row from its cursor (rounded down to a
// multiple of 4 entries, so every load is aligned to its size).
template <int DT, int NRW, int EPL, int NP, bool DELTA>
__device__ __forceinline__ void residual_load(ResPass<DT, NRW, EPL, NP, DELTA>& st, __amdgpu_buffer_rsrc_t rc,
                                              __amdgpu_buffer_rsrc_t rv, int lane) {
    using R = ResPass<DT, NRW, EPL, NP, DELTA>;
    constexpr int ES = SN<DT>::ES, IB = DELTA ? 1 : 4;        // value / index bytes per entry
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
        st.ld[j] = st.lo[j] & ~3;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            // below 2^31 + 2^12 entries' bytes: the host keeps nnz * IB under 2^31
            const uint32_t e0 = (uint32_t)st.ld[j] + (uint32_t)(R::PASS * p + EPL * lane);
            const uint32_t oc = st.open[j] ? e0 * IB : kOob;
            const uint32_t ov = st.open[j] ? e0 * ES : kOob;
            if constexpr (DELTA) {
                if constexpr (EPL == 4) st.cw[j][p][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rc, oc, 0, 0);
                else st.cw[j][p][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rc, oc, 0, 0);
            } else if constexpr (EPL == 4) {
                const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, 0);
                __builtin_memcpy(st.cw[j][p], &v, 16);
            } else {
                const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, oc, 0, 0);
                __builtin_memcpy(st.cw[j][p], &v, 8);
            }
            if constexpr (EPL * ES == 8) {
                const i32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rv, ov, 0, 0);
                __builtin_memcpy(st.vw[j][p], &v, 8);
            } else if constexpr (EPL * ES == 4) {
                st.vw[j][p][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rv, ov, 0, 0);
            } else {
                st.vw[j][p][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, ov, 0, 0);
            }
        }
    }
}

// Consume the loaded passes, row by row, pass by pass; the row's column sums
// are reduced across the wave once per row and added to res[row][16].
// Returns whether a row still has entries of this chunk past its NP passes.
template <int DT, int NRW, int EPL, int NP, bool DELTA>
__device__ __forceinline__ bool residual_consume(ResPass<DT, NRW, EPL, NP, DELTA>& st, const uint8_t* ldsb,
                                                 void* res, int64_t kc0, int64_t kc1, int wave, int waves,
                                                 int lane) {
    using R = ResPass<DT, NRW, EPL, NP, DELTA>;
    constexpr int ES = SN<DT>::ES;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    bool any = false;
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
        if (!st.open[j]) continue;
        S acc[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[n] = S(0);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (!st.open[j]) break;
            const int64_t e0 = (int64_t)st.ld[j] + R::PASS * p + EPL * lane;
            bool v[EPL];
#pragma unroll
            for (int i = 0; i < EPL; ++i) v[i] = e0 + i >= st.lo[j] && e0 + i < st.hi[j];
            int32_t col[EPL];
            if constexpr (DELTA) {
                int pre[EPL], sum = 0;
#pragma unroll
                for (int i = 0; i < EPL; ++i) {
                    sum += v[i] ? (int)((st.cw[j][p][0] >> (8 * i)) & 0xFFu) : 0;
                    pre[i] = sum;
                }
                const int incl = wave_incl_sum(sum, lane);
#pragma unroll
                for (int i = 0; i < EPL; ++i) col[i] = st.base[j] + (incl - sum) + pre[i];
            } else {
#pragma unroll
                for (int i = 0; i < EPL; ++i) col[i] = (int32_t)st.cw[j][p][i];
            }
            // B rows of the pass's entries in this chunk (row 0 for the
            // others, whose value is zeroed), all reads before the products
            uint4 w[EPL][2];
            S vv[EPL];
            int taken = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int32_t cc = v[i] ? col[i] : (int32_t)kc1;
                taken += __popcll(__ballot(cc < kc1));
                const bool inch = cc >= kc0 && cc < kc1;
                const uint8_t* brow = ldsb + (inch ? (int)(cc - kc0) : 0) * 16 * ES;
                w[i][0] = *reinterpret_cast<const uint4*>(brow);
                if constexpr (ES == 2) w[i][1] = *reinterpret_cast<const uint4*>(brow + 16);
                if constexpr (DT == DT_I8) {
                    const int32_t x = (int32_t)(int8_t)(st.vw[j][p][0] >> (8 * i));
                    vv[i] = inch ? x : 0;
                } else if constexpr (ES == 1) {
                    vv[i] = inch ? elem_to_f32<DT>(st.vw[j][p][0] >> (8 * i)) : 0.0f;
                } else {
                    const uint16_t x = (uint16_t)(st.vw[j][p][i >> 1] >> (16 * (i & 1)));
                    vv[i] = inch ? elem_to_f32<DT>(x) : 0.0f;
                }
            }
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                if constexpr (DT == DT_I8) {
                    int8_t bv[16];
                    __builtin_memcpy(bv, &w[i][0], 16);
#pragma unroll
                    for (int n = 0; n < 16; ++n) acc[n] += vv[i] * (int32_t)bv[n];
                } else if constexpr (ES == 1) {
                    uint8_t bv[16];
                    __builtin_memcpy(bv, &w[i][0], 16);
#pragma unroll
                    for (int n = 0; n < 16; ++n) acc[n] = fmaf(vv[i], elem_to_f32<DT>(bv[n]), acc[n]);
                } else {
                    uint16_t bv[16];
                    __builtin_memcpy(bv, &w[i][0], 16);
                    __builtin_memcpy(bv + 8, &w[i][1], 16);
#pragma unroll
                    for (int n = 0; n < 16; ++n) acc[n] = fmaf(vv[i], elem_to_f32<DT>(bv[n]), acc[n]);
                }
            }
            if constexpr (DELTA) {
                // the column of the last entry taken is the next base
                if (taken > 0) {
                    const int t = st.lo[j] + taken - 1 - (st.ld[j] + R::PASS * p);
#pragma unroll
                    for (int i = 0; i < EPL; ++i)
                        if (t % EPL == i) st.base[j] = __builtin_amdgcn_readlane(col[i], t / EPL);
                }
            }
            st.lo[j] += taken;
            // the pass was consumed to its end: the row goes on in the next
            // pass; otherwise it reached a column of a later chunk or its end
            st.open[j] = st.lo[j] < st.hi[j] && st.lo[j] == st.ld[j] + R::PASS * (p + 1);
        }
        const S tot = transpose_sum16<S>(acc, lane);
        const int rl = wave + waves * j;
        if (lane < 16) reinterpret_cast<S*>(res)[rl * 16 + transpose_col(lane)] += tot;
        any |= st.open[j];
    }
    return any;
}

// Rows closed at the end of a chunk that still have entries go on in the next.
template <int DT, int NRW, int EPL, int NP, bool DELTA>
__device__ __forceinline__ void residual_reopen(ResPass<DT, NRW, EPL, NP, DELTA>& st) {
#pragma unroll
    for (int j = 0; j < NRW; ++j) st.open[j] = st.lo[j] < st.hi[j];
}

template <int DT, int NRW, int EPL, int NP, bool DELTA>
__device__ __forceinline__ void residual_end(const ResPass<DT, NRW, EPL, NP, DELTA>& st, int32_t* cursor, int nrows,
                                             int wave, int waves, int lane) {
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
        const int rl = wave + waves * j;
        if (rl < nrows && lane == 0) {
            cursor[rl] = st.lo[j];
            if constexpr (DELTA) cursor[64 + rl] = st.base[j];
        }
    }
}

// One workgroup owns a slab of <= 16*TM rows and all of K.  Wave w takes the
// k-steps w, w + W, w + 2W, ... (W waves), so the waves walk K together and
// share each B chunk.  A wave keeps the sparse fragments of its next P
// k-steps in flight in a register ring and refills a slot as soon as the
// slot's k-step has been multiplied: the weight stream of every CU stays
// P x TM KiB per wave deep from the first cycle to the last.
template <int DT, int TM, int P, bool DELTA>
__global__ void __launch_bounds__(kWaves * 64) k_spmm_small_n(SpmmArgs a, int rows_per_wg, int chunk_steps,
                                                              int vec_b, int vec_m) {
    constexpr int W = kWaves;
    constexpr int kResRows = (16 * TM + W - 1) / W;   // residual rows per wave (dealt round-robin)
    constexpr int kResEPL = kResRows > 4 ? 2 : 4;        // residual entries per lane per pass
    constexpr int kResNP = kResRows > 4 ? 1 : 2;         // residual passes per row loaded at once
    using T = SN<DT>;
    using Acc = AccT<DT>;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsData + kLdsRes + kLdsCursor];
    uint8_t* ldsb = lds;
    uint8_t* ldsm = lds + chunk_steps * 16 * T::ES * T::KS;
    void* res = lds + kLdsData;
    int32_t* cursor = reinterpret_cast<int32_t*>(lds + kLdsData + kLdsRes);
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(const lds_void*)lds;   // LDS byte address of `lds`

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)min<int64_t>(rows_per_wg, a.M - r0);
    const int64_t ksteps = a.K / T::KS;
    const bool residual = a.row_ptr != nullptr;
    const bool l24 = a.vals != nullptr;                 // false: the residual alone (unstructured product)
    const int q = lane >> 4, rl = lane & 15;
    // residual arrays as buffers (the host keeps each under 2^31 bytes and
    // aligns it to 4 entries' bytes)
    const __amdgpu_buffer_rsrc_t rcol = DELTA ? rsrc_aligned<4>(a.dcol, a.nnz_r) : rsrc_aligned<16>(a.col, a.nnz_r * 4);
    const __amdgpu_buffer_rsrc_t rval = rsrc_aligned<4 * T::ES>(a.rvals, a.nnz_r * T::ES);

    // sparse operand of lane l for k-step g, tile t: row r0 + 16t + l%16,
    // stored values [q*VALS/4, (q+1)*VALS/4) of the k-step, q = l/16
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vals) + (r0 + rl) * a.ldv * T::ES + q * 16;
    const int64_t vstep = (int64_t)T::VALS * T::ES;
    const int64_t vtile = 16 * a.ldv * T::ES;
    auto load_a = [&](int64_t g, uint4 (&f)[TM]) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
            f[t] = (16 * t + rl < nrows && g < ksteps) ? *reinterpret_cast<const uint4*>(vbase + t * vtile + g * vstep)
                                                      : make_uint4(0, 0, 0, 0);
    };

    if (residual)
        for (int i = threadIdx.x; i < kTMax * 16 * 16; i += blockDim.x) reinterpret_cast<S*>(res)[i] = S(0);

    Acc acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = Acc{0, 0, 0, 0};

    uint4 ring[P][TM];
    const int64_t nchunks = (ksteps + chunk_steps - 1) / chunk_steps;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t c0 = c * chunk_steps;
        const int csteps = (int)min<int64_t>(chunk_steps, ksteps - c0);
        const int pitch = csteps * T::META + 4;
        if (c > 0) lds_barrier();                         // previous chunk's B and metadata consumed
        // The ring's first loads go out before the chunk's B rows and
        // metadata: waiting for the staging loads then also waits for them
        // (loads complete in order), but the weight stream is already running.
        if (vec_b) dma_b<DT>(a, lds_addr, c0 * T::KS, csteps * T::KS, wave);
        if (vec_m && l24) dma_meta<DT>(a, lds_addr + (uint32_t)(ldsm - lds), r0, nrows, c0, csteps, pitch, wave);
        if (c == 0 && l24) {
#pragma unroll
            for (int u = 0; u < P; ++u) load_a(wave + (int64_t)W * u, ring[u]);
        }
        // this wave's B and metadata loads have landed (with the ring's first
        // loads, which the first multiply waits for anyway)
        wait_vm<0>();
        // the chunk's first residual passes are in flight during its 2:4 work
        ResPass<DT, kResRows, kResEPL, kResNP, DELTA> rp;
        if (residual) {
            residual_begin(rp, a, cursor, r0, nrows, c == 0, wave, W);
            residual_load(rp, rcol, rval, lane);
        }
        if (!vec_b) stage_b<DT>(a, ldsb, c0 * T::KS, csteps * T::KS, false);
        if (!vec_m && l24) stage_meta<DT>(a, ldsm, r0, nrows, c0, csteps, pitch, false);
        lds_barrier();

        // this wave's k-steps of the chunk: local kk = wave + W*i; a full
        // chunk holds a multiple of W*P k-steps, so ring slot i % P belongs
        // to the wave's global k-step sequence across chunks
        const int nw = l24 && csteps > wave ? (csteps - wave + W - 1) / W : 0;
        for (int i0 = 0; i0 < nw; i0 += P) {
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const int i = i0 + u;
                if (i < nw) {
                    const int kk = wave + W * i;
                    uint4 b[2];
                    load_b_operand<DT>(ldsb, kk, lane, b);
#pragma unroll
                    for (int t = 0; t < TM; ++t) {
                        const uint8_t* mp = ldsm + (16 * t + rl) * pitch + kk * T::META + q * (T::META / 4);
                        uint32_t ix;
                        if constexpr (SN<DT>::META == 16) ix = *reinterpret_cast<const uint32_t*>(mp);
                        else ix = *reinterpret_cast<const uint16_t*>(mp);
                        acc[t] = smfmac<DT>(ring[u][t], b, acc[t], ix);
                    }
                    load_a(c0 + kk + (int64_t)W * P, ring[u]);
                }
            }
        }
        if (residual) {
            while (residual_consume(rp, ldsb, res, c0 * T::KS, (c0 + csteps) * T::KS, wave, W, lane))
                residual_load(rp, rcol, rval, lane);
            residual_end(rp, cursor, nrows, wave, W, lane);
        }
    }
    lds_barrier();

    // fixed-order reduction of the waves' partial tiles
    Acc* red = reinterpret_cast<Acc*>(ldsb);
#pragma unroll
    for (int t = 0; t < TM; ++t) red[(wave * kTMax + t) * 64 + lane] = acc[t];
    lds_barrier();
    const int tiles = (nrows + 15) >> 4;
    for (int i = threadIdx.x; i < tiles * 256; i += blockDim.x) {
        const int t = i >> 8, ln = (i >> 2) & 63, r = i & 3;
        S sum = S(0);
#pragma unroll
        for (int w = 0; w < W; ++w) sum += reinterpret_cast<const S*>(red)[((w * kTMax + t) * 64 + ln) * 4 + r];
        const int row = 16 * t + 4 * (ln >> 4) + r, col = ln & 15;
        if (row < nrows && col < a.N) {
            if (residual) sum += reinterpret_cast<const S*>(res)[row * 16 + col];
            reinterpret_cast<S*>(a.C)[(r0 + row) * a.ldc + col] = sum;
        }
    }
}

// Variant for products whose B is one contiguous K x 16 block.  The slab's
// metadata rows (all of K) are staged once, in 256-byte row segments,
// behind the only barrier before the final reduction.  After that every
// wave fetches what its k-steps need on its own -- the two 1 KiB pieces of
// B rows (direct to a private LDS slot) and the sparse fragments (to
// registers) -- as buffer loads from inline assembly.  A k-step beyond K or
// a row beyond the slab uses an offset past its buffer, which reads zero, so
// every wave issues the same GOPS loads per k-step and one hand-counted wait
// per k-step is exact.
//
// With a residual (RES), the 2:4 sums go to LDS instead of C and the
// residual follows as an epilogue: the whole LDS (but the row sums) then
// holds chunks of B in turn, and each wave's residual rows are consumed
// chunk by chunk, their first passes loaded while the 2:4 stream drains and
// the next chunk's while its B rows are staged.  A workgroup that finishes
// its weight stream early runs its epilogue while others still stream.
template <int DT, int TM, int P, bool RES, bool DELTA>
__global__ void __launch_bounds__(kWaves * 64) k_spmm_small_n_ring(SpmmArgs a, int rows_per_wg) {
    constexpr int W = kWaves;
    using T = SN<DT>;
    using Acc = AccT<DT>;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    constexpr int BSTEP = 16 * T::ES * T::KS;           // B bytes per k-step (2 KiB)
    constexpr int GOPS = 2 + TM;                        // loads per k-step per wave
    static_assert(P * GOPS < 64, "vmcnt");
    static_assert(W * kTMax * 1024 <= W * P * BSTEP, "LDS");
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];   // B slots, then the metadata rows
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(const lds_void*)lds;
    uint8_t* ldsm = lds + W * P * BSTEP;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int nrows = (int)min<int64_t>(rows_per_wg, a.M - r0);
    const int64_t ksteps = a.K / T::KS;
    const int q = lane >> 4, rl = lane & 15;
    const int pitch = (int)(ksteps * T::META) + 4;      // metadata row pitch in LDS (padded against conflicts)

    const __amdgpu_buffer_rsrc_t rv = rsrc(reinterpret_cast<const uint8_t*>(a.vals) + r0 * a.ldv * T::ES,
                                           ((a.M - r0 - 1) * a.ldv + a.K / 2) * T::ES);
    const __amdgpu_buffer_rsrc_t rb = rsrc(a.B, a.K * 16 * T::ES);
    uint32_t voff[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
        voff[t] = 16 * t + rl < nrows ? (uint32_t)((16 * t + rl) * a.ldv * T::ES + q * 16) : kOob;

    i32x4 av[P][TM] = {};   // native vector registers, so they can be tied to the waits below
    // k-step g of this wave into ring slot u
    auto issue = [&](int64_t g, int u) {
        const bool in = g < ksteps;
        const uint32_t slot = lds_addr + (uint32_t)((wave * P + u) * BSTEP);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            dma<16>(rb, slot + j * 1024, in ? (uint32_t)(g * BSTEP + j * 1024 + lane * 16) : kOob);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const uint32_t o = in ? voff[t] + (uint32_t)(g * T::VALS * T::ES) : kOob;
            asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(av[u][t]) : "v"(o), "s"(rv) : "memory");
        }
    };

    Acc acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = Acc{0, 0, 0, 0};
    // without a 2:4 layer (an unstructured product of the residual alone)
    // the weight stream is empty
    const bool l24 = a.vals != nullptr;
    if (l24) {
        dma_meta<DT>(a, lds_addr + (uint32_t)(W * P * BSTEP), r0, nrows, 0, (int)ksteps, pitch, wave);
#pragma unroll
        for (int u = 0; u < P; ++u) issue(wave + (int64_t)W * u, u);
    }
    // residual rows of this wave: their bounds are read now, behind the
    // first k-steps' loads
    constexpr int kResRows = (16 * TM + W - 1) / W;
    constexpr int kResEPL = kResRows > 4 ? 2 : 4;
    constexpr int kResNP = kResRows > 4 ? 1 : 2;
    ResPass<DT, kResRows, kResEPL, kResNP, DELTA> rp;
    if constexpr (RES) residual_begin(rp, a, nullptr, r0, nrows, true, wave, W);
    wait_vm<P * GOPS>();                                // this wave's metadata segments have landed
    lds_barrier();                                      // and every other wave's
    const int nw = l24 && ksteps > wave ? (int)((ksteps - wave + W - 1) / W) : 0;
    for (int i0 = 0; i0 < nw; i0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int i = i0 + u;
            if (i < nw) {
                // the oldest k-step in flight has landed once only the P-1
                // younger ones remain; its registers are tied to the wait so
                // no use moves above it
                wait_vm<(P - 1) * GOPS>();
#pragma unroll
                for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(av[u][t]));
                uint4 b[2];
                load_b_operand<DT>(lds + (wave * P + u) * BSTEP, 0, lane, b);
                const int64_t g = wave + (int64_t)W * i;
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    const uint8_t* mp = ldsm + (16 * t + rl) * pitch + g * T::META + q * (T::META / 4);
                    uint32_t ix;
                    if constexpr (SN<DT>::META == 16) ix = *reinterpret_cast<const uint32_t*>(mp);
                    else ix = *reinterpret_cast<const uint16_t*>(mp);
                    uint4 f;
                    __builtin_memcpy(&f, &av[u][t], 16);
                    acc[t] = smfmac<DT>(f, b, acc[t], ix);
                }
                // the slot's LDS reads are done before its next B rows land
                __builtin_amdgcn_s_waitcnt(0xC07F);
                issue(wave + (int64_t)W * (i + P), u);
            }
        }
    }
    // residual: the first passes go out while the weight stream drains
    const __amdgpu_buffer_rsrc_t rcol = DELTA ? rsrc_aligned<4>(a.dcol, a.nnz_r)
                                              : rsrc_aligned<16>(a.col, a.nnz_r * 4);
    const __amdgpu_buffer_rsrc_t rval = rsrc_aligned<4 * T::ES>(a.rvals, a.nnz_r * T::ES);
    if constexpr (RES) residual_load(rp, rcol, rval, lane);
    // the loads past the wave's last k-step land before the LDS is reused --
    // and before their registers are: the compiler takes an asm load's
    // output as written when the load is issued, so the ring stays in use
    // until the wait (else a late load could overwrite a reassigned register)
    wait_vm<0>();
#pragma unroll
    for (int u = 0; u < P; ++u)
#pragma unroll
        for (int t = 0; t < TM; ++t) asm volatile("" ::"v"(av[u][t]));
    lds_barrier();

    // fixed-order reduction of the waves' partial tiles
    Acc* red = reinterpret_cast<Acc*>(lds);
    S* res = reinterpret_cast<S*>(lds + kRingResOff);   // RES: the slab's row sums [64][16]
#pragma unroll
    for (int t = 0; t < TM; ++t) red[(wave * kTMax + t) * 64 + lane] = acc[t];
    lds_barrier();
    const int tiles = (nrows + 15) >> 4;
    for (int i = threadIdx.x; i < tiles * 256; i += blockDim.x) {
        const int t = i >> 8, ln = (i >> 2) & 63, r = i & 3;
        S sum = S(0);
#pragma unroll
        for (int w = 0; w < W; ++w) sum += reinterpret_cast<const S*>(red)[((w * kTMax + t) * 64 + ln) * 4 + r];
        const int row = 16 * t + 4 * (ln >> 4) + r, col = ln & 15;
        if constexpr (RES) res[row * 16 + col] = sum;
        else if (row < nrows && col < a.N) reinterpret_cast<S*>(a.C)[(r0 + row) * a.ldc + col] = sum;
    }
    if constexpr (RES) {
        // B in chunks over the LDS below the row sums
        constexpr int64_t kChunkRows = kRingResOff / (16 * T::ES);
        for (int64_t k0 = 0; k0 < a.K; k0 += kChunkRows) {
            const int rows = (int)min<int64_t>(kChunkRows, a.K - k0);
            lds_barrier();                                  // the previous chunk (or the partial tiles) consumed
            dma_b<DT>(a, lds_addr, k0, rows, wave);
            wait_vm<0>();                                   // this wave's B rows and residual passes
            lds_barrier();
            while (residual_consume(rp, lds, res, k0, k0 + rows, wave, W, lane)) residual_load(rp, rcol, rval, lane);
            if (k0 + rows < a.K) {
                residual_reopen(rp);
                residual_load(rp, rcol, rval, lane);
            }
        }
        lds_barrier();
        for (int i = threadIdx.x; i < nrows * 16; i += blockDim.x) {
            const int row = i >> 4, col = i & 15;
            if (col < a.N) reinterpret_cast<S*>(a.C)[(r0 + row) * a.ldc + col] = res[i];
        }
    }
}

// ---- packed decode layout --------------------------------------------------
//
// The decode kernel's sparse operand in the order it is consumed: for each
// 16-row tile and k-step, the 64 lanes' fragments (lane l = 16q + r holds
// row r's stored values [q*VALS/4, (q+1)*VALS/4) of the k-step, 16 bytes)
// as one 1 KiB block, and their index words (the 2 or 4 metadata bytes the
// sparse MFMA takes per lane) as one 128- or 256-byte block.  A tile's
// blocks are consecutive in k.  Rows past M are zero.  The product reads
// each block with one fully coalesced load per wave instead of 16 row
// pieces of 64 bytes, and needs no metadata staging.

template <int DT>
__global__ void __launch_bounds__(256) k_pack(int64_t M, int64_t K, const uint8_t* vals, int64_t ldv_bytes,
                                              const uint8_t* meta, int64_t ldm, uint8_t* pvals, uint8_t* pmeta) {
    using T = SN<DT>;
    constexpr int IDXB = T::META / 4;
    const int64_t ksteps = K / T::KS, tiles = (M + 15) / 16;
    const int64_t n = tiles * ksteps * 64;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(i & 63);
        const int64_t blk = i >> 6, tile = blk / ksteps, g = blk - tile * ksteps;
        const int64_t row = 16 * tile + (lane & 15);
        const int q = lane >> 4;
        uint4 v = make_uint4(0, 0, 0, 0);
        uint8_t mb[IDXB] = {};
        if (row < M) {
            v = *reinterpret_cast<const uint4*>(vals + row * ldv_bytes + g * T::VALS * T::ES + q * 16);
#pragma unroll
            for (int b = 0; b < IDXB; ++b) mb[b] = meta[row * ldm + g * T::META + q * IDXB + b];
        }
        *reinterpret_cast<uint4*>(pvals + i * 16) = v;
#pragma unroll
        for (int b = 0; b < IDXB; ++b) pmeta[i * IDXB + b] = mb[b];
    }
}

// Product on the packed layout (B one contiguous K x 16 block): the ring
// kernel's scheme with the index words loaded per k-step next to the
// fragments, so nothing is staged before the loop.  Workgroup b takes the
// tiles [b*T/G, (b+1)*T/G) (at most TM); tiles past its range read zero.
// With a residual (RES) the workgroup's rows get the ring kernel's residual
// epilogue: the 2:4 sums go to LDS, the first residual passes are loaded
// while the weight stream drains, then B is staged in chunks over the LDS
// below the row sums and the residual rows are consumed chunk by chunk.
// With activation-major B (BT: a.B is Bt [N, K] row-major, N <= 16, row
// stride a.ldb) each lane loads its own B operand of a k-step straight into
// registers: column n = l % 16, block bb = l / 16 holds dense k (e / H) *
// (KS / 2) + H * bb + e % H, which is two 16-byte pieces of row n of Bt, at k
// offsets H * bb and KS / 2 + H * bb (H = KS / 8 elements).  A load then
// reads 64 contiguous bytes of each of 16 rows, nothing passes through LDS
// and no transposing read is needed; rows past N read zero.
template <int DT, int TM, int P, bool RES, bool DELTA, bool BT = false>
__global__ void __launch_bounds__(kWaves * 64) k_spmm_packed(SpmmArgs a, const uint8_t* pvals, const uint8_t* pmeta,
                                                             int64_t tiles) {
    constexpr int W = kWaves;
    using T = SN<DT>;
    using Acc = AccT<DT>;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    constexpr int IDXB = T::META / 4;                   // index bytes per lane per k-step
    constexpr int BSTEP = 16 * T::ES * T::KS;           // B bytes per k-step (2 KiB)
    constexpr int GOPS = 2 + 2 * TM;                    // loads per k-step per wave
    static_assert(P * GOPS < 64, "vmcnt");
    static_assert(W * kTMax * 1024 <= W * P * BSTEP, "LDS");
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];   // the waves' B slots
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(const lds_void*)lds;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)blockIdx.x * tiles / gridDim.x, t1 = ((int64_t)blockIdx.x + 1) * tiles / gridDim.x;
    const int nt = (int)(t1 - t0);
    const int64_t ksteps = a.K / T::KS;

    const __amdgpu_buffer_rsrc_t rv = rsrc(pvals, tiles * ksteps * 1024);
    const __amdgpu_buffer_rsrc_t rm = rsrc(pmeta, tiles * ksteps * 64 * IDXB);
    const __amdgpu_buffer_rsrc_t rb = BT ? rsrc(a.B, ((a.N - 1) * a.ldb + a.K) * T::ES) : rsrc(a.B, a.K * 16 * T::ES);
    uint32_t voff[TM], moff[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        voff[t] = t < nt ? (uint32_t)(((t0 + t) * ksteps * 64 + lane) * 16) : kOob;
        moff[t] = t < nt ? (uint32_t)(((t0 + t) * ksteps * 64 + lane) * IDXB) : kOob;
    }
    // BT: this lane's piece of row lane % 16 of Bt at k-step 0 (a row past N
    // is an offset past the buffer)
    const uint32_t bt_off = (lane & 15) < a.N
                                ? (uint32_t)(((lane & 15) * a.ldb + (lane >> 4) * (T::KS / 8)) * T::ES)
                                : kOob;

    i32x4 av[P][TM] = {};   // native vector registers, so they can be tied to the waits below
    int mv[P][TM] = {};
    i32x4 bv[P][2] = {};    // BT: the wave's B operand of each k-step in flight
    auto issue = [&](int64_t g, int u) {
        const bool in = g < ksteps;
        const uint32_t slot = lds_addr + (uint32_t)((wave * P + u) * BSTEP);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (BT) {
                const uint32_t ob = in && bt_off != kOob ? bt_off + (uint32_t)((g * T::KS + j * (T::KS / 2)) * T::ES) : kOob;
                asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(bv[u][j]) : "v"(ob), "s"(rb) : "memory");
            } else {
                dma<16>(rb, slot + j * 1024, in ? (uint32_t)(g * BSTEP + j * 1024 + lane * 16) : kOob);
            }
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const uint32_t o = in ? voff[t] + (uint32_t)(g * 1024) : kOob;
            const uint32_t om = in ? moff[t] + (uint32_t)(g * 64 * IDXB) : kOob;
            // non-temporal: every line of the packed blocks is read once, whole,
            // so nothing is lost by not keeping it, and B stays in L2
            asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen nt" : "=v"(av[u][t]) : "v"(o), "s"(rv) : "memory");
            if constexpr (IDXB == 4)
                asm volatile("buffer_load_dword %0, %1, %2, 0 offen nt" : "=v"(mv[u][t]) : "v"(om), "s"(rm) : "memory");
            else
                asm volatile("buffer_load_ushort %0, %1, %2, 0 offen nt" : "=v"(mv[u][t]) : "v"(om), "s"(rm) : "memory");
        }
    };

    Acc acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = Acc{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < P; ++u) issue(wave + (int64_t)W * u, u);
    // residual rows of the workgroup (rows [r0, r0 + nrows)): their bounds
    // are read now, behind the first k-steps' loads
    const int64_t r0 = 16 * t0;
    const int nrows = (int)min<int64_t>(16 * nt, a.M - r0);
    constexpr int kResRows = (16 * TM + W - 1) / W;
    constexpr int kResEPL = kResRows > 4 ? 2 : 4;
    constexpr int kResNP = kResRows > 4 ? 1 : 2;
    ResPass<DT, kResRows, kResEPL, kResNP, DELTA> rp;
    if constexpr (RES) residual_begin(rp, a, nullptr, r0, nrows, true, wave, W);
    const int nw = ksteps > wave ? (int)((ksteps - wave + W - 1) / W) : 0;
    for (int i0 = 0; i0 < nw; i0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int i = i0 + u;
            if (i < nw) {
                // the oldest k-step in flight has landed once only the P-1
                // younger ones remain; its registers are tied to the wait so
                // no use moves above it
                wait_vm<(P - 1) * GOPS>();
#pragma unroll
                for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(av[u][t]), "+v"(mv[u][t]));
                uint4 b[2];
                if constexpr (BT) {
                    asm volatile("" : "+v"(bv[u][0]));
                    asm volatile("" : "+v"(bv[u][1]));
                    __builtin_memcpy(&b[0], &bv[u][0], 16);
                    __builtin_memcpy(&b[1], &bv[u][1], 16);
                } else {
                    load_b_operand<DT>(lds + (wave * P + u) * BSTEP, 0, lane, b);
                }
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    uint4 f;
                    __builtin_memcpy(&f, &av[u][t], 16);
                    acc[t] = smfmac<DT>(f, b, acc[t], (uint32_t)mv[u][t]);
                }
                // the slot's LDS reads are done before its next B rows land
                __builtin_amdgcn_s_waitcnt(0xC07F);
                issue(wave + (int64_t)W * (i + P), u);
            }
        }
    }
    // residual: the first passes go out while the weight stream drains
    const __amdgpu_buffer_rsrc_t rcol = DELTA ? rsrc_aligned<4>(a.dcol, a.nnz_r)
                                              : rsrc_aligned<16>(a.col, a.nnz_r * 4);
    const __amdgpu_buffer_rsrc_t rval = rsrc_aligned<4 * T::ES>(a.rvals, a.nnz_r * T::ES);
    if constexpr (RES) residual_load(rp, rcol, rval, lane);
    // the loads past the wave's last k-step land before the LDS is reused,
    // and before their registers are (an asm load's output counts as
    // written when issued, so the ring stays in use until the wait)
    wait_vm<0>();
#pragma unroll
    for (int u = 0; u < P; ++u) {
#pragma unroll
        for (int t = 0; t < TM; ++t) asm volatile("" ::"v"(av[u][t]), "v"(mv[u][t]));
        if constexpr (BT) asm volatile("" ::"v"(bv[u][0]), "v"(bv[u][1]));
    }
    lds_barrier();

    // fixed-order reduction of the waves' partial tiles
    Acc* red = reinterpret_cast<Acc*>(lds);
    S* res = reinterpret_cast<S*>(lds + kRingResOff);   // RES: the rows' sums [64][16]
#pragma unroll
    for (int t = 0; t < TM; ++t) red[(wave * kTMax + t) * 64 + lane] = acc[t];
    lds_barrier();
    for (int i = threadIdx.x; i < nt * 256; i += blockDim.x) {
        const int t = i >> 8, ln = (i >> 2) & 63, r = i & 3;
        S sum = S(0);
#pragma unroll
        for (int w = 0; w < W; ++w) sum += reinterpret_cast<const S*>(red)[((w * kTMax + t) * 64 + ln) * 4 + r];
        const int lrow = 16 * t + 4 * (ln >> 4) + r;
        const int64_t row = r0 + lrow;
        const int col = ln & 15;
        if constexpr (RES) res[lrow * 16 + col] = sum;
        else if (row < a.M && col < a.N) reinterpret_cast<S*>(a.C)[row * a.ldc + col] = sum;
    }
    if constexpr (RES) {
        // B in chunks over the LDS below the row sums
        constexpr int64_t kChunkRows = kRingResOff / (16 * T::ES);
        for (int64_t k0 = 0; k0 < a.K; k0 += kChunkRows) {
            const int rows = (int)min<int64_t>(kChunkRows, a.K - k0);
            lds_barrier();                                  // the previous chunk (or the partial tiles) consumed
            dma_b<DT>(a, lds_addr, k0, rows, wave);
            wait_vm<0>();                                   // this wave's B rows and residual passes
            lds_barrier();
            while (residual_consume(rp, lds, res, k0, k0 + rows, wave, W, lane)) residual_load(rp, rcol, rval, lane);
            if (k0 + rows < a.K) {
                residual_reopen(rp);
                residual_load(rp, rcol, rval, lane);
            }
        }
        lds_barrier();
        for (int i = threadIdx.x; i < nrows * 16; i += blockDim.x) {
            const int row = i >> 4, col = i & 15;
            if (col < a.N) reinterpret_cast<S*>(a.C)[(r0 + row) * a.ldc + col] = res[i];
        }
    }
}

// ---- complement-bitmap residual, fused into the packed decode product -------
//
// A residual entry of a group can only sit at one of the two positions the
// 2:4 layer did not keep.  Stored per packed block (16 rows x one k-step) as
// a 2-bit-per-group mask word per lane over those positions, a block offset
// and the values in lane order, the residual's share of a lane's operand is
// itself a 2:4 operand: the values at the complement positions (zeros where
// the mask bit is clear) with the index word whose nibbles are the
// complements of the 2:4 layer's.  It rides the same B operand and the same
// sparse MFMA in every k-step, so the residual bytes stream with the 2:4
// layer's instead of after them ("How sparse LLM weights cut GPU inference
// cost without quantization", section "How the three-layer format makes
// moderate sparsity fast": the layers are decoded on chip in one pipeline).

// Complement of every nibble of an index word: kept pair {i0, i1} -> the
// other two positions, ascending.  For the six valid nibbles this is
// n ^ 0xA for the pairs (0, 1) and (2, 3) -- the nibbles with bit 3 clear or
// bits 2 and 1 both set -- and n ^ 0x5 for the other four.
__device__ __forceinline__ uint32_t complement_index(uint32_t n) {
    const uint32_t pair01_23 = ((~n >> 3) | ((n >> 2) & (n >> 1))) & 0x11111111u;
    return n ^ 0x55555555u ^ ((pair01_23 << 4) - pair01_23);
}

template <int DT> struct Cbm {
    static constexpr int IDXB = SN<DT>::META / 4;          // index bytes per lane per k-step (2 / 4)
    static constexpr int MB = IDXB / 2;                    // mask bytes per lane (1 / 2)
    static constexpr int SLOTS = 8 * MB;                   // complement slots per lane (8 / 16)
    static constexpr int BSTEP = 16 * SN<DT>::ES * SN<DT>::KS;
    static constexpr int LX = 4;                           // k-steps of fragments, masks, offsets and B in flight
    static constexpr int LY = 2;                           // k-steps of residual value windows in flight
    static constexpr int YWIN = 2048;                      // a block's values: at most 1 KiB plus alignment
    // LDS per wave: B slots (row-major B only), value windows, 16 zero bytes
    template <int TM, bool BT> static constexpr int wave_lds() {
        return (BT ? 0 : LX * BSTEP) + LY * TM * YWIN + 16;
    }
};

// Residual operand of a lane from its block's value window in LDS: slot s
// (group s / 2, complement position s % 2) holds the value of rank
// popcount(mask below s) among the lane's values if mask bit s is set, else
// zero (read from a zeroed pad, so no slot takes a branch).
template <int DT>
__device__ __forceinline__ uint4 cbm_operand(const uint8_t* win, uint32_t zoff, uint32_t e0, uint32_t mask) {
    constexpr int ES = SN<DT>::ES;
    uint32_t w[4];
    if constexpr (ES == 2) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t h[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int sl = 2 * d + j;
                const uint32_t rank = __popc(mask & ((1u << sl) - 1u));
                const uint32_t off = (mask >> sl & 1u) ? 2u * (e0 + rank) : zoff;
                h[j] = *reinterpret_cast<const uint16_t*>(win + off);
            }
            w[d] = h[0] | (h[1] << 16);
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t x = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sl = 4 * d + j;
                const uint32_t rank = __popc(mask & ((1u << sl) - 1u));
                const uint32_t off = (mask >> sl & 1u) ? e0 + rank : zoff;
                x |= (uint32_t)win[off] << (8 * j);
            }
            w[d] = x;
        }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Packed decode product with a complement-bitmap residual (B one contiguous
// K x 16 block).  Per wave and k-step g: the 2:4 fragments, index words and
// mask words of its tiles plus its two 1 KiB pieces of B rows (group X(g),
// LX k-steps ahead, with the tiles' block offsets by scalar loads), and the
// value windows of its tiles' blocks (group Y(g), LY k-steps ahead: one
// direct-to-LDS load of 1 KiB per tile, two for the rare block whose values
// span more than that from the 16-byte piece holding its first; their
// addresses need the block offsets, so a Y group is issued once its X group
// has landed).  Iteration i waits until only the previous iteration's two
// groups are outstanding, multiplies k-step g_i, then issues Y(g_{i+LY})
// and X(g_{i+LX}).  Every wave issues at least the vector loads the waits
// count (a k-step past K, a tile past the range or a window piece past a
// block's values reads zero from an out-of-range offset), so each wait is
// exact or, after a second window load, stricter.  Partial tiles are summed
// in wave order as in the plain packed product.  With activation-major B
// (BT) the two B pieces of an X group are the lane's own B operand, loaded
// straight into registers as in the plain packed product.
template <int DT, int TM, int W, bool BT = false>
__global__ void __launch_bounds__(W * 64) k_spmm_packed_cbm(SpmmArgs a, const uint8_t* pvals, const uint8_t* pmeta,
                                                            const uint8_t* rmask, const int32_t* roff,
                                                            const uint8_t* cvals, int64_t nvals, int64_t tiles) {
    using T = SN<DT>;
    using C = Cbm<DT>;
    using Acc = AccT<DT>;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    constexpr int LX = C::LX, LY = C::LY, IDXB = C::IDXB, MB = C::MB;
    constexpr int GX = 2 + 3 * TM;                      // vector loads of an X group per wave
    // loads of a Y group per wave: one per tile, plus one for a tile whose
    // window (its block's values, from the 16-byte piece that holds the
    // first) spans more than 1 KiB.  The waits count one per tile: an extra
    // load makes a wait stricter (loads complete in issue order), never
    // looser.
    constexpr int GY = TM;
    constexpr int WL = C::template wave_lds<TM, BT>();
    static_assert(LX % LY == 0 && GX + GY < 64, "ring");
    static_assert(W * WL <= 160 * 1024 && W * kTMax * 1024 <= W * WL, "LDS");
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(const lds_void*)lds;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)blockIdx.x * TM;
    const int nt = (int)min<int64_t>(TM, tiles - t0);
    const int64_t ksteps = a.K / T::KS;
    const uint32_t wbase = (uint32_t)(wave * WL);                 // this wave's LDS region
    const uint32_t ybase = wbase + (BT ? 0 : LX * C::BSTEP);     // its value windows
    const uint32_t zpad = ybase + LY * TM * C::YWIN;              // 16 zero bytes
    if (lane == 0) *reinterpret_cast<uint4*>(lds + zpad) = make_uint4(0, 0, 0, 0);

    const __amdgpu_buffer_rsrc_t rv = rsrc(pvals, tiles * ksteps * 1024);
    const __amdgpu_buffer_rsrc_t rm = rsrc(pmeta, tiles * ksteps * 64 * IDXB);
    const __amdgpu_buffer_rsrc_t rb = BT ? rsrc(a.B, ((a.N - 1) * a.ldb + a.K) * T::ES) : rsrc(a.B, a.K * 16 * T::ES);
    const __amdgpu_buffer_rsrc_t rk = rsrc(rmask, tiles * ksteps * 64 * MB);
    const uint32_t bt_off = (lane & 15) < a.N
                                ? (uint32_t)(((lane & 15) * a.ldb + (lane >> 4) * (T::KS / 8)) * T::ES)
                                : kOob;
    // values: the host aligns cvals to 16 bytes, so the 16-byte block that
    // holds the last value is mapped; bytes past the array are never used
    const __amdgpu_buffer_rsrc_t rc = rsrc(cvals, (nvals * T::ES + 15) / 16 * 16);
    uint32_t voff[TM], moff[TM], koff[TM];
    int64_t bidx[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int64_t blk0 = (t0 + t) * ksteps;           // block of the tile's k-step 0
        voff[t] = t < nt ? (uint32_t)((blk0 * 64 + lane) * 16) : kOob;
        moff[t] = t < nt ? (uint32_t)((blk0 * 64 + lane) * IDXB) : kOob;
        koff[t] = t < nt ? (uint32_t)((blk0 * 64 + lane) * MB) : kOob;
        bidx[t] = t < nt ? blk0 : -1;
    }

    i32x4 av[LX][TM] = {};   // native vector registers, so they can be tied to the waits below
    int mv[LX][TM] = {};
    int kv[LX][TM] = {};
    i32x4 bv[LX][2] = {};    // BT: the wave's B operand of each k-step in flight
    // block offsets (roff[b], roff[b + 1]) of a group's tiles: wave-uniform,
    // so scalar loads (through the constant address space), which the
    // compiler waits for itself; past K or past the tiles they read as an
    // empty range
    int2 ov[LX][TM] = {};
    bool lv[LX][TM] = {};
    const __attribute__((address_space(4))) int32_t* roff_c =
        (const __attribute__((address_space(4))) int32_t*)(uintptr_t)roff;
    auto issue_x = [&](int64_t g, int u) {
        const bool in = g < ksteps;
        const uint32_t slot = lds_addr + wbase + (uint32_t)(u * C::BSTEP);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (BT) {
                const uint32_t ob = in && bt_off != kOob ? bt_off + (uint32_t)((g * T::KS + j * (T::KS / 2)) * T::ES) : kOob;
                asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(bv[u][j]) : "v"(ob), "s"(rb) : "memory");
            } else {
                dma<16>(rb, slot + j * 1024, in ? (uint32_t)(g * C::BSTEP + j * 1024 + lane * 16) : kOob);
            }
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const uint32_t o = in ? voff[t] + (uint32_t)(g * 1024) : kOob;
            const uint32_t om = in ? moff[t] + (uint32_t)(g * 64 * IDXB) : kOob;
            const uint32_t ok = in ? koff[t] + (uint32_t)(g * 64 * MB) : kOob;
            asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen nt" : "=v"(av[u][t]) : "v"(o), "s"(rv) : "memory");
            if constexpr (IDXB == 4)
                asm volatile("buffer_load_dword %0, %1, %2, 0 offen nt" : "=v"(mv[u][t]) : "v"(om), "s"(rm) : "memory");
            else
                asm volatile("buffer_load_ushort %0, %1, %2, 0 offen nt" : "=v"(mv[u][t]) : "v"(om), "s"(rm) : "memory");
            if constexpr (MB == 2)
                asm volatile("buffer_load_ushort %0, %1, %2, 0 offen nt" : "=v"(kv[u][t]) : "v"(ok), "s"(rk) : "memory");
            else
                asm volatile("buffer_load_ubyte %0, %1, %2, 0 offen nt" : "=v"(kv[u][t]) : "v"(ok), "s"(rk) : "memory");
            // the range is emptied where it is used, not here, so the
            // compiler's wait for the scalar load sits at the use
            lv[u][t] = in && bidx[t] >= 0;
            const int64_t b = lv[u][t] ? bidx[t] + g : 0;
            ov[u][t] = make_int2(roff_c[b], roff_c[b + 1]);
        }
    };
    // the value windows of k-step g's blocks (X slot u landed) into Y slot y
    auto issue_y = [&](int u, int y) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const uint32_t start = lv[u][t] ? ((uint32_t)ov[u][t].x * T::ES) & ~15u : 0u;
            const uint32_t end = lv[u][t] ? (uint32_t)ov[u][t].y * T::ES : 0u;
            const uint32_t win = lds_addr + ybase + (uint32_t)((y * TM + t) * C::YWIN);
            const uint32_t o = start + (uint32_t)(lane * 16);
            dma<16>(rc, win, o < end ? o : kOob);
            if (end > start + 1024u) dma<16>(rc, win + 1024, o + 1024u < end ? o + 1024u : kOob);   // wave-uniform
        }
    };

    Acc acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = Acc{0, 0, 0, 0};
    // prologue: X(g0), X(g1), Y(g0), X(g2), Y(g1), X(g3) -- the state an
    // iteration expects: its own X and Y landed once only the previous
    // iteration's Y and X groups remain outstanding
    issue_x(wave, 0);
    issue_x(wave + (int64_t)W, 1);
    wait_vm<GX>();
    issue_y(0, 0);
    issue_x(wave + (int64_t)2 * W, 2);
    wait_vm<GY + GX>();
    issue_y(1, 1);
    issue_x(wave + (int64_t)3 * W, 3);

    const int nw = ksteps > wave ? (int)((ksteps - wave + W - 1) / W) : 0;
    for (int i0 = 0; i0 < nw; i0 += LX) {
#pragma unroll
        for (int u = 0; u < LX; ++u) {
            const int i = i0 + u;
            if (i < nw) {
                const int y = u % LY, u2 = (u + LY) % LX;
                wait_vm<GY + GX>();
#pragma unroll
                for (int t = 0; t < TM; ++t)
                    asm volatile("" : "+v"(av[u][t]), "+v"(mv[u][t]), "+v"(kv[u][t]));
                uint4 b[2];
                if constexpr (BT) {
                    asm volatile("" : "+v"(bv[u][0]));
                    asm volatile("" : "+v"(bv[u][1]));
                    __builtin_memcpy(&b[0], &bv[u][0], 16);
                    __builtin_memcpy(&b[1], &bv[u][1], 16);
                } else {
                    load_b_operand<DT>(lds + wbase + u * C::BSTEP, 0, lane, b);
                }
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    uint4 f;
                    __builtin_memcpy(&f, &av[u][t], 16);
                    acc[t] = smfmac<DT>(f, b, acc[t], (uint32_t)mv[u][t]);
                }
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    const uint32_t mask = (uint32_t)kv[u][t];
                    if (__builtin_amdgcn_ballot_w64(mask != 0u) != 0) {      // wave-uniform
                        const int pc = __popc(mask);
                        const uint32_t before = (uint32_t)(wave_incl_sum(pc, lane) - pc);
                        const uint32_t ro0 = (uint32_t)ov[u][t].x;
                        const uint32_t e0 = ((ro0 * T::ES) & 15u) / T::ES + before;
                        const uint8_t* win = lds + ybase + (y * TM + t) * C::YWIN;
                        const uint4 f = cbm_operand<DT>(win, zpad - (ybase + (uint32_t)((y * TM + t) * C::YWIN)), e0,
                                                        mask);
                        acc[t] = smfmac<DT>(f, b, acc[t], complement_index((uint32_t)mv[u][t]));
                    }
                }
                // the slots' LDS reads are done before their next loads land
                __builtin_amdgcn_s_waitcnt(0xC07F);
                issue_y(u2, y);
                issue_x(wave + (int64_t)W * (i + LX), u);
            }
        }
    }
    // the loads past the wave's last k-step land before the LDS is reused,
    // and before their registers are (an asm load's output counts as
    // written when issued, so the ring stays in use until the wait)
    wait_vm<0>();
#pragma unroll
    for (int u = 0; u < LX; ++u) {
#pragma unroll
        for (int t = 0; t < TM; ++t) asm volatile("" ::"v"(av[u][t]), "v"(mv[u][t]), "v"(kv[u][t]));
        if constexpr (BT) asm volatile("" ::"v"(bv[u][0]), "v"(bv[u][1]));
    }
    lds_barrier();

    // fixed-order reduction of the waves' partial tiles
    Acc* red = reinterpret_cast<Acc*>(lds);
#pragma unroll
    for (int t = 0; t < TM; ++t) red[(wave * kTMax + t) * 64 + lane] = acc[t];
    lds_barrier();
    const int64_t r0 = 16 * t0;
    for (int i = threadIdx.x; i < nt * 256; i += blockDim.x) {
        const int t = i >> 8, ln = (i >> 2) & 63, r = i & 3;
        S sum = S(0);
#pragma unroll
        for (int w = 0; w < W; ++w) sum += reinterpret_cast<const S*>(red)[((w * kTMax + t) * 64 + ln) * 4 + r];
        const int64_t row = r0 + 16 * t + 4 * (ln >> 4) + r;
        const int col = ln & 15;
        if (row < a.M && col < a.N) reinterpret_cast<S*>(a.C)[row * a.ldc + col] = sum;
    }
}

template <int DT, int TM, int W, bool BT>
void launch_packed_cbm_w(const SpmmArgs& a, const uint8_t* pv, const uint8_t* pm, const uint8_t* rmask,
                         const int32_t* roff, const uint8_t* cvals, int64_t nvals, int64_t tiles, hipStream_t s) {
    hipLaunchKernelGGL((k_spmm_packed_cbm<DT, TM, W, BT>), dim3((unsigned)((tiles + TM - 1) / TM)), dim3(64 * W),
                       (W * Cbm<DT>::template wave_lds<TM, BT>()), s, a, pv, pm, rmask, roff, cvals, nvals, tiles);
}

template <int DT, bool BT = false>
hipError_t launch_packed_cbm_t(const SpmmArgs& a, const uint8_t* pv, const uint8_t* pm, const uint8_t* rmask,
                               const int32_t* roff, const uint8_t* cvals, int64_t nvals, hipStream_t s) {
    const int64_t tiles = (a.M + 15) / 16;
    if (tiles <= 256) launch_packed_cbm_w<DT, 1, kWaves, BT>(a, pv, pm, rmask, roff, cvals, nvals, tiles, s);
    else launch_packed_cbm_w<DT, 2, kWaves, BT>(a, pv, pm, rmask, roff, cvals, nvals, tiles, s);
    return hipGetLastError();
}

// Ring depth of the packed product by tiles per workgroup: about 3 to 8
// fragments (KiB) in flight per wave.  Deeper rings put most of a decode-size
// operand in flight at once and measured slower (fp16 11008 x 4096: 12.5 us
// at 7 k-steps deep, 11.0 us at 2; 8192 x 8192: 17.7 us at 8, 15.0 us at 2).
template <int TM> constexpr int kPackedP = TM == 1 ? 3 : 2;

// with a residual: the shallower ring (registers for the epilogue) and the
// whole LDS (B chunks below the row sums)
template <int TM> constexpr int kPackedResP = TM == 4 ? 2 : 3;

template <int DT, int TM, bool BT = false>
hipError_t launch_packed_tm(const SpmmArgs& a, const uint8_t* pv, const uint8_t* pm, int64_t tiles, int64_t G,
                            hipStream_t s) {
    if (BT || a.row_ptr == nullptr) {
        constexpr int P = kPackedP<TM>;
        const unsigned shm = (unsigned)(kWaves * P * 16 * SN<DT>::ES * SN<DT>::KS);
        hipLaunchKernelGGL((k_spmm_packed<DT, TM, P, false, false, BT>), dim3((unsigned)G), dim3(64 * kWaves), shm, s,
                           a, pv, pm, tiles);
    } else {
        constexpr int P = kPackedResP<TM>;
        static_assert(kWaves * P * 16 * 2 * 64 <= kRingResOff, "ring slots below the row sums");
        if (a.dcol != nullptr)
            hipLaunchKernelGGL((k_spmm_packed<DT, TM, P, true, true>), dim3((unsigned)G), dim3(64 * kWaves),
                               160 * 1024, s, a, pv, pm, tiles);
        else
            hipLaunchKernelGGL((k_spmm_packed<DT, TM, P, true, false>), dim3((unsigned)G), dim3(64 * kWaves),
                               160 * 1024, s, a, pv, pm, tiles);
    }
    return hipGetLastError();
}

template <int DT, bool BT = false>
hipError_t launch_packed_t(const SpmmArgs& a, const uint8_t* pv, const uint8_t* pm, hipStream_t s) {
    const int64_t tiles = (a.M + 15) / 16;
    int64_t G = tiles < 256 ? tiles : 256;
    if (G * kTMax < tiles) G = (tiles + kTMax - 1) / kTMax;
    const int tm = (int)((tiles + G - 1) / G);
    switch (tm) {
        case 1: return launch_packed_tm<DT, 1, BT>(a, pv, pm, tiles, G, s);
        case 2: return launch_packed_tm<DT, 2, BT>(a, pv, pm, tiles, G, s);
        case 3: return launch_packed_tm<DT, 3, BT>(a, pv, pm, tiles, G, s);
        default: return launch_packed_tm<DT, 4, BT>(a, pv, pm, tiles, G, s);
    }
}

// Ring depths (k-steps in flight per wave).  As for the packed product,
// shallow rings measured faster than deep ones (fp16 11008 x 4096 x 16:
// 16.2 us at 8 k-steps, 14.9 us at 4, 14.3 us at 3).
template <int TM> constexpr int kRingP = TM == 4 ? 2 : 3;      // deepest ring
template <int TM> constexpr int kRingPLow = 2;                 // when the deepest does not fit

// LDS of the ring variant: the waves' B slots and the slab's metadata rows
template <int DT, int TM>
int64_t ring_lds(const SpmmArgs& a, int P) {
    using T = SN<DT>;
    return (int64_t)kWaves * P * 16 * T::ES * T::KS + 16 * TM * ((a.K / T::KS) * T::META + 4);
}

// Ring depth for this problem: the deepest that fits (0: none).  Products
// with a residual take the shallower ring, which leaves more registers for
// the epilogue.
template <int DT, int TM>
int ring_depth(const SpmmArgs& a) {
    constexpr int64_t kLds = 160 * 1024;
    if (a.row_ptr == nullptr && ring_lds<DT, TM>(a, kRingP<TM>) <= kLds) return kRingP<TM>;
    return ring_lds<DT, TM>(a, kRingPLow<TM>) <= kLds ? kRingPLow<TM> : 0;
}

template <int DT, int TM, int P>
void launch_ring_p(const SpmmArgs& a, int64_t G, int64_t rows_per_wg, hipStream_t s) {
    if (a.row_ptr == nullptr) {
        const unsigned shm = (unsigned)ring_lds<DT, TM>(a, P);
        hipLaunchKernelGGL((k_spmm_small_n_ring<DT, TM, P, false, false>), dim3((unsigned)G), dim3(64 * kWaves), shm,
                           s, a, (int)rows_per_wg);
    } else if constexpr (P == kRingPLow<TM>) {
        // the residual epilogue uses the whole LDS
        if (a.dcol != nullptr)
            hipLaunchKernelGGL((k_spmm_small_n_ring<DT, TM, P, true, true>), dim3((unsigned)G), dim3(64 * kWaves),
                               160 * 1024, s, a, (int)rows_per_wg);
        else
            hipLaunchKernelGGL((k_spmm_small_n_ring<DT, TM, P, true, false>), dim3((unsigned)G), dim3(64 * kWaves),
                               160 * 1024, s, a, (int)rows_per_wg);
    }
}

template <int DT, int TM>
hipError_t launch_ring(const SpmmArgs& a, int64_t G, int64_t rows_per_wg, hipStream_t s) {
    const int P = ring_depth<DT, TM>(a);
    if (P == kRingP<TM>) launch_ring_p<DT, TM, kRingP<TM>>(a, G, rows_per_wg, s);
    else if (P == kRingPLow<TM>) launch_ring_p<DT, TM, kRingPLow<TM>>(a, G, rows_per_wg, s);
    else return hipErrorInvalidConfiguration;   // excluded by ring_ok
    return hipGetLastError();
}

// The barrier-free variant takes products whose B is one contiguous K x 16
// block, whose ring fits the LDS and whose buffers are addressed with
// 31-bit offsets (a residual has passed supported_t: aligned arrays, 31-bit
// offsets).
template <int DT>
bool ring_ok(const SpmmArgs& a, int tm) {
    using T = SN<DT>;
    const uintptr_t bp = reinterpret_cast<uintptr_t>(a.B), mp = reinterpret_cast<uintptr_t>(a.meta);
    const int P = tm == 1 ? ring_depth<DT, 1>(a) : tm == 2 ? ring_depth<DT, 2>(a) : tm == 3 ? ring_depth<DT, 3>(a)
                                                                                          : ring_depth<DT, 4>(a);
    // B rows of 16 readable elements: N == 16, or a narrower B that the host
    // padded into the workspace (columns past N are computed and never stored)
    return P > 0 && (a.N == 16 || (a.N < 16 && a.b_pad16)) && a.ldb == 16 && bp % 16 == 0 && mp % 4 == 0 &&
           a.ldm % 4 == 0 &&
           a.K * 16 * T::ES < 0x7fffffff && a.M * a.ldv * T::ES < 0x7fffffff && a.M * a.ldm < 0x7fffffff;
}

template <int DT>
bool supported_t(const SpmmArgs& a) {
    using T = SN<DT>;
    const uintptr_t v = reinterpret_cast<uintptr_t>(a.vals);
    // vals rows 16-byte aligned; every index fits the kernel's 32-bit LDS math
    const bool dense_ok = a.N >= 1 && a.N <= 16 && a.K > 0 && a.K % T::KS == 0 && v % 16 == 0 &&
                          (a.ldv * T::ES) % 16 == 0 && a.M > 0;
    if (!dense_ok || a.row_ptr == nullptr) return dense_ok;
    // residual arrays: aligned for the widest per-lane load (4 entries) and
    // addressed with 31-bit byte offsets
    const uintptr_t ip = a.dcol ? reinterpret_cast<uintptr_t>(a.dcol) : reinterpret_cast<uintptr_t>(a.col);
    const uintptr_t rp = reinterpret_cast<uintptr_t>(a.rvals);
    const int64_t ib = a.dcol ? 1 : 4;
    return ip % (4 * ib) == 0 && rp % (4 * T::ES) == 0 && a.nnz_r * ib < 0x7fff0000 && a.nnz_r * T::ES < 0x7fff0000;
}

// Ring depth by tiles per slab: about 16 fragments (KiB) in flight per wave.
template <int TM> constexpr int kRing = TM == 1 ? 16 : TM == 2 ? 8 : 4;

// K-steps one LDS chunk holds: the chunk's B rows (16 columns) and the
// padded metadata rows of the slab's 16*TM rows share the LDS data region.
template <int DT, int TM>
constexpr int64_t chunk_capacity() {
    using T = SN<DT>;
    return (kLdsData - 16 * TM * 4) / (16 * T::ES * T::KS + 16 * TM * T::META);
}

// Whether TM tiles can walk K: in one chunk, or in chunks that each hold a
// multiple of W*P k-steps (so ring slot i % P follows the wave's k-steps
// across chunks).
template <int DT, int TM>
bool chunks_fit(int64_t ksteps) {
    return ksteps <= chunk_capacity<DT, TM>() || chunk_capacity<DT, TM>() >= kWaves * kRing<TM>;
}

static_assert(chunk_capacity<DT_F16, 4>() >= kWaves * kRing<4> && chunk_capacity<DT_I8, 4>() >= kWaves * kRing<4>,
              "the widest slab must walk any K");

template <int DT, int TM>
hipError_t launch_tm(const SpmmArgs& a, int64_t G, int64_t rows_per_wg, hipStream_t s) {
    using T = SN<DT>;
    constexpr int P = kRing<TM>;
    const int64_t ksteps = a.K / T::KS;
    const int64_t max_steps = chunk_capacity<DT, TM>();
    int64_t chunk = ksteps;
    if (chunk > max_steps) chunk = max_steps / (kWaves * P) * (kWaves * P);
    if (chunk <= 0) return hipErrorInvalidConfiguration;   // excluded by launch_t (chunks_fit)
    const uintptr_t bp = reinterpret_cast<uintptr_t>(a.B), mp = reinterpret_cast<uintptr_t>(a.meta);
    const bool vec_b = a.N == 16 && a.ldb == 16 && bp % 16 == 0 &&
                       a.K * 16 * T::ES < 0x7fffffff;                // one contiguous block of B
    const bool vec_m = mp % 4 == 0 && a.ldm % 4 == 0 && (a.M - 1) * a.ldm + (a.K + 7) / 8 < 0x7fffffff;
    if (a.row_ptr != nullptr && a.dcol != nullptr)
        hipLaunchKernelGGL((k_spmm_small_n<DT, TM, P, true>), dim3((unsigned)G), dim3(64 * kWaves), 0, s, a,
                           (int)rows_per_wg, (int)chunk, (int)vec_b, (int)vec_m);
    else
        hipLaunchKernelGGL((k_spmm_small_n<DT, TM, P, false>), dim3((unsigned)G), dim3(64 * kWaves), 0, s, a,
                           (int)rows_per_wg, (int)chunk, (int)vec_b, (int)vec_m);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_t(const SpmmArgs& a, hipStream_t s) {
    const int64_t tiles = (a.M + 15) / 16;
    int64_t G = tiles < 256 ? tiles : 256;
    const int64_t min_g = (tiles + kTMax - 1) / kTMax;
    if (G < min_g) G = min_g;
    const int64_t rows_per_wg = (a.M + G - 1) / G;
    G = (a.M + rows_per_wg - 1) / rows_per_wg;
    if (ring_ok<DT>(a, (int)((rows_per_wg + 15) / 16))) {
        switch ((rows_per_wg + 15) / 16) {
            case 1: return launch_ring<DT, 1>(a, G, rows_per_wg, s);
            case 2: return launch_ring<DT, 2>(a, G, rows_per_wg, s);
            case 3: return launch_ring<DT, 3>(a, G, rows_per_wg, s);
            default: return launch_ring<DT, 4>(a, G, rows_per_wg, s);
        }
    }
    // a slab of fewer tiles than its deepest ring can chunk runs as a wider
    // slab (its rows past rows_per_wg are masked)
    int tm = (int)((rows_per_wg + 15) / 16);
    const int64_t ksteps = a.K / SN<DT>::KS;
    if (tm == 1 && !chunks_fit<DT, 1>(ksteps)) tm = 2;
    if (tm == 2 && !chunks_fit<DT, 2>(ksteps)) tm = 3;
    if (tm == 3 && !chunks_fit<DT, 3>(ksteps)) tm = 4;
    switch (tm) {
        case 1: return launch_tm<DT, 1>(a, G, rows_per_wg, s);
        case 2: return launch_tm<DT, 2>(a, G, rows_per_wg, s);
        case 3: return launch_tm<DT, 3>(a, G, rows_per_wg, s);
        default: return launch_tm<DT, 4>(a, G, rows_per_wg, s);
    }
}

}  // namespace

bool supported_small_n(const SpmmArgs& a) {
    switch (a.dt) {
        case DT_F16: return supported_t<DT_F16>(a);
        case DT_BF16: return supported_t<DT_BF16>(a);
        case DT_I8: return supported_t<DT_I8>(a);
        case DT_E4M3: return supported_t<DT_E4M3>(a);
        case DT_E5M2: return supported_t<DT_E5M2>(a);
        default: return false;
    }
}

hipError_t launch_pack_decode(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                              int64_t ldm, void* pvals, void* pmeta, hipStream_t s) {
    const int64_t ks = dt_bytes(dt) == 1 ? SN<DT_I8>::KS : SN<DT_F16>::KS;
    const int64_t n = ((M + 15) / 16) * (K / ks) * 64;
    if (n == 0) return hipSuccess;
    const unsigned grid = (unsigned)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
    const int64_t es = dt_bytes(dt);
    switch (dt) {
        case DT_F16: case DT_BF16:
            hipLaunchKernelGGL(k_pack<DT_F16>, dim3(grid), dim3(256), 0, s, M, K, (const uint8_t*)vals, ldv * es, meta,
                               ldm, (uint8_t*)pvals, (uint8_t*)pmeta);
            break;
        case DT_I8: case DT_E4M3: case DT_E5M2:
            hipLaunchKernelGGL(k_pack<DT_I8>, dim3(grid), dim3(256), 0, s, M, K, (const uint8_t*)vals, ldv * es, meta,
                               ldm, (uint8_t*)pvals, (uint8_t*)pmeta);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// B [K, N] (N < 16, row stride ldb) copied to K x 16 with zero columns past N,
// so the decode kernels that take B as one contiguous K x 16 block apply.
template <typename E>
__global__ void __launch_bounds__(256) k_pad_b(int64_t K, int64_t N, const E* B, int64_t ldb, E* out) {
    const int64_t n = K * 16;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k = i >> 4, c = i & 15;
        out[i] = c < N ? B[k * ldb + c] : E(0);
    }
}

hipError_t launch_pad_b(int dt, int64_t K, int64_t N, const void* B, int64_t ldb, void* out, hipStream_t s) {
    const int64_t n = K * 16;
    const unsigned grid = (unsigned)std::min<int64_t>((n + 255) / 256, 2048);
    if (dt_bytes(dt) == 2)
        hipLaunchKernelGGL(k_pad_b<uint16_t>, dim3(grid), dim3(256), 0, s, K, N, (const uint16_t*)B, ldb, (uint16_t*)out);
    else
        hipLaunchKernelGGL(k_pad_b<uint8_t>, dim3(grid), dim3(256), 0, s, K, N, (const uint8_t*)B, ldb, (uint8_t*)out);
    return hipGetLastError();
}

hipError_t launch_spmm_packed(const SpmmArgs& a, const void* pvals, const void* pmeta, hipStream_t s) {
    const uint8_t* pv = (const uint8_t*)pvals;
    const uint8_t* pm = (const uint8_t*)pmeta;
    switch (a.dt) {
        case DT_F16: return launch_packed_t<DT_F16>(a, pv, pm, s);
        case DT_BF16: return launch_packed_t<DT_BF16>(a, pv, pm, s);
        case DT_I8: return launch_packed_t<DT_I8>(a, pv, pm, s);
        case DT_E4M3: return launch_packed_t<DT_E4M3>(a, pv, pm, s);
        case DT_E5M2: return launch_packed_t<DT_E5M2>(a, pv, pm, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_spmm_packed_bt(const SpmmArgs& a, const void* pvals, const void* pmeta, hipStream_t s) {
    const uint8_t* pv = (const uint8_t*)pvals;
    const uint8_t* pm = (const uint8_t*)pmeta;
    switch (a.dt) {
        case DT_F16: return launch_packed_t<DT_F16, true>(a, pv, pm, s);
        case DT_BF16: return launch_packed_t<DT_BF16, true>(a, pv, pm, s);
        case DT_I8: return launch_packed_t<DT_I8, true>(a, pv, pm, s);
        case DT_E4M3: return launch_packed_t<DT_E4M3, true>(a, pv, pm, s);
        case DT_E5M2: return launch_packed_t<DT_E5M2, true>(a, pv, pm, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_spmm_packed_cbm(const SpmmArgs& a, const void* pvals, const void* pmeta, const void* rmask,
                                  const int32_t* roff, const void* cvals, int64_t nvals, hipStream_t s) {
    const uint8_t* pv = (const uint8_t*)pvals;
    const uint8_t* pm = (const uint8_t*)pmeta;
    const uint8_t* rk = (const uint8_t*)rmask;
    const uint8_t* cv = (const uint8_t*)cvals;
    switch (a.dt) {
        case DT_F16: return launch_packed_cbm_t<DT_F16>(a, pv, pm, rk, roff, cv, nvals, s);
        case DT_BF16: return launch_packed_cbm_t<DT_BF16>(a, pv, pm, rk, roff, cv, nvals, s);
        case DT_I8: return launch_packed_cbm_t<DT_I8>(a, pv, pm, rk, roff, cv, nvals, s);
        case DT_E4M3: return launch_packed_cbm_t<DT_E4M3>(a, pv, pm, rk, roff, cv, nvals, s);
        case DT_E5M2: return launch_packed_cbm_t<DT_E5M2>(a, pv, pm, rk, roff, cv, nvals, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_spmm_packed_cbm_bt(const SpmmArgs& a, const void* pvals, const void* pmeta, const void* rmask,
                                  const int32_t* roff, const void* cvals, int64_t nvals, hipStream_t s) {
    const uint8_t* pv = (const uint8_t*)pvals;
    const uint8_t* pm = (const uint8_t*)pmeta;
    const uint8_t* rk = (const uint8_t*)rmask;
    const uint8_t* cv = (const uint8_t*)cvals;
    switch (a.dt) {
        case DT_F16: return launch_packed_cbm_t<DT_F16, true>(a, pv, pm, rk, roff, cv, nvals, s);
        case DT_BF16: return launch_packed_cbm_t<DT_BF16, true>(a, pv, pm, rk, roff, cv, nvals, s);
        case DT_I8: return launch_packed_cbm_t<DT_I8, true>(a, pv, pm, rk, roff, cv, nvals, s);
        case DT_E4M3: return launch_packed_cbm_t<DT_E4M3, true>(a, pv, pm, rk, roff, cv, nvals, s);
        case DT_E5M2: return launch_packed_cbm_t<DT_E5M2, true>(a, pv, pm, rk, roff, cv, nvals, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_spmm_small_n(const SpmmArgs& a, hipStream_t s) {
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
