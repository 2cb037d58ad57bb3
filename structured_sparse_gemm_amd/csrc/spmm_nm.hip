// spmm_nm.hip -- N:M structured sparsity other than 2:4 (1:4, 2:8, 4:8, and
// 2:4 in the same storage for comparison): compress a dense weight into its
// kept values and a keep mask, expand it back, and the decode-shape product
// on the dense MFMA.
//
// "Chapter 26 -- Sparsity: The Hardware View", section "Block Sparsity, N:M
// Generalizations, and Channel Pruning", lists these patterns; the page
// gives no selection rule and no storage.  The reading here widens the 2:4
// rule: each group of MM consecutive elements along K keeps its NN largest
// magnitudes (ties to the lower position); vals[M, K/MM*NN] holds them in
// ascending position order and mask[M, ceil(K/8)] has bit k%8 of byte k/8
// set iff element k is kept.
//
// gfx950's sparse MFMA takes 2:4 only, so the gain of these patterns on this
// chip is the bytes a product streams: in the memory-bound regime
// ("Chapter 26", section "2:4 in the Memory-Bound Regime") they set the time.
// The product therefore expands the operand to dense in registers and runs
// the dense MFMA:
// * Super-step: lane l = 16q + r of a wave owns the D consecutive dense k
//   [s*4D + q*D, s*4D + (q+1)*D) of row r of its tile, where D is what one
//   16-byte load of stored values covers (D = 16/ES * MM/NN).  Its values
//   are that one load from the row, its mask bits one 2-, 4- or 8-byte load.
//   A dense MFMA sums over its k in any order provided the A and B fragments
//   agree element by element, so the lane cuts its range into fragments in
//   place and B is read to match.
// * Expansion: per group, one byte permute (v_perm_b32) per output dword of
//   the group's stored bytes under selectors looked up in an LDS table
//   indexed by the group's mask bits (built at kernel start).
// * B rows of each super-step arrive by direct-to-LDS loads into a per-wave
//   ring slot and are read back transposed (ds_read_b64_tr_b16 / _b8).
// * A workgroup owns up to 4 tiles (64 rows) and one 16-column slice of B;
//   its waves split the super-steps; partial tiles are summed through LDS in
//   wave order, so fp32 results are the same on every run.
#include "ssg_device.hpp"
#include "ssg_kernels.hpp"
#include "ssg_stream.hpp"

namespace ssg {

namespace {

constexpr int kNmWaves = 8;
constexpr int kNmTMax = 4;

// Working element of the compress / expand kernels: the storage word, or
// for 4-bit weights the value widened to int8 (stored two per byte).
template <int DT> struct NmStore { using T = uint16_t; };
template <> struct NmStore<DT_I8> { using T = int8_t; };
template <> struct NmStore<DT_E4M3> { using T = uint8_t; };
template <> struct NmStore<DT_E5M2> { using T = uint8_t; };
template <> struct NmStore<DT_I4> { using T = int8_t; };

template <int DT>
__device__ __forceinline__ uint32_t nm_key(typename NmStore<DT>::T x) {
    if constexpr (DT == DT_I8 || DT == DT_I4) return mag_key8((int32_t)x);
    else if constexpr (dt_is_fp8(DT)) return mag_key_fp8((uint32_t)x);
    else return mag_key16((uint32_t)x);
}

// ---- compress / expand ------------------------------------------------------
//
// One thread per chunk of 32 dense elements of a row (32 / MM whole groups):
// it writes 4 whole mask bytes and 32*NN/MM values, so no byte is shared
// (4-bit weights: NN is even, so a chunk's values fill whole bytes).  The
// ragged last chunk of a row (K % 32) takes element-wise accesses.

constexpr int kNmChunk = 32;

// n elements of a row from `row` (element index i0 on) into x; 4-bit
// weights are sign-extended from their nibbles.  `vec`: 16-byte loads.
template <int DT>
__device__ __forceinline__ void nm_load(const void* row, int64_t i0, int n, bool vec,
                                        typename NmStore<DT>::T (&x)[kNmChunk]) {
    using T = typename NmStore<DT>::T;
    if constexpr (DT == DT_I4) {
        const uint8_t* b = reinterpret_cast<const uint8_t*>(row) + i0 / 2;
        uint8_t by[kNmChunk / 2];
        if (vec && n == kNmChunk) {
            const uint4 w = *reinterpret_cast<const uint4*>(b);
            __builtin_memcpy(by, &w, 16);
        } else {
#pragma unroll
            for (int i = 0; i < kNmChunk / 2; ++i) by[i] = 2 * i < n ? b[i] : 0;
        }
#pragma unroll
        for (int i = 0; i < kNmChunk; ++i) {
            const int nib = (by[i / 2] >> (4 * (i % 2))) & 0xF;
            x[i] = (T)(nib >= 8 ? nib - 16 : nib);
        }
    } else {
        const T* a = reinterpret_cast<const T*>(row) + i0;
        if (vec && n == kNmChunk) {
            uint4 w[kNmChunk * sizeof(T) / 16];
#pragma unroll
            for (int i = 0; i < (int)(kNmChunk * sizeof(T) / 16); ++i) w[i] = reinterpret_cast<const uint4*>(a)[i];
            __builtin_memcpy(x, w, sizeof(x));
        } else {
#pragma unroll
            for (int i = 0; i < kNmChunk; ++i) x[i] = i < n ? a[i] : T(0);
        }
    }
}

// The first n of v (NV entries) to `row` from element i0 on; 4-bit values
// are packed two per byte (n and i0 even).  `vec`: NV entries as 8-byte stores.
template <int DT, int NV>
__device__ __forceinline__ void nm_store(void* row, int64_t i0, int n, bool vec, const typename NmStore<DT>::T (&v)[NV]) {
    using T = typename NmStore<DT>::T;
    if constexpr (DT == DT_I4) {
        uint8_t* b = reinterpret_cast<uint8_t*>(row) + i0 / 2;
        uint8_t by[NV / 2];
#pragma unroll
        for (int i = 0; i < NV / 2; ++i) by[i] = (uint8_t)((v[2 * i] & 0xF) | ((v[2 * i + 1] & 0xF) << 4));
        if (vec && n == NV) {
            if constexpr (NV / 2 >= 8) {
                uint2 w[NV / 16];
                __builtin_memcpy(w, by, NV / 2);
#pragma unroll
                for (int i = 0; i < NV / 16; ++i) reinterpret_cast<uint2*>(b)[i] = w[i];
            } else {
                uint32_t w;
                __builtin_memcpy(&w, by, 4);
                *reinterpret_cast<uint32_t*>(b) = w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV / 2; ++i)
                if (2 * i < n) b[i] = by[i];
        }
    } else {
        T* a = reinterpret_cast<T*>(row) + i0;
        if (vec && n == NV) {
            constexpr int VB = NV * (int)sizeof(T);           // 8, 16 or 32 bytes
            uint2 w[VB / 8];
            __builtin_memcpy(w, v, VB);
#pragma unroll
            for (int i = 0; i < VB / 8; ++i) reinterpret_cast<uint2*>(a)[i] = w[i];
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (i < n) a[i] = v[i];
        }
    }
}

// Bytes of a row of ld elements.
template <int DT> __device__ __forceinline__ int64_t nm_row_bytes(int64_t ld) {
    return DT == DT_I4 ? ld / 2 : ld * (int64_t)sizeof(typename NmStore<DT>::T);
}

template <int DT, int NN, int MM>
__global__ void __launch_bounds__(256) k_compress_nm(int64_t M, int64_t K, const void* A, int64_t lda, void* vals,
                                                     int64_t ldv, uint8_t* mask, int64_t ldm, int vec) {
    using T = typename NmStore<DT>::T;
    constexpr int G = kNmChunk / MM, NV = kNmChunk / MM * NN;
    const int64_t chunks = (K + kNmChunk - 1) / kNmChunk;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < M * chunks;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = t / chunks, c = t - m * chunks;
        const int ne = (int)min<int64_t>(kNmChunk, K - c * kNmChunk);   // a multiple of MM
        T x[kNmChunk];
        nm_load<DT>(reinterpret_cast<const uint8_t*>(A) + m * nm_row_bytes<DT>(lda), c * kNmChunk, ne, vec != 0, x);
        uint32_t bits = 0;
        T v[NV];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            uint32_t key[MM];
#pragma unroll
            for (int p = 0; p < MM; ++p) key[p] = nm_key<DT>(x[g * MM + p]);
            int cnt = 0;
#pragma unroll
            for (int j = 0; j < NN; ++j) v[g * NN + j] = T(0);
#pragma unroll
            for (int p = 0; p < MM; ++p) {
                int rank = 0;
#pragma unroll
                for (int q = 0; q < MM; ++q)
                    if (q != p) rank += (key[q] > key[p] || (key[q] == key[p] && q < p)) ? 1 : 0;
                const bool keep = rank < NN;
#pragma unroll
                for (int j = 0; j < NN; ++j)
                    if (keep && cnt == j) v[g * NN + j] = x[g * MM + p];
                cnt += keep ? 1 : 0;
                if (keep && g * MM < ne) bits |= 1u << (g * MM + p);
            }
        }
        nm_store<DT, NV>(reinterpret_cast<uint8_t*>(vals) + m * nm_row_bytes<DT>(ldv), c * NV, ne / MM * NN,
                         vec != 0, v);
        uint8_t* mrow = mask + m * ldm + c * (kNmChunk / 8);
        if (vec && ne == kNmChunk) {
            *reinterpret_cast<uint32_t*>(mrow) = bits;
        } else {
#pragma unroll
            for (int b = 0; b < kNmChunk / 8; ++b)
                if (8 * b < ne) mrow[b] = (uint8_t)(bits >> (8 * b));
        }
    }
}

// Dense expansion; a group whose mask does not hold exactly NN bits is
// written as zeros and counted into *bad (if not null).
template <int DT, int NN, int MM>
__global__ void __launch_bounds__(256) k_decompress_nm(int64_t M, int64_t K, const void* vals, int64_t ldv,
                                                       const uint8_t* mask, int64_t ldm, void* D, int64_t ldd,
                                                       int32_t* bad) {
    using T = typename NmStore<DT>::T;
    constexpr int G = kNmChunk / MM, NV = kNmChunk / MM * NN;
    const int64_t chunks = (K + kNmChunk - 1) / kNmChunk;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < M * chunks;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = t / chunks, c = t - m * chunks;
        const int ne = (int)min<int64_t>(kNmChunk, K - c * kNmChunk);
        T vin[kNmChunk];                                   // the chunk's stored values (NV of them)
        nm_load<DT>(reinterpret_cast<const uint8_t*>(vals) + m * nm_row_bytes<DT>(ldv), c * NV, ne / MM * NN, false,
                    vin);
        const uint8_t* mrow = mask + m * ldm + c * (kNmChunk / 8);
        uint32_t bits = 0;
#pragma unroll
        for (int b = 0; b < kNmChunk / 8; ++b)
            if (8 * b < ne) bits |= (uint32_t)mrow[b] << (8 * b);
        T out[kNmChunk];
        int nbad = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint32_t gb = (bits >> (g * MM)) & ((1u << MM) - 1u);
            const bool ok = __builtin_popcount(gb) == NN;
            if (g * MM < ne && !ok) ++nbad;
            int cnt = 0;
#pragma unroll
            for (int p = 0; p < MM; ++p) {
                const bool on = ok && ((gb >> p) & 1u);
                T val = T(0);
#pragma unroll
                for (int j = 0; j < NN; ++j)
                    if (on && cnt == j && g * MM < ne) val = vin[g * NN + j];
                out[g * MM + p] = val;
                cnt += on ? 1 : 0;
            }
        }
        nm_store<DT, kNmChunk>(reinterpret_cast<uint8_t*>(D) + m * nm_row_bytes<DT>(ldd), c * kNmChunk, ne, false,
                               out);
        if (bad && nbad) atomicAdd(bad, nbad);
    }
}

// ---- product ----------------------------------------------------------------

// 4-bit weights (W4) run as fp16: their values are widened to fp16 in
// registers before the expansion, and B is fp16.
template <int DT, int NN, int MM>
struct NmShape {
    static constexpr bool W4 = DT == DT_I4;
    static constexpr int ES = W4 ? 2 : dt_bytes(DT);    // element bytes of the MFMA operands (and B)
    static constexpr int FB = dt_is_fp8(DT) ? 8 : 16;   // A (and B) bytes per lane per MFMA
    static constexpr int E = FB / ES;                    // dense k per lane per MFMA
    static constexpr int D = W4 ? 32 : 16 / ES * MM / NN;   // dense k per lane per super-step
    static constexpr int V = D * NN / MM;                // stored values per lane per super-step
    static constexpr int VB = W4 ? V / 2 : 16;           // their bytes: one 16-, 8- or 4-byte load
    static constexpr int VW = V * ES / 4;                // dwords of them (widened for W4)
    static constexpr int F = D / E;                      // MFMAs per tile per super-step
    static constexpr int SK = 4 * D;                     // dense k per super-step
    static constexpr int GL = D / MM;                    // groups per lane per super-step
    static constexpr int GB = NN * ES;                   // stored (widened) bytes per group
    static constexpr int OW = MM * ES / 4;               // dense dwords per group
    static constexpr int MB = D / 8;                     // mask bytes per lane per super-step
    static constexpr int BSTEP = SK * 16 * ES;           // B bytes per super-step (16 columns)
    static constexpr int NB = BSTEP / 1024;              // direct-to-LDS loads of B per super-step
    // super-steps in flight per wave: shallow rings measured faster than
    // deep ones (fp16 11008 x 4096 x 16, packed: 1:4 11.5 us at 4, 9.3 us at
    // 2; 2:4 13.5 us at 6, 11.6 us at 2)
    static constexpr int P = 2;
    static constexpr int LUT = (1 << MM) * OW * 4;       // selector table bytes
    static_assert(D % MM == 0 && D % E == 0 && D % 8 == 0 && V % 8 == 0, "shape");
    static_assert(!W4 || NN % 2 == 0, "4-bit weights: whole bytes per group");
    static_assert((GB <= 4 && 4 % GB == 0) || GB == 8, "a group's stored bytes lie in one or two whole dwords");
    static_assert(BSTEP % 1024 == 0, "B rows per super-step");
};

template <int DT> using NmAcc = typename std::conditional<DT == DT_I8, i32x4, f32x4>::type;

// Registers of one lane's stored values per super-step, loaded as one
// buffer load of VB bytes.
template <int VB> struct ValReg { using T = i32x4; };
template <> struct ValReg<8> { using T = i32x2; };
template <> struct ValReg<4> { using T = int; };

// NT: a non-temporal load, for the packed layout, whose lines are each read
// once and whole (in the row-major layout a line's halves are read in
// different super-steps, and the second half wants the line still in L2).
#define SSG_NM_LOAD(OP, POL) asm volatile("buffer_load_" OP " %0, %1, %2, 0 offen" POL : "=v"(r) : "v"(off), "s"(rs) : "memory")
template <int VB, bool NT>
__device__ __forceinline__ void load_vals(typename ValReg<VB>::T& r, uint32_t off, __amdgpu_buffer_rsrc_t rs) {
    if constexpr (VB == 16) {
        if constexpr (NT) SSG_NM_LOAD("dwordx4", " nt"); else SSG_NM_LOAD("dwordx4", "");
    } else if constexpr (VB == 8) {
        if constexpr (NT) SSG_NM_LOAD("dwordx2", " nt"); else SSG_NM_LOAD("dwordx2", "");
    } else {
        if constexpr (NT) SSG_NM_LOAD("dword", " nt"); else SSG_NM_LOAD("dword", "");
    }
}

typedef _Float16 nm_h2 __attribute__((ext_vector_type(2)));

// The lane's stored values as VW dwords of MFMA elements: a copy, or for
// 4-bit weights each byte's two nibbles widened to a pair of fp16.  A
// nibble u (two's complement) becomes fp16 1024 + (u ^ 8) by placing u ^ 8
// in the low mantissa bits of 0x6400, and 1024 + 8 is then subtracted:
// exact, since every value involved is an integer below 2048.
template <int DT, int NN, int MM>
__device__ __forceinline__ void widen_vals(const typename ValReg<NmShape<DT, NN, MM>::VB>::T& r, uint32_t (&vw)[NmShape<DT, NN, MM>::VW]) {
    using S = NmShape<DT, NN, MM>;
    if constexpr (S::W4) {
        uint32_t raw[S::VB / 4];
        __builtin_memcpy(raw, &r, S::VB);
#pragma unroll
        for (int i = 0; i < S::VW; ++i) {
            const uint32_t b = (raw[i / 4] >> (8 * (i % 4))) & 0xFFu;
            const uint32_t w = ((b & 0xFu) | ((b & 0xF0u) << 12)) ^ 0x64086408u;
            nm_h2 h;
            __builtin_memcpy(&h, &w, 4);
            h = h - nm_h2{(_Float16)1032.0f, (_Float16)1032.0f};
            __builtin_memcpy(&vw[i], &h, 4);
        }
    } else {
        __builtin_memcpy(vw, &r, 16);
    }
}

template <int DT>
__device__ __forceinline__ NmAcc<DT> nm_mfma(const uint32_t* a, const uint32_t* b, NmAcc<DT> c) {
    if constexpr (DT == DT_I8) {
        i32x4 av, bv;
        __builtin_memcpy(&av, a, 16);
        __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
    } else if constexpr (dt_is_fp8(DT)) {
        long av, bv;
        __builtin_memcpy(&av, a, 8);
        __builtin_memcpy(&bv, b, 8);
        if constexpr (DT == DT_E4M3) return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(av, bv, c, 0, 0, 0);
        else return __builtin_amdgcn_mfma_f32_16x16x32_bf8_bf8(av, bv, c, 0, 0, 0);
    } else if constexpr (DT == DT_F16) {
        f16x8 av, bv;
        __builtin_memcpy(&av, a, 16);
        __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
    } else {
        bf16x8 av, bv;
        __builtin_memcpy(&av, a, 16);
        __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
    }
}

typedef __attribute__((address_space(3))) i16x4 nm_lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 nm_lds_i32x2;

// Selector table: entry (mask, s) is the v_perm_b32 selector of dense dword s
// of a group whose keep bits are `mask`, the group's stored bytes sitting at
// bytes 0..GB-1 of the permute source: byte b of the dword is element
// p = (4s + b) / ES of the group, byte e = (4s + b) % ES of it; a kept p
// takes stored byte j*ES + e with j the number of kept positions below p,
// a dropped p takes the constant zero (selector 0x0C).
template <int DT, int NN, int MM>
__device__ __forceinline__ void build_lut(uint32_t* lut) {
    using S = NmShape<DT, NN, MM>;
    for (int i = threadIdx.x; i < (1 << MM) * S::OW; i += blockDim.x) {
        const uint32_t mk = (uint32_t)i / S::OW, s = (uint32_t)i % S::OW;
        uint32_t sel = 0;
        for (int b = 0; b < 4; ++b) {
            const uint32_t x = 4 * s + b, p = x / S::ES, e = x % S::ES;
            uint32_t v = 0x0Cu;
            if ((mk >> p) & 1u) {
                const uint32_t j = __builtin_popcount(mk & ((1u << p) - 1u));
                const uint32_t src = j * S::ES + e;
                if (src < 8) v = src;
            }
            sel |= v << (8 * b);
        }
        lut[i] = sel;
    }
}

// B fragment f of the lane's range from the super-step's LDS slot (rows of
// 16 columns): element j = row q*D + f*E + j of column l%16.
template <int DT, int NN, int MM>
__device__ __forceinline__ void nm_load_b(const uint8_t* slot, int lane, int f, uint32_t* b) {
    using S = NmShape<DT, NN, MM>;
    const int i = lane & 15, q = lane >> 4;
    if constexpr (S::ES == 2) {
        // tr16: lane i of a 16-lane block names row i/4, columns [4(i%4), +4); it gets column i of the 4 rows
#pragma unroll
        for (int h = 0; h < S::E / 4; ++h) {
            const int row = q * S::D + f * S::E + 4 * h + (i >> 2);
            i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((nm_lds_i16x4*)(slot + row * 32 + (i & 3) * 8));
            __builtin_memcpy(b + 2 * h, &v, 8);
        }
    } else {
        // tr8: lane i names row i/2, bytes [8(i%2), +8); it gets column i of the 8 rows
#pragma unroll
        for (int h = 0; h < S::E / 8; ++h) {
            const int row = q * S::D + f * S::E + 8 * h + (i >> 1);
            i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((nm_lds_i32x2*)(slot + row * 16 + (i & 1) * 8));
            __builtin_memcpy(b + 2 * h, &v, 8);
        }
    }
}

template <int MB> struct MaskReg { using T = int; };
template <> struct MaskReg<8> { using T = i32x2; };

template <int MB, bool NT>
__device__ __forceinline__ void load_mask(typename MaskReg<MB>::T& r, uint32_t off, __amdgpu_buffer_rsrc_t rs) {
    if constexpr (MB == 8) {
        if constexpr (NT) SSG_NM_LOAD("dwordx2", " nt"); else SSG_NM_LOAD("dwordx2", "");
    } else if constexpr (MB == 4) {
        if constexpr (NT) SSG_NM_LOAD("dword", " nt"); else SSG_NM_LOAD("dword", "");
    } else {
        if constexpr (NT) SSG_NM_LOAD("ushort", " nt"); else SSG_NM_LOAD("ushort", "");
    }
}
#undef SSG_NM_LOAD

template <int MB>
__device__ __forceinline__ uint64_t mask_bits(const typename MaskReg<MB>::T& r) {
    if constexpr (MB == 8) return (uint64_t)(uint32_t)r[0] | ((uint64_t)(uint32_t)r[1] << 32);
    else return (uint64_t)(uint32_t)r;
}

// C[:, 16*blockIdx.y + (0..15)] for the workgroup's tiles.  a.vals / a.meta
// are the stored values and the keep mask (rows 16- and 8-byte aligned), or
// with PK their packed decode layout (k_pack_nm).
template <int DT, int NN, int MM, int TM, bool PK>
__global__ void __launch_bounds__(kNmWaves * 64) k_spmm_nm(SpmmArgs a, int64_t tiles) {
    using S = NmShape<DT, NN, MM>;
    constexpr int W = kNmWaves, P = S::P;
    constexpr int GOPS = S::NB + 2 * TM;                 // loads per super-step per wave
    static_assert(P * GOPS < 64, "vmcnt");
    static_assert(W * kNmTMax * 1024 <= W * P * S::BSTEP, "LDS for the reduction");
    using Acc = NmAcc<DT>;
    using Out = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    using MR = typename MaskReg<S::MB>::T;
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];   // ring slots, then the selector table
    uint32_t* lut = reinterpret_cast<uint32_t*>(lds + W * P * S::BSTEP);
    const uint32_t lds_addr = (uint32_t)(uintptr_t)(const lds_void*)lds;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)blockIdx.x * tiles / gridDim.x, t1 = ((int64_t)blockIdx.x + 1) * tiles / gridDim.x;
    const int nt = (int)(t1 - t0);
    const int64_t r0 = 16 * t0;
    const int64_t rows = min<int64_t>(16 * nt, a.M - r0);
    const int64_t ct = blockIdx.y;
    const int64_t nsteps = (a.K + S::SK - 1) / S::SK;
    const int64_t ldvb = S::W4 ? a.ldv / 2 : a.ldv * S::ES, ldbb = a.ldb * S::ES;

    // row-major: ranges rounded up to the load sizes (bases are aligned to
    // them), so a single row whose stride is not a multiple of them still
    // reads whole.  Packed: the workgroup's tiles' blocks, consecutive.
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.vals);
    const __amdgpu_buffer_rsrc_t rv =
        PK ? rsrc(vbase + t0 * nsteps * 64 * S::VB, nt * nsteps * 64 * S::VB)
           : rsrc_aligned<16>(vbase + r0 * ldvb, rows * ldvb);
    const __amdgpu_buffer_rsrc_t rm =
        PK ? rsrc(a.meta + t0 * nsteps * 64 * S::MB, nt * nsteps * 64 * S::MB)
           : rsrc_aligned<8>(a.meta + r0 * a.ldm, rows * a.ldm);
    const __amdgpu_buffer_rsrc_t rb = rsrc_aligned<16>(a.B, a.K * ldbb);
    const int r = lane & 15, q = lane >> 4;
    constexpr uint32_t VSTEP = PK ? 64 * S::VB : 4 * S::VB, MSTEP = PK ? 64 * S::MB : 4 * S::MB;   // bytes per super-step
    uint32_t voff[TM], moff[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        voff[t] = PK ? (uint32_t)((t * nsteps * 64 + lane) * S::VB) : (uint32_t)((16 * t + r) * ldvb + S::VB * q);
        moff[t] = PK ? (uint32_t)((t * nsteps * 64 + lane) * S::MB) : (uint32_t)((16 * t + r) * a.ldm + S::MB * q);
    }
    // lane's B piece of one direct-to-LDS load: 16 bytes of row
    // (j*1024 + 16*lane) / (16*ES) of the super-step
    const int brow = 16 * lane / (16 * S::ES), bcol = 16 * lane % (16 * S::ES);

    build_lut<DT, NN, MM>(lut);

    typename ValReg<S::VB>::T av[P][TM] = {};
    MR mv[P][TM] = {};
    auto issue = [&](int64_t g, int u) {
        const bool in = g < nsteps;
        const uint32_t slot = lds_addr + (uint32_t)((wave * P + u) * S::BSTEP);
#pragma unroll
        for (int j = 0; j < S::NB; ++j) {
            const int64_t k = g * S::SK + j * (1024 / (16 * S::ES)) + brow;
            const uint32_t o = in && k < a.K ? (uint32_t)(k * ldbb + ct * 16 * S::ES + bcol) : kOob;
            dma<16>(rb, slot + j * 1024, o);
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const bool live = in && t < nt;
            const uint32_t o = live ? voff[t] + (uint32_t)(g * VSTEP) : kOob;
            const uint32_t om = live ? moff[t] + (uint32_t)(g * MSTEP) : kOob;
            load_vals<S::VB, PK>(av[u][t], o, rv);
            load_mask<S::MB, PK>(mv[u][t], om, rm);
        }
    };

    Acc acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = Acc{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < P; ++u) issue(wave + (int64_t)W * u, u);
    lds_barrier();                                       // selector table written
    const int nw = nsteps > wave ? (int)((nsteps - wave + W - 1) / W) : 0;
    for (int i0 = 0; i0 < nw; i0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int i = i0 + u;
            if (i < nw) {
                // the oldest super-step in flight has landed once only the
                // P-1 younger ones remain; its registers are tied to the wait
                wait_vm<(P - 1) * GOPS>();
#pragma unroll
                for (int t = 0; t < TM; ++t) asm volatile("" : "+v"(av[u][t]), "+v"(mv[u][t]));
                const int64_t g = wave + (int64_t)W * i;
                const uint8_t* slot = lds + (wave * P + u) * S::BSTEP;
                uint32_t bf[S::F][S::FB / 4];
#pragma unroll
                for (int f = 0; f < S::F; ++f) nm_load_b<DT, NN, MM>(slot, lane, f, bf[f]);
                // dense k of the lane's range still inside K (K % MM == 0, so whole groups)
                const int64_t nv = a.K - (g * S::SK + q * S::D);
                const uint64_t keepm = nv >= S::D ? ~0ull : (nv <= 0 ? 0ull : ((1ull << nv) - 1ull));
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    uint32_t vw[S::VW];
                    widen_vals<DT, NN, MM>(av[u][t], vw);
                    const uint64_t mk = mask_bits<S::MB>(mv[u][t]) & keepm;
                    uint32_t dense[S::GL * S::OW];
#pragma unroll
                    for (int gg = 0; gg < S::GL; ++gg) {
                        const uint32_t gm = (uint32_t)(mk >> (gg * MM)) & ((1u << MM) - 1u);
                        const int byte0 = gg * S::GB;
                        const uint32_t s1 = S::GB == 8 ? vw[byte0 / 4] : vw[byte0 / 4] >> (8 * (byte0 % 4));
                        const uint32_t s0 = S::GB == 8 ? vw[byte0 / 4 + 1] : 0u;
                        uint32_t sv[S::OW];
                        if constexpr (S::OW == 4) {
                            const uint4 x = *reinterpret_cast<const uint4*>(lut + gm * 4);
                            sv[0] = x.x; sv[1] = x.y; sv[2] = x.z; sv[3] = x.w;
                        } else if constexpr (S::OW == 2) {
                            const uint2 x = *reinterpret_cast<const uint2*>(lut + gm * 2);
                            sv[0] = x.x; sv[1] = x.y;
                        } else {
                            sv[0] = lut[gm];
                        }
#pragma unroll
                        for (int s = 0; s < S::OW; ++s) dense[gg * S::OW + s] = __builtin_amdgcn_perm(s0, s1, sv[s]);
                    }
#pragma unroll
                    for (int f = 0; f < S::F; ++f)
                        acc[t] = nm_mfma<S::W4 ? DT_F16 : DT>(dense + f * (S::FB / 4), bf[f], acc[t]);
                }
                // the slot's LDS reads are done before its next B rows land
                __builtin_amdgcn_s_waitcnt(0xC07F);
                issue(wave + (int64_t)W * (i + P), u);
            }
        }
    }
    // the loads past the wave's last super-step land before the LDS is
    // reused, and before their registers are (an asm load's output counts as
    // written when issued, so the ring stays in use until the wait)
    wait_vm<0>();
#pragma unroll
    for (int u = 0; u < P; ++u)
#pragma unroll
        for (int t = 0; t < TM; ++t) asm volatile("" ::"v"(av[u][t]), "v"(mv[u][t]));
    lds_barrier();

    // fixed-order reduction of the waves' partial tiles
    Acc* red = reinterpret_cast<Acc*>(lds);
#pragma unroll
    for (int t = 0; t < TM; ++t) red[(wave * kNmTMax + t) * 64 + lane] = acc[t];
    lds_barrier();
    for (int i = threadIdx.x; i < nt * 256; i += blockDim.x) {
        const int t = i >> 8, ln = (i >> 2) & 63, e = i & 3;
        Out sum = Out(0);
#pragma unroll
        for (int w = 0; w < W; ++w) sum += reinterpret_cast<const Out*>(red)[((w * kNmTMax + t) * 64 + ln) * 4 + e];
        const int64_t row = 16 * (t0 + t) + 4 * (ln >> 4) + e;
        const int64_t col = 16 * ct + (ln & 15);
        if (row < a.M && col < a.N) reinterpret_cast<Out*>(a.C)[row * a.ldc + col] = sum;
    }
}

template <int DT, int NN, int MM, int TM, bool PK>
hipError_t launch_nm_tm(const SpmmArgs& a, int64_t tiles, int64_t G, hipStream_t s) {
    using S = NmShape<DT, NN, MM>;
    const unsigned shm = (unsigned)(kNmWaves * S::P * S::BSTEP + S::LUT);
    const dim3 grid((unsigned)G, (unsigned)((a.N + 15) / 16));
    hipLaunchKernelGGL((k_spmm_nm<DT, NN, MM, TM, PK>), grid, dim3(64 * kNmWaves), shm, s, a, tiles);
    return hipGetLastError();
}

template <int DT, int NN, int MM, bool PK>
hipError_t launch_nm_t(const SpmmArgs& a, hipStream_t s) {
    const int64_t tiles = (a.M + 15) / 16;
    int64_t G = tiles < 256 ? tiles : 256;
    if (G * kNmTMax < tiles) G = (tiles + kNmTMax - 1) / kNmTMax;
    switch ((int)((tiles + G - 1) / G)) {
        case 1: return launch_nm_tm<DT, NN, MM, 1, PK>(a, tiles, G, s);
        case 2: return launch_nm_tm<DT, NN, MM, 2, PK>(a, tiles, G, s);
        case 3: return launch_nm_tm<DT, NN, MM, 3, PK>(a, tiles, G, s);
        default: return launch_nm_tm<DT, NN, MM, 4, PK>(a, tiles, G, s);
    }
}

// ---- packed decode layout ----------------------------------------------------
//
// The product's operand in the order it is consumed: for each 16-row tile
// and super-step, the 64 lanes' VB value bytes (lane l = 16q + r: row r's
// stored bytes [4g*VB + q*VB, +VB) of super-step g; VB = 16, or 8 / 4 for
// 4-bit weights) as one block of 64*VB bytes, and their MB mask bytes (row
// r's mask bytes [4g*MB + q*MB, +MB)) as one block of 64*MB bytes.  A
// tile's blocks follow each other in g; bytes past a row's end and rows
// past M are zero.  Each load of the product is then one fully coalesced
// block instead of 16 row pieces.
__global__ void __launch_bounds__(256) k_pack_nm(int64_t M, int64_t tiles, int64_t nsteps, const uint8_t* vals,
                                                 int64_t ldvb, int64_t vrow, int vb, const uint8_t* mask, int64_t ldm,
                                                 int64_t mrow, int mb, uint8_t* pvals, uint8_t* pmask) {
    const int64_t n = tiles * nsteps * 64;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(i & 63);
        const int64_t blk = i >> 6, tile = blk / nsteps, g = blk - tile * nsteps;
        const int64_t row = 16 * tile + (lane & 15);
        const int q = lane >> 4;
        const int64_t v0 = g * 4 * vb + (int64_t)q * vb, m0 = g * 4 * mb + (int64_t)q * mb;
        for (int b = 0; b < vb; ++b) pvals[i * vb + b] = row < M && v0 + b < vrow ? vals[row * ldvb + v0 + b] : 0;
        for (int b = 0; b < mb; ++b) pmask[i * mb + b] = row < M && m0 + b < mrow ? mask[row * ldm + m0 + b] : 0;
    }
}

// Op<DT, NN, MM>::run(args...) for the runtime (dt, n, m).
template <template <int, int, int> class Op, int D, typename... Args>
hipError_t nm_pat(int n, int m, Args... args) {
    if (n == 1 && m == 4) {
        if constexpr (D == DT_I4) return hipErrorInvalidValue;   // 4-bit weights: whole bytes per group
        else return Op<D, 1, 4>::run(args...);
    }
    if (n == 2 && m == 4) return Op<D, 2, 4>::run(args...);
    if (n == 2 && m == 8) return Op<D, 2, 8>::run(args...);
    if (n == 4 && m == 8) return Op<D, 4, 8>::run(args...);
    return hipErrorInvalidValue;
}

template <template <int, int, int> class Op, typename... Args>
hipError_t nm_dispatch(int dt, int n, int m, Args... args) {
    switch (dt) {
        case DT_F16: return nm_pat<Op, DT_F16>(n, m, args...);
        case DT_BF16: return nm_pat<Op, DT_BF16>(n, m, args...);
        case DT_I8: return nm_pat<Op, DT_I8>(n, m, args...);
        case DT_E4M3: return nm_pat<Op, DT_E4M3>(n, m, args...);
        case DT_E5M2: return nm_pat<Op, DT_E5M2>(n, m, args...);
        case DT_I4: return nm_pat<Op, DT_I4>(n, m, args...);
        default: return hipErrorInvalidValue;
    }
}

unsigned nm_grid(int64_t M, int64_t K) {
    const int64_t n = M * ((K + kNmChunk - 1) / kNmChunk);
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < 4096 ? g : 4096);
}

}  // namespace

bool nm_pattern_supported(int n, int m) {
    return (n == 1 && m == 4) || (n == 2 && m == 4) || (n == 2 && m == 8) || (n == 4 && m == 8);
}

template <int D, int NN, int MM>
struct CompressNm {
    static hipError_t run(int64_t M, int64_t K, const void* A, int64_t lda, void* vals, int64_t ldv, uint8_t* mask,
                          int64_t ldm, bool vec, hipStream_t s) {
        hipLaunchKernelGGL((k_compress_nm<D, NN, MM>), dim3(nm_grid(M, K)), dim3(256), 0, s, M, K, A, lda, vals, ldv,
                           mask, ldm, (int)vec);
        return hipGetLastError();
    }
};

template <int D, int NN, int MM>
struct DecompressNm {
    static hipError_t run(int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* mask, int64_t ldm,
                          void* Dm, int64_t ldd, int32_t* bad, hipStream_t s) {
        hipLaunchKernelGGL((k_decompress_nm<D, NN, MM>), dim3(nm_grid(M, K)), dim3(256), 0, s, M, K, vals, ldv, mask,
                           ldm, Dm, ldd, bad);
        return hipGetLastError();
    }
};

template <int D, int NN, int MM>
struct SpmmNm {
    static hipError_t run(const SpmmArgs* a, bool packed, hipStream_t s) {
        return packed ? launch_nm_t<D, NN, MM, true>(*a, s) : launch_nm_t<D, NN, MM, false>(*a, s);
    }
};

hipError_t launch_compress_nm(int dt, int n, int m, int64_t M, int64_t K, const void* A, int64_t lda, void* vals,
                              int64_t ldv, uint8_t* mask, int64_t ldm, bool vec, hipStream_t s) {
    if (M == 0 || K == 0) return hipSuccess;
    return nm_dispatch<CompressNm>(dt, n, m, M, K, A, lda, vals, ldv, mask, ldm, vec, s);
}

hipError_t launch_decompress_nm(int dt, int n, int m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                                const uint8_t* mask, int64_t ldm, void* D, int64_t ldd, int32_t* bad, hipStream_t s) {
    if (M == 0 || K == 0) return hipSuccess;
    return nm_dispatch<DecompressNm>(dt, n, m, M, K, vals, ldv, mask, ldm, D, ldd, bad, s);
}

hipError_t launch_spmm_nm(int n, int m, const SpmmArgs& a, bool packed, hipStream_t s) {
    return nm_dispatch<SpmmNm>(a.dt, n, m, &a, packed, s);
}

void nm_packed_geometry(int dt, int n, int m, int64_t M, int64_t K, int64_t* tiles, int64_t* nsteps, int* vb,
                        int* mb) {
    // dense k per lane per super-step, as NmShape
    const int64_t d = dt == DT_I4 ? 32 : (16 / dt_bytes(dt)) * m / n;
    *tiles = (M + 15) / 16;
    *nsteps = (K + 4 * d - 1) / (4 * d);
    *vb = dt == DT_I4 ? (int)(d * n / m / 2) : 16;
    *mb = (int)(d / 8);
}

hipError_t launch_pack_nm(int dt, int n, int m, int64_t M, int64_t K, const void* vals, int64_t ldv,
                          const uint8_t* mask, int64_t ldm, void* pvals, void* pmask, hipStream_t s) {
    int64_t tiles, nsteps;
    int vb, mb;
    nm_packed_geometry(dt, n, m, M, K, &tiles, &nsteps, &vb, &mb);
    const int64_t lanes = tiles * nsteps * 64;
    if (lanes == 0) return hipSuccess;
    const int64_t g = (lanes + 255) / 256;
    // row bytes of the stored values: 4-bit weights are two per byte
    const int64_t ldvb = dt == DT_I4 ? ldv / 2 : ldv * dt_bytes(dt);
    const int64_t vrow = dt == DT_I4 ? K / m * n / 2 : K / m * n * dt_bytes(dt);
    hipLaunchKernelGGL(k_pack_nm, dim3((unsigned)(g < 8192 ? g : 8192)), dim3(256), 0, s, M, tiles, nsteps,
                       (const uint8_t*)vals, ldvb, vrow, vb, mask, ldm, (K + 7) / 8, mb, (uint8_t*)pvals,
                       (uint8_t*)pmask);
    return hipGetLastError();
}

}  // namespace ssg
