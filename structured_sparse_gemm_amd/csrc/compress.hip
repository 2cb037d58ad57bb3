// compress.hip -- HIP kernels that turn a dense weight into its 2:4 form:
// magnitude prune, compress (values + 2-bit positions), expand back, and the
// two-pass split of a moderately unstructured weight into a 2:4 layer plus a
// CSR residual of the dropped non-zeros.
//
// Selection follows "Chapter 26 -- Sparsity: The Hardware View", section
// "Python: Build a 2:4 Mask, Compress It, ..." (keep the two largest
// magnitudes of each group of 4 along K, positions ascending); the storage
// follows the worked example of its section "2:4 Fine-Grained Structured
// Sparsity"; the residual follows "How sparse LLM weights cut GPU inference
// cost without quantization", section "How the three-layer format makes
// moderate sparsity fast".
//
// Work unit: one thread owns a chunk of 8 groups (32 elements) of one row,
// so it writes whole metadata bytes (4 bytes = 8 nibbles) and never shares a
// byte with another thread.  Full chunks with aligned rows use 16-byte loads
// and stores; the ragged last chunk of a row and unaligned operands take
// element-wise accesses in the same kernels.  All of these kernels are
// HBM-bound streaming passes.
#include "ssg_device.hpp"
#include "ssg_kernels.hpp"

namespace ssg {

namespace {

constexpr int kChunkGroups = 8;
constexpr int kChunkElems = 32;
#ifndef SSG_COMPRESS_BLOCKS
#define SSG_COMPRESS_BLOCKS 2048
#endif
constexpr int64_t kCompressBlocks = SSG_COMPRESS_BLOCKS;   // grid cap of the compress pass

// Raw storage word of one element: uint16_t for fp16/bf16, int8_t for int8,
// uint8_t for the 8-bit floats.
template <int DT> struct Store { using T = uint16_t; };
template <> struct Store<DT_I8> { using T = int8_t; };
template <> struct Store<DT_E4M3> { using T = uint8_t; };
template <> struct Store<DT_E5M2> { using T = uint8_t; };

template <int DT>
__device__ __forceinline__ uint32_t key_of(typename Store<DT>::T x) {
    if constexpr (DT == DT_I8) return mag_key8((int32_t)x);
    else if constexpr (dt_is_fp8(DT)) return mag_key_fp8((uint32_t)x);
    else return mag_key16((uint32_t)x);
}

// Loads the chunk's 4*ng elements (ng <= 8) into x[0..31]; missing ones are 0.
template <int DT>
__device__ __forceinline__ void load_chunk(const typename Store<DT>::T* a, int ng, bool vec,
                                           typename Store<DT>::T (&x)[kChunkElems]) {
    using T = typename Store<DT>::T;
    if (vec && ng == kChunkGroups) {
        constexpr int kVecs = kChunkElems * sizeof(T) / 16;
        uint4 w[kVecs];
#pragma unroll
        for (int i = 0; i < kVecs; ++i) w[i] = reinterpret_cast<const uint4*>(a)[i];
        __builtin_memcpy(x, w, sizeof(w));
    } else {
#pragma unroll
        for (int i = 0; i < kChunkElems; ++i) x[i] = (i < 4 * ng) ? a[i] : T(0);
    }
}

template <typename T>
__device__ __forceinline__ T pick_low(uint32_t i0, T x0, T x1, T x2) { return i0 == 0 ? x0 : (i0 == 1 ? x1 : x2); }
template <typename T>
__device__ __forceinline__ T pick_high(uint32_t i1, T x1, T x2, T x3) { return i1 == 1 ? x1 : (i1 == 2 ? x2 : x3); }

// Nibbles of the chunk (nibble g at bits 4g..4g+3) and the kept values.
template <int DT>
__device__ __forceinline__ uint32_t select_chunk(const typename Store<DT>::T (&x)[kChunkElems], int ng,
                                                 typename Store<DT>::T (&v)[2 * kChunkGroups]) {
    uint32_t word = 0;
#pragma unroll
    for (int g = 0; g < kChunkGroups; ++g) {
        const uint32_t nib = select_nibble(key_of<DT>(x[4 * g]), key_of<DT>(x[4 * g + 1]),
                                           key_of<DT>(x[4 * g + 2]), key_of<DT>(x[4 * g + 3]));
        v[2 * g] = pick_low(nib & 3u, x[4 * g], x[4 * g + 1], x[4 * g + 2]);
        v[2 * g + 1] = pick_high(nib >> 2, x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]);
        if (g < ng) word |= nib << (4 * g);
    }
    return word;
}

template <int DT>
__device__ __forceinline__ void store_compressed(typename Store<DT>::T* vrow, uint8_t* mrow, int ng, bool vec,
                                                 const typename Store<DT>::T (&v)[2 * kChunkGroups], uint32_t word) {
    using T = typename Store<DT>::T;
    if (vec && ng == kChunkGroups) {
        constexpr int kVecs = 2 * kChunkGroups * sizeof(T) / 16;
        uint4 w[kVecs];
        __builtin_memcpy(w, v, sizeof(w));
#pragma unroll
        for (int i = 0; i < kVecs; ++i) reinterpret_cast<uint4*>(vrow)[i] = w[i];
        *reinterpret_cast<uint32_t*>(mrow) = word;
    } else {
#pragma unroll
        for (int i = 0; i < 2 * kChunkGroups; ++i)
            if (i < 2 * ng) vrow[i] = v[i];
#pragma unroll
        for (int j = 0; j < kChunkGroups / 2; ++j)
            if (2 * j < ng) mrow[j] = (uint8_t)(word >> (8 * j));
    }
}

// Grid-stride loop over chunks with the next chunk's loads in flight while
// the current one is selected and stored, so reads and writes of the pass
// overlap instead of running as one load phase followed by one store phase.
template <int DT>
__global__ void __launch_bounds__(256) k_compress(int64_t M, int64_t K, const typename Store<DT>::T* __restrict__ A,
                                                  int64_t lda, typename Store<DT>::T* __restrict__ vals, int64_t ldv,
                                                  uint8_t* __restrict__ meta, int64_t ldm, int vec) {
    using T = typename Store<DT>::T;
    const int64_t chunks = (K + kChunkElems - 1) / kChunkElems;
    const int64_t total = M * chunks;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= total) return;
    int64_t m = t / chunks, c = t - m * chunks;
    int ng = (int)min<int64_t>(kChunkGroups, (K - c * kChunkElems) / 4);
    T x[kChunkElems];
    load_chunk<DT>(A + m * lda + c * kChunkElems, ng, vec != 0, x);
    for (;;) {
        const int64_t tn = t + stride;
        const bool more = tn < total;
        int64_t mn = 0, cn = 0;
        int ngn = 0;
        T xn[kChunkElems];
        if (more) {
            mn = tn / chunks;
            cn = tn - mn * chunks;
            ngn = (int)min<int64_t>(kChunkGroups, (K - cn * kChunkElems) / 4);
            load_chunk<DT>(A + mn * lda + cn * kChunkElems, ngn, vec != 0, xn);
        }
        T v[2 * kChunkGroups];
        uint32_t word = select_chunk<DT>(x, ng, v);
        store_compressed<DT>(vals + m * ldv + c * 2 * kChunkGroups, meta + m * ldm + c * (kChunkGroups / 2), ng,
                             vec != 0, v, word);
        if (!more) break;
#pragma unroll
        for (int i = 0; i < kChunkElems; ++i) x[i] = xn[i];
        t = tn;
        m = mn;
        c = cn;
        ng = ngn;
    }
}

// Packed prefill output, one workgroup per (256-row tile, metadata block):
// the block's stored values (4 stages of 64 stored bytes per row for 16-bit
// types, 2 for 8-bit ones) and its metadata block are assembled in LDS at
// their positions in the layout and then written out as the two contiguous
// runs they are in HBM (16, 32 or 64 KiB of values, 8 KiB of metadata), so
// every store is a whole 16-byte piece and every line is written whole.
// Thread t of 512 takes chunk c = t % 8 (32 dense k) of rows t / 8 + 64 i,
// all 4 chunk loads in flight before the first selection; two workgroups fit
// a CU, so one streams while the other selects and stores.  Rows past M and
// chunks past K are zeros.
constexpr int kPrefillThreads = 512;

template <int DT>
__global__ void __launch_bounds__(kPrefillThreads) k_compress_prefill(int64_t M, int64_t K, const typename Store<DT>::T* A,
                                                          int64_t lda, uint8_t* __restrict__ pvals,
                                                          uint8_t* __restrict__ pmeta, int vec, int64_t stages,
                                                          int64_t mblocks) {
    using T = typename Store<DT>::T;
    constexpr int ES = (int)sizeof(T);
    constexpr int SPB = 2 * ES;                  // stages per metadata block (256 dense k)
    constexpr int CPS = 4 / ES;                  // 32-element chunks per stage
    constexpr int IW = ES == 1 ? 4 : 2;          // index-word bytes
    constexpr int kRows = 256 / (kPrefillThreads / 8);   // rows per thread
    __shared__ __attribute__((aligned(16))) uint8_t lds[SPB * 16384 + 8192];
    uint8_t* const lmeta = lds + SPB * 16384;
    const int64_t tile = blockIdx.x / mblocks, g = blockIdx.x - tile * mblocks;
    const int nst = (int)min<int64_t>(SPB, stages - g * SPB);   // stages of this block inside K
    const int c = threadIdx.x & 7, r0 = threadIdx.x >> 3;
    const bool in_k = c < nst * CPS;
    const int64_t k0 = g * 256 + (int64_t)c * kChunkElems;

    // raw 16-byte pieces of the chunks (kept packed until each is selected)
    constexpr int kVecs = kChunkElems * ES / 16;
    const bool fast = vec != 0;
    uint4 raw[kRows][kVecs];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int64_t m = tile * 256 + r0 + (kPrefillThreads / 8) * i;
        const bool ld = in_k && m < M;
#pragma unroll
        for (int j = 0; j < kVecs; ++j) raw[i][j] = make_uint4(0, 0, 0, 0);
        if (ld && fast) {
#pragma unroll
            for (int j = 0; j < kVecs; ++j) raw[i][j] = reinterpret_cast<const uint4*>(A + m * lda + k0)[j];
        } else if (ld) {
            T x[kChunkElems];
            load_chunk<DT>(A + m * lda + k0, kChunkGroups, false, x);
            __builtin_memcpy(raw[i], x, sizeof(x));
        }
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        const int r = r0 + (kPrefillThreads / 8) * i;
        const bool live = in_k && tile * 256 + r < M;
        T x[kChunkElems];
        __builtin_memcpy(x, raw[i], sizeof(x));
        T v[2 * kChunkGroups];
        uint32_t word = select_chunk<DT>(x, kChunkGroups, v);
        if (!live) {
            word = 0;
#pragma unroll
            for (int e = 0; e < 2 * kChunkGroups; ++e) v[e] = T(0);
        }
        // the chunk's stored values: bytes [16 c ES, 16 c ES + 16 ES) of the
        // row's stored bytes in this block, i.e. ES 16-byte pieces of stage
        // c / CPS (pieces past the block's last stage are never written out)
        uint4 w[ES];
        __builtin_memcpy(w, v, sizeof(w));
        const int st = c / CPS;
#pragma unroll
        for (int j = 0; j < ES; ++j) {
            const int piece = (c % CPS) * ES + j;
            *reinterpret_cast<uint4*>(lds + st * 16384 + (prefill_vals_unit(r, piece) << 4)) = w[j];
        }
        // its 4 metadata bytes (block bytes [4 c, 4 c + 4) of the row): one
        // index word for 8-bit types, two for 16-bit ones, each whole at its
        // position in the block
#pragma unroll
        for (int j = 0; j < 4 / IW; ++j) {
            const int pos = prefill_meta_pos(r, 4 * c + IW * j, IW);
            if constexpr (IW == 4) *reinterpret_cast<uint32_t*>(lmeta + pos) = word;
            else *reinterpret_cast<uint16_t*>(lmeta + pos) = (uint16_t)(word >> (16 * j));
        }
    }
    __syncthreads();
    uint8_t* const vdst = pvals + ((tile * stages + g * SPB) << 14);
    for (int o = threadIdx.x * 16; o < nst * 16384; o += kPrefillThreads * 16)
        *reinterpret_cast<uint4*>(vdst + o) = *reinterpret_cast<const uint4*>(lds + o);
    uint8_t* const mdst = pmeta + ((tile * mblocks + g) << 13);
    for (int o = threadIdx.x * 16; o < 8192; o += kPrefillThreads * 16)
        *reinterpret_cast<uint4*>(mdst + o) = *reinterpret_cast<const uint4*>(lmeta + o);
}

template <int DT>
__global__ void __launch_bounds__(256) k_prune(int64_t M, int64_t K, const typename Store<DT>::T* A, int64_t lda,
                                               typename Store<DT>::T* P, int64_t ldp, int vec) {
    using T = typename Store<DT>::T;
    const int64_t chunks = (K + kChunkElems - 1) / kChunkElems;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= M * chunks) return;
    const int64_t m = t / chunks, c = t - m * chunks;
    const int ng = (int)min<int64_t>(kChunkGroups, (K - c * kChunkElems) / 4);
    T x[kChunkElems], v[2 * kChunkGroups];
    load_chunk<DT>(A + m * lda + c * kChunkElems, ng, vec != 0, x);   // whole chunk read before any write
    const uint32_t word = select_chunk<DT>(x, ng, v);
#pragma unroll
    for (int g = 0; g < kChunkGroups; ++g) {
        const uint32_t nib = (word >> (4 * g)) & 0xFu, i0 = nib & 3u, i1 = nib >> 2;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            if (p != (int)i0 && p != (int)i1) x[4 * g + p] = T(0);
    }
    T* prow = P + m * ldp + c * kChunkElems;
    if (vec && ng == kChunkGroups) {
        constexpr int kVecs = kChunkElems * sizeof(T) / 16;
        uint4 w[kVecs];
        __builtin_memcpy(w, x, sizeof(w));
#pragma unroll
        for (int i = 0; i < kVecs; ++i) reinterpret_cast<uint4*>(prow)[i] = w[i];
    } else {
#pragma unroll
        for (int i = 0; i < kChunkElems; ++i)
            if (i < 4 * ng) prow[i] = x[i];
    }
}

template <int DT>
__global__ void __launch_bounds__(256) k_decompress(int64_t M, int64_t K, const typename Store<DT>::T* vals,
                                                    int64_t ldv, const uint8_t* meta, int64_t ldm,
                                                    typename Store<DT>::T* D, int64_t ldd, int32_t* bad_count,
                                                    int vec) {
    using T = typename Store<DT>::T;
    const int64_t chunks = (K + kChunkElems - 1) / kChunkElems;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= M * chunks) return;
    const int64_t m = t / chunks, c = t - m * chunks;
    const int ng = (int)min<int64_t>(kChunkGroups, (K - c * kChunkElems) / 4);
    const T* vrow = vals + m * ldv + c * 2 * kChunkGroups;
    const uint8_t* mrow = meta + m * ldm + c * (kChunkGroups / 2);
    T v[2 * kChunkGroups];
    uint32_t word = 0;
    if (vec && ng == kChunkGroups) {
        constexpr int kVecs = 2 * kChunkGroups * sizeof(T) / 16;
        uint4 w[kVecs];
#pragma unroll
        for (int i = 0; i < kVecs; ++i) w[i] = reinterpret_cast<const uint4*>(vrow)[i];
        __builtin_memcpy(v, w, sizeof(w));
        word = *reinterpret_cast<const uint32_t*>(mrow);
    } else {
#pragma unroll
        for (int i = 0; i < 2 * kChunkGroups; ++i) v[i] = (i < 2 * ng) ? vrow[i] : T(0);
#pragma unroll
        for (int j = 0; j < kChunkGroups / 2; ++j)
            if (2 * j < ng) word |= (uint32_t)mrow[j] << (8 * j);
    }
    T x[kChunkElems];
    int bad = 0;
#pragma unroll
    for (int g = 0; g < kChunkGroups; ++g) {
        const uint32_t nib = (word >> (4 * g)) & 0xFu, i0 = nib & 3u, i1 = nib >> 2;
        const bool ok = nibble_valid(nib);
        if (g < ng && !ok) ++bad;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            x[4 * g + p] = (ok && p == (int)i0) ? v[2 * g] : ((ok && p == (int)i1) ? v[2 * g + 1] : T(0));
    }
    T* drow = D + m * ldd + c * kChunkElems;
    if (vec && ng == kChunkGroups) {
        constexpr int kVecs = kChunkElems * sizeof(T) / 16;
        uint4 w[kVecs];
        __builtin_memcpy(w, x, sizeof(w));
#pragma unroll
        for (int i = 0; i < kVecs; ++i) reinterpret_cast<uint4*>(drow)[i] = w[i];
    } else {
#pragma unroll
        for (int i = 0; i < kChunkElems; ++i)
            if (i < 4 * ng) drow[i] = x[i];
    }
    if (bad && bad_count) atomicAdd(bad_count, bad);
}

// ---- residual split -------------------------------------------------------

constexpr int kSplitThreads = 256;

// Exclusive prefix sum over a 256-thread block; *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* lds4) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) lds4[wid] = x;
    __syncthreads();
    int before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < kSplitThreads / 64; ++w) {
        const int s = lds4[w];
        before += (w < wid) ? s : 0;
        sum += s;
    }
    __syncthreads();
    *total = sum;
    return before + x - v;
}

// Dropped non-zeros of a chunk as a bit mask over its 32 elements.
template <int DT>
__device__ __forceinline__ uint32_t overflow_mask(const typename Store<DT>::T (&x)[kChunkElems], uint32_t word,
                                                  int ng) {
    uint32_t mask = 0;
#pragma unroll
    for (int g = 0; g < kChunkGroups; ++g) {
        const uint32_t nib = (word >> (4 * g)) & 0xFu, i0 = nib & 3u, i1 = nib >> 2;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const bool dropped_nonzero = p != (int)i0 && p != (int)i1 && key_of<DT>(x[4 * g + p]) != 0u;
            if (g < ng && dropped_nonzero) mask |= 1u << (4 * g + p);
        }
    }
    return mask;
}

// Pass 1: per-row counts into row_ptr[m + 1]; one block per row (grid-stride).
template <int DT>
__global__ void __launch_bounds__(kSplitThreads) k_split_count(int64_t M, int64_t K, const typename Store<DT>::T* A,
                                                               int64_t lda, int32_t* row_ptr, int vec) {
    using T = typename Store<DT>::T;
    __shared__ int lds4[kSplitThreads / 64];
    const int64_t chunks = (K + kChunkElems - 1) / kChunkElems;
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
        int cnt = 0;
        for (int64_t c = threadIdx.x; c < chunks; c += kSplitThreads) {
            const int ng = (int)min<int64_t>(kChunkGroups, (K - c * kChunkElems) / 4);
            T x[kChunkElems], v[2 * kChunkGroups];
            load_chunk<DT>(A + m * lda + c * kChunkElems, ng, vec != 0, x);
            const uint32_t word = select_chunk<DT>(x, ng, v);
            cnt += __popc(overflow_mask<DT>(x, word, ng));
        }
        int total;
        block_exclusive_scan(cnt, &total, lds4);
        if (threadIdx.x == 0) row_ptr[m + 1] = total;
    }
}

// Inclusive scan of row_ptr[1..M] in place, row_ptr[0] = 0; one block.
__global__ void __launch_bounds__(1024) k_scan_rows(int64_t M, int32_t* row_ptr) {
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (threadIdx.x == 0) { row_ptr[0] = 0; carry_s = 0; }
    __syncthreads();
    for (int64_t base = 0; base < M; base += 1024) {
        const int64_t i = base + threadIdx.x;
        const int v = (i < M) ? row_ptr[i + 1] : 0;
        int x = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wsum[wid] = x;
        __syncthreads();
        int before = carry_s, sum = 0;
        for (int w = 0; w < 16; ++w) {
            before += (w < wid) ? wsum[w] : 0;
            sum += wsum[w];
        }
        if (i < M) row_ptr[i + 1] = before + x;
        __syncthreads();
        if (threadIdx.x == 0) carry_s += sum;
        __syncthreads();
    }
}

// Pass 2: the 2:4 layer and the CSR residual; one block per row (grid-stride).
// Chunks are taken 256 at a time in K order; a block scan places each
// thread's dropped non-zeros after those of lower chunks, so columns come
// out ascending.
template <int DT>
__global__ void __launch_bounds__(kSplitThreads) k_split_fill(int64_t M, int64_t K, const typename Store<DT>::T* A,
                                                              int64_t lda, typename Store<DT>::T* vals, int64_t ldv,
                                                              uint8_t* meta, int64_t ldm, const int32_t* row_ptr,
                                                              int32_t* col, typename Store<DT>::T* rvals, int vec) {
    using T = typename Store<DT>::T;
    __shared__ int lds4[kSplitThreads / 64];
    const int64_t chunks = (K + kChunkElems - 1) / kChunkElems;
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
        int64_t carry = row_ptr[m];
        for (int64_t c0 = 0; c0 < chunks; c0 += kSplitThreads) {
            const int64_t c = c0 + threadIdx.x;
            uint32_t mask = 0;
            T x[kChunkElems];
            if (c < chunks) {
                const int ng = (int)min<int64_t>(kChunkGroups, (K - c * kChunkElems) / 4);
                T v[2 * kChunkGroups];
                load_chunk<DT>(A + m * lda + c * kChunkElems, ng, vec != 0, x);
                const uint32_t word = select_chunk<DT>(x, ng, v);
                store_compressed<DT>(vals + m * ldv + c * 2 * kChunkGroups, meta + m * ldm + c * (kChunkGroups / 2),
                                     ng, vec != 0, v, word);
                mask = overflow_mask<DT>(x, word, ng);
            }
            int total;
            const int before = block_exclusive_scan(__popc(mask), &total, lds4);
            if (col != nullptr) {
                int64_t pos = carry + before;
#pragma unroll
                for (int i = 0; i < kChunkElems; ++i) {
                    if (mask & (1u << i)) {
                        col[pos] = (int32_t)(c * kChunkElems + i);
                        rvals[pos] = x[i];
                        ++pos;
                    }
                }
            }
            carry += total;
        }
    }
}

// ---- delta-coded residual --------------------------------------------------
//
// Compact residual: entry j of a row stores its column as the one-byte gap
// d = col_j - col_(j-1) (col_(-1) = -1), and a gap above 255 is bridged by
// filler entries (d = 255, value +0) in front of it, floor((gap - 1) / 255)
// of them.  "How sparse LLM weights cut GPU inference cost without
// quantization", section "How the three-layer format makes moderate sparsity
// fast", names such a differential position code decoded on chip; the byte
// layout is this library's own.  Both passes read the CSR through the same
// clamps (entries to [0, nnz), columns to [0, K - 1], a gap below 1 taken as
// 1), so the fill writes exactly the entries the count gave each row, even
// for a malformed CSR.

struct DeltaEntry {
    int fillers;   // filler entries in front of the entry
    int d;         // the entry's own gap byte, in [1, 255]
};

__device__ __forceinline__ DeltaEntry delta_entry(const int32_t* col, int64_t j, int64_t lo, int64_t K) {
    const int64_t c = min<int64_t>(max<int64_t>(col[j], 0), K - 1);
    const int64_t p = j > lo ? min<int64_t>(max<int64_t>(col[j - 1], 0), K - 1) : -1;
    const int64_t gap = max<int64_t>(c - p, 1);
    const int f = (int)((gap - 1) / 255);
    return DeltaEntry{f, (int)(gap - 255 * (int64_t)f)};
}

__device__ __forceinline__ void csr_row_range(const int32_t* row_ptr, int64_t m, int64_t nnz, int64_t* lo,
                                              int64_t* hi) {
    *lo = min<int64_t>(max<int64_t>(row_ptr[m], 0), nnz);
    *hi = min<int64_t>(max<int64_t>(row_ptr[m + 1], *lo), nnz);
}

// Pass 1: entries of row m (fillers included) into drow_ptr[m + 1]; one block
// per row (grid-stride).
__global__ void __launch_bounds__(kSplitThreads) k_delta_count(int64_t M, int64_t K, const int32_t* row_ptr,
                                                               const int32_t* col, int64_t nnz, int32_t* drow_ptr) {
    __shared__ int lds4[kSplitThreads / 64];
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
        int64_t lo, hi;
        csr_row_range(row_ptr, m, nnz, &lo, &hi);
        int cnt = 0;
        for (int64_t j = lo + threadIdx.x; j < hi; j += kSplitThreads) cnt += 1 + delta_entry(col, j, lo, K).fillers;
        int total;
        block_exclusive_scan(cnt, &total, lds4);
        if (threadIdx.x == 0) drow_ptr[m + 1] = total;
    }
}

// Pass 2: the gap bytes and values; 256 entries of a row at a time, a block
// scan placing each entry (and its fillers) after those of lower threads.
template <int DT>
__global__ void __launch_bounds__(kSplitThreads) k_delta_fill(int64_t M, int64_t K, const int32_t* row_ptr,
                                                              const int32_t* col, const typename Store<DT>::T* rvals,
                                                              int64_t nnz, const int32_t* drow_ptr, uint8_t* dcol,
                                                              typename Store<DT>::T* dvals) {
    using T = typename Store<DT>::T;
    __shared__ int lds4[kSplitThreads / 64];
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
        int64_t lo, hi;
        csr_row_range(row_ptr, m, nnz, &lo, &hi);
        const int64_t end = drow_ptr[m + 1];
        int64_t carry = drow_ptr[m];
        for (int64_t j0 = lo; j0 < hi; j0 += kSplitThreads) {
            const int64_t j = j0 + threadIdx.x;
            const bool have = j < hi;
            DeltaEntry e{0, 0};
            if (have) e = delta_entry(col, j, lo, K);
            int total;
            const int before = block_exclusive_scan(have ? 1 + e.fillers : 0, &total, lds4);
            int64_t pos = carry + before;
            for (int i = 0; i < e.fillers; ++i, ++pos) {
                if (pos < end) {
                    dcol[pos] = 255;
                    dvals[pos] = T(0);
                }
            }
            if (have && pos < end) {
                dcol[pos] = (uint8_t)e.d;
                dvals[pos] = rvals[j];
            }
            carry += total;
        }
    }
}

inline unsigned blocks_for(int64_t threads, int per_block) {
    return (unsigned)((threads + per_block - 1) / per_block);
}

}  // namespace

// ---- host launchers --------------------------------------------------------

#define SSG_DISPATCH_DT(dt, BODY)                                        \
    switch (dt) {                                                        \
        case DT_F16: { constexpr int D = DT_F16; BODY; } break;           \
        case DT_BF16: { constexpr int D = DT_BF16; BODY; } break;         \
        case DT_I8: { constexpr int D = DT_I8; BODY; } break;             \
        case DT_E4M3: { constexpr int D = DT_E4M3; BODY; } break;         \
        case DT_E5M2: { constexpr int D = DT_E5M2; BODY; } break;         \
        default: return hipErrorInvalidValue;                            \
    }

hipError_t launch_compress(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* vals, int64_t ldv,
                           uint8_t* meta, int64_t ldm, bool vec, hipStream_t s) {
    const int64_t threads = M * ((K + kChunkElems - 1) / kChunkElems);
    if (threads == 0) return hipSuccess;
    // a few chunks per thread: enough waves to cover latency, few enough that
    // each thread's loop overlaps its next loads with its stores
    int64_t blocks = blocks_for(threads, 256);
    if (blocks > kCompressBlocks) blocks = kCompressBlocks;
    SSG_DISPATCH_DT(dt, {
        using T = typename Store<D>::T;
        hipLaunchKernelGGL((k_compress<D>), dim3((unsigned)blocks), dim3(256), 0, s, M, K, (const T*)A, lda,
                           (T*)vals, ldv, meta, ldm, (int)vec);
    });
    return hipGetLastError();
}

hipError_t launch_compress_prefill(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* pvals,
                                   void* pmeta, bool vec, hipStream_t s) {
    int64_t tiles, stages, mblocks;
    prefill_geometry(dt, M, K, &tiles, &stages, &mblocks);
    const int64_t blocks = tiles * mblocks;
    if (blocks == 0) return hipSuccess;
    SSG_DISPATCH_DT(dt, {
        using T = typename Store<D>::T;
        hipLaunchKernelGGL(k_compress_prefill<D>, dim3((unsigned)blocks), dim3(kPrefillThreads), 0, s, M, K, (const T*)A, lda,
                           (uint8_t*)pvals, (uint8_t*)pmeta, (int)vec, stages, mblocks);
    });
    return hipGetLastError();
}

hipError_t launch_prune(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* P, int64_t ldp, bool vec,
                        hipStream_t s) {
    const int64_t threads = M * ((K + kChunkElems - 1) / kChunkElems);
    if (threads == 0) return hipSuccess;
    SSG_DISPATCH_DT(dt, {
        using T = typename Store<D>::T;
        hipLaunchKernelGGL(k_prune<D>, dim3(blocks_for(threads, 256)), dim3(256), 0, s, M, K, (const T*)A, lda,
                           (T*)P, ldp, (int)vec);
    });
    return hipGetLastError();
}

hipError_t launch_decompress(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                             int64_t ldm, void* D_, int64_t ldd, int32_t* bad, bool vec, hipStream_t s) {
    const int64_t threads = M * ((K + kChunkElems - 1) / kChunkElems);
    if (threads == 0) return hipSuccess;
    SSG_DISPATCH_DT(dt, {
        using T = typename Store<D>::T;
        hipLaunchKernelGGL(k_decompress<D>, dim3(blocks_for(threads, 256)), dim3(256), 0, s, M, K, (const T*)vals,
                           ldv, meta, ldm, (T*)D_, ldd, bad, (int)vec);
    });
    return hipGetLastError();
}

hipError_t launch_split_count(int dt, int64_t M, int64_t K, const void* A, int64_t lda, int32_t* row_ptr, bool vec,
                              hipStream_t s) {
    const unsigned grid = (unsigned)(M < 65536 ? M : 65536);
    if (M > 0) {
        SSG_DISPATCH_DT(dt, {
            using T = typename Store<D>::T;
            hipLaunchKernelGGL(k_split_count<D>, dim3(grid), dim3(kSplitThreads), 0, s, M, K, (const T*)A, lda,
                               row_ptr, (int)vec);
        });
    }
    hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(1024), 0, s, M, row_ptr);
    return hipGetLastError();
}

hipError_t launch_split_fill(int dt, int64_t M, int64_t K, const void* A, int64_t lda, void* vals, int64_t ldv,
                             uint8_t* meta, int64_t ldm, const int32_t* row_ptr, int32_t* col, void* rvals, bool vec,
                             hipStream_t s) {
    if (M == 0) return hipSuccess;
    const unsigned grid = (unsigned)(M < 65536 ? M : 65536);
    SSG_DISPATCH_DT(dt, {
        using T = typename Store<D>::T;
        hipLaunchKernelGGL(k_split_fill<D>, dim3(grid), dim3(kSplitThreads), 0, s, M, K, (const T*)A, lda, (T*)vals,
                           ldv, meta, ldm, row_ptr, col, (T*)rvals, (int)vec);
    });
    return hipGetLastError();
}

hipError_t launch_delta_count(int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col, int64_t nnz,
                              int32_t* drow_ptr, hipStream_t s) {
    if (M > 0 && K > 0) {
        const unsigned grid = (unsigned)(M < 65536 ? M : 65536);
        hipLaunchKernelGGL(k_delta_count, dim3(grid), dim3(kSplitThreads), 0, s, M, K, row_ptr, col, nnz, drow_ptr);
    } else if (M > 0) {
        // no columns: every row is empty
        hipLaunchKernelGGL(k_delta_count, dim3(1), dim3(kSplitThreads), 0, s, M, K, row_ptr, col, (int64_t)0,
                           drow_ptr);
    }
    hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(1024), 0, s, M, drow_ptr);
    return hipGetLastError();
}

hipError_t launch_scan_counts(int64_t n, int32_t* a, hipStream_t s) {
    hipLaunchKernelGGL(k_scan_rows, dim3(1), dim3(1024), 0, s, n, a);
    return hipGetLastError();
}

hipError_t launch_delta_fill(int dt, int64_t M, int64_t K, const int32_t* row_ptr, const int32_t* col,
                             const void* rvals, int64_t nnz, const int32_t* drow_ptr, uint8_t* dcol, void* dvals,
                             hipStream_t s) {
    if (M == 0 || K == 0 || nnz == 0) return hipSuccess;
    const unsigned grid = (unsigned)(M < 65536 ? M : 65536);
    SSG_DISPATCH_DT(dt, {
        using T = typename Store<D>::T;
        hipLaunchKernelGGL(k_delta_fill<D>, dim3(grid), dim3(kSplitThreads), 0, s, M, K, row_ptr, col,
                           (const T*)rvals, nnz, drow_ptr, dcol, (T*)dvals);
    });
    return hipGetLastError();
}

}  // namespace ssg
