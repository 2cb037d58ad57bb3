// residual_cbm.hip -- encoder of the complement-bitmap residual, the
// residual layer in the packed decode product's block order.
//
// "How sparse LLM weights cut GPU inference cost without quantization",
// section "How the three-layer format makes moderate sparsity fast", keeps
// what the 2:4 layer drops in a residual layer that is decoded in parallel on
// chip and runs in the same pipeline as the structured layer; it gives no
// layout.  This one rests on a fact of the split: a residual entry of a group
// can only sit at one of the two positions the 2:4 layer did not keep (its
// complement positions).  So, for every lane of a packed decode block (16
// rows x one k-step; lane l = 16q + r: row r, dense columns [q*EB, (q+1)*EB)
// of the k-step, EB = 16 for 16-bit types and 32 for 8-bit ones):
//   rmask  one little-endian word of 2 bits per group (1 byte for 16-bit
//          types, 2 for 8-bit): bit 2*gi + j set iff the residual holds a
//          value at complement position c_j (c0 < c1) of the lane's group gi;
//   roff   int32 per block, the number of entries in the blocks before it,
//          plus one final entry holding the total;
//   cvals  the values, bit-copied, in block, lane and bit order.
// The encoder takes the CSR residual (columns ascending) and the row-major
// metadata of the 2:4 layer.  Pass 1 writes every lane's mask word and the
// block's entry count into roff[b + 1]; a scan turns the counts into offsets;
// pass 2 writes the values, each lane after the lanes before it (a wave
// prefix sum of the mask popcounts).  An entry at a kept position of its
// group (or one whose group has an invalid nibble) is counted into *bad and
// left out.
#include "ssg_device.hpp"
#include "ssg_kernels.hpp"

namespace ssg {

namespace {

constexpr int kCbmThreads = 256;   // four waves, one block each

struct CbmGeom {
    int64_t M, K, tiles, ksteps;
    int ks, eb, gl;                // dense k per k-step, per lane, groups per lane
};

__device__ __forceinline__ int wave_excl_sum(int x, int lane) {
    int v = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(v, d, 64);
        if (lane >= d) v += y;
    }
    return v - x;
}

// The lane's residual entries [j0, j1) (columns in its range) and its mask
// word.  Entries at kept positions are flagged in `badmask` (bit per entry
// index from j0) and have no mask bit.
__device__ __forceinline__ uint32_t lane_mask(const CbmGeom& g, const uint8_t* meta, int64_t ldm,
                                              const int32_t* row_ptr, const int32_t* col, int64_t nnz, int64_t m,
                                              int64_t kb, int64_t* j0_out, int* n_out, uint32_t* badmask) {
    *j0_out = 0;
    *n_out = 0;
    *badmask = 0;
    if (m >= g.M) return 0;
    int64_t lo = min<int64_t>(max<int64_t>(row_ptr[m], 0), nnz), hi = min<int64_t>(max<int64_t>(row_ptr[m + 1], lo), nnz);
    // first entry with col >= kb (columns ascend within the row)
    int64_t a = lo, b = hi;
    while (a < b) {
        const int64_t mid = (a + b) >> 1;
        if (col[mid] < kb) a = mid + 1;
        else b = mid;
    }
    uint32_t word = 0;
    int n = 0;
    // at most EB (<= 32) entries fall in the lane's columns of a valid CSR
    for (int64_t j = a; j < hi && col[j] >= kb && col[j] < kb + g.eb && n < g.eb; ++j, ++n) {
        const int c = (int)(col[j] - kb), gi = c >> 2, p = c & 3;
        const int64_t grp = (kb >> 2) + gi;
        const uint32_t nib = (meta[m * ldm + (grp >> 1)] >> (4 * (grp & 1))) & 0xFu;
        const int i0 = (int)(nib & 3u), i1 = (int)(nib >> 2);
        // slot 0 is the lower complement position: p is slot 1 iff a lower
        // position is also not kept
        int below = 0;
        for (int x = 0; x < p; ++x) below += (x != i0 && x != i1);
        const uint32_t bit = 1u << (2 * gi + below);
        // an entry at a kept position, in a group with an invalid nibble, or
        // repeating a column (the CSR contract is strictly ascending columns)
        if (!nibble_valid(nib) || p == i0 || p == i1 || (word & bit)) {
            *badmask |= 1u << n;
            continue;
        }
        word |= bit;
    }
    *j0_out = a;
    *n_out = n;
    return word;
}

__global__ void __launch_bounds__(kCbmThreads) k_cbm_count(CbmGeom g, const uint8_t* meta, int64_t ldm,
                                                           const int32_t* row_ptr, const int32_t* col, int64_t nnz,
                                                           uint8_t* rmask, int32_t* roff, int32_t* bad) {
    const int lane = threadIdx.x & 63;
    const int64_t blocks = g.tiles * g.ksteps;
    const int mb = g.gl / 4;
    for (int64_t b = (int64_t)blockIdx.x * (kCbmThreads / 64) + (threadIdx.x >> 6); b < blocks;
         b += (int64_t)gridDim.x * (kCbmThreads / 64)) {
        const int64_t t = b / g.ksteps, s = b - t * g.ksteps;
        const int q = lane >> 4, r = lane & 15;
        const int64_t m = 16 * t + r, kb = s * g.ks + (int64_t)q * g.eb;
        int64_t j0;
        int n;
        uint32_t badm;
        const uint32_t word = lane_mask(g, meta, ldm, row_ptr, col, nnz, m, kb, &j0, &n, &badm);
        for (int y = 0; y < mb; ++y) rmask[(b * 64 + lane) * mb + y] = (uint8_t)(word >> (8 * y));
        int cnt = __popc(word);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d, 64);
        if (lane == 0) roff[b + 1] = cnt;
        if (bad != nullptr && badm != 0u) atomicAdd(bad, __popc(badm));
    }
}

template <int ES>
__global__ void __launch_bounds__(kCbmThreads) k_cbm_fill(CbmGeom g, const uint8_t* meta, int64_t ldm,
                                                          const int32_t* row_ptr, const int32_t* col, int64_t nnz,
                                                          const uint8_t* rvals, const int32_t* roff, uint8_t* cvals) {
    const int lane = threadIdx.x & 63;
    const int64_t blocks = g.tiles * g.ksteps;
    for (int64_t b = (int64_t)blockIdx.x * (kCbmThreads / 64) + (threadIdx.x >> 6); b < blocks;
         b += (int64_t)gridDim.x * (kCbmThreads / 64)) {
        const int64_t t = b / g.ksteps, s = b - t * g.ksteps;
        const int q = lane >> 4, r = lane & 15;
        const int64_t m = 16 * t + r, kb = s * g.ks + (int64_t)q * g.eb;
        int64_t j0;
        int n;
        uint32_t badm;
        const uint32_t word = lane_mask(g, meta, ldm, row_ptr, col, nnz, m, kb, &j0, &n, &badm);
        int64_t out = (int64_t)roff[b] + wave_excl_sum(__popc(word), lane);
        // the entries in column order are the mask bits in bit order
        for (int e = 0; e < n; ++e) {
            if (badm >> e & 1u) continue;
#pragma unroll
            for (int y = 0; y < ES; ++y) cvals[out * ES + y] = rvals[(j0 + e) * ES + y];
            ++out;
        }
    }
}

CbmGeom cbm_geom(int dt, int64_t M, int64_t K) {
    CbmGeom g;
    g.M = M;
    g.K = K;
    g.ks = dt_bytes(dt) == 1 ? 128 : 64;
    g.eb = g.ks / 4;
    g.gl = g.eb / 4;
    g.tiles = (M + 15) / 16;
    g.ksteps = K / g.ks;
    return g;
}

}  // namespace

void cbm_geometry(int dt, int64_t M, int64_t K, int64_t* blocks, int64_t* mask_bytes) {
    const CbmGeom g = cbm_geom(dt, M, K);
    *blocks = g.tiles * g.ksteps;
    *mask_bytes = *blocks * 64 * (g.gl / 4);
}

hipError_t launch_pack_cbm(int dt, int64_t M, int64_t K, const uint8_t* meta, int64_t ldm, const int32_t* row_ptr,
                           const int32_t* col, const void* rvals, int64_t nnz, void* rmask, int32_t* roff,
                           void* cvals, int32_t* bad, hipStream_t s) {
    const CbmGeom g = cbm_geom(dt, M, K);
    const int64_t blocks = g.tiles * g.ksteps;
    if (blocks > 0) {
        const unsigned grid = (unsigned)((blocks + 3) / 4 < 65536 ? (blocks + 3) / 4 : 65536);
        hipLaunchKernelGGL(k_cbm_count, dim3(grid), dim3(kCbmThreads), 0, s, g, meta, ldm, row_ptr, col, nnz,
                           (uint8_t*)rmask, roff, bad);
    }
    hipError_t e = launch_scan_counts(blocks, roff, s);
    if (e != hipSuccess || blocks == 0 || nnz == 0) return e;
    const unsigned grid = (unsigned)((blocks + 3) / 4 < 65536 ? (blocks + 3) / 4 : 65536);
    if (dt_bytes(dt) == 2)
        hipLaunchKernelGGL(k_cbm_fill<2>, dim3(grid), dim3(kCbmThreads), 0, s, g, meta, ldm, row_ptr, col, nnz,
                           (const uint8_t*)rvals, (const int32_t*)roff, (uint8_t*)cvals);
    else
        hipLaunchKernelGGL(k_cbm_fill<1>, dim3(grid), dim3(kCbmThreads), 0, s, g, meta, ldm, row_ptr, col, nnz,
                           (const uint8_t*)rvals, (const int32_t*)roff, (uint8_t*)cvals);
    return hipGetLastError();
}

}  // namespace ssg
