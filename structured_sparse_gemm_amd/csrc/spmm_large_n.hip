// spmm_large_n.hip -- pipelined 2:4 SpMM for compute-bound shapes (prefill,
// large N) on gfx950's sparse MFMA.
//
// What it computes: C = expand(vals, meta) x B, each stored pair of a group
// meeting the two rows of B its 2-bit positions select ("Chapter 26 --
// Sparsity: The Hardware View", section "2:4 Fine-Grained Structured
// Sparsity"); in the compute-bound regime the doubled rate of the sparse
// matrix units is what pays (same chapter, sections "2:4: ~2x on the Matmul,
// Less End-to-End" and "2:4 in the Memory-Bound Regime").
//
// Mapping:
// * Workgroup tile 256 x 256, 4 waves (one per SIMD) in 2 x 2, each wave a
//   4 x 4 grid of 32 x 32 sparse MFMA tiles: v_smfmac_f32_32x32x32_{f16,bf16}
//   (32 dense k) or v_smfmac_i32_32x32x64_i8 (64 dense k); two of them per
//   k-block (BK = 64 dense k for 16-bit, 128 for int8).  The packed operand
//   with activation-major B runs 8 waves (two per SIMD) in 2 x 4, each a
//   4 x 2 grid: with one wave per SIMD every non-MFMA instruction of the
//   wave delays its next MFMA, and a second wave fills those gaps.
// * Every operand reaches LDS through direct-to-LDS buffer loads
//   (buffer_load ... lds): no register staging, and a row or column beyond
//   the matrix is an out-of-range buffer offset that reads as zero, so edge
//   tiles need no branches.  Three LDS stages; the loads of k-block i+2 are
//   issued right after the barrier that opens k-block i, and the wait before
//   that barrier counts only k-block i's loads.
// * Loads are shaped for the texture path, whose cost grows with the number
//   of distinct rows a quarter-wave touches: sparse values arrive 16 rows x
//   64 bytes per load (each row's stored values of the stage, 16-byte chunks
//   XOR-swizzled by row so the ds_read_b128 that builds a lane's operand --
//   row l%32, chunk 2s + l/32 -- is bank-conflict free); metadata arrives in
//   blocks of 32 bytes per row covering 4 (16-bit) or 2 (int8) stages, two
//   blocks resident, 8 rows per load.
// * B rows are stored unpadded with the 16-byte chunks of row r XOR-swizzled
//   (chunk c at slot c ^ 4*(r%4) for 16-bit, c ^ 2*(r%8) for int8); the
//   transposing reads (ds_read_b64_tr_b16 / _b8) that build the B operand
//   then hit 16 distinct 16-byte bank groups per 256 bytes.
// * Tiles are ordered so each XCD (workgroups are dealt round-robin to the 8
//   XCDs) gets a contiguous range of tiles, walked 8 row tiles at a time, so
//   the 32 tiles in flight on an XCD share their A and B panels in its L2.
// * Packed prefill operand (PK): the sparse values and metadata arrive
//   already in this kernel's LDS image, one contiguous 16 KiB block of values
//   per 256-row tile and stage (rows 64 bytes apart, chunks swizzled as
//   above) and one 8 KiB block of metadata per tile and metadata block.  Each
//   of their loads is then a contiguous 1 KiB / 256 B piece instead of 16 rows
//   x 64 bytes / 8 rows x 32 bytes, which halves the cache lines the load
//   path must track for the values and quarters them for the metadata.  The
//   metadata block is ordered in 16-byte lane chunks, so one LDS read gives
//   a lane the index words of its 4 row tiles for a whole stage (16-bit
//   types, two words per index register, picked by the MFMA's index-set
//   select) or a k-step (8-bit types), instead of one read per row tile and
//   k-step: the LDS issues reads at a fixed rate per instruction, and these
//   small reads cost as much of it as the operand reads.  The loads of a
//   stage are also spread over the reads and MFMAs of the next k-step
//   instead of being issued in one burst after the barrier.
#include <algorithm>

#include "ssg_device.hpp"
#include "ssg_kernels.hpp"

namespace ssg {

namespace {

constexpr int kBM = 256, kBN = 256, kStages = 3;
constexpr int kGroupM = 8;             // row tiles walked together per XCD
constexpr uint32_t kOob = 0x80000000u; // buffer offset that reads as zero

template <int DT> struct PT;
template <> struct PT<DT_F16> {
    static constexpr int ES = 2;       // element bytes
    static constexpr int KSUB = 32;    // dense k per MFMA
    static constexpr int BK = 64;      // dense k per stage
    static constexpr int MSTAGE = 8;   // metadata bytes per row per stage
    static constexpr int IDXB = 2;     // metadata bytes per lane per MFMA
    static constexpr int EPC = 8;      // elements per 16-byte chunk
    static constexpr int MB = 4;       // stages per 32-byte metadata block
};
template <> struct PT<DT_BF16> : PT<DT_F16> {};
template <> struct PT<DT_I8> {
    static constexpr int ES = 1;
    static constexpr int KSUB = 64;
    static constexpr int BK = 128;
    static constexpr int MSTAGE = 16;
    static constexpr int IDXB = 4;
    static constexpr int EPC = 16;
    static constexpr int MB = 2;
};
template <> struct PT<DT_E4M3> : PT<DT_I8> {};   // 8-bit floats: the int8 shapes
template <> struct PT<DT_E5M2> : PT<DT_I8> {};

// NW waves per workgroup: two along M (128 rows each), NW / 2 along N
template <int DT, int BN = kBN, int NW = 4>
struct Lay {
    using T = PT<DT>;
    static constexpr int WN = NW / 2;                      // waves along N
    static constexpr int NJ = BN / (32 * WN);              // 32-column MFMA tiles per wave
    static constexpr int ROWB = BN * T::ES;                // B tile row bytes
    static constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
    static constexpr int B_BYTES = T::BK * ROWB;           // 32 KiB
    static constexpr int A_ROWB = T::BK / 2 * T::ES;      // stored bytes per row per stage (64)
    static constexpr int A_BYTES = kBM * A_ROWB;           // 16 KiB
    static constexpr int STAGE = B_BYTES + A_BYTES;
    static constexpr int MBLK_ROWB = T::MB * T::MSTAGE;    // metadata bytes per row per block (32)
    static constexpr int MBLK = kBM * MBLK_ROWB;           // 8 KiB, two blocks resident
    static constexpr int LDS = kStages * STAGE + 2 * MBLK;
    static constexpr int B_LOADS = B_BYTES / 1024 / NW;    // per wave per stage (1 KiB each)
    static constexpr int A_LOADS = A_BYTES / 1024 / NW;
    static constexpr int M_LOADS = MBLK / 256 / NW;        // per wave per block (256 B each)
    static constexpr int VM_PER_STAGE = B_LOADS + A_LOADS;
    static_assert(A_ROWB == 64 && MBLK_ROWB == 32, "layout");
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert((NW == 4 || NW == 8) && NJ >= 1, "waves");
    static_assert(B_LOADS % NJ == 0 && B_LOADS >= 1 && A_LOADS >= 1 && A_LOADS <= 4 && M_LOADS >= 1,
                  "loads per wave per stage");
};

// Row-major operand: 16-byte chunk c of row r of the sparse-value tile sits
// at chunk c ^ swz_a(r) of the row's 64 bytes.  The permutation was chosen
// by measurement (the LDS read probe over every pair of row-bit parities):
// with it a sparse-operand read (32 rows, two chunks each) runs at the rate
// of a lane-contiguous read, where the XOR of row bits 1 and 3 ran at 0.6
// of it.  (The packed prefill operand instead arrives in the lane order of
// the reads, prefill_vals_unit, and each read is lane-contiguous.)
__device__ __forceinline__ int swz_a(int r) { return ((r >> 2) & 1) | (((r ^ (r >> 4)) & 1) << 1); }

template <int DT, int BN = kBN> __device__ __forceinline__ int swz(int r) {
    // a permutation of the row's 16-byte chunks (8-bit rows of 128 columns
    // have 8 of them)
    if constexpr (dt_bytes(DT) == 1) return BN == 256 ? 2 * (r & 7) : 2 * (r & 3);
    else return 4 * (r & 3);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int DT> using Acc16 = typename std::conditional<DT == DT_I8, i32x16, f32x16>::type;

// One sparse MFMA.  16-bit types take 16 index bits per lane: ABID selects
// the half of idx that holds them (the instruction's index-set select), so
// two MFMAs can share one register of two packed index words.
template <int DT, int ABID = 0>
__device__ __forceinline__ Acc16<DT> mma(uint4 a, const uint4 (&b)[2], Acc16<DT> c, uint32_t idx) {
    static_assert(ABID == 0 || dt_bytes(DT) == 2, "8-bit types use the whole index register");
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
        return __builtin_amdgcn_smfmac_f32_32x32x32_f16(av, bv, c, (int)idx, 0, ABID);
    } else {
        bf16x8 av;
        bf16x16 bv;
        __builtin_memcpy(&av, &a, 16);
        __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(av, bv, c, (int)idx, 0, ABID);
    }
}

// B operand (32 columns from tile column `cb`, MFMA k-step `s` of the stage)
// from the swizzled LDS tile.  Lane l: column cb + l%32, block bb = l/32;
// element e is dense k = (e / H) * (KSUB / 2) + H * bb + e % H within the
// k-step, H = 8 (16-bit) / 16 (int8).  Transposing reads act on 16-lane
// groups: source lane 4q+r (tr16) / 2q+r (tr8) names a row and 4 / 8
// consecutive columns; output lane i gets column i of 4 / 8 consecutive rows.
template <int DT, int BN>
__device__ __forceinline__ void b_frag(const uint8_t* bt, int s, int cb, int lane, uint4 (&b)[2]) {
    using L = Lay<DT, BN>;
    const int bb = lane >> 5, h = (lane >> 4) & 1, i = lane & 15;
    if constexpr (dt_bytes(DT) == 1) {
        const int q = i >> 1, r = i & 1;
        const int c = (cb >> 4) + h;                       // 16-byte chunk of the 16 columns
        i32x2 v[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = s * 64 + (p >> 1) * 32 + 16 * bb + (p & 1) * 8 + q;
            v[p] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2*)(bt + row * L::ROWB + ((c ^ swz<DT, BN>(row)) << 4) + 8 * r));
        }
        b[0] = make_uint4(v[0][0], v[0][1], v[1][0], v[1][1]);
        b[1] = make_uint4(v[2][0], v[2][1], v[3][0], v[3][1]);
    } else {
        const int q = i >> 2, r = i & 3;
        const int c = (cb >> 3) + 2 * h + (r >> 1);          // 16-byte chunk of the 4 columns
        uint2 w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int row = s * 32 + (p >> 1) * 16 + 8 * bb + (p & 1) * 4 + q;
            i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(bt + row * L::ROWB + ((c ^ swz<DT, BN>(row)) << 4) + 8 * (r & 1)));
            __builtin_memcpy(&w[p], &v, 8);
        }
        b[0] = make_uint4(w[0].x, w[0].y, w[1].x, w[1].y);
        b[1] = make_uint4(w[2].x, w[2].y, w[3].x, w[3].y);
    }
}

// Activation-major B (BT): the B operand given as its transpose Bt [N, K]
// row-major (one row of K per output column, as token-major activations
// arrive).  Its LDS tile holds BN rows of the stage's BK * ES = 128 bytes,
// the 8 16-byte chunks of row n XOR-swizzled by (n / 2) % 8, so the 16
// consecutive rows that a 16-byte read serves together hit 16 distinct
// 16-byte bank windows.  Lane l's B fragment (column cb + l%32, block
// bb = l/32) is then two plain 16-byte reads: chunks 4s + bb and 4s + 2 + bb
// of its row hold exactly its elements e < H and e >= H (dense k
// (e / H) * (KSUB / 2) + H * bb + e % H of k-step s, as in b_frag).
__device__ __forceinline__ int swz_bt(int n) { return (n >> 1) & 7; }

template <int DT>
__device__ __forceinline__ void b_frag_bt(const uint8_t* bt, int s, int cb, int lane, uint4 (&b)[2]) {
    const int bb = lane >> 5, n = cb + (lane & 31);
    const uint8_t* row = bt + n * 128;
    b[0] = *reinterpret_cast<const uint4*>(row + (((4 * s + bb) ^ swz_bt(n)) << 4));
    b[1] = *reinterpret_cast<const uint4*>(row + (((4 * s + 2 + bb) ^ swz_bt(n)) << 4));
}

struct Ctx {
    const uint8_t* vbase;   // vals row m0
    const uint8_t* mbase;   // meta row m0
    const uint8_t* bbase;   // B column n0
    int64_t vbytes, mbytes, bbytes;   // bytes from each base to the end of its buffer
    int64_t vstage, bstage;           // bytes per stage along K
    int64_t mstep;                    // bytes per metadata block along K
    uint32_t boff[8], aoff[4], moff[8];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int64_t remaining) {
    const int64_t n = remaining < 0 ? 0 : (remaining > 0x7fffffff ? 0x7fffffff : remaining);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)n, 0x00020000);
}

// One direct-to-LDS load: each lane's `BYTES` (4 or 16) from the buffer at
// byte offset `voff` land at LDS address m0 + lane * BYTES.  Issued as inline
// assembly so the compiler neither tracks these loads nor inserts its own
// conservative waits for them; the kernel counts them itself (wait_vm).  The
// s_nop is the wait state GFX9 needs between an SALU write of M0 and an
// LDS-DMA load that reads it.
template <int BYTES>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, uint32_t lds_dst, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
                     : "memory", "m0");
}

// s_waitcnt vmcnt(N): at most N of this wave's vector-memory operations are
// still outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that is also a compiler memory barrier; unlike
// __syncthreads it does not make the compiler drain the direct-to-LDS loads.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Scheduling pattern for a block of NM MFMAs and ND LDS reads: one MFMA,
// then one or two reads (two for the first ND - NM MFMAs), so the reads of
// the next k-step are spread over the current one's MFMAs instead of
// clustering in front of the first use.
template <int NM, int ND>
__device__ __forceinline__ void interleave() {
    if constexpr (NM > 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (ND > NM) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            interleave<NM - 1, ND - 2>();
        } else if constexpr (ND > 0) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            interleave<NM - 1, ND - 1>();
        } else {
            interleave<NM - 1, 0>();
        }
    }
}

// LDS reads of one k-step's operands: 4 sparse fragments, NJ x 4 transposing
// reads of B and 4 index words

// Issue the direct-to-LDS loads of stage `it` into `st` (this wave's share).
template <int DT, int BN, int NW>
__device__ __forceinline__ void issue(const Ctx& x, uint32_t st, int64_t it, int wave) {
    using L = Lay<DT, BN, NW>;
    using T = PT<DT>;
    const __amdgpu_buffer_rsrc_t rb = rsrc(x.bbase + it * x.bstage, x.bbytes - it * x.bstage);
    const __amdgpu_buffer_rsrc_t ra = rsrc(x.vbase + it * x.vstage, x.vbytes - it * x.vstage);
#pragma unroll
    for (int j = 0; j < L::B_LOADS; ++j) dma<16>(rb, st + (wave * L::B_LOADS + j) * 1024, x.boff[j]);
#pragma unroll
    for (int j = 0; j < L::A_LOADS; ++j) dma<16>(ra, st + L::B_BYTES + (wave * L::A_LOADS + j) * 1024, x.aoff[j]);
}

// Issue the direct-to-LDS loads of metadata block `g` (the 32 bytes of each
// of the tile's rows that cover stages [g * MB, (g + 1) * MB)) into `mt`.
template <int DT, int BN, int NW>
__device__ __forceinline__ void issue_meta(const Ctx& x, uint32_t mt, int64_t g, int wave) {
    using L = Lay<DT, BN, NW>;
    const __amdgpu_buffer_rsrc_t rm = rsrc(x.mbase + g * x.mstep, x.mbytes - g * x.mstep);
#pragma unroll
    for (int j = 0; j < L::M_LOADS; ++j) dma<4>(rm, mt + (wave * L::M_LOADS + j) * 256, x.moff[j]);
}

// Tile (tm, tn) of width BN (256, or 128 for the half-width tiles that fill
// the last wave of a launch): rows [256 tm, +256), columns [BN tn, +BN).
template <int DT, bool PK, int BN, bool BT, int NW>
__device__ __forceinline__ void spmm_tile(const SpmmArgs& a, int tm, int tn, uint8_t* lds) {
    using T = PT<DT>;
    using L = Lay<DT, BN, NW>;
    using Acc = Acc16<DT>;
    using S = typename std::conditional<DT == DT_I8, int32_t, float>::type;
    constexpr int NJ = L::NJ;
    uint8_t* const mlds = lds + kStages * L::STAGE;   // two metadata blocks
    // LDS byte addresses of the same, for the loads' M0 (32-bit arithmetic,
    // so no generic-pointer conversion per load)
    const uint32_t lds32 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void*)lds);
    const uint32_t mlds32 = lds32 + kStages * L::STAGE;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / L::WN, wn = wave % L::WN;     // rows [128 wm, +128), columns [32 NJ wn, +32 NJ)
    constexpr int WCOLS = 32 * NJ;
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * BN;

    // per-lane load offsets (constant across stages)
    const int64_t nit = a.K / T::BK;
    const int64_t nmb = (nit + T::MB - 1) / T::MB;       // metadata blocks along K
    Ctx x;
    if constexpr (PK) {
        // this tile's stage blocks of values and metadata blocks; a stage or
        // block past K is an empty range and reads zero
        x.vbase = reinterpret_cast<const uint8_t*>(a.vals) + tm * nit * L::A_BYTES;
        x.mbase = a.meta + tm * nmb * L::MBLK;
        x.vbytes = nit * L::A_BYTES;
        x.mbytes = nmb * L::MBLK;
        x.vstage = L::A_BYTES;
        x.mstep = L::MBLK;
    } else {
        x.vbase = reinterpret_cast<const uint8_t*>(a.vals) + m0 * a.ldv * T::ES;
        x.mbase = a.meta + m0 * a.ldm;
        x.vbytes = ((a.M - 1) * a.ldv + a.K / 2 - m0 * a.ldv) * T::ES;
        x.mbytes = (a.M - 1) * a.ldm + (a.K + 7) / 8 - m0 * a.ldm;
        x.vstage = L::A_ROWB;
        x.mstep = L::MBLK_ROWB;
    }
    if constexpr (BT) {
        // rows n0.. of Bt, advancing BK elements along them per stage; a
        // stage past K reads the next row's elements (or zeros past the
        // buffer) into a slot that is never multiplied
        x.bbase = reinterpret_cast<const uint8_t*>(a.B) + n0 * a.ldb * T::ES;
        x.bbytes = ((a.N - 1 - n0) * a.ldb + a.K) * T::ES;
        x.bstage = (int64_t)T::BK * T::ES;
    } else {
        x.bbase = reinterpret_cast<const uint8_t*>(a.B) + n0 * T::ES;
        x.bbytes = ((a.K - 1) * a.ldb + a.N - n0) * T::ES;
        x.bstage = (int64_t)T::BK * a.ldb * T::ES;
    }
#pragma unroll
    for (int j = 0; j < L::B_LOADS; ++j) {
        const int slot = (wave * L::B_LOADS + j) * 64 + lane;
        if constexpr (BT) {
            // 8 rows x 128 bytes per load: lane -> row slot / 8, LDS chunk slot % 8
            const int r = slot >> 3, c = (slot & 7) ^ swz_bt(r);
            x.boff[j] = (n0 + r < a.N) ? (uint32_t)(r * a.ldb * T::ES + 16 * c) : kOob;
        } else {
            const int r = slot / L::CPR, c = (slot % L::CPR) ^ swz<DT, BN>(r);
            x.boff[j] = (n0 + (int64_t)c * T::EPC < a.N) ? (uint32_t)((r * a.ldb + c * T::EPC) * T::ES) : kOob;
        }
    }
#pragma unroll
    for (int j = 0; j < L::A_LOADS; ++j) {
        // 16 rows x 64 bytes per load: lane -> row 16*ins + lane/4, LDS chunk lane%4
        const int row = 16 * (wave * L::A_LOADS + j) + (lane >> 2);
        const int c = (lane & 3) ^ swz_a(row);
        x.aoff[j] = (m0 + row < a.M) ? (uint32_t)(row * a.ldv * T::ES + 16 * c) : kOob;
        if constexpr (PK) x.aoff[j] = (uint32_t)((wave * L::A_LOADS + j) * 1024 + lane * 16);
    }
#pragma unroll
    for (int j = 0; j < L::M_LOADS; ++j) {
        // 8 rows x 32 bytes per load: lane -> row 8*ins + lane/8, dword lane%8
        const int row = 8 * (wave * L::M_LOADS + j) + (lane >> 3);
        x.moff[j] = (m0 + row < a.M) ? (uint32_t)(row * a.ldm + 4 * (lane & 7)) : kOob;
        if constexpr (PK) x.moff[j] = (uint32_t)((wave * L::M_LOADS + j) * 256 + lane * 4);
    }

    Acc acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = S(0);

    const int q = lane >> 5, rl = lane & 31;

    // Operands of one MFMA k-step (sub-step) from an LDS stage: 4 sparse
    // fragments of this wave's row tiles and NJ B fragments of its columns.
    struct Ops {
        uint4 av[4];
        uint4 b[NJ][2];
    };
    auto read_ops = [&](const uint8_t* st, int s, Ops& o) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 32 * (wm * 4 + i) + rl;
            if constexpr (PK)
                o.av[i] = *reinterpret_cast<const uint4*>(st + L::B_BYTES + (((wm * 4 + i) * 2 + s) << 10) + lane * 16);
            else
                o.av[i] = *reinterpret_cast<const uint4*>(st + L::B_BYTES + row * L::A_ROWB +
                                                          (((2 * s + q) ^ swz_a(row)) << 4));
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if constexpr (BT) b_frag_bt<DT>(st, s, wn * WCOLS + 32 * j, lane, o.b[j]);
            else b_frag<DT, BN>(st, s, wn * WCOLS + 32 * j, lane, o.b[j]);
        }
    };
    // Index words of sub-step s of stage t for this lane, read so that no
    // per-lane selection follows the read.  Row-major metadata: 16-bit -- the
    // 16 bits at byte 4s + 2q of the row's 8 (a zero-extending u16 read);
    // int8 -- dword 2s + q of the row's 16; stage t's bytes are at
    // (t % MB) * MSTAGE of each row of metadata block t / MB.  Packed: the
    // lane's 16-byte chunk of the block holds the words of its 4 row tiles
    // for KPC k-steps (both of a stage for 16-bit types, whose MFMAs then
    // take them two per register, one for 8-bit ones).
    auto read_idx = [&](int64_t t, int s, uint32_t (&ix)[4]) {
        const uint8_t* mt = mlds + ((t / T::MB) & 1) * L::MBLK + (t % T::MB) * T::MSTAGE + s * (T::MSTAGE / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint8_t* mp = mt + (32 * (wm * 4 + i) + rl) * L::MBLK_ROWB + q * T::IDXB;
            if constexpr (T::IDXB == 4) ix[i] = *reinterpret_cast<const uint32_t*>(mp);
            else ix[i] = *reinterpret_cast<const uint16_t*>(mp);
        }
    };
    constexpr int KPC = 4 / T::IDXB;                    // k-steps per packed index chunk
    auto read_idx_pk = [&](int64_t t, int s) -> uint4 {
        const uint8_t* mb = mlds + ((t / T::MB) & 1) * L::MBLK;
        const int h = (int)(t % T::MB) * 2 + s;          // k-step of the block
        return *reinterpret_cast<const uint4*>(mb + (((h / KPC) * 2 + wm) * 64 + lane) * 16);
    };
    // ix[i]: the index register of row tile i; with HALVES (16-bit types,
    // packed) row tile i's word is half i % 2 of it
    auto mmas = [&](const Ops& o, const uint32_t (&ix)[4], auto halves) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                acc[i][j] = mma<DT>(o.av[i], o.b[j], acc[i][j], ix[i]);
                acc[i + 1][j] = mma<DT, decltype(halves)::value ? 1 : 0>(o.av[i + 1], o.b[j], acc[i + 1][j], ix[i + 1]);
            }
    };

    // Pipeline: DMA stages run two ahead of the stage being multiplied; the
    // LDS reads of the next sub-step are in flight while the current one's
    // MFMAs execute.  The loop has no branches: a stage past the end of K is
    // a load with an empty buffer range, which writes zeros to a slot that is
    // never multiplied.
    //
    // Metadata comes in blocks of MB stages, two resident: block g is issued
    // right after the A/B loads of stage (g - 1) * MB + 2 (the iteration
    // after every wave's last read of block g - 2, whose buffer it takes) and
    // is first read MB - 1 iterations later.  The wait of an iteration that
    // follows such an issue leaves the block's loads outstanding too.
    issue_meta<DT, BN, NW>(x, mlds32, 0, wave);
    issue<DT, BN, NW>(x, lds32, 0, wave);
    issue<DT, BN, NW>(x, lds32 + L::STAGE, 1, wave);
    wait_vm<L::VM_PER_STAGE>();
    barrier();
    issue<DT, BN, NW>(x, lds32 + 2 * L::STAGE, 2, wave);
    issue_meta<DT, BN, NW>(x, mlds32 + L::MBLK, 1, wave);

    // Index words: packed 16-bit -- one chunk per stage (dn: both k-steps'
    // words, two per register); packed 8-bit -- one chunk per k-step;
    // row-major -- one read per row tile and k-step.
    constexpr bool PK16 = PK && T::IDXB == 2;
    constexpr int NIX0 = PK16 ? 0 : PK ? 1 : 4, NIX1 = PK ? 1 : 4;   // index reads per half-iteration
    constexpr int NB = BT ? 2 : 4;                                     // B reads per fragment
    using Halves = std::integral_constant<bool, PK16>;
    auto load_ix = [&](int64_t t, int s, uint32_t (&ix)[4]) {
        if constexpr (PK) {
            const uint4 d = read_idx_pk(t, s);
            ix[0] = d.x; ix[1] = d.y; ix[2] = d.z; ix[3] = d.w;
        } else {
            read_idx(t, s, ix);
        }
    };
    Ops o0, o1;
    uint32_t ix0[4], ix1[4];
    uint4 dn = make_uint4(0, 0, 0, 0);
    if constexpr (PK16) dn = read_idx_pk(0, 0);
    else load_ix(0, 0, ix0);
    read_ops(lds, 0, o0);
    int slot = 0;
    for (int64_t it = 0; it < nit; ++it) {
        const uint8_t* st = lds + slot * L::STAGE;
        read_ops(st, 1, o1);
        if constexpr (PK16) {
            ix0[0] = dn.x; ix0[1] = dn.x; ix0[2] = dn.y; ix0[3] = dn.y;
            ix1[0] = dn.z; ix1[1] = dn.z; ix1[2] = dn.w; ix1[3] = dn.w;
        } else {
            load_ix(it, 1, ix1);
        }
        mmas(o0, ix0, Halves{});
        interleave<4 * NJ, 4 + NB * NJ + NIX0>();
        // stage it+1 has landed once only stage it+2's loads remain; this
        // wave's reads of stage it are done (s_waitcnt lgkmcnt(0), through the
        // builtin so the compiler knows they have landed) before the barrier
        // lets stage it+3's loads overwrite its slot
        if (it % T::MB == 0) wait_vm<L::VM_PER_STAGE + L::M_LOADS>();
        else wait_vm<L::VM_PER_STAGE>();
        __builtin_amdgcn_s_waitcnt(0xC07F);
        barrier();
        const uint32_t dst = lds32 + slot * L::STAGE;
        if constexpr (!PK) issue<DT, BN, NW>(x, dst, it + 3, wave);
        if ((it + 1) % T::MB == 0)
            issue_meta<DT, BN, NW>(x, mlds32 + (((it + 1) / T::MB + 1) & 1) * L::MBLK, (it + 1) / T::MB + 1, wave);
        slot = slot == kStages - 1 ? 0 : slot + 1;
        const uint8_t* nx = lds + slot * L::STAGE;
        if constexpr (PK) {
            // the same loads as issue(), each placed after one of the reads
            // of the next k-step so they leave the wave between its MFMAs
            const __amdgpu_buffer_rsrc_t rb = rsrc(x.bbase + (it + 3) * x.bstage, x.bbytes - (it + 3) * x.bstage);
            const __amdgpu_buffer_rsrc_t ra = rsrc(x.vbase + (it + 3) * x.vstage, x.vbytes - (it + 3) * x.vstage);
            // the A_LOADS (at most 4) loads of values follow the first reads
            constexpr int BPJ = L::B_LOADS / NJ;        // B loads placed after each column tile's reads
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o0.av[i] = *reinterpret_cast<const uint4*>(nx + L::B_BYTES + ((wm * 4 + i) << 11) + lane * 16);
                if (i < L::A_LOADS) dma<16>(ra, dst + L::B_BYTES + (wave * L::A_LOADS + i) * 1024, x.aoff[i]);
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if constexpr (BT) b_frag_bt<DT>(nx, 0, wn * WCOLS + 32 * j, lane, o0.b[j]);
                else b_frag<DT, BN>(nx, 0, wn * WCOLS + 32 * j, lane, o0.b[j]);
#pragma unroll
                for (int u = 0; u < BPJ; ++u)
                    dma<16>(rb, dst + (wave * L::B_LOADS + BPJ * j + u) * 1024, x.boff[BPJ * j + u]);
            }
        } else {
            read_ops(nx, 0, o0);
        }
        if constexpr (PK16) dn = read_idx_pk(it + 1, 0);
        else load_ix(it + 1, 0, ix0);
        mmas(o1, ix1, Halves{});
        interleave<4 * NJ, 4 + NB * NJ + NIX1>();
    }
    // the zero-filling loads of the stages past K land before the LDS is released
    wait_vm<0>();

    // epilogue: D element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32.
    // C is written once and not read back here: non-temporal stores keep it
    // from displacing the operand panels the other tiles still stream.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int64_t col = n0 + wn * WCOLS + 32 * j + rl;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * q + (e & 3);
                if (row < a.M && col < a.N)
                    __builtin_nontemporal_store((S)acc[i][j][e], reinterpret_cast<S*>(a.C) + row * a.ldc + col);
            }
        }
    }
}

// One launch: tiles of full width for row tiles [0, full_rows), and two
// half-width tiles per tile for row tiles [full_rows, tiles_m), dispatched
// after the full ones.  When the tiles of a launch leave the last wave of
// workgroups at most half full, its tiles are cut in half so that the last
// wave is full of half-length work instead of half empty.  An output's k
// order is the same in both widths, so the result is the same bits.  Within
// each part the order is XCD-aware: workgroups are dealt round-robin to the
// 8 XCDs, and each XCD gets a contiguous range of tiles, walked kGroupM row
// tiles at a time, so the tiles in flight on an XCD share their A and B
// panels in its L2.
__device__ __forceinline__ void xcd_order(int bid, int tiles_m, int tiles_n, int* tm, int* tn) {
    const int tiles = tiles_m * tiles_n;
    const int per_xcd = tiles / 8;
    if (bid < per_xcd * 8) bid = (bid & 7) * per_xcd + (bid >> 3);
    const int group = bid / (kGroupM * tiles_n);
    const int first_m = group * kGroupM;
    const int gm = min(kGroupM, tiles_m - first_m);
    const int in_group = bid - group * kGroupM * tiles_n;
    *tm = first_m + in_group % gm;
    *tn = in_group / gm;
}

template <int DT, bool PK, bool BT = false, int NW = 4>
__global__ void __launch_bounds__(NW * 64) k_spmm_pipe(SpmmArgs a, int tiles_m, int tiles_n, int full_rows) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[Lay<DT>::LDS];
    const int nfull = full_rows * tiles_n;
    int tm, tn;
    if ((int)blockIdx.x < nfull) {
        xcd_order(blockIdx.x, full_rows, tiles_n, &tm, &tn);
        spmm_tile<DT, PK, kBN, BT, NW>(a, tm, tn, lds);
    } else {
        xcd_order(blockIdx.x - nfull, tiles_m - full_rows, 2 * tiles_n, &tm, &tn);
        spmm_tile<DT, PK, kBN / 2, BT, NW>(a, full_rows + tm, tn, lds);
    }
}

template <int DT>
bool pipe_supported(const SpmmArgs& a) {
    using T = PT<DT>;
    const uintptr_t v = reinterpret_cast<uintptr_t>(a.vals), m = reinterpret_cast<uintptr_t>(a.meta),
                    b = reinterpret_cast<uintptr_t>(a.B);
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    return a.M > 0 && a.N > 0 && a.K > 0 && a.K % T::BK == 0 && a.N % T::EPC == 0 &&
           v % 16 == 0 && (a.ldv * T::ES) % 16 == 0 && b % 16 == 0 && (a.ldb * T::ES) % 16 == 0 &&
           m % 4 == 0 && a.ldm % 4 == 0 &&
           // every buffer addressed with 31-bit offsets
           ((a.M - 1) * a.ldv + a.K / 2) * T::ES < 0x7fffffff && (a.M - 1) * a.ldm + a.K / 8 < 0x7fffffff &&
           ((a.K - 1) * a.ldb + a.N) * T::ES < 0x7fffffff && tiles < 0x7fffffff;
}

// Row tiles that run at full width: all of them, unless the launch's last
// wave of workgroups (256 CUs) would be at most half full -- then enough of
// the last row tiles run as half-width tiles to fill it with half-length
// work (the converted tiles number between the remainder and 256 minus it,
// so the launch needs no more waves than before).
int full_row_tiles(int tiles_m, int tiles_n) {
    constexpr int kCUs = 256;
    const int tiles = tiles_m * tiles_n, rem = tiles % kCUs;
    if (rem == 0) return tiles_m;
    const int half_rows = (rem + tiles_n - 1) / tiles_n, conv = half_rows * tiles_n;
    return conv <= kCUs - rem ? tiles_m - half_rows : tiles_m;
}

template <int DT, bool PK = false, bool BT = false, int NW = 4>
hipError_t pipe_launch(const SpmmArgs& a, hipStream_t s) {
    const int tm = (int)((a.M + kBM - 1) / kBM), tn = (int)((a.N + kBN - 1) / kBN);
    const int full = full_row_tiles(tm, tn);
    const unsigned grid = (unsigned)(full * tn + 2 * (tm - full) * tn);
    hipLaunchKernelGGL((k_spmm_pipe<DT, PK, BT, NW>), dim3(grid), dim3(NW * 64), 0, s, a, tm, tn, full);
    return hipGetLastError();
}

// Row-major (vals, meta) -> packed prefill layout.  One thread per 16-byte
// chunk of pvals (a copy of one 16-byte chunk of a vals row, or zeros past
// M) and per 4 bytes of pmeta (gathered bytewise from the lane-chunk
// positions: meta rows need no alignment; zeros past M and past K / 8).
__global__ void __launch_bounds__(256) k_pack_prefill(int64_t M, int64_t K, const uint8_t* vals, int64_t ldv_bytes,
                                                      const uint8_t* meta, int64_t ldm, int64_t stages, int64_t mblocks,
                                                      int64_t vchunks, int64_t mwords, int iw, uint8_t* pvals,
                                                      uint8_t* pmeta) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < vchunks + mwords; i += stride) {
        if (i < vchunks) {
            // 16-byte unit u of block (t, s): chunk c of the stage's bytes of row r
            const int64_t blk = i >> 10, t = blk / stages, st = blk - t * stages;
            int r, c;
            prefill_vals_unit_inv((int)(i & 1023), &r, &c);
            const int64_t m = t * 256 + r;
            uint4 w = make_uint4(0, 0, 0, 0);
            if (m < M) w = *reinterpret_cast<const uint4*>(vals + m * ldv_bytes + st * 64 + (c << 4));
            *reinterpret_cast<uint4*>(pvals + (i << 4)) = w;
        } else {
            const int64_t k = i - vchunks;     // 4-byte word k of pmeta
            const int64_t blk = k >> 11, t = blk / mblocks, g = blk - t * mblocks;
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // byte o of the block: metadata byte j of row r of the block
                int r, j;
                prefill_meta_inv((int)((k & 2047) * 4 + e), iw, &r, &j);
                const int64_t m = t * 256 + r;
                if (m < M && g * 32 + j < K / 8) w |= (uint32_t)meta[m * ldm + g * 32 + j] << (8 * e);
            }
            *reinterpret_cast<uint32_t*>(pmeta + (k << 2)) = w;
        }
    }
}

bool pipe_ok(const SpmmArgs& a) {
    switch (a.dt) {
        case DT_F16: return pipe_supported<DT_F16>(a);
        case DT_BF16: return pipe_supported<DT_BF16>(a);
        case DT_I8: return pipe_supported<DT_I8>(a);
        case DT_E4M3: return pipe_supported<DT_E4M3>(a);
        case DT_E5M2: return pipe_supported<DT_E5M2>(a);
        default: return false;
    }
}

}  // namespace

void prefill_geometry(int dt, int64_t M, int64_t K, int64_t* tiles, int64_t* stages, int64_t* mblocks) {
    *tiles = (M + kBM - 1) / kBM;
    *stages = K / 2 * dt_bytes(dt) / 64;
    *mblocks = (K + 255) / 256;
}

hipError_t launch_pack_prefill(int dt, int64_t M, int64_t K, const void* vals, int64_t ldv, const uint8_t* meta,
                               int64_t ldm, void* pvals, void* pmeta, hipStream_t s) {
    int64_t tiles, stages, mblocks;
    prefill_geometry(dt, M, K, &tiles, &stages, &mblocks);
    const int64_t vchunks = tiles * stages * 1024, mwords = tiles * mblocks * 2048;
    if (vchunks + mwords == 0) return hipSuccess;
    const int64_t grid = std::min<int64_t>((vchunks + mwords + 255) / 256, 8192);
    hipLaunchKernelGGL(k_pack_prefill, dim3((unsigned)grid), dim3(256), 0, s, M, K, (const uint8_t*)vals,
                       ldv * dt_bytes(dt), meta, ldm, stages, mblocks, vchunks, mwords, dt_bytes(dt) == 1 ? 4 : 2,
                       (uint8_t*)pvals, (uint8_t*)pmeta);
    return hipGetLastError();
}

bool supported_prefill_packed(const SpmmArgs& a) {
    const int es = dt_bytes(a.dt), bk = es == 1 ? 128 : 64, epc = 16 / es;
    const uintptr_t v = reinterpret_cast<uintptr_t>(a.vals), m = reinterpret_cast<uintptr_t>(a.meta),
                    b = reinterpret_cast<uintptr_t>(a.B);
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    return a.M > 0 && a.N > 0 && a.K > 0 && a.K % bk == 0 && a.N % epc == 0 && v % 16 == 0 && m % 4 == 0 &&
           b % 16 == 0 && (a.ldb * es) % 16 == 0 &&
           // one tile's blocks and all of B addressed with 31-bit offsets
           a.K / 2 * es * 256 < 0x7fffffff && ((a.K - 1) * a.ldb + a.N) * es < 0x7fffffff && tiles < 0x7fffffff;
}

hipError_t launch_spmm_prefill_packed(const SpmmArgs& a, hipStream_t s) {
    switch (a.dt) {
        case DT_F16: return pipe_launch<DT_F16, true>(a, s);
        case DT_BF16: return pipe_launch<DT_BF16, true>(a, s);
        case DT_I8: return pipe_launch<DT_I8, true>(a, s);
        case DT_E4M3: return pipe_launch<DT_E4M3, true>(a, s);
        case DT_E5M2: return pipe_launch<DT_E5M2, true>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// Activation-major B: a.B is Bt [N, K] row-major with row stride a.ldb.
bool supported_prefill_packed_bt(const SpmmArgs& a) {
    const int es = dt_bytes(a.dt), bk = es == 1 ? 128 : 64;
    const uintptr_t v = reinterpret_cast<uintptr_t>(a.vals), m = reinterpret_cast<uintptr_t>(a.meta),
                    b = reinterpret_cast<uintptr_t>(a.B);
    const int64_t tiles = ((a.M + kBM - 1) / kBM) * ((a.N + kBN - 1) / kBN);
    return a.M > 0 && a.N > 0 && a.K > 0 && a.K % bk == 0 && a.ldb >= a.K && v % 16 == 0 && m % 4 == 0 &&
           b % 16 == 0 && (a.ldb * es) % 16 == 0 &&
           // one tile's blocks, and a tile's 256 rows of Bt, addressed with 31-bit offsets
           a.K / 2 * es * 256 < 0x7fffffff && 256 * a.ldb * es < 0x7fffffff && tiles < 0x7fffffff;
}

hipError_t launch_spmm_prefill_packed_bt(const SpmmArgs& a, hipStream_t s) {
    switch (a.dt) {
        case DT_F16: return pipe_launch<DT_F16, true, true, 8>(a, s);
        case DT_BF16: return pipe_launch<DT_BF16, true, true, 8>(a, s);
        case DT_I8: return pipe_launch<DT_I8, true, true, 8>(a, s);
        case DT_E4M3: return pipe_launch<DT_E4M3, true, true, 8>(a, s);
        case DT_E5M2: return pipe_launch<DT_E5M2, true, true, 8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

bool supported_large_n(const SpmmArgs& a) { return pipe_ok(a) || supported_large_n_basic(a); }

hipError_t launch_spmm_large_n(const SpmmArgs& a, hipStream_t s) {
    if (!pipe_ok(a)) return launch_spmm_large_n_basic(a, s);
    switch (a.dt) {
        case DT_F16: return pipe_launch<DT_F16>(a, s);
        case DT_BF16: return pipe_launch<DT_BF16>(a, s);
        case DT_I8: return pipe_launch<DT_I8>(a, s);
        case DT_E4M3: return pipe_launch<DT_E4M3>(a, s);
        case DT_E5M2: return pipe_launch<DT_E5M2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ssg
