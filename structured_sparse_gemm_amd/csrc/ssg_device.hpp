// ssg_device.hpp -- device-side building blocks shared by the HIP kernels of
// libssgemm: element traits, the 2:4 selection rule on integer magnitude
// keys, vector types for the gfx950 sparse/dense MFMA builtins.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssg_kernels.hpp"

namespace ssg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Magnitude keys.  For finite IEEE binary16 and bfloat16 values the bit
// pattern with the sign cleared orders exactly like |x| (sign-magnitude
// encoding with a monotone exponent/fraction field), and -0 maps to the same
// key as +0.  For int8 the key is |x| as an integer, so -128 -> 128.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t mag_key16(uint32_t bits) { return bits & 0x7FFFu; }
__device__ __forceinline__ uint32_t mag_key8(int32_t v) { return (uint32_t)(v < 0 ? -v : v); }
// 8-bit floats are sign-magnitude too: the 7 low bits order like |x|.
__device__ __forceinline__ uint32_t mag_key_fp8(uint32_t bits) { return bits & 0x7Fu; }

// The two kept positions of a group as a nibble i0 | (i1 << 2), i0 < i1.
// Position p is kept iff fewer than two others outrank it; q outranks p when
// key_q > key_p, or key_q == key_p and q < p (ties go to the lower position).
// With b_pq = (key_p >= key_q) for p < q ("p wins against q"):
//   rank0 = !b01 + !b02 + !b03      rank1 = b01 + !b12 + !b13
//   rank2 = b02 + b12 + !b23        rank3 = b03 + b13 + b23
__device__ __forceinline__ uint32_t select_nibble(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
    const uint32_t b01 = k0 >= k1, b02 = k0 >= k2, b03 = k0 >= k3;
    const uint32_t b12 = k1 >= k2, b13 = k1 >= k3, b23 = k2 >= k3;
    const uint32_t r0 = 3u - b01 - b02 - b03;
    const uint32_t r1 = b01 + 2u - b12 - b13;
    const uint32_t r2 = b02 + b12 + 1u - b23;
    const uint32_t r3 = b03 + b13 + b23;
    const uint32_t keep = (uint32_t)(r0 < 2) | ((uint32_t)(r1 < 2) << 1) | ((uint32_t)(r2 < 2) << 2) |
                          ((uint32_t)(r3 < 2) << 3);
    // keep mask (exactly two bits) -> nibble: 0011->0x4 0101->0x8 0110->0x9
    // 1001->0xC 1010->0xD 1100->0xE
    constexpr uint64_t kTable = (0x4ull << (4 * 3)) | (0x8ull << (4 * 5)) | (0x9ull << (4 * 6)) |
                                (0xCull << (4 * 9)) | (0xDull << (4 * 10)) | (0xEull << (4 * 12));
    return (uint32_t)(kTable >> (4 * keep)) & 0xFu;
}

__device__ __forceinline__ bool nibble_valid(uint32_t nib) { return (nib & 3u) < (nib >> 2); }

// ---------------------------------------------------------------------------
// Packed prefill layout of a 2:4 operand: the large-N kernel's LDS image of
// each 256-row tile, so that kernel loads it in contiguous pieces.  In bytes
// it is the same for every element type: a stage is 64 stored-value bytes of
// every row (64 dense k for fp16/bf16, 128 for 8-bit types) and a metadata
// block 32 metadata bytes of every row (256 dense k).
// * pvals: tile t, stage s -> 16 KiB block (t * stages + s) of 16-byte lane
//   chunks in the order of the kernel's sparse-operand reads: 1 KiB piece
//   (32-row group rt, MFMA k-step s2 of the stage) holds, at lane
//   position 32 q + rl, 16-byte chunk 2 s2 + q of the stage's 64 bytes of
//   row 32 rt + rl (prefill_vals_unit).  One lane-contiguous 16-byte read
//   then gives every lane of a wave its sparse operand.
// * pmeta: tile t, block g -> 8 KiB block (t * mblocks + g) of 16-byte lane
//   chunks, one per (MFMA k-step group, 128-row half, lane) of the kernel:
//   chunk u = (hq * 2 + wm) * 64 + 32 q + rl holds the index words of rows
//   128 wm + 32 i + rl (i = 0..3) for lane half q of k-steps hq * KPC + hs
//   (hs < KPC), word (hs, i) at bytes ((hs * 4 + i) * IW, + IW).  IW = index-
//   word bytes (2 for 16-bit types, 4 for 8-bit), KPC = 4 / IW k-steps per
//   chunk; k-step h of the block is metadata bytes [2 IW h, 2 IW (h + 1)) of
//   each row, lane half q its bytes [2 IW h + q IW, + IW).  One 16-byte LDS
//   read then gives a lane every index word of its 4 row tiles for KPC
//   k-steps.
// Rows past M and metadata bytes past K / 8 hold zeros.
// ---------------------------------------------------------------------------
// 16-byte unit of a pvals stage block that holds chunk c (0..3) of the
// stage's 64 bytes of tile row r (0..255), and the inverse.
__host__ __device__ __forceinline__ int prefill_vals_unit(int r, int c) {
    return ((((r >> 5) << 1) + (c >> 1)) << 6) + ((c & 1) << 5) + (r & 31);
}
__host__ __device__ __forceinline__ void prefill_vals_unit_inv(int u, int* r, int* c) {
    *r = ((u >> 7) << 5) + (u & 31);
    *c = (((u >> 6) & 1) << 1) + ((u >> 5) & 1);
}

// Position in its 8 KiB metadata block of byte j (0..31) of row r (0..255)
// of the block, and the inverse.
__host__ __device__ __forceinline__ int prefill_meta_pos(int r, int j, int iw) {
    const int kpc = 4 / iw, h = j / (2 * iw), q = (j / iw) & 1, e = j % iw;
    const int wm = r >> 7, i = (r >> 5) & 3, rl = r & 31;
    return (((h / kpc) * 2 + wm) * 64 + 32 * q + rl) * 16 + ((h % kpc) * 4 + i) * iw + e;
}
__host__ __device__ __forceinline__ void prefill_meta_inv(int o, int iw, int* r, int* j) {
    const int kpc = 4 / iw, u = o >> 4, b = o & 15;
    const int wm = (u >> 6) & 1, hq = u >> 7, q = (u >> 5) & 1, rl = u & 31;
    const int wi = b / iw, hs = wi >> 2, i = wi & 3, e = b % iw;
    *r = 128 * wm + 32 * i + rl;
    *j = (hq * kpc + hs) * 2 * iw + q * iw + e;
}

// Element conversion to fp32 (bit-exact widening).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return (float)h;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// 8-bit floats, exact: E4M3 (bias 7, S.1111.111 = NaN, no infinities) and
// E5M2 (bias 15, IEEE-style infinities and NaNs), from their bit fields.
__device__ __forceinline__ float e4m3_bits_to_f32(uint32_t b) {
    const uint32_t s = (b & 0x80u) << 24, e = (b >> 3) & 0xFu, m = b & 7u;
    if (e == 0xFu && m == 7u) return __uint_as_float(s | 0x7FC00000u);
    if (e == 0u) return __uint_as_float(s | __float_as_uint((float)m * 0.001953125f));   // m * 2^-9
    return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}
__device__ __forceinline__ float e5m2_bits_to_f32(uint32_t b) {
    const uint32_t s = (b & 0x80u) << 24, e = (b >> 2) & 0x1Fu, m = b & 3u;
    if (e == 0x1Fu) return __uint_as_float(s | (m ? 0x7FC00000u : 0x7F800000u));
    if (e == 0u) return __uint_as_float(s | __float_as_uint((float)m * 1.52587890625e-05f));   // m * 2^-16
    return __uint_as_float(s | ((e + 112u) << 23) | (m << 21));
}

// Element bits (the low 16 or 8 bits of b) to fp32 for the float types.
template <int DT>
__device__ __forceinline__ float elem_to_f32(uint32_t b) {
    if constexpr (DT == DT_F16) return f16_bits_to_f32((uint16_t)b);
    else if constexpr (DT == DT_BF16) return bf16_bits_to_f32((uint16_t)b);
    else if constexpr (DT == DT_E4M3) return e4m3_bits_to_f32(b & 0xFFu);
    else return e5m2_bits_to_f32(b & 0xFFu);
}

}  // namespace ssg
