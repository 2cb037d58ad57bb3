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

// Element conversion to fp32 (bit-exact widening).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    _Float16 h;
    __builtin_memcpy(&h, &b, 2);
    return (float)h;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

template <int DT>
__device__ __forceinline__ float elem_to_f32(uint16_t b) {
    if constexpr (DT == DT_F16) return f16_bits_to_f32(b);
    else return bf16_bits_to_f32(b);
}

}  // namespace ssg
