// probe.hip -- measured ceilings the products are compared against.
//
// A plain streaming read of device memory, the ceiling of the
// bandwidth-bound products.  It reads every byte of a buffer once, in
// contiguous 16-byte pieces per lane (1 KiB per wave per load), with several
// loads in flight per lane, and does nothing with the data but fold it into
// one word per workgroup (stored only if the fold hits a value chosen so that
// it practically never does, which keeps the loads alive).  Same grid shape
// rules as the products: many more workgroups than CUs, and non-temporal
// loads, as the decode products use for their weights.
//
// The issue rate of one matrix-core instruction form, sparse or dense, the
// ceiling of the compute-bound products and the measure for choosing between
// the sparse MFMA and a decode to dense operands followed by the dense MFMA.
// Every wave runs a chain of independent accumulators through the one
// instruction with operands from a hash of its lane (bf16 values in
// [2^-63, 2), int8 bytes uniform, fp8 bytes uniform over the finite
// E4M3 values of magnitude at most 240, valid 2:4 index nibbles), so
// the instruction stream is nothing but that form.
//
// The rate of 16-byte LDS reads (ds_read_b128) for one pattern of per-lane
// addresses, the measure behind the LDS images of the large-N kernel.
// Every wave repeats eight reads of its lanes' addresses, 4 KiB apart, and
// folds the data into a word as the other probes do.
#include <algorithm>

#include "ssg_device.hpp"
#include "ssg_kernels.hpp"

namespace ssg {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 4;

__global__ void __launch_bounds__(kProbeThreads) k_stream_read(const i32x4* __restrict__ src, int64_t n16,
                                                              uint32_t* sink) {
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        i32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) x ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
    }
    for (; i < n16; i += stride) {
        const i32x4 v = __builtin_nontemporal_load(src + i);
        x ^= (uint32_t)(v.x ^ v.y ^ v.z ^ v.w);
    }
    if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

constexpr int kMfmaThreads = 256;                  // one wave per SIMD of a CU

__device__ __forceinline__ uint32_t lane_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    return x ^ (x >> 16);
}

// One instruction of form F on accumulator c; a holds 8 words, b 8 words.
template <int F> struct MfmaForm;
template <> struct MfmaForm<0> {                     // sparse bf16, 32 x 32, 32 dense k
    using Acc = f32x16;
    static constexpr int NACC = 8;
    static __device__ Acc op(const int* a, const int* b, Acc c, int idx) {
        bf16x8 av; bf16x16 bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(av, bv, c, idx, 0, 0);
    }
};
template <> struct MfmaForm<1> {                     // dense bf16, 32 x 32 x 16
    using Acc = f32x16;
    static constexpr int NACC = 8;
    static __device__ Acc op(const int* a, const int* b, Acc c, int) {
        bf16x8 av, bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
    }
};
template <> struct MfmaForm<2> {                     // sparse bf16, 16 x 16, 64 dense k
    using Acc = f32x4;
    static constexpr int NACC = 16;
    static __device__ Acc op(const int* a, const int* b, Acc c, int idx) {
        bf16x8 av; bf16x16 bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(av, bv, c, idx, 0, 0);
    }
};
template <> struct MfmaForm<3> {                     // dense bf16, 16 x 16 x 32
    using Acc = f32x4;
    static constexpr int NACC = 16;
    static __device__ Acc op(const int* a, const int* b, Acc c, int) {
        bf16x8 av, bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
    }
};
template <> struct MfmaForm<4> {                     // sparse int8, 32 x 32, 64 dense k
    using Acc = i32x16;
    static constexpr int NACC = 8;
    static __device__ Acc op(const int* a, const int* b, Acc c, int idx) {
        i32x4 av; i32x8 bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_i32_32x32x64_i8(av, bv, c, idx, 0, 0);
    }
};
template <> struct MfmaForm<5> {                     // dense int8, 32 x 32 x 32
    using Acc = i32x16;
    static constexpr int NACC = 8;
    static __device__ Acc op(const int* a, const int* b, Acc c, int) {
        i32x4 av, bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, c, 0, 0, 0);
    }
};
template <> struct MfmaForm<6> {                     // sparse int8, 16 x 16, 128 dense k
    using Acc = i32x4;
    static constexpr int NACC = 16;
    static __device__ Acc op(const int* a, const int* b, Acc c, int idx) {
        i32x4 av; i32x8 bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_i32_16x16x128_i8(av, bv, c, idx, 0, 0);
    }
};
template <> struct MfmaForm<7> {                     // dense int8, 16 x 16 x 64
    using Acc = i32x4;
    static constexpr int NACC = 16;
    static __device__ Acc op(const int* a, const int* b, Acc c, int) {
        i32x4 av, bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
    }
};
template <> struct MfmaForm<8> {                     // sparse fp8 (E4M3), 32 x 32, 64 dense k
    using Acc = f32x16;
    static constexpr int NACC = 8;
    static __device__ Acc op(const int* a, const int* b, Acc c, int idx) {
        i32x4 av; i32x8 bv;
        __builtin_memcpy(&av, a, 16); __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(av, bv, c, idx, 0, 0);
    }
};
template <> struct MfmaForm<9> {                     // dense fp8 (E4M3), 32 x 32 x 64, unit scales
    using Acc = f32x16;
    static constexpr int NACC = 8;
    static __device__ Acc op(const int* a, const int* b, Acc c, int) {
        i32x8 av, bv;
        __builtin_memcpy(&av, a, 32); __builtin_memcpy(&bv, b, 32);
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
    }
};

template <int F>
__global__ void __launch_bounds__(kMfmaThreads) k_mfma_rate(int64_t iters, uint32_t seed, uint32_t* sink) {
    using Fm = MfmaForm<F>;
    using Acc = typename Fm::Acc;
    const uint32_t id = (uint32_t)blockIdx.x * kMfmaThreads + threadIdx.x;
    // bf16 forms: both halves positive with exponent fields in [64, 127]
    constexpr bool kBf16 = F <= 3;
    int a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t ha = lane_hash(id * 16u + (uint32_t)i + seed), hb = lane_hash(id * 16u + 8u + (uint32_t)i + seed);
        a[i] = (int)(kBf16 ? (ha & 0x3fff3fffu) | 0x20002000u : ha);
        b[i] = (int)(kBf16 ? (hb & 0x3fff3fffu) | 0x20002000u : hb);
        if (F == 8 || F == 9) {                      // no NaN bytes (E4M3: 0x7f / 0xff)
            a[i] &= 0x77777777;
            b[i] &= 0x77777777;
        }
    }
    // valid 2:4 index nibbles (first kept position below the second)
    constexpr uint32_t kValid[6] = {0x4u, 0x8u, 0xCu, 0x9u, 0xDu, 0xEu};
    const uint32_t hi = lane_hash(id ^ 0xA511E9B3u ^ seed);
    uint32_t idx = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) idx |= kValid[((hi >> (4 * j)) & 0xFu) % 6u] << (4 * j);
    Acc acc[Fm::NACC];
#pragma unroll
    for (int j = 0; j < Fm::NACC; ++j) acc[j] = Acc{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < Fm::NACC; ++j) acc[j] = Fm::op(a, b, acc[j], (int)idx);
        a[0] ^= 1;                                   // keeps the operands loop-variant
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < Fm::NACC; ++j)
        for (int e = 0; e < (int)(sizeof(Acc) / 4); ++e) s += (float)acc[j][e];
    if (__float_as_uint(s) == 0x9E3779B9u) sink[blockIdx.x] = 1u;
}

struct FormInfo {
    const char* name;
    int64_t ops;     // dense-equivalent operations per instruction: 2 * 32 * 32 * k or 2 * 16 * 16 * k
    int nacc;
};

constexpr FormInfo kForms[] = {
    {"v_smfmac_f32_32x32x32_bf16", 2LL * 32 * 32 * 32, 8},
    {"v_mfma_f32_32x32x16_bf16", 2LL * 32 * 32 * 16, 8},
    {"v_smfmac_f32_16x16x64_bf16", 2LL * 16 * 16 * 64, 16},
    {"v_mfma_f32_16x16x32_bf16", 2LL * 16 * 16 * 32, 16},
    {"v_smfmac_i32_32x32x64_i8", 2LL * 32 * 32 * 64, 8},
    {"v_mfma_i32_32x32x32_i8", 2LL * 32 * 32 * 32, 8},
    {"v_smfmac_i32_16x16x128_i8", 2LL * 16 * 16 * 128, 16},
    {"v_mfma_i32_16x16x64_i8", 2LL * 16 * 16 * 64, 16},
    {"v_smfmac_f32_32x32x64_fp8_fp8", 2LL * 32 * 32 * 64, 8},
    {"v_mfma_f32_32x32x64_f8f6f4", 2LL * 32 * 32 * 64, 8},
};
constexpr int kNumForms = (int)(sizeof(kForms) / sizeof(kForms[0]));

template <int F>
void launch_rate(int64_t workgroups, int64_t iters, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL(k_mfma_rate<F>, dim3((unsigned)workgroups), dim3(kMfmaThreads), 0, s, iters, 0x5EEDu, sink);
}

}  // namespace

int mfma_probe_forms() { return kNumForms; }

const char* mfma_probe_name(int form) { return form >= 0 && form < kNumForms ? kForms[form].name : nullptr; }

int64_t mfma_probe_ops(int form, int64_t workgroups, int64_t iters) {
    if (form < 0 || form >= kNumForms || workgroups <= 0 || iters <= 0) return 0;
    return kForms[form].ops * kForms[form].nacc * iters * workgroups * (kMfmaThreads / 64);
}

constexpr int kLdsProbeThreads = 256;
typedef __attribute__((address_space(3))) const void lds_cvoid;

__global__ void __launch_bounds__(kLdsProbeThreads) k_lds_read(LdsPattern pat, int64_t iters, uint32_t* sink) {
    __shared__ __attribute__((aligned(1024))) i32x4 buf[4096];     // 64 KiB
    for (int i = threadIdx.x; i < 4096; i += kLdsProbeThreads) buf[i] = i32x4{i, 3 * i, i ^ 0x55, i + 7};
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint32_t addr = (uint32_t)(uintptr_t)(lds_cvoid*)buf + pat.off[lane];
    i32x4 x = {0, 0, 0, 0};
    for (int64_t it = 0; it < iters; ++it) {
        // eight reads in flight, then one wait, in one statement: no output
        // register is reused while its read is outstanding
        i32x4 r0, r1, r2, r3, r4, r5, r6, r7;
        asm volatile(
            "ds_read_b128 %0, %8 offset:0\n\t"
            "ds_read_b128 %1, %8 offset:4096\n\t"
            "ds_read_b128 %2, %8 offset:8192\n\t"
            "ds_read_b128 %3, %8 offset:12288\n\t"
            "ds_read_b128 %4, %8 offset:16384\n\t"
            "ds_read_b128 %5, %8 offset:20480\n\t"
            "ds_read_b128 %6, %8 offset:24576\n\t"
            "ds_read_b128 %7, %8 offset:28672\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
            : "v"(addr)
            : "memory");
        x ^= r0 ^ r1 ^ r2 ^ r3 ^ r4 ^ r5 ^ r6 ^ r7;
    }
    const uint32_t f = (uint32_t)(x.x ^ x.y ^ x.z ^ x.w);
    if (f == 0x9E3779B9u) sink[blockIdx.x] = f;
}

hipError_t launch_lds_read_probe(const LdsPattern& pat, int64_t workgroups, int64_t iters, uint32_t* sink,
                                 hipStream_t s) {
    hipLaunchKernelGGL(k_lds_read, dim3((unsigned)workgroups), dim3(kLdsProbeThreads), 0, s, pat, iters, sink);
    return hipGetLastError();
}

hipError_t launch_mfma_probe(int form, int64_t workgroups, int64_t iters, uint32_t* sink, hipStream_t s) {
    switch (form) {
    case 0: launch_rate<0>(workgroups, iters, sink, s); break;
    case 1: launch_rate<1>(workgroups, iters, sink, s); break;
    case 2: launch_rate<2>(workgroups, iters, sink, s); break;
    case 3: launch_rate<3>(workgroups, iters, sink, s); break;
    case 4: launch_rate<4>(workgroups, iters, sink, s); break;
    case 5: launch_rate<5>(workgroups, iters, sink, s); break;
    case 6: launch_rate<6>(workgroups, iters, sink, s); break;
    case 7: launch_rate<7>(workgroups, iters, sink, s); break;
    case 8: launch_rate<8>(workgroups, iters, sink, s); break;
    case 9: launch_rate<9>(workgroups, iters, sink, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int64_t stream_read_grid(int64_t bytes) {
    const int64_t n16 = bytes / 16;
    return std::max<int64_t>(1, std::min<int64_t>((n16 + kProbeThreads * kProbeUnroll - 1) /
                                                      (kProbeThreads * kProbeUnroll), 8192));
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
    const int64_t grid = stream_read_grid(bytes);
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(kProbeThreads), 0, s,
                       reinterpret_cast<const i32x4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace ssg
