// ssg_stream.hpp -- buffer-resource loads, direct-to-LDS loads and the
// hand-counted memory waits of the streaming SpMM kernels (the 2:4 decode
// kernels and the N:M decode kernel).  Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssg {

typedef __attribute__((address_space(3))) void lds_void;

constexpr uint32_t kOob = 0x80000000u;   // buffer offset that reads as zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}

// Buffer over an array of `bytes` whose base is ALIGN-aligned, read with
// loads of at most ALIGN bytes at multiples of their size.  The range is
// rounded up to ALIGN: a load that holds the array's last bytes is then
// performed whole (the hardware range check would zero the partial word),
// and it stays inside the ALIGN-aligned block of the last byte, so it reads
// only mapped memory; the bytes past the array are masked by the caller.
template <int ALIGN>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_aligned(const void* base, int64_t bytes) {
    return rsrc(base, (bytes + ALIGN - 1) / ALIGN * ALIGN);
}

// Direct-to-LDS load of BYTES (4 or 16) per active lane: lane l's bytes from
// buffer offset `voff` land at LDS byte address `dst` + l * BYTES (`dst`
// wave-uniform, passed in M0); an offset past the buffer reads as zero.
// GFX9 needs one wait state between an SALU write of M0 and an LDS-DMA load
// that reads it (else the load may take the previous M0), hence the s_nop.  Inline assembly, so the compiler does not count it: the
// kernel waits for these loads itself (vmcnt), and issues them before the
// weight loads the compiler does count, so the compiler's own waits for
// those (loads complete in order) also cover them.
template <int BYTES>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, uint32_t dst, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(dst);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
                     : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS barrier without the release fence of __syncthreads (which would also
// wait for this wave's outstanding weight loads): the wave's own LDS
// accesses are made complete first (lgkmcnt(0)), then the workgroup meets.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("s_barrier" ::: "memory");
}

}  // namespace ssg
