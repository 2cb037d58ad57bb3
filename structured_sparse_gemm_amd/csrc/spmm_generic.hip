// spmm_generic.hip -- the plain-layout SpMM kernels: one thread per output
// element walking its row's groups (decode nibble -> the two kept positions
// -> two multiply-adds: the 2-bit positions choose the two activations of
// the four that meet the stored weights, as in "Chapter 26 -- Sparsity: The
// Hardware View", section "2:4 Fine-Grained Structured Sparsity"), plus the
// residual term (CSR or delta-coded) of "How sparse LLM weights cut GPU
// inference cost without quantization", section "How the three-layer format
// makes moderate sparsity fast".
//
// These kernels take any shape, leading dimension and alignment.  They are
// the fallback for operands the tiled kernels do not take, and the residual
// pass of the large-N path (launch_residual_add).  fp16/bf16 accumulate in
// fp32 with fmaf in k order; int8 accumulates in int32.
#include "ssg_device.hpp"
#include "ssg_kernels.hpp"

namespace ssg {

namespace {

template <int DT> struct Acc { using T = float; };
template <> struct Acc<DT_I8> { using T = int32_t; };

template <int DT>
__device__ __forceinline__ void mac(typename Acc<DT>::T& acc, const void* a, int64_t ia, const void* b, int64_t ib) {
    if constexpr (DT == DT_I8) {
        acc += (int32_t)((const int8_t*)a)[ia] * (int32_t)((const int8_t*)b)[ib];
    } else if constexpr (dt_is_fp8(DT)) {
        acc = fmaf(elem_to_f32<DT>(((const uint8_t*)a)[ia]), elem_to_f32<DT>(((const uint8_t*)b)[ib]), acc);
    } else {
        acc = fmaf(elem_to_f32<DT>(((const uint16_t*)a)[ia]), elem_to_f32<DT>(((const uint16_t*)b)[ib]), acc);
    }
}

// Residual contribution to C[m, n]; the entry range is clamped to
// [0, nnz_r) and columns outside [0, K) are skipped, so a corrupt residual
// cannot cause an out-of-bounds access.  A delta-coded residual (dcol set)
// gives each entry's column as the running sum of the row's gap bytes from
// column -1; its filler entries hold +0.
template <int DT>
__device__ __forceinline__ void residual_row(typename Acc<DT>::T& acc, const SpmmArgs& a, int64_t m, int64_t n) {
    const int64_t lo = max<int64_t>(a.row_ptr[m], 0), hi = min<int64_t>(a.row_ptr[m + 1], a.nnz_r);
    if (a.dcol) {
        int64_t k = -1;
        for (int64_t j = lo; j < hi; ++j) {
            k += a.dcol[j];
            if (k >= 0 && k < a.K) mac<DT>(acc, a.rvals, j, a.B, k * a.ldb + n);
        }
        return;
    }
    for (int64_t j = lo; j < hi; ++j) {
        const int64_t k = a.col[j];
        if (k >= 0 && k < a.K) mac<DT>(acc, a.rvals, j, a.B, k * a.ldb + n);
    }
}

template <int DT>
__global__ void __launch_bounds__(256) k_spmm_generic(SpmmArgs a) {
    using AT = typename Acc<DT>::T;
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= a.N) return;
    for (int64_t m = blockIdx.y; m < a.M; m += gridDim.y) {
        AT acc = AT(0);
        const uint8_t* mrow = a.meta + m * a.ldm;
        const int64_t vbase = m * a.ldv;
        // no 2:4 layer (vals == nullptr): an unstructured sparse product
        for (int64_t g = 0; a.vals != nullptr && g < a.K / 4; ++g) {
            const uint32_t nib = (mrow[g >> 1] >> (4 * (g & 1))) & 0xFu;
            mac<DT>(acc, a.vals, vbase + 2 * g, a.B, (4 * g + (nib & 3u)) * a.ldb + n);
            mac<DT>(acc, a.vals, vbase + 2 * g + 1, a.B, (4 * g + (nib >> 2)) * a.ldb + n);
        }
        if (a.row_ptr) residual_row<DT>(acc, a, m, n);
        reinterpret_cast<AT*>(a.C)[m * a.ldc + n] = acc;
    }
}

template <int DT>
__global__ void __launch_bounds__(256) k_residual_add(SpmmArgs a) {
    using AT = typename Acc<DT>::T;
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= a.N) return;
    for (int64_t m = blockIdx.y; m < a.M; m += gridDim.y) {
        AT acc = AT(0);
        residual_row<DT>(acc, a, m, n);
        reinterpret_cast<AT*>(a.C)[m * a.ldc + n] += acc;
    }
}

dim3 grid_for(const SpmmArgs& a, int threads) {
    return dim3((unsigned)((a.N + threads - 1) / threads), (unsigned)(a.M < 65535 ? a.M : 65535));
}

}  // namespace

hipError_t launch_spmm_generic(const SpmmArgs& a, hipStream_t s) {
    if (a.M == 0 || a.N == 0) return hipSuccess;
    const int threads = a.N >= 256 ? 256 : 64;
    switch (a.dt) {
        case DT_F16: hipLaunchKernelGGL(k_spmm_generic<DT_F16>, grid_for(a, threads), dim3(threads), 0, s, a); break;
        case DT_BF16: hipLaunchKernelGGL(k_spmm_generic<DT_BF16>, grid_for(a, threads), dim3(threads), 0, s, a); break;
        case DT_I8: hipLaunchKernelGGL(k_spmm_generic<DT_I8>, grid_for(a, threads), dim3(threads), 0, s, a); break;
        case DT_E4M3:
            hipLaunchKernelGGL(k_spmm_generic<DT_E4M3>, grid_for(a, threads), dim3(threads), 0, s, a);
            break;
        case DT_E5M2:
            hipLaunchKernelGGL(k_spmm_generic<DT_E5M2>, grid_for(a, threads), dim3(threads), 0, s, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_residual_add(const SpmmArgs& a, hipStream_t s) {
    if (a.M == 0 || a.N == 0 || a.row_ptr == nullptr) return hipSuccess;
    const int threads = a.N >= 256 ? 256 : 64;
    switch (a.dt) {
        case DT_F16: hipLaunchKernelGGL(k_residual_add<DT_F16>, grid_for(a, threads), dim3(threads), 0, s, a); break;
        case DT_BF16: hipLaunchKernelGGL(k_residual_add<DT_BF16>, grid_for(a, threads), dim3(threads), 0, s, a); break;
        case DT_I8: hipLaunchKernelGGL(k_residual_add<DT_I8>, grid_for(a, threads), dim3(threads), 0, s, a); break;
        case DT_E4M3:
            hipLaunchKernelGGL(k_residual_add<DT_E4M3>, grid_for(a, threads), dim3(threads), 0, s, a);
            break;
        case DT_E5M2:
            hipLaunchKernelGGL(k_residual_add<DT_E5M2>, grid_for(a, threads), dim3(threads), 0, s, a);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssg
