// Standalone elementwise tanh-GELU for gfx950 (declared in include/spgelu.h).
//
// The loop fusion of the XLA:GPU emitters page's "Loop emitter" example (a bf16
// [6,512,4096] tensor through the tanh approximation of GELU), written the way
// the Triton lecture notes' GeLU kernel splits it: each workgroup owns a
// contiguous block of the flat array and masks the tail.  The work is a stream
// through HBM (2 bytes in, 2 bytes out per bf16 element, ~20 flops), so the
// design is about bytes in flight, not arithmetic:
//  * 16 bytes per lane per access (8 fp16/bf16 or 4 fp32 elements), 64 lanes of
//    a wave covering 1 KiB of consecutive bytes;
//  * one 16-byte vector per lane and one workgroup per 256 vectors: 6144
//    workgroups for the [6,512,4096] tensor, ~24 per CU, so every CU keeps many
//    waves' reads in flight (2, 4, 8 or 16 vectors per lane measured 3-30%
//    slower: fewer workgroups, later first stores);
//  * loads and stores marked nontemporal: the data is touched once.
// The arithmetic is the GEMM epilogue's (gelu_tanh in gemm_kernels.hpp): fp32,
// then round-to-nearest-even into the element type.
#include "spgelu.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "errors.hpp"
#include "gemm_kernels.hpp"

namespace spg {
namespace {

constexpr int kGeluThreads = 256;
constexpr int kGeluUnroll = 1;   // measured best: more per lane only cuts the workgroup count

template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
    if constexpr (DT == GEMM_F32) return ((const float*)p)[i];
    else return bits_to_f32(((const uint16_t*)p)[i], DT == GEMM_BF16);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
    if constexpr (DT == GEMM_F32) ((float*)p)[i] = v;
    else ((uint16_t*)p)[i] = f32_to_bits(v, DT == GEMM_BF16);
}

// One 16-byte vector: EPV elements widened to fp32, GELU, narrowed back.
template <int DT>
__device__ __forceinline__ u32x4 gelu_vec(u32x4 v) {
    if constexpr (DT == GEMM_F32) {
        // each element goes through a scalar first: a bit cast applied directly to an
        // element of a vector value read element 0 whatever the index (seen with this
        // toolchain: 4 of 16 exponentials left in the kernel)
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t b = v[e];
            r[e] = __builtin_bit_cast(uint32_t, gelu_tanh(__builtin_bit_cast(float, b)));
        }
        return r;
    } else {
        constexpr bool BF = DT == GEMM_BF16;
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = gelu_tanh(bits_to_f32((uint16_t)(v[e] & 0xffffu), BF));
            const float hi = gelu_tanh(bits_to_f32((uint16_t)(v[e] >> 16), BF));
            r[e] = (uint32_t)f32_to_bits(lo, BF) | ((uint32_t)f32_to_bits(hi, BF) << 16);
        }
        return r;
    }
}

// Vector path: x and y 16-byte aligned.  Workgroup b handles vectors
// [b*256*UNROLL, (b+1)*256*UNROLL) of the nv = n / EPV whole vectors, lane-
// contiguous within each of its UNROLL rounds; the last workgroup also handles
// the n % EPV trailing elements.
template <int DT>
__global__ void __launch_bounds__(kGeluThreads) gelu_vec_kernel(const void* x, void* y, int64_t n) {
    constexpr int EPV = DT == GEMM_F32 ? 4 : 8;   // elements per 16-byte vector
    const int64_t nv = n / EPV;
    const int64_t base = (int64_t)blockIdx.x * (kGeluThreads * kGeluUnroll) + threadIdx.x;
    const u32x4* xv = (const u32x4*)x;
    u32x4* yv = (u32x4*)y;
    u32x4 v[kGeluUnroll];
#pragma unroll
    for (int u = 0; u < kGeluUnroll; ++u) {
        const int64_t i = base + u * kGeluThreads;
        if (i < nv) v[u] = __builtin_nontemporal_load(xv + i);
    }
#pragma unroll
    for (int u = 0; u < kGeluUnroll; ++u) {
        const int64_t i = base + u * kGeluThreads;
        if (i < nv) __builtin_nontemporal_store(gelu_vec<DT>(v[u]), yv + i);
    }
    if (blockIdx.x == gridDim.x - 1) {
        const int64_t i = nv * EPV + threadIdx.x;
        if (i < n) store_elem<DT>(y, i, gelu_tanh(load_elem<DT>(x, i)));
    }
}

// Element path for unaligned pointers: a grid-stride loop, one element per lane.
template <int DT>
__global__ void __launch_bounds__(kGeluThreads) gelu_elem_kernel(const void* x, void* y, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kGeluThreads;
    for (int64_t i = (int64_t)blockIdx.x * kGeluThreads + threadIdx.x; i < n; i += stride)
        store_elem<DT>(y, i, gelu_tanh(load_elem<DT>(x, i)));
}

template <int DT>
void launch_gelu(const void* x, void* y, int64_t n, hipStream_t st) {
    constexpr int EPV = DT == GEMM_F32 ? 4 : 8;
    const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0);
    if (aligned) {
        const int64_t nv = n / EPV;
        const int64_t per = (int64_t)kGeluThreads * kGeluUnroll;
        int64_t blocks = (nv + per - 1) / per;
        if (blocks < 1) blocks = 1;   // the tail alone
        hipLaunchKernelGGL(gelu_vec_kernel<DT>, dim3((uint32_t)blocks), dim3(kGeluThreads), 0, st,
                           x, y, n);
    } else {
        int64_t blocks = (n + kGeluThreads - 1) / kGeluThreads;
        if (blocks > 8192) blocks = 8192;
        hipLaunchKernelGGL(gelu_elem_kernel<DT>, dim3((uint32_t)blocks), dim3(kGeluThreads), 0, st,
                           x, y, n);
    }
}

}  // namespace
}  // namespace spg

extern "C" gemm_status gelu_run(const void* x, void* y, int64_t n, gemm_dtype dtype,
                                hipStream_t stream) {
    if (n < 0) return GEMM_ERR_INVALID_ARG;
    if (dtype != GEMM_F16 && dtype != GEMM_BF16 && dtype != GEMM_F32) return GEMM_ERR_INVALID_ARG;
    if (n == 0) return GEMM_OK;
    if (!x || !y) return GEMM_ERR_INVALID_ARG;
    // a grid of at most 2^32 work-items: n / 4 / 4 (vector path) and 8192 workgroups
    // (element path) stay within it for n < 2^36 elements (256 GiB of fp32)
    if (n >= ((int64_t)1 << 36)) return GEMM_ERR_UNSUPPORTED;
    if (dtype == GEMM_F16) spg::launch_gelu<GEMM_F16>(x, y, n, stream);
    else if (dtype == GEMM_BF16) spg::launch_gelu<GEMM_BF16>(x, y, n, stream);
    else spg::launch_gelu<GEMM_F32>(x, y, n, stream);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? GEMM_OK : spg::hip_fail(e);
}
