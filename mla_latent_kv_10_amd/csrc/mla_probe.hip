// Measurement aids: what this GPU reaches on its own, for context beside the
// published peaks that the decode's roofline fractions are taken against.
// Neither kernel is part of the decode path.
//
//  * mfma_loop_kernel: every wave runs `iters` steps of four independent
//    accumulation chains of v_mfma_f32_32x32x16_bf16 on register operands
//    (no memory traffic in the loop), so the MFMA pipes of every SIMD that
//    holds a wave stay busy back to back. Four chains per wave keep each
//    MFMA's result latency covered by the other three.
//  * hbm_read_kernel: reads a buffer once with non-temporal 16-byte loads;
//    each workgroup streams a contiguous range (consecutive lanes, consecutive
//    16 bytes), eight loads in flight per thread; each thread folds what it
//    read into a 32-bit sum.
#include "mla_probe.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float value, float* __restrict__ sink) {
    // every A and B element is bf16(value): the argument keeps the compiler
    // from folding the products
    const __bf16 v = (__bf16)value;
    const bf16x8 a = {v, v, v, v, v, v, v, v};
    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    for (int i = 0; i < iters; ++i) {
        #pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
    }
    float s = 0.f;
    #pragma unroll
    for (int c = 0; c < 4; ++c)
        #pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                       unsigned* __restrict__ sink) {
    // workgroup b streams its own contiguous range of the buffer, 4 KB per
    // step of its 256 threads, eight steps' loads in flight before any is used
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < n16 ? lo + per : n16;
    int64_t i = lo + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 7 * 256 < hi; i += 8 * 256) {
        u32x4 x[8];
        #pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_nontemporal_load(src + i + j * 256);
        #pragma unroll
        for (int j = 0; j < 8; ++j) acc += x[j];
    }
    for (; i < hi; i += 256) acc += __builtin_nontemporal_load(src + i);
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

}  // namespace

hipError_t launch_probe_mfma(int iters, int blocks, float value, float* sink, hipStream_t s) {
    hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(256), 0, s, iters, value, sink);
    return hipGetLastError();
}

hipError_t launch_probe_hbm_read(const void* src, int64_t bytes, int blocks, unsigned* sink, hipStream_t s) {
    hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)src, bytes / 16,
                       sink);
    return hipGetLastError();
}

}  // namespace mla
