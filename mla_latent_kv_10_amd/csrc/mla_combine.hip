// Split-KV LSE merge kernel.
//
// [Walkthrough] §七 "split-KV：把长序列切开": partial results over disjoint
// KV ranges merge as m = max m_k, l = sum l_k e^{m_k - m},
// o = sum o_k l_k e^{m_k - m} / l. The split kernel stores each partial
// normalised (o_k = O_k / l_k) with lse_k = m_k + ln l_k, so the merge is
// lse = ln sum_k e^{lse_k} and o = sum_k e^{lse_k - lse} o_k. Empty partials
// (lse_k = -inf) weigh zero; a row with no partial at all gets o = 0 and
// lse = -inf.
//
// One wave per query row: lanes split the 512 output dims (8 each) and share
// the reduction over splits through wave shuffles.
#include "mla_common.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;

__device__ __forceinline__ float wave_max(float v) {
    #pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    #pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t rowg = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int Q = p.batch * p.n_rg;
    const int q = (int)(rowg / p.rg);
    const int rr = (int)(rowg - (int64_t)q * p.rg);
    if (q >= Q) return;
    const int b = q / p.n_rg;
    const int rgi = q - b * p.n_rg;
    const int i = rgi / p.n_hb;
    const int h = (rgi - i * p.n_hb) * p.rg + rr;
    if (h >= p.h_q) return;
    const int s0 = p.split_offsets[q];
    const int n = p.split_offsets[q + 1] - s0;
    if (n == 1) return;  // the split kernel wrote the final row
    const int64_t orow = ((int64_t)b * p.s_q + i) * p.h_q + h;
    uint16_t* op = p.o + orow * kDv + 8 * lane;
    const float* lse_k = p.ws_lse + (int64_t)s0 * p.rg + rr;

    float m = -INFINITY;
    for (int k = lane; k < n; k += 64) m = fmaxf(m, lse_k[(int64_t)k * p.rg]);
    m = wave_max(m);
    if (n == 0 || m == -INFINITY) {
        *(i16x8*)op = i16x8{};
        if (lane == 0) p.lse[orow] = -INFINITY;
        return;
    }
    float s = 0.f;
    for (int k = lane; k < n; k += 64) s += __expf(lse_k[(int64_t)k * p.rg] - m);
    s = wave_sum(s);
    const float lse = m + __logf(s);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const float* ob = p.ws_o + ((int64_t)s0 * p.rg + rr) * kDv + 8 * lane;
    for (int k = 0; k < n; ++k) {
        const float lk = lse_k[(int64_t)k * p.rg];
        if (lk == -INFINITY) continue;
        const float w = __expf(lk - lse);
        const float* src = ob + (int64_t)k * p.rg * kDv;
        const f32x4 a = *(const f32x4*)src;
        const f32x4 c = *(const f32x4*)(src + 4);
        acc[0] += w * a[0]; acc[1] += w * a[1]; acc[2] += w * a[2]; acc[3] += w * a[3];
        acc[4] += w * c[0]; acc[5] += w * c[1]; acc[6] += w * c[2]; acc[7] += w * c[3];
    }
    i16x8 out;
    #pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = __builtin_bit_cast(short, (__bf16)acc[e]);
    *(i16x8*)op = out;
    if (lane == 0) p.lse[orow] = lse;
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, hipStream_t s) {
    const int64_t rows = (int64_t)p.batch * p.n_rg * p.rg;
    const int64_t blocks = (rows + 3) / 4;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace mla
