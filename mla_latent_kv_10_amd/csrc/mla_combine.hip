// Split-KV LSE merge kernel.
//
// [Walkthrough] §七 "split-KV：把长序列切开": partial results over disjoint
// KV ranges merge as m = max m_k, l = sum l_k e^{m_k - m},
// o = sum o_k l_k e^{m_k - m} / l. The split kernel stores each partial
// normalised (o_k = O_k / l_k) with lse_k = m_k + ln l_k, so the merge is
// lse = ln sum_k e^{lse_k} and o = sum_k e^{lse_k - lse} o_k. Empty partials
// (lse_k = -inf) weigh zero; a row with no partial at all gets o = 0 and
// lse = -inf; a row with exactly one split was written by the split kernel.
//
// Workspace layout of one slot (RG rows x 512 dims, fp32):
//   RG = 128 or 64: blocked as the split kernel's MFMA registers hold it, float4
//     index ((w * 16 + dd) * 4 + g) * 64 + lane for row 32 w + (lane & 31),
//     dims 32 dd + 8 g + 4 (lane >> 5) + 0..3;
//   RG = 16: row-major [row][512].
// Each thread owns one row and a fixed set of float4s; consecutive threads
// read consecutive float4s of a slot.
#include <type_traits>

#include "mla_common.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;

template <int RG>
struct CombineMap {
    // blocks per row-group sequence, float4s per thread per slot
    static constexpr int kBlocksPerQ = RG == 16 ? 4 : RG / 4;  // 128 -> 32, 64 -> 16
    static constexpr int kVec = 2;
    // thread -> (row, float4 offsets within the slot, dims of each float4)
    __device__ static void map(int blk, int t, int& row, int (&f4)[kVec], int (&dim)[kVec]) {
        if constexpr (RG != 16) {
            const int w = blk >> 3, dq = blk & 7;
            const int lane = t & 63, g = (t >> 6) & 3;
            row = 32 * w + (lane & 31);
            #pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const int dd = 2 * dq + j;
                f4[j] = ((w * 16 + dd) * 4 + g) * 64 + lane;
                dim[j] = 32 * dd + 8 * g + 4 * (lane >> 5);
            }
        } else {
            const int dq = blk;
            row = t >> 4;
            const int c = t & 15;
            #pragma unroll
            for (int j = 0; j < kVec; ++j) {
                dim[j] = 128 * dq + 4 * c + 64 * j;
                f4[j] = (row * 512 + dim[j]) >> 2;
            }
        }
    }
};

// One pass over the splits, kU at a time: every load of a chunk (its lse
// values and its partial rows) is issued before any of them is used, and the
// running reference m moves with a rescale of the sums, as in the online
// softmax ([Walkthrough] §五). Result: o = sum_k e^{lse_k - m} o_k / s with
// s = sum_k e^{lse_k - m}, lse = m + ln s.
template <int RG>
__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p) {
    using M = CombineMap<RG>;
    // XCD-aware numbering, as in the split kernel: the parts of one sequence
    // run on one XCD, so its partials are merged on the XCD that wrote them.
    int lb = blockIdx.x;
    if ((gridDim.x & 7) == 0) lb = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int q = lb / M::kBlocksPerQ;
    const int blk = lb - q * M::kBlocksPerQ;
    const int b = q / p.n_rg;
    const int rgi = q - b * p.n_rg;
    const int i = rgi / p.n_hb;
    int row, f4[M::kVec], dim[M::kVec];
    M::map(blk, threadIdx.x, row, f4, dim);
    const int h = (rgi - i * p.n_hb) * RG + row;
    if (h >= p.h_q) return;
    const int s0 = p.split_offsets[q];
    const int n = p.split_offsets[q + 1] - s0;
    if (n == 1) return;  // the split kernel wrote the final row
    const int64_t orow = ((int64_t)b * p.s_q + i) * p.h_q + h;
    uint16_t* op = p.o + orow * kDv;
    const float* lse_k = p.ws_lse + (int64_t)s0 * RG + row;
    const bool lse_writer = dim[0] == 0;  // exactly one thread per row holds dim 0
    const f32x4* base = (const f32x4*)(p.ws_o + (int64_t)s0 * RG * kDv);
    constexpr int kSlot4 = RG * kDv / 4;  // float4s per slot
    constexpr int kU = 16;                // splits in flight
    float m = -INFINITY, s = 0.f;
    f32x4 acc[M::kVec];
    #pragma unroll
    for (int j = 0; j < M::kVec; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Each partial is read exactly once. With three or more splits the loads
    // are non-temporal (measured faster); with two (long sequences, many
    // workgroups) the default policy measured faster.
    auto merge = [&](auto nt_tag) {
        constexpr bool NT = decltype(nt_tag)::value;
        for (int k0 = 0; k0 < n; k0 += kU) {
            float lv[kU];
            f32x4 v[kU][M::kVec];
            #pragma unroll
            for (int u = 0; u < kU; ++u) {
                const bool in = k0 + u < n;
                lv[u] = in ? lse_k[(int64_t)(k0 + u) * RG] : -INFINITY;
                #pragma unroll
                for (int j = 0; j < M::kVec; ++j) {
                    const f32x4* src = &base[(int64_t)(k0 + u) * kSlot4 + f4[j]];
                    if constexpr (NT) v[u][j] = in ? __builtin_nontemporal_load(src) : f32x4{0.f, 0.f, 0.f, 0.f};
                    else v[u][j] = in ? *src : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            float mc = m;
            #pragma unroll
            for (int u = 0; u < kU; ++u) mc = fmaxf(mc, lv[u]);
            if (mc == -INFINITY) continue;  // nothing attended so far
            const float r = (m == -INFINITY) ? 0.f : __expf(m - mc);
            s *= r;
            #pragma unroll
            for (int j = 0; j < M::kVec; ++j) acc[j] *= r;
            #pragma unroll
            for (int u = 0; u < kU; ++u) {
                const float wgt = lv[u] == -INFINITY ? 0.f : __expf(lv[u] - mc);
                s += wgt;
                #pragma unroll
                for (int j = 0; j < M::kVec; ++j) acc[j] += wgt * v[u][j];
            }
            m = mc;
        }
    };
    if (n >= 3) merge(std::true_type{});
    else merge(std::false_type{});
    // no split attended anything (or no split at all): o = 0, lse = -inf
    const bool empty = m == -INFINITY;
    const float inv = empty ? 0.f : 1.f / s;
    #pragma unroll
    for (int j = 0; j < M::kVec; ++j) {
        i16x4 o4;
        #pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = __builtin_bit_cast(short, (__bf16)(acc[j][e] * inv));
        *(i16x4*)(op + dim[j]) = o4;
    }
    if (lse_writer) p.lse[orow] = empty ? -INFINITY : m + __logf(s);
}

}  // namespace

hipError_t launch_combine(const DecodeParams& p, hipStream_t s) {
    const int Q = p.batch * p.n_rg;
    if (p.rg == 128) {
        hipLaunchKernelGGL(combine_kernel<128>, dim3((unsigned)Q * CombineMap<128>::kBlocksPerQ), dim3(256), 0, s, p);
    } else if (p.rg == 64) {
        hipLaunchKernelGGL(combine_kernel<64>, dim3((unsigned)Q * CombineMap<64>::kBlocksPerQ), dim3(256), 0, s, p);
    } else {
        hipLaunchKernelGGL(combine_kernel<16>, dim3((unsigned)Q * CombineMap<16>::kBlocksPerQ), dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace mla
