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
// Workspace layout of one slot (RG rows x 512 dims, fp16 values o_k / c_k,
// where c_k, a power of two per slot and row, sits in ws_scale):
//   RG = 128 or 64: blocked as the split kernel's MFMA registers hold it, 4-value
//     group index ((w * 16 + dd) * 4 + g) * 64 + lane for row 32 w + (lane & 31),
//     dims 32 dd + 8 g + 4 (lane >> 5) + 0..3;
//   RG = 16: row-major [row][512].
// Each thread owns one row and a fixed set of 4-value groups; consecutive
// threads read consecutive groups of a slot.
#include <type_traits>

#include "mla_common.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// VEC 4-value groups per thread per slot: 2, or 8 for the blocked layouts
// when sequences have few splits (a quarter of the workgroups, each thread
// doing four times the work).
template <int RG, int VEC>
struct CombineMap {
    static_assert(VEC == 2 || (VEC == 8 && RG != 16), "VEC 8 is for the blocked layouts");
    static constexpr int kPerBlock = 16 / VEC;  // workgroups per 32-row block (blocked layouts)
    // workgroups per row-group sequence: VEC 2 -> 32 (RG 128), 16 (RG 64), 4 (RG 16); VEC 8 -> 8, 4
    static constexpr int kBlocksPerQ = RG == 16 ? 4 : (RG / 32) * kPerBlock;
    static constexpr int kVec = VEC;
    // thread -> (row, group offsets within the slot, dims of each group)
    __device__ static void map(int blk, int t, int& row, int (&f4)[kVec], int (&dim)[kVec]) {
        if constexpr (RG != 16) {
            const int w = blk / kPerBlock, dq = blk % kPerBlock;
            const int lane = t & 63, g = (t >> 6) & 3;
            row = 32 * w + (lane & 31);
            #pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const int dd = VEC * dq + j;
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
// values, scales and partial rows) is issued before any of them is used, and
// the running reference m moves with a rescale of the sums, as in the online
// softmax ([Walkthrough] §五). Result: o = sum_k e^{lse_k - m} c_k h_k / s
// with h_k the stored fp16 row, s = sum_k e^{lse_k - m}, lse = m + ln s.
// split_offsets travels as a separate leading argument (the same pointer as
// p.split_offsets), preloaded into SGPRs at dispatch, so the split-count
// loads issue without waiting for the argument block.
// DV: value dims of o (512, or 448 for 528-byte rows). Slots always hold 512
// dims per row; groups at dims >= DV are merged like the others (from slot
// bytes the split kernel did not write) and never stored.
template <int RG, int VEC, int KU_MAX, int DV>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ split_offsets, DecodeParams p) {
    using M = CombineMap<RG, VEC>;
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
    const int h = (rgi - i * p.n_hb) * RG + row;  // row of the row space (see Layout)
    if (h >= p.rows_b) return;
    const int s0 = split_offsets[q];
    const int n = split_offsets[q + 1] - s0;
    if (n == 1) return;  // the split kernel wrote the final row
    const int64_t orow = ((int64_t)b * p.n_pos + i) * p.rows_b + h;
    uint16_t* op = p.o + orow * DV;
    const bool lse_writer = dim[0] == 0;  // exactly one thread per row holds dim 0
    constexpr int kSlotBytes = RG * kDv * 2;  // fp16 partial rows of one slot
    float m = -INFINITY, s = 0.f;
    f32x4 acc[M::kVec];
    #pragma unroll
    for (int j = 0; j < M::kVec; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Each partial is read exactly once. With three or more splits the loads
    // are non-temporal (measured faster); with two (long sequences, many
    // workgroups) the default policy measured faster.
    // kU splits in flight per chunk: the power of two in 2..KU_MAX nearest
    // above n, so a sequence with few splits issues few loads.
    auto merge = [&](auto nt_tag, auto ku_tag) {
        constexpr int AUX = decltype(nt_tag)::value ? 2 : 0;  // 2: nt
        constexpr int kU = decltype(ku_tag)::value;
        for (int k0 = 0; k0 < n; k0 += kU) {
            // All kU loads issue unconditionally (a conditional load would
            // become a branch closed by a wait, one round trip per split).
            // Slots past the chunk's last split re-read its first split and
            // weigh zero: the split's offset travels in soffset, which the
            // buffer range check does not cover, so it is chosen in range.
            const int nc = min(kU, n - k0);
            const int64_t slot0 = (int64_t)s0 + k0;
            const __amdgpu_buffer_rsrc_t o_rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(p.ws_o + slot0 * RG * kDv), (short)0, nc * kSlotBytes, 0x00020000);
            const __amdgpu_buffer_rsrc_t l_rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(p.ws_lse + slot0 * RG), (short)0, nc * RG * 4, 0x00020000);
            const __amdgpu_buffer_rsrc_t c_rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)(p.ws_scale + slot0 * RG), (short)0, nc * RG * 4, 0x00020000);
            float lv[kU], cv[kU];
            u32x2 v[kU][M::kVec];
            // per-lane byte offsets in VGPRs, the split's offset in the
            // (uniform) soffset field: no VGPR per load for addressing
            #pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int su = u < nc ? u : 0;  // uniform
                lv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(l_rs, row * 4, su * RG * 4, 0));
                cv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(c_rs, row * 4, su * RG * 4, 0));
                #pragma unroll
                for (int j = 0; j < M::kVec; ++j)
                    v[u][j] = __builtin_amdgcn_raw_buffer_load_b64(o_rs, f4[j] * 8, su * kSlotBytes, AUX);
            }
            // keep every load of the chunk ahead of the first use (left alone,
            // the scheduler issues the data loads only after the lse maximum)
            __builtin_amdgcn_sched_barrier(0);
            #pragma unroll
            for (int u = 0; u < kU; ++u)
                if (u >= nc) lv[u] = -INFINITY;
            float mc = m;
            #pragma unroll
            for (int u = 0; u < kU; ++u) mc = fmaxf(mc, lv[u]);
            // Branch-free (a branch here would let the compiler sink the data
            // loads below it, a second round trip): while nothing is attended
            // (mc = -inf) every weight is 0 and the sums stay 0.
            const float r = (m == -INFINITY) ? 0.f : __expf(m - mc);
            s *= r;
            #pragma unroll
            for (int j = 0; j < M::kVec; ++j) acc[j] *= r;
            #pragma unroll
            for (int u = 0; u < kU; ++u) {
                const float wgt = lv[u] == -INFINITY ? 0.f : __expf(lv[u] - mc);
                s += wgt;
                const float wc = wgt * cv[u];
                #pragma unroll
                for (int j = 0; j < M::kVec; ++j)
                    acc[j] += wc * __builtin_convertvector(__builtin_bit_cast(f16x4, v[u][j]), f32x4);
            }
            m = mc;
        }
    };
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    using I16 = std::integral_constant<int, 16>;
    if (n <= 2) merge(std::false_type{}, I2{});
    else if (KU_MAX == 4 || n <= 4) merge(std::true_type{}, I4{});
    else if constexpr (KU_MAX >= 16) {
        if (n <= 8) merge(std::true_type{}, I8{});
        else merge(std::true_type{}, I16{});
    }
    // no split attended anything (or no split at all): o = 0, lse = -inf
    const bool empty = m == -INFINITY;
    const float inv = empty ? 0.f : 1.f / s;
    #pragma unroll
    for (int j = 0; j < M::kVec; ++j) {
        i16x4 o4;
        #pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = __builtin_bit_cast(short, (__bf16)(acc[j][e] * inv));
        if (DV == kDv || dim[j] < DV) *(i16x4*)(op + dim[j]) = o4;
    }
    if (lse_writer) p.lse[orow] = empty ? -INFINITY : m + __logf(s);
}

}  // namespace

template <int RG, int VEC, int KU_MAX, int DV>
void launch_map(const DecodeParams& p, int Q, hipStream_t s) {
    hipLaunchKernelGGL((combine_kernel<RG, VEC, KU_MAX, DV>), dim3((unsigned)Q * CombineMap<RG, VEC>::kBlocksPerQ),
                       dim3(256), 0, s, p.split_offsets, p);
}

template <int DV>
void launch_dv(const DecodeParams& p, hipStream_t s) {
    const int Q = p.batch * p.n_rg;
    // At most one split per sequence on average (num_parts <= Q): most rows
    // were finished by the split kernel and the merge is mostly launch
    // overhead, so the wide mapping (a quarter of the workgroups, chunks of up
    // to 4 splits) is used. Any split count is merged correctly either way;
    // this only picks the faster one (sparse prefill, one split per sequence:
    // 21.4 -> 8.0 us; two splits per sequence: 11.6 -> 12.8 us, so not there).
    const bool wide = p.num_parts <= Q;
    if (p.rg == 128) {
        if (wide) launch_map<128, 8, 4, DV>(p, Q, s);
        else launch_map<128, 2, 16, DV>(p, Q, s);
    } else if (p.rg == 64) {
        if (wide) launch_map<64, 8, 4, DV>(p, Q, s);
        else launch_map<64, 2, 16, DV>(p, Q, s);
    } else {
        launch_map<16, 2, 16, DV>(p, Q, s);
    }
}

hipError_t launch_combine(const DecodeParams& p, int format, hipStream_t s) {
    if (format == kFmtFp8Mx) launch_dv<448>(p, s);
    else launch_dv<kDv>(p, s);
    return hipGetLastError();
}

}  // namespace mla
