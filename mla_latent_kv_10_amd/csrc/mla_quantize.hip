// FP8 cache writer: quantise new cache rows on write.
//
// Layout of the 656-byte row from [Guide] §"FP8 缓存怎么把 KV 压掉四成":
// 512 e4m3 codes of the latent, one fp32 scale per 128 latent values, then
// the 64 RoPE values kept in bf16; [Guide] §"容易踩的坑" is why the writer has
// to produce exactly this layout (a decode reading 656-byte rows from a cache
// written otherwise returns garbage). [Walkthrough] §三 gives e4m3's 3
// mantissa bits and its largest finite value, 448, and why the scale is per
// block rather than per tensor.
//
// Per group of 128 values: scale = amax / 448 in fp32 (1 for an all-zero
// group), code = e4m3 round-to-nearest-even of clamp(x / scale, +-448), both
// divisions IEEE fp32. Streaming work: one wave64 per row, each lane holding
// 8 latent values (a 16-byte load), so a 128-value group is 16 lanes and its
// amax a 4-step butterfly within them; lanes 0-7 also carry the 128 RoPE
// bytes. The codes leave as two 4-byte stores per lane. The row's loads go
// out before its slot is tested, so a wave waits for one memory round trip,
// not two; source rows are read once and the written rows are not read back
// by this kernel, so both streams are non-temporal.
#include "mla_quantize.h"

namespace mla {

namespace {

constexpr int kRowsPerBlock = kThreads / 64;  // one wave per row

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt(const uint4* ptr) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_nt(uint8_t* dst, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(dst));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 values (|y| <= 448) -> two e4m3 codes in the low or high half of `old`
// (v_cvt_pk_fp8_f32: OCP e4m3 on gfx950, round to nearest even).
template <bool HIGH>
__device__ __forceinline__ uint32_t pack_fp8(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HIGH);
}

__device__ __forceinline__ float quotient(float x, float scale) {
    return fminf(fmaxf(x / scale, -448.f), 448.f);
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= p.n) return;

    const uint4* src = reinterpret_cast<const uint4*>(p.src + row * kDqk);
    const uint4 w = load_nt(src + lane);            // latent values 8*lane .. 8*lane+7
    uint4 rope = make_uint4(0, 0, 0, 0);
    if (lane < 8) rope = load_nt(src + 64 + lane);  // the 64 RoPE values, 16 bytes per lane
    const int slot = __builtin_amdgcn_readfirstlane(p.slots[row]);
    if (slot < 0 || slot >= p.num_rows) return;  // -1 (and anything outside the cache) writes nothing

    float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                  bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
    float amax = 0.f;
    #pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    #pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));  // 16-lane group
    const float scale = amax == 0.f ? 1.f : amax / 448.f;

    uint32_t c0 = pack_fp8<false>(quotient(x[0], scale), quotient(x[1], scale), 0u);
    c0 = pack_fp8<true>(quotient(x[2], scale), quotient(x[3], scale), c0);
    uint32_t c1 = pack_fp8<false>(quotient(x[4], scale), quotient(x[5], scale), 0u);
    c1 = pack_fp8<true>(quotient(x[6], scale), quotient(x[7], scale), c1);

    uint8_t* dst = p.kv + (int64_t)slot * kRawRow;
    store_nt(dst + lane * 8, c0);
    store_nt(dst + lane * 8 + 4, c1);
    if ((lane & 15) == 0) store_nt(dst + kDv + (lane >> 4) * 4, __float_as_uint(scale));
    if (lane < 8) {
        uint8_t* r = dst + kDv + 16 + lane * 16;
        store_nt(r, rope.x);
        store_nt(r + 4, rope.y);
        store_nt(r + 8, rope.z);
        store_nt(r + 12, rope.w);
    }
}

}  // namespace

hipError_t launch_quantize(const QuantParams& p, hipStream_t s) {
    const int64_t blocks = (p.n + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mla
