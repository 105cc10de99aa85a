// Device helpers shared by the split-decode kernels (gfx950 only).
#pragma once

#include "mla_common.h"

namespace mla {
namespace dev {

#define LDS_AS __attribute__((address_space(3)))
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;  // exponent reference moves when a row max grows by > 2^8
constexpr unsigned kOOB = 0xFFFFFFFFu;

// ---------------------------------------------------------------- cache row formats

// What a cache row format fixes for the split kernel.
//   bf16:     576 bf16 values (1152 B): 512 latent + 64 RoPE; the tile is used as loaded.
//   fp8:      656 B: 512 e4m3 latent codes, 4 fp32 scales (one per 128), 64 bf16 RoPE.
//   fp8_528:  528 B: 512 e4m3 codes (448 latent + 64 RoPE), 16 UE8M0 scales (one per 32).
// Raw (FP8) rows land in LDS as stored and are dequantised into a bf16 tile of
// kDqk values per token: kDqk / 8 16-byte units, grouped 8 to a 1 KB chunk
// per 8 tokens (kUg unit groups per row).
template <int FMT>
struct Fmt {
    static constexpr bool kRaw = FMT != kFmtBf16;
    static constexpr bool kMx = FMT == kFmtFp8Mx;
    static constexpr int kDqk = kMx ? 512 : 576;            // key and query dims
    static constexpr int kDv = kMx ? 448 : 512;             // value (latent) dims
    static constexpr int kUg = kDqk / 64;                   // unit groups per token group
    static constexpr int kTile = kBlock * kDqk * 2;         // bf16 tile bytes in LDS
    static constexpr int kRawRow = kMx ? 528 : 656;
    static constexpr int kRawUnits = kRawRow / 16;          // 16-byte units per raw row (33, 41)
    static constexpr int kRawTile = kBlock * kRawRow;       // kRawUnits KB
    static constexpr int kRawSlots = (kRawUnits + 3) / 4;   // 1 KB chunk slots per wave per raw tile
    // x * kDivMagic >> 16 == x / kRawUnits for 0 <= x < 64 * (kRawUnits + 1)
    static constexpr unsigned kDivMagic = kMx ? 1986u : 1599u;
};

// ---------------------------------------------------------------- LDS layout

template <int FMT>
struct Smem {
    // bf16: two tiles (double buffer). FP8: two raw tiles + one bf16 tile.
    using F = Fmt<FMT>;
    static constexpr int kTileA = 0;
    static constexpr int kTileB = F::kRaw ? -1 : F::kTile;
    static constexpr int kRaw0 = F::kRaw ? F::kTile : -1;
    static constexpr int kRaw1 = F::kRaw ? F::kTile + F::kRawTile : -1;
    static constexpr int kBytes = F::kRaw ? F::kTile + 2 * F::kRawTile : 2 * F::kTile;
};

// ---------------------------------------------------------------- waits

__device__ __forceinline__ void wait_vm(int n) {
    // vmcnt takes an immediate (0..63 on gfx950); n is wave-uniform. Counts past that wait for everything.
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
        case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
        case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
        case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
        case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
        case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
        case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
        case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
        case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
        case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
        case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
        case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
        case 25: asm volatile("s_waitcnt vmcnt(25)" ::: "memory"); break;
        case 26: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
        case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
        case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
        case 29: asm volatile("s_waitcnt vmcnt(29)" ::: "memory"); break;
        case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
        case 31: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
        case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
        case 33: asm volatile("s_waitcnt vmcnt(33)" ::: "memory"); break;
        case 34: asm volatile("s_waitcnt vmcnt(34)" ::: "memory"); break;
        case 35: asm volatile("s_waitcnt vmcnt(35)" ::: "memory"); break;
        case 36: asm volatile("s_waitcnt vmcnt(36)" ::: "memory"); break;
        case 37: asm volatile("s_waitcnt vmcnt(37)" ::: "memory"); break;
        case 38: asm volatile("s_waitcnt vmcnt(38)" ::: "memory"); break;
        case 39: asm volatile("s_waitcnt vmcnt(39)" ::: "memory"); break;
        case 40: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
        case 41: asm volatile("s_waitcnt vmcnt(41)" ::: "memory"); break;
        case 42: asm volatile("s_waitcnt vmcnt(42)" ::: "memory"); break;
        case 43: asm volatile("s_waitcnt vmcnt(43)" ::: "memory"); break;
        case 44: asm volatile("s_waitcnt vmcnt(44)" ::: "memory"); break;
        case 45: asm volatile("s_waitcnt vmcnt(45)" ::: "memory"); break;
        case 46: asm volatile("s_waitcnt vmcnt(46)" ::: "memory"); break;
        case 47: asm volatile("s_waitcnt vmcnt(47)" ::: "memory"); break;
        case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
        case 49: asm volatile("s_waitcnt vmcnt(49)" ::: "memory"); break;
        case 50: asm volatile("s_waitcnt vmcnt(50)" ::: "memory"); break;
        case 51: asm volatile("s_waitcnt vmcnt(51)" ::: "memory"); break;
        case 52: asm volatile("s_waitcnt vmcnt(52)" ::: "memory"); break;
        case 53: asm volatile("s_waitcnt vmcnt(53)" ::: "memory"); break;
        case 54: asm volatile("s_waitcnt vmcnt(54)" ::: "memory"); break;
        case 55: asm volatile("s_waitcnt vmcnt(55)" ::: "memory"); break;
        case 56: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
        case 57: asm volatile("s_waitcnt vmcnt(57)" ::: "memory"); break;
        case 58: asm volatile("s_waitcnt vmcnt(58)" ::: "memory"); break;
        case 59: asm volatile("s_waitcnt vmcnt(59)" ::: "memory"); break;
        case 60: asm volatile("s_waitcnt vmcnt(60)" ::: "memory"); break;
        case 61: asm volatile("s_waitcnt vmcnt(61)" ::: "memory"); break;
        case 62: asm volatile("s_waitcnt vmcnt(62)" ::: "memory"); break;
        case 63: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

__device__ __forceinline__ void block_sync_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 16-byte-per-lane direct load into LDS: lane i's bytes land at dst + 16 i.
// Global address = base + vindex * stride + voffset + soffset; an out-of-range
// vindex writes zeros.
// The KV cache is streamed through once per sequence: the loads are
// non-temporal (nt), which measured faster on every workload than the default
// policy (the low-head workload at L=16K: 66.5 -> 58.5 us).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char LDS_AS* dst, unsigned vindex, unsigned voffset,
                                      int soffset) {
    __builtin_amdgcn_struct_ptr_buffer_load_lds(r, (void LDS_AS*)dst, 16, vindex, voffset, soffset, 0, /*nt*/ 2);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Buffer descriptor words (gfx9 V#): base, stride, record count, and a 32-bit
// data format so that the bounds check applies to every access; the same
// descriptor as __builtin_amdgcn_make_buffer_rsrc(base, stride, records, 0x20000).
__device__ __forceinline__ u32x4 make_rsrc_words(const void* base, int stride, unsigned num_records) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    u32x4 r;
    r[0] = (unsigned)a;
    r[1] = ((unsigned)(a >> 32) & 0xFFFFu) | ((unsigned)stride << 16);
    r[2] = num_records;
    r[3] = 0x00020000u;
    return r;
}

// One 4-byte-per-lane direct load into LDS as inline asm, raw buffer with a
// byte offset per lane (lane i's word lands at lds + 4 i; an offset past the
// record count reads 0). Same rules as dma16_asm below.
__device__ __forceinline__ void dma4_asm(const u32x4& rsrc, unsigned lds, unsigned voffset) {
    u32x4 rs;
    rs[0] = __builtin_amdgcn_readfirstlane(rsrc[0]);
    rs[1] = __builtin_amdgcn_readfirstlane(rsrc[1]);
    rs[2] = __builtin_amdgcn_readfirstlane(rsrc[2]);
    rs[3] = __builtin_amdgcn_readfirstlane(rsrc[3]);
    unsigned saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, 0 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voffset), "s"(rs));
}

// LDS byte address of an LDS pointer (what M0 takes).
__device__ __forceinline__ unsigned lds_addr(const char LDS_AS* p) { return (unsigned)(uintptr_t)p; }

// One 16-byte-per-lane direct load into LDS as inline asm, non-temporal like
// dma16 (lane i's bytes land at LDS address lds + 16 i; global address =
// base + vindex * stride + voffset + soffset; an out-of-range vindex writes
// zeros). The compiler does not see a
// memory operation here: it neither counts it in its own vmcnt bookkeeping nor
// waits for it before LDS reads it cannot prove disjoint. Callers wait with
// wait_vm (the hardware counter does count it) and order LDS reuse with
// workgroup barriers. lds and rsrc must be wave-uniform. M0 (the LDS base of
// the load) is saved and restored around it: the compiler does not honour an
// M0 clobber, so the asm leaves M0 as it found it.
__device__ __forceinline__ void dma16_asm(const u32x4& rsrc, unsigned lds, unsigned vindex, unsigned voffset,
                                          int soffset = 0) {
    typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
    const u32x2 va = {vindex, voffset};
    u32x4 rs;
    rs[0] = __builtin_amdgcn_readfirstlane(rsrc[0]);
    rs[1] = __builtin_amdgcn_readfirstlane(rsrc[1]);
    rs[2] = __builtin_amdgcn_readfirstlane(rsrc[2]);
    rs[3] = __builtin_amdgcn_readfirstlane(rsrc[3]);
    unsigned saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, %4 idxen offen nt lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(va), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(soffset)));
}

// This lane's index in the wave (0..63), computed afresh where it is used: an
// asm with no inputs is not hoisted out of a loop, so nothing derived from it
// is held (or spilled) across the tile loop.
__device__ __forceinline__ int lane_fresh() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// A wave-uniform value unchanged, but opaque to the optimiser: what is derived
// from it inside a loop is computed there, not hoisted out of the loop and
// held (and spilled) in scalar registers across it.
__device__ __forceinline__ int opaque_s(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

// The value unchanged, but opaque to the optimiser: lane-dependent addresses
// computed from it inside a loop are not hoisted out of the loop (and then
// spilled to scratch across it).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// The value of lane (this lane ^ m), 0 < m < 64, as one ds_bpermute (the
// lane id computed afresh: nothing is held across loops for it).
__device__ __forceinline__ float wave_shfl_xor(float v, int m) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane_fresh() ^ m) << 2, __float_as_int(v)));
}
// The value of lane src (0..63), as one ds_bpermute.
__device__ __forceinline__ int wave_shfl(int v, int src) { return __builtin_amdgcn_ds_bpermute(src << 2, v); }

// bf16x8 from eight floats (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5, float a6, float a7) {
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

__device__ __forceinline__ bf16x8 lds_read16(const char LDS_AS* p) { return *(const bf16x8 LDS_AS*)p; }

__device__ __forceinline__ i16x4 lds_read_tr(const char LDS_AS* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)p);
}


// acc *= alpha for an accumulator held in AGPRs. Written as inline asm on the
// AGPRs themselves so the register allocator keeps MFMA accumulators in the
// AGPR file (a VALU multiply in C++ would make it migrate them to VGPRs). The
// trailing s_nop covers the VALU-write -> MFMA-srcC hazard; the last MFMA
// that wrote acc is hundreds of cycles back (a whole QK phase).
template <typename V, int N>
__device__ __forceinline__ void scale_agpr(V& acc, float alpha) {
    #pragma unroll
    for (int e = 0; e < N; ++e) {
        float x = acc[e], t;
        asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                     : "+a"(x), "=&v"(t) : "v"(alpha));
        acc[e] = x;
    }
}


// O += V^T P^T on the AGPR-resident accumulator (v_mfma_f32_32x32x16_bf16).
// Inline asm pins the accumulator to AGPRs; the rest of the kernel's MFMAs
// use VGPR accumulators. Hazards around this asm are covered explicitly:
// callers separate it from VALU producers of its operands and from later
// AGPR reads with s_nop (mfma_fence).
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// >= 24 wait states: covers XDL-result -> VALU/accvgpr-read and VALU-write -> XDL-read hazards.
__device__ __forceinline__ void mfma_fence() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// ---------------------------------------------------------------- split partials

typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

// Split partials are stored as fp16 of o_k * 2^-e, with 2^-e chosen from the
// row's largest |o_k| (amax) so that it lands in [2^14, 2^15): fp16 keeps 11
// significant bits over that row's range, and the power of two makes the
// scaling itself exact. Returns the biased fp32 exponent field of 2^e
// (2^e = 1 for amax = 0; e never below -126).
__device__ __forceinline__ unsigned partial_exp_field(float amax) {
    if (!(amax > 0.f)) return 127u;
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 14;  // amax < 2^(field - 126)
    return (unsigned)max(e, 1);
}
// 2^e and 2^-e from that field (both normal floats: field in [1, 241])
__device__ __forceinline__ float exp_field_pow2(unsigned f) { return __uint_as_float(f << 23); }
__device__ __forceinline__ float exp_field_inv_pow2(unsigned f) { return __uint_as_float((254u - f) << 23); }

__device__ __forceinline__ f16x4 to_f16x4(float a, float b, float c, float d) {
    return f16x4{(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
}

// ---------------------------------------------------------------- segment context

struct Seg {
    int b, i, h0, limit, t_end, split, n_splits, slot, mask_rows;
    int k_cut;  // dense: first tile where rows of later positions see more tokens (else INT_MAX)
};

// Row index of token t of tile k (dense): page base from the block table.
// Returns kOOB for masked tokens.
__device__ __forceinline__ unsigned dense_row(int page_row0, int n_valid, int t) {
    return (page_row0 >= 0 && t < n_valid) ? (unsigned)(page_row0 + t) : kOOB;
}

}  // namespace dev
}  // namespace mla
