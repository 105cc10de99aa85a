// Shared device/host definitions of the gfx950 MLA decode library.
//
// Pages cited (by title, then section):
//   [Walkthrough] "矩阵、注意力与 GPU：拆解 DeepGEMM 与 FlashMLA" (msy.plus)
//   [Guide]       "FlashMLA 实战：MLA 注意力加速指南" (m.lsln.cn)
//   [ETAP]        the FlashMLA-ETAP article (ocdem.com)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kBlock = 64;          // tokens per KV page and per tile
constexpr int kDqk = 576;           // 512 latent + 64 rope ([Walkthrough] §六)
constexpr int kDv = 512;            // value = latent
constexpr int kUnits = 72;          // 16-byte units per bf16 row (1152 B)
constexpr int kTileBytes = kBlock * 1152;       // one bf16 tile in LDS (swizzled)
constexpr int kRawRow = 656;        // FP8 row ([Guide] §"FP8 缓存怎么把 KV 压掉四成")
constexpr int kRawUnits = 41;       // 656 / 16
constexpr int kRawTileBytes = kBlock * kRawRow; // one FP8 tile as stored, 41 x 1 KB
constexpr int kMaxUnits = 8192;     // row-group sequences per call (metadata LDS)
// Longest sequence a call attends (tokens): cache_seqlens entries above it are
// read as this value, max_blocks_per_seq and topk are bounded by it. With at
// most kMaxUnits sequences of at most 2^17 tiles, every schedule position
// and tile index stays below 2^31.
constexpr int kMaxSeqTokens = 1 << 23;
constexpr int kThreads = 256;       // four wave64s per workgroup

enum Variant { kV128 = 0, kV16 = 1, kV64 = 2 };
// Cache row formats (the kv_format values of include/mla.h).
enum Format { kFmtBf16 = 0, kFmtFp8 = 1, kFmtFp8Mx = 2 };

// Row-group policy; it is part of the ABI contract (see include/mla.h).
//
// The rows of a batch entry are its query rows in q's order, (position i,
// head h) -> row i * h_q + h. A dense call packs all s_q positions of a
// sequence into one row space of R = s_q * h_q rows: they attend the same
// cache, so one pass over it serves them all (row i sees the first
// L - s_q + 1 + i tokens when causal). A sparse call keeps one row space of
// h_q rows per position: each position has its own index list.
// R <= 16: 16-row groups (four waves splitting each tile's tokens);
// 16 < R <= 64: 64-row groups (two row waves x two token waves);
// R > 64: 128-row groups (four row waves, every token).
struct Layout {
    int rg;           // rows per row group
    int rows_b;       // rows of one row space: s_q * h_q (dense), h_q (sparse)
    int n_pos;        // row spaces per batch entry: 1 (dense), s_q (sparse)
    int n_hb;         // row groups per row space
    int n_rg;         // row groups per batch entry (n_pos * n_hb)
    int fixed_cost;   // schedule positions charged per row-group sequence
    int min_payload;  // minimum schedule positions per part
    int variant;
};

inline Layout layout_for(int h_q, int s_q, bool sparse) {
    Layout l;
    l.rows_b = sparse ? h_q : s_q * h_q;
    l.n_pos = sparse ? s_q : 1;
    if (l.rows_b <= 16) {
        l.rg = 16; l.fixed_cost = 0; l.min_payload = 1; l.variant = kV16;
    } else if (l.rows_b <= 64) {
        l.rg = 64; l.fixed_cost = 2; l.min_payload = 2; l.variant = kV64;
    } else {
        l.rg = 128; l.fixed_cost = 2; l.min_payload = 3; l.variant = kV128;
    }
    l.n_hb = (l.rows_b + l.rg - 1) / l.rg;
    l.n_rg = l.n_pos * l.n_hb;
    return l;
}

struct MetaParams {
    const int32_t* seqlens;
    int32_t* tile_meta;
    int32_t* split_offsets;
    int batch, n_rg, topk, num_parts, fixed_cost, min_payload;
};

struct DecodeParams {
    const uint16_t* q;          // bf16 bits [B, s_q, h_q, 576]
    const uint8_t* kv;          // [num_rows, row_bytes]
    const int32_t* block_table; // [B, mbps]
    const int32_t* seqlens;     // [B]
    const int32_t* indices;     // [B, s_q, topk]
    const int32_t* tile_meta;   // [num_parts, 8]
    const int32_t* split_offsets;
    uint16_t* ws_o;             // fp16 bits [slots, rg, 512]: partial o times 1 / ws_scale
    float* ws_lse;              // [slots, rg]
    float* ws_scale;            // [slots, rg]: power of two the stored partial row is scaled by
    uint16_t* o;                // bf16 bits [B, s_q, h_q, 512]
    float* lse;                 // [B, s_q, h_q]
    int batch, s_q, h_q, n_hb, n_rg, rg, mbps, topk, causal, num_rows, num_parts, row_bytes;
    int rows_b, n_pos;          // the row spaces (see Layout)
    float scale_log2;           // softmax_scale * log2(e)
};

// Host-side launchers (defined in the .hip files).
hipError_t launch_metadata(const MetaParams& p, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int variant, int format, bool sparse, hipStream_t s);
hipError_t launch_combine(const DecodeParams& p, int format, hipStream_t s);

}  // namespace mla
