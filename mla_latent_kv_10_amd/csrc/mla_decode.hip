// MLA decode split kernel for gfx950 (CDNA4), plus its launcher.
//
// What it computes ([Walkthrough] §六 "结果：decode 变成 MQA", §五 "公式";
// §七 "split-KV"): for each row group (RG consecutive query rows of one
// sequence: rows (position i, head h) -> i * h_q + h of all its positions
// when dense, since they all read the same cache, or the heads of one
// position when sparse) and a contiguous range of 64-token tiles, the online-
// softmax attention state (running max m, running sum l, unnormalised output
// O) over those tokens; then either the final o = O / l and lse, or the
// normalised partial (O / l, lse) for the split merge.
//
// gfx950 design (differs from the pages' Hopper designs):
//  * Tiles go HBM -> LDS with buffer_load ... lds (no VGPR staging), through a
//    structured buffer descriptor (stride = row bytes, records = cache rows):
//    each lane names its token's row; a masked token gets an out-of-range
//    index and the hardware writes zeros, so masked rows are never read.
//    Two tiles are in flight (double buffering); waits are explicit vmcnt
//    counts plus raw s_barrier, so prefetches stay outstanding. With 128-row
//    groups (and 64-row bf16 groups) the next tile's loads are spread over the
//    current tile's score MFMAs: a CU accepts an LDS-direct load only every
//    ~25 cycles, so loads issued back to back stall the waves issuing them.
//  * The bf16 tile sits in LDS as 72 chunks of 1 KB (8 tokens x 8 16-byte
//    units), with the unit index XOR-swizzled by (token/2) so that 16 lanes
//    reading 16 tokens at one unit hit 16 distinct bank groups.
//  * Scores are computed transposed, S^T = K . Q^T, with tokens on the MFMA
//    M dimension ([ETAP] §2.1-2.3 puts the long KV axis on M): each lane then
//    owns one query row, so the softmax max/sum are in-lane plus one cross-
//    half (or cross-quarter) shuffle, and P^T feeds the PV MFMA straight from
//    registers. The V operand is the transposed view of the same LDS tile,
//    read with ds_read_b64_tr_b16.
//  * FP8 rows (656 B) land raw in LDS, then every thread dequantises
//    bf16_rne(fp32(e4m3) * fp32 scale) into the bf16 tile once for all waves
//    ([Guide] §"Crossover" explains the dequant cost; on CDNA4 one workgroup
//    dequantises a tile once instead of exchanging halves between CTAs).
//    528-byte rows ([Walkthrough] §八, the V4.1 row) scale each 32 codes by a
//    power of two (a UE8M0 byte), which gfx950's scaled conversion applies
//    exactly in the same instruction that widens two codes to bf16.
//  * The running max is updated lazily: the exponent reference moves only
//    when a row's max grows by more than 2^8 (exact in real arithmetic; keeps
//    the O rescale off the common path).
#include <type_traits>

#include "mla_common.h"
#include "mla_device.h"

namespace mla {
namespace {

using namespace dev;

// A race-check build (MLA_DRAIN_PIPELINE defined) waits for every tile's loads
// right after issuing them, so each lands at the earliest point the schedule
// allows; its outputs must equal the pipelined build's bit for bit. A load
// issued into LDS that a wave may still read would show up as a difference.
#ifdef MLA_DRAIN_PIPELINE
constexpr bool kDrainPipeline = true;
#else
constexpr bool kDrainPipeline = false;
#endif

// ---------------------------------------------------------------- kernel

// MIXED (dense, causal only): some row group holds rows of more than one query
// position, so tokens between the first and the last row's causal limit are
// masked per row. A separate instantiation keeps that masking, and the scalar
// registers it holds across the tile loop, out of every other kernel.
template <int FMT, bool SPARSE, int VAR, bool MIXED>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeParams p) {
    static_assert(!(SPARSE && MIXED), "a sparse row group holds one position");
    using F = Fmt<FMT>;
    using S = Smem<FMT>;
    constexpr bool FP8 = F::kRaw;  // raw FP8 rows, dequantised in LDS
    // FP8 with 128-head groups spreads each tile's loads over the score MFMAs
    // of the tile two ahead (see the tile pipeline). Its bf16 tile and its two
    // raw tiles are separate LDS arrays; each raw array has a spare 1 KB after
    // the tile for the padding load of waves 1..3 (41 chunks over 4 waves). The
    // other variants use one array (the 64- and 16-head ones reuse all of it
    // for their end-of-segment merge).
    constexpr bool kFp8Pipe = FP8 && VAR == kV128;
    // bf16 with 128- or 64-row groups (dense or sparse) issues each tile's
    // loads between the score MFMAs of the tile before it (see the tile
    // pipeline).
    constexpr bool kQkLoads = !FP8 && (VAR == kV128 || VAR == kV64);
    // Every dense variant reads block-table words as scalar loads and issues
    // its tile loads as inline asm the compiler does not track, so that no
    // compiler wait for a load in flight lands inside the tile loop (in the
    // generic pipeline below, such a wait before the transposed V reads made
    // each tile wait for the next one's loads).
    constexpr bool kScalarIdx = !SPARSE;
    __shared__ __attribute__((aligned(1024))) char smem_raw[kFp8Pipe ? 1024 : S::kBytes];
    __shared__ __attribute__((aligned(1024))) char lds_tile[kFp8Pipe ? F::kTile : 1024];
    __shared__ __attribute__((aligned(1024))) char lds_raw0[kFp8Pipe ? F::kRawTile + 1024 : 1024];
    __shared__ __attribute__((aligned(1024))) char lds_raw1[kFp8Pipe ? F::kRawTile + 1024 : 1024];
    // sparse index words of four tiles (tile x in slot x & 3), 64 per tile
    __shared__ __attribute__((aligned(256))) int32_t lds_ring[kFp8Pipe && SPARSE ? 4 * 64 : 1];
    // per wave, a dense unit's per-row cut data (first row's limit, its
    // position, the unit's first row): kept here rather than in registers
    // across the tile loop; each wave reads only what it wrote
    __shared__ __attribute__((aligned(16))) int32_t lds_cut[4][4];
    char LDS_AS* smem = (char LDS_AS*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6) & 3;  // the & 3 tells the compiler the range (4 waves)

    // XCD-aware part numbering: hardware places workgroup x on XCD x % 8, so
    // consecutive logical parts (same sequence) share an XCD and its L2.
    int part = blockIdx.x;
    if ((gridDim.x & 7) == 0) part = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    // the part's schedule row: one scalar load of all its fields, then the
    // empty test (testing first would make the other fields a second round trip)
    typedef const int32_t __attribute__((address_space(4))) cint32_t;
    const cint32_t* tm = (const cint32_t*)p.tile_meta + (int64_t)part * 8;
    const int qb = tm[0], tb = tm[1], qe = tm[2], te = tm[3], fs = tm[4], empty = tm[5];
    if (empty) return;

    const __amdgpu_buffer_rsrc_t kv_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.kv, (short)p.row_bytes, p.num_rows, 0x00020000);

    constexpr int RG = (VAR == kV128) ? 128 : (VAR == kV64 ? 64 : 16);

    for (int qq = qb; qq <= qe; ++qq) {
        Seg sg;
        sg.b = qq / p.n_rg;
        const int rgi = qq - sg.b * p.n_rg;
        sg.i = rgi / p.n_hb;
        sg.h0 = (rgi - sg.i * p.n_hb) * RG;
        const int t0 = (qq == qb) ? tb : 0;
        // global index of the row space's row 0: rows h < rows_b of this unit
        // are q rows qrow0 + h (dense: all positions of sequence b; sparse:
        // position i of sequence b)
        const int64_t qrow0 = ((int64_t)sg.b * p.n_pos + sg.i) * p.rows_b;
        const int32_t* idx_row = SPARSE ? p.indices + ((int64_t)sg.b * p.s_q + sg.i) * p.topk : nullptr;

        // Index word of tile k: sparse -> a VMEM load, lane l holds the raw index
        // entry of token l (range-checked where the tile is issued); dense -> a
        // scalar load of the tile's page id. `kmax` bounds the block-table read;
        // words past the segment's last tile are never used.
        auto load_index = [&](int k, int kmax) -> unsigned {
            unsigned r = kOOB;
            if constexpr (SPARSE) {
                // branch-free and unchecked: the load is always issued, at a
                // position clamped into the row (topk >= 1), and its value is
                // not used here, so no wait for it lands here; tile_src drops
                // the entries past topk, and words past the segment are unused
                r = (unsigned)idx_row[min(k * kBlock + lane_fresh(), p.topk - 1)];
            } else if (k <= kmax) {
                if constexpr (kScalarIdx) {
                    // read-only for the whole kernel: a scalar load (lgkmcnt),
                    // outside the vmcnt count that tracks the tile loads
                    typedef const int32_t __attribute__((address_space(4))) cint32;
                    r = (unsigned)((cint32*)p.block_table)[(int64_t)sg.b * p.mbps + k];
                } else {
                    r = (unsigned)p.block_table[(int64_t)sg.b * p.mbps + k];
                }
            }
            return r;
        };

        // Everything that gates the first tile goes out as one batch before any
        // of it is used: the index words of tiles t0..t0+2 (bounded by the
        // block-table row, so they need not wait for the sequence length), the
        // length and split offsets, then q. The first tile's load is issued as
        // soon as its index word arrives, while q is still in flight.
        const int kmax0 = SPARSE ? (p.topk + kBlock - 1) / kBlock - 1 : p.mbps - 1;
        // Sparse, FP8, 128-head groups: the index words travel to the LDS ring
        // (every wave loads the whole slot and reads only what it loaded), so
        // no register carries a pending load across tile-loop iterations.
        // batch * s_q * topk < 2^29 (checked on the host): byte offsets fit 32 bits
        const u32x4 ix_words = make_rsrc_words(p.indices, 0, (unsigned)(p.batch * p.s_q * p.topk) * 4u);
        const int ix_row0 = ((sg.b * p.s_q + sg.i) * p.topk);
        auto ring_load = [&](int k) {
            dma4_asm(ix_words, lds_addr((const char LDS_AS*)(lds_ring + (k & 3) * 64)),
                     (unsigned)(ix_row0 + k * kBlock + lane_fresh()) * 4u);
        };
        unsigned idx_a = kOOB, idx_b = kOOB, idx_c = kOOB;
        if constexpr (kFp8Pipe && SPARSE) {
            ring_load(t0);
            ring_load(t0 + 1);
            ring_load(t0 + 2);
            // The wait before the first tile counts the VMEM loads issued
            // after these three (the NQ q loads below): no later memory
            // access may be moved above them.
            asm volatile("" ::: "memory");
        } else {
            idx_a = load_index(t0, kmax0);
            idx_b = load_index(t0 + 1, kmax0);
            idx_c = load_index(t0 + 2, kmax0);
        }
        // read-only for the whole kernel: scalar loads (lgkmcnt), so that the
        // wait for them does not also wait for the VMEM loads above
        const int len_raw = SPARSE ? 0 : ((cint32_t*)p.seqlens)[sg.b];
        const int so_raw = ((cint32_t*)p.split_offsets)[qq], so_end_raw = ((cint32_t*)p.split_offsets)[qq + 1];

        constexpr bool R32 = VAR != kV16;               // 32 rows per wave, 32x32x16 MFMA
        constexpr int NQ = R32 ? F::kDqk / 16 : F::kDqk / 32;   // k-steps over the key dims
        bf16x8 qreg[NQ];
        {
            const int ln = lane_fresh();
            int row, dsub;
            if constexpr (R32) { row = 32 * ((VAR == kV64) ? (wave >> 1) : wave) + (ln & 31); dsub = 8 * (ln >> 5); }
            else { row = ln & 15; dsub = 8 * (ln >> 4); }
            // Rows past the row space (padding of the last row group) load its
            // row 0: rows are independent and a padded row's output is never stored.
            const int h = sg.h0 + row;
            const uint16_t* qbase = p.q + qrow0 * F::kDqk;              // row 0 of the row space
            const int qoff = (h < p.rows_b ? h : 0) * F::kDqk + dsub;   // this lane's row and sub-block
            #pragma unroll
            for (int kk = 0; kk < NQ; ++kk) {
                const int dim0 = R32 ? 16 * kk : 32 * kk;
                qreg[kk] = __builtin_bit_cast(bf16x8, *(const i16x8*)(qbase + qoff + dim0));
            }
            // issue the q loads here, before the waits for the length and the
            // index words below (left to itself the compiler sinks them past
            // the test for an empty segment, behind that wait)
            asm volatile("" ::: "memory");
        }

        int T_q;
        if (SPARSE) {
            T_q = (p.topk + kBlock - 1) / kBlock;
            sg.limit = p.topk;
            sg.k_cut = 0x7fffffff;
        } else {
            const int L = min(uniform(len_raw), kMaxSeqTokens);  // as the schedule reads it
            T_q = L > 0 ? (L + kBlock - 1) / kBlock : 0;
            // causal: position i sees L - s_q + 1 + i tokens. The unit's rows
            // span positions pos_lo .. pos_hi (one position unless dense rows
            // pack several); the tiles run to the last row's limit and
            // tokens between the first and last row's limits are masked per row.
            int pos_lo = sg.i, pos_hi = sg.i;
            if (p.n_pos == 1) {
                pos_lo = sg.h0 / p.h_q;
                pos_hi = (min(sg.h0 + RG, p.rows_b) - 1) / p.h_q;
            }
            const int cap = min(L, p.mbps * kBlock);
            sg.limit = max(min(p.causal ? L - p.s_q + 1 + pos_hi : L, cap), 0);
            const int lim_lo = max(min(p.causal ? L - p.s_q + 1 + pos_lo : L, cap), 0);
            sg.k_cut = 0x7fffffff;
            if (MIXED && lim_lo != sg.limit) {
                sg.k_cut = lim_lo / kBlock;   // first tile with tokens past the first row's limit
                // the first row's causal limit before clamping: below 0 when
                // L < s_q - 1 - pos_lo, so that the rows of positions that see
                // no token stay fully masked (their limit + offset is <= 0)
                lds_cut[wave][0] = L - p.s_q + 1 + pos_lo;
                lds_cut[wave][1] = pos_lo;
                lds_cut[wave][2] = sg.h0;
            }
        }
        int t1 = (qq == qe) ? te : T_q - 1;
        sg.split = (qq == qb) ? fs : 0;
        const int so = uniform(so_raw);
        sg.n_splits = uniform(so_end_raw) - so;
        sg.slot = so + sg.split;
        const int t_eff = (sg.limit + kBlock - 1) / kBlock;  // tiles holding any attended token
        t1 = min(t1, t_eff - 1);
        sg.t_end = t1;

        // ------------------------------------------------ per-segment state
        // Index words of later tiles (three tiles ahead of use).
        auto fetch_index = [&](int k) -> unsigned { return load_index(k, t1); };
        // Dense: row of token 0 of tile k, or -1 when the page id is invalid.
        auto dense_page_row0 = [&](unsigned blk_bits) -> int {
            const int blk = uniform((int)blk_bits);
            return (blk >= 0 && (int64_t)blk * kBlock < (int64_t)p.num_rows) ? blk * kBlock : -1;
        };

        const u32x4 kv_words = make_rsrc_words(p.kv, p.row_bytes, (unsigned)p.num_rows);
        // One 1 KB chunk of a tile into LDS: dense -> untracked asm load (see
        // kScalarIdx); sparse -> the builtin (its index words are VMEM loads
        // held in registers, which the compiler must be able to count).
        auto tile_load = [&](char LDS_AS* dst, unsigned row, unsigned voff, int soff) {
            if constexpr (!SPARSE) dma16_asm(kv_words, lds_addr(dst), row, voff, soff);
            else dma16(kv_rsrc, dst, row, voff, soff);
        };

        // Where tile k's rows come from, given its index word: dense -> the
        // page's first cache row and the attended token count; sparse -> each
        // lane's (token's) validated cache row. mask: bit t set = token t attended.
        struct TileSrc {
            int page0, n_valid;
            unsigned srow;
            uint64_t mask;
        };
        auto tile_src = [&](int k, unsigned word) -> TileSrc {
            TileSrc ts{0, 0, kOOB, 0ull};
            if (!SPARSE) {
                ts.page0 = dense_page_row0(word);
                ts.n_valid = min(kBlock, sg.limit - k * kBlock);
                ts.mask = (ts.page0 < 0 || ts.n_valid <= 0) ? 0ull
                          : (ts.n_valid >= 64 ? ~0ull : ((1ull << ts.n_valid) - 1ull));
            } else {
                const bool in_row = k * kBlock + lane_fresh() < p.topk;  // ring words past topk belong to other rows
                ts.srow = (in_row && (int)word >= 0 && (int)word < p.num_rows) ? word : kOOB;  // -1, out of range
                ts.mask = __builtin_amdgcn_ballot_w64(ts.srow != kOOB);
            }
            return ts;
        };
        // Issue the loads of tile k into LDS region `dst` back to back (the
        // two-tiles-ahead pipeline: 16-row groups, FP8 64-row groups); returns
        // the tile's validity mask. The
        // number of VMEM instructions per wave is fixed per variant (n_dma).
        // UNROLL: straight-line issue (the prologue).
        auto issue_tile = [&](auto unroll_tag, int k, char LDS_AS* dst, unsigned word) -> uint64_t {
            constexpr bool UNROLL = decltype(unroll_tag)::value;
            const TileSrc ts = tile_src(k, word);
            const int page0 = ts.page0, n_valid = ts.n_valid;
            const unsigned srow = ts.srow;
            const uint64_t mask = ts.mask;
            const int w = opaque_s(wave) & 3;  // chunk geometry computed per tile, not held across the loop
            if (!FP8) {
                // 72 chunks, 18 per wave: token groups 2w, 2w+1; unit groups 0..8.
                auto group = [&](int g) {
                    // lane geometry recomputed here (not hoisted and spilled: a
                    // scratch reload would make the issue wait for q)
                    const int ln = lane_fresh();
                    const int tg = 2 * w + g;
                    const int t = tg * 8 + (ln >> 3);
                    const int uu = (ln & 7) ^ ((t >> 1) & 7);
                    unsigned row;
                    if (SPARSE) row = (unsigned)wave_shfl((int)srow, t);
                    else row = dense_row(page0, n_valid, t);
                    if constexpr (UNROLL) {
                        #pragma unroll
                        for (int ug = 0; ug < F::kUg; ++ug)
                            tile_load(dst + ((tg * F::kUg + ug) << 10), row, (unsigned)(uu << 4), ug * 128);
                    } else {
                        #pragma unroll 1
                        for (int ug = 0; ug < F::kUg; ++ug)
                            tile_load(dst + ((tg * F::kUg + ug) << 10), row, (unsigned)(uu << 4), ug * 128);
                    }
                };
                if constexpr (UNROLL) {
                    group(0);
                    group(1);
                } else {
                    #pragma unroll 1
                    for (int g = 0; g < 2; ++g) group(g);
                }
            } else {
                // kRawUnits (41 or 33) chunks of the raw tile image, chunk c
                // to wave c % 4. Chunk c holds 16-byte units kk = 64 c + lane of
                // the image: token kk / kRawUnits, unit kk % kRawUnits. From chunk
                // c to c + 4, kk grows by 256 = kStepT * kRawUnits + kStepU, so
                // (token, unit) step without a division.
                constexpr int kStepT = 256 / F::kRawUnits, kStepU = 256 % F::kRawUnits;
                const int kk0 = 64 * w + lane_fresh();
                int t = (int)(((unsigned)kk0 * F::kDivMagic) >> 16);  // kk0 / kRawUnits
                int u = kk0 - t * F::kRawUnits;
                auto chunk = [&](int c) {
                    unsigned row;
                    if (SPARSE) row = (unsigned)wave_shfl((int)srow, t);
                    else row = dense_row(page0, n_valid, t);
                    tile_load(dst + (c << 10), row, (unsigned)(u << 4), 0);
                    u += kStepU;
                    t += kStepT;
                    if (u >= F::kRawUnits) { u -= F::kRawUnits; t += 1; }
                };
                if constexpr (UNROLL) {
                    #pragma unroll
                    for (int j = 0; j < F::kRawUnits / 4; ++j) chunk(w + 4 * j);
                    if (w < F::kRawUnits % 4) chunk(w + 4 * (F::kRawUnits / 4));
                } else {
                    #pragma unroll 1
                    for (int c = w; c < F::kRawUnits; c += 4) chunk(c);
                }
            }
            return mask;
        };
        const int n_dma = FP8 ? (wave < F::kRawUnits % 4 ? F::kRawUnits / 4 + 1 : F::kRawUnits / 4) : 18;

        // FP8, 128-head groups: chunk slot j (0 .. kRawSlots - 1) of a tile's
        // raw image; chunk c = wave + 4 j holds 16-byte units kk = 64 c + lane
        // (token kk / kRawUnits, unit kk % kRawUnits). Branch-free, so it can
        // sit between MFMAs: a wave whose last slot is past the image loads
        // nothing into the spare 1 KB after the tile instead, and a tile past
        // the segment (no rows) loads nothing.
        struct ChunkAddr {
            unsigned row, voff;
        };
        auto chunk_addr = [&](int j, const TileSrc& ts) -> ChunkAddr {
            const int c = (opaque_s(wave) & 3) + 4 * j;
            const int kk = 64 * c + lane_fresh();
            const int t = (int)(__umul24((unsigned)kk, F::kDivMagic) >> 16);  // kk / kRawUnits
            const int u = kk - (int)__umul24((unsigned)t, (unsigned)F::kRawUnits);
            unsigned row;
            if (SPARSE) {
                // the chunk's 64 units span tokens tA .. tA + 2
                const int tA = uniform((int)(((unsigned)(64 * c) * F::kDivMagic) >> 16));
                const unsigned rA = (unsigned)__builtin_amdgcn_readlane((int)ts.srow, min(tA, 63));
                const unsigned rB = (unsigned)__builtin_amdgcn_readlane((int)ts.srow, min(tA + 1, 63));
                const unsigned rC = (unsigned)__builtin_amdgcn_readlane((int)ts.srow, min(tA + 2, 63));
                row = t == tA ? rA : (t == tA + 1 ? rB : rC);
            } else {
                row = dense_row(ts.page0, ts.n_valid, t);
            }
            return ChunkAddr{c < F::kRawUnits ? row : kOOB, (unsigned)(u << 4)};
        };
        auto chunk_issue = [&](int j, char LDS_AS* dst, const ChunkAddr& a) {
            const int c = (opaque_s(wave) & 3) + 4 * j;
            dma16_asm(kv_words, lds_addr(dst + ((c < F::kRawUnits ? c : F::kRawUnits) << 10)), a.row, a.voff);
        };
        auto raw_chunk = [&](int j, char LDS_AS* dst, const TileSrc& ts) { chunk_issue(j, dst, chunk_addr(j, ts)); };

        // Dequantise raw FP8 tile `raw` into the bf16 tile at `tile`. Lane l
        // handles token l; wave w handles raw code units w, w+4, .., w+28
        // (16 codes each; bf16 units 2u, 2u+1) and, for 656-byte rows, rope
        // units w, w+4. All LDS reads are issued before any conversion.
        const int dq_x = (lane >> 1) & 7;  // swizzle of token `lane`
        const int dq_base = ((lane >> 3) * F::kUg << 10) + ((lane & 7) << 7);
        const int dq_c0 = (((2 * wave) ^ dq_x) & 7) << 4;      // unit 2*(w+4j) & 7 == 2w
        const int dq_c1 = (((2 * wave + 1) ^ dq_x) & 7) << 4;
        auto dequant = [&](const char LDS_AS* raw, char LDS_AS* tile) {
            const char LDS_AS* rrow = raw + lane * F::kRawRow;
            if constexpr (F::kMx) {
                // 528-byte rows: code unit u (values 16u .. 16u + 15) takes
                // the UE8M0 scale byte 512 + u / 2 (blocks of 32 values). The
                // scaled conversion multiplies by 2^(byte - 127) exactly: the
                // fp32 operand's exponent field is the byte itself.
                u32x4 c[8];
                #pragma unroll
                for (int j = 0; j < 8; ++j) c[j] = *(const u32x4 LDS_AS*)(rrow + (wave + 4 * j) * 16);
                const u32x4 e4 = *(const u32x4 LDS_AS*)(rrow + 512);
                #pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int blk = 2 * j + (wave >> 1);               // (wave + 4 j) / 2
                    const unsigned eb = (e4[j >> 1] >> (8 * (blk & 3))) & 0xFFu;
                    const float sc = __uint_as_float(eb << 23);
                    u32x4 w0, w1;
                    #pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j][d], sc, false);
                        const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[j][d], sc, true);
                        const unsigned a = __builtin_bit_cast(unsigned, lo), b = __builtin_bit_cast(unsigned, hi);
                        if (d < 2) { w0[2 * d] = a; w0[2 * d + 1] = b; }
                        else { w1[2 * d - 4] = a; w1[2 * d - 3] = b; }
                    }
                    char LDS_AS* dst = tile + dq_base + (j << 10);
                    *(u32x4 LDS_AS*)(dst + dq_c0) = w0;
                    *(u32x4 LDS_AS*)(dst + dq_c1) = w1;
                }
                return;
            }
            u32x4 c[8], rp[2];
            #pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = *(const u32x4 LDS_AS*)(rrow + (wave + 4 * j) * 16);
            const f32x4 sc4 = *(const f32x4 LDS_AS*)(rrow + 512);
            #pragma unroll
            for (int j = 0; j < 2; ++j) rp[j] = *(const u32x4 LDS_AS*)(rrow + 528 + (wave + 4 * j) * 16);
            #pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float sc = sc4[j >> 1];  // unit w + 4j lies in scale group (w + 4j) / 8 == j / 2
                float v[16];
                #pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[j][d], false);
                    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[j][d], true);
                    v[4 * d + 0] = lo[0] * sc; v[4 * d + 1] = lo[1] * sc;
                    v[4 * d + 2] = hi[0] * sc; v[4 * d + 3] = hi[1] * sc;
                }
                char LDS_AS* dst = tile + dq_base + (j << 10);
                *(bf16x8 LDS_AS*)(dst + dq_c0) = pack8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]);
                *(bf16x8 LDS_AS*)(dst + dq_c1) = pack8(v[8], v[9], v[10], v[11], v[12], v[13], v[14], v[15]);
            }
            #pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int u = 64 + wave + 4 * j;
                *(u32x4 LDS_AS*)(tile + dq_base + (8 << 10) + ((((u & 7) ^ dq_x) & 7) << 4)) = rp[j];
            }
        };

        // ------------------------------------------------ compute state
        // V128: wave owns rows 32*wave + (lane & 31); all 64 tokens of a tile.
        // V64 : wave owns rows 32*rw + (lane & 31) and tokens 32*tw .. +31 of
        //       each tile (rw = wave >> 1, tw = wave & 1).
        // V16 : wave owns tokens 16*wave .. +15 of each tile; all 16 rows.
        constexpr int NB = (VAR == kV128) ? 2 : 1;      // 32-token blocks per wave per tile
        const int rw = (VAR == kV64) ? (wave >> 1) : wave;
        const int tw = (VAR == kV64) ? (wave & 1) : 0;
        constexpr int NO = R32 ? F::kDv / 32 : F::kDv / 16;   // output blocks over the value dims
        typedef typename std::conditional<R32, f32x16, f32x4>::type Acc;
        Acc oacc[NO];
        #pragma unroll
        for (int d = 0; d < NO; ++d) oacc[d] = Acc{};
        float m_run = -INFINITY;  // exponent reference (log2 units), per row
        float l_run = 0.f;        // partial sum of p over this lane's tokens

        // Per-lane LDS offsets (see the layout derivation in the comments).
        int koff[2][4];   // 32-row variants: [token block][k-step & 3]; V16 uses koff[0][0..1]
        int voff[4];      // 32-row variants: [lohi*2 + (d&1)]; V16: [d&3]
        if constexpr (R32) {
            const int hh = lane >> 5;
            #pragma unroll
            for (int blk = 0; blk < NB; ++blk) {
                const int t = 32 * (VAR == kV128 ? blk : tw) + (lane & 31);
                const int base = ((t >> 3) * F::kUg << 10) + ((t & 7) << 7);
                const int x = (t >> 1) & 7;
                #pragma unroll
                for (int j = 0; j < 4; ++j) koff[blk][j] = base + ((((2 * j + hh) ^ x) & 7) << 4);
            }
            const int q16 = lane >> 4, r = (lane >> 2) & 3, c4 = lane & 3;
            #pragma unroll
            for (int lohi = 0; lohi < 2; ++lohi) {
                #pragma unroll
                for (int dp = 0; dp < 2; ++dp) {
                    const int tt = 4 * hh + r;                          // token & 7
                    const int x = (4 * lohi + 2 * hh + (r >> 1)) & 7;   // (token >> 1) & 7
                    const int u7 = 4 * dp + 2 * (q16 & 1) + (c4 >> 1);  // unit & 7
                    voff[lohi * 2 + dp] = (((tt << 3) | (u7 ^ x)) << 4) + 8 * (c4 & 1);
                }
            }
        } else {
            const int g = lane >> 4;
            const int t = 16 * wave + (lane & 15);
            #pragma unroll
            for (int j = 0; j < 2; ++j)
                koff[0][j] = ((t >> 3) * F::kUg << 10) + ((((t & 7) << 3) | (((4 * j + g) ^ ((t >> 1) & 7)) & 7)) << 4);
            koff[1][0] = koff[1][1] = koff[1][2] = koff[1][3] = koff[0][2] = koff[0][3] = 0;
            const int r = (lane >> 2) & 3, c4 = lane & 3;
            const int tv = 16 * wave + 4 * g + r;
            #pragma unroll
            for (int dq = 0; dq < 4; ++dq) {
                const int u7 = 2 * dq + (c4 >> 1);
                voff[dq] = ((tv >> 3) * F::kUg << 10) + ((((tv & 7) << 3) | ((u7 ^ ((tv >> 1) & 7)) & 7)) << 4) + 8 * (c4 & 1);
            }
        }

        // ------------------------------------------------ compute one tile
        // Side work between the score MFMAs (tile loads; see the tile
        // pipeline): side(j), j = 0 .. NQ/2 - 1, after the MFMAs of k-step 2 j
        // (j < NQ/2 - 1) or NQ - 3 (the last j), when the tag is true.
        // Row r's token limit relative to tile k, in a dense unit whose rows
        // span positions: the first row's limit plus r's position offset.
        auto row_cut = [&](int k, int r) -> int {
            const int lim_lo = uniform(lds_cut[wave][0]), pos_lo = uniform(lds_cut[wave][1]);
            const int h0 = uniform(lds_cut[wave][2]);
            return lim_lo - k * kBlock + (h0 + r) / p.h_q - pos_lo;
        };
        auto compute_tile = [&](const char LDS_AS* tile, uint64_t mask, int k, auto side_tag, auto&& side) {
            constexpr bool kSideQk = decltype(side_tag)::value;
            if constexpr (R32) {
                // S^T = K Q^T on 32x32x16 MFMAs: two accumulation chains (the two
                // token blocks for V128; even/odd k-steps of the one block for V64).
                f32x16 sc[2] = {f32x16{}, f32x16{}};
                constexpr int kPF = (NB == 2) ? 2 : 4;
                bf16x8 ka[kPF + 1][NB];
                #pragma unroll
                for (int j = 0; j < kPF; ++j)
                    #pragma unroll
                    for (int bb = 0; bb < NB; ++bb) ka[j][bb] = lds_read16(tile + koff[bb][j & 3] + ((j >> 2) << 10));
                #pragma unroll
                for (int kk = 0; kk < NQ; ++kk) {
                    const int nk = kk + kPF;
                    if (nk < NQ) {
                        #pragma unroll
                        for (int bb = 0; bb < NB; ++bb)
                            ka[nk % (kPF + 1)][bb] = lds_read16(tile + koff[bb][nk & 3] + ((nk >> 2) << 10));
                    }
                    #pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        const int ch = (NB == 2) ? bb : (kk & 1);
                        sc[ch] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % (kPF + 1)][bb], qreg[kk], sc[ch], 0, 0, 0);
                    }
                    if constexpr (kSideQk) {
                        if (kk < NQ - 3 && kk % 2 == 0) side(kk / 2);
                        else if (kk == NQ - 3) side(NQ / 2 - 1);
                    }
                }
                // keep the read-ahead: reads first, then (NB MFMA, NB reads) groups
                __builtin_amdgcn_sched_group_barrier(0x100, NB * kPF, 0);
                #pragma unroll
                for (int kk = 0; kk < NQ - kPF; ++kk) {
                    __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, NB, 0);
                    if constexpr (kSideQk) {
                        if ((kk < NQ - 3 && kk % 2 == 0) || kk == NQ - 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    }
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NB * kPF, 0);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (NB == 1) sc[0] += sc[1];
                // lane holds row (lane&31), token 32*tb + 8*(v>>2) + 4*(lane>>5) + (v&3)
                const int hh = lane >> 5;
                #pragma unroll
                for (int bb = 0; bb < NB; ++bb)
                    #pragma unroll
                    for (int v = 0; v < 16; ++v) sc[bb][v] *= p.scale_log2;
                if (mask != ~0ull) {
                    const uint64_t mh = mask >> (4 * (lane_fresh() >> 5));  // this lane's token half
                    #pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        const int tb = (VAR == kV128) ? bb : tw;
                        #pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int t = 32 * tb + 8 * (v >> 2) + (v & 3);
                            if (!((mh >> t) & 1ull)) sc[bb][v] = -INFINITY;
                        }
                    }
                }
                // a causal dense unit whose rows span positions: tokens past
                // the first position's limit are masked per row
                if (MIXED && k >= sg.k_cut) {
                    const int ln2 = lane_fresh();
                    const int rcut = row_cut(k, 32 * rw + (ln2 & 31)) - 4 * (ln2 >> 5);
                    #pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        const int tb = (VAR == kV128) ? bb : tw;
                        #pragma unroll
                        for (int v = 0; v < 16; ++v)
                            if (32 * tb + 8 * (v >> 2) + (v & 3) >= rcut) sc[bb][v] = -INFINITY;
                    }
                }
                float mt = sc[0][0];
                #pragma unroll
                for (int bb = 0; bb < NB; ++bb)
                    #pragma unroll
                    for (int v = 0; v < 16; ++v) mt = fmaxf(mt, sc[bb][v]);
                mt = fmaxf(mt, wave_shfl_xor(mt, 32));
                const bool need = mt > m_run + kLazyMax;
                if (__builtin_amdgcn_ballot_w64(need)) {
                    const float m_new = fmaxf(m_run, mt);
                    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                    // rows with nothing accumulated yet hold O = 0: skip the scaling
                    if (__builtin_amdgcn_ballot_w64(m_run != -INFINITY)) {
                        l_run *= alpha;
                        #pragma unroll
                        for (int d = 0; d < NO; ++d) scale_agpr<f32x16, 16>(oacc[d], alpha);
                        asm volatile("s_nop 2" ::: "memory");
                    }
                    m_run = m_new;
                }
                const float mu = (m_run == -INFINITY) ? 0.f : m_run;
                float ps = 0.f;
                #pragma unroll
                for (int bb = 0; bb < NB; ++bb)
                    #pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        sc[bb][v] = __builtin_amdgcn_exp2f(sc[bb][v] - mu);
                        ps += sc[bb][v];
                    }
                l_run += ps;
                bf16x8 pb[2 * NB];
                #pragma unroll
                for (int bb = 0; bb < NB; ++bb)
                    #pragma unroll
                    for (int c = 0; c < 2; ++c)
                        pb[2 * bb + c] = pack8(sc[bb][8 * c + 0], sc[bb][8 * c + 1], sc[bb][8 * c + 2], sc[bb][8 * c + 3],
                                               sc[bb][8 * c + 4], sc[bb][8 * c + 5], sc[bb][8 * c + 6], sc[bb][8 * c + 7]);
                __builtin_amdgcn_sched_barrier(0);
                // V operands (transposed reads) kVF MFMAs ahead; c = the tile's 16-token chunk
                constexpr int kVF = 3;
                constexpr int NPV = NO * 2 * NB;   // (16-token chunk, 32-dim block) pairs
                auto vread = [&](int n) -> bf16x8 {
                    const int cl = n / NO, d = n % NO;
                    const int c = (VAR == kV128) ? cl : 2 * tw + cl;
                    const i16x4 lo = lds_read_tr(tile + voff[d & 1] + (((2 * c) * F::kUg + (d >> 1)) << 10));
                    const i16x4 hi = lds_read_tr(tile + voff[2 + (d & 1)] + (((2 * c + 1) * F::kUg + (d >> 1)) << 10));
                    const i16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    return __builtin_bit_cast(bf16x8, av);
                };
                bf16x8 va[kVF + 1];
                #pragma unroll
                for (int j = 0; j < kVF; ++j) va[j] = vread(j);
                mfma_fence();  // pb (VALU) -> MFMA operand
                #pragma unroll
                for (int n = 0; n < NPV; ++n) {
                    if (n + kVF < NPV) va[(n + kVF) % (kVF + 1)] = vread(n + kVF);
                    const int cl = n / NO, d = n % NO;
                    mfma32_agpr(oacc[d], va[n % (kVF + 1)], pb[cl]);
                }
                mfma_fence();  // MFMA results -> later AGPR reads / scaling
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVF, 0);
                #pragma unroll
                for (int n = 0; n < NPV - kVF; ++n) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, kVF, 0);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                f32x4 s = {};
                constexpr int kPF = 3;
                bf16x8 ka[kPF + 1];
                #pragma unroll
                for (int j = 0; j < kPF; ++j) ka[j] = lds_read16(tile + koff[0][j & 1] + ((j >> 1) << 10));
                #pragma unroll
                for (int kk = 0; kk < NQ; ++kk) {
                    const int nk = kk + kPF;
                    if (nk < NQ) ka[nk % (kPF + 1)] = lds_read16(tile + koff[0][nk & 1] + ((nk >> 1) << 10));
                    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk % (kPF + 1)], qreg[kk], s, 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, kPF, 0);
                #pragma unroll
                for (int kk = 0; kk < NQ - kPF; ++kk) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, kPF, 0);
                __builtin_amdgcn_sched_barrier(0);
                // lane holds row (lane&15), tokens 16*wave + 4*(lane>>4) + v
                const int g = lane >> 4;
                float x[4];
                #pragma unroll
                for (int v = 0; v < 4; ++v) {
                    x[v] = s[v] * p.scale_log2;
                    const int t = 16 * wave + 4 * g + v;
                    if (!((mask >> t) & 1ull)) x[v] = -INFINITY;
                }
                // a causal dense unit whose rows span positions: tokens past
                // the first position's limit are masked per row
                if (MIXED && k >= sg.k_cut) {
                    const int rcut = row_cut(k, lane_fresh() & 15);
                    #pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (16 * wave + 4 * g + v >= rcut) x[v] = -INFINITY;
                }
                float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
                mt = fmaxf(mt, wave_shfl_xor(mt, 16));
                mt = fmaxf(mt, wave_shfl_xor(mt, 32));
                const bool need = mt > m_run + kLazyMax;
                if (__builtin_amdgcn_ballot_w64(need)) {
                    const float m_new = fmaxf(m_run, mt);
                    const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                    if (__builtin_amdgcn_ballot_w64(m_run != -INFINITY)) {
                        l_run *= alpha;
                        #pragma unroll
                        for (int d = 0; d < NO; ++d) scale_agpr<f32x4, 4>(oacc[d], alpha);
                        asm volatile("s_nop 2" ::: "memory");
                    }
                    m_run = m_new;
                }
                const float mu = (m_run == -INFINITY) ? 0.f : m_run;
                #pragma unroll
                for (int v = 0; v < 4; ++v) { x[v] = __builtin_amdgcn_exp2f(x[v] - mu); l_run += x[v]; }
                const bf16x8 pb = pack8(x[0], x[1], x[2], x[3], 0.f, 0.f, 0.f, 0.f);
                __builtin_amdgcn_sched_barrier(0);
                constexpr int kVF = 4;
                i16x4 va[kVF + 1];
                #pragma unroll
                for (int j = 0; j < kVF; ++j) va[j] = lds_read_tr(tile + voff[j & 3] + ((j >> 2) << 10));
                #pragma unroll
                for (int d = 0; d < NO; ++d) {
                    if (d + kVF < NO) va[(d + kVF) % (kVF + 1)] = lds_read_tr(tile + voff[(d + kVF) & 3] + (((d + kVF) >> 2) << 10));
                    const i16x4 lo = va[d % (kVF + 1)];
                    const i16x8 av = {lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
                    oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb, oacc[d], 0, 0, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, kVF, 0);
                #pragma unroll
                for (int d = 0; d < NO - kVF; ++d) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, kVF, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // ------------------------------------------------ tile pipeline
        if constexpr (kFp8Pipe) {
          if (t0 <= t1) {
            // Tile k: wait for its raw image, dequantise it into the bf16 tile,
            // then compute it while tile k + 2's loads (into the raw buffer just
            // dequantised) go out between its score MFMAs, one every two
            // k-steps per wave: a CU takes an LDS-direct load every ~25 cycles,
            // so loads issued back to back stall the issuing waves, but spread
            // this way they do not. (Between the PV MFMAs instead: 2 % slower.)
            char LDS_AS* tile = (char LDS_AS*)lds_tile;
            char LDS_AS* raw0 = (char LDS_AS*)lds_raw0;
            char LDS_AS* raw1 = (char LDS_AS*)lds_raw1;
            const TileSrc none{-1, 0, kOOB, 0ull};
            // index word of tile k (sparse: from the ring, its load complete)
            auto word_of = [&](int k, unsigned reg) -> unsigned {
                if constexpr (SPARSE) return (unsigned)lds_ring[(k & 3) * 64 + lane];
                else return reg;
            };
            if constexpr (SPARSE) wait_vm(NQ);  // the ring loads of t0..t0+2 (older than the split offsets and the NQ q loads)
            TileSrc ts = tile_src(t0, word_of(t0, idx_a));
            uint64_t mask_a = ts.mask, mask_b = 0;
            #pragma unroll
            for (int j = 0; j < F::kRawSlots; ++j) raw_chunk(j, raw0, ts);
            if constexpr (kDrainPipeline) wait_vm(0);
            if (t0 + 1 <= t1) {
                ts = tile_src(t0 + 1, word_of(t0 + 1, idx_b));
                mask_b = ts.mask;
                #pragma unroll
                for (int j = 0; j < F::kRawSlots; ++j) raw_chunk(j, raw1, ts);
                if constexpr (kDrainPipeline) wait_vm(0);
            }
            // q was loaded before these tiles: have it in registers here. (The
            // compiler does not see the tile loads, so its wait for q also
            // waits for them: once per segment. Issuing tile t0 + 1 after that
            // wait measured no faster here.)
            #pragma unroll
            for (int kk = 0; kk < NQ; ++kk) asm volatile("" ::"v"(qreg[kk]));
            for (int k = t0; k <= t1; ++k) {
                char LDS_AS* cur = ((k - t0) & 1) ? raw1 : raw0;
                unsigned idx_d = kOOB;
                if constexpr (SPARSE) ring_load(k + 3);  // always issued: a fixed count per iteration
                else idx_d = fetch_index(k + 3);
                // VMEM instructions issued after tile k's loads: tile k + 1's
                // (kRawSlots; in the prologue only if that tile exists), and for
                // the sparse index the ring loads of tiles k + 2 and k + 3 (dense
                // index words are scalar loads).
                int after;
                if (k == t0) after = (k + 1 <= t1 ? F::kRawSlots : 0) + (SPARSE ? 1 : 0);
                else after = F::kRawSlots + (SPARSE ? 2 : 0);
                wait_vm(after);
                block_sync_lds();
                dequant(cur, tile);
                block_sync_lds();
                // sparse: the ring load of tile k + 2 (followed by tile k + 1's
                // loads and the ring load of k + 3); at k = t0 it is already in
                if (SPARSE && k > t0) wait_vm(F::kRawSlots + 1);
                const TileSrc tn = (k + 2 <= t1) ? tile_src(k + 2, word_of(k + 2, idx_c)) : none;
                // chunk j is issued with the address computed after chunk j - 1,
                // so its VALU fills the MFMA slots between the two loads
                ChunkAddr ca = chunk_addr(0, tn);
                compute_tile(tile, mask_a, k, std::true_type{}, [&](int j) {
                    if (j < F::kRawSlots) {
                        chunk_issue(j, cur, ca);
                        if (kDrainPipeline && j == F::kRawSlots - 1) wait_vm(0);
                        if (j + 1 < F::kRawSlots) ca = chunk_addr(j + 1, tn);
                    }
                });
                idx_a = idx_b; idx_b = idx_c; idx_c = idx_d;
                mask_a = mask_b; mask_b = tn.mask;
            }
            wait_vm(0);        // the loads for tiles past the segment have landed
            block_sync_lds();  // every wave is done with the tiles before LDS is reused
          }
        } else if constexpr (kQkLoads) {
          if (t0 <= t1) {
            // Tile k + 1's loads go out between tile k's score MFMAs (one per
            // two k-steps per wave, ~one per 32 cycles per CU) into the other
            // buffer, which held tile k - 1 (every wave is past it at the
            // barrier). Issued back to back after the tile they block the waves
            // for ~1800 cycles (a CU accepts an LDS-direct load every ~25).
            char LDS_AS* buf0 = smem + S::kTileA;
            char LDS_AS* buf1 = smem + S::kTileB;
            const TileSrc none{-1, 0, kOOB, 0ull};
            // lane geometry of this wave's chunks: token groups tg = 2w + g
            const int ln = lane_fresh();
            int trow[2], uu16[2];
            #pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int t = (2 * wave + g) * 8 + (ln >> 3);
                trow[g] = t;
                uu16[g] = ((ln & 7) ^ ((t >> 1) & 7)) << 4;
            }
            // chunk j of a tile: token group g = j / 9, unit group ug = j % 9
            auto qk_chunk = [&](int j, char LDS_AS* dst, const unsigned (&rows)[2]) {
                const int g = j / 9, ug = j % 9;
                dma16_asm(kv_words, lds_addr(dst + (((2 * (opaque_s(wave) & 3) + g) * 9 + ug) << 10)), rows[g], (unsigned)uu16[g], ug * 128);
            };
            // each chunk's cache row: dense -> from the page; sparse -> the
            // index entry of the chunk's token, held by the lane of that token
            auto tile_rows = [&](const TileSrc& tsrc, unsigned (&rows)[2]) {
                #pragma unroll
                for (int g = 0; g < 2; ++g) {
                    if constexpr (SPARSE) rows[g] = (unsigned)wave_shfl((int)tsrc.srow, trow[g]);
                    else rows[g] = dense_row(tsrc.page0, tsrc.n_valid, trow[g]);
                }
            };
            TileSrc ts = tile_src(t0, idx_a);
            uint64_t mask_a = ts.mask;
            unsigned rows0[2];
            tile_rows(ts, rows0);
            #pragma unroll
            for (int j = 0; j < 18; ++j) qk_chunk(j, buf0, rows0);
            if constexpr (kDrainPipeline) wait_vm(0);
            // q was loaded before the tile: have it in registers here.
            #pragma unroll
            for (int kk = 0; kk < NQ; ++kk) asm volatile("" ::"v"(qreg[kk]));
            unsigned idx_n = idx_b;  // index word of tile k + 1
            for (int k = t0; k <= t1; ++k) {
                char LDS_AS* cur = ((k - t0) & 1) ? buf1 : buf0;
                char LDS_AS* nxt = ((k - t0) & 1) ? buf0 : buf1;
                // index word of tile k + 2: dense -> a scalar load, issued early;
                // sparse -> a VMEM load, issued after the wait below so that the
                // wait never includes it (it has a whole tile to land)
                unsigned idx_f = kOOB;
                if constexpr (!SPARSE) idx_f = fetch_index(k + 2);
                wait_vm(0);        // tile k's loads (and a sparse index word) are all the VMEM in flight
                block_sync_lds();  // ... and every wave is done with nxt (tile k - 1)
                if constexpr (SPARSE) idx_f = fetch_index(k + 2);
                const TileSrc tn = (k + 1 <= t1) ? tile_src(k + 1, idx_n) : none;
                unsigned rows[2];
                tile_rows(tn, rows);
                compute_tile(cur, mask_a, k, std::true_type{}, [&](int j) {
                    qk_chunk(j, nxt, rows);
                    if (kDrainPipeline && j == 17) wait_vm(0);
                });
                mask_a = tn.mask;
                idx_n = idx_f;
            }
            wait_vm(0);        // the loads for a tile past the segment have landed
            block_sync_lds();  // every wave is done with the tiles before LDS is reused
          }
        } else if (t0 <= t1) {
            char LDS_AS* stage0 = smem + (FP8 ? S::kRaw0 : S::kTileA);
            char LDS_AS* stage1 = smem + (FP8 ? S::kRaw1 : S::kTileB);
            char LDS_AS* ctile = smem + S::kTileA;  // FP8: the single bf16 tile
            // index prefetch ring: tiles k, k+1, k+2 (loaded above)
            constexpr std::true_type kUnrolled{};
            constexpr std::false_type kLooped{};
            // q was loaded before tile t0: it is pinned in registers before the
            // loop, so no wait for it lands inside the tile loop. Its wait also
            // covers the tile loads issued before it where they are untracked
            // asm (the dense variants). bf16: the wait sits between tile t0's
            // loads and tile t0 + 1's, so the first tile does not also wait for
            // the second (low-head split kernel, alternating runs: L = 4K -1.8 %,
            // 16K -1.0 %, 64K -0.3 %; one-tile parts, L <= 1K, +3 %: their
            // accumulators are then cleared after the wait). FP8 (the dequant
            // waits for the raw tile anyway) keeps it after both.
            auto pin_q = [&] {
                #pragma unroll
                for (int kk = 0; kk < NQ; ++kk) asm volatile("" ::"v"(qreg[kk]));
            };
            uint64_t mask_a = issue_tile(kUnrolled, t0, stage0, idx_a), mask_b = 0;
            if constexpr (kDrainPipeline) wait_vm(0);
            if constexpr (!FP8) pin_q();
            if (t0 + 1 <= t1) mask_b = issue_tile(kUnrolled, t0 + 1, stage1, idx_b);
            if constexpr (kDrainPipeline) wait_vm(0);
            if constexpr (FP8) pin_q();
            for (int k = t0; k <= t1; ++k) {
                const bool odd = ((k - t0) & 1) != 0;
                char LDS_AS* cur = odd ? stage1 : stage0;
                const unsigned idx_d = fetch_index(k + 3);
                // VMEM instructions this wave issued after tile k's DMA (a
                // lower bound is safe: it only waits longer): tile k + 1's loads,
                // and for the sparse index (VMEM) the words of k + 2 and k + 3
                // (dense index words are scalar loads).
                int after = 0;
                if (k + 1 <= t1) {
                    after += n_dma;
                    if (SPARSE && k > t0 && k + 2 <= t1) after += 1;
                    if (SPARSE && k + 3 <= t1) after += 1;
                }
                wait_vm(after);
                block_sync_lds();
                uint64_t mask_c = 0;
                if (FP8) {
                    dequant(cur, ctile);
                    block_sync_lds();
                    if (k + 2 <= t1) mask_c = issue_tile(kLooped, k + 2, cur, idx_c);
                    if constexpr (kDrainPipeline) wait_vm(0);
                    compute_tile(ctile, mask_a, k, std::false_type{}, [](int) {});
                } else {
                    compute_tile(cur, mask_a, k, std::false_type{}, [](int) {});
                    block_sync_lds();
                    if (k + 2 <= t1) mask_c = issue_tile(kLooped, k + 2, cur, idx_c);
                    if constexpr (kDrainPipeline) wait_vm(0);
                }
                idx_a = idx_b; idx_b = idx_c; idx_c = idx_d;
                mask_a = mask_b; mask_b = mask_c;
            }
            block_sync_lds();  // every wave is done with the tiles before LDS is reused
        }

        // ------------------------------------------------ epilogue
        const bool final_out = sg.n_splits == 1;
        // V64: token-half 1 hands (m, l, O) to token-half 0 of the same rows
        // through LDS; half 0 folds them in as it stores (o4 below), so its
        // accumulators are read once and never rewritten.
        float LDS_AS* xo = (float LDS_AS*)smem;                          // [2][16][4][64] float4
        float LDS_AS* xm = (float LDS_AS*)(smem + 2 * 16 * 4 * 64 * 16);  // [2][64] m, then [2][64] l
        float e_self = 1.f, e_part = 0.f;
        if constexpr (VAR == kV64) {
            if (tw == 1) {
                const int ln = lane_fresh();
                #pragma unroll
                for (int d = 0; d < NO; ++d)
                    #pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *(f32x4 LDS_AS*)(xo + ((((rw * 16 + d) * 4 + g) * 64) + ln) * 4) =
                            f32x4{oacc[d][4 * g], oacc[d][4 * g + 1], oacc[d][4 * g + 2], oacc[d][4 * g + 3]};
                xm[rw * 64 + ln] = m_run;
                xm[128 + rw * 64 + ln] = l_run;
            }
            block_sync_lds();
            if (tw == 0) {
                const int ln = lane_fresh();
                const float m1 = xm[rw * 64 + ln], l1 = xm[128 + rw * 64 + ln];
                const float mx = fmaxf(m_run, m1);
                e_self = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
                e_part = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - mx);
                l_run = l_run * e_self + l1 * e_part;
                m_run = mx;
            }
        }
        if constexpr (R32) {
          if (VAR == kV128 || tw == 0) {
            const float l_tot = l_run + wave_shfl_xor(l_run, 32);
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            const float lse_v = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
            // addresses from an opaque lane id: computed here, not held
            // across the tile loop
            const int ln = lane_fresh();
            const int rloc = 32 * rw + (ln & 31);
            const int h = sg.h0 + rloc;
            const int hh = ln >> 5;
            // the 4 output values of (d, g) times a factor: this wave's
            // (times a), plus for V64 the other token half's from LDS (times b)
            auto o4 = [&](int d, int g, float a, float b) -> f32x4 {
                f32x4 r = {oacc[d][4 * g] * a, oacc[d][4 * g + 1] * a, oacc[d][4 * g + 2] * a, oacc[d][4 * g + 3] * a};
                if constexpr (VAR == kV64) {
                    const f32x4 v = *(const f32x4 LDS_AS*)(xo + ((((rw * 16 + d) * 4 + g) * 64) + ln) * 4);
                    r += v * b;
                }
                return r;
            };
            if (final_out && VAR == kV128) {
                // Rows leave through LDS (free once the tile loop is done): a
                // lane holds 4 dims of one row per accumulator group, so direct
                // stores would write 32 separate 16-byte pieces per instruction.
                // Staged, each store writes one row's half contiguously. Per
                // wave 32 rows x half the dims, rows padded by 8 dims.
                constexpr int kHalfD = 32 * (NO / 2);            // dims per half (256, or 224)
                constexpr int kStg = kHalfD + 8;                  // staged row stride (dims)
                uint16_t LDS_AS* stg = (uint16_t LDS_AS*)(kFp8Pipe ? (char LDS_AS*)lds_tile : smem) + wave * 32 * kStg;
                const int rl = ln & 31;
                #pragma unroll
                for (int half = 0; half < 2; ++half) {
                    #pragma unroll
                    for (int dd = 0; dd < NO / 2; ++dd) {
                        const int d = half * (NO / 2) + dd;
                        #pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const f32x4 v = o4(d, g, e_self * inv, e_part * inv);
                            i16x4 w;
                            #pragma unroll
                            for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(short, (__bf16)v[e]);
                            *(i16x4 LDS_AS*)(stg + rl * kStg + 32 * dd + 8 * g + 4 * hh) = w;
                        }
                    }
                    // the wave reads back what it wrote (LDS ops of one wave stay in order)
                    #pragma unroll 4
                    for (int r = 0; r < 32; ++r) {
                        const int hr = sg.h0 + 32 * rw + r;
                        if (hr < p.rows_b && 4 * ln < kHalfD) {
                            const i16x4 w = *(const i16x4 LDS_AS*)(stg + r * kStg + 4 * ln);
                            *(i16x4*)(p.o + (qrow0 + hr) * F::kDv + half * kHalfD + 4 * ln) = w;
                        }
                    }
                }
                if (hh == 0 && h < p.rows_b) p.lse[qrow0 + h] = lse_v;
                block_sync_lds();  // every wave has read its staged rows before the next segment's loads
            } else if (final_out) {
                if (h < p.rows_b) {
                    uint16_t* op = p.o + (qrow0 + h) * F::kDv;
                    #pragma unroll
                    for (int d = 0; d < NO; ++d) {
                        #pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const int dim = 32 * d + 8 * g + 4 * hh;
                            const f32x4 v = o4(d, g, e_self * inv, e_part * inv);
                            i16x4 w;
                            #pragma unroll
                            for (int e = 0; e < 4; ++e) w[e] = __builtin_bit_cast(short, (__bf16)v[e]);
                            *(i16x4*)(op + dim) = w;
                        }
                    }
                    if (hh == 0) p.lse[qrow0 + h] = lse_v;
                }
            } else {
                // fp16 partial o * 2^-e, e from the row's largest |o| (its two
                // lanes hold 256 dims each). Blocked layout: one 512-byte
                // contiguous store per (d, g) per wave.
                float amax = 0.f;
                #pragma unroll
                for (int d = 0; d < NO; ++d)
                    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 v = o4(d, g, e_self, e_part);
                        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
                    }
                amax = fmaxf(amax, wave_shfl_xor(amax, 32));
                // V64: the store pass reads the other half's values again
                // and scales afresh instead of holding the pass above's
                if constexpr (VAR == kV64) asm volatile("" ::: "memory");
                const unsigned ef = partial_exp_field(amax * inv);
                const float sc = inv * exp_field_inv_pow2(ef);  // exact: inv times a power of two
                // (a slot holds 512 dims per row whatever the value width)
                f16x4* wp = (f16x4*)(p.ws_o + (int64_t)sg.slot * RG * kDv) + (rw * 16 * 4) * 64 + ln;
                #pragma unroll
                for (int d = 0; d < NO; ++d) {
                    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 v = o4(d, g, e_self * sc, e_part * sc);
                        wp[(d * 4 + g) * 64] = to_f16x4(v[0], v[1], v[2], v[3]);
                    }
                }
                if (hh == 0) {
                    p.ws_lse[(int64_t)sg.slot * RG + rloc] = lse_v;
                    p.ws_scale[(int64_t)sg.slot * RG + rloc] = exp_field_pow2(ef);
                }
            }
          }
          if constexpr (VAR == kV64) block_sync_lds();  // merge buffer read before the next segment's DMA
        } else {
            // merge the four waves' states through LDS
            float l_w = l_run + wave_shfl_xor(l_run, 16);
            l_w += wave_shfl_xor(l_w, 32);
            // [4][16][kMoStride]: rows padded by 4 floats, so the 16 rows a
            // ds_write_b128 covers start 4 banks apart (at 512 floats every row
            // began in the same bank: a 16-way conflict on every write)
            constexpr int kMoStride = 516;
            float LDS_AS* mo = (float LDS_AS*)smem;
            float LDS_AS* mm = (float LDS_AS*)(smem + 4 * 16 * kMoStride * 4);  // [4][16] m, then [4][16] l
            static_assert(4 * 16 * kMoStride * 4 + 2 * 64 * 4 <= S::kBytes, "merge buffers fit the tile area");
            const int row = lane & 15, g = lane >> 4;
            #pragma unroll
            for (int d = 0; d < NO; ++d)
                *(f32x4 LDS_AS*)(mo + (wave * 16 + row) * kMoStride + 16 * d + 4 * g) = oacc[d];
            if (g == 0) { mm[wave * 16 + row] = m_run; mm[64 + wave * 16 + row] = l_w; }
            block_sync_lds();
            // thread -> row mr, dims 4c + 64j (j < kDv / 64): 16 threads cover 64 contiguous dims
            constexpr int NJ = F::kDv / 64;
            const int mr = tid >> 4;
            const int c4 = (tid & 15) * 4;
            float mw[4], lw[4];
            float mx = -INFINITY;
            #pragma unroll
            for (int w = 0; w < 4; ++w) { mw[w] = mm[w * 16 + mr]; lw[w] = mm[64 + w * 16 + mr]; mx = fmaxf(mx, mw[w]); }
            float e[4], l_tot = 0.f;
            #pragma unroll
            for (int w = 0; w < 4; ++w) { e[w] = (mw[w] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - mx); l_tot += e[w] * lw[w]; }
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            const float lse_v = l_tot > 0.f ? (mx + __log2f(l_tot)) * kLn2 : -INFINITY;
            const int h = sg.h0 + mr;
            f32x4 acc[NJ];
            #pragma unroll
            for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            #pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float ew = e[w] * inv;
                #pragma unroll
                for (int j = 0; j < NJ; ++j) acc[j] += ew * *(const f32x4 LDS_AS*)(mo + (w * 16 + mr) * kMoStride + c4 + 64 * j);
            }
            if (final_out) {
                if (h < p.rows_b) {
                    uint16_t* op = p.o + (qrow0 + h) * F::kDv + c4;
                    #pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        i16x4 w4;
                        #pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2) w4[e2] = __builtin_bit_cast(short, (__bf16)acc[j][e2]);
                        *(i16x4*)(op + 64 * j) = w4;
                    }
                    if ((tid & 15) == 0) p.lse[qrow0 + h] = lse_v;
                }
            } else {
                // fp16 partial o * 2^-e, e from the row's largest |o| (16 lanes
                // hold its 512 dims)
                float amax = 0.f;
                #pragma unroll
                for (int j = 0; j < NJ; ++j)
                    #pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) amax = fmaxf(amax, fabsf(acc[j][e2]));
                #pragma unroll
                for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, wave_shfl_xor(amax, m));
                const unsigned ef = partial_exp_field(amax);
                const float sc = exp_field_inv_pow2(ef);
                uint16_t* wp = p.ws_o + ((int64_t)sg.slot * RG + mr) * kDv + c4;  // 512-dim slot rows
                #pragma unroll
                for (int j = 0; j < NJ; ++j)
                    *(f16x4*)(wp + 64 * j) = to_f16x4(acc[j][0] * sc, acc[j][1] * sc, acc[j][2] * sc, acc[j][3] * sc);
                if ((tid & 15) == 0) {
                    p.ws_lse[(int64_t)sg.slot * RG + mr] = lse_v;
                    p.ws_scale[(int64_t)sg.slot * RG + mr] = exp_field_pow2(ef);
                }
            }
            block_sync_lds();  // merge buffers are read before the next segment's DMA
        }
    }
}

template <int FMT, int VAR>
hipError_t launch_one(const DecodeParams& p, bool sparse, bool mixed, hipStream_t s) {
    if (sparse)
        hipLaunchKernelGGL((decode_kernel<FMT, true, VAR, false>), dim3(p.num_parts), dim3(kThreads), 0, s, p);
    else if (mixed)
        hipLaunchKernelGGL((decode_kernel<FMT, false, VAR, true>), dim3(p.num_parts), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((decode_kernel<FMT, false, VAR, false>), dim3(p.num_parts), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_format(const DecodeParams& p, int variant, bool sparse, hipStream_t s) {
    // A dense causal call packs s_q positions of h_q rows into one row space;
    // a group of rg rows straddles two positions exactly when h_q is not a
    // multiple of rg (the group holding rows h_q - 1 and h_q).
    const int rg = (variant == kV128) ? 128 : (variant == kV64 ? 64 : 16);
    const bool mixed = !sparse && p.causal && p.s_q > 1 && p.h_q % rg != 0;
    if (variant == kV128) return launch_one<FMT, kV128>(p, sparse, mixed, s);
    if (variant == kV64) return launch_one<FMT, kV64>(p, sparse, mixed, s);
    return launch_one<FMT, kV16>(p, sparse, mixed, s);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int variant, int format, bool sparse, hipStream_t s) {
    if (format == kFmtFp8) return launch_format<kFmtFp8>(p, variant, sparse, s);
    if (format == kFmtFp8Mx) return launch_format<kFmtFp8Mx>(p, variant, sparse, s);
    return launch_format<kFmtBf16>(p, variant, sparse, s);
}

}  // namespace mla
