/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA decode library, libmla_mi355x.so.
 *
 * Computes DeepSeek-style Multi-head Latent Attention decode over a paged
 * latent KV cache. Pages cited below (by title, then section):
 *   [Walkthrough] "矩阵、注意力与 GPU：拆解 DeepGEMM 与 FlashMLA" (msy.plus)
 *   [Guide]       "FlashMLA 实战：MLA 注意力加速指南" (m.lsln.cn)
 *   [ETAP]        the FlashMLA-ETAP article (ocdem.com)
 *
 * The operation ([Walkthrough] §六 "吸收", "结果：decode 变成 MQA"; §五
 * "公式"): after weight absorption every query head h scores each cached
 * token against the same 576-dim row [latent c (512) ; rope k^R (64)],
 * score = softmax_scale * <q[b,i,h,:], row>, and the output is the softmax-
 * weighted sum of the 512-dim latents. Outputs o[b,i,h,:512] (bf16) and
 * lse[b,i,h] = ln(sum_t exp(score_t)) (fp32, natural log).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device pointers owned by the caller;
 *     the library never frees, retains or allocates device memory and never
 *     synchronises the stream. "host" pointers are read before return.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All device work is enqueued on it; launches are graph-capturable.
 *   - Return value: MLA_OK (0) or a negative status. On a negative status
 *     mla_last_error() (thread-local) describes it. Every argument check runs
 *     on the host before any HIP call, so an invalid call enqueues nothing.
 *   - Tensors are contiguous, row-major, in the shapes given.
 */
#ifndef MLA_MI355X_H
#define MLA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_INVALID (-1)     /* bad argument (null pointer, size, flag combination) */
#define MLA_ERR_UNSUPPORTED (-2) /* well-formed but outside what the kernels handle */
#define MLA_ERR_WORKSPACE (-3)   /* workspace or metadata buffers too small */
#define MLA_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed */

/* KV cache row formats ([Guide] §"FP8 缓存怎么把 KV 压掉四成", §"容易踩的坑"). */
#define MLA_KV_BF16 0    /* 576 bf16 = 1152 B per token: latent 512, then rope 64 */
#define MLA_KV_FP8_656 1 /* 656 B per token: 512 e4m3 latent codes, 4 fp32 scales
                            (one per 128 latent dims), 64 bf16 rope values */
#define MLA_KV_FP8_528 2 /* 528 B per token ([Walkthrough] §八, the V4.1 row; §九 data
                            before scales): 512 e4m3 codes of the whole key, 448
                            latent dims then 64 rope dims, then 16 UE8M0 scale
                            bytes, byte j scaling codes 32 j .. 32 j + 31 by
                            2^(byte - 127). With this format the key (and q) has
                            512 dims and the value (o) 448: q is
                            [batch, s_q, h_q, 512], o is [batch, s_q, h_q, 448]. */

#define MLA_BLOCK_SIZE 64 /* tokens per KV page */
#define MLA_D_QK 576
#define MLA_D_V 512
#define MLA_MAX_UNITS 8192 /* max row-group sequences (see below) per call */
#define MLA_MAX_SEQ_TOKENS (1 << 23) /* tokens one sequence may attend: cache_seqlens
                                        entries above it read as this value; bounds
                                        max_blocks_per_seq (2^17 pages) and topk */

/*
 * Split policy (the library's own rule; the pages give the metadata's role,
 * [Walkthrough] §七 "split-KV", but no format):
 *   The query rows of sequence b are its rows of q in order, (position i,
 *   head h) -> i * h_q + h. A dense call (topk == 0) puts all R = s_q * h_q
 *   of them in one row space: they attend the same cache, so one pass over
 *   it serves every position ([Walkthrough] §七 "先算清楚瓶颈": a decode
 *   request's h_q * s_q query rows share the KV). A sparse call has s_q row spaces of R = h_q
 *   rows, one per position (each position has its own indices). Rows are
 *   grouped into "row groups" of RG consecutive rows of a row space: RG = 16
 *   when R <= 16, RG = 64 when 16 < R <= 64, else RG = 128. A row-group
 *   sequence q = b * n_rg + i * n_hb + hb, with n_hb = ceil(R / RG) and
 *   n_rg = n_pos * n_hb (n_pos = 1 dense, s_q sparse; i = the row space),
 *   covers T_q = ceil(L_b / 64) tiles of 64 tokens (dense)
 *   or ceil(topk / 64) tiles (sparse). Units are laid end to end, each
 *   non-empty one first taking FIXED_COST positions, then one per tile; with
 *   total = sum(FIXED_COST + T_q) and W = max(ceil(total / num_parts),
 *   MIN_PAYLOAD), the tile at position x goes to work part floor(x / W).
 *   FIXED_COST and MIN_PAYLOAD: RG 128 -> 2 and 3; RG 64 -> 2 and 2;
 *   RG 16 -> 0 and 1; FIXED_COST is 0 for every RG when topk > 0 (all units
 *   of a sparse call have the same tile count).
 *   Placement: when num_parts is a multiple of 8, with used = ceil(total / W)
 *   and k = ceil(used / 8), work part j is row (j / k) * (num_parts / 8) +
 *   j % k of tile_meta and every other row is empty (the decode grid runs
 *   row r on XCD r / (num_parts / 8), so the parts with work are spread over
 *   the eight XCDs); otherwise work part j is row j.
 */

/* Message for the last non-OK status on this thread ("" if none). */
const char* mla_last_error(void);

/* Number of compute units of HIP device `device`, the default num_parts. */
int mla_default_num_parts(int device, int* num_parts);

/*
 * Element counts of the two metadata buffers for a call shape:
 * tile_meta holds num_parts * 8 int32, split_offsets holds Q + 1 int32 where
 * Q = batch * n_rg, the larger of the dense and the sparse n_rg (the sizes do
 * not depend on topk, so they cover either kind of call; a shape whose sparse
 * Q exceeds MLA_MAX_UNITS gets the dense sizes). Pure host arithmetic.
 */
int mla_metadata_size(int batch, int s_q, int h_q, int num_parts,
                      int64_t* tile_meta_elems, int64_t* split_offsets_elems);

/*
 * Bytes of split workspace mla_decode_with_kvcache needs: enough for a dense
 * or a sparse call of this shape (the larger). Layout, with
 * S = Q + num_parts slots (Q and RG of the call's kind): partial outputs, S slots of RG x 512 fp16; then, at
 * the next 256-byte boundary, partial lse fp32 [S][RG]; then partial scales
 * fp32 [S][RG]. A partial row o_k (already divided by its own softmax sum) is
 * stored as fp16(o_k / c), c = its scale, a power of two chosen so that the
 * row's largest |o_k / c| lies in [2^14, 2^15) (c = 1 for an all-zero row):
 * 11 significant bits over the row's own range, far below the bf16 rounding
 * of the final o. Inside a slot, RG = 16 is row-major [row][512]; RG = 128
 * and 64 are blocked as the split kernel's registers hold it: the group of 4
 * values at index ((w * 16 + dd) * 4 + g) * 64 + lane holds row
 * 32 w + (lane & 31), dims 32 dd + 8 g + 4 (lane >> 5) + 0..3. The slots of
 * row-group sequence q are split_offsets[q] .. split_offsets[q + 1] - 1, in
 * KV order.
 */
int mla_workspace_size(int batch, int s_q, int h_q, int num_parts, size_t* bytes);

/*
 * Split-KV work schedule ([Walkthrough] §七 "split-KV：把长序列切开":
 * computed once per decode step, reused by every layer).
 *   cache_seqlens  device int32 [batch], 4-byte aligned; ignored when topk > 0
 *                  (may be NULL)
 *   topk           0 for dense attention, else the sparse index count
 *   num_parts      parts (workgroups) of the decode grid, 1..65535
 *   tile_meta      device int32 [num_parts][8], 16-byte aligned, written: per row
 *                  (placed as above) {q_begin, t_begin, q_end, t_end
 *                  (inclusive), first_split, empty, 0, 0}
 *   split_offsets  device int32 [Q + 1], 4-byte aligned, written: prefix sums
 *                  of the number of splits of each row-group sequence
 * The result is a pure function of (cache_seqlens, batch, s_q, h_q, topk,
 * num_parts). Reusing it after any of these change gives wrong splits
 * silently; the caller must recompute it ([Walkthrough] §七 warns the same).
 * Errors: MLA_ERR_INVALID for null or misaligned buffers, batch/s_q/h_q < 1,
 * topk < 0, num_parts out of range; MLA_ERR_UNSUPPORTED if Q > MLA_MAX_UNITS or
 * topk > MLA_MAX_SEQ_TOKENS.
 */
int mla_get_metadata(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int topk,
                     int num_parts, int32_t* tile_meta, int32_t* split_offsets, void* stream);

typedef struct mla_decode_args {
    int32_t struct_size;       /* must equal sizeof(mla_decode_args) */
    int32_t batch, s_q, h_q;   /* num_heads_k is 1 ([Walkthrough] §六) */
    const void* q;             /* device bf16 [batch, s_q, h_q, 576], 16-byte aligned:
                                  absorbed latent query (512) then rope query (64);
                                  512 dims (448 + 64) with MLA_KV_FP8_528 */
    const void* kv;            /* device uint8 [num_blocks, 64, row_bytes], 16-byte
                                  aligned */
    int64_t num_blocks;        /* pages in the cache; num_blocks * 64 * row_bytes
                                  <= 2^32 (4 GiB: rows are addressed with 32-bit
                                  byte offsets from kv) */
    int32_t block_size;        /* must be 64 */
    int32_t row_bytes;         /* 1152 for MLA_KV_BF16, 656 for MLA_KV_FP8_656, 528 for
                                  MLA_KV_FP8_528; a mismatch is rejected ([Guide]
                                  §"容易踩的坑") */
    int32_t kv_format;         /* MLA_KV_BF16, MLA_KV_FP8_656 or MLA_KV_FP8_528 */
    const int32_t* block_table;   /* dense: device int32 [batch, max_blocks_per_seq],
                                     4-byte aligned; token t of sequence b is row
                                     block_table[b, t/64]*64 + t%64 */
    int32_t max_blocks_per_seq;   /* 1 .. MLA_MAX_SEQ_TOKENS / 64 */
    const int32_t* cache_seqlens; /* dense: device int32 [batch], 4-byte aligned, tokens
                                     per sequence */
    const int32_t* indices;       /* sparse: device int32 [batch, s_q, topk], 4-byte
                                     aligned: absolute cache rows
                                     (page*64 + offset), -1 = unused
                                     ([Walkthrough] §八 "当前 master 已经是稀疏注意力");
                                     NULL selects dense attention */
    int32_t topk;              /* sparse: 1 .. MLA_MAX_SEQ_TOKENS, with
                                  batch * s_q * topk < 2^29 */
    float softmax_scale;
    int32_t causal;            /* dense only: query i sees t <= L - s_q + i.
                                  causal with indices -> MLA_ERR_INVALID
                                  ([Guide] §"容易踩的坑") */
    const int32_t* tile_meta;     /* from mla_get_metadata with the same shapes;
                                     16-byte aligned */
    const int32_t* split_offsets; /* from the same call; 4-byte aligned */
    int32_t num_parts;
    void* workspace;           /* device, >= mla_workspace_size bytes, 256-B aligned */
    size_t workspace_bytes;
    void* o;                   /* device bf16 [batch, s_q, h_q, 512] (448 with
                                  MLA_KV_FP8_528), 16-byte aligned, written */
    float* lse;                /* device fp32 [batch, s_q, h_q], 4-byte aligned,
                                  written */
} mla_decode_args;

/*
 * Decode attention over the cache.
 * Enqueues the split kernel, then mla_combine's kernel. Masked tokens (past
 * L, causal-excluded, -1 or out-of-range sparse entries, tokens whose page id
 * is outside [0, num_blocks) or past max_blocks_per_seq) are never read and
 * never contribute. A query row with no attended token gets o = 0 and
 * lse = -inf. Errors: MLA_ERR_INVALID (see field notes), MLA_ERR_WORKSPACE,
 * MLA_ERR_UNSUPPORTED (block_size other than 64, a cache above 4 GiB,
 * max_blocks_per_seq or topk above their bounds, Q > MLA_MAX_UNITS),
 * MLA_ERR_HIP.
 */
int mla_decode_with_kvcache(const mla_decode_args* args, void* stream);

/*
 * The split kernel of mla_decode_with_kvcache alone: each part attends its
 * tile ranges ([Walkthrough] §七, split-KV). Rows of a sequence with a
 * single split are finished (o, lse); the others leave partials in the
 * workspace for mla_combine, which must follow on the same stream with the
 * same arguments before o and lse are read. Lets a caller place work between
 * the two kernels. Same arguments and errors as mla_decode_with_kvcache.
 */
int mla_decode_splits(const mla_decode_args* args, void* stream);

/*
 * Split-KV LSE merge ([Walkthrough] §七: m = max m_k,
 * l = sum l_k e^{m_k - m}, o = sum o_k l_k e^{m_k - m} / l). For every query
 * row whose sequence has more than one split, merges the partials in the
 * workspace into o and lse; rows with no split get o = 0, lse = -inf; rows
 * with one split are left as the split kernel wrote them. Reads the same
 * fields as mla_decode_with_kvcache (q, kv, block_table, indices unused).
 */
int mla_combine(const mla_decode_args* args, void* stream);

/*
 * mla_decode_with_kvcache without a caller workspace: for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The split workspace is the library's
 * own static device array of MLA_STATIC_SCRATCH_BYTES, one per GPU, held
 * until the process ends; this call allocates nothing (no hipMalloc, no
 * allocating library routine). Same arguments, kernels and results as
 * mla_decode_with_kvcache, except that args->workspace and
 * args->workspace_bytes are ignored. The stream must belong to the current
 * HIP device. No part of the scratch needs clearing: every slot the merge
 * reads is written earlier in the same call. All calls on one GPU share its
 * scratch: calls that overlap in time on one GPU (other streams, other host
 * threads) race and give wrong results; order them.
 * Errors: those of mla_decode_with_kvcache, plus MLA_ERR_UNSUPPORTED when
 * the split workspace this call needs (the layout under mla_workspace_size
 * for the call's own kind, dense or sparse) exceeds MLA_STATIC_SCRATCH_BYTES;
 * that is checked first, on the host, before any HIP call.
 */
#define MLA_STATIC_SCRATCH_BYTES (64u << 20)
int mla_decode_with_kvcache_static(const mla_decode_args* args, void* stream);

/*
 * FP8 cache writer (quantise on write): turns n bf16 cache rows into the
 * 656-byte FP8 layout of [Guide] §"FP8 缓存怎么把 KV 压掉四成" and stores
 * row i at absolute cache row slots[i] (= page * 64 + offset, the row
 * numbering sparse indices use). [Guide] §"容易踩的坑" is why the writer must
 * match this layout exactly.
 *   src    device bf16 [n, 576]: latent (512) then RoPE (64), the row a bf16
 *          cache would hold; 16-byte aligned; read only. Values are finite.
 *   slots  device int32 [n]; -1, or any value outside [0, num_blocks * 64),
 *          writes nothing. Two rows aimed at one slot race (one of them lands).
 *   kv     device [num_blocks, 64, 656] bytes, 16-byte aligned; only the
 *          addressed rows are written.
 * Per 128 latent values: scale = amax / 448 in fp32 (1 if the group is all
 * zero; [Walkthrough] §三 for e4m3's 448 maximum), code = e4m3 (OCP, finite
 * only) round-to-nearest-even of clamp(x / scale, -448, 448); both divisions
 * are IEEE fp32. Bytes [0, 512) codes, [512, 528) the four scales
 * (little-endian fp32), [528, 656) the RoPE bf16 values unchanged.
 * n == 0 enqueues nothing. Errors: MLA_ERR_INVALID (negative n, NULL or
 * misaligned pointers, num_blocks < 1), MLA_ERR_UNSUPPORTED (n >= 2^31 or
 * num_blocks * 64 >= 2^31), MLA_ERR_HIP (launch failure). Asynchronous on
 * `stream`; allocates nothing.
 */
int mla_quantize_fp8_append(const void* src, const int32_t* slots, int64_t n, void* kv, int64_t num_blocks,
                            void* stream);

/*
 * Absorbed query ([Walkthrough] §六, the absorption passage): per token t and
 * head i, q[t, i, 0:512] = W^UK_i^T q^C[t, i] and q[t, i, 512:576] = q^R[t, i],
 * the 576-value query row the decode takes (its [batch, s_q, h_q, 576] q with
 * tokens = batch * s_q, heads = h_q).
 *   q_nope  device bf16 [tokens, heads, 128]: q^C
 *   q_rope  device bf16 [tokens, heads, 64]: q^R, already rotated; copied
 *   w_uk_t  device bf16 [heads, 512, 128]: per head the transpose of W^UK_i
 *           (W^UK_i is 128 x 512, latent -> key); row n holds the 128
 *           weights of latent dim n. Arranged once when weights are loaded.
 *   q       device bf16 [tokens, heads, 576], written
 * All pointers 16-byte aligned. fp32 accumulation, one round to bf16 (nearest
 * even). tokens == 0 enqueues nothing. Errors: MLA_ERR_INVALID (negative
 * tokens, heads < 1, NULL or misaligned pointers), MLA_ERR_UNSUPPORTED
 * (heads > 4096, tokens * heads >= 2^31), MLA_ERR_HIP.
 */
int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk_t, int64_t tokens, int heads, void* q,
                 void* stream);

/*
 * Value up-projection after the decode ([Walkthrough] §六: o_i = W^UV_i times
 * the attention-weighted sum of latents): out[t, i] = W^UV_i o[t, i].
 *   o_latent  device bf16 [tokens, heads, 512]: the decode's o
 *   w_uv      device bf16 [heads, 128, 512]: W^UV_i (latent -> value)
 *   out       device bf16 [tokens, heads, 128], written
 * Alignment, rounding, empty calls and errors as mla_absorb_q.
 */
int mla_unabsorb_o(const void* o_latent, const void* w_uv, int64_t tokens, int heads, void* out, void* stream);

/*
 * Measurement aids, not part of the decode path: what this GPU reaches on its
 * own, reported beside the published peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16
 * MFMA) that the decode's roofline fractions are taken against.
 *
 * mla_probe_mfma_bf16: `blocks` workgroups of four wave64s; every wave runs
 *   `iters` steps of four independent v_mfma_f32_32x32x16_bf16 accumulation
 *   chains on register operands whose elements all equal bf16(value). FLOPs
 *   per launch: blocks * 4 * iters * 4 * 32768.
 *   sink  device float [blocks * 256], written: per thread the sum of its 64
 *         accumulator values, 1024 * iters * bf16(value)^2 in exact
 *         arithmetic (exact in fp32 while that stays below 2^24).
 * mla_probe_hbm_read: reads `bytes` of src once, with non-temporal 16-byte
 *   loads from `blocks` workgroups of 256 threads.
 *   src   device, 16-byte aligned, bytes a positive multiple of 16; read only.
 *   sink  device uint32 [blocks * 256], written: per thread the sum modulo
 *         2^32 of the 32-bit words it read (the sum over all threads is the
 *         sum of every word of src).
 * Errors: MLA_ERR_INVALID (iters < 1, blocks outside [1, 2^20], NULL or
 * misaligned pointers, bytes not a positive multiple of 16), MLA_ERR_HIP
 * (launch failure). Asynchronous on `stream`; allocate nothing.
 */
int mla_probe_mfma_bf16(int iters, int blocks, float value, float* sink, void* stream);
int mla_probe_hbm_read(const void* src, int64_t bytes, int blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MLA_MI355X_H */
