// C ABI of the library (declared in include/mla.h): argument validation on
// the host, buffer sizing, and kernel launches. Every check runs before any
// HIP call so that an invalid call enqueues nothing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "mla.h"
#include "mla_common.h"
#include "mla_probe.h"
#include "mla_quantize.h"
#include "mla_absorb.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return MLA_OK;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

bool fits(int batch, int s_q, int h_q, bool sparse) {
    return (int64_t)batch * mla::layout_for(h_q, s_q, sparse).n_rg <= mla::kMaxUnits;
}

// Shape checks. mode: 0 dense, 1 sparse, -1 the size queries, which do not
// know the kind of call: they cover every kind the shape allows (a sparse
// shape has at least as many row groups as the dense one, so dense is the
// one that can fit alone).
int check_shape(int batch, int s_q, int h_q, int num_parts, int mode) {
    if (batch < 1) return fail(MLA_ERR_INVALID, "batch must be >= 1 (got %d)", batch);
    if (s_q < 1) return fail(MLA_ERR_INVALID, "s_q must be >= 1 (got %d)", s_q);
    if (h_q < 1) return fail(MLA_ERR_INVALID, "h_q must be >= 1 (got %d)", h_q);
    if (num_parts < 1 || num_parts > 65535)
        return fail(MLA_ERR_INVALID, "num_parts must be in [1, 65535] (got %d)", num_parts);
    const bool sparse = mode == 1;
    if (!fits(batch, s_q, h_q, sparse)) {
        const mla::Layout l = mla::layout_for(h_q, s_q, sparse);
        return fail(MLA_ERR_UNSUPPORTED, "%s: batch * %d row groups of %d rows = %lld exceeds %d row-group sequences",
                    sparse ? "sparse" : "dense", l.n_rg, l.rg, (long long)batch * l.n_rg, mla::kMaxUnits);
    }
    return MLA_OK;
}

size_t workspace_bytes_for(int batch, int num_parts, const mla::Layout& l) {
    const size_t slots = (size_t)batch * l.n_rg + (size_t)num_parts;
    const size_t o_bytes = slots * l.rg * mla::kDv * sizeof(uint16_t);
    const size_t lse_bytes = slots * l.rg * sizeof(float);
    return ((o_bytes + 255) & ~(size_t)255) + 2 * lse_bytes;
}

// Workspace bytes of a call (mode 0 dense, 1 sparse) or, for mode -1, enough
// for every kind of call the shape allows.
size_t workspace_bytes(int batch, int s_q, int h_q, int num_parts, int mode) {
    size_t need = 0;
    for (int m = 0; m < 2; ++m) {
        if (mode >= 0 ? m != mode : !fits(batch, s_q, h_q, m == 1)) continue;
        const size_t b = workspace_bytes_for(batch, num_parts, mla::layout_for(h_q, s_q, m == 1));
        need = b > need ? b : need;
    }
    return need;
}

// Validates a decode call; fills the kernel parameters.
int prepare(const mla_decode_args* a, mla::DecodeParams* p) {
    if (!a) return fail(MLA_ERR_INVALID, "args is NULL");
    if (a->struct_size != (int32_t)sizeof(mla_decode_args))
        return fail(MLA_ERR_INVALID, "struct_size %d != sizeof(mla_decode_args) %d", a->struct_size,
                    (int)sizeof(mla_decode_args));
    const bool sparse = a->indices != nullptr;
    int st = check_shape(a->batch, a->s_q, a->h_q, a->num_parts, sparse ? 1 : 0);
    if (st) return st;
    if (!a->q || !a->kv || !a->o || !a->lse) return fail(MLA_ERR_INVALID, "q, kv, o and lse must be non-NULL");
    if (!aligned(a->q, 16) || !aligned(a->o, 16) || !aligned(a->kv, 16) || !aligned(a->lse, 4))
        return fail(MLA_ERR_INVALID, "q, o and kv must be 16-byte aligned, lse 4-byte aligned");
    if (a->block_size != mla::kBlock) return fail(MLA_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", a->block_size);
    if (a->kv_format != MLA_KV_BF16 && a->kv_format != MLA_KV_FP8_656 && a->kv_format != MLA_KV_FP8_528)
        return fail(MLA_ERR_INVALID, "unknown kv_format %d", a->kv_format);
    const int want_row = a->kv_format == MLA_KV_BF16 ? 1152 : (a->kv_format == MLA_KV_FP8_656 ? 656 : 528);
    if (a->row_bytes != want_row)
        return fail(MLA_ERR_INVALID, "row_bytes %d does not match kv_format %s (%d bytes per token)", a->row_bytes,
                    a->kv_format == MLA_KV_BF16 ? "bf16" : (a->kv_format == MLA_KV_FP8_656 ? "fp8-656" : "fp8-528"),
                    want_row);
    if (a->num_blocks < 1) return fail(MLA_ERR_INVALID, "num_blocks must be >= 1");
    if (a->num_blocks * (int64_t)mla::kBlock >= ((int64_t)1 << 31))
        return fail(MLA_ERR_UNSUPPORTED, "num_blocks * 64 must be < 2^31");
    // the split kernel addresses rows through buffer descriptors, whose byte
    // offsets are 32-bit: the whole cache must lie within 4 GiB of its start
    if (a->num_blocks * (int64_t)mla::kBlock * a->row_bytes > ((int64_t)1 << 32))
        return fail(MLA_ERR_UNSUPPORTED, "the cache (num_blocks * 64 * row_bytes = %lld bytes) must be at most 4 GiB",
                    (long long)(a->num_blocks * (int64_t)mla::kBlock * a->row_bytes));
    if (sparse) {
        if (a->topk < 1) return fail(MLA_ERR_INVALID, "topk must be >= 1 with indices");
        if (a->causal) return fail(MLA_ERR_INVALID, "causal masking is not defined with sparse indices");
        if (a->topk > mla::kMaxSeqTokens)
            return fail(MLA_ERR_UNSUPPORTED, "topk must be <= 2^23 (got %d)", a->topk);
        if (!aligned(a->indices, 4)) return fail(MLA_ERR_INVALID, "indices must be 4-byte aligned");
        if ((int64_t)a->batch * a->s_q * a->topk >= ((int64_t)1 << 29))
            return fail(MLA_ERR_UNSUPPORTED, "batch * s_q * topk must be < 2^29 index entries");
    } else {
        if (!a->block_table || !a->cache_seqlens)
            return fail(MLA_ERR_INVALID, "dense attention needs block_table and cache_seqlens");
        if (!aligned(a->block_table, 4) || !aligned(a->cache_seqlens, 4))
            return fail(MLA_ERR_INVALID, "block_table and cache_seqlens must be 4-byte aligned");
        if (a->max_blocks_per_seq < 1) return fail(MLA_ERR_INVALID, "max_blocks_per_seq must be >= 1");
        if (a->max_blocks_per_seq > mla::kMaxSeqTokens / mla::kBlock)
            return fail(MLA_ERR_UNSUPPORTED, "max_blocks_per_seq must be <= 2^17 (got %d)", a->max_blocks_per_seq);
        if (a->topk != 0) return fail(MLA_ERR_INVALID, "topk must be 0 without indices");
    }
    if (!std::isfinite(a->softmax_scale)) return fail(MLA_ERR_INVALID, "softmax_scale must be finite");
    if (!a->tile_meta || !a->split_offsets) return fail(MLA_ERR_INVALID, "tile_meta and split_offsets are required");
    if (!aligned(a->tile_meta, 16) || !aligned(a->split_offsets, 4))
        return fail(MLA_ERR_INVALID, "tile_meta must be 16-byte aligned, split_offsets 4-byte aligned");
    if (!a->workspace) return fail(MLA_ERR_INVALID, "workspace is required");
    if (!aligned(a->workspace, 256)) return fail(MLA_ERR_INVALID, "workspace must be 256-byte aligned");
    const size_t need = workspace_bytes(a->batch, a->s_q, a->h_q, a->num_parts, sparse ? 1 : 0);
    if (a->workspace_bytes < need)
        return fail(MLA_ERR_WORKSPACE, "workspace_bytes %zu < required %zu", a->workspace_bytes, need);

    const mla::Layout l = mla::layout_for(a->h_q, a->s_q, sparse);
    const size_t slots = (size_t)a->batch * l.n_rg + (size_t)a->num_parts;
    const size_t o_bytes = ((slots * l.rg * mla::kDv * sizeof(uint16_t)) + 255) & ~(size_t)255;
    p->q = static_cast<const uint16_t*>(a->q);
    p->kv = static_cast<const uint8_t*>(a->kv);
    p->block_table = a->block_table;
    p->seqlens = a->cache_seqlens;
    p->indices = a->indices;
    p->tile_meta = a->tile_meta;
    p->split_offsets = a->split_offsets;
    p->ws_o = static_cast<uint16_t*>(a->workspace);
    p->ws_lse = reinterpret_cast<float*>(static_cast<char*>(a->workspace) + o_bytes);
    p->ws_scale = p->ws_lse + slots * l.rg;
    p->o = static_cast<uint16_t*>(a->o);
    p->lse = a->lse;
    p->batch = a->batch;
    p->s_q = a->s_q;
    p->h_q = a->h_q;
    p->n_hb = l.n_hb;
    p->n_rg = l.n_rg;
    p->rg = l.rg;
    p->rows_b = l.rows_b;
    p->n_pos = l.n_pos;
    p->mbps = sparse ? 0 : a->max_blocks_per_seq;
    p->topk = sparse ? a->topk : 0;
    p->causal = a->causal ? 1 : 0;
    p->num_rows = (int)(a->num_blocks * mla::kBlock);
    p->num_parts = a->num_parts;
    p->row_bytes = a->row_bytes;
    p->scale_log2 = a->softmax_scale * 1.4426950408889634f;
    return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_last_error(void) { return g_err; }

int mla_default_num_parts(int device, int* num_parts) {
    if (!num_parts) return fail(MLA_ERR_INVALID, "num_parts is NULL");
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    *num_parts = n;
    return ok();
}

int mla_metadata_size(int batch, int s_q, int h_q, int num_parts, int64_t* tile_meta_elems,
                      int64_t* split_offsets_elems) {
    if (!tile_meta_elems || !split_offsets_elems) return fail(MLA_ERR_INVALID, "output pointers are NULL");
    int st = check_shape(batch, s_q, h_q, num_parts, -1);
    if (st) return st;
    int n_rg = mla::layout_for(h_q, s_q, false).n_rg;
    if (fits(batch, s_q, h_q, true)) n_rg = std::max(n_rg, mla::layout_for(h_q, s_q, true).n_rg);
    *tile_meta_elems = (int64_t)num_parts * 8;
    *split_offsets_elems = (int64_t)batch * n_rg + 1;
    return ok();
}

int mla_workspace_size(int batch, int s_q, int h_q, int num_parts, size_t* bytes) {
    if (!bytes) return fail(MLA_ERR_INVALID, "bytes is NULL");
    int st = check_shape(batch, s_q, h_q, num_parts, -1);
    if (st) return st;
    *bytes = workspace_bytes(batch, s_q, h_q, num_parts, -1);
    return ok();
}

int mla_get_metadata(const int32_t* cache_seqlens, int batch, int s_q, int h_q, int topk, int num_parts,
                     int32_t* tile_meta, int32_t* split_offsets, void* stream) {
    int st = check_shape(batch, s_q, h_q, num_parts, topk > 0 ? 1 : 0);
    if (st) return st;
    if (topk < 0) return fail(MLA_ERR_INVALID, "topk must be >= 0 (got %d)", topk);
    if (topk > mla::kMaxSeqTokens) return fail(MLA_ERR_UNSUPPORTED, "topk must be <= 2^23 (got %d)", topk);
    if (topk == 0 && !cache_seqlens) return fail(MLA_ERR_INVALID, "cache_seqlens is required for dense attention");
    if (topk == 0 && !aligned(cache_seqlens, 4)) return fail(MLA_ERR_INVALID, "cache_seqlens must be 4-byte aligned");
    if (!tile_meta || !split_offsets) return fail(MLA_ERR_INVALID, "tile_meta and split_offsets are required");
    if (!aligned(tile_meta, 16) || !aligned(split_offsets, 4))
        return fail(MLA_ERR_INVALID, "tile_meta must be 16-byte aligned, split_offsets 4-byte aligned");
    const mla::Layout l = mla::layout_for(h_q, s_q, topk > 0);
    mla::MetaParams p;
    p.seqlens = cache_seqlens;
    p.tile_meta = tile_meta;
    p.split_offsets = split_offsets;
    p.batch = batch;
    p.n_rg = l.n_rg;
    p.topk = topk;
    p.num_parts = num_parts;
    // A sparse call gives every row-group sequence the same tile count: a
    // per-sequence fixed cost would only push part boundaries off sequence
    // boundaries, so sparse calls use none.
    p.fixed_cost = topk > 0 ? 0 : l.fixed_cost;
    p.min_payload = l.min_payload;
    hipError_t e = mla::launch_metadata(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "metadata launch: %s", hipGetErrorString(e));
    return ok();
}

int mla_decode_with_kvcache(const mla_decode_args* args, void* stream) {
    mla::DecodeParams p;
    int st = prepare(args, &p);
    if (st) return st;
    const mla::Layout l = mla::layout_for(args->h_q, args->s_q, args->indices != nullptr);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = mla::launch_decode(p, l.variant, args->kv_format, args->indices != nullptr, s);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    e = mla::launch_combine(p, args->kv_format, s);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
    return ok();
}

int mla_decode_splits(const mla_decode_args* args, void* stream) {
    mla::DecodeParams p;
    int st = prepare(args, &p);
    if (st) return st;
    const mla::Layout l = mla::layout_for(args->h_q, args->s_q, args->indices != nullptr);
    hipError_t e = mla::launch_decode(p, l.variant, args->kv_format, args->indices != nullptr,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

int mla_combine(const mla_decode_args* args, void* stream) {
    mla::DecodeParams p;
    int st = prepare(args, &p);
    if (st) return st;
    hipError_t e = mla::launch_combine(p, args->kv_format, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

// Workspace of mla_decode_with_kvcache_static: device memory of the library
// itself, one copy on every GPU the library runs on, held until the process
// ends. In host code `scratch` names a host-side stand-in, never the device
// memory: kernels get the address hipGetSymbolAddress gives for the current
// device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[MLA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_with_kvcache_static(const mla_decode_args* args, void* stream) {
    if (!args) return fail(MLA_ERR_INVALID, "args is NULL");
    if (args->struct_size != (int32_t)sizeof(mla_decode_args))
        return fail(MLA_ERR_INVALID, "struct_size %d != sizeof(mla_decode_args) %d", args->struct_size,
                    (int)sizeof(mla_decode_args));
    int st = check_shape(args->batch, args->s_q, args->h_q, args->num_parts, args->indices != nullptr ? 1 : 0);
    if (st) return st;
    const size_t need = workspace_bytes(args->batch, args->s_q, args->h_q, args->num_parts, args->indices != nullptr ? 1 : 0);
    if (need > (size_t)MLA_STATIC_SCRATCH_BYTES)
        return fail(MLA_ERR_UNSUPPORTED,
                    "this call needs %zu bytes of split workspace; the static scratch holds %zu "
                    "(use mla_decode_with_kvcache with a workspace)",
                    need, (size_t)MLA_STATIC_SCRATCH_BYTES);
    // every other check, on the host, before any HIP call (the workspace
    // fields of args are ignored: a placeholder stands in for the scratch)
    mla_decode_args a = *args;
    a.workspace = reinterpret_cast<void*>((uintptr_t)256);
    a.workspace_bytes = MLA_STATIC_SCRATCH_BYTES;
    mla::DecodeParams p;
    st = prepare(&a, &p);
    if (st) return st;
    void* ptr = nullptr;
    st = scratch_address(&ptr);
    if (st) return st;
    a.workspace = ptr;
    st = prepare(&a, &p);
    if (st) return st;
    const mla::Layout l = mla::layout_for(a.h_q, a.s_q, a.indices != nullptr);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = mla::launch_decode(p, l.variant, a.kv_format, a.indices != nullptr, s);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    e = mla::launch_combine(p, a.kv_format, s);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
    return ok();
}

int mla_quantize_fp8_append(const void* src, const int32_t* slots, int64_t n, void* kv, int64_t num_blocks,
                            void* stream) {
    if (n < 0) return fail(MLA_ERR_INVALID, "n must be >= 0 (got %lld)", (long long)n);
    if (n >= ((int64_t)1 << 31)) return fail(MLA_ERR_UNSUPPORTED, "n must be < 2^31 rows per call");
    if (num_blocks < 1) return fail(MLA_ERR_INVALID, "num_blocks must be >= 1");
    if (num_blocks * (int64_t)mla::kBlock >= ((int64_t)1 << 31))
        return fail(MLA_ERR_UNSUPPORTED, "num_blocks * 64 must be < 2^31");
    if (n == 0) return ok();
    if (!src || !slots || !kv) return fail(MLA_ERR_INVALID, "src, slots and kv must be non-NULL");
    if (!aligned(src, 16) || !aligned(kv, 16) || !aligned(slots, 4))
        return fail(MLA_ERR_INVALID, "src and kv must be 16-byte aligned, slots 4-byte aligned");
    mla::QuantParams p;
    p.src = static_cast<const uint16_t*>(src);
    p.slots = slots;
    p.kv = static_cast<uint8_t*>(kv);
    p.n = n;
    p.num_rows = (int)(num_blocks * mla::kBlock);
    hipError_t e = mla::launch_quantize(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "quantize launch: %s", hipGetErrorString(e));
    return ok();
}

int mla_probe_mfma_bf16(int iters, int blocks, float value, float* sink, void* stream) {
    if (iters < 1) return fail(MLA_ERR_INVALID, "iters must be >= 1 (got %d)", iters);
    if (blocks < 1 || blocks > (1 << 20)) return fail(MLA_ERR_INVALID, "blocks must be in [1, 2^20] (got %d)", blocks);
    if (!sink || !aligned(sink, 4)) return fail(MLA_ERR_INVALID, "sink must be non-NULL and 4-byte aligned");
    hipError_t e = mla::launch_probe_mfma(iters, blocks, value, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
    return ok();
}

int mla_probe_hbm_read(const void* src, int64_t bytes, int blocks, uint32_t* sink, void* stream) {
    if (bytes < 16 || bytes % 16 != 0) return fail(MLA_ERR_INVALID, "bytes must be a positive multiple of 16");
    if (blocks < 1 || blocks > (1 << 20)) return fail(MLA_ERR_INVALID, "blocks must be in [1, 2^20] (got %d)", blocks);
    if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4))
        return fail(MLA_ERR_INVALID, "src must be non-NULL and 16-byte aligned, sink non-NULL and 4-byte aligned");
    hipError_t e = mla::launch_probe_hbm_read(src, bytes, blocks, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

int check_absorb(int64_t tokens, int heads) {
    if (tokens < 0) return fail(MLA_ERR_INVALID, "tokens must be >= 0 (got %lld)", (long long)tokens);
    if (heads < 1) return fail(MLA_ERR_INVALID, "heads must be >= 1 (got %d)", heads);
    if (heads > 4096) return fail(MLA_ERR_UNSUPPORTED, "heads must be <= 4096 (got %d)", heads);
    if (tokens >= ((int64_t)1 << 31) / heads) return fail(MLA_ERR_UNSUPPORTED, "tokens * heads must be < 2^31");
    return MLA_OK;
}

}  // namespace

extern "C" {

int mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk_t, int64_t tokens, int heads, void* q,
                 void* stream) {
    int st = check_absorb(tokens, heads);
    if (st) return st;
    if (tokens == 0) return ok();
    if (!q_nope || !q_rope || !w_uk_t || !q) return fail(MLA_ERR_INVALID, "q_nope, q_rope, w_uk_t and q must be non-NULL");
    if (!aligned(q_nope, 16) || !aligned(q_rope, 16) || !aligned(w_uk_t, 16) || !aligned(q, 16))
        return fail(MLA_ERR_INVALID, "q_nope, q_rope, w_uk_t and q must be 16-byte aligned");
    mla::AbsorbParams p;
    p.x = static_cast<const uint16_t*>(q_nope);
    p.w = static_cast<const uint16_t*>(w_uk_t);
    p.rope = static_cast<const uint16_t*>(q_rope);
    p.out = static_cast<uint16_t*>(q);
    p.tokens = tokens;
    p.heads = heads;
    p.out_stride = mla::kDqk;
    hipError_t e = mla::launch_absorb_q(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "absorb launch: %s", hipGetErrorString(e));
    return ok();
}

int mla_unabsorb_o(const void* o_latent, const void* w_uv, int64_t tokens, int heads, void* out, void* stream) {
    int st = check_absorb(tokens, heads);
    if (st) return st;
    if (tokens == 0) return ok();
    if (!o_latent || !w_uv || !out) return fail(MLA_ERR_INVALID, "o_latent, w_uv and out must be non-NULL");
    if (!aligned(o_latent, 16) || !aligned(w_uv, 16) || !aligned(out, 16))
        return fail(MLA_ERR_INVALID, "o_latent, w_uv and out must be 16-byte aligned");
    mla::AbsorbParams p;
    p.x = static_cast<const uint16_t*>(o_latent);
    p.w = static_cast<const uint16_t*>(w_uv);
    p.rope = nullptr;
    p.out = static_cast<uint16_t*>(out);
    p.tokens = tokens;
    p.heads = heads;
    p.out_stride = 128;
    hipError_t e = mla::launch_unabsorb_o(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "unabsorb launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
