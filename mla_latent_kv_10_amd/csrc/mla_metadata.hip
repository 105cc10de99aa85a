// Split-KV work schedule kernel.
//
// Role from [Walkthrough] §七 "split-KV：把长序列切开": once per decode step,
// decide which row-group sequences and which 64-token tiles each part (one
// workgroup of the decode grid) processes, and how many splits each
// sequence has; every layer reuses the result. The rule (see include/mla.h):
// units laid end to end, fixed_cost positions then one per tile, work part
// floor(position / W); then the work parts are placed on the grid so that the
// ones holding work are spread evenly over the eight XCDs. One workgroup of
// 256 threads computes it: block-wide exclusive scans built from DPP wave
// scans with one barrier each (positions with the last non-empty unit in one
// pass, then split counts), then a binary search per part.
#include "mla_common.h"

namespace mla {

namespace {

constexpr int kMT = 256;
constexpr int kWaves = kMT / 64;

enum ScanOp { kSum, kMax };

template <ScanOp OP>
__device__ __forceinline__ int combine(int a, int b) { return OP == kSum ? a + b : max(a, b); }

// One DPP move: lane i takes `v` from the lane the control names (row_shr:n
// within rows of 16 lanes, row_bcast:15 / row_bcast:31 across rows). Lanes
// whose source lies outside the pattern get an unspecified value; callers
// use the result only in lanes where it is defined.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }

// Inclusive scan of one value per lane across the wave64: doubling steps
// inside each row of 16 lanes, then the last lane of rows 0 and 2 into rows 1
// and 3, then lane 31 into rows 2 and 3. No LDS, no barrier.
template <ScanOp OP>
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    const int lane = threadIdx.x & 63, rl = lane & 15;
    int t;
    t = dpp_mov<0x111>(x); if (rl >= 1) x = combine<OP>(t, x);   // row_shr:1
    t = dpp_mov<0x112>(x); if (rl >= 2) x = combine<OP>(t, x);   // row_shr:2
    t = dpp_mov<0x114>(x); if (rl >= 4) x = combine<OP>(t, x);   // row_shr:4
    t = dpp_mov<0x118>(x); if (rl >= 8) x = combine<OP>(t, x);   // row_shr:8
    t = dpp_mov<0x142>(x); if ((lane & 31) >= 16) x = combine<OP>(t, x);  // row_bcast:15
    t = dpp_mov<0x143>(x); if (lane >= 32) x = combine<OP>(t, x);         // row_bcast:31
    return x;
}

// Exclusive scan of one value per thread across the workgroup (thread order):
// wave scans, then the wave totals through `scratch` (kWaves ints, used by
// this scan only) behind one barrier. *total receives the reduction over all
// threads.
template <ScanOp OP>
__device__ int block_exclusive_scan(int v, int identity, int* scratch, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int inc = wave_inclusive_scan<OP>(v);
    int exc = __shfl_up(inc, 1, 64);
    if (lane == 0) exc = identity;
    if (lane == 63) scratch[w] = inc;
    __syncthreads();
    int before = identity, tot = identity;
    #pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int s = scratch[i];
        if (i < w) before = combine<OP>(before, s);
        tot = combine<OP>(tot, s);
    }
    *total = tot;
    return combine<OP>(before, exc);
}

// Exclusive scans of two values per thread at once, a sum and a max, behind
// one barrier (`scratch`: kWaves int2, used by this scan only). Returns (sum
// before, max before); *sum_total receives the sum over all threads.
__device__ int2 block_exclusive_scan_sum_max(int vs, int vm, int2* scratch, int* sum_total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int is = wave_inclusive_scan<kSum>(vs), im = wave_inclusive_scan<kMax>(vm);
    int es = is - vs, em = __shfl_up(im, 1, 64);
    if (lane == 0) em = -1;
    if (lane == 63) scratch[w] = make_int2(is, im);
    __syncthreads();
    int bs = 0, bm = -1, ts = 0;
    #pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        const int2 s2 = scratch[i];
        if (i < w) { bs += s2.x; bm = max(bm, s2.y); }
        ts += s2.x;
    }
    *sum_total = ts;
    return make_int2(bs + es, max(bm, em));
}

// Smallest q in [0, n) with cum[q + 1] > v (cum has n + 1 entries, non-decreasing).
__device__ int first_unit_past(const int* cum, int n, int v) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (cum[mid + 1] > v) hi = mid; else lo = mid + 1;
    }
    return lo;
}

// Scalar arguments rather than one struct: they are preloaded into SGPRs at
// dispatch, so the length loads issue without waiting for the argument block.
__global__ __launch_bounds__(kMT) void metadata_kernel(const int32_t* seqlens, int32_t* tile_meta, int32_t* split_offsets,
                                                       int batch, int n_rg, int topk, int num_parts, int fixed_cost,
                                                       int min_payload) {
    const MetaParams p{seqlens, tile_meta, split_offsets, batch, n_rg, topk, num_parts, fixed_cost, min_payload};
    __shared__ int s_cum[kMaxUnits + 1];    // exclusive scan of per-unit cost (positions)
    __shared__ int s_T[kMaxUnits];          // tiles per unit
    __shared__ int s_prev[kMaxUnits];       // last non-empty unit at or before q (-1 if none)
    __shared__ int s_scan[kWaves];    // wave totals of the split-count scan
    __shared__ int2 s_scan2[kWaves];  // wave totals of the position scan
    const int Q = p.batch * p.n_rg;
    const int tid = threadIdx.x;
    const int C = p.fixed_cost;
    const int per = (Q + kMT - 1) / kMT;    // <= 32 units per thread
    const int b0 = tid * per, e0 = min(Q, b0 + per);

    // tiles and cost of this thread's (contiguous) units
    int cost_sum = 0, last_ne = -1;
    for (int q = b0; q < e0; ++q) {
        int T;
        if (p.topk > 0) {
            T = (p.topk + kBlock - 1) / kBlock;
        } else {
            const int L = min(p.seqlens[q / p.n_rg], kMaxSeqTokens);
            T = L > 0 ? (L + kBlock - 1) / kBlock : 0;
        }
        s_T[q] = T;
        cost_sum += T > 0 ? C + T : 0;
        if (T > 0) last_ne = q;
    }
    int total;
    const int2 before = block_exclusive_scan_sum_max(cost_sum, last_ne, s_scan2, &total);
    const int cost_before = before.x, ne_before = before.y;
    {
        int run = cost_before, prev = ne_before;
        for (int q = b0; q < e0; ++q) {
            s_cum[q] = run;
            run += s_T[q] > 0 ? C + s_T[q] : 0;
            if (s_T[q] > 0) prev = q;
            s_prev[q] = prev;
        }
        if (tid == 0) s_cum[Q] = total;
    }
    int W = total > 0 ? (total + p.num_parts - 1) / p.num_parts : 1;
    W = max(W, max(p.min_payload, 1));

    // split counts (distinct parts among a unit's tiles) and their prefix sums
    int ns_sum = 0;
    for (int q = b0; q < e0; ++q) {
        const int T = s_T[q];
        if (T > 0) {
            const int x0 = s_cum[q] + C;
            ns_sum += (x0 + T - 1) / W - x0 / W + 1;
        }
    }
    int total_splits;
    const int ns_before = block_exclusive_scan<kSum>(ns_sum, 0, s_scan, &total_splits);
    {
        int run = ns_before;
        for (int q = b0; q < e0; ++q) {
            p.split_offsets[q] = run;
            const int T = s_T[q];
            if (T > 0) {
                const int x0 = s_cum[q] + C;
                run += (x0 + T - 1) / W - x0 / W + 1;
            }
        }
        if (tid == 0) p.split_offsets[Q] = total_splits;
    }
    __syncthreads();  // s_cum / s_prev complete before the searches

    // Placement. The decode grid runs row r of tile_meta on XCD r / (P / 8)
    // when P % 8 == 0, so work part j goes to row (j / k) * (P / 8) + j % k,
    // k = ceil(used / 8): every XCD gets k consecutive work parts (adjacent
    // parts share a sequence, hence its q in that XCD's L2), and the rows
    // past them stay empty. Otherwise row r holds work part r.
    const int used = total > 0 ? (int)((total + W - 1) / W) : 0;  // work parts that may hold tiles
    const int per_xcd = p.num_parts >> 3;
    const bool spread = (p.num_parts & 7) == 0;
    const int kx = (used + 7) >> 3;
    for (int r = tid; r < p.num_parts; r += kMT) {
        int32_t* out = p.tile_meta + (int64_t)r * 8;
        int part = r;
        if (spread) {
            const int x = r / per_xcd, c = r - x * per_xcd;
            part = c < kx ? x * kx + c : p.num_parts;  // num_parts: no work part
        }
        const long long start = (long long)part * W;
        const long long end = start + W - 1;  // inclusive
        int row[8] = {0, 0, 0, 0, 0, 1, 0, 0};
        if (Q > 0 && part < p.num_parts && start < total) {
            const int qb = first_unit_past(s_cum, Q, (int)start);
            const int x0b = s_cum[qb] + C;
            const int tb = (int)max(0LL, start - x0b);
            int qe, te;
            if (end >= total) {
                qe = s_prev[Q - 1];
                te = s_T[qe] - 1;
            } else {
                const int qq = first_unit_past(s_cum, Q, (int)end);
                const int x0 = s_cum[qq] + C;
                if (x0 <= end) { qe = qq; te = (int)(end - x0); }
                else { qe = qq > 0 ? s_prev[qq - 1] : -1; te = qe >= 0 ? s_T[qe] - 1 : -1; }
            }
            const bool nonempty = qe >= 0 && (qb < qe || (qb == qe && tb <= te));
            if (nonempty) {
                row[0] = qb; row[1] = tb; row[2] = qe; row[3] = te;
                row[4] = part - x0b / W;
                row[5] = 0;
            }
        }
        *(int4*)out = make_int4(row[0], row[1], row[2], row[3]);
        *(int4*)(out + 4) = make_int4(row[4], row[5], row[6], row[7]);
    }
}

}  // namespace

hipError_t launch_metadata(const MetaParams& p, hipStream_t s) {
    hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kMT), 0, s, p.seqlens, p.tile_meta, p.split_offsets, p.batch,
                       p.n_rg, p.topk, p.num_parts, p.fixed_cost, p.min_payload);
    return hipGetLastError();
}

}  // namespace mla
