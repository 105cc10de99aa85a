// Split-KV work schedule kernel.
//
// Role from [Walkthrough] §七 "split-KV：把长序列切开": once per decode step,
// decide which row-group sequences and which 64-token tiles each part (one
// workgroup of the decode grid) processes, and how many splits each
// sequence has; every layer reuses the result. The rule (see include/mla.h):
// units laid end to end, fixed_cost positions then one per tile, part =
// floor(position / W). One workgroup computes it in parallel: two block
// scans (positions, split counts), then a binary search per part.
#include "mla_common.h"

namespace mla {

namespace {

constexpr int kMT = 256;

// Exclusive scan of vals[0..n) in place (LDS), returning the total. Each
// thread owns one contiguous chunk; chunk sums are scanned by thread 0.
__device__ int block_exclusive_scan(int* vals, int n, int* chunk_sums) {
    const int tid = threadIdx.x;
    const int per = (n + kMT - 1) / kMT;
    const int b = tid * per;
    const int e = min(n, b + per);
    int s = 0;
    for (int k = b; k < e; ++k) s += vals[k];
    chunk_sums[tid] = s;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int k = 0; k < kMT; ++k) { int v = chunk_sums[k]; chunk_sums[k] = run; run += v; }
        chunk_sums[kMT] = run;
    }
    __syncthreads();
    int run = chunk_sums[tid];
    for (int k = b; k < e; ++k) { int v = vals[k]; vals[k] = run; run += v; }
    __syncthreads();
    return chunk_sums[kMT];
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

__global__ __launch_bounds__(kMT) void metadata_kernel(MetaParams p) {
    __shared__ int s_cum[kMaxUnits + 1];    // positions: exclusive scan of per-unit cost
    __shared__ int s_T[kMaxUnits];          // tiles per unit
    __shared__ int s_prev[kMaxUnits];       // last non-empty unit at or before q (-1 if none)
    __shared__ int s_ns[kMaxUnits];         // splits per unit, then their exclusive prefix sums
    __shared__ int s_chunk[kMT + 1];
    const int Q = p.batch * p.n_rg;
    const int tid = threadIdx.x;
    const int C = p.fixed_cost;

    for (int q = tid; q < Q; q += kMT) {
        int T;
        if (p.topk > 0) {
            T = (p.topk + kBlock - 1) / kBlock;
        } else {
            int L = p.seqlens[q / p.n_rg];
            T = L > 0 ? (L + kBlock - 1) / kBlock : 0;
        }
        s_T[q] = T;
        s_cum[q] = T > 0 ? C + T : 0;
    }
    __syncthreads();
    const int total = block_exclusive_scan(s_cum, Q, s_chunk);
    if (tid == 0) s_cum[Q] = total;
    // last non-empty unit at or before q, by a sequential pass over chunks
    {
        const int per = (Q + kMT - 1) / kMT;
        const int b = tid * per, e = min(Q, b + per);
        int last = -1;
        for (int k = b; k < e; ++k) if (s_T[k] > 0) last = k;
        s_chunk[tid] = last;
        __syncthreads();
        if (tid == 0) {
            int run = -1;
            for (int k = 0; k < kMT; ++k) { int v = s_chunk[k]; s_chunk[k] = run; if (v >= 0) run = v; }
        }
        __syncthreads();
        int run = s_chunk[tid];
        for (int k = b; k < e; ++k) { if (s_T[k] > 0) run = k; s_prev[k] = run; }
        __syncthreads();
    }
    int W = total > 0 ? (total + p.num_parts - 1) / p.num_parts : 1;
    W = max(W, max(p.min_payload, 1));

    // split counts (distinct parts among a unit's tiles), then their prefix sums
    for (int q = tid; q < Q; q += kMT) {
        int T = s_T[q];
        int ns = 0;
        if (T > 0) {
            int x0 = s_cum[q] + C;
            ns = (x0 + T - 1) / W - x0 / W + 1;
        }
        s_ns[q] = ns;
    }
    __syncthreads();
    const int total_splits = block_exclusive_scan(s_ns, Q, s_chunk);
    for (int q = tid; q < Q; q += kMT) p.split_offsets[q] = s_ns[q];
    if (tid == 0) p.split_offsets[Q] = total_splits;

    for (int part = tid; part < p.num_parts; part += kMT) {
        int32_t* out = p.tile_meta + (int64_t)part * 8;
        const long long start = (long long)part * W;
        const long long end = start + W - 1;  // inclusive
        int row[8] = {0, 0, 0, 0, 0, 1, 0, 0};
        if (Q > 0 && start < total) {
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
        for (int k = 0; k < 8; ++k) out[k] = row[k];
    }
}

}  // namespace

hipError_t launch_metadata(const MetaParams& p, hipStream_t s) {
    hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kMT), 0, s, p);
    return hipGetLastError();
}

}  // namespace mla
