// Absorption products on either side of the decode.
//
// [Walkthrough] §六 (the absorption passage; "结果：decode 变成 MQA"): per
// head i the key up-projection folds into the query, q~_i = W^UK_i^T q^C_i
// (128 -> 512), which is what makes the decode an MQA over the 576-value
// cache row; after the decode W^UV_i maps each head's latent output back to
// 128 values. Both are batched products with the head as the batch:
// out[t, h, n] = sum_k W_h[n, k] x[t, h, k], with W_h stored row n = output n
// (for the query side that is W^UK_i transposed, arranged once when the
// weights are loaded), so both operands are contiguous along k.
//
// A workgroup (four waves) computes one head's 128 output columns for 32
// tokens. Its 128 weight rows and 32 activation rows stream in 128 k-values
// at a time with fully coalesced 16-byte loads (a thread per 16 bytes, 16
// threads per 256-byte row segment) into an LDS tile whose 16-byte chunks are
// XOR-swizzled by row, so the MFMA operand reads (32 rows at one chunk
// index) spread over all banks; the next k-chunk's loads are in flight while
// the current one's MFMAs run. Wave w multiplies weight rows 32w..32w+31 (the
// A operand, M = output column) by the 32 token rows (the B operand, N =
// token) with v_mfma_f32_32x32x16_bf16, fp32 accumulation. The 32 x 128
// result goes back through LDS so that each token's 128 outputs leave as one
// contiguous 256-byte row segment. For decode-sized token counts the bytes
// are the weights (H x 128 x 512 bf16 per product) and the activations, each
// read from HBM once: HBM-bound work. All workgroups of one head run on one
// XCD (block % 8 picks it), so the weight rows re-read by a head's token
// tiles and the activation rows re-read by its column blocks come from that
// XCD's L2.
#include "mla_absorb.h"

namespace mla {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kXcds = 8;

constexpr int kKc = 128;            // k-values per LDS stage (256-byte row segments)
constexpr int kWRows = 128;         // weight rows (output columns) per workgroup
constexpr int kTRows = 32;          // token rows per workgroup
constexpr int kRows = kWRows + kTRows;
constexpr int kPieces = kRows * kKc / 8 / 256;  // 16-byte pieces per thread per stage (10)
constexpr int kOutPitch = kWRows + 8;           // output staging row pitch (elements)

// LDS element offset of 16-byte chunk c of row r (chunks XOR-swizzled by row)
__device__ __forceinline__ int tile_at(int r, int c) { return r * kKc + ((c ^ (r & 15)) << 3); }

template <int K, int N, bool ROPE>
__global__ __launch_bounds__(256) void absorb_kernel(AbsorbParams p, int token_tiles) {
    constexpr int kStages = K / kKc;
    constexpr int kColBlocks = N / kWRows;
    __shared__ __attribute__((aligned(16))) uint16_t lds[kRows * kKc];  // 40 KB

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 31, kh = lane >> 5;

    // block -> (head, column block, token tile); with H % 8 == 0 every block
    // of a head runs on XCD (block % 8), otherwise blocks map in order
    const int per_head = kColBlocks * token_tiles;
    int h, j;
    const int id = blockIdx.x;
    if ((p.heads % kXcds) == 0) {
        const int x = id % kXcds, r = id / kXcds;
        h = (r / per_head) * kXcds + x;
        j = r % per_head;
    } else {
        h = id / per_head;
        j = id % per_head;
    }
    const int cb = j / token_tiles;
    const int n0 = cb * kWRows;
    const int64_t t0 = (int64_t)(j % token_tiles) * kTRows;

    // this thread's 16-byte pieces: piece q = tid + 256 i is chunk (q & 15) of tile row (q >> 4);
    // rows 0..127 are weight rows n0 + row, rows 128..159 token rows t0 + row - 128
    uint4 stage[kPieces];
    auto fetch = [&](int kc) {
        #pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int q = tid + 256 * i, row = q >> 4, c = q & 15;
            const uint16_t* src = nullptr;
            if (row < kWRows) {
                src = p.w + ((int64_t)h * N + n0 + row) * K + kc * kKc + c * 8;
            } else {
                const int64_t t = t0 + row - kWRows;
                if (t < p.tokens) src = p.x + (t * p.heads + h) * K + kc * kKc + c * 8;
            }
            stage[i] = src ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
        }
    };
    auto put = [&]() {
        #pragma unroll
        for (int i = 0; i < kPieces; ++i) {
            const int q = tid + 256 * i;
            *reinterpret_cast<uint4*>(lds + tile_at(q >> 4, q & 15)) = stage[i];
        }
    };

    f32x16_t acc = {};
    fetch(0);
    #pragma unroll
    for (int kc = 0; kc < kStages; ++kc) {
        if (kc > 0) __syncthreads();       // every wave is done reading the previous stage
        put();
        __syncthreads();
        if (kc + 1 < kStages) fetch(kc + 1);
        #pragma unroll
        for (int s = 0; s < kKc / 16; ++s) {
            const int c = 2 * s + kh;      // k = kc * 128 + 16 s + 8 kh + 0..7
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(lds + tile_at(32 * wave + m, c));
            const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(lds + tile_at(kWRows + m, c));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
    }

    // acc[r] = out[t0 + m, n0 + 32 wave + 8 (r / 4) + 4 kh + (r % 4)]; stage the 32 x 128 tile in LDS
    __syncthreads();
    #pragma unroll
    for (int g = 0; g < 4; ++g) {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
        const bf16x4_t v = {(__bf16)acc[4 * g], (__bf16)acc[4 * g + 1], (__bf16)acc[4 * g + 2], (__bf16)acc[4 * g + 3]};
        *reinterpret_cast<bf16x4_t*>(lds + m * kOutPitch + 32 * wave + 8 * g + 4 * kh) = v;
    }
    __syncthreads();
    #pragma unroll
    for (int i = 0; i < kTRows * kWRows / 8 / 256; ++i) {  // 2 pieces per thread
        const int q = tid + 256 * i, tok = q >> 4, c = q & 15;
        const int64_t t = t0 + tok;
        if (t < p.tokens)
            *reinterpret_cast<uint4*>(p.out + (t * p.heads + h) * p.out_stride + n0 + c * 8) =
                *reinterpret_cast<const uint4*>(lds + tok * kOutPitch + c * 8);
    }
    if (ROPE && cb == 0) {  // the query's RoPE part: 32 tokens x 128 bytes, a piece per thread
        const int tok = tid >> 3, c = tid & 7;
        const int64_t t = t0 + tok;
        if (t < p.tokens)
            *reinterpret_cast<uint4*>(p.out + (t * p.heads + h) * p.out_stride + kDv + c * 8) =
                *reinterpret_cast<const uint4*>(p.rope + (t * p.heads + h) * 64 + c * 8);
    }
}

template <int K, int N, bool ROPE>
hipError_t launch(const AbsorbParams& p, hipStream_t s) {
    const int token_tiles = (int)((p.tokens + kTRows - 1) / kTRows);
    const int64_t blocks = (int64_t)p.heads * (N / kWRows) * token_tiles;
    if (blocks >= ((int64_t)1 << 31)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((absorb_kernel<K, N, ROPE>), dim3((unsigned)blocks), dim3(256), 0, s, p, token_tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_absorb_q(const AbsorbParams& p, hipStream_t s) { return launch<128, 512, true>(p, s); }
hipError_t launch_unabsorb_o(const AbsorbParams& p, hipStream_t s) { return launch<512, 128, false>(p, s); }

}  // namespace mla
