// Host/device definitions of the absorption products around the decode.
#pragma once

#include "mla_common.h"

namespace mla {

// out[t, h, :N] = W_h x[t, h, :K] for every token t and head h, W_h = w[h] stored
// [N, K] (row n holds the K weights of output n); optionally out[t, h, 512:576]
// = rope[t, h, :64].
struct AbsorbParams {
    const uint16_t* x;      // bf16 [T, H, K]
    const uint16_t* w;      // bf16 [H, N, K]
    const uint16_t* rope;   // bf16 [T, H, 64] or null
    uint16_t* out;          // bf16 [T, H, out_stride]
    int64_t tokens;
    int heads;
    int out_stride;
};

hipError_t launch_absorb_q(const AbsorbParams& p, hipStream_t s);    // K = 128, N = 512, RoPE copied
hipError_t launch_unabsorb_o(const AbsorbParams& p, hipStream_t s);  // K = 512, N = 128

}  // namespace mla
