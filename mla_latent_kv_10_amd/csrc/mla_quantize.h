// Host/device definitions of the FP8 cache writer (quantise on write).
#pragma once

#include "mla_common.h"

namespace mla {

struct QuantParams {
    const uint16_t* src;        // bf16 bits [n, 576]
    const int32_t* slots;       // [n] absolute cache rows (page * 64 + offset)
    uint8_t* kv;                // [num_rows, 656]
    int64_t n;
    int num_rows;
};

hipError_t launch_quantize(const QuantParams& p, hipStream_t s);

}  // namespace mla
