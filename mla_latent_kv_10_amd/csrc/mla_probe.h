// Host/device declarations of the measurement aids (achievable MFMA and HBM
// read rates of the GPU; not part of the decode path).
#pragma once

#include "mla_common.h"

namespace mla {

hipError_t launch_probe_mfma(int iters, int blocks, float value, float* sink, hipStream_t s);
hipError_t launch_probe_hbm_read(const void* src, int64_t bytes, int blocks, unsigned* sink, hipStream_t s);

}  // namespace mla
