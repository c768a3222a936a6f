// Launch of the lse merge kernel (lse_merge.hip), shared with the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace splash {

// dtypes: 0 = bf16, 1 = f32.  dv % 8 == 0 and 64 % (dv / 8) == 0.
hipError_t launch_lse_merge(const void *oa, const float *la, int dta, const void *ob, const float *lb, int dtb,
                            void *oo, float *lo, int dto, int64_t rows, int dv, hipStream_t stream);

}  // namespace splash
