// Backward selective-scan kernels for gfx950 (recomputation-based).
#include "ss_device.h"
#include "ss_kernels.h"
#include "ss_plan.h"

namespace ss {

int64_t bwd_reduce_blocks(const Plan& p) { return (p.B * p.D + 255) / 256; }
size_t bwd_partial_bytes(const Plan& p) { return 0; }

}  // namespace ss

extern "C" int ss_bwd(const ss_dims* dims, const void*, const void*, const float*, const float*,
                      const void*, const void*, const float*, const void*, const float*,
                      const float*, const float*, float*, float*, float*, float*, float*, float*,
                      float*, float*, float*, void*, size_t, hipStream_t) {
    if (!dims) return SS_ERR_NULL;
    return SS_ERR_UNSUPPORTED;
}
