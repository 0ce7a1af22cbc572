// attend_bwd.hip -- segment-wise backward of the routed attention (placeholder
// until the backward kernels land: reports "not supported").
#include "hga_internal.h"

namespace hga {

size_t bwd_workspace_bytes(int64_t Hq, int64_t Hkv, int64_t n_q)
{
    (void)Hkv;
    return (size_t)(Hq * n_q) * sizeof(float);
}

hipError_t launch_attend_bwd(const uint16_t *, const uint16_t *, const uint16_t *, int64_t,
                             int64_t, int64_t, int64_t, int64_t, const int32_t *, int32_t,
                             float, const uint16_t *, const float *, const uint16_t *, float *,
                             float *, float *, void *, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace hga
