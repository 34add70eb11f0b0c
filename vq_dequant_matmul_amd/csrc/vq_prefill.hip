// vq_prefill.hip -- grouped MFMA GEMM path for large token counts (gfx950).
#include "vq_common.hpp"
#include "vq_internal.hpp"

namespace vq {

size_t gemm_workspace_bytes(const TensorDev &, int) { return 0; }

hipError_t launch_expert_gemm(const TensorDev &, int, const void *, int, const int32_t *, float *,
                              void *, hipStream_t)
{
    return hipErrorNotSupported;
}

size_t moe_prefill_workspace_bytes(const TensorDev &, const TensorDev &, const TensorDev &, int, int)
{
    return 0;
}

hipError_t launch_moe_prefill(const TensorDev &, const TensorDev &, const TensorDev &, int, int,
                              const void *, int, const int32_t *, const float *, float *, void *,
                              hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace vq
