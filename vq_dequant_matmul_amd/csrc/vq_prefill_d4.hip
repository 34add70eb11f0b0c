// vq_prefill_d4.hip -- grouped MFMA GEMM instantiations for d = 4.
#include "vq_prefill_impl.hpp"

namespace vq {

template hipError_t gemm_d<4>(int, int, int, const GemmArgs &, int, hipStream_t);

}  // namespace vq
