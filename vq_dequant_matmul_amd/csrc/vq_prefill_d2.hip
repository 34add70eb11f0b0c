// vq_prefill_d2.hip -- grouped MFMA GEMM instantiations for d = 2.
#include "vq_prefill_impl.hpp"

namespace vq {

template hipError_t gemm_d<2>(int, int, int, const GemmArgs &, int, hipStream_t);

}  // namespace vq
