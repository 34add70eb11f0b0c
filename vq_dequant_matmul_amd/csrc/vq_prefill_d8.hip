// vq_prefill_d8.hip -- grouped MFMA GEMM instantiations for d = 8.
#include "vq_prefill_impl.hpp"

namespace vq {

template hipError_t gemm_d<8>(int, int, int, const GemmArgs &, int, hipStream_t);

}  // namespace vq
