// vq_decode_d4.hip -- decode-engine instantiations for d = 4.
#include "vq_decode_impl.hpp"

namespace vq {

template hipError_t rows_d<4>(int, const RowsArgs &, int, int, int, int64_t, int, size_t,
                               hipStream_t);
template hipError_t dequantize_d<4>(const TensorDev &, int, float *, hipStream_t);
template hipError_t mix_d<4>(int, const MixArgs &, size_t, hipStream_t);

}  // namespace vq
