// vq_decode_d8.hip -- decode-engine instantiations for d = 8.
#include "vq_decode_impl.hpp"

namespace vq {

template hipError_t rows_d<8>(int, const RowsArgs &, int, int, bool, int64_t, int, size_t,
                               hipStream_t);
template hipError_t dequantize_d<8>(const TensorDev &, int, float *, hipStream_t);
template hipError_t mix_d<8>(int, const MixArgs &, size_t, hipStream_t);

}  // namespace vq
