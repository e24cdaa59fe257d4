// VALU engine kernels for f16 V, plain product.
#include "valu_launch.hpp"

template hipError_t gqa_av_launch::valu<gqa_av::kF16, false>(int, int, bool, const gqa_av::Pass1Args&, hipStream_t);
