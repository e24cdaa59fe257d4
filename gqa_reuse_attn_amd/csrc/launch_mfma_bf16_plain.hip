// bf16 matrix engine kernels, plain product.
#include "mfma_bf16_launch.hpp"

template hipError_t gqa_av_launch::mfma_bf16<false>(int64_t, int, int, const gqa_av::Pass1Args&, hipStream_t);
