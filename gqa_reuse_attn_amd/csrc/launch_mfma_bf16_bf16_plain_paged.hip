// bf16 matrix engine kernels, paged bf16 V, plain product.
#include "mfma_bf16_launch.hpp"

template hipError_t gqa_av_launch::mfma_bf16<gqa_av::kBF16, false, true, false>(int64_t, int, int, int, const gqa_av::Pass1Args&,
                                                                       hipStream_t);
