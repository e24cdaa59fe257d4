// Score-step kernels for bf16 K.
#include "qk_launch.hpp"

template hipError_t gqa_av_launch::qk<gqa_av::kBF16>(int64_t, int, const gqa_av::QkArgs&, hipStream_t);
