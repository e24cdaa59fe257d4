// Score-step kernels for f32 K.
#include "qk_launch.hpp"

template hipError_t gqa_av_launch::qk<gqa_av::kF32>(int64_t, int, const gqa_av::QkArgs&, hipStream_t);
