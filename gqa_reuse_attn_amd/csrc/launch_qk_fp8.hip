// Score-step kernels for fp8 (OCP E4M3) K.
#include "qk_launch.hpp"

template hipError_t gqa_av_launch::qk<gqa_av::kFP8>(int64_t, int, const gqa_av::QkArgs&, hipStream_t);
