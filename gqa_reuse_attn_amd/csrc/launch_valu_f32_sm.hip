// VALU engine kernels for f32 V, fused softmax.
#include "valu_launch.hpp"

template hipError_t gqa_av_launch::valu<gqa_av::kF32, true>(int, int, bool, const gqa_av::Pass1Args&, hipStream_t);
