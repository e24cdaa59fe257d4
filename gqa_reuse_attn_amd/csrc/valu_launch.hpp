// The VALU engine's kernel instantiations, included by the launch_valu_*.hip
// translation units (one per element type and softmax flag).
#pragma once

#include "dispatch.hpp"

namespace gqa_av_launch {
namespace detail {

template <int DT, int VB, int GT, bool SM, bool PG>
hipError_t launch_valu(const gqa_av::Pass1Args& a, hipStream_t s) {
    constexpr int U = gqa_av::valu_unroll(GT, DT, SM, PG);
    hipLaunchKernelGGL((gqa_av::av_pass1_valu<DT, VB, GT, U, SM, PG>), dim3(a.nblocks), dim3(gqa_av::kThreads), 0, s,
                       a);
    return hipGetLastError();
}

template <int DT, int VB, bool SM, bool PG = false>
hipError_t launch_valu_gt(int GT, const gqa_av::Pass1Args& a, hipStream_t s) {
    switch (GT) {
    case 1: return launch_valu<DT, VB, 1, SM, PG>(a, s);
    case 2: return launch_valu<DT, VB, 2, SM, PG>(a, s);
    case 3: return launch_valu<DT, VB, 3, SM, PG>(a, s);
    case 4: return launch_valu<DT, VB, 4, SM, PG>(a, s);
    default: break;
    }
    // fp8 with 16-byte lane loads (16 values) only for tiles of up to 4 heads.
    if constexpr (DT == gqa_av::kFP8 && VB == 16) {
        return hipErrorInvalidValue;
    } else {
        switch (GT) {
        case 5: return launch_valu<DT, VB, 5, SM, PG>(a, s);
        case 6: return launch_valu<DT, VB, 6, SM, PG>(a, s);
        case 7: return launch_valu<DT, VB, 7, SM, PG>(a, s);
        case 8: return launch_valu<DT, VB, 8, SM, PG>(a, s);
        case 16: return launch_valu<DT, VB, 16, SM, PG>(a, s);
        default: return hipErrorInvalidValue;
        }
    }
}

template <int DT, bool SM>
hipError_t launch_valu_vb(int VB, int GT, const gqa_av::Pass1Args& a, hipStream_t s) {
    switch (VB) {
    case 16: return launch_valu_gt<DT, 16, SM>(GT, a, s);
    case 8: return launch_valu_gt<DT, 8, SM>(GT, a, s);
    case 4: return launch_valu_gt<DT, 4, SM>(GT, a, s);
    case 2:
        if constexpr (DT != gqa_av::kF32) return launch_valu_gt<DT, 2, SM>(GT, a, s);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace detail

template <int DT, bool SM>
hipError_t valu(int VB, int GT, bool paged, const gqa_av::Pass1Args& a, hipStream_t s) {
    if (paged)   // paged V: 16-byte lane loads only (fp8: tiles of up to 4 heads)
        return VB == 16 ? detail::launch_valu_gt<DT, 16, SM, true>(GT, a, s) : hipErrorInvalidValue;
    return detail::launch_valu_vb<DT, SM>(VB, GT, a, s);
}

}  // namespace gqa_av_launch
