// The score step's kernel instantiations, included by the launch_qk_*.hip
// translation units (one per K element type).
#pragma once

#include "dispatch.hpp"

namespace gqa_av_launch {
namespace detail {

template <int KDT, int NBLK, int NSET, bool PG>
hipError_t launch_qk_pg(const gqa_av::QkArgs& a, hipStream_t s) {
    const dim3 grid(a.nblocks), block(gqa_av::kThreads);
    switch (a.ht) {
    case 1: hipLaunchKernelGGL((gqa_av::qk_scores<KDT, NBLK, NSET, 1, PG>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gqa_av::qk_scores<KDT, NBLK, NSET, 2, PG>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gqa_av::qk_scores<KDT, NBLK, NSET, 4, PG>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Paged K when the arguments carry a block table.
template <int KDT, int NBLK, int NSET>
hipError_t launch_qk_ht(const gqa_av::QkArgs& a, hipStream_t s) {
    return a.block_table ? launch_qk_pg<KDT, NBLK, NSET, true>(a, s) : launch_qk_pg<KDT, NBLK, NSET, false>(a, s);
}

template <int KDT, int NBLK>
hipError_t launch_qk_nset(int nset, const gqa_av::QkArgs& a, hipStream_t s) {
    if constexpr (KDT == gqa_av::kFP8 && NBLK % 2 != 0) {
        return hipErrorInvalidValue;                 // fp8 K: D a multiple of 64 (the plan checks it)
    } else {
        if (nset == 1) return launch_qk_ht<KDT, NBLK, 1>(a, s);
        if constexpr (NBLK <= 4) {
            if (nset == 2) return launch_qk_ht<KDT, NBLK, 2>(a, s);
        }
        return hipErrorInvalidValue;
    }
}

template <int KDT>
hipError_t launch_qk_nblk(int64_t D, int nset, const gqa_av::QkArgs& a, hipStream_t s) {
    switch (D / 32) {
    case 1: return launch_qk_nset<KDT, 1>(nset, a, s);
    case 2: return launch_qk_nset<KDT, 2>(nset, a, s);
    case 3: return launch_qk_nset<KDT, 3>(nset, a, s);
    case 4: return launch_qk_nset<KDT, 4>(nset, a, s);
    case 5: return launch_qk_nset<KDT, 5>(nset, a, s);
    case 6: return launch_qk_nset<KDT, 6>(nset, a, s);
    case 7: return launch_qk_nset<KDT, 7>(nset, a, s);
    case 8: return launch_qk_nset<KDT, 8>(nset, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace detail

template <int KDT>
hipError_t qk(int64_t D, int nset, const gqa_av::QkArgs& a, hipStream_t s) {
    return detail::launch_qk_nblk<KDT>(D, nset, a, s);
}

}  // namespace gqa_av_launch
