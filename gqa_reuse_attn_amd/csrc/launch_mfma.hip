// fp32 matrix engine kernels.
#include "dispatch.hpp"

namespace gqa_av_launch {
namespace {

template <int DT, int DE, int NSET>
hipError_t launch_mfma(const gqa_av::Pass1Args& a, hipStream_t s) {
    constexpr int U = gqa_av::mfma_unroll(DE * gqa_av::esize<DT>());
    hipLaunchKernelGGL((gqa_av::av_pass1_mfma<DT, DE, NSET, U>), dim3(a.nblocks), dim3(gqa_av::kThreads), 0, s, a);
    return hipGetLastError();
}

template <int DT, int DE>
hipError_t launch_mfma_set(int nset, const gqa_av::Pass1Args& a, hipStream_t s) {
    if (nset == 1) return launch_mfma<DT, DE, 1>(a, s);
    if constexpr (DE <= 8) {
        if (nset == 2) return launch_mfma<DT, DE, 2>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_mfma_de(int DE, int nset, const gqa_av::Pass1Args& a, hipStream_t s) {
    switch (DE) {
    case 2: return launch_mfma_set<DT, 2>(nset, a, s);
    case 4: return launch_mfma_set<DT, 4>(nset, a, s);
    case 6:
        if constexpr (DT != gqa_av::kF32) return launch_mfma_set<DT, 6>(nset, a, s);
        return hipErrorInvalidValue;
    case 8: return launch_mfma_set<DT, 8>(nset, a, s);
    case 16:
        if constexpr (DT != gqa_av::kF32) return launch_mfma_set<DT, 16>(nset, a, s);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t mfma(int DT, int DE, int nset, const gqa_av::Pass1Args& a, hipStream_t s) {
    switch (DT) {
    case gqa_av::kF32: return launch_mfma_de<gqa_av::kF32>(DE, nset, a, s);
    case gqa_av::kF16: return launch_mfma_de<gqa_av::kF16>(DE, nset, a, s);
    case gqa_av::kBF16: return launch_mfma_de<gqa_av::kBF16>(DE, nset, a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gqa_av_launch
