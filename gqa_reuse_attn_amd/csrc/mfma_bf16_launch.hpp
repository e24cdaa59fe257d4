// The bf16 matrix engine's kernel instantiations, included by the
// launch_mfma_bf16_*.hip translation units.
#pragma once

#include "dispatch.hpp"

namespace gqa_av_launch {
namespace detail {

template <int VDT, int PR, int NSET, int HT, bool SM, bool PG, bool QK, int NW>
hipError_t launch_mfma_bf16(const gqa_av::Pass1Args& a, hipStream_t s) {
    hipLaunchKernelGGL((gqa_av::av_pass1_mfma_bf16<PR, NSET, GQA_AV_MFMA_BF16_CHUNKS, HT, SM, VDT, PG, QK, NW>),
                       dim3(a.nblocks), dim3(64 * NW), 0, s, a);
    return hipGetLastError();
}

// Eight waves per workgroup for the plain product, and for the fused softmax
// with eight KV heads (fused attention keeps four).
template <int VDT, int PR, int NSET, int HT, bool SM, bool PG, bool QK>
hipError_t launch_mfma_bf16_nw(int nw, const gqa_av::Pass1Args& a, hipStream_t s) {
    if constexpr (HT <= 4) {
        if (nw == 4) return launch_mfma_bf16<VDT, PR, NSET, HT, SM, PG, QK, 4>(a, s);
    }
    if constexpr (!QK && (!SM || HT == 8)) {
        if (nw == 8) return launch_mfma_bf16<VDT, PR, NSET, HT, SM, PG, QK, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int VDT, int PR, int NSET, bool SM, bool PG, bool QK>
hipError_t launch_mfma_bf16_ht(int ht, int nw, const gqa_av::Pass1Args& a, hipStream_t s) {
    switch (ht) {
    case 1: return launch_mfma_bf16_nw<VDT, PR, NSET, 1, SM, PG, QK>(nw, a, s);
    case 2: return launch_mfma_bf16_nw<VDT, PR, NSET, 2, SM, PG, QK>(nw, a, s);
    case 4: return launch_mfma_bf16_nw<VDT, PR, NSET, 4, SM, PG, QK>(nw, a, s);
    case 8:
        // Eight KV heads, a wave each: not fused attention.
        if constexpr (!QK) return launch_mfma_bf16_nw<VDT, PR, NSET, 8, SM, PG, QK>(nw, a, s);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

template <int VDT, bool SM, bool PG, bool QK>
hipError_t mfma_bf16_pr(int64_t D, int nset, int ht, int nw, const gqa_av::Pass1Args& a, hipStream_t s) {
    switch (D) {
    case 64:
        return nset == 1 ? launch_mfma_bf16_ht<VDT, 8, 1, SM, PG, QK>(ht, nw, a, s)
                         : launch_mfma_bf16_ht<VDT, 8, 2, SM, PG, QK>(ht, nw, a, s);
    case 128:
        return nset == 1 ? launch_mfma_bf16_ht<VDT, 16, 1, SM, PG, QK>(ht, nw, a, s)
                         : launch_mfma_bf16_ht<VDT, 16, 2, SM, PG, QK>(ht, nw, a, s);
    case 256: return nset == 1 ? launch_mfma_bf16_ht<VDT, 32, 1, SM, PG, QK>(ht, nw, a, s) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace detail

template <int VDT, bool SM, bool PG, bool QK>
hipError_t mfma_bf16(int64_t D, int nset, int ht, int nw, const gqa_av::Pass1Args& a, hipStream_t s) {
    return detail::mfma_bf16_pr<VDT, SM, PG, QK>(D, nset, ht, nw, a, s);
}

}  // namespace gqa_av_launch
