// Kernel launches of libgqa_av.so, one entry per engine. Each is defined in a
// translation unit of its own (launch_*.hip) that instantiates only its
// engine's kernels, so the library's kernels compile in parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "av_kernels.hpp"
#include "qk_kernels.hpp"

namespace gqa_av_launch {

// VALU engine, element type DT (gqa_av::kF32 ...), fused softmax SM: VB-byte
// lane loads, GT heads per tile, paged V when `paged` (16-byte loads only).
template <int DT, bool SM>
hipError_t valu(int VB, int GT, bool paged, const gqa_av::Pass1Args& a, hipStream_t s);

// fp32 matrix engine: DE = D / 16 values per lane, nset sets of 16 heads.
hipError_t mfma(int DT, int DE, int nset, const gqa_av::Pass1Args& a, hipStream_t s);

// bf16 matrix engine, V of element type VDT (gqa_av::kBF16 or kFP8), paged V
// when PG, fused attention (scores from q and K) when QK: D of 64, 128 or
// 256, nset sets of 16 heads, ht KV heads per tile (1, 2, 4 or 8), nw waves
// per workgroup (4, or 8 for the plain product or eight KV heads per tile).
template <int VDT, bool SM, bool PG = false, bool QK = false>
hipError_t mfma_bf16(int64_t D, int nset, int ht, int nw, const gqa_av::Pass1Args& a, hipStream_t s);

// Score step, K of element type KDT: D / 32 blocks, nset sets of 16 heads.
template <int KDT>
hipError_t qk(int64_t D, int nset, const gqa_av::QkArgs& a, hipStream_t s);

// Plain streaming read of `bytes` from src (the bandwidth ceiling): nblocks
// workgroups, loads_in_flight 16-byte loads per lane and batch (4, 8 or 16);
// pattern 0: `slice` contiguous bytes per workgroup; 1: grid-stride batches.
hipError_t stream_read(int pattern, const uint8_t* src, int64_t bytes, int64_t slice, int nblocks,
                       int loads_in_flight, uint32_t* sink, hipStream_t s);

}  // namespace gqa_av_launch
