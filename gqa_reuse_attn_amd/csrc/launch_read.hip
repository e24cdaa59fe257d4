// The plain streaming read (read_kernels.hpp), for the bandwidth ceiling.
#include "dispatch.hpp"
#include "read_kernels.hpp"

namespace gqa_av_launch {

hipError_t stream_read(const uint8_t* src, int64_t bytes, int64_t slice, int nblocks, int loads_in_flight,
                       uint32_t* sink, hipStream_t s) {
    switch (loads_in_flight) {
    case 4:
        hipLaunchKernelGGL(gqa_av::stream_read<4>, dim3(nblocks), dim3(gqa_av::kThreads), 0, s, src, bytes, slice,
                           sink);
        break;
    case 8:
        hipLaunchKernelGGL(gqa_av::stream_read<8>, dim3(nblocks), dim3(gqa_av::kThreads), 0, s, src, bytes, slice,
                           sink);
        break;
    case 16:
        hipLaunchKernelGGL(gqa_av::stream_read<16>, dim3(nblocks), dim3(gqa_av::kThreads), 0, s, src, bytes, slice,
                           sink);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gqa_av_launch
