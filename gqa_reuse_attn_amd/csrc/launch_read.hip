// The plain streaming reads (read_kernels.hpp), for the bandwidth ceiling.
#include "dispatch.hpp"
#include "read_kernels.hpp"

namespace gqa_av_launch {

namespace {

template <int U>
void launch(int pattern, const uint8_t* src, int64_t bytes, int64_t slice, int nblocks, uint32_t* sink,
            hipStream_t s) {
    if (pattern == 0)
        hipLaunchKernelGGL(gqa_av::stream_read<U>, dim3(nblocks), dim3(gqa_av::kThreads), 0, s, src, bytes, slice,
                           sink);
    else
        hipLaunchKernelGGL(gqa_av::stream_read_strided<U>, dim3(nblocks), dim3(gqa_av::kThreads), 0, s, src, bytes,
                           sink);
}

}  // namespace

hipError_t stream_read(int pattern, const uint8_t* src, int64_t bytes, int64_t slice, int nblocks,
                       int loads_in_flight, uint32_t* sink, hipStream_t s) {
    switch (loads_in_flight) {
    case 4: launch<4>(pattern, src, bytes, slice, nblocks, sink, s); break;
    case 8: launch<8>(pattern, src, bytes, slice, nblocks, sink, s); break;
    case 16: launch<16>(pattern, src, bytes, slice, nblocks, sink, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gqa_av_launch
