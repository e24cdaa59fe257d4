/*
 * gqa_bench.h -- measurement aid of libgqa_av.so: a plain streaming read.
 *
 * The AV product is bound by the rate at which a GPU streams V out of HBM
 * (ExecuTorch PR #21063, "...GEMV", introduction: the kernel is bandwidth
 * bound and V is the dominant traffic). A published peak is one bound; the
 * rate a trivial read kernel reaches on the same device, for the same number
 * of bytes, is the practical one. This entry point is that kernel. It
 * computes nothing of the product and is not part of it.
 */
#ifndef GQA_BENCH_H
#define GQA_BENCH_H

#include <stdint.h>

#include "gqa_av.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `src` once with `workgroups`
 * workgroups of 256 threads and 16-byte non-temporal loads, `loads_in_flight`
 * (4, 8 or 16) loads per lane and batch (a batch is 4, 8 or 16 KB of
 * consecutive bytes). pattern 0: each workgroup reads one contiguous slice of
 * ceil(bytes / workgroups) bytes (rounded up to 16), two batches in flight;
 * pattern 1: batch j goes to workgroup j mod workgroups (grid stride), one
 * batch in flight, and a tail shorter than a batch is not read. The loaded
 * words are folded into one value per workgroup, which is written to
 * sink[0..255] only if it equals a fixed 32-bit constant (so the loads cannot
 * be dropped); sink is otherwise untouched.
 *
 * src: device pointer, 16-byte aligned, caller-owned; bytes > 0, a multiple
 * of 16; slices must stay below 2^31 bytes. sink: device pointer to 256
 * uint32, 4-byte aligned, caller-owned. Asynchronous on `stream` (a
 * hipStream_t, NULL = default). Returns a gqa_av_status: INVALID_ARG for a
 * bad argument (nothing launched, pattern not 0 or 1 included), HIP for a
 * launch failure; details from
 * gqa_av_last_error(). */
int gqa_bench_stream_read(const void *src, int64_t bytes, int32_t workgroups, int32_t loads_in_flight,
                          int32_t pattern, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_BENCH_H */
