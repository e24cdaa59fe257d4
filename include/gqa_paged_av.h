/*
 * gqa_paged_av.h -- C ABI of the attention-times-V product (and its fused
 * softmax form) over a paged V cache, in libgqa_av.so (MI355X, gfx950).
 *
 * The operation is the page's (ExecuTorch PR #21063, "...GEMV",
 * introduction) -- out[b, q_h, d] = sum_c w[b, c, q_h] * V[b, c, kv_h, d],
 * kv_h = q_h / G, each V row read once for its group in reuse mode -- or the
 * fused softmax form of gqa_softmax_av.h, with V held the way decode servers
 * keep their caches (a layout the page does not cover):
 *
 *   pages        [num_pages][page_size][Hkv][D] of v_dtype: fixed-size blocks
 *                of consecutive context rows, shared by all sequences;
 *   block_table  [B][max_pages] int32: row c of sequence b is row
 *                c % page_size of page block_table[b][c / page_size];
 *   seq_lens     [B] int32: sequence b has seq_lens[b] rows; only rows
 *                c < seq_lens[b] take part (a length of 0 gives zeros).
 *
 * The weights -- or, with softmax, the scores -- keep the dense layout
 * w [B][C][Hq] float32, C being the capacity (C <= max_pages * page_size);
 * out [B][Hq][D] float32. A dense cache V[B][C][Hkv][D] with per-sequence
 * lengths is the case page_size = C, block_table[b][0] = b, when C is a power
 * of two; for any capacity it is pages of one row, block_table[b][c] =
 * b * C + c (or, with every sequence at the same length,
 * gqa_av_decode_strided in gqa_av.h).
 *
 * All pointers are DEVICE pointers on the current HIP device, owned by the
 * caller. pages must be 16-byte aligned and (D * element size) a multiple of
 * 16 (whole 16-byte lane loads); page_size a power of two. block_table and
 * seq_lens live on the device, so their values are not checked on the host:
 * lengths are clamped into [0, C] and block-table entries into
 * [0, num_pages), so bad tables give wrong results, never a fault.
 *
 * Plans come from gqa_av_make_plan with hint->page_size = page_size (and
 * hint->softmax for the fused form); they carry plan->page_size and run with
 * the kernel combine on the VALU engine or, in reuse mode for bf16 or fp8 V
 * with D of 64, 128 or 256, the bf16 matrix engine (automatic for G >= 5, as
 * for dense V); never on the fp32 matrix engine. Modes, workspace,
 * asynchrony, errors and threading are as in gqa_av.h.
 */
#ifndef GQA_PAGED_AV_H
#define GQA_PAGED_AV_H

#include <stdint.h>

#include "gqa_av.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out as defined above, with an automatic plan for the current device;
 * softmax = 1 takes w as scores and applies the softmax over each sequence's
 * rows (gqa_softmax_av.h). Sizes as in gqa_av_decode, plus page_size >= 1 (a
 * power of two), max_pages >= 1 and num_pages >= 1 when B * C > 0. */
int gqa_av_paged_decode(const float *w, const void *pages, const int32_t *block_table, const int32_t *seq_lens,
                        float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                        int64_t page_size, int64_t max_pages, int64_t num_pages,
                        int v_dtype, int softmax, int mode, void *stream);

/* Same, with an explicit plan (plan->page_size == page_size; plan->softmax
 * selects the fused form); GQA_AV_ERR_INVALID_ARG if it does not match. */
int gqa_av_paged_decode_plan(const float *w, const void *pages, const int32_t *block_table,
                             const int32_t *seq_lens, float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                             int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages,
                             int v_dtype, const gqa_av_plan *plan, void *stream);

/* The two launches of gqa_av_paged_decode_plan, for callers that schedule or
 * time them separately: same arguments, checks and order as
 * gqa_av_decode_pass1 / gqa_av_decode_combine (gqa_av.h); `out` is complete
 * only after the combine. */
int gqa_av_paged_decode_pass1(const float *w, const void *pages, const int32_t *block_table,
                              const int32_t *seq_lens, float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                              int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages,
                              int v_dtype, const gqa_av_plan *plan, void *stream);
int gqa_av_paged_decode_combine(const float *w, const void *pages, const int32_t *block_table,
                                const int32_t *seq_lens, float *out, int64_t B, int64_t C, int64_t Hq,
                                int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages,
                                int v_dtype, const gqa_av_plan *plan, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PAGED_AV_H */
