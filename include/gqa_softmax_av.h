/*
 * gqa_softmax_av.h -- C ABI of the fused softmax and attention-times-V product
 * in libgqa_av.so (MI355X, gfx950).
 *
 * The operation: the page's weights (ExecuTorch PR #21063, "...GEMV",
 * introduction) are, in decode attention, a softmax over the context of the
 * step's scores. This call takes the scores and applies that softmax inside
 * the product, so the [B][C][Hq] weights never travel through memory:
 *
 *     out[b, q_h, d] = sum_{c < C} p[b, c, q_h] * V[b, c, kv_h, d],    kv_h = q_h / G
 *     p[b, c, q_h]   = exp(s[b, c, q_h] - m) / sum_{c' < C} exp(s[b, c', q_h] - m)
 *     m              = max_{c < C} s[b, c, q_h]
 *
 * The page gives no softmax; the plain definition above is taken. Reuse and
 * per-head modes are those of gqa_av.h (each V row read once per group, or
 * once per query head as the measured baseline).
 *
 * Memory layout: scores [B][C][Hq] float32 -- the layout of gqa_av.h's attn
 * and of gqa_qk_decode's output -- and V, out as in gqa_av.h. All DEVICE
 * pointers on the current HIP device, owned by the caller; scores and out
 * 4-byte aligned, V aligned to its element size.
 *
 * Values: a score of -inf gives weight 0 (a mask); a (b, q_h) whose scores
 * are all -inf gives NaN (0 / 0), as the definition does; NaN or +inf scores
 * give NaN. C == 0 writes zeros (an empty sum, as gqa_av_decode does).
 *
 * Arithmetic: float32. Each weight is exp2((s - r) * log2(e)) with r a
 * running maximum of the scores one lane (or wave) has seen -- the difference
 * first, so the weight's error grows with s - r and not with the size of the
 * scores -- and when r grows the running sums are rescaled. Splits of the
 * context keep their own maximum and weight sum and are merged by the
 * combine kernel with the log-sum-exp rule. The products weight * V and the
 * sums are fp32 as in gqa_av.h (the bf16 matrix engine splits each weight
 * exactly into three bf16 terms); the result is the weighted sum divided once
 * by the weight sum.
 *
 * Plans, workspace, asynchrony, errors and threading are as in gqa_av.h. A
 * plan for this call comes from gqa_av_make_plan with hint->softmax = 1 and
 * carries plan->softmax = 1: its engine is GQA_AV_ENGINE_VALU or
 * GQA_AV_ENGINE_MFMA_BF16 (forcing GQA_AV_ENGINE_MFMA is UNSUPPORTED), its
 * combine GQA_AV_COMBINE_KERNEL, at most 4 KV
 * heads per tile. gqa_av_decode_plan and its split entry points refuse such a
 * plan (INVALID_ARG), and this call refuses the others.
 */
#ifndef GQA_SOFTMAX_AV_H
#define GQA_SOFTMAX_AV_H

#include <stdint.h>

#include "gqa_av.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out = softmax over c of scores, times V, as defined above, with an
 * automatic plan for the current device. Sizes as in gqa_av_decode. */
int gqa_softmax_av_decode(const float *scores, const void *V, float *out,
                          int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                          int v_dtype, int mode, void *stream);

/* Same, with an explicit fused softmax plan (plan->softmax == 1) from
 * gqa_av_make_plan for the same problem; GQA_AV_ERR_INVALID_ARG if the plan
 * does not match it. */
int gqa_softmax_av_decode_plan(const float *scores, const void *V, float *out,
                               int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                               int v_dtype, const gqa_av_plan *plan, void *stream);

/* The two launches of gqa_softmax_av_decode_plan, for callers that schedule
 * or time them separately (same arguments and checks; see
 * gqa_av_decode_pass1): pass 1 writes `out` when plan->nsplit == 1, else it
 * leaves each split's partial sums and (maximum, weight sum) statistics in
 * the workspace of (current device, stream), and the combine, enqueued next
 * on the same stream, merges them into `out`. */
int gqa_softmax_av_decode_pass1(const float *scores, const void *V, float *out,
                                int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                                int v_dtype, const gqa_av_plan *plan, void *stream);
int gqa_softmax_av_decode_combine(const float *scores, const void *V, float *out,
                                  int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                                  int v_dtype, const gqa_av_plan *plan, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_SOFTMAX_AV_H */
