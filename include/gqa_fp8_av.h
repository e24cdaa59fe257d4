/*
 * gqa_fp8_av.h -- C ABI of the attention-times-V product (and its fused
 * softmax form) over an fp8 V cache with a scale per KV head, in libgqa_av.so
 * (MI355X, gfx950).
 *
 * The operation is the page's (ExecuTorch PR #21063, "...GEMV",
 * introduction): out[b, q_h, d] = sum_c w[b, c, q_h] * V[b, c, kv_h, d],
 * kv_h = q_h / G, each V row read once for its group in reuse mode -- or the
 * fused softmax form of gqa_softmax_av.h when softmax = 1 (w then holds the
 * scores). Here V is stored compressed, which the page does not cover:
 *
 *   V        [B][C][Hkv][D] bytes in OCP FP8 E4M3 (1 sign bit, 4 exponent bits
 *            with bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN),
 *   v_scale  [Hkv] float32 or NULL (all 1): element value = decode(byte) * v_scale[kv_h].
 *
 * half the bytes of a bf16 cache. w [B][C][Hq] and out [B][Hq][D] float32 as
 * in gqa_av.h. All DEVICE pointers on the current HIP device, owned by the
 * caller; v_scale 4-byte aligned, V aligned to the plan's lane loads (2 to
 * 16 bytes: 16 only for tiles of up to 4 query heads; D even).
 *
 * Arithmetic: gfx950 widens fp8 to fp32 exactly (v_cvt_pk_f32_fp8), the
 * products with the fp32 weights and the sums are fp32 as in gqa_av.h, and
 * each output is multiplied by its KV head's scale once (the sums are linear
 * in V, so this equals scaling every element, up to that one rounding).
 *
 * Plans come from gqa_av_make_plan with v_dtype = GQA_AV_FP8_E4M3 (and
 * hint->softmax for the fused form): the VALU engine. Paged fp8 caches are not supported. gqa_av_decode and
 * gqa_softmax_av_decode also take GQA_AV_FP8_E4M3 V, with unit scales.
 * Modes, workspace, asynchrony, errors and threading are as in gqa_av.h.
 */
#ifndef GQA_FP8_AV_H
#define GQA_FP8_AV_H

#include <stdint.h>

#include "gqa_av.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out as defined above, with an automatic plan for the current device. */
int gqa_av_fp8_decode(const float *w, const void *V, const float *v_scale, float *out,
                      int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                      int softmax, int mode, void *stream);

/* Same, with an explicit plan (v_dtype GQA_AV_FP8_E4M3; plan->softmax selects
 * the fused form); GQA_AV_ERR_INVALID_ARG if it does not match the problem. */
int gqa_av_fp8_decode_plan(const float *w, const void *V, const float *v_scale, float *out,
                           int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                           const gqa_av_plan *plan, void *stream);

/* The two launches of gqa_av_fp8_decode_plan, for callers that schedule or
 * time them separately: same arguments, checks and order as
 * gqa_av_decode_pass1 / gqa_av_decode_combine (gqa_av.h); `out` is complete
 * only after the combine. */
int gqa_av_fp8_decode_pass1(const float *w, const void *V, const float *v_scale, float *out,
                            int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                            const gqa_av_plan *plan, void *stream);
int gqa_av_fp8_decode_combine(const float *w, const void *V, const float *v_scale, float *out,
                              int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                              const gqa_av_plan *plan, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_FP8_AV_H */
