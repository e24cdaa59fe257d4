/*
 * gqa_attention.h -- C ABI of fused GQA decode attention in libgqa_av.so
 * (MI355X, gfx950): the score step, the softmax and the attention-times-V
 * product in one pass over K and V.
 *
 * The operation: the page (ExecuTorch PR #21063, "...GEMV", introduction)
 * covers the product of the softmax weights with V; the weights are the
 * softmax over the context of the decode step's scores. This call computes
 * the scores from q and K itself, so neither scores nor weights travel
 * through memory:
 *
 *     out[b, q_h, d] = sum_{c < C} p[b, c, q_h] * V[b, c, kv_h, d],    kv_h = q_h / G
 *     p[b, c, q_h]   = softmax over c of s[b, c, q_h]
 *     s[b, c, q_h]   = scale * sum_{d < D} q[b, q_h, d] * K[b, c, kv_h, d]
 *
 * Each K and V row is read once for the G query heads of its group (reuse
 * mode only: mode GQA_AV_PER_HEAD, or GQA_AV_AUTO with G = 1, is
 * GQA_AV_ERR_UNSUPPORTED; GQA_AV_REUSE with G = 1 is GQA_AV_ERR_INELIGIBLE as
 * in gqa_av.h).
 *
 * Memory layout: q [B][Hq][D] float32; K and V [B][C][Hkv][D] bfloat16
 * (kv_dtype GQA_AV_BF16; fp8 below); out [B][Hq][D] float32. All DEVICE pointers on the
 * current HIP device, owned by the caller; q and out 4-byte aligned, K and V
 * 16-byte aligned. D must be 64, 128 or 256; otherwise GQA_AV_ERR_UNSUPPORTED.
 *
 * Arithmetic: float32. The scores come from the matrix cores with each q
 * value split exactly into three bfloat16 terms (every product exact, fp32
 * sums), times scale; the softmax and the product are those of
 * gqa_softmax_av.h (online maximum per wave, log-sum-exp merge of context
 * splits in the combine kernel). C == 0 writes zeros.
 *
 * Plans: gqa_av_make_plan with hint->attention = 1 (kv_dtype as v_dtype); the
 * plan carries plan->attention = 1 and plan->softmax = 1 and runs only on
 * this header's _plan entry point. Workspace, asynchrony, errors and threading
 * are as in gqa_av.h.
 */
#ifndef GQA_ATTENTION_H
#define GQA_ATTENTION_H

#include <stdint.h>

#include "gqa_av.h"

#ifdef __cplusplus
extern "C" {
#endif

/* out as defined above, with an automatic plan for the current device. */
int gqa_attention_decode(const float *q, const void *K, const void *V, float *out,
                         int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                         int kv_dtype, float scale, int mode, void *stream);

/* Same, with an explicit plan (plan->attention == 1); GQA_AV_ERR_INVALID_ARG
 * if it does not match the problem. */
int gqa_attention_decode_plan(const float *q, const void *K, const void *V, float *out,
                              int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                              int kv_dtype, float scale, const gqa_av_plan *plan, void *stream);

/* The two launches of gqa_attention_decode_plan, for callers that schedule or
 * time them separately: same arguments, checks and order as
 * gqa_av_decode_pass1 / gqa_av_decode_combine (gqa_av.h). */
int gqa_attention_decode_pass1(const float *q, const void *K, const void *V, float *out,
                               int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                               int kv_dtype, float scale, const gqa_av_plan *plan, void *stream);
int gqa_attention_decode_combine(const float *q, const void *K, const void *V, float *out,
                                 int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                                 int kv_dtype, float scale, const gqa_av_plan *plan, void *stream);

/* fp8 K and V (an fp8 KV cache, not on the page): K and V hold OCP FP8 E4M3
 * bytes [B][C][Hkv][D] (8-byte aligned) with float32 scales per KV head,
 * k_scale and v_scale [Hkv] on the device (NULL: 1): each element is
 * decode(byte) * scale[kv_h]. The values widen exactly to bfloat16 and run
 * as above; k_scale joins scale on the scores, v_scale multiplies each
 * output once. Plans: gqa_av_make_plan with hint->attention = 1 and v_dtype
 * GQA_AV_FP8_E4M3. */
int gqa_attention_fp8_decode(const float *q, const void *K, const float *k_scale, const void *V,
                             const float *v_scale, float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                             int64_t D, float scale, int mode, void *stream);
int gqa_attention_fp8_decode_plan(const float *q, const void *K, const float *k_scale, const void *V,
                                  const float *v_scale, float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                  int64_t D, float scale, const gqa_av_plan *plan, void *stream);
int gqa_attention_fp8_decode_pass1(const float *q, const void *K, const float *k_scale, const void *V,
                                   const float *v_scale, float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                   int64_t D, float scale, const gqa_av_plan *plan, void *stream);
int gqa_attention_fp8_decode_combine(const float *q, const void *K, const float *k_scale, const void *V,
                                     const float *v_scale, float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                     int64_t D, float scale, const gqa_av_plan *plan, void *stream);

/* A paged K and V cache (the serving layout; not on the page): K and V each
 * live in a page pool [num_pages][page_size][Hkv][D] of kv_dtype (bf16, or
 * fp8 E4M3 with k_scale and v_scale as above; with bf16 both scales must be
 * NULL), and the two pools share one block table: row c of sequence b is row
 * c mod page_size of page block_table[b][c / page_size] in both. block_table
 * [B][max_pages] and seq_lens [B] are int32 device arrays; only rows
 * c < seq_lens[b] take part, and a length of 0 writes zeros. C is the
 * capacity (C <= max_pages * page_size; lengths are clamped into [0, C] and
 * table entries into [0, num_pages) on the device, so a bad table gives wrong
 * numbers, never a fault, as in gqa_paged_av.h). page_size is a power of two;
 * the pools are aligned as K and V above. Plans: gqa_av_make_plan with
 * hint->attention = 1 and hint->page_size = page_size. */
int gqa_attention_paged_decode(const float *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                               const int32_t *seq_lens, const float *k_scale, const float *v_scale, float *out,
                               int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t max_pages, int64_t num_pages, int kv_dtype, float scale, int mode,
                               void *stream);
int gqa_attention_paged_decode_plan(const float *q, const void *k_pages, const void *v_pages,
                                    const int32_t *block_table, const int32_t *seq_lens, const float *k_scale,
                                    const float *v_scale, float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                    int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages, int kv_dtype,
                                    float scale, const gqa_av_plan *plan, void *stream);
int gqa_attention_paged_decode_pass1(const float *q, const void *k_pages, const void *v_pages,
                                     const int32_t *block_table, const int32_t *seq_lens, const float *k_scale,
                                     const float *v_scale, float *out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                     int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages, int kv_dtype,
                                     float scale, const gqa_av_plan *plan, void *stream);
int gqa_attention_paged_decode_combine(const float *q, const void *k_pages, const void *v_pages,
                                       const int32_t *block_table, const int32_t *seq_lens, const float *k_scale,
                                       const float *v_scale, float *out, int64_t B, int64_t C, int64_t Hq,
                                       int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages,
                                       int64_t num_pages, int kv_dtype, float scale, const gqa_av_plan *plan,
                                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTENTION_H */
