/*
 * gqa_qk.h -- C ABI of the decode score step in libgqa_av.so (MI355X, gfx950).
 *
 * The operation: in grouped-query attention the Hq = G * Hkv query heads come
 * in groups of G that share one KV head (ExecuTorch PR #21063, "...GEMV",
 * introduction), and the decode step's scores are
 *
 *     scores[b, c, q_h] = scale * sum_{d < D} q[b, q_h, d] * K[b, c, kv_h, d]
 *     kv_h              = q_h / G            (integer division)
 *
 * for every sequence b < B, context position c < C and query head q_h < Hq.
 * That page covers the attention-times-V product that follows (gqa_av.h); this
 * step is not on it. It is the standard first half of decode attention with the
 * same head grouping: after a softmax over c, `scores` is the `attn` input of
 * gqa_av_decode, in the same layout. The page's reuse idea carries over: in
 * GQA_AV_REUSE mode each K row is read once for all G query heads of its
 * group; GQA_AV_PER_HEAD reads it once per query head (the measured baseline).
 * Mode values and their resolution are those of gqa_av_resolve_mode.
 *
 * Memory layout: dense, row-major, no padding or strides.
 *   q       [B][Hq][D]      float32
 *   K       [B][C][Hkv][D]  float32, float16, bfloat16 or OCP FP8 E4M3 bytes
 *                           (k_dtype, a gqa_av_dtype)
 *   scores  [B][C][Hq]      float32, fully overwritten
 * All three are DEVICE pointers on the current HIP device, owned by the caller.
 * Accumulation is in float32: with bf16 K every product q * K is exact (q is
 * split exactly into three bf16 terms) and only the sums round; with fp16 K,
 * q is scaled by a power of two and split into three fp16 terms, the products
 * are exact and the split drops less than 2^-33 of the largest q value; with
 * fp32 K the products are fp32 fused multiply-adds. The scale multiplies the
 * sum once at the end.
 *
 * fp8 K (a compressed cache, not on the page): each element is decode(byte) *
 * k_scale[kv_h], decode being OCP FP8 E4M3 (bias 7, no infinities,
 * S.1111.111 NaN) and k_scale one float32 per KV head (gqa_qk_fp8_decode; the
 * plain entry points take fp8 K with all scales 1). Every E4M3 value is a
 * bfloat16 value, so K is widened exactly and the products are exact as for
 * bf16 K; k_scale joins the scale on each head's sum.
 *
 * Requirements of this build: D a multiple of 32 (of 64 for fp8 K) and at
 * most 256, K 16-byte aligned, q, scores and k_scale 4-byte aligned; otherwise GQA_AV_ERR_UNSUPPORTED (or
 * GQA_AV_ERR_INVALID_ARG for bad sizes, as in gqa_av.h). No workspace: the
 * context is never split.
 *
 * Asynchrony, errors and threading are as in gqa_av.h: calls enqueue on
 * `stream` and return a gqa_av_status; gqa_av_last_error() gives the detail.
 */
#ifndef GQA_QK_H
#define GQA_QK_H

#include <stdint.h>

#include "gqa_av.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Optional planning hints. Zero-initialise; every field at 0 means automatic. */
typedef struct gqa_qk_hint {
    int64_t rows_per_block;  /* context rows per workgroup (rounded up to a multiple of 64) */
    int32_t cu_count;        /* compute units to plan for (make_plan: 256; decode: the device's) */
    int32_t kv_tile;         /* adjacent KV heads per workgroup in reuse mode: 1, 2 or 4 */
    int32_t page_size;       /* paged K (gqa_qk_paged_decode_plan): rows per page, a power of two; 0: dense */
    int32_t reserved[3];
} gqa_qk_hint;

/* Launch plan of the score step. */
typedef struct gqa_qk_plan {
    int32_t mode;            /* resolved: GQA_AV_PER_HEAD or GQA_AV_REUSE */
    int32_t engine;          /* GQA_AV_ENGINE_MFMA_BF16 (16-bit matrix path: bf16, fp16 and fp8 K) or GQA_AV_ENGINE_MFMA (fp32 K) */
    int32_t heads_per_tile;  /* query heads per KV head in one workgroup: 16 or 32 (reuse), 1 (per-head) */
    int32_t subgroups;       /* workgroups along the heads of one KV head (reuse: ceil(G / heads_per_tile)) */
    int64_t rows_per_block;  /* context rows per workgroup (a multiple of 64) */
    int64_t grid;            /* workgroups launched */
    int64_t k_bytes_read;    /* K bytes the plan reads from memory (G x more for per-head) */
    int32_t kv_heads_per_tile; /* adjacent KV heads one workgroup streams (reuse: 1, 2 or 4; per-head: 1) */
    int32_t page_size;         /* paged K: rows per page (rows_per_block then <= 1023 pages); 0: dense K */
    int32_t reserved[2];
} gqa_qk_plan;

/* Build the plan. Host-only: needs no GPU. hint may be NULL. Returns a gqa_av_status. */
int gqa_qk_make_plan(int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int k_dtype, int mode,
                     const gqa_qk_hint *hint, gqa_qk_plan *plan);

/* scores = scale * q . K as defined above, with an automatic plan for the
 * current device. B == 0 or C == 0 does nothing (scores is empty). */
int gqa_qk_decode(const float *q, const void *K, float *scores,
                  int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                  int k_dtype, float scale, int mode, void *stream);

/* Same, with an explicit plan from gqa_qk_make_plan for the same problem;
 * GQA_AV_ERR_INVALID_ARG if the plan does not match it. */
int gqa_qk_decode_plan(const float *q, const void *K, float *scores,
                       int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                       int k_dtype, float scale, const gqa_qk_plan *plan, void *stream);

/* fp8 K with per-KV-head scales: K holds [B][C][Hkv][D] OCP FP8 E4M3 bytes
 * and k_scale [Hkv] float32 on the device (NULL: all 1); the rest as
 * gqa_qk_decode. The _plan form takes a plan made with k_dtype
 * GQA_AV_FP8_E4M3. */
int gqa_qk_fp8_decode(const float *q, const void *K, const float *k_scale, float *scores,
                      int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                      float scale, int mode, void *stream);
int gqa_qk_fp8_decode_plan(const float *q, const void *K, const float *k_scale, float *scores,
                           int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                           float scale, const gqa_qk_plan *plan, void *stream);

/* Paged K (a decode cache layout, not on the page; the layout and tables of
 * gqa_paged_av.h): pages [num_pages][page_size][Hkv][D] of k_dtype, row c of
 * sequence b being row c % page_size of page block_table[b][c / page_size]
 * (block_table [B][max_pages] int32, seq_lens [B] int32, device data). scores
 * keeps the dense [B][C][Hq] layout with C the capacity (C <= max_pages *
 * page_size); the scores of rows c < seq_lens[b] are written as defined
 * above and the rows past each length are left as they were. k_scale [Hkv]
 * (fp8 K only; NULL: 1). page_size a power of two; lengths are clamped into
 * [0, C] and block-table entries into [0, num_pages), so bad tables give
 * wrong numbers, never a fault. The _plan form takes a plan made with
 * hint->page_size = page_size (plan->page_size). */
int gqa_qk_paged_decode(const float *q, const void *pages, const int32_t *block_table, const int32_t *seq_lens,
                        const float *k_scale, float *scores, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                        int64_t page_size, int64_t max_pages, int64_t num_pages, int k_dtype, float scale, int mode,
                        void *stream);
int gqa_qk_paged_decode_plan(const float *q, const void *pages, const int32_t *block_table, const int32_t *seq_lens,
                             const float *k_scale, float *scores, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                             int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages, int k_dtype,
                             float scale, const gqa_qk_plan *plan, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_QK_H */
