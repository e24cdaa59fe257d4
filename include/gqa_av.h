/*
 * gqa_av.h -- C ABI of the MI355X (gfx950) GQA decode attention-times-V library
 * (libgqa_av.so, built from gqa_reuse_attn_amd/csrc/).
 *
 * The operation (ExecuTorch PR #21063, "...GEMV" -- GQA-reuse AV coop GEMV for
 * the Vulkan backend -- introduction): in grouped-query attention the
 * Hq = G * Hkv query heads come in groups of G that share one KV head, and the
 * decode step's attention-times-V product is
 *
 *     out[b, q_h, d] = sum_{c < C} attn[b, c, q_h] * V[b, c, kv_h, d]
 *     kv_h           = q_h / G            (integer division)
 *
 * for every sequence b < B, query head q_h < Hq and d < D. The page writes it
 * without the batch index; b indexes independent sequences of equal length C.
 * attn holds already-normalised weights: no softmax, scale or mask is applied.
 *
 * Two ways to compute it, chosen by `mode` (the page's override knob, in its
 * implementation section, with the same three values):
 *   GQA_AV_REUSE     each V row is read once and used for all G query heads of
 *                    its group (the page's GQA-reuse variant).
 *   GQA_AV_PER_HEAD  each query head reads its KV head's V rows itself, so V
 *                    is read G times (the page's per-query-head shader; kept
 *                    as the measured baseline).
 *   GQA_AV_AUTO      reuse when the shape is eligible (G >= 2), per-head
 *                    otherwise (the page's dispatch bullet, without its cap of
 *                    8 on G: any G is accepted here).
 *
 * Memory layout: dense, row-major, no padding or strides (a V cache with a
 * per-sequence capacity stride: gqa_av_decode_strided below).
 *   attn  [B][C][Hq]      float32
 *   V     [B][C][Hkv][D]  float32, float16 or bfloat16 (v_dtype)
 *   out   [B][Hq][D]      float32, fully overwritten
 * All three are DEVICE pointers on the current HIP device, owned by the
 * caller; the library keeps no pointer to them after a call returns.
 * Accumulation is in float32 (fused multiply-add, round to nearest even).
 *
 * Asynchrony: gqa_av_decode* enqueue work on `stream` (a hipStream_t; NULL is
 * the default stream) and return without synchronising. The buffers must stay
 * valid until the stream has passed the call. A fault inside a kernel shows up
 * at the caller's next synchronisation, not as a return value.
 *
 * Errors: every entry point returns an int status (enum gqa_av_status) and
 * never throws. Arguments are validated before anything is launched; on an
 * error `out` is left untouched. gqa_av_last_error() gives a one-line detail
 * for the calling thread's last failing call.
 *
 * Workspace: when a plan splits the context (nsplit > 1) the library needs
 * nsplit planes of partial sums, plus, for a fused softmax plan
 * (gqa_softmax_av.h), nsplit * B * Hq pairs of floats of per-split statistics
 * (plan->workspace_bytes in total). It allocates that itself (hipMalloc) per
 * (device, stream), keeps it for reuse, and grows it on demand: the larger
 * buffer replaces the old one, which is kept (not freed) until
 * gqa_av_release(), so a HIP graph captured from an earlier call on the
 * stream stays valid. Growth allocates and is therefore refused while the
 * stream is being captured (GQA_AV_ERR_UNSUPPORTED, nothing launched): make
 * one call with the largest plan on the stream before capturing. Calls on
 * different streams never share a workspace; calls on one stream are ordered
 * by the stream. A captured graph uses the workspace of the stream it was
 * captured from, wherever it is replayed: do not replay it concurrently with
 * calls on that stream or with other replays of graphs captured from it. No
 * call clears memory with a memset.
 *
 * Thread safety: all entry points may be called from several host threads.
 */
#ifndef GQA_AV_H
#define GQA_AV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of V (and of K in gqa_qk.h, which takes the first three). attn
 * and out are always float32. */
typedef enum gqa_av_dtype {
    GQA_AV_F32 = 0,
    GQA_AV_F16 = 1,   /* IEEE binary16 */
    GQA_AV_BF16 = 2,  /* bfloat16: the upper 16 bits of a binary32 */
    GQA_AV_FP8_E4M3 = 3  /* OCP FP8 E4M3 (bias 7, no infinities, S.1111.111 = NaN): V only, on the
                            VALU and bf16 matrix engines; here with unit scale, per-KV-head scales
                            in gqa_fp8_av.h */
} gqa_av_dtype;

/* How V is shared across the query heads of a group (see above). */
typedef enum gqa_av_mode {
    GQA_AV_AUTO = -1,
    GQA_AV_PER_HEAD = 0,
    GQA_AV_REUSE = 1
} gqa_av_mode;

typedef enum gqa_av_status {
    GQA_AV_OK = 0,
    GQA_AV_ERR_INVALID_ARG = 1,  /* negative/zero sizes, Hq % Hkv != 0, bad enum, null pointer */
    GQA_AV_ERR_INELIGIBLE = 2,   /* GQA_AV_REUSE forced on a shape with G < 2 */
    GQA_AV_ERR_UNSUPPORTED = 3,  /* valid request this build cannot run (e.g. misaligned pointer for a forced plan) */
    GQA_AV_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} gqa_av_status;

/* Inner-product engine of the reuse kernel. */
typedef enum gqa_av_engine {
    GQA_AV_ENGINE_AUTO = 0,
    GQA_AV_ENGINE_VALU = 1,      /* per-lane fp32 FMAs, any G, any D */
    GQA_AV_ENGINE_MFMA = 2,      /* fp32 matrix-core tiles over 16 query heads */
    GQA_AV_ENGINE_MFMA_BF16 = 3  /* bf16 V only (D = 64, 128 or 256, V 16-byte aligned): bf16
                                    matrix-core tiles over 16 query heads and 32 rows; each fp32
                                    weight is split exactly into three bf16 terms, so every
                                    product is exact and the sums are fp32 as in the others */
} gqa_av_engine;

/* How the partial sums of a split context are added: a second kernel over
 * per-split planes, in a fixed order, so results are reproducible bit for bit.
 * (A plan without splits records AUTO.) */
typedef enum gqa_av_combine {
    GQA_AV_COMBINE_AUTO = 0,
    GQA_AV_COMBINE_KERNEL = 1    /* a second kernel over per-split planes */
} gqa_av_combine;

/* Optional planning hints. Zero-initialise, then set what you want to force:
 * every field at 0 (or below) means "choose automatically". */
typedef struct gqa_av_hint {
    int32_t engine;     /* gqa_av_engine */
    int32_t nsplit;     /* number of context splits */
    int32_t cu_count;   /* compute units to plan for; auto = the device's (decode) or 256 (make_plan) */
    int32_t v_align;    /* byte alignment of V's base address; auto = 16 */
    int32_t combine;    /* gqa_av_combine for context splits (AUTO or KERNEL; others are INVALID_ARG) */
    int32_t kv_tile;    /* adjacent KV heads per workgroup (their D-rows are contiguous), reuse mode on
                           the VALU engine (a divisor of Hkv, tile rows within 256 lanes) or the bf16
                           matrix engine (1, 2, 4; 8 for the plain product, on eight waves); a value
                           that does not divide Hkv is INVALID_ARG, other misfits UNSUPPORTED */
    int32_t softmax;    /* 1: plan the fused softmax product of gqa_softmax_av.h; 0: this header's product */
    int32_t page_size;  /* > 0: plan for a paged V cache of this many rows per page (gqa_paged_av.h) */
    int32_t attention;  /* 1: plan the fused decode attention of gqa_attention.h (implies softmax = 1) */
    int32_t waves;      /* waves (of 64 threads) per workgroup: 4, or 8 for the plain product on the bf16
                           matrix engine (eight KV heads per tile take 8: UNSUPPORTED with 4); other
                           values are INVALID_ARG */
    int32_t split_order;/* how a split context is cut: 0 automatic, 1 contiguous ranges, 2 interleaved
                           blocks (dense V on the VALU or bf16 matrix engine, not fused attention;
                           UNSUPPORTED elsewhere) */
    int32_t reserved[2];
} gqa_av_hint;

/* A launch plan: what gqa_av_decode_plan will run. Produced by gqa_av_make_plan. */
typedef struct gqa_av_plan {
    int32_t mode;            /* resolved: GQA_AV_PER_HEAD or GQA_AV_REUSE */
    int32_t engine;          /* resolved gqa_av_engine (VALU, MFMA or MFMA_BF16) */
    int32_t heads_per_tile;  /* query heads one workgroup computes (reuse: VALU 1-8 or 16; MFMA engines 16 or 32; per-head: 1) */
    int32_t subgroups;       /* workgroups that share one KV head's rows (ceil(G / heads_per_tile)) */
    int32_t vec_bytes;       /* bytes of V each lane loads per row (VALU: 16, 8, 4, 2; MFMA: D/16 elements; MFMA_BF16: 16) */
    int32_t lanes_per_row;   /* lanes covering one row of the tile (kv_heads_per_tile D-rows) */
    int32_t row_slots;       /* rows a workgroup loads side by side for one KV head (MFMA_BF16: 32 per
                                wave streaming that KV head) */
    int32_t d_tiles;         /* workgroups along D */
    int32_t nsplit;          /* context splits (1 = no partial sums) */
    int32_t threads;         /* threads per workgroup (256, or 512 on the bf16 matrix engine) */
    int64_t rows_per_split;  /* contiguous splits: context rows per split (the last may be shorter);
                                interleaved: rows of one block (see interleave) */
    int64_t grid;            /* workgroups launched by the first kernel */
    int64_t workspace_bytes; /* device workspace the plan needs (0 if nsplit == 1) */
    int64_t v_bytes_read;    /* V bytes the plan reads from memory (G x more for per-head) */
    int32_t combine;         /* resolved gqa_av_combine: KERNEL when nsplit > 1, else AUTO */
    int32_t kv_heads_per_tile; /* adjacent KV heads one workgroup streams (VALU reuse; else 1) */
    int32_t softmax;         /* 1: a plan of the fused softmax product (gqa_softmax_av.h), which only
                                gqa_softmax_av_decode_plan runs; 0: a plan of this header's product */
    int32_t page_size;       /* > 0: a plan for a paged V cache (gqa_paged_av.h) with this many rows per
                                page, which only gqa_av_paged_decode_plan runs; 0: dense V */
    int32_t attention;       /* 1: a plan of the fused decode attention (gqa_attention.h), which only
                                gqa_attention_decode_plan runs */
    int32_t interleave;      /* 1: split s takes the blocks s, s + nsplit, s + 2 nsplit, ... of
                                rows_per_split rows of the sequence (every split at least one);
                                0: split s takes rows [s rows_per_split, (s + 1) rows_per_split) */
} gqa_av_plan;

/* Resolve `mode` for a head shape. Host-only: needs no GPU.
 * Returns GQA_AV_PER_HEAD or GQA_AV_REUSE (>= 0) on success, or the negated
 * gqa_av_status on error: -GQA_AV_ERR_INVALID_ARG for Hq < 1, Hkv < 1,
 * Hq % Hkv != 0 or an unknown mode; -GQA_AV_ERR_INELIGIBLE for GQA_AV_REUSE
 * with G = Hq / Hkv < 2 (the page checks forced reuse against eligibility). */
int gqa_av_resolve_mode(int64_t Hq, int64_t Hkv, int mode);

/* Build the launch plan for a problem. Host-only: needs no GPU.
 * hint may be NULL. Returns a gqa_av_status; fills *plan on success. */
int gqa_av_make_plan(int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                     int v_dtype, int mode, const gqa_av_hint *hint, gqa_av_plan *plan);

/* out = attn x V as defined above, with an automatic plan for the current
 * device. Sizes: B >= 0, C >= 0, Hq >= 1, Hkv >= 1, D >= 1, Hq % Hkv == 0.
 * C == 0 writes zeros (empty sum); B == 0 does nothing. Pointers may be NULL
 * only when B * Hq * D == 0. attn and out must be 4-byte aligned; V needs only
 * its element alignment (the plan narrows its loads to what V allows). */
int gqa_av_decode(const float *attn, const void *V, float *out,
                  int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                  int v_dtype, int mode, void *stream);

/* Same, with an explicit plan from gqa_av_make_plan for the same sizes, dtype
 * and mode. Returns GQA_AV_ERR_INVALID_ARG if the plan does not match the
 * problem and GQA_AV_ERR_UNSUPPORTED if V is not aligned to plan->vec_bytes. */
int gqa_av_decode_plan(const float *attn, const void *V, float *out,
                       int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                       int v_dtype, const gqa_av_plan *plan, void *stream);

/* The two launches of gqa_av_decode_plan, for callers that schedule or time
 * them separately (same arguments and checks). gqa_av_decode_pass1 streams V
 * and writes `out` directly when plan->nsplit == 1; otherwise it leaves the
 * split partials in the
 * workspace of (current device, stream), and gqa_av_decode_combine, enqueued
 * next on the same stream, adds them into `out` (a no-op for the other
 * cases). Calling both in this order on one stream is exactly
 * gqa_av_decode_plan; `out` is complete only after the combine. */
int gqa_av_decode_pass1(const float *attn, const void *V, float *out,
                        int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                        int v_dtype, const gqa_av_plan *plan, void *stream);
int gqa_av_decode_combine(const float *attn, const void *V, float *out,
                          int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                          int v_dtype, const gqa_av_plan *plan, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, hosts that forbid hipMalloc): gqa_av_decode
 * with the same automatic plan and kernels, its split partials kept in a
 * fixed device array of GQA_AV_NOALLOC_SCRATCH_BYTES (8 MiB) inside the
 * library instead of an allocated workspace. It calls no hipMalloc, hipFree
 * or other allocating routine; the array exists once per device the library
 * runs on and lives until the process ends. A problem whose plan needs more
 * partial-sum space (plan->workspace_bytes) is refused with
 * GQA_AV_ERR_UNSUPPORTED before anything is launched. Every call on one
 * device shares that device's array, which keeps the last call's partials
 * (nothing in it needs clearing: each call writes all it reads): calls that
 * overlap in time on one device (other streams, concurrent graph replays)
 * race and must be ordered by the caller. Same arguments, results and
 * errors as gqa_av_decode otherwise. */
#define GQA_AV_NOALLOC_SCRATCH_BYTES (8 << 20)
int gqa_av_decode_noalloc(const float *attn, const void *V, float *out,
                          int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                          int v_dtype, int mode, void *stream);

/* The same product over a capacity-strided V cache: V is [B][C_max][Hkv][D]
 * (each sequence owns C_max rows, C_max >= C, any value) and rows c < C of
 * every sequence take part; attn [B][C][Hq] and out [B][Hq][D] are dense as
 * above. This is the dense layout of a decode cache allocated for a maximum
 * length (ExecuTorch PR #21063, "...GEMV", introduction: each V row is read
 * once for its group; the page keeps no stride), with all sequences at the
 * same length C (per-sequence lengths: gqa_paged_av.h). The plan is the
 * dense one for (B, C, Hq, Hkv, D); C_max changes only where a sequence's
 * rows start. Errors as gqa_av_decode, plus INVALID_ARG for C_max < C. */
int gqa_av_decode_strided(const float *attn, const void *V, float *out,
                          int64_t B, int64_t C, int64_t C_max, int64_t Hq, int64_t Hkv, int64_t D,
                          int v_dtype, int mode, void *stream);
int gqa_av_decode_strided_plan(const float *attn, const void *V, float *out,
                               int64_t B, int64_t C, int64_t C_max, int64_t Hq, int64_t Hkv, int64_t D,
                               int v_dtype, const gqa_av_plan *plan, void *stream);

/* Static description of a status code. */
const char *gqa_av_status_string(int status);

/* Detail of the calling thread's last failing call ("" if none). */
const char *gqa_av_last_error(void);

/* Free every workspace buffer the library has allocated (live and retired),
 * after synchronising the devices that hold one. Returns a gqa_av_status.
 * Later calls allocate again. A HIP graph captured from a split call refers
 * to its stream's workspace: release invalidates every such graph, so call
 * it only when no captured graph will be replayed again. */
int gqa_av_release(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_AV_H */
