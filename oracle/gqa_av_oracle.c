/*
 * CPU oracle for the GQA decode attention-times-V contraction.
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library. The product
 * path (gqa_reuse_attn_amd/) never links, imports or executes it, and it
 * shares no code, header or table with the HIP kernels.
 *
 * What it computes -- ExecuTorch PR #21063, "...GEMV" (GQA-reuse AV coop GEMV
 * for the Vulkan backend), introduction: query heads come in groups of
 * G = Hq / Hkv that share one KV head, and each output element is the sum
 * over context positions c of attn[c, q_h] * V[c, kv_h, d]. A batch index b
 * of independent sequences is added in front of every tensor:
 *
 *   out[b, q_h, d] = sum_{c=0}^{C-1} attn[b, c, q_h] * V[b, c, kv_h(q_h), d]
 *   kv_h(q_h)      = floor(q_h / G)      (contiguous groups of G heads)
 *
 * The page never states which KV head a query head reads. Contiguous groups
 * are taken: the page has G query heads sharing one KV head and one workgroup
 * per KV head producing that group's G outputs, and consecutive query heads
 * are the plain grouping for that.
 *
 * How: every input element is widened exactly to double with decoders written
 * here from the IEEE-754 binary16 and bfloat16 bit layouts; each product of a
 * float32 weight and a V value is exact in double (at most 24 x 24 significand
 * bits); the products are added in double in increasing c. The only rounding
 * is that summation, bounded by gamma_{C-1} * sum_c |attn * V|.
 *
 * Layouts are dense row-major: attn [B][C][Hq] float32, V [B][C][Hkv][D] of
 * the given dtype, out [B][Hq][D] double.
 *
 * The score step that precedes it in decode attention is not on the page; it
 * is the standard first half of decode attention with the same head grouping
 * (each K row shared by the G query heads of its group), and its output has
 * the layout of attn above:
 *
 *   scores[b, c, q_h] = scale * sum_{d=0}^{D-1} q[b, q_h, d] * K[b, c, kv_h(q_h), d]
 *
 * with q [B][Hq][D] float32, K [B][C][Hkv][D] of the given dtype and scores
 * [B][C][Hq] double. Each product is exact in double, the sum runs in double
 * in increasing d, and the scale multiplies the sum.
 *
 * The fused variant takes the scores instead of the weights: the page's attn
 * is a softmax over the context of the scores, and the fused product applies
 * that softmax itself,
 *
 *   out[b, q_h, d] = sum_c p[b, c, q_h] * V[b, c, kv_h(q_h), d]
 *   p[b, c, q_h]   = exp(s[b, c, q_h] - m) / sum_{c'} exp(s[b, c', q_h] - m)
 *   m              = max_c s[b, c, q_h]
 *
 * with s [B][C][Hq] float32. Written out in double: the maximum, then
 * e_c = exp(s_c - m) (libm), the sums of e_c * V and of e_c in increasing c,
 * and one division at the end. C = 0 gives zeros (an empty sum, as above); a
 * row whose scores are all -inf gives NaN, as the definition does.
 *
 * Fused decode attention (the score step, the softmax and the product in one
 * pass; the page covers the product only):
 *
 *   out[b, q_h, d] = sum_c p_c V[b, c, kv_h, d],  p = softmax_c(s),
 *   s_c = scale * sum_d q[b, q_h, d] * K[b, c, kv_h, d]
 *
 * written out in double: each score from exact products summed in increasing
 * d and multiplied by scale, then the maximum, exp(s_c - m) (libm), the sums
 * of exp * V and of exp in increasing c, and one division.
 *
 * fp8 V (a compressed cache, not on the page): V holds OCP FP8 E4M3 bytes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities,
 * S.1111.111 is NaN) and each KV head has a float32 scale: the value of an
 * element is decode(byte) * v_scale[kv_h], exact in double. The products and
 * sums are those of the plain or fused definitions above. fp8 K in the score
 * step is read the same way, with its own per-KV-head k_scale:
 * scores = scale * sum_d q * (decode(K byte) * k_scale[kv_h]).
 *
 * Paged V (a decode cache layout, not on the page): sequence b has seq_lens[b]
 * context rows; row c of it lives in page block_table[b][c / page_size], at
 * row c % page_size of that page, pages being [page_size][Hkv][D] blocks of
 * one array. The weights (or scores) keep the dense [B][C][Hq] layout with C
 * the capacity, and only rows c < seq_lens[b] take part: the sums above run
 * over those rows (a sequence of length 0 gives zeros). Paged K in the score
 * step uses the same layout and tables: the scores of rows c < seq_lens[b]
 * follow the score definition with K's row c read from its page; rows at or
 * past the length have no score (NaN here: the kernel leaves them unwritten).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_OK = 0, ORC_BAD_ARG = 1 };

/* bfloat16 is the upper half of an IEEE binary32: shift into place. */
static double orc_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double orc_f16(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^(1-15-10) */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);   /* (1 + m/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

static double orc_f32(const float *p)
{
    return (double)*p;
}

static double orc_load(const void *V, int dtype, int64_t i)
{
    switch (dtype) {
    case ORC_F32: return orc_f32((const float *)V + i);
    case ORC_F16: return orc_f16(((const uint16_t *)V)[i]);
    default:      return orc_bf16(((const uint16_t *)V)[i]);
    }
}

static int orc_check(int dtype, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D)
{
    if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16) return ORC_BAD_ARG;
    if (B < 0 || C < 0 || Hq < 1 || Hkv < 1 || D < 1) return ORC_BAD_ARG;
    if (Hq % Hkv != 0) return ORC_BAD_ARG;
    return ORC_OK;
}

/* Widen n elements of V to double (exposed so tests can pin the decoders). */
int gqa_av_oracle_decode(const void *V, int dtype, int64_t n, double *out)
{
    if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16) return ORC_BAD_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = orc_load(V, dtype, i);
    return ORC_OK;
}

/* All 65536 binary16 values, filled once from orc_f16 (a speed-up only). */
static double orc_f16_table[65536];
static pthread_once_t orc_f16_once = PTHREAD_ONCE_INIT;
static void orc_f16_fill(void)
{
    for (uint32_t h = 0; h < 65536u; ++h) orc_f16_table[h] = orc_f16((uint16_t)h);
}

/* One output row out[b, q, 0:D]: the definition, summed in increasing c. */
static void orc_row(const float *attn, const void *V, int dtype,
                    int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                    int64_t b, int64_t q, double *acc)
{
    const int64_t G = Hq / Hkv;
    const int64_t kv = q / G;
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t c = 0; c < C; ++c) {
        const double a = (double)attn[(b * C + c) * Hq + q];
        const int64_t row = ((b * C + c) * Hkv + kv) * D;
        if (dtype == ORC_F32) {
            const float *r = (const float *)V + row;
            for (int64_t d = 0; d < D; ++d) acc[d] += a * orc_f32(r + d);
        } else if (dtype == ORC_F16) {
            const uint16_t *r = (const uint16_t *)V + row;
            for (int64_t d = 0; d < D; ++d) acc[d] += a * orc_f16_table[r[d]];
        } else {
            const uint16_t *r = (const uint16_t *)V + row;
            for (int64_t d = 0; d < D; ++d) acc[d] += a * orc_bf16(r[d]);
        }
    }
}

/* Full output: out[B][Hq][D] in double. nthreads <= 0 uses the OpenMP default. */
int gqa_av_oracle(const float *attn, const void *V, int dtype,
                  int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                  double *out, int nthreads)
{
    int rc = orc_check(dtype, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    pthread_once(&orc_f16_once, orc_f16_fill);
    const int64_t rows = B * Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i)
        orc_row(attn, V, dtype, C, Hq, Hkv, D, i / Hq, i % Hq, out + i * D);
    (void)nthreads;
    return ORC_OK;
}

/* Selected outputs: idx holds npts triples (b, q_h, d); out[k] is that element. */
int gqa_av_oracle_points(const float *attn, const void *V, int dtype,
                         int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                         const int64_t *idx, int64_t npts, double *out, int nthreads)
{
    int rc = orc_check(dtype, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    for (int64_t k = 0; k < npts; ++k) {
        const int64_t b = idx[3 * k], q = idx[3 * k + 1], d = idx[3 * k + 2];
        if (b < 0 || b >= B || q < 0 || q >= Hq || d < 0 || d >= D) return ORC_BAD_ARG;
    }
    const int64_t G = Hq / Hkv;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
#endif
    for (int64_t k = 0; k < npts; ++k) {
        const int64_t b = idx[3 * k], q = idx[3 * k + 1], d = idx[3 * k + 2];
        const int64_t kv = q / G;
        double acc = 0.0;
        for (int64_t c = 0; c < C; ++c)
            acc += (double)attn[(b * C + c) * Hq + q] *
                   orc_load(V, dtype, ((b * C + c) * Hkv + kv) * D + d);
        out[k] = acc;
    }
    (void)nthreads;
    return ORC_OK;
}

/* Scores of one context row: scores[b, c, 0:Hq], the definition above. */
static void orc_qk_row(const float *q, const void *K, int dtype,
                       int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                       int64_t b, int64_t c, double scale, double *out)
{
    const int64_t G = Hq / Hkv;
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t kvh = h / G;
        const float *qrow = q + (b * Hq + h) * D;
        const int64_t krow = ((b * C + c) * Hkv + kvh) * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * orc_load(K, dtype, krow + d);
        out[h] = dot * scale;
    }
}

/* Full scores: out[B][C][Hq] in double. nthreads <= 0 uses the OpenMP default. */
int gqa_qk_oracle(const float *q, const void *K, int dtype,
                  int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                  double scale, double *out, int nthreads)
{
    int rc = orc_check(dtype, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    const int64_t rows = B * C;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i)
        orc_qk_row(q, K, dtype, C, Hq, Hkv, D, i / C, i % C, scale, out + i * Hq);
    (void)nthreads;
    return ORC_OK;
}

/* One output row of the fused softmax and AV product (see the header). */
static void orc_sav_row(const float *scores, const void *V, int dtype,
                        int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                        int64_t b, int64_t q, double *acc)
{
    const int64_t G = Hq / Hkv;
    const int64_t kv = q / G;
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    if (C == 0) return;
    double m = -INFINITY;
    for (int64_t c = 0; c < C; ++c) {
        const double s = (double)scores[(b * C + c) * Hq + q];
        if (s > m) m = s;
    }
    double l = 0.0;
    for (int64_t c = 0; c < C; ++c) {
        const double e = exp((double)scores[(b * C + c) * Hq + q] - m);
        l += e;
        const int64_t row = ((b * C + c) * Hkv + kv) * D;
        for (int64_t d = 0; d < D; ++d) acc[d] += e * orc_load(V, dtype, row + d);
    }
    for (int64_t d = 0; d < D; ++d) acc[d] /= l;
}

/* Full fused output: out[B][Hq][D] in double. nthreads <= 0 uses the OpenMP default. */
int gqa_softmax_av_oracle(const float *scores, const void *V, int dtype,
                          int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                          double *out, int nthreads)
{
    int rc = orc_check(dtype, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    pthread_once(&orc_f16_once, orc_f16_fill);
    const int64_t rows = B * Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i)
        orc_sav_row(scores, V, dtype, C, Hq, Hkv, D, i / Hq, i % Hq, out + i * D);
    (void)nthreads;
    return ORC_OK;
}

/* Paged V, one output row: the plain product (softmax = 0) or the fused
 * softmax product (softmax = 1) over the rows c < len of sequence b. */
static void orc_paged_row(const float *w, const void *pages, const int32_t *bt, int dtype, int softmax,
                          int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int64_t P, int64_t max_pages,
                          int64_t len, int64_t b, int64_t q, double *acc)
{
    const int64_t G = Hq / Hkv;
    const int64_t kv = q / G;
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    if (len == 0) return;
    double m = 0.0, l = 0.0;
    if (softmax) {
        m = -INFINITY;
        for (int64_t c = 0; c < len; ++c) {
            const double s = (double)w[(b * C + c) * Hq + q];
            if (s > m) m = s;
        }
    }
    for (int64_t c = 0; c < len; ++c) {
        const double x = (double)w[(b * C + c) * Hq + q];
        const double a = softmax ? exp(x - m) : x;
        l += a;
        const int64_t page = bt[b * max_pages + c / P];
        const int64_t row = ((page * P + c % P) * Hkv + kv) * D;
        for (int64_t d = 0; d < D; ++d) acc[d] += a * orc_load(pages, dtype, row + d);
    }
    if (softmax)
        for (int64_t d = 0; d < D; ++d) acc[d] /= l;
}

/* Full paged output: out[B][Hq][D] in double. Rejects lengths outside [0, C],
 * block-table entries outside [0, num_pages) for used rows, and a capacity C
 * above max_pages * P. */
int gqa_av_paged_oracle(const float *w, const void *pages, const int32_t *block_table, const int32_t *seq_lens,
                        int dtype, int softmax, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                        int64_t P, int64_t max_pages, int64_t num_pages, double *out, int nthreads)
{
    int rc = orc_check(dtype, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    if (P < 1 || max_pages < 0 || num_pages < 0 || C > max_pages * P) return ORC_BAD_ARG;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t len = seq_lens[b];
        if (len < 0 || len > C) return ORC_BAD_ARG;
        for (int64_t c = 0; c < len; c += P) {
            const int64_t page = block_table[b * max_pages + c / P];
            if (page < 0 || page >= num_pages) return ORC_BAD_ARG;
        }
    }
    pthread_once(&orc_f16_once, orc_f16_fill);
    const int64_t rows = B * Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i)
        orc_paged_row(w, pages, block_table, dtype, softmax, C, Hq, Hkv, D, P, max_pages, seq_lens[i / Hq],
                      i / Hq, i % Hq, out + i * D);
    (void)nthreads;
    return ORC_OK;
}

/* OCP FP8 E4M3: written out from the bit layout. */
static double orc_e4m3(uint8_t x)
{
    const int sign = x >> 7, e = (x >> 3) & 15, m = x & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);                  /* subnormal: m / 8 * 2^-6 */
    else v = ldexp((double)(8 + m), e - 10);               /* (1 + m / 8) * 2^(e - 7) */
    return sign ? -v : v;
}

/* Widen n fp8 E4M3 bytes to double (exposed so tests can pin the decoder). */
int gqa_fp8_oracle_decode(const uint8_t *V, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3(V[i]);
    return ORC_OK;
}

/* fp8 V with per-KV-head scales, one output row: the plain product
 * (softmax = 0) or the fused softmax product (softmax = 1). */
static void orc_fp8_row(const float *w, const uint8_t *V, const float *v_scale, int softmax,
                        int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int64_t b, int64_t q, double *acc)
{
    const int64_t G = Hq / Hkv;
    const int64_t kv = q / G;
    const double sc = v_scale ? (double)v_scale[kv] : 1.0;
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    if (C == 0) return;
    double m = 0.0, l = 0.0;
    if (softmax) {
        m = -INFINITY;
        for (int64_t c = 0; c < C; ++c) {
            const double x = (double)w[(b * C + c) * Hq + q];
            if (x > m) m = x;
        }
    }
    for (int64_t c = 0; c < C; ++c) {
        const double x = (double)w[(b * C + c) * Hq + q];
        const double a = softmax ? exp(x - m) : x;
        l += a;
        const uint8_t *r = V + ((b * C + c) * Hkv + kv) * D;
        for (int64_t d = 0; d < D; ++d) acc[d] += a * (orc_e4m3(r[d]) * sc);
    }
    if (softmax)
        for (int64_t d = 0; d < D; ++d) acc[d] /= l;
}

/* Full fp8 output: out[B][Hq][D] in double; v_scale [Hkv] or NULL (all 1). */
int gqa_fp8_oracle(const float *w, const uint8_t *V, const float *v_scale, int softmax,
                   int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, double *out, int nthreads)
{
    int rc = orc_check(ORC_F32, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    const int64_t rows = B * Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i)
        orc_fp8_row(w, V, v_scale, softmax, C, Hq, Hkv, D, i / Hq, i % Hq, out + i * D);
    (void)nthreads;
    return ORC_OK;
}

/* Score step over fp8 K with per-KV-head scales (k_scale [Hkv] or NULL: all
 * 1): out[B][C][Hq] in double, the score definition above with each K element
 * decode(byte) * k_scale[kv_h]; the dot product runs in increasing d. */
static void orc_qk_fp8_row(const float *q, const uint8_t *K, const float *k_scale,
                           int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                           int64_t b, int64_t c, double scale, double *out)
{
    const int64_t G = Hq / Hkv;
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t kvh = h / G;
        const double ks = k_scale ? (double)k_scale[kvh] : 1.0;
        const float *qrow = q + (b * Hq + h) * D;
        const uint8_t *krow = K + ((b * C + c) * Hkv + kvh) * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (orc_e4m3(krow[d]) * ks);
        out[h] = dot * scale;
    }
}

int gqa_qk_fp8_oracle(const float *q, const uint8_t *K, const float *k_scale,
                      int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                      double scale, double *out, int nthreads)
{
    int rc = orc_check(ORC_F32, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    const int64_t rows = B * C;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i)
        orc_qk_fp8_row(q, K, k_scale, C, Hq, Hkv, D, i / C, i % C, scale, out + i * Hq);
    (void)nthreads;
    return ORC_OK;
}

/* Score step over paged K: out[B][C][Hq] in double, rows c < seq_lens[b] as
 * the score definition with K row c from its page, other rows NaN. dtype as
 * for K (0..2), or 3 for fp8 E4M3 bytes with k_scale [Hkv] (NULL: all 1).
 * Rejects what gqa_av_paged_oracle rejects. */
int gqa_qk_paged_oracle(const float *q, const void *pages, const int32_t *block_table, const int32_t *seq_lens,
                        int dtype, const float *k_scale, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                        int64_t D, int64_t P, int64_t max_pages, int64_t num_pages, double scale, double *out,
                        int nthreads)
{
    int rc = orc_check(dtype == 3 ? ORC_F32 : dtype, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    if (P < 1 || max_pages < 0 || num_pages < 0 || C > max_pages * P) return ORC_BAD_ARG;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t len = seq_lens[b];
        if (len < 0 || len > C) return ORC_BAD_ARG;
        for (int64_t c = 0; c < len; c += P) {
            const int64_t page = block_table[b * max_pages + c / P];
            if (page < 0 || page >= num_pages) return ORC_BAD_ARG;
        }
    }
    pthread_once(&orc_f16_once, orc_f16_fill);
    const int64_t G = Hq / Hkv;
    const int64_t rows = B * C;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i) {
        const int64_t b = i / C, c = i % C;
        double *o = out + i * Hq;
        if (c >= seq_lens[b]) {
            for (int64_t h = 0; h < Hq; ++h) o[h] = NAN;
            continue;
        }
        const int64_t page = block_table[b * max_pages + c / P];
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t kvh = h / G;
            const int64_t row = ((page * P + c % P) * Hkv + kvh) * D;
            const float *qrow = q + (b * Hq + h) * D;
            double dot = 0.0;
            if (dtype == 3) {
                const double ks = k_scale ? (double)k_scale[kvh] : 1.0;
                const uint8_t *kr = (const uint8_t *)pages + row;
                for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (orc_e4m3(kr[d]) * ks);
            } else {
                for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * orc_load(pages, dtype, row + d);
            }
            o[h] = dot * scale;
        }
    }
    (void)nthreads;
    return ORC_OK;
}

/* Fused decode attention: out[B][Hq][D] in double (definition above). K and
 * V share dtype (0..2). C = 0 gives zeros. */
int gqa_attention_oracle(const float *q, const void *K, const void *V, int dtype,
                         int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, double scale, double *out,
                         int nthreads)
{
    int rc = orc_check(dtype, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    pthread_once(&orc_f16_once, orc_f16_fill);
    const int64_t G = Hq / Hkv;
    const int64_t rows = B * Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i) {
        const int64_t b = i / Hq, h = i % Hq, kv = h / G;
        double *o = out + i * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (C == 0) continue;
        const float *qrow = q + (b * Hq + h) * D;
        double m = -INFINITY;
        for (int64_t c = 0; c < C; ++c) {
            const int64_t krow = ((b * C + c) * Hkv + kv) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * orc_load(K, dtype, krow + d);
            const double sc = dot * scale;
            if (sc > m) m = sc;
        }
        double l = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            const int64_t krow = ((b * C + c) * Hkv + kv) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * orc_load(K, dtype, krow + d);
            const double e = exp(dot * scale - m);
            l += e;
            for (int64_t d = 0; d < D; ++d) o[d] += e * orc_load(V, dtype, krow + d);
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= l;
    }
    (void)nthreads;
    return ORC_OK;
}

/* Fused decode attention over fp8 K and V (OCP E4M3 bytes) with per-KV-head
 * scales (NULL: all 1): the definition above with K and V elements
 * decode(byte) * k_scale[kv_h] and decode(byte) * v_scale[kv_h]. */
int gqa_attention_fp8_oracle(const float *q, const uint8_t *K, const float *k_scale, const uint8_t *V,
                             const float *v_scale, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                             double scale, double *out, int nthreads)
{
    int rc = orc_check(ORC_F32, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    const int64_t G = Hq / Hkv;
    const int64_t rows = B * Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i) {
        const int64_t b = i / Hq, h = i % Hq, kv = h / G;
        const double ks = k_scale ? (double)k_scale[kv] : 1.0;
        const double vs = v_scale ? (double)v_scale[kv] : 1.0;
        double *o = out + i * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (C == 0) continue;
        const float *qrow = q + (b * Hq + h) * D;
        double m = -INFINITY;
        for (int64_t c = 0; c < C; ++c) {
            const uint8_t *kr = K + ((b * C + c) * Hkv + kv) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (orc_e4m3(kr[d]) * ks);
            const double sc = dot * scale;
            if (sc > m) m = sc;
        }
        double l = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            const uint8_t *kr = K + ((b * C + c) * Hkv + kv) * D;
            const uint8_t *vr = V + ((b * C + c) * Hkv + kv) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (orc_e4m3(kr[d]) * ks);
            const double e = exp(dot * scale - m);
            l += e;
            for (int64_t d = 0; d < D; ++d) o[d] += e * (orc_e4m3(vr[d]) * vs);
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= l;
    }
    (void)nthreads;
    return ORC_OK;
}

/* One element of a paged K or V cache: dtype 0..2 as for V, or 3 for fp8
 * E4M3 bytes times the KV head's scale (NULL: 1). */
static double orc_kv_elem(const void *pages, int dtype, const float *sc, int64_t kv, int64_t i)
{
    if (dtype == 3) return orc_e4m3(((const uint8_t *)pages)[i]) * (sc ? (double)sc[kv] : 1.0);
    return orc_load(pages, dtype, i);
}

/* Fused decode attention over a paged K and V cache: out[B][Hq][D] in double.
 * K and V live in two page pools of one layout [num_pages][P][Hkv][D] that
 * share the block table: row c of sequence b is row c mod P of page
 * block_table[b][c / P] in both. Only rows c < seq_lens[b] take part; a
 * length of 0 gives zeros. dtype 0..2, or 3 for fp8 E4M3 with k_scale and
 * v_scale [Hkv] (NULL: all 1). Rejects what gqa_av_paged_oracle rejects. */
int gqa_attention_paged_oracle(const float *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                               const int32_t *seq_lens, int dtype, const float *k_scale, const float *v_scale,
                               int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int64_t P,
                               int64_t max_pages, int64_t num_pages, double scale, double *out, int nthreads)
{
    int rc = orc_check(dtype == 3 ? ORC_F32 : dtype, B, C, Hq, Hkv, D);
    if (rc != ORC_OK) return rc;
    if (P < 1 || max_pages < 0 || num_pages < 0 || C > max_pages * P) return ORC_BAD_ARG;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t len = seq_lens[b];
        if (len < 0 || len > C) return ORC_BAD_ARG;
        for (int64_t c = 0; c < len; c += P) {
            const int64_t page = block_table[b * max_pages + c / P];
            if (page < 0 || page >= num_pages) return ORC_BAD_ARG;
        }
    }
    pthread_once(&orc_f16_once, orc_f16_fill);
    const int64_t G = Hq / Hkv;
    const int64_t rows = B * Hq;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < rows; ++i) {
        const int64_t b = i / Hq, h = i % Hq, kv = h / G;
        const int64_t len = seq_lens[b];
        double *o = out + i * D;
        for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
        if (len == 0) continue;
        const float *qrow = q + (b * Hq + h) * D;
        double m = -INFINITY;
        for (int64_t c = 0; c < len; ++c) {
            const int64_t page = block_table[b * max_pages + c / P];
            const int64_t row = ((page * P + c % P) * Hkv + kv) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * orc_kv_elem(k_pages, dtype, k_scale, kv, row + d);
            const double sc = dot * scale;
            if (sc > m) m = sc;
        }
        double l = 0.0;
        for (int64_t c = 0; c < len; ++c) {
            const int64_t page = block_table[b * max_pages + c / P];
            const int64_t row = ((page * P + c % P) * Hkv + kv) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * orc_kv_elem(k_pages, dtype, k_scale, kv, row + d);
            const double e = exp(dot * scale - m);
            l += e;
            for (int64_t d = 0; d < D; ++d) o[d] += e * orc_kv_elem(v_pages, dtype, v_scale, kv, row + d);
        }
        for (int64_t d = 0; d < D; ++d) o[d] /= l;
    }
    (void)nthreads;
    return ORC_OK;
}
