// Host side of the decode score step (include/gqa_qk.h): planning, checks and
// launches. Included at the end of gqa_av.hip, whose error, size and device
// helpers it shares.
#pragma once

#include "dispatch.hpp"
#include "gqa_qk.h"

namespace {

using gqa_av::QkArgs;

constexpr int64_t kQkRowsQuantum = 64;        // 4 waves x 16 rows
constexpr int64_t kQkTargetWgPerCu = 2;
constexpr int64_t kQkMinRowsWide = 256;       // shortest chunk worth a wider KV tile

int qk_plan_impl(int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int k_dtype, int mode,
                 int64_t rows_hint, int cus, int kv_tile, gqa_qk_plan* plan, int64_t page_size = 0) {
    int rc = check_sizes(B, C, Hq, Hkv, D, k_dtype);
    if (rc != GQA_AV_OK) return rc;
    const int resolved = gqa_av_resolve_mode(Hq, Hkv, mode);
    if (resolved < 0) return -resolved;
    if (!plan) return fail(GQA_AV_ERR_INVALID_ARG, "plan is NULL");
    if (D % 32 != 0 || D > 256)
        return fail(GQA_AV_ERR_UNSUPPORTED, "score step: D=%lld must be a multiple of 32 and at most 256", (long long)D);
    if (k_dtype == GQA_AV_FP8_E4M3 && D % 64 != 0)
        return fail(GQA_AV_ERR_UNSUPPORTED, "score step: fp8 K needs D a multiple of 64 (D=%lld)", (long long)D);
    if (page_size < 0 || page_size > INT32_MAX || (page_size > 0 && (page_size & (page_size - 1)) != 0))
        return fail(GQA_AV_ERR_INVALID_ARG, "score step: page_size %lld must be a power of two", (long long)page_size);
    const int es = elem_bytes(k_dtype);
    const int64_t G = Hq / Hkv;
    const int64_t krow = Hkv * D * es;
    if (krow > (int64_t{1} << 20)) return fail(GQA_AV_ERR_UNSUPPORTED, "score step: a row of K exceeds 1 MB");

    int hpt, nsg;
    if (resolved == GQA_AV_PER_HEAD) {
        hpt = 1;
        nsg = 1;
    } else {
        // 32-head tiles for larger groups while the q operand stays small.
        hpt = (G > 16 && D <= 128) ? 32 : 16;
        nsg = static_cast<int>(ceil_div(G, hpt));
    }
    const int64_t minor = resolved == GQA_AV_PER_HEAD ? G : nsg;
    if (cus <= 0) cus = kDefaultCUs;
    const int64_t target = kQkTargetWgPerCu * cus;
    // KV heads per tile: forced, or the widest of 4 and 2 whose grid still
    // reaches the target with chunks of at least kQkMinRowsWide rows (a plain
    // read of 2 KB rows streams faster in wider slices).
    int ht = kv_tile > 0 ? kv_tile : 1;
    if (kv_tile <= 0 && resolved == GQA_AV_REUSE) {
        for (int cand : {4, 2}) {
            if (Hkv % cand != 0) continue;
            const int64_t tw = B * (Hkv / cand) * minor;
            if (tw > 0 && tw * std::min<int64_t>(ceil_div(target, tw), std::max<int64_t>(1, C / kQkMinRowsWide)) >= target) {
                ht = cand;
                break;
            }
        }
    }
    if (ht != 1 && ht != 2 && ht != 4)
        return fail(GQA_AV_ERR_UNSUPPORTED, "score step: kv_tile %d (1, 2 or 4)", ht);
    if (Hkv % ht != 0) return fail(GQA_AV_ERR_INVALID_ARG, "score step: kv_tile %d does not divide Hkv", ht);
    if (ht > 1 && resolved != GQA_AV_REUSE)
        return fail(GQA_AV_ERR_UNSUPPORTED, "score step: kv_tile > 1 needs reuse mode");
    const int64_t tiles = B * (Hkv / ht) * minor;

    // Context rows per workgroup: enough workgroups for about two per CU, in
    // whole 64-row steps; 32-bit K offsets for the chunk and its overrun.
    int64_t rows = rows_hint;
    if (rows <= 0) {
        const int64_t nchunk = tiles > 0 ? std::max<int64_t>(1, ceil_div(target, tiles)) : 1;
        rows = std::max<int64_t>(1, ceil_div(C, nchunk));
    }
    rows = ceil_div(rows, kQkRowsQuantum) * kQkRowsQuantum;
    // K and score offsets inside a chunk stay below 2^30 bytes, with room for
    // the reads and the scalar row offsets past its end.
    const int64_t max_rows =
        ((int64_t{1} << 30) / std::max(krow, 4 * Hq) - 2 * kQkRowsQuantum) / kQkRowsQuantum * kQkRowsQuantum;
    if (max_rows < kQkRowsQuantum) return fail(GQA_AV_ERR_UNSUPPORTED, "score step: rows of K too large");
    if (rows > max_rows) rows = max_rows;
    if (rows > INT32_MAX) rows = max_rows;
    if (page_size > 0) {
        // Paged K: a block's page list (at most ceil(rows / P) + 1 entries) sits in LDS.
        const int64_t cap = (gqa_av::kMaxSplitPages - 1) * page_size / kQkRowsQuantum * kQkRowsQuantum;
        if (rows > cap) rows = cap;
        if (rows < kQkRowsQuantum)
            return fail(GQA_AV_ERR_UNSUPPORTED, "score step: pages of %lld rows are too small", (long long)page_size);
    }
    const int64_t nchunk = C > 0 ? ceil_div(C, rows) : 0;
    const int64_t grid = tiles * nchunk;
    if (grid > INT32_MAX || nchunk > INT32_MAX) return fail(GQA_AV_ERR_UNSUPPORTED, "score step: grid too large");

    std::memset(plan, 0, sizeof *plan);
    plan->mode = resolved;
    // The 16-bit matrix path for bf16, fp16 and fp8 K, the fp32 one for fp32 K.
    plan->engine = k_dtype == GQA_AV_F32 ? GQA_AV_ENGINE_MFMA : GQA_AV_ENGINE_MFMA_BF16;
    plan->heads_per_tile = hpt;
    plan->subgroups = nsg;
    plan->rows_per_block = rows;
    plan->grid = grid;
    plan->k_bytes_read = B * C * Hkv * D * es * (resolved == GQA_AV_PER_HEAD ? G : nsg);
    plan->kv_heads_per_tile = ht;
    plan->page_size = static_cast<int32_t>(page_size);
    return GQA_AV_OK;
}

// The paged-cache arguments of the paged score step.
struct QkPaged {
    const int32_t* block_table;
    const int32_t* seq_lens;
    int64_t page_size, max_pages, num_pages;
};

int qk_run(const float* q, const void* K, float* scores, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
           int64_t D, int k_dtype, float scale, const gqa_qk_plan* plan, void* stream,
           const float* k_scale = nullptr, const QkPaged* pg = nullptr) {
    if (!plan) return fail(GQA_AV_ERR_INVALID_ARG, "plan is NULL");
    if ((plan->page_size > 0) != (pg != nullptr))
        return fail(GQA_AV_ERR_INVALID_ARG, pg ? "not a paged score plan (plan->page_size == 0)"
                                                : "a paged score plan: run it with gqa_qk_paged_decode_plan");
    gqa_qk_plan check;
    int rc = qk_plan_impl(B, C, Hq, Hkv, D, k_dtype, plan->mode, plan->rows_per_block, kDefaultCUs,
                          plan->kv_heads_per_tile, &check, plan->page_size);
    if (rc != GQA_AV_OK) return rc;
    if (check.mode != plan->mode || check.engine != plan->engine || check.heads_per_tile != plan->heads_per_tile ||
        check.subgroups != plan->subgroups || check.rows_per_block != plan->rows_per_block ||
        check.grid != plan->grid || check.k_bytes_read != plan->k_bytes_read ||
        check.kv_heads_per_tile != plan->kv_heads_per_tile || check.page_size != plan->page_size)
        return fail(GQA_AV_ERR_INVALID_ARG, "score plan does not belong to this problem");
    if (k_scale && k_dtype != GQA_AV_FP8_E4M3) return fail(GQA_AV_ERR_INVALID_ARG, "k_scale is for fp8 K");
    if (pg) {
        if (pg->page_size != plan->page_size)
            return fail(GQA_AV_ERR_INVALID_ARG, "page_size %lld does not match the plan's %d",
                        (long long)pg->page_size, plan->page_size);
        if (pg->max_pages < 1 || pg->max_pages > INT32_MAX || pg->num_pages < 1)
            return fail(GQA_AV_ERR_INVALID_ARG, "max_pages and num_pages must be >= 1");
        if (C > pg->max_pages * pg->page_size)
            return fail(GQA_AV_ERR_INVALID_ARG, "capacity C=%lld exceeds max_pages * page_size", (long long)C);
        if (B > 0 && C > 0 && (!pg->block_table || !pg->seq_lens))
            return fail(GQA_AV_ERR_INVALID_ARG, "block_table and seq_lens must not be NULL");
    }
    if (B == 0 || C == 0) return GQA_AV_OK;
    if (!q || !K || !scores) return fail(GQA_AV_ERR_INVALID_ARG, "q, K and scores must not be NULL");
    if ((reinterpret_cast<uintptr_t>(q) & 3u) || (reinterpret_cast<uintptr_t>(scores) & 3u))
        return fail(GQA_AV_ERR_INVALID_ARG, "q and scores must be 4-byte aligned");
    if (reinterpret_cast<uintptr_t>(K) & 15u) return fail(GQA_AV_ERR_UNSUPPORTED, "K must be 16-byte aligned");
    if (k_scale && (reinterpret_cast<uintptr_t>(k_scale) & 3u))
        return fail(GQA_AV_ERR_INVALID_ARG, "k_scale must be 4-byte aligned");

    QkArgs a;
    a.q = q;
    a.K = static_cast<const uint8_t*>(K);
    a.scores = scores;
    a.scale = scale;
    a.k_scale = k_scale;
    a.block_table = pg ? pg->block_table : nullptr;
    a.seq_lens = pg ? pg->seq_lens : nullptr;
    a.num_pages = pg ? pg->num_pages : 0;
    a.max_pages = pg ? static_cast<int32_t>(pg->max_pages) : 0;
    a.page_shift = 0;
    if (pg)
        while ((int64_t{1} << a.page_shift) < pg->page_size) ++a.page_shift;
    a.C = C;
    a.rows_per_block = static_cast<int32_t>(plan->rows_per_block);
    a.nchunk = static_cast<int32_t>(ceil_div(C, plan->rows_per_block));
    a.B = static_cast<int32_t>(B);
    a.Hq = static_cast<int32_t>(Hq);
    a.Hkv = static_cast<int32_t>(Hkv);
    a.G = static_cast<int32_t>(Hq / Hkv);
    a.per_head = plan->mode == GQA_AV_PER_HEAD;
    a.nsg = plan->subgroups;
    a.ht = plan->kv_heads_per_tile;
    a.nblocks = static_cast<uint32_t>(plan->grid);
    // 16-byte score stores: each tile's heads are one run (one head subgroup)
    // starting at a multiple of 4 heads (kv_heads_per_tile * G a multiple of
    // 4), rows are whole 16-byte groups, and scores is 16-byte aligned.
    a.vec4 = plan->mode == GQA_AV_REUSE && plan->subgroups == 1 && (plan->kv_heads_per_tile * a.G) % 4 == 0 &&
             Hq % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15u) == 0;
    const int nset = plan->mode == GQA_AV_PER_HEAD ? 1 : plan->heads_per_tile / 16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (k_dtype) {
    case GQA_AV_F32: e = gqa_av_launch::qk<gqa_av::kF32>(D, nset, a, s); break;
    case GQA_AV_F16: e = gqa_av_launch::qk<gqa_av::kF16>(D, nset, a, s); break;
    case GQA_AV_FP8_E4M3: e = gqa_av_launch::qk<gqa_av::kFP8>(D, nset, a, s); break;
    default: e = gqa_av_launch::qk<gqa_av::kBF16>(D, nset, a, s); break;
    }
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "score launch: %s", hipGetErrorString(e));
    return GQA_AV_OK;
}

}  // namespace

extern "C" {

int gqa_qk_make_plan(int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int k_dtype, int mode,
                     const gqa_qk_hint* hint, gqa_qk_plan* plan) {
    gqa_qk_hint h;
    std::memset(&h, 0, sizeof h);
    if (hint) h = *hint;
    return qk_plan_impl(B, C, Hq, Hkv, D, k_dtype, mode, h.rows_per_block, h.cu_count > 0 ? h.cu_count : kDefaultCUs,
                        h.kv_tile, plan, h.page_size);
}

int gqa_qk_decode_plan(const float* q, const void* K, float* scores, int64_t B, int64_t C, int64_t Hq,
                       int64_t Hkv, int64_t D, int k_dtype, float scale, const gqa_qk_plan* plan, void* stream) {
    return qk_run(q, K, scores, B, C, Hq, Hkv, D, k_dtype, scale, plan, stream);
}

}  // extern "C"

namespace {

int qk_auto(const float* q, const void* K, const float* k_scale, float* scores, int64_t B, int64_t C, int64_t Hq,
            int64_t Hkv, int64_t D, int k_dtype, float scale, int mode, void* stream, const QkPaged* pg = nullptr) {
    int rc = check_sizes(B, C, Hq, Hkv, D, k_dtype);
    if (rc != GQA_AV_OK) return rc;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    int cus = kDefaultCUs;
    rc = device_cus(dev, &cus);
    if (rc != GQA_AV_OK) return rc;
    gqa_qk_plan plan;
    rc = qk_plan_impl(B, C, Hq, Hkv, D, k_dtype, mode, 0, cus, 0, &plan, pg ? pg->page_size : 0);
    if (rc != GQA_AV_OK) return rc;
    return qk_run(q, K, scores, B, C, Hq, Hkv, D, k_dtype, scale, &plan, stream, k_scale, pg);
}

}  // namespace

extern "C" {

int gqa_qk_decode(const float* q, const void* K, float* scores, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                  int64_t D, int k_dtype, float scale, int mode, void* stream) {
    return qk_auto(q, K, nullptr, scores, B, C, Hq, Hkv, D, k_dtype, scale, mode, stream);
}

int gqa_qk_fp8_decode(const float* q, const void* K, const float* k_scale, float* scores, int64_t B, int64_t C,
                      int64_t Hq, int64_t Hkv, int64_t D, float scale, int mode, void* stream) {
    return qk_auto(q, K, k_scale, scores, B, C, Hq, Hkv, D, GQA_AV_FP8_E4M3, scale, mode, stream);
}

int gqa_qk_fp8_decode_plan(const float* q, const void* K, const float* k_scale, float* scores, int64_t B,
                           int64_t C, int64_t Hq, int64_t Hkv, int64_t D, float scale, const gqa_qk_plan* plan,
                           void* stream) {
    return qk_run(q, K, scores, B, C, Hq, Hkv, D, GQA_AV_FP8_E4M3, scale, plan, stream, k_scale);
}

int gqa_qk_paged_decode(const float* q, const void* pages, const int32_t* block_table, const int32_t* seq_lens,
                        const float* k_scale, float* scores, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D,
                        int64_t page_size, int64_t max_pages, int64_t num_pages, int k_dtype, float scale, int mode,
                        void* stream) {
    if (page_size < 1) return fail(GQA_AV_ERR_INVALID_ARG, "page_size must be >= 1");
    QkPaged pg{block_table, seq_lens, page_size, max_pages, num_pages};
    return qk_auto(q, pages, k_scale, scores, B, C, Hq, Hkv, D, k_dtype, scale, mode, stream, &pg);
}

int gqa_qk_paged_decode_plan(const float* q, const void* pages, const int32_t* block_table, const int32_t* seq_lens,
                             const float* k_scale, float* scores, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                             int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages, int k_dtype,
                             float scale, const gqa_qk_plan* plan, void* stream) {
    QkPaged pg{block_table, seq_lens, page_size, max_pages, num_pages};
    return qk_run(q, pages, scores, B, C, Hq, Hkv, D, k_dtype, scale, plan, stream, k_scale, &pg);
}

}  // extern "C"
