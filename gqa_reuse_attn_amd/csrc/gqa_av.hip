// Host side of libgqa_av.so: argument checks, mode resolution, planning,
// workspace management and kernel launches behind the C ABI in include/gqa_av.h.
//
// Mode resolution and eligibility follow the dispatch and override bullets of
// ExecuTorch PR #21063, "...GEMV", implementation section: the reuse variant
// is picked when Hq > Hkv and Hq divides evenly by Hkv, the per-head kernel
// otherwise, and a forced reuse on an ineligible shape is an error. The page
// also caps G at 8 and sends larger groups to the per-head kernel; that cap
// is not kept: any G takes the reuse path (G > 16 in sub-groups of 16 heads).
#include "gqa_av.h"
#include "gqa_fp8_av.h"
#include "gqa_paged_av.h"
#include "gqa_attention.h"
#include "gqa_softmax_av.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "combine_kernels.hpp"
#include "dispatch.hpp"

namespace {

using gqa_av::Pass1Args;

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int elem_bytes(int dt) { return dt == GQA_AV_F32 ? 4 : (dt == GQA_AV_FP8_E4M3 ? 1 : 2); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compile-time head capacity of a VALU reuse tile for a group of G heads:
// exactly G up to 8, two tiles of 8 for 9..15, tiles of 16 beyond. Never more
// than Hq (>= G), so a tile's weight window fits inside an attn row.
int head_capacity(int64_t G) {
    if (G <= 8) return static_cast<int>(G);
    if (G < 16) return 8;
    return 16;
}


constexpr int kDefaultCUs = 256;
// Context-split sizing, measured on MI355X. The engines stream best with few
// long-running workgroups (VALU about 2 per CU, the matrix engines about 1):
// a plain streaming read shows the same (7.0 TB/s with 512-1024 blocks, 6.8
// with 4096).
constexpr int64_t kMinRowsPerSplit = 128;     // VALU: below this a split's epilogue dominates
constexpr int64_t kMinRowsPerSplitMfma = 256;
constexpr int64_t kTargetWgPerCuValu = 2;
constexpr int64_t kTargetWgPerCuMfma = 1;
constexpr int64_t kMinRowsPerSplitBf16 = 512;  // bf16 matrix engine: measured best for MQA at B = 4, C = 32768
constexpr int64_t kTargetWgPerCuBf16 = 1;
// The fused softmax product and fused attention over fp8 values do twice the
// matrix, LDS and exp work per byte read and run better with two workgroups
// per CU. Measured on MI355X, B = 64, C = 8192, Hkv = 8, G = 8: attention
// takes 204 us on 512 workgroups against 225 on 256, the fused softmax
// product 130 against 143; attention at B = 4, C = 32768, Hkv = 8, G = 2
// takes 60 against 64.5. (The plain fp8 product stays at one: 112.6 against
// 118.4.)
constexpr int64_t kTargetWgPerCuBf16Fp8Sm = 2;
// Fused attention on grids smaller than the chip (B = 1, C = 4096, Hkv = 8,
// G = 4): 32 splits of 128 rows take 10.2 us (fp8 K and V: 11.2) against
// 14.2 (16.3) for 8 splits of 512 rows.
constexpr int64_t kMinRowsPerSplitAttn = 128;

// Split-C workspace of one (device, stream). The per-tile counters live in a
// buffer of their own: they must be zero before a call, every call leaves the
// ones it used at zero again, and no partial sum may ever land on them,
// whatever the next plan's layout.
struct Workspace {
    void* counters = nullptr;
    size_t counter_bytes = 0;
    void* part = nullptr;
    size_t part_bytes = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

std::mutex g_cu_mutex;
std::map<int, int> g_cu_count;

int device_cus(int dev, int* cus) {
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    auto it = g_cu_count.find(dev);
    if (it != g_cu_count.end()) {
        *cus = it->second;
        return GQA_AV_OK;
    }
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    g_cu_count[dev] = n;
    *cus = n;
    return GQA_AV_OK;
}

// Grow `*buf` to at least `bytes`. Earlier calls on `stream` may still use the
// old buffer, so the stream is synchronised before it is freed. A new counter
// buffer is zeroed on the stream.
int grow(void** buf, size_t* have, size_t bytes, hipStream_t stream, bool zero) {
    if (*have >= bytes) return GQA_AV_OK;
    if (*buf) {
        hipError_t e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
        e = hipFree(*buf);
        *buf = nullptr;
        *have = 0;
        if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipFree: %s", hipGetErrorString(e));
    }
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipMalloc(%zu) for split-C workspace: %s", bytes, hipGetErrorString(e));
    if (zero) {
        e = hipMemsetAsync(p, 0, bytes, stream);
        if (e != hipSuccess) {
            (void)hipFree(p);
            return fail(GQA_AV_ERR_HIP, "hipMemsetAsync: %s", hipGetErrorString(e));
        }
    }
    *buf = p;
    *have = bytes;
    return GQA_AV_OK;
}

int get_workspace(int dev, hipStream_t stream, size_t counter_bytes, size_t part_bytes, uint32_t** counters,
                  float** part) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& ws = g_ws[{dev, stream}];
    int rc = GQA_AV_OK;
    if (counter_bytes > 0) rc = grow(&ws.counters, &ws.counter_bytes, counter_bytes, stream, true);
    if (rc == GQA_AV_OK) rc = grow(&ws.part, &ws.part_bytes, part_bytes, stream, false);
    if (rc != GQA_AV_OK) return rc;
    *counters = static_cast<uint32_t*>(ws.counters);
    *part = static_cast<float*>(ws.part);
    return GQA_AV_OK;
}

int check_sizes(int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int v_dtype) {
    if (B < 0 || C < 0) return fail(GQA_AV_ERR_INVALID_ARG, "B=%lld and C=%lld must be >= 0", (long long)B, (long long)C);
    if (Hq < 1 || Hkv < 1 || D < 1)
        return fail(GQA_AV_ERR_INVALID_ARG, "Hq=%lld, Hkv=%lld and D=%lld must be >= 1", (long long)Hq, (long long)Hkv, (long long)D);
    if (Hq % Hkv != 0)
        return fail(GQA_AV_ERR_INVALID_ARG, "Hq=%lld is not a multiple of Hkv=%lld", (long long)Hq, (long long)Hkv);
    if (v_dtype != GQA_AV_F32 && v_dtype != GQA_AV_F16 && v_dtype != GQA_AV_BF16 && v_dtype != GQA_AV_FP8_E4M3)
        return fail(GQA_AV_ERR_INVALID_ARG, "unknown v_dtype %d", v_dtype);
    // Index arithmetic inside the kernels keeps these in 32 bits.
    if (B > INT32_MAX || Hq > INT32_MAX || D > INT32_MAX)
        return fail(GQA_AV_ERR_UNSUPPORTED, "B, Hq and D must each fit in 31 bits");
    return GQA_AV_OK;
}

// ---- kernel dispatch ----------------------------------------------------------

hipError_t launch_pass1(int v_dtype, const gqa_av_plan& p, int64_t D, const Pass1Args& a, hipStream_t s) {
    const int dt = v_dtype == GQA_AV_F32 ? gqa_av::kF32
                 : v_dtype == GQA_AV_F16 ? gqa_av::kF16
                 : v_dtype == GQA_AV_BF16 ? gqa_av::kBF16 : gqa_av::kFP8;
    if (p.attention) {
        if ((v_dtype != GQA_AV_BF16 && v_dtype != GQA_AV_FP8_E4M3) || p.engine != GQA_AV_ENGINE_MFMA_BF16 ||
            !p.softmax)
            return hipErrorInvalidValue;
        const int nset = p.heads_per_tile / 16, ht = p.kv_heads_per_tile;
        using namespace gqa_av_launch;
        if (p.page_size > 0)
            return v_dtype == GQA_AV_FP8_E4M3 ? mfma_bf16<gqa_av::kFP8, true, true, true>(D, nset, ht, a, s)
                                              : mfma_bf16<gqa_av::kBF16, true, true, true>(D, nset, ht, a, s);
        return v_dtype == GQA_AV_FP8_E4M3 ? mfma_bf16<gqa_av::kFP8, true, false, true>(D, nset, ht, a, s)
                                          : mfma_bf16<gqa_av::kBF16, true, false, true>(D, nset, ht, a, s);
    }
    if (p.engine == GQA_AV_ENGINE_MFMA_BF16) {
        if (v_dtype != GQA_AV_BF16 && v_dtype != GQA_AV_FP8_E4M3) return hipErrorInvalidValue;
        const int nset = p.heads_per_tile / 16, ht = p.kv_heads_per_tile;
        using namespace gqa_av_launch;
        if (p.page_size > 0) {
            if (v_dtype == GQA_AV_FP8_E4M3)
                return p.softmax ? mfma_bf16<gqa_av::kFP8, true, true>(D, nset, ht, a, s)
                                 : mfma_bf16<gqa_av::kFP8, false, true>(D, nset, ht, a, s);
            return p.softmax ? mfma_bf16<gqa_av::kBF16, true, true>(D, nset, ht, a, s)
                             : mfma_bf16<gqa_av::kBF16, false, true>(D, nset, ht, a, s);
        }
        if (v_dtype == GQA_AV_FP8_E4M3)
            return p.softmax ? mfma_bf16<gqa_av::kFP8, true>(D, nset, ht, a, s)
                             : mfma_bf16<gqa_av::kFP8, false>(D, nset, ht, a, s);
        return p.softmax ? mfma_bf16<gqa_av::kBF16, true>(D, nset, ht, a, s)
                         : mfma_bf16<gqa_av::kBF16, false>(D, nset, ht, a, s);
    }
    if (p.engine == GQA_AV_ENGINE_MFMA) {
        if (p.softmax || p.page_size > 0 || v_dtype == GQA_AV_FP8_E4M3) return hipErrorInvalidValue;
        return gqa_av_launch::mfma(dt, static_cast<int>(D / 16), p.heads_per_tile / 16, a, s);
    }
    const bool pg = p.page_size > 0;
    const int VB = p.vec_bytes, GT = p.heads_per_tile;
    switch (dt) {
    case gqa_av::kF32:
        return p.softmax ? gqa_av_launch::valu<gqa_av::kF32, true>(VB, GT, pg, a, s)
                         : gqa_av_launch::valu<gqa_av::kF32, false>(VB, GT, pg, a, s);
    case gqa_av::kF16:
        return p.softmax ? gqa_av_launch::valu<gqa_av::kF16, true>(VB, GT, pg, a, s)
                         : gqa_av_launch::valu<gqa_av::kF16, false>(VB, GT, pg, a, s);
    case gqa_av::kBF16:
        return p.softmax ? gqa_av_launch::valu<gqa_av::kBF16, true>(VB, GT, pg, a, s)
                         : gqa_av_launch::valu<gqa_av::kBF16, false>(VB, GT, pg, a, s);
    default:
        return p.softmax ? gqa_av_launch::valu<gqa_av::kFP8, true>(VB, GT, pg, a, s)
                         : gqa_av_launch::valu<gqa_av::kFP8, false>(VB, GT, pg, a, s);
    }
}

// Address alignment a lane load of `vec_bytes` needs: its own size up to 16
// bytes (a 32-byte load is two 16-byte ones); 12-byte loads need 4.
int load_alignment(int vec_bytes) {
    if (vec_bytes == 12) return 4;
    return vec_bytes > 16 ? 16 : vec_bytes;
}

// Can the MFMA engine take this problem? D splits into 16 lane chunks whose
// byte size is one of the engine's load widths, V is aligned for that width,
// and the four waves' 16 x D tiles fit the 64 KB LDS reduction buffer.
bool mfma_fits(int64_t D, int es, int v_align, int nset) {
    if (D % 16 != 0) return false;
    const int64_t DE = D / 16, NB = DE * es;
    if (!(NB == 4 || NB == 8 || NB == 12 || NB == 16 || NB == 32)) return false;
    if (v_align % load_alignment(static_cast<int>(NB)) != 0) return false;
    return nset * DE <= 16 && (nset == 1 || DE <= 8);
}

// Can the bf16 matrix-core engine take this problem? bf16 V, D of 64, 128 or
// 256 (whole 16-byte pieces per row, a power of two of them for the LDS
// swizzle), 16-byte aligned V, rows of V and attn of at most 1 MB, and the
// same 64 KB bound on the four waves' tiles as the fp32 engine.
bool mfma_bf16_fits(int v_dtype, int64_t Hq, int64_t Hkv, int64_t D, int v_align, int nset) {
    if ((v_dtype != GQA_AV_BF16 && v_dtype != GQA_AV_FP8_E4M3) || !(D == 64 || D == 128 || D == 256)) return false;
    const int es = v_dtype == GQA_AV_FP8_E4M3 ? 1 : 2;
    if (Hkv * D * es > (int64_t{1} << 20) || Hq * 4 > (int64_t{1} << 20)) return false;  // row bytes for 32-bit offsets
    if (v_align % (8 * es) != 0) return false;       // 8-value pieces
    return nset * D <= 256;
}

constexpr int64_t kMfmaMinGroup = 5;     // below this the VALU engine does less work

constexpr int64_t kCounterBytes = 256;          // the counter block is padded to this

int64_t counter_bytes(int64_t tiles) { return ceil_div(tiles * 4, kCounterBytes) * kCounterBytes; }

// Floats from the start of the split planes to the fused softmax's statistics
// (the planes rounded up to whole 16-byte groups).
int64_t stats_offset(int64_t nsplit, int64_t B, int64_t Hq, int64_t D) { return (nsplit * B * Hq * D + 3) / 4 * 4; }

// KERNEL: one fp32 plane of `out` per split, and for the fused softmax one
// (maximum, weight sum) pair per split and (b, q_h) after the planes. LAST:
// [tiles][nsplit][tile outputs] partials plus one counter per tile.
int64_t workspace_bytes(int64_t B, int64_t Hq, int64_t D, int64_t tiles, int64_t nsplit, int64_t tile_outputs,
                        int combine, bool softmax) {
    if (nsplit <= 1) return 0;
    if (combine == GQA_AV_COMBINE_LAST)
        return counter_bytes(tiles) + tiles * nsplit * gqa_av::padded_outputs(static_cast<int>(tile_outputs)) * 4;
    if (softmax) return stats_offset(nsplit, B, Hq, D) * 4 + nsplit * B * Hq * 2 * 4;
    return nsplit * B * Hq * D * 4;
}

int plan_impl(int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int v_dtype, int mode,
              const gqa_av_hint* hint, int cu_default, gqa_av_plan* plan) {
    int rc = check_sizes(B, C, Hq, Hkv, D, v_dtype);
    if (rc != GQA_AV_OK) return rc;
    const int resolved = gqa_av_resolve_mode(Hq, Hkv, mode);
    if (resolved < 0) return -resolved;
    if (!plan) return fail(GQA_AV_ERR_INVALID_ARG, "plan is NULL");

    gqa_av_hint h;
    std::memset(&h, 0, sizeof h);
    if (hint) h = *hint;
    if (h.engine < GQA_AV_ENGINE_AUTO || h.engine > GQA_AV_ENGINE_MFMA_BF16)
        return fail(GQA_AV_ERR_INVALID_ARG, "unknown engine %d", h.engine);
    if (h.combine < GQA_AV_COMBINE_AUTO || h.combine > GQA_AV_COMBINE_LAST)
        return fail(GQA_AV_ERR_INVALID_ARG, "unknown combine %d", h.combine);
    if (h.softmax != 0 && h.softmax != 1) return fail(GQA_AV_ERR_INVALID_ARG, "hint softmax must be 0 or 1");
    if (h.attention != 0 && h.attention != 1) return fail(GQA_AV_ERR_INVALID_ARG, "hint attention must be 0 or 1");
    // Fused attention: the fused softmax product on the bf16 matrix engine, its
    // scores computed from q and K.
    const bool attention = h.attention == 1;
    if (attention) {
        if (v_dtype != GQA_AV_BF16 && v_dtype != GQA_AV_FP8_E4M3)
            return fail(GQA_AV_ERR_UNSUPPORTED, "fused attention takes bf16 or fp8 K and V");
        if (h.engine != GQA_AV_ENGINE_AUTO && h.engine != GQA_AV_ENGINE_MFMA_BF16)
            return fail(GQA_AV_ERR_UNSUPPORTED, "fused attention runs on the bf16 matrix engine");
        h.softmax = 1;
        h.engine = GQA_AV_ENGINE_MFMA_BF16;
    }
    const bool sm = h.softmax == 1;
    // Paged V: the VALU engine with 16-byte lane loads or the bf16 matrix
    // engine, the kernel combine, and splits short enough for their page list
    // to fit in LDS.
    const int64_t P = h.page_size;
    const bool paged = P > 0;
    if (P < 0 || (paged && (P & (P - 1)) != 0))
        return fail(GQA_AV_ERR_INVALID_ARG, "page_size %lld must be a power of two", (long long)P);
    if (paged && h.engine == GQA_AV_ENGINE_MFMA)
        return fail(GQA_AV_ERR_UNSUPPORTED, "paged V runs on the VALU or bf16 matrix engine");
    const int cus = h.cu_count > 0 ? h.cu_count : cu_default;
    const int v_align = h.v_align > 0 ? h.v_align : 16;

    const int es = elem_bytes(v_dtype);
    const int64_t G = Hq / Hkv;

    // Engine. The matrix-core engines always compute 16 (or 32) heads per
    // tile, so they only pay off for larger groups; the per-head baseline is
    // always the VALU engine with one head per tile. For bf16 V the bf16
    // matrix engine is preferred: the fp32 one keeps the SIMDs about 80 %
    // busy at full bandwidth with 16 heads per tile.
    const int nset = (G > 16 && mfma_fits(D, es, v_align, 2)) ? 2 : 1;
    const bool mfma_ok = resolved == GQA_AV_REUSE && mfma_fits(D, es, v_align, nset);
    const int nset16 = (G > 16 && mfma_bf16_fits(v_dtype, Hq, Hkv, D, v_align, 2)) ? 2 : 1;
    const bool mfma16_ok = resolved == GQA_AV_REUSE && mfma_bf16_fits(v_dtype, Hq, Hkv, D, v_align, nset16);
    int engine = h.engine;
    if (engine == GQA_AV_ENGINE_AUTO) {
        engine = GQA_AV_ENGINE_VALU;
        if (G >= kMfmaMinGroup && mfma16_ok) engine = GQA_AV_ENGINE_MFMA_BF16;
        else if (G >= kMfmaMinGroup && mfma_ok && !sm && !paged && v_dtype != GQA_AV_FP8_E4M3)
            engine = GQA_AV_ENGINE_MFMA;
    }
    if (sm && engine == GQA_AV_ENGINE_MFMA)
        return fail(GQA_AV_ERR_UNSUPPORTED, "the fused softmax runs on the VALU or bf16 matrix engine");
    if (v_dtype == GQA_AV_FP8_E4M3 && engine == GQA_AV_ENGINE_MFMA)
        return fail(GQA_AV_ERR_UNSUPPORTED, "fp8 V runs on the VALU or bf16 matrix engine");
    if (engine == GQA_AV_ENGINE_MFMA && !mfma_ok)
        return fail(GQA_AV_ERR_UNSUPPORTED,
                    "MFMA engine needs reuse mode, D %% 16 == 0 with a 4/8/12/16/32-byte lane chunk and matching V alignment");
    if (engine == GQA_AV_ENGINE_MFMA_BF16 && !mfma16_ok)
        return fail(GQA_AV_ERR_UNSUPPORTED,
                    "bf16 MFMA engine needs reuse mode, bf16 or fp8 V, D of 64, 128 or 256 and V aligned to 8 values");
    const bool matrix = engine == GQA_AV_ENGINE_MFMA || engine == GQA_AV_ENGINE_MFMA_BF16;

    // KV heads per tile: the VALU and bf16 matrix engines in reuse mode can
    // stream several adjacent KV heads, i.e. a contiguous ht x D slice of each
    // row. Automatic: the widest tile (VALU: 2 heads; bf16 matrix: 4, else 2)
    // whose split grid still reaches the engine's workgroup target with
    // splits of its minimum length. Measured on MI355X: two heads run 4-12 %
    // faster than one for VALU; a plain streaming read of 2 KB rows in
    // 512-byte slices runs at 7.1 TB/s against 6.8 TB/s in 256-byte slices;
    // the bf16 matrix engine on B = 64, C = 8192, Hkv = 8, G = 8 takes 193 us
    // with one head per tile, 181 with two and 177 with four. fp8 V differs:
    // there two heads without a split take 112 us against 117.7 with four
    // heads and two splits, and the VALU engine also takes four heads while a
    // tile row stays within 512 bytes (G = 3, D = 96: 26.6 us against 28.1).
    int ht = h.kv_tile > 0 ? h.kv_tile : 1;
    const bool bf16_engine = engine == GQA_AV_ENGINE_MFMA_BF16;
    const int64_t wg_per_cu_bf16 =
        h.softmax == 1 && v_dtype == GQA_AV_FP8_E4M3 ? kTargetWgPerCuBf16Fp8Sm : kTargetWgPerCuBf16;
    if (h.kv_tile <= 0 && resolved == GQA_AV_REUSE &&
        (engine == GQA_AV_ENGINE_VALU || bf16_engine)) {
        const bool fp8 = v_dtype == GQA_AV_FP8_E4M3;
        const int64_t lanes = (D * es) / 16 > 0 && (D * es) % 16 == 0 ? (D * es) / 16 : 0;
        const int64_t nsgw = ceil_div(G, bf16_engine ? 16 * nset16 : head_capacity(G));
        const int64_t target = (bf16_engine ? wg_per_cu_bf16 : kTargetWgPerCuValu) * cus;
        const int64_t min_rows = bf16_engine ? kMinRowsPerSplitBf16 : kMinRowsPerSplit;
        for (int cand : {4, 2}) {
            const bool four = bf16_engine ? !fp8 : (fp8 && 4 * D * es <= 512);
            if ((cand == 4 && !four) || Hkv % cand != 0) continue;
            const int64_t tiles_w = B * (Hkv / cand) * nsgw;
            if (lanes > 0 && (bf16_engine || cand * lanes <= gqa_av::kThreads) && v_align % 16 == 0 &&
                tiles_w > 0 &&
                tiles_w * std::min<int64_t>(ceil_div(target, tiles_w), std::max<int64_t>(1, C / min_rows)) >= target) {
                ht = cand;
                break;
            }
        }
    }
    if (ht > 1) {
        if (resolved != GQA_AV_REUSE || !(engine == GQA_AV_ENGINE_VALU || bf16_engine))
            return fail(GQA_AV_ERR_UNSUPPORTED, "kv_tile > 1 needs the VALU or bf16 matrix engine in reuse mode");
        if (Hkv % ht != 0)
            return fail(GQA_AV_ERR_INVALID_ARG, "kv_tile %d does not divide Hkv=%lld", ht, (long long)Hkv);
        if (bf16_engine && ht != 2 && ht != 4)
            return fail(GQA_AV_ERR_UNSUPPORTED, "the bf16 matrix engine takes 1, 2 or 4 KV heads per tile");
        if (sm && ht > 4) return fail(GQA_AV_ERR_UNSUPPORTED, "the fused softmax takes at most 4 KV heads per tile");
    }

    int VB, GT, nsg;
    int64_t Lc, rps, ndt, rows_per_step, tile_outputs;
    int64_t heads_major;  // tiles along the head axis per KV head
    if (engine == GQA_AV_ENGINE_MFMA_BF16) {
        VB = v_dtype == GQA_AV_FP8_E4M3 ? 8 : 16;    // one 8-value piece per lane load
        GT = 16 * nset16;
        nsg = static_cast<int>(ceil_div(G, GT));
        heads_major = nsg;
        Lc = ht * D / 8;                // 16-byte pieces of a tile row
        rps = 32 * gqa_av::kWaves / ht; // one 32-row chunk per wave, kWaves / ht waves per KV head
        ndt = 1;
        rows_per_step = rps * GQA_AV_MFMA_BF16_CHUNKS;
        tile_outputs = static_cast<int64_t>(ht) * GT * D;
    } else if (engine == GQA_AV_ENGINE_MFMA) {
        const int64_t DE = D / 16;
        VB = static_cast<int>(DE * es);
        GT = 16 * nset;
        nsg = static_cast<int>(ceil_div(G, GT));
        heads_major = nsg;
        Lc = 16;
        rps = 16;                       // 4 waves x 4 rows per MFMA
        ndt = 1;
        rows_per_step = 4 * gqa_av::kWaves * gqa_av::mfma_unroll(VB);
        tile_outputs = static_cast<int64_t>(GT) * D;
    } else {
        // Widest lane load that divides a D-row and respects V's alignment
        // (fp8: 16 values per lane only for tiles of up to 4 heads, else 8, so
        // a lane holds at most 64 or GT x 8 accumulators).
        const int gt_planned = resolved == GQA_AV_REUSE ? head_capacity(G) : 1;
        VB = 0;
        for (int cand = (v_dtype == GQA_AV_FP8_E4M3 && gt_planned > 4) ? 8 : 16; cand >= std::max(es, 2);
             cand /= 2) {
            if ((D * es) % cand == 0 && v_align % cand == 0) { VB = cand; break; }
        }
        if (VB == 0)
            return fail(GQA_AV_ERR_UNSUPPORTED, "V must be aligned to its element size (%d bytes)", es);
        if (paged && VB != 16)
            return fail(GQA_AV_ERR_UNSUPPORTED, "paged V needs rows of whole 16-byte pieces and 16-byte aligned pages");
        const int64_t E = VB / es;
        const int64_t L = D / E;
        if (ht > 1) {
            // Several adjacent KV heads per workgroup: their D-rows form one
            // contiguous tile row, which must fit the workgroup's lanes.
            if (L * ht > gqa_av::kThreads)
                return fail(GQA_AV_ERR_UNSUPPORTED, "kv_tile %d: %lld lanes per tile row exceed %d", ht,
                            (long long)(L * ht), gqa_av::kThreads);
            Lc = L * ht;
            ndt = 1;
        } else {
            Lc = L < gqa_av::kThreads ? L : gqa_av::kThreads;
            ndt = ceil_div(L, Lc);
        }
        rps = gqa_av::kThreads / Lc;
        if (rps > gqa_av::kMaxRowSlots) rps = gqa_av::kMaxRowSlots;
        if (resolved == GQA_AV_REUSE) {
            GT = head_capacity(G);
            nsg = static_cast<int>(ceil_div(G, GT));
            heads_major = nsg;
        } else {
            GT = 1;
            nsg = 1;
            heads_major = G;
        }
        rows_per_step = rps * gqa_av::valu_unroll(GT);
        tile_outputs = static_cast<int64_t>(GT) * E * Lc;
    }
    const int64_t tiles = B * (Hkv / ht) * heads_major * ndt;

    int64_t nsplit = 1, rows_per_split = C;
    if (C > 0) {
        if (h.nsplit > 0) {
            nsplit = h.nsplit < C ? h.nsplit : C;
            rows_per_split = ceil_div(C, nsplit);
        } else {
            const int64_t target =
                (bf16_engine ? wg_per_cu_bf16 : matrix ? kTargetWgPerCuMfma : kTargetWgPerCuValu) * cus;
            nsplit = tiles > 0 ? ceil_div(target, tiles) : 1;
            const int64_t cap =
                ceil_div(C, bf16_engine ? kMinRowsPerSplitBf16 : matrix ? kMinRowsPerSplitMfma : kMinRowsPerSplit);
            if (nsplit > cap) nsplit = cap;
            if (attention && tiles * nsplit < cus) {
                // Fused attention with fewer workgroups than CUs: shorter
                // splits, down to kMinRowsPerSplitAttn rows, give each CU one.
                nsplit = std::min(ceil_div(cus, tiles), ceil_div(C, kMinRowsPerSplitAttn));
            }
            if (nsplit < 1) nsplit = 1;
            rows_per_split = ceil_div(ceil_div(C, nsplit), rows_per_step) * rows_per_step;
        }
        nsplit = ceil_div(C, rows_per_split);
        if (engine != GQA_AV_ENGINE_MFMA) {
            // The VALU and bf16 matrix engines address one split of V and attn
            // through buffer resources with 32-bit offsets (the pipeline's last
            // reads run up to two steps past the split): keep a split under 1 GB.
            const int64_t row_bytes = std::max<int64_t>(Hkv * D * es, Hq * 4);
            const int64_t max_rows = (int64_t{1} << 30) / row_bytes - 2 * rows_per_step;
            if (max_rows < 1) return fail(GQA_AV_ERR_UNSUPPORTED, "one context row of V or attn exceeds 1 GB");
            if (rows_per_split > max_rows) {
                rows_per_split = max_rows;
                nsplit = ceil_div(C, rows_per_split);
            }
        }
    }
    if (paged && C > 0) {
        // A split of R rows touches at most ceil(R / P) + 1 pages.
        const int64_t max_rows = (gqa_av::kMaxSplitPages - 1) * P;
        if (rows_per_split > max_rows) {
            if (h.nsplit > 0)
                return fail(GQA_AV_ERR_UNSUPPORTED, "paged V: a split of %lld rows spans more than %d pages",
                            (long long)rows_per_split, gqa_av::kMaxSplitPages);
            rows_per_split = max_rows / rows_per_step * rows_per_step;
            if (rows_per_split < 1) rows_per_split = max_rows;
            nsplit = ceil_div(C, rows_per_split);
        }
    }
    if (nsplit > INT32_MAX) return fail(GQA_AV_ERR_UNSUPPORTED, "too many context splits");
    const int64_t grid = tiles * nsplit;
    if (grid > INT32_MAX) return fail(GQA_AV_ERR_UNSUPPORTED, "grid of %lld workgroups is too large", (long long)grid);

    std::memset(plan, 0, sizeof *plan);
    plan->mode = resolved;
    plan->engine = engine;
    plan->heads_per_tile = GT;
    plan->subgroups = nsg;
    plan->vec_bytes = VB;
    plan->lanes_per_row = static_cast<int32_t>(Lc);
    plan->row_slots = static_cast<int32_t>(rps);
    plan->d_tiles = static_cast<int32_t>(ndt);
    plan->nsplit = static_cast<int32_t>(nsplit);
    plan->threads = gqa_av::kThreads;
    plan->rows_per_split = rows_per_split;
    plan->grid = grid;
    int combine = GQA_AV_COMBINE_AUTO;
    if (nsplit > 1) {
        combine = h.combine;
        // Measured on MI355X: the second kernel is faster on every decode
        // workload (the last-workgroup combine pays for device-coherent
        // stores and loads of the partials), so it is the automatic choice.
        if (combine == GQA_AV_COMBINE_AUTO) combine = GQA_AV_COMBINE_KERNEL;
        if ((sm || paged) && combine != GQA_AV_COMBINE_KERNEL)
            return fail(GQA_AV_ERR_UNSUPPORTED, "the fused softmax combines its splits in a second kernel");
        // One tile's block is addressed through a 32-bit buffer offset.
        if (combine == GQA_AV_COMBINE_LAST && nsplit * gqa_av::padded_outputs(static_cast<int>(tile_outputs)) * 4 > INT32_MAX)
            return fail(GQA_AV_ERR_UNSUPPORTED, "a tile's split partials exceed 2 GB; use the kernel combine");
    }
    plan->combine = combine;
    plan->kv_heads_per_tile = ht;
    plan->workspace_bytes = workspace_bytes(B, Hq, D, tiles, nsplit, tile_outputs, combine, sm);
    plan->v_bytes_read = B * C * Hkv * D * es * heads_major;
    plan->softmax = sm ? 1 : 0;
    plan->page_size = static_cast<int32_t>(P);
    plan->attention = attention ? 1 : 0;
    return GQA_AV_OK;
}

bool same_plan(const gqa_av_plan& a, const gqa_av_plan& b) {
    return a.mode == b.mode && a.engine == b.engine && a.heads_per_tile == b.heads_per_tile &&
           a.subgroups == b.subgroups && a.vec_bytes == b.vec_bytes && a.lanes_per_row == b.lanes_per_row &&
           a.row_slots == b.row_slots && a.d_tiles == b.d_tiles && a.nsplit == b.nsplit &&
           a.threads == b.threads && a.rows_per_split == b.rows_per_split && a.grid == b.grid &&
           a.workspace_bytes == b.workspace_bytes && a.kv_heads_per_tile == b.kv_heads_per_tile &&
           a.softmax == b.softmax && a.page_size == b.page_size && a.attention == b.attention;
}

}  // namespace

extern "C" {

int gqa_av_resolve_mode(int64_t Hq, int64_t Hkv, int mode) {
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) {
        fail(GQA_AV_ERR_INVALID_ARG, "head shape Hq=%lld, Hkv=%lld: need Hq, Hkv >= 1 and Hq %% Hkv == 0",
             (long long)Hq, (long long)Hkv);
        return -GQA_AV_ERR_INVALID_ARG;
    }
    const bool eligible = Hq / Hkv >= 2;
    switch (mode) {
    case GQA_AV_AUTO: return eligible ? GQA_AV_REUSE : GQA_AV_PER_HEAD;
    case GQA_AV_PER_HEAD: return GQA_AV_PER_HEAD;
    case GQA_AV_REUSE:
        if (!eligible) {
            fail(GQA_AV_ERR_INELIGIBLE, "reuse forced with Hq=%lld, Hkv=%lld: group size %lld < 2",
                 (long long)Hq, (long long)Hkv, (long long)(Hq / Hkv));
            return -GQA_AV_ERR_INELIGIBLE;
        }
        return GQA_AV_REUSE;
    default:
        fail(GQA_AV_ERR_INVALID_ARG, "unknown mode %d", mode);
        return -GQA_AV_ERR_INVALID_ARG;
    }
}

int gqa_av_make_plan(int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int v_dtype, int mode,
                     const gqa_av_hint* hint, gqa_av_plan* plan) {
    return plan_impl(B, C, Hq, Hkv, D, v_dtype, mode, hint, kDefaultCUs, plan);
}

}  // extern "C"

namespace {

constexpr int kRunPass1 = 1, kRunCombine = 2;

// Validate (attn, V, out, sizes, plan) and launch the parts of the call named
// by `which`. Validation is the same for every part, so a caller splitting
// the call gets the same errors as gqa_av_decode_plan.
// The paged-cache arguments of gqa_av_paged_decode_plan.
struct PagedArgs {
    const int32_t* block_table;
    const int32_t* seq_lens;
    int64_t page_size, max_pages, num_pages;
};

// The query and key arguments of the fused attention entry points.
struct AttnArgs {
    const float* q;
    const void* K;
    float scale;
    const float* k_scale;   // fp8 K: [Hkv] or NULL
};

// softmax: 1 for the fused softmax entry points (attn then holds the scores);
// pg: the paged cache (V then points at its pages), or NULL for dense V.
int run_plan(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
             int64_t D, int v_dtype, const gqa_av_plan* plan, void* stream, int which, int softmax,
             const PagedArgs* pg = nullptr, const float* v_scale = nullptr, const AttnArgs* at = nullptr) {
    if (!plan) return fail(GQA_AV_ERR_INVALID_ARG, "plan is NULL");
    int rc = check_sizes(B, C, Hq, Hkv, D, v_dtype);
    if (rc != GQA_AV_OK) return rc;
    if ((plan->attention == 1) != (at != nullptr))
        return fail(GQA_AV_ERR_INVALID_ARG, at ? "not a fused attention plan (plan->attention == 0)"
                                                : "a fused attention plan: run it with gqa_attention_decode_plan");
    if ((plan->page_size > 0) != (pg != nullptr))
        return fail(GQA_AV_ERR_INVALID_ARG, pg ? "not a paged plan (plan->page_size == 0)"
                                                : "a paged plan: run it with gqa_av_paged_decode_plan");
    if (pg) {
        if (pg->page_size != plan->page_size)
            return fail(GQA_AV_ERR_INVALID_ARG, "page_size %lld does not match the plan's %d",
                        (long long)pg->page_size, plan->page_size);
        if (pg->max_pages < 1 || pg->max_pages > INT32_MAX || pg->num_pages < 1)
            return fail(GQA_AV_ERR_INVALID_ARG, "max_pages and num_pages must be >= 1 (max_pages < 2^31)");
        if (C > pg->max_pages * pg->page_size)
            return fail(GQA_AV_ERR_INVALID_ARG, "capacity C=%lld exceeds max_pages * page_size", (long long)C);
        if (B > 0 && (!pg->block_table || !pg->seq_lens))
            return fail(GQA_AV_ERR_INVALID_ARG, "block_table and seq_lens must not be NULL");
    }
    if (plan->softmax != softmax)
        return fail(GQA_AV_ERR_INVALID_ARG, softmax ? "not a fused softmax plan (plan->softmax == 0)"
                                                    : "a fused softmax plan: run it with gqa_softmax_av_decode_plan");
    // Re-derive the plan from its own choices and insist it matches.
    gqa_av_hint h;
    std::memset(&h, 0, sizeof h);
    h.engine = plan->engine;
    h.nsplit = plan->nsplit;
    h.v_align = plan->vec_bytes;
    h.combine = plan->combine;
    h.kv_tile = plan->kv_heads_per_tile;
    h.softmax = plan->softmax;
    h.page_size = plan->page_size;
    h.attention = plan->attention;
    gqa_av_plan check;
    const int mode = plan->mode;
    // Re-plan with the split count fixed: rows_per_split then follows from C.
    rc = plan_impl(B, C, Hq, Hkv, D, v_dtype, mode, &h, kDefaultCUs, &check);
    if (rc != GQA_AV_OK) return rc;
    check.rows_per_split = plan->rows_per_split;
    check.nsplit = plan->nsplit;
    check.grid = plan->grid;
    check.workspace_bytes = plan->workspace_bytes;
    check.combine = plan->combine;
    if (!same_plan(check, *plan)) return fail(GQA_AV_ERR_INVALID_ARG, "plan does not belong to this problem");
    if (plan->nsplit > 1 ? (plan->combine != GQA_AV_COMBINE_KERNEL && plan->combine != GQA_AV_COMBINE_LAST)
                         : plan->combine != GQA_AV_COMBINE_AUTO)
        return fail(GQA_AV_ERR_INVALID_ARG, "plan combine %d does not fit nsplit %d", plan->combine, plan->nsplit);
    // The split fields must still tile [0, C) exactly.
    if (C > 0) {
        if (plan->nsplit < 1 || plan->rows_per_split < 1 ||
            ceil_div(C, plan->rows_per_split) != plan->nsplit)
            return fail(GQA_AV_ERR_INVALID_ARG, "plan splits do not cover C=%lld", (long long)C);
    } else if (plan->nsplit != 1) {
        return fail(GQA_AV_ERR_INVALID_ARG, "C == 0 needs nsplit == 1");
    }
    const int64_t tiles_per_split = plan->grid / plan->nsplit;
    const int64_t heads_major = plan->mode == GQA_AV_REUSE ? plan->subgroups : Hq / Hkv;
    if (plan->kv_heads_per_tile < 1 || Hkv % plan->kv_heads_per_tile != 0)
        return fail(GQA_AV_ERR_INVALID_ARG, "plan kv_heads_per_tile does not divide Hkv");
    if (plan->grid % plan->nsplit != 0 ||
        tiles_per_split != B * (Hkv / plan->kv_heads_per_tile) * heads_major * plan->d_tiles)
        return fail(GQA_AV_ERR_INVALID_ARG, "plan grid does not match the problem");
    const int64_t tile_outputs = (plan->engine == GQA_AV_ENGINE_MFMA || plan->engine == GQA_AV_ENGINE_MFMA_BF16)
        ? static_cast<int64_t>(plan->heads_per_tile) * D * plan->kv_heads_per_tile
        : static_cast<int64_t>(plan->heads_per_tile) * (plan->vec_bytes / elem_bytes(v_dtype)) * plan->lanes_per_row;
    if (plan->workspace_bytes !=
        workspace_bytes(B, Hq, D, tiles_per_split, plan->nsplit, tile_outputs, plan->combine, plan->softmax == 1))
        return fail(GQA_AV_ERR_INVALID_ARG, "plan workspace does not match the problem");

    if (B == 0) return GQA_AV_OK;
    if (at) {
        if (C > 0 && (!at->q || !at->K)) return fail(GQA_AV_ERR_INVALID_ARG, "q and K must not be NULL");
        if (reinterpret_cast<uintptr_t>(at->q) & 3u) return fail(GQA_AV_ERR_INVALID_ARG, "q must be 4-byte aligned");
        if (reinterpret_cast<uintptr_t>(at->K) % static_cast<uintptr_t>(load_alignment(plan->vec_bytes)))
            return fail(GQA_AV_ERR_UNSUPPORTED, "K is not aligned to the plan's %d-byte loads", plan->vec_bytes);
    } else if (!attn && C > 0) {
        return fail(GQA_AV_ERR_INVALID_ARG, softmax ? "scores is NULL" : "attn is NULL");
    }
    if (!V && C > 0) return fail(GQA_AV_ERR_INVALID_ARG, "V is NULL");
    if (!out) return fail(GQA_AV_ERR_INVALID_ARG, "out is NULL");
    if ((reinterpret_cast<uintptr_t>(attn) & 3u) || (reinterpret_cast<uintptr_t>(out) & 3u))
        return fail(GQA_AV_ERR_INVALID_ARG, "attn and out must be 4-byte aligned");
    if (reinterpret_cast<uintptr_t>(V) % static_cast<uintptr_t>(load_alignment(plan->vec_bytes)))
        return fail(GQA_AV_ERR_UNSUPPORTED, "V is not aligned to the plan's %d-byte loads", plan->vec_bytes);

    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));

    float* part = nullptr;
    uint32_t* counters = nullptr;
    const bool last = plan->nsplit > 1 && plan->combine == GQA_AV_COMBINE_LAST;
    if (plan->nsplit > 1) {
        const int64_t cbytes = last ? counter_bytes(tiles_per_split) : 0;
        rc = get_workspace(dev, s, static_cast<size_t>(cbytes), static_cast<size_t>(plan->workspace_bytes - cbytes),
                           &counters, &part);
        if (rc != GQA_AV_OK) return rc;
    }

    Pass1Args a;
    a.attn = attn;
    a.V = static_cast<const uint8_t*>(V);
    a.out = out;
    a.part = part;
    a.stats = (softmax && plan->nsplit > 1) ? part + stats_offset(plan->nsplit, B, Hq, D) : nullptr;
    a.counters = counters;
    a.v_scale = v_scale;
    a.q = at ? at->q : nullptr;
    a.K = at ? static_cast<const uint8_t*>(at->K) : nullptr;
    a.qk_scale = at ? at->scale : 0.0f;
    a.k_scale = at ? at->k_scale : nullptr;
    a.block_table = pg ? pg->block_table : nullptr;
    a.seq_lens = pg ? pg->seq_lens : nullptr;
    a.num_pages = pg ? pg->num_pages : 0;
    a.max_pages = pg ? static_cast<int32_t>(pg->max_pages) : 0;
    a.page_shift = 0;
    if (pg)
        while ((int64_t{1} << a.page_shift) < pg->page_size) ++a.page_shift;
    a.combine = last ? 1 : 0;
    a.C = C;
    a.rows_per_split = plan->rows_per_split;
    a.B = static_cast<int32_t>(B);
    a.Hq = static_cast<int32_t>(Hq);
    a.Hkv = static_cast<int32_t>(Hkv);
    a.D = static_cast<int32_t>(D);
    a.G = static_cast<int32_t>(Hq / Hkv);
    a.per_head = plan->mode == GQA_AV_PER_HEAD;
    a.nsg = plan->subgroups;
    a.ndt = plan->d_tiles;
    a.nsplit = plan->nsplit;
    a.L = static_cast<int32_t>(D * elem_bytes(v_dtype) / plan->vec_bytes);
    a.ht = plan->kv_heads_per_tile;
    a.Lc = plan->lanes_per_row;
    a.rps = plan->row_slots;
    a.nblocks = static_cast<uint32_t>(plan->grid);

    if (which & kRunPass1) {
        e = launch_pass1(v_dtype, *plan, D, a, s);
        if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "pass-1 launch: %s", hipGetErrorString(e));
    }
    if ((which & kRunCombine) && plan->nsplit > 1 && softmax) {
        if (plan->nsplit <= gqa_av::kCombineBatch) {
            const int64_t threads = B * Hq * ceil_div(D, 4);
            const int64_t blocks = ceil_div(threads, gqa_av::kThreads);
            if (blocks > INT32_MAX) return fail(GQA_AV_ERR_UNSUPPORTED, "output too large for the softmax combine");
            if (D % 4 == 0)
                hipLaunchKernelGGL(gqa_av::av_pass2_softmax_combine_few<true>, dim3(static_cast<uint32_t>(blocks)),
                                   dim3(gqa_av::kThreads), 0, s, static_cast<const float*>(part),
                                   static_cast<const float*>(a.stats), out, a.D, B * Hq, a.nsplit);
            else
                hipLaunchKernelGGL(gqa_av::av_pass2_softmax_combine_few<false>, dim3(static_cast<uint32_t>(blocks)),
                                   dim3(gqa_av::kThreads), 0, s, static_cast<const float*>(part),
                                   static_cast<const float*>(a.stats), out, a.D, B * Hq, a.nsplit);
        } else if (D % 4 == 0) {
            hipLaunchKernelGGL(gqa_av::av_pass2_softmax_combine<true>, dim3(static_cast<uint32_t>(B * Hq)),
                               dim3(gqa_av::kThreads), 0, s, static_cast<const float*>(part),
                               static_cast<const float*>(a.stats), out, a.D, B * Hq, a.nsplit);
        } else {
            hipLaunchKernelGGL(gqa_av::av_pass2_softmax_combine<false>, dim3(static_cast<uint32_t>(B * Hq)),
                               dim3(gqa_av::kThreads), 0, s, static_cast<const float*>(part),
                               static_cast<const float*>(a.stats), out, a.D, B * Hq, a.nsplit);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "softmax combine launch: %s", hipGetErrorString(e));
    } else if ((which & kRunCombine) && plan->nsplit > 1 && !last) {
        const int64_t plane = B * Hq * D;
        const int64_t per_block = 4 * gqa_av::kQuadsPerBlock;
        const int64_t blocks = ceil_div(plane, per_block);
        if (blocks > INT32_MAX) return fail(GQA_AV_ERR_UNSUPPORTED, "output too large for the split-C combine");
        hipLaunchKernelGGL(gqa_av::av_pass2_combine, dim3(static_cast<uint32_t>(blocks)), dim3(gqa_av::kThreads),
                           0, s, static_cast<const float*>(part), out, plane, a.nsplit);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "pass-2 launch: %s", hipGetErrorString(e));
    }
    return GQA_AV_OK;
}

// The automatic plan for the current device and V's address alignment.
int auto_plan(const void* V, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int v_dtype, int mode,
              int softmax, gqa_av_plan* plan, int64_t page_size = 0, int attention = 0) {
    int rc = check_sizes(B, C, Hq, Hkv, D, v_dtype);
    if (rc != GQA_AV_OK) return rc;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    int cus = kDefaultCUs;
    rc = device_cus(dev, &cus);
    if (rc != GQA_AV_OK) return rc;
    gqa_av_hint h;
    std::memset(&h, 0, sizeof h);
    h.engine = GQA_AV_ENGINE_AUTO;
    h.cu_count = cus;
    h.softmax = softmax;
    h.attention = attention;
    if (page_size < 0 || page_size > INT32_MAX)
        return fail(GQA_AV_ERR_INVALID_ARG, "page_size %lld out of range", (long long)page_size);
    h.page_size = static_cast<int32_t>(page_size);
    // Alignment of V's address: its lowest set bit, at most 16.
    const uintptr_t addr = reinterpret_cast<uintptr_t>(V);
    const uintptr_t low = addr & (~addr + 1);
    h.v_align = (addr == 0 || low >= 16) ? 16 : static_cast<int32_t>(low);
    return plan_impl(B, C, Hq, Hkv, D, v_dtype, mode, &h, cus, plan);
}

}  // namespace

extern "C" {

int gqa_av_decode_plan(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                       int64_t Hkv, int64_t D, int v_dtype, const gqa_av_plan* plan, void* stream) {
    return run_plan(attn, V, out, B, C, Hq, Hkv, D, v_dtype, plan, stream, kRunPass1 | kRunCombine, 0);
}

int gqa_av_decode_pass1(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                        int64_t Hkv, int64_t D, int v_dtype, const gqa_av_plan* plan, void* stream) {
    return run_plan(attn, V, out, B, C, Hq, Hkv, D, v_dtype, plan, stream, kRunPass1, 0);
}

int gqa_av_decode_combine(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                          int64_t Hkv, int64_t D, int v_dtype, const gqa_av_plan* plan, void* stream) {
    return run_plan(attn, V, out, B, C, Hq, Hkv, D, v_dtype, plan, stream, kRunCombine, 0);
}

int gqa_av_decode(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                  int64_t D, int v_dtype, int mode, void* stream) {
    gqa_av_plan plan;
    int rc = auto_plan(V, B, C, Hq, Hkv, D, v_dtype, mode, 0, &plan);
    if (rc != GQA_AV_OK) return rc;
    return gqa_av_decode_plan(attn, V, out, B, C, Hq, Hkv, D, v_dtype, &plan, stream);
}

int gqa_softmax_av_decode(const float* scores, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                          int64_t Hkv, int64_t D, int v_dtype, int mode, void* stream) {
    gqa_av_plan plan;
    int rc = auto_plan(V, B, C, Hq, Hkv, D, v_dtype, mode, 1, &plan);
    if (rc != GQA_AV_OK) return rc;
    return gqa_softmax_av_decode_plan(scores, V, out, B, C, Hq, Hkv, D, v_dtype, &plan, stream);
}

int gqa_softmax_av_decode_plan(const float* scores, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                               int64_t Hkv, int64_t D, int v_dtype, const gqa_av_plan* plan, void* stream) {
    return run_plan(scores, V, out, B, C, Hq, Hkv, D, v_dtype, plan, stream, kRunPass1 | kRunCombine, 1);
}

int gqa_av_fp8_decode(const float* w, const void* V, const float* v_scale, float* out, int64_t B, int64_t C,
                      int64_t Hq, int64_t Hkv, int64_t D, int softmax, int mode, void* stream) {
    if (softmax != 0 && softmax != 1) return fail(GQA_AV_ERR_INVALID_ARG, "softmax must be 0 or 1");
    gqa_av_plan plan;
    int rc = auto_plan(V, B, C, Hq, Hkv, D, GQA_AV_FP8_E4M3, mode, softmax, &plan);
    if (rc != GQA_AV_OK) return rc;
    return gqa_av_fp8_decode_plan(w, V, v_scale, out, B, C, Hq, Hkv, D, &plan, stream);
}

}  // extern "C"

namespace {

int run_fp8(const float* w, const void* V, const float* v_scale, float* out, int64_t B, int64_t C, int64_t Hq,
            int64_t Hkv, int64_t D, const gqa_av_plan* plan, void* stream, int which) {
    if (!plan) return fail(GQA_AV_ERR_INVALID_ARG, "plan is NULL");
    if (v_scale && (reinterpret_cast<uintptr_t>(v_scale) & 3u))
        return fail(GQA_AV_ERR_INVALID_ARG, "v_scale must be 4-byte aligned");
    return run_plan(w, V, out, B, C, Hq, Hkv, D, GQA_AV_FP8_E4M3, plan, stream, which, plan->softmax, nullptr,
                    v_scale);
}

int run_paged(const float* w, const void* pages, const int32_t* block_table, const int32_t* seq_lens, float* out,
              int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages,
              int64_t num_pages, int v_dtype, const gqa_av_plan* plan, void* stream, int which) {
    if (!plan) return fail(GQA_AV_ERR_INVALID_ARG, "plan is NULL");
    PagedArgs pa{block_table, seq_lens, page_size, max_pages, num_pages};
    return run_plan(w, pages, out, B, C, Hq, Hkv, D, v_dtype, plan, stream, which, plan->softmax, &pa);
}

}  // namespace

extern "C" {

int gqa_av_fp8_decode_plan(const float* w, const void* V, const float* v_scale, float* out, int64_t B, int64_t C,
                           int64_t Hq, int64_t Hkv, int64_t D, const gqa_av_plan* plan, void* stream) {
    return run_fp8(w, V, v_scale, out, B, C, Hq, Hkv, D, plan, stream, kRunPass1 | kRunCombine);
}

int gqa_av_fp8_decode_pass1(const float* w, const void* V, const float* v_scale, float* out, int64_t B, int64_t C,
                            int64_t Hq, int64_t Hkv, int64_t D, const gqa_av_plan* plan, void* stream) {
    return run_fp8(w, V, v_scale, out, B, C, Hq, Hkv, D, plan, stream, kRunPass1);
}

int gqa_av_fp8_decode_combine(const float* w, const void* V, const float* v_scale, float* out, int64_t B, int64_t C,
                              int64_t Hq, int64_t Hkv, int64_t D, const gqa_av_plan* plan, void* stream) {
    return run_fp8(w, V, v_scale, out, B, C, Hq, Hkv, D, plan, stream, kRunCombine);
}

int gqa_av_paged_decode(const float* w, const void* pages, const int32_t* block_table, const int32_t* seq_lens,
                        float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                        int64_t max_pages, int64_t num_pages, int v_dtype, int softmax, int mode, void* stream) {
    if (softmax != 0 && softmax != 1) return fail(GQA_AV_ERR_INVALID_ARG, "softmax must be 0 or 1");
    if (page_size < 1) return fail(GQA_AV_ERR_INVALID_ARG, "page_size must be >= 1");
    gqa_av_plan plan;
    int rc = auto_plan(pages, B, C, Hq, Hkv, D, v_dtype, mode, softmax, &plan, page_size);
    if (rc != GQA_AV_OK) return rc;
    return gqa_av_paged_decode_plan(w, pages, block_table, seq_lens, out, B, C, Hq, Hkv, D, page_size, max_pages,
                                    num_pages, v_dtype, &plan, stream);
}

int gqa_av_paged_decode_plan(const float* w, const void* pages, const int32_t* block_table,
                             const int32_t* seq_lens, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                             int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages, int v_dtype,
                             const gqa_av_plan* plan, void* stream) {
    return run_paged(w, pages, block_table, seq_lens, out, B, C, Hq, Hkv, D, page_size, max_pages, num_pages, v_dtype,
                     plan, stream, kRunPass1 | kRunCombine);
}

int gqa_av_paged_decode_pass1(const float* w, const void* pages, const int32_t* block_table,
                              const int32_t* seq_lens, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                              int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages, int v_dtype,
                              const gqa_av_plan* plan, void* stream) {
    return run_paged(w, pages, block_table, seq_lens, out, B, C, Hq, Hkv, D, page_size, max_pages, num_pages, v_dtype,
                     plan, stream, kRunPass1);
}

int gqa_av_paged_decode_combine(const float* w, const void* pages, const int32_t* block_table,
                                const int32_t* seq_lens, float* out, int64_t B, int64_t C, int64_t Hq,
                                int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages,
                                int v_dtype, const gqa_av_plan* plan, void* stream) {
    return run_paged(w, pages, block_table, seq_lens, out, B, C, Hq, Hkv, D, page_size, max_pages, num_pages, v_dtype,
                     plan, stream, kRunCombine);
}

int gqa_softmax_av_decode_pass1(const float* scores, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                                int64_t Hkv, int64_t D, int v_dtype, const gqa_av_plan* plan, void* stream) {
    return run_plan(scores, V, out, B, C, Hq, Hkv, D, v_dtype, plan, stream, kRunPass1, 1);
}

int gqa_softmax_av_decode_combine(const float* scores, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                                  int64_t Hkv, int64_t D, int v_dtype, const gqa_av_plan* plan, void* stream) {
    return run_plan(scores, V, out, B, C, Hq, Hkv, D, v_dtype, plan, stream, kRunCombine, 1);
}

int gqa_attention_decode_plan(const float* q, const void* K, const void* V, float* out, int64_t B, int64_t C,
                              int64_t Hq, int64_t Hkv, int64_t D, int kv_dtype, float scale, const gqa_av_plan* plan,
                              void* stream) {
    const AttnArgs at{q, K, scale, nullptr};
    return run_plan(nullptr, V, out, B, C, Hq, Hkv, D, kv_dtype, plan, stream, kRunPass1 | kRunCombine, 1, nullptr,
                    nullptr, &at);
}

int gqa_attention_decode_pass1(const float* q, const void* K, const void* V, float* out, int64_t B, int64_t C,
                               int64_t Hq, int64_t Hkv, int64_t D, int kv_dtype, float scale,
                               const gqa_av_plan* plan, void* stream) {
    const AttnArgs at{q, K, scale, nullptr};
    return run_plan(nullptr, V, out, B, C, Hq, Hkv, D, kv_dtype, plan, stream, kRunPass1, 1, nullptr, nullptr, &at);
}

int gqa_attention_decode_combine(const float* q, const void* K, const void* V, float* out, int64_t B, int64_t C,
                                 int64_t Hq, int64_t Hkv, int64_t D, int kv_dtype, float scale,
                                 const gqa_av_plan* plan, void* stream) {
    const AttnArgs at{q, K, scale, nullptr};
    return run_plan(nullptr, V, out, B, C, Hq, Hkv, D, kv_dtype, plan, stream, kRunCombine, 1, nullptr, nullptr, &at);
}

int gqa_attention_decode(const float* q, const void* K, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                         int64_t Hkv, int64_t D, int kv_dtype, float scale, int mode, void* stream) {
    gqa_av_plan plan;
    int rc = auto_plan(V, B, C, Hq, Hkv, D, kv_dtype, mode, 1, &plan, 0, 1);
    if (rc != GQA_AV_OK) return rc;
    return gqa_attention_decode_plan(q, K, V, out, B, C, Hq, Hkv, D, kv_dtype, scale, &plan, stream);
}

}  // extern "C"

namespace {

int run_attention_fp8(const float* q, const void* K, const float* k_scale, const void* V, const float* v_scale,
                      float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                      const gqa_av_plan* plan, void* stream, int which) {
    if ((k_scale && (reinterpret_cast<uintptr_t>(k_scale) & 3u)) ||
        (v_scale && (reinterpret_cast<uintptr_t>(v_scale) & 3u)))
        return fail(GQA_AV_ERR_INVALID_ARG, "k_scale and v_scale must be 4-byte aligned");
    const AttnArgs at{q, K, scale, k_scale};
    return run_plan(nullptr, V, out, B, C, Hq, Hkv, D, GQA_AV_FP8_E4M3, plan, stream, which, 1, nullptr, v_scale, &at);
}

}  // namespace

extern "C" {

int gqa_attention_fp8_decode_plan(const float* q, const void* K, const float* k_scale, const void* V,
                                  const float* v_scale, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                  int64_t D, float scale, const gqa_av_plan* plan, void* stream) {
    return run_attention_fp8(q, K, k_scale, V, v_scale, out, B, C, Hq, Hkv, D, scale, plan, stream,
                             kRunPass1 | kRunCombine);
}

int gqa_attention_fp8_decode_pass1(const float* q, const void* K, const float* k_scale, const void* V,
                                   const float* v_scale, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                   int64_t D, float scale, const gqa_av_plan* plan, void* stream) {
    return run_attention_fp8(q, K, k_scale, V, v_scale, out, B, C, Hq, Hkv, D, scale, plan, stream, kRunPass1);
}

int gqa_attention_fp8_decode_combine(const float* q, const void* K, const float* k_scale, const void* V,
                                     const float* v_scale, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                     int64_t D, float scale, const gqa_av_plan* plan, void* stream) {
    return run_attention_fp8(q, K, k_scale, V, v_scale, out, B, C, Hq, Hkv, D, scale, plan, stream, kRunCombine);
}

int gqa_attention_fp8_decode(const float* q, const void* K, const float* k_scale, const void* V,
                             const float* v_scale, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                             int64_t D, float scale, int mode, void* stream) {
    gqa_av_plan plan;
    int rc = auto_plan(V, B, C, Hq, Hkv, D, GQA_AV_FP8_E4M3, mode, 1, &plan, 0, 1);
    if (rc != GQA_AV_OK) return rc;
    return gqa_attention_fp8_decode_plan(q, K, k_scale, V, v_scale, out, B, C, Hq, Hkv, D, scale, &plan, stream);
}

}  // extern "C"

namespace {

int run_attention_paged(const float* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                        const int32_t* seq_lens, const float* k_scale, const float* v_scale, float* out, int64_t B,
                        int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages,
                        int64_t num_pages, int kv_dtype, float scale, const gqa_av_plan* plan, void* stream,
                        int which) {
    if (kv_dtype != GQA_AV_BF16 && kv_dtype != GQA_AV_FP8_E4M3)
        return fail(GQA_AV_ERR_UNSUPPORTED, "fused attention takes bf16 or fp8 K and V");
    if (kv_dtype != GQA_AV_FP8_E4M3 && (k_scale || v_scale))
        return fail(GQA_AV_ERR_INVALID_ARG, "k_scale and v_scale are for fp8 K and V");
    if ((k_scale && (reinterpret_cast<uintptr_t>(k_scale) & 3u)) ||
        (v_scale && (reinterpret_cast<uintptr_t>(v_scale) & 3u)))
        return fail(GQA_AV_ERR_INVALID_ARG, "k_scale and v_scale must be 4-byte aligned");
    const PagedArgs pa{block_table, seq_lens, page_size, max_pages, num_pages};
    const AttnArgs at{q, k_pages, scale, k_scale};
    return run_plan(nullptr, v_pages, out, B, C, Hq, Hkv, D, kv_dtype, plan, stream, which, 1, &pa, v_scale, &at);
}

}  // namespace

extern "C" {

int gqa_attention_paged_decode_plan(const float* q, const void* k_pages, const void* v_pages,
                                    const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                                    const float* v_scale, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                    int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages, int kv_dtype,
                                    float scale, const gqa_av_plan* plan, void* stream) {
    return run_attention_paged(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale, out, B, C, Hq, Hkv, D,
                               page_size, max_pages, num_pages, kv_dtype, scale, plan, stream,
                               kRunPass1 | kRunCombine);
}

int gqa_attention_paged_decode_pass1(const float* q, const void* k_pages, const void* v_pages,
                                     const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                                     const float* v_scale, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
                                     int64_t D, int64_t page_size, int64_t max_pages, int64_t num_pages, int kv_dtype,
                                     float scale, const gqa_av_plan* plan, void* stream) {
    return run_attention_paged(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale, out, B, C, Hq, Hkv, D,
                               page_size, max_pages, num_pages, kv_dtype, scale, plan, stream, kRunPass1);
}

int gqa_attention_paged_decode_combine(const float* q, const void* k_pages, const void* v_pages,
                                       const int32_t* block_table, const int32_t* seq_lens, const float* k_scale,
                                       const float* v_scale, float* out, int64_t B, int64_t C, int64_t Hq,
                                       int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages,
                                       int64_t num_pages, int kv_dtype, float scale, const gqa_av_plan* plan,
                                       void* stream) {
    return run_attention_paged(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale, out, B, C, Hq, Hkv, D,
                               page_size, max_pages, num_pages, kv_dtype, scale, plan, stream, kRunCombine);
}

int gqa_attention_paged_decode(const float* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                               const int32_t* seq_lens, const float* k_scale, const float* v_scale, float* out,
                               int64_t B, int64_t C, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t max_pages, int64_t num_pages, int kv_dtype, float scale, int mode,
                               void* stream) {
    if (page_size < 1) return fail(GQA_AV_ERR_INVALID_ARG, "page_size must be >= 1");
    gqa_av_plan plan;
    int rc = auto_plan(v_pages, B, C, Hq, Hkv, D, kv_dtype, mode, 1, &plan, page_size, 1);
    if (rc != GQA_AV_OK) return rc;
    return gqa_attention_paged_decode_plan(q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale, out, B, C,
                                           Hq, Hkv, D, page_size, max_pages, num_pages, kv_dtype, scale, &plan,
                                           stream);
}

const char* gqa_av_status_string(int status) {
    switch (status) {
    case GQA_AV_OK: return "ok";
    case GQA_AV_ERR_INVALID_ARG: return "invalid argument";
    case GQA_AV_ERR_INELIGIBLE: return "shape not eligible for GQA reuse (group size < 2)";
    case GQA_AV_ERR_UNSUPPORTED: return "unsupported by this build";
    case GQA_AV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char* gqa_av_last_error(void) { return g_last_error.c_str(); }

int gqa_av_release(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int prev = 0;
    bool have_prev = hipGetDevice(&prev) == hipSuccess;
    int status = GQA_AV_OK;
    for (auto& kv : g_ws) {
        Workspace& ws = kv.second;
        if (!ws.counters && !ws.part) continue;
        hipError_t e = hipSetDevice(kv.first.first);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e == hipSuccess && ws.counters) e = hipFree(ws.counters);
        if (e == hipSuccess && ws.part) e = hipFree(ws.part);
        if (e != hipSuccess) status = fail(GQA_AV_ERR_HIP, "release: %s", hipGetErrorString(e));
        ws = Workspace();
    }
    g_ws.clear();
    if (have_prev) (void)hipSetDevice(prev);
    return status;
}

}  // extern "C"

// The decode score step shares this library's error, size and device helpers.
#include "qk_host.hpp"
