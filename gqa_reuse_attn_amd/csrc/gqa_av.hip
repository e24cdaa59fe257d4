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
#include "gqa_bench.h"
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
#include <vector>

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
// Eight KV heads per workgroup on the bf16 matrix engine (see the KV-tile
// choice below) only while every split keeps at least this many rows ...
constexpr int64_t kMinRowsPerSplitBf16Wide = 1024;
constexpr int64_t kMaxSplitsBf16Wide = 8;     // ... and the grid fills with at most this many splits
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

// Split-C workspace of one (device, stream): the buffer the split partials of
// the calls on that stream go to. A HIP graph captured from such a call keeps
// the buffer's address, so a buffer that has been handed out is never freed
// before gqa_av_release(): when a later call needs more, the old buffer is
// retired (kept) and a larger one takes its place.
struct Workspace {
    void* part = nullptr;
    size_t part_bytes = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<std::pair<int, void*>> g_ws_retired;   // (device, buffer), freed by gqa_av_release

// Per-device state lives in fixed tables (no host allocation on the call path).
constexpr int kMaxDevices = 64;

std::mutex g_cu_mutex;
int g_cu_count[kMaxDevices];   // 0: not asked yet

int device_cus(int dev, int* cus) {
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GQA_AV_ERR_UNSUPPORTED, "device %d: this library handles devices 0 .. %d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (g_cu_count[dev] > 0) {
        *cus = g_cu_count[dev];
        return GQA_AV_OK;
    }
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    g_cu_count[dev] = n;
    *cus = n;
    return GQA_AV_OK;
}

// Is `stream` being captured into a HIP graph?
int stream_capturing(hipStream_t stream, bool* capturing) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &st);
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
    *capturing = st != hipStreamCaptureStatusNone;
    return GQA_AV_OK;
}

// The split workspace of (dev, stream), at least `bytes` long. Growing it
// allocates (hipMalloc, rounded up to a power of two so that the retired
// buffers of a growing caller total less than the live one) and is refused
// while the stream is being captured: a graph must not record an allocation,
// and the call that first needs the space has to run outside the capture.
int get_workspace(int dev, hipStream_t stream, size_t bytes, float** part) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& ws = g_ws[{dev, stream}];
    if (ws.part_bytes < bytes) {
        bool capturing = false;
        int rc = stream_capturing(stream, &capturing);
        if (rc != GQA_AV_OK) return rc;
        if (capturing)
            return fail(GQA_AV_ERR_UNSUPPORTED,
                        "the split workspace of this stream must grow to %zu bytes, which cannot happen during "
                        "graph capture: make one call with this plan (or a larger one) on the stream before "
                        "capturing", bytes);
        size_t n = size_t{1} << 16;
        while (n < bytes) n <<= 1;
        void* p = nullptr;
        const hipError_t e = hipMalloc(&p, n);
        if (e != hipSuccess)
            return fail(GQA_AV_ERR_HIP, "hipMalloc(%zu) for the split-C workspace: %s", n, hipGetErrorString(e));
        if (ws.part) g_ws_retired.emplace_back(dev, ws.part);
        ws.part = p;
        ws.part_bytes = n;
    }
    *part = static_cast<float*>(ws.part);
    return GQA_AV_OK;
}

}  // namespace

// Split partials of gqa_av_decode_noalloc: a fixed device array instead of an
// allocated workspace. Host code never passes this name to a kernel or a copy
// (on the host it is only a stand-in); it uses the device address that
// hipGetSymbolAddress gives for the current device, kept per device below.
static __device__ __align__(256) uint8_t scratch[GQA_AV_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// The device address of `scratch` on device `dev`, which must be current:
// looked up once per device (hipGetSymbolAddress allocates nothing).
int scratch_address(int dev, float** p) {
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GQA_AV_ERR_UNSUPPORTED, "device %d: this library handles devices 0 .. %d", dev, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* q = nullptr;
        const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !q)
            return fail(GQA_AV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = q;
    }
    *p = static_cast<float*>(g_scratch_ptr[dev]);
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
        const int nset = p.heads_per_tile / 16, ht = p.kv_heads_per_tile, nw = p.threads / 64;
        using namespace gqa_av_launch;
        if (p.page_size > 0)
            return v_dtype == GQA_AV_FP8_E4M3 ? mfma_bf16<gqa_av::kFP8, true, true, true>(D, nset, ht, nw, a, s)
                                              : mfma_bf16<gqa_av::kBF16, true, true, true>(D, nset, ht, nw, a, s);
        return v_dtype == GQA_AV_FP8_E4M3 ? mfma_bf16<gqa_av::kFP8, true, false, true>(D, nset, ht, nw, a, s)
                                          : mfma_bf16<gqa_av::kBF16, true, false, true>(D, nset, ht, nw, a, s);
    }
    if (p.engine == GQA_AV_ENGINE_MFMA_BF16) {
        if (v_dtype != GQA_AV_BF16 && v_dtype != GQA_AV_FP8_E4M3) return hipErrorInvalidValue;
        const int nset = p.heads_per_tile / 16, ht = p.kv_heads_per_tile, nw = p.threads / 64;
        using namespace gqa_av_launch;
        if (p.page_size > 0) {
            if (v_dtype == GQA_AV_FP8_E4M3)
                return p.softmax ? mfma_bf16<gqa_av::kFP8, true, true>(D, nset, ht, nw, a, s)
                                 : mfma_bf16<gqa_av::kFP8, false, true>(D, nset, ht, nw, a, s);
            return p.softmax ? mfma_bf16<gqa_av::kBF16, true, true>(D, nset, ht, nw, a, s)
                             : mfma_bf16<gqa_av::kBF16, false, true>(D, nset, ht, nw, a, s);
        }
        if (v_dtype == GQA_AV_FP8_E4M3)
            return p.softmax ? mfma_bf16<gqa_av::kFP8, true>(D, nset, ht, nw, a, s)
                             : mfma_bf16<gqa_av::kFP8, false>(D, nset, ht, nw, a, s);
        return p.softmax ? mfma_bf16<gqa_av::kBF16, true>(D, nset, ht, nw, a, s)
                         : mfma_bf16<gqa_av::kBF16, false>(D, nset, ht, nw, a, s);
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

// Floats from the start of the split planes to the fused softmax's statistics
// (the planes rounded up to whole 16-byte groups).
int64_t stats_offset(int64_t nsplit, int64_t B, int64_t Hq, int64_t D) { return (nsplit * B * Hq * D + 3) / 4 * 4; }

// One fp32 plane of `out` per split, and for the fused softmax one (maximum,
// weight sum) pair per split and (b, q_h) after the planes.
int64_t workspace_bytes(int64_t B, int64_t Hq, int64_t D, int64_t nsplit, bool softmax) {
    if (nsplit <= 1) return 0;
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
    if (h.combine < GQA_AV_COMBINE_AUTO || h.combine > GQA_AV_COMBINE_KERNEL)
        return fail(GQA_AV_ERR_INVALID_ARG, "unknown combine %d", h.combine);
    if (h.softmax != 0 && h.softmax != 1) return fail(GQA_AV_ERR_INVALID_ARG, "hint softmax must be 0 or 1");
    if (h.attention != 0 && h.attention != 1) return fail(GQA_AV_ERR_INVALID_ARG, "hint attention must be 0 or 1");
    if (h.waves != 0 && h.waves != 4 && h.waves != 8)
        return fail(GQA_AV_ERR_INVALID_ARG, "hint waves must be 0 (automatic), 4 or 8");
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
    // bf16 V at G = 8 goes one step further, to eight heads (eight waves, a
    // wave per head: a workgroup streams whole rows), while the grid fills
    // with at most 8 splits of at least 1024 rows; D <= 128 for the plain
    // product, D = 128 for the fused softmax. Measured on MI355X (calls,
    // four heads -> eight), plain product, B = 64, C = 8192, Hkv = 8:
    // 177.4 -> 174.8 us; B = 48: 185.0 -> 180.3; B = 32: 93.5 -> 92.7;
    // Hkv = 16, B = 32: 184.2 -> 177.5; D = 64: 100.1 -> 98.6; B = 64,
    // C = 4096: 92.3 -> 91.7; B = 128, C = 4096 and B = 16, C = 16384 even;
    // fused softmax, B = 64: 179.7 -> 177.4; B = 48: 190.8 -> 183.9; B = 32:
    // 95.0 -> 93.6; Hkv = 16: 186.7 -> 180.7; D = 64: 97.2 -> 100.1. Other
    // head ratios lose with eight heads (G = 4: 166.3 -> 172.2, G = 5:
    // 166.1 -> 175.4, G = 6: 168.3 -> 180.2, G = 16: 101.7 -> 102.9 and
    // 56.4 -> 58.5), so do D = 256 (169.0 -> 196.0), fp8 V (the fused
    // softmax 116.4 -> 124.5) and grids that need 16 or more splits (B = 16,
    // C = 16384, fused softmax: 95.2 -> 95.8; B = 4, C = 32768: 50.1 -> 50.5,
    // 52.3 -> 53.1).
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
        for (int cand : {8, 4, 2}) {
            const bool eight = bf16_engine && !fp8 && !attention && G == 8 && (sm ? D == 128 : D <= 128) &&
                               (h.waves == 0 || h.waves == 8);
            const bool four = bf16_engine ? !fp8 : (fp8 && 4 * D * es <= 512);
            if ((cand == 8 && !eight) || (cand == 4 && !four) || Hkv % cand != 0) continue;
            const int64_t tiles_w = B * (Hkv / cand) * nsgw;
            if (cand == 8 && tiles_w * kMaxSplitsBf16Wide < target) continue;
            const int64_t rows_w = cand == 8 ? kMinRowsPerSplitBf16Wide : min_rows;
            if (lanes > 0 && (bf16_engine || cand * lanes <= gqa_av::kThreads) && v_align % 16 == 0 &&
                tiles_w > 0 &&
                tiles_w * std::min<int64_t>(ceil_div(target, tiles_w), std::max<int64_t>(1, C / rows_w)) >= target) {
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
        if (bf16_engine && ht != 2 && ht != 4 && !(ht == 8 && !attention))
            return fail(GQA_AV_ERR_UNSUPPORTED,
                        "the bf16 matrix engine takes 1, 2, 4 or 8 KV heads per tile (fused attention: up to 4)");
        if (sm && ht > 4 && !bf16_engine)
            return fail(GQA_AV_ERR_UNSUPPORTED, "the fused softmax on the VALU engine takes at most 4 KV heads per tile");
    }

    // Waves per workgroup: four, or eight on the bf16 matrix engine for the
    // plain product or eight KV heads per tile (more rows in flight per
    // workgroup without more splits).
    int nw = gqa_av::kWaves;
    // Automatic: eight waves on the bf16 matrix engine when a workgroup
    // streams one KV head of the plain product, or eight KV heads (set below,
    // once the KV heads per tile are known).
    if (h.waves > 0 && h.waves != nw) {
        if (!bf16_engine || (sm && ht != 8))
            return fail(GQA_AV_ERR_UNSUPPORTED, "%d waves per workgroup: only the bf16 matrix engine takes eight, "
                        "for the plain product or eight KV heads per tile", h.waves);
        nw = h.waves;
    }

    int VB, GT, nsg;
    int64_t Lc, rps, ndt, rows_per_step;
    int64_t heads_major;  // tiles along the head axis per KV head
    if (engine == GQA_AV_ENGINE_MFMA_BF16) {
        // Eight waves when one KV head per workgroup (plain product): more
        // rows in flight per CU without more splits. Measured on MI355X,
        // B = 4, C = 32768, Hq = 16, Hkv = 1: pass 1 10.4 -> 9.9 us; with four
        // KV heads per workgroup (B = 64, C = 8192, Hq = 64, Hkv = 8) eight
        // waves were slower (176 -> 190 us). Eight KV heads take eight waves,
        // one per head.
        if (h.waves == 0 && ((ht == 1 && !sm) || ht == 8)) nw = 8;
        if (ht == 8 && nw != 8)
            return fail(GQA_AV_ERR_UNSUPPORTED, "eight KV heads per tile take eight waves (a wave per KV head)");
        VB = v_dtype == GQA_AV_FP8_E4M3 ? 8 : 16;    // one 8-value piece per lane load
        GT = 16 * nset16;
        nsg = static_cast<int>(ceil_div(G, GT));
        heads_major = nsg;
        Lc = ht * D / 8;                // 16-byte pieces of a tile row
        rps = 32 * nw / ht;             // one 32-row chunk per wave, nw / ht waves per KV head
        ndt = 1;
        rows_per_step = rps * GQA_AV_MFMA_BF16_CHUNKS;
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
        rows_per_step = rps * gqa_av::valu_unroll(static_cast<int>(GT), v_dtype, h.softmax == 1, paged);
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
    // Interleaved splits (dense V on the VALU and bf16 matrix engines): split
    // s takes the pipeline steps s, s + nsplit, ... of the whole sequence, so
    // the splits of a tile, which run side by side, stream neighbouring rows.
    // The buffer resources then span the whole sequence: its rows, plus the
    // pipeline's reloads up to two steps of every split past the end, must
    // stay under 1 GB for 32-bit offsets.
    bool interleave = false;
    if (h.split_order < 0 || h.split_order > 2)
        return fail(GQA_AV_ERR_INVALID_ARG, "hint split_order must be 0 (automatic), 1 (contiguous) or 2 (interleaved)");
    if (h.split_order != 1 && C > 0 && nsplit > 1) {
        const int64_t row_bytes = std::max<int64_t>(Hkv * D * es, Hq * 4);
        const bool can = !paged && !attention && engine != GQA_AV_ENGINE_MFMA &&
                         (C + 3 * nsplit * rows_per_step) * row_bytes < (int64_t{1} << 30);
        if (h.split_order == 2 && !can)
            return fail(GQA_AV_ERR_UNSUPPORTED, "interleaved splits need dense V on the VALU or bf16 matrix engine "
                        "(not fused attention) and a sequence under 1 GB of V");
        // Automatic: interleaved for the plain product (measured on MI355X),
        // contiguous for the fused softmax and fused attention.
        interleave = can && (h.split_order == 2 || !sm);
    }
    if (interleave) {
        rows_per_split = rows_per_step;            // one block per step
        nsplit = std::min(nsplit, ceil_div(C, rows_per_step));
        interleave = nsplit > 1;
        if (!interleave) rows_per_split = C;
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
    plan->threads = 64 * nw;
    plan->rows_per_split = rows_per_split;
    plan->interleave = interleave ? 1 : 0;
    plan->grid = grid;
    // Split partials are added by a second kernel.
    plan->combine = nsplit > 1 ? GQA_AV_COMBINE_KERNEL : GQA_AV_COMBINE_AUTO;
    plan->kv_heads_per_tile = ht;
    plan->workspace_bytes = workspace_bytes(B, Hq, D, nsplit, sm);
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
           a.softmax == b.softmax && a.page_size == b.page_size && a.attention == b.attention &&
           a.interleave == b.interleave;
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
// no_alloc: the split partials go to the fixed `scratch` array instead of the
// stream's workspace (gqa_av_decode_noalloc).
int run_plan(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t Hq, int64_t Hkv,
             int64_t D, int v_dtype, const gqa_av_plan* plan, void* stream, int which, int softmax,
             const PagedArgs* pg = nullptr, const float* v_scale = nullptr, const AttnArgs* at = nullptr,
             bool no_alloc = false, int64_t v_seq_rows = -1) {
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
    h.waves = plan->threads / 64;
    h.split_order = plan->interleave ? 2 : 1;
    gqa_av_plan check;
    const int mode = plan->mode;
    // Re-plan with the split count fixed: rows_per_split then follows from C.
    rc = plan_impl(B, C, Hq, Hkv, D, v_dtype, mode, &h, kDefaultCUs, &check);
    if (rc != GQA_AV_OK) return rc;
    if (plan->interleave && check.rows_per_split != plan->rows_per_split)
        return fail(GQA_AV_ERR_INVALID_ARG, "an interleaved plan's blocks must be one pipeline step of %lld rows",
                    (long long)check.rows_per_split);
    check.rows_per_split = plan->rows_per_split;
    check.nsplit = plan->nsplit;
    check.grid = plan->grid;
    check.workspace_bytes = plan->workspace_bytes;
    check.combine = plan->combine;
    if (!same_plan(check, *plan)) return fail(GQA_AV_ERR_INVALID_ARG, "plan does not belong to this problem");
    if (plan->nsplit > 1 ? plan->combine != GQA_AV_COMBINE_KERNEL : plan->combine != GQA_AV_COMBINE_AUTO)
        return fail(GQA_AV_ERR_INVALID_ARG, "plan combine %d does not fit nsplit %d", plan->combine, plan->nsplit);
    // The split fields must still tile [0, C) exactly: contiguous splits of
    // rows_per_split rows, or (interleaved) blocks of one pipeline step, at
    // least one per split.
    if (C > 0) {
        if (plan->interleave != 0 && plan->interleave != 1)
            return fail(GQA_AV_ERR_INVALID_ARG, "plan interleave must be 0 or 1");
        if (plan->nsplit < 1 || plan->rows_per_split < 1 ||
            (plan->interleave ? plan->nsplit > ceil_div(C, plan->rows_per_split) || plan->nsplit < 2
                              : ceil_div(C, plan->rows_per_split) != plan->nsplit))
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
    if (plan->workspace_bytes != workspace_bytes(B, Hq, D, plan->nsplit, plan->softmax == 1))
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
    if (plan->nsplit > 1) {
        if (no_alloc) {
            if (plan->workspace_bytes > static_cast<int64_t>(GQA_AV_NOALLOC_SCRATCH_BYTES))
                return fail(GQA_AV_ERR_UNSUPPORTED,
                            "the plan needs %lld bytes of split partials; the allocation-free entry point has a "
                            "fixed %d-byte scratch array (use gqa_av_decode)",
                            (long long)plan->workspace_bytes, GQA_AV_NOALLOC_SCRATCH_BYTES);
            rc = scratch_address(dev, &part);
        } else {
            rc = get_workspace(dev, s, static_cast<size_t>(plan->workspace_bytes), &part);
        }
        if (rc != GQA_AV_OK) return rc;
    }

    Pass1Args a;
    a.attn = attn;
    a.V = static_cast<const uint8_t*>(V);
    a.out = out;
    a.part = part;
    a.stats = (softmax && plan->nsplit > 1) ? part + stats_offset(plan->nsplit, B, Hq, D) : nullptr;
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
    a.C = C;
    a.v_seq_rows = v_seq_rows < 0 ? C : v_seq_rows;
    a.rows_per_split = plan->rows_per_split;
    a.interleave = plan->interleave;
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
    } else if ((which & kRunCombine) && plan->nsplit > 1) {
        const int64_t plane = B * Hq * D;
        const int groups = gqa_av::combine_groups(a.nsplit, plane);
        const int64_t per_block = 4 * (gqa_av::kThreads / groups);
        const int64_t blocks = ceil_div(plane, per_block);
        if (blocks > INT32_MAX) return fail(GQA_AV_ERR_UNSUPPORTED, "output too large for the split-C combine");
        const dim3 grid(static_cast<uint32_t>(blocks)), block(gqa_av::kThreads);
        const float* const pp = part;
        switch (groups) {
        case 1: hipLaunchKernelGGL(gqa_av::av_pass2_combine<1>, grid, block, 0, s, pp, out, plane, a.nsplit); break;
        case 2: hipLaunchKernelGGL(gqa_av::av_pass2_combine<2>, grid, block, 0, s, pp, out, plane, a.nsplit); break;
        case 4: hipLaunchKernelGGL(gqa_av::av_pass2_combine<4>, grid, block, 0, s, pp, out, plane, a.nsplit); break;
        case 8: hipLaunchKernelGGL(gqa_av::av_pass2_combine<8>, grid, block, 0, s, pp, out, plane, a.nsplit); break;
        case 16: hipLaunchKernelGGL(gqa_av::av_pass2_combine<16>, grid, block, 0, s, pp, out, plane, a.nsplit); break;
        case 32: hipLaunchKernelGGL(gqa_av::av_pass2_combine<32>, grid, block, 0, s, pp, out, plane, a.nsplit); break;
        default: hipLaunchKernelGGL(gqa_av::av_pass2_combine<64>, grid, block, 0, s, pp, out, plane, a.nsplit); break;
        }
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

int gqa_av_decode_noalloc(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t Hq,
                          int64_t Hkv, int64_t D, int v_dtype, int mode, void* stream) {
    gqa_av_plan plan;
    int rc = auto_plan(V, B, C, Hq, Hkv, D, v_dtype, mode, 0, &plan);
    if (rc != GQA_AV_OK) return rc;
    return run_plan(attn, V, out, B, C, Hq, Hkv, D, v_dtype, &plan, stream, kRunPass1 | kRunCombine, 0, nullptr,
                    nullptr, nullptr, true);
}

}  // extern "C"

namespace {

int check_capacity(int64_t B, int64_t C, int64_t C_max, int64_t Hq, int64_t Hkv, int64_t D, int v_dtype) {
    int rc = check_sizes(B, C, Hq, Hkv, D, v_dtype);
    if (rc != GQA_AV_OK) return rc;
    if (C_max < C) return fail(GQA_AV_ERR_INVALID_ARG, "capacity C_max=%lld is below C=%lld", (long long)C_max,
                               (long long)C);
    if (C_max > INT64_MAX / (Hkv * D * elem_bytes(v_dtype)) / (B > 0 ? B : 1))
        return fail(GQA_AV_ERR_INVALID_ARG, "B * C_max rows of V overflow 64-bit offsets");
    return GQA_AV_OK;
}

}  // namespace

extern "C" {

int gqa_av_decode_strided_plan(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t C_max,
                               int64_t Hq, int64_t Hkv, int64_t D, int v_dtype, const gqa_av_plan* plan,
                               void* stream) {
    int rc = check_capacity(B, C, C_max, Hq, Hkv, D, v_dtype);
    if (rc != GQA_AV_OK) return rc;
    return run_plan(attn, V, out, B, C, Hq, Hkv, D, v_dtype, plan, stream, kRunPass1 | kRunCombine, 0, nullptr,
                    nullptr, nullptr, false, C_max);
}

int gqa_av_decode_strided(const float* attn, const void* V, float* out, int64_t B, int64_t C, int64_t C_max,
                          int64_t Hq, int64_t Hkv, int64_t D, int v_dtype, int mode, void* stream) {
    int rc = check_capacity(B, C, C_max, Hq, Hkv, D, v_dtype);
    if (rc != GQA_AV_OK) return rc;
    gqa_av_plan plan;
    rc = auto_plan(V, B, C, Hq, Hkv, D, v_dtype, mode, 0, &plan);
    if (rc != GQA_AV_OK) return rc;
    return gqa_av_decode_strided_plan(attn, V, out, B, C, C_max, Hq, Hkv, D, v_dtype, &plan, stream);
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

int gqa_bench_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t loads_in_flight,
                          int32_t pattern, uint32_t* sink, void* stream) {
    if (pattern != 0 && pattern != 1) return fail(GQA_AV_ERR_INVALID_ARG, "pattern must be 0 or 1");
    if (!src || !sink) return fail(GQA_AV_ERR_INVALID_ARG, "src and sink must not be NULL");
    if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return fail(GQA_AV_ERR_INVALID_ARG, "src must be 16-byte and sink 4-byte aligned");
    if (bytes <= 0 || bytes % 16 != 0) return fail(GQA_AV_ERR_INVALID_ARG, "bytes must be > 0 and a multiple of 16");
    if (workgroups < 1) return fail(GQA_AV_ERR_INVALID_ARG, "workgroups must be >= 1");
    if (loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16)
        return fail(GQA_AV_ERR_INVALID_ARG, "loads_in_flight must be 4, 8 or 16");
    const int64_t slice = ceil_div(ceil_div(bytes, workgroups), 16) * 16;
    if (slice > INT32_MAX) return fail(GQA_AV_ERR_INVALID_ARG, "a slice of %lld bytes exceeds 2^31", (long long)slice);
    const hipError_t e = gqa_av_launch::stream_read(pattern, static_cast<const uint8_t*>(src), bytes, slice,
                                                    workgroups, loads_in_flight, sink,
                                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GQA_AV_ERR_HIP, "stream read launch: %s", hipGetErrorString(e));
    return GQA_AV_OK;
}

int gqa_av_release(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int prev = 0;
    bool have_prev = hipGetDevice(&prev) == hipSuccess;
    int status = GQA_AV_OK;
    // Every buffer ever handed out, live or retired, per device.
    std::vector<std::pair<int, void*>> bufs = g_ws_retired;
    for (auto& kv : g_ws)
        if (kv.second.part) bufs.emplace_back(kv.first.first, kv.second.part);
    std::sort(bufs.begin(), bufs.end());
    int synced = -1;
    for (auto& db : bufs) {
        hipError_t e = hipSuccess;
        if (db.first != synced) {
            e = hipSetDevice(db.first);
            if (e == hipSuccess) e = hipDeviceSynchronize();
            synced = db.first;
        }
        if (e == hipSuccess) e = hipFree(db.second);
        if (e != hipSuccess) status = fail(GQA_AV_ERR_HIP, "release: %s", hipGetErrorString(e));
    }
    g_ws.clear();
    g_ws_retired.clear();
    if (have_prev) (void)hipSetDevice(prev);
    return status;
}

}  // extern "C"

// The decode score step shares this library's error, size and device helpers.
#include "qk_host.hpp"
