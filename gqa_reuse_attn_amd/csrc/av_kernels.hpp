// Device code of the GQA decode attention-times-V path for gfx950 (MI355X).
//
// Operation (ExecuTorch PR #21063, "...GEMV", introduction), batch index added:
//   out[b, q_h, d] = sum_c attn[b, c, q_h] * V[b, c, kv_h, d],  kv_h = q_h / G.
// The page's GQA-reuse variant gives one workgroup a whole KV head and makes
// it produce the G outputs of that head's group from one read of each V row;
// its per-query-head shader (kept here as the baseline) reads V once per head.
//
// A workgroup owns a tile = (b, kv_h, head sub-group, D-tile) -- or
// (b, q_h, D-tile) for the per-head baseline -- and one context split
// [cb, ce). It streams the tile's V rows of that split once and keeps fp32
// accumulators for every query head of the tile. Without a context split it
// writes `out` directly. With one, it writes its split's partial sums to a
// plane of the workspace and a second kernel adds the planes in a fixed
// order (the kernel boundary orders them), so a plan is bitwise
// reproducible.
//
// Two inner-product engines, both fp32 FMA arithmetic:
//  * VALU  -- any G and D. Lc lanes cover a D-row with VB-byte loads (one
//             16-byte global_load_dwordx4 each when D allows); rps row slots
//             load different rows side by side. Each lane widens its V chunk
//             once and applies it to the GT query heads of the tile, whose
//             weights are staged in LDS per stage of rps * U rows
//             (double-buffered) and read as broadcasts. Row slots are summed
//             through LDS at the end.
//  * MFMA  -- G >= 5: the group's weights form a 16 x 4 A operand and four V
//             rows a 4 x 16 B operand of v_mfma_f32_16x16x4_f32, so the matrix
//             core does the G-fold reuse and the sum over four rows at once.
//             Lane 16k + n loads row k's D-chunk n (D/16 elements) and the
//             weight of head n of row k; nothing goes through LDS until the
//             four waves' tiles are added at the end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gqa_av {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies, one L2 each
constexpr int kMaxRowSlots = 64;  // rows a VALU workgroup loads side by side, at most
constexpr int kMaxSplitPages = 1024;  // paged V: pages one context split may touch (its page list sits in LDS)

// Tuning constants (compile-time; -D overrides build variants for sweeps).
#ifndef GQA_AV_VALU_UNROLL
#define GQA_AV_VALU_UNROLL 4      // rows per lane per iteration, groups of up to 4 heads (see valu_unroll;
                                  // 4 measured best on MI355X for 2 and 4 heads: 6 and 8 cost 0.5-1 us at G = 2)
#endif
#ifndef GQA_AV_MFMA_UNROLL
#define GQA_AV_MFMA_UNROLL 4      // row groups of four per wave and step (16-byte lanes)
#endif
#ifndef GQA_AV_MFMA_BF16_CHUNKS
#define GQA_AV_MFMA_BF16_CHUNKS 1 // bf16 matrix engine: 32-row chunks per wave and buffer (two buffers)
#endif
constexpr int mfma_unroll(int NB) { return NB > 16 ? (GQA_AV_MFMA_UNROLL + 1) / 2 : GQA_AV_MFMA_UNROLL; }

enum : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };   // kFP8: OCP FP8 E4M3 (V only)

// Rows per lane and step of the VALU engine for GT heads per tile, element
// type DT, fused softmax SM, paged V PG (the planner's step and the kernel's
// template argument both come from here). Tiles of three heads over dense
// fp16 V take twice the rows: measured on MI355X (B = 8, C = 16384, Hkv = 8,
// G = 3, D = 96), pass 1 33.7-33.8 us against 34.05-34.08 with four, while
// the paged, fp8 and fused softmax products of that shape lost 1-1.6 us.
constexpr int valu_unroll(int GT, int DT, bool SM, bool PG) {
    return GT == 3 && DT == kF16 && !SM && !PG ? 2 * GQA_AV_VALU_UNROLL
           : GT <= 4                           ? GQA_AV_VALU_UNROLL
           : GT <= 8                           ? (GQA_AV_VALU_UNROLL + 1) / 2
                                               : (GQA_AV_VALU_UNROLL + 3) / 4;
}

// Fused softmax: a weight is exp2((s - r) * log2(e)) for a running maximum r of
// the scores. The difference is taken first (exact when s and r are within a
// factor of two), so the weight's error grows with s - r, not with s. exp2 is
// the hardware's v_exp_f32 (about 1 ulp), whose results below 2^-126 may be
// flushed to zero: a weight that small beside the maximum's 1 changes no fp32
// result.
constexpr float kLog2e = 1.4426950408889634f;

template <int DT>
constexpr int esize() { return DT == kF32 ? 4 : (DT == kFP8 ? 1 : 2); }

// Workgroups are handed to the XCDs round-robin (block i -> XCD i % 8). Remap
// so that each XCD walks a contiguous range of logical tiles: the KV heads of
// one (b, split) -- which share the cache lines of their attn rows -- then run
// on one XCD at about the same time and share its L2.
__device__ inline uint32_t xcd_remap(uint32_t i, uint32_t n) {
    const uint32_t per = n / kXcds, rem = n % kXcds;
    const uint32_t x = i % kXcds, k = i / kXcds;
    return x < rem ? x * (per + 1) + k : rem * (per + 1) + (x - rem) * per + k;
}

struct Pass1Args {
    const float* attn;      // [B][C][Hq]
    const uint8_t* V;       // [B][C][Hkv][D] of DT
    float* out;             // [B][Hq][D]
    float* part;            // nsplit > 1: [nsplit][B][Hq][D] partial sums
    float* stats;           // fused softmax with nsplit > 1: [nsplit][B][Hq] pairs (maximum score, weight sum),
                            // 16-byte aligned
    const int32_t* block_table;  // paged V: [B][max_pages], the page of each page-long run of a sequence's rows
    const int32_t* seq_lens;     // paged V: [B] rows of each sequence (clamped into [0, C])
    int64_t num_pages;           // paged V: pages in the cache (block-table entries are clamped into range)
    int32_t page_shift;          // paged V: log2 of the rows per page
    int32_t max_pages;           // paged V: length of a block-table row
    const float* v_scale;        // fp8 V: [Hkv] scale of each KV head's values (NULL: 1)
    const float* q;              // fused attention: [B][Hq][D] queries (the scores are computed, not read)
    const uint8_t* K;            // fused attention: [B][C][Hkv][D] keys, V's element type
    float qk_scale;              // fused attention: the scores are qk_scale * q . K
    const float* k_scale;        // fused attention over fp8 K: [Hkv] scale of each KV head's keys (NULL: 1)
    int64_t C;
    int64_t v_seq_rows;      // rows of V from one sequence to the next (C, or a larger capacity)
    int64_t rows_per_split;  // contiguous splits: rows of each; interleaved: rows of one block (a pipeline step)
    int32_t interleave;      // 1: split s takes the blocks s, s + nsplit, s + 2 nsplit, ... of the sequence
    int32_t B, Hq, Hkv, D;
    int32_t G;              // Hq / Hkv
    int32_t per_head;       // 0: reuse tiles, 1: one query head per tile
    int32_t nsg;            // head sub-groups per KV head (reuse)
    int32_t ndt;            // D-tiles (VALU)
    int32_t nsplit;
    int32_t L;              // VALU: lanes per full D-row of one KV head
    int32_t ht;             // VALU: adjacent KV heads per tile (their D-rows are contiguous)
    int32_t Lc;             // VALU: lanes per tile row inside a workgroup (<= 256; ht * L when ht > 1)
    int32_t rps;            // VALU: row slots = min(256 / Lc, kMaxRowSlots)
    uint32_t nblocks;
};

// ---- V loads and conversion -------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Buffer-resource word 3 for raw (untyped) buffer access on gfx9-family parts.
constexpr int kRawBufferFlags = 0x00020000;
constexpr int kCachePolicySc1 = 16;   // device-scope coherence (same policy as agent-scope atomics)
constexpr int kCachePolicyNt = 2;     // non-temporal (streamed once)
// A buffer offset past every resource the kernels build (their ranges stay
// below 2^30 bytes and their scalar offsets add less than 2^30): an access
// there fails the range check, so a load reads zero and a store is dropped.
constexpr int kOutOfRange = 0x40000000;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));

template <int NB>
struct Raw {
    uint32_t w[NB >= 4 ? NB / 4 : 1];
};

// Load NB bytes (2, 4, 8, 12, 16 or 32) from p, which is NB-aligned (12: 4-aligned).
// V is read exactly once per call, so the loads carry the non-temporal cache
// policy: on MI355X this streams at about 7 TB/s against about 6.1 TB/s for
// default-policy loads of the same pattern.
template <int NB>
__device__ inline Raw<NB> load_raw(const uint8_t* p) {
    Raw<NB> r;
    if constexpr (NB == 32) {
        const u32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const u32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
        r.w[0] = v0.x; r.w[1] = v0.y; r.w[2] = v0.z; r.w[3] = v0.w;
        r.w[4] = v1.x; r.w[5] = v1.y; r.w[6] = v1.z; r.w[7] = v1.w;
    } else if constexpr (NB == 16) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (NB == 12) {
        const u32x3 v = __builtin_nontemporal_load(reinterpret_cast<const u32x3*>(p));
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z;
    } else if constexpr (NB == 8) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        r.w[0] = v.x; r.w[1] = v.y;
    } else if constexpr (NB == 4) {
        r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else {
        r.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
    }
    return r;
}

// Buffer-resource forms: NB bytes (2, 4, 8 or 16) at voffset + soffset of
// the resource, non-temporal; zero when the range check of the resource fails.
template <int NB>
__device__ inline Raw<NB> load_raw_buf(__amdgpu_buffer_rsrc_t rs, int voffset, int soffset) {
    Raw<NB> r;
    if constexpr (NB == 16) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, soffset, kCachePolicyNt);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (NB == 8) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, voffset, soffset, kCachePolicyNt);
        r.w[0] = v.x; r.w[1] = v.y;
    } else if constexpr (NB == 4) {
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voffset, soffset, kCachePolicyNt);
    } else {
        static_assert(NB == 2, "lane loads are 2, 4, 8 or 16 bytes");
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, voffset, soffset, kCachePolicyNt);
    }
    return r;
}

// N consecutive floats at voffset + soffset of the resource (4-byte aligned),
// in loads of up to 16 bytes.
template <int N>
__device__ inline void load_floats(__amdgpu_buffer_rsrc_t rs, int voffset, int soffset, float* out) {
    int k = 0;
#pragma unroll
    for (; k + 4 <= N; k += 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voffset + 4 * k, soffset, 0);
        out[k] = __uint_as_float(v.x); out[k + 1] = __uint_as_float(v.y);
        out[k + 2] = __uint_as_float(v.z); out[k + 3] = __uint_as_float(v.w);
    }
    if constexpr (N % 4 == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rs, voffset + 4 * k, soffset, 0);
        out[k] = __uint_as_float(v.x); out[k + 1] = __uint_as_float(v.y); out[k + 2] = __uint_as_float(v.z);
    } else if constexpr (N % 4 == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, voffset + 4 * k, soffset, 0);
        out[k] = __uint_as_float(v.x); out[k + 1] = __uint_as_float(v.y);
    } else if constexpr (N % 4 == 1) {
        out[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, voffset + 4 * k, soffset, 0));
    }
}

// Exact split of an fp32 value w into three bfloat16 terms by truncation:
// th = trunc(w), tm = trunc(w - th), tl = w - th - tm. Both subtractions are
// exact (Sterbenz) and tl has at most 8 significant bits, so th + tm + tl = w
// for every normal w down to 2^-103. Returned as fp32 bit patterns whose low
// 16 bits are zero (the upper halves are the bfloat16 encodings).
__device__ inline void split_bf16x3(float w, uint32_t& th, uint32_t& tm, uint32_t& tl) {
    th = __float_as_uint(w) & 0xffff0000u;
    const float r1 = w - __uint_as_float(th);
    tm = __float_as_uint(r1) & 0xffff0000u;
    tl = __float_as_uint(r1 - __uint_as_float(tm)) & 0xffff0000u;
}

__device__ inline float f16_bits_to_f32(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Widen the NB / esize elements of one lane-load to fp32 (exact for all three types).
template <int DT, int NB>
__device__ inline void widen(const Raw<NB>& r, float* f) {
    if constexpr (DT == kFP8) {
        // v_cvt_pk_f32_fp8 decodes two OCP E4M3 bytes exactly on gfx950 (all 256
        // patterns checked on MI355X against the format's definition).
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        static_assert(NB == 2 || NB % 4 == 0, "fp8 lane loads are 2, 4 or 8 bytes");
        if constexpr (NB == 2) {
            const f32x2 p = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[0]), false);
            f[0] = p.x;
            f[1] = p.y;
        } else {
#pragma unroll
            for (int i = 0; i < NB / 4; ++i) {
                const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[i]), false);
                const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.w[i]), true);
                f[4 * i] = lo.x;
                f[4 * i + 1] = lo.y;
                f[4 * i + 2] = hi.x;
                f[4 * i + 3] = hi.y;
            }
        }
    } else if constexpr (DT == kF32) {
#pragma unroll
        for (int i = 0; i < NB / 4; ++i) f[i] = __uint_as_float(r.w[i]);
    } else if constexpr (NB == 2) {
        f[0] = DT == kBF16 ? __uint_as_float(r.w[0] << 16) : f16_bits_to_f32(r.w[0]);
    } else if constexpr (DT == kBF16) {
#pragma unroll
        for (int i = 0; i < NB / 4; ++i) {
            f[2 * i] = __uint_as_float(r.w[i] << 16);
            f[2 * i + 1] = __uint_as_float(r.w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NB / 4; ++i) {
            f[2 * i] = f16_bits_to_f32(r.w[i] & 0xffffu);
            f[2 * i + 1] = f16_bits_to_f32(r.w[i] >> 16);
        }
    }
}

// A value that is the same in every lane, moved to scalar registers.
__device__ inline int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// ---- tile decode ------------------------------------------------------------

struct Tile {
    int b, kv, s, dt, q_first, nq;
};

// Logical order, fastest first: (sub-group, D-tile), kv_h, split, b, and for
// the per-head baseline the head's position g inside its group slowest, so the
// G re-reads of one V row are far apart in time and not merged by the caches.
__device__ inline Tile decode_tile(const Pass1Args& a, int GT) {
    uint32_t t = xcd_remap(blockIdx.x, a.nblocks);
    Tile T;
    const uint32_t nminor = a.per_head ? a.ndt : a.nsg * a.ndt;
    const uint32_t nkvt = a.Hkv / a.ht;              // tiles along the KV heads
    const uint32_t minor = t % nminor; t /= nminor;
    const uint32_t kvt = t % nkvt; t /= nkvt;
    T.kv = kvt * a.ht;                               // first KV head of the tile
    T.s = t % a.nsplit; t /= a.nsplit;
    T.b = t % a.B; t /= a.B;
    const uint32_t major = t;
    if (a.per_head) {
        T.dt = minor;
        T.q_first = T.kv * a.G + major;
        T.nq = 1;
    } else {
        const int sg = minor / a.ndt;
        T.dt = minor % a.ndt;
        T.q_first = T.kv * a.G + sg * GT;
        T.nq = min(GT, a.G - sg * GT);
    }
    return T;
}

// ---- split partials ---------------------------------------------------------

// The fused softmax's second-kernel combine adds split partials as
// kSplitGroups contiguous ranges of splits (see av_pass2_softmax_combine).
constexpr int kSplitGroups = 8;

// ---- pass 1: VALU engine ----------------------------------------------------

// SM: fused softmax. attn then holds raw scores s; a lane's weight for a row is
// exp2((s - mx) log2 e) with mx the running maximum of the scores the lane has
// seen (per head). When a step raises mx, the lane's accumulators and weight
// sum are multiplied by exp2((old - new) log2 e) (skipped when no lane of the
// wave saw a new maximum). At the end of the split the row slots are brought
// to the workgroup's maximum before they are summed; the split's result is the
// weighted sum divided by the weight sum, or, with several splits, the
// unnormalised sum with its (maximum, weight sum) for the combine.
//
// PG: paged V. Sequence b has seq_lens[b] rows; row c is row c % P of page
// block_table[b][c / P] (P = 2^page_shift rows of Hkv * D values). The
// workgroup copies the block-table entries its split touches into LDS once
// (clamped into the cache), and each lane computes its rows' addresses from
// them; rows past the sequence's length take weight 0 (and read the split's
// last valid row). The weights keep the dense [B][C][Hq] layout, C being the
// capacity. Needs 16-byte lane loads.
template <int DT, int VB, int GT, int U, bool SM = false, bool PG = false>
__global__ __launch_bounds__(kThreads) void av_pass1_valu(Pass1Args a) {
    static_assert(!PG || VB == 16, "paged V takes 16-byte lane loads");
    constexpr int ES = esize<DT>();
    constexpr int E = VB / ES;
    constexpr int NACC = GT * E;
    constexpr int CH = NACC < 32 ? NACC : 32;       // accumulator slots per LDS reduction pass
    constexpr int RED = CH * kThreads;
    __shared__ __align__(16) float smem[RED];

    const Tile T = decode_tile(a, GT);
    const int tid = threadIdx.x;
    const int Lc = a.Lc, rps = a.rps;
    const int r = tid / Lc;
    const int j = tid - r * Lc;
    const int kvl = j / a.L;                         // which KV head of the tile (0 when ht == 1)
    const int lane_d = T.dt * Lc + (j - kvl * a.L);  // which VB-chunk of that head's D-row
    const bool active = (r < rps) && (lane_d < a.L);

    // Rows of the split: contiguous, [cb, ce); or interleaved (dense V), the
    // blocks of R rows s, s + nsplit, s + 2 nsplit, ... of the whole sequence
    // (then cb = 0 and ce = C), so the splits of a tile, which run at the same
    // time, stream neighbouring rows (a plain read over such blocks runs a few
    // per cent faster on MI355X than one contiguous slice per workgroup).
    const bool il = !PG && a.interleave;
    const int64_t cb = il ? 0 : static_cast<int64_t>(T.s) * a.rows_per_split;
    int64_t ce_ = il ? a.C : min(a.C, cb + a.rows_per_split);
    if constexpr (PG) {
        const int64_t len = a.seq_lens[T.b];
        ce_ = min(ce_, len < 0 ? int64_t{0} : min(len, a.C));
    }
    const int64_t ce = ce_;
    const int64_t nrows_split = ce > cb ? ce - cb : 0;
    const int R = rps * U;                           // rows per stage

    const size_t vrow = static_cast<size_t>(a.Hkv) * a.D * ES;   // bytes from row c to c+1

    float acc[GT][E];
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = 0.0f;
    float mx[GT], lsum[GT];                          // SM: running maximum score and weight sum
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        mx[g] = -INFINITY;
        lsum[g] = 0.0f;
    }
    __shared__ float s_stat[2][4 * GT];              // SM: the workgroup's maximum and weight sum per head

    // The tile's weights are read as a window of GT consecutive heads starting at
    // q_lo, shifted down when the tile's last sub-group is short, so every lane
    // loads GT words at constant offsets and the window never leaves the attn
    // row (the planner keeps GT <= Hq). Accumulators outside the tile's own
    // heads are computed and dropped.
    // With ht > 1 every lane uses the window of its own KV head kv + kvl.
    auto lane_q_lo = [&](int kl) { return min(T.q_first + kl * a.G, a.Hq - GT); };
    const int q_lo = lane_q_lo(kvl);
    // V and attn are read through buffer resources that end with the split's
    // last row: rows at or past ce read as zero (and add nothing), so every
    // step is a full one, and a row's address is a per-lane constant plus a
    // workgroup-uniform offset held in a scalar register. The plan keeps a
    // split's span under 1 GB so 32-bit offsets suffice.
    const int nrows = static_cast<int>(uniform64(nrows_split));
    const int vrow32 = static_cast<int>(vrow);
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.V) + ((static_cast<size_t>(T.b) * a.v_seq_rows + cb) * a.Hkv + T.kv) * a.D * ES, 0,
        nrows > 0 ? (nrows - 1) * vrow32 + a.ht * a.D * ES : 0, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.attn) + (static_cast<size_t>(T.b) * a.C + cb) * a.Hq, 0, nrows * a.Hq * 4,
        kRawBufferFlags);
    const int voff = r * vrow32 + (kvl * a.D * ES + lane_d * VB);
    const int woff = (r * a.Hq + q_lo) * 4;
    const int nblk = (nrows + R - 1) / R;           // blocks of R rows in [cb, ce)
    const int nsteps = il ? (nblk > T.s ? (nblk - T.s + a.nsplit - 1) / a.nsplit : 0) : nblk;
    // First row (from cb) of this workgroup's step st.
    auto step_row = [&](int st) { return (il ? st * a.nsplit + T.s : st) * R; };
    // PG: the split's pages, from the block table into LDS.
    __shared__ int32_t s_pages[PG ? kMaxSplitPages : 1];
    const int64_t pg0 = PG ? (cb >> a.page_shift) : 0;
    if constexpr (PG) {
        const int npg = nrows > 0 ? static_cast<int>(((cb + nrows - 1) >> a.page_shift) - pg0 + 1) : 0;
        const int32_t* const btr = a.block_table + static_cast<size_t>(T.b) * a.max_pages + pg0;
        for (int i = tid; i < npg; i += kThreads) {
            const int32_t pg = btr[i];
            s_pages[i] = pg < 0 ? 0 : (pg >= a.num_pages ? static_cast<int32_t>(a.num_pages - 1) : pg);
        }
        __syncthreads();
    }
    const int64_t pmask = PG ? (int64_t{1} << a.page_shift) - 1 : 0;
    const int pcol = (T.kv + kvl) * a.D * ES + lane_d * VB;     // PG: this lane's bytes inside a row of a page
    struct Buf {
        Raw<VB> v[U];
        float w[U][GT];
    };
    auto load = [&](Buf& bf, int st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = step_row(st) + u * rps;  // of this step's slot 0; the lane adds r
            if constexpr (PG) {
                // Rows past the split read its last row (their weight is 0).
                const int64_t c = cb + min(row + r, nrows - 1);
                const int64_t page = s_pages[(c >> a.page_shift) - pg0];
                bf.v[u] = load_raw<VB>(a.V + ((page << a.page_shift) + (c & pmask)) * vrow + pcol);
            } else {
                bf.v[u] = load_raw_buf<VB>(vres, voff, row * vrow32);
            }
            load_floats<GT>(wres, woff, row * a.Hq * 4, bf.w[u]);
        }
    };
    auto compute = [&](const Buf& bf, int st) {
        if constexpr (SM) {
            // Rows past the split read as zero; they must not count as scores.
            float x[U][GT], nm[GT];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = step_row(st) + u * rps + r < nrows;
#pragma unroll
                for (int g = 0; g < GT; ++g) x[u][g] = ok ? bf.w[u][g] : -INFINITY;
            }
            bool up = false;
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                float t = mx[g];
#pragma unroll
                for (int u = 0; u < U; ++u) t = fmaxf(t, x[u][g]);
                nm[g] = t;
                up |= t > mx[g];
            }
            if (__any(up)) {
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    const float al = nm[g] > mx[g] ? __builtin_amdgcn_exp2f((mx[g] - nm[g]) * kLog2e) : 1.0f;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[g][e] *= al;
                    lsum[g] *= al;
                    mx[g] = nm[g];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[E];
                widen<DT, VB>(bf.v[u], f);
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    const float w = __builtin_amdgcn_exp2f((x[u][g] - (mx[g] == -INFINITY ? 0.0f : mx[g])) * kLog2e);
                    lsum[g] += w;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[g][e] = __builtin_fmaf(w, f[e], acc[g][e]);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float f[E];
                widen<DT, VB>(bf.v[u], f);
#pragma unroll
                for (int g = 0; g < GT; ++g)
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[g][e] = __builtin_fmaf(bf.w[u][g], f[e], acc[g][e]);
            }
        }
    };
    if (active) {
        // Two buffers in flight; the reload of bA is unconditional (a step
        // past ce reads zeros and is never computed).
        Buf bA, bB;
        int st = 0;
        // PG: keep each step's loads ahead of the other buffer's arithmetic (the
        // page lookups through LDS otherwise let the scheduler move the
        // arithmetic first, which then waits for every load in flight).
        auto fence = [] {
            __builtin_amdgcn_sched_barrier(0);
        };
        if (nsteps > 0) load(bA, 0);
        for (; st + 1 < nsteps; st += 2) {
            load(bB, st + 1);
            fence();
            compute(bA, st);
            load(bA, st + 2);
            fence();
            compute(bB, st + 1);
        }
        if (st < nsteps) compute(bA, st);
    }
    __syncthreads();                                  // LDS is reused below

    // SM: bring every row slot to the workgroup's maximum per (KV head of the
    // tile, head): the first lane of each slot and KV head holds the slot's
    // values (the other lanes of the slot saw the same rows and weights).
    const int nst = a.ht * GT;                        // <= 4 GT: the plan keeps ht <= 4 here
    if constexpr (SM) {
        const bool lead = active && j - kvl * a.L == 0;
        if (lead)
#pragma unroll
            for (int g = 0; g < GT; ++g) smem[(r * a.ht + kvl) * GT + g] = mx[g];
        __syncthreads();
        if (tid < nst) {
            float M = -INFINITY;
            for (int rr = 0; rr < rps; ++rr) M = fmaxf(M, smem[rr * nst + tid]);
            s_stat[0][tid] = M;
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                const float al = mx[g] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mx[g] - s_stat[0][kvl * GT + g]) * kLog2e);
#pragma unroll
                for (int e = 0; e < E; ++e) acc[g][e] *= al;
                lsum[g] *= al;
            }
        }
        if (lead)
#pragma unroll
            for (int g = 0; g < GT; ++g) smem[(r * a.ht + kvl) * GT + g] = lsum[g];
        __syncthreads();
        if (tid < nst) {
            float L = 0.0f;
            for (int rr = 0; rr < rps; ++rr) L += smem[rr * nst + tid];
            s_stat[1][tid] = L;
        }
        __syncthreads();
    }

    // Sum the row slots, CHH heads at a time (CHH * E <= 32 accumulators of a
    // lane): every active thread stores its E consecutive columns of each head
    // of the chunk into LDS rows [row slot][KV head of the tile][head][column]
    // of RL floats (the workgroup's columns of one KV head), 16 bytes at a
    // time when E allows; then each thread adds a quad of columns (or one
    // column) of one head over the row slots, in slot order, and writes it
    // with one store.
    constexpr int CHH = E >= 32 ? 1 : (32 / E < GT ? 32 / E : GT);   // heads per chunk
    constexpr int QW = E % 4 == 0 ? 4 : 1;           // columns a reader adds and stores at once
    const int Lh = Lc / a.ht;                        // lane chunks of one KV head in the workgroup
    const int RL = Lh * E;                           // columns of one KV head in the workgroup
    const int jl = j - kvl * a.L;                    // this lane's chunk within its KV head
    float* const plane = a.nsplit > 1 ? a.part + static_cast<size_t>(T.s) * a.B * a.Hq * a.D : a.out;
    const bool vec_store = QW == 4 && (reinterpret_cast<uintptr_t>(plane) & 15u) == 0;
    typedef __attribute__((address_space(3))) float lds_fl;
    typedef __attribute__((address_space(3))) f32x4 lds_f4;
    lds_fl* const red = (lds_fl*)(smem);
#pragma unroll
    for (int g0 = 0; g0 < GT; g0 += CHH) {
        if (active) {
#pragma unroll
            for (int gl = 0; gl < CHH; ++gl) {
                if (g0 + gl >= GT) break;
                lds_fl* const dst = red + ((r * a.ht + kvl) * CHH + gl) * RL + jl * E;
                if constexpr (E % 4 == 0) {
#pragma unroll
                    for (int e = 0; e < E; e += 4)
                        *(lds_f4*)(dst + e) = f32x4{acc[g0 + gl][e], acc[g0 + gl][e + 1], acc[g0 + gl][e + 2],
                                                    acc[g0 + gl][e + 3]};
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) dst[e] = acc[g0 + gl][e];
                }
            }
        }
        __syncthreads();
        const int nh = GT - g0 < CHH ? GT - g0 : CHH;
        const int units = a.ht * nh * (RL / QW);
        for (int q = tid; q < units; q += kThreads) {
            const int kl = q / (nh * (RL / QW));
            const int gl = (q / (RL / QW)) % nh;
            const int dl = (q % (RL / QW)) * QW;       // column within the workgroup's columns of the KV head
            const int d = (a.ht > 1 ? 0 : T.dt * Lc * E) + dl;
            const int g = g0 + gl;
            const int ql = lane_q_lo(kl);
            const int go = T.q_first + kl * a.G - ql;  // accumulator of the tile's first head
            if (d >= a.D || g < go || g >= go + T.nq) continue;
            f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int rr = 0; rr < rps; ++rr) {
                const lds_fl* const src = red + ((rr * a.ht + kl) * CHH + gl) * RL + dl;
                if constexpr (QW == 4) {
                    sum += *(const lds_f4*)src;
                } else {
                    sum[0] += src[0];
                }
            }
            if constexpr (SM) {
                // One split: normalise here (C = 0 gives zeros); several: the
                // combine does, from the statistics written below.
                if (a.nsplit == 1) {
                    const float l = s_stat[1][kl * GT + g];
                    sum = nrows_split > 0 ? sum / l : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
            if constexpr (DT == kFP8) {
                // The KV head's scale, once per output (the sums are linear in V).
                if (a.v_scale) sum *= a.v_scale[(ql + g) / a.G];
            }
            float* const o = plane + (static_cast<size_t>(T.b) * a.Hq + ql + g) * a.D + d;
            if (vec_store) {
                *reinterpret_cast<f32x4*>(o) = sum;
            } else {
#pragma unroll
                for (int c = 0; c < QW; ++c) o[c] = sum[c];
            }
        }
        __syncthreads();
    }
    if constexpr (SM) {
        if (a.nsplit > 1 && T.dt == 0 && tid < nst) {
            const int kl = tid / GT, g = tid - kl * GT;
            const int ql = lane_q_lo(kl);
            const int go = T.q_first + kl * a.G - ql;
            if (g >= go && g < go + T.nq) {
                float* const st = a.stats + ((static_cast<size_t>(T.s) * a.B + T.b) * a.Hq + ql + g) * 2;
                // PG: a sequence of length 0 (its first split is empty) hands the
                // combine maximum 0 and weight sum 1 beside zero partials, so its
                // outputs come out as zeros rather than 0 / 0.
                const bool empty = PG && T.s == 0 && nrows_split == 0;
                st[0] = empty ? 0.0f : s_stat[0][tid];
                st[1] = empty ? 1.0f : s_stat[1][tid];
            }
        }
    }
}

// ---- pass 1: MFMA engine ----------------------------------------------------

// NSET sets of 16 query heads; DE = D / 16 elements of V per lane and row.
// Rows are taken in groups of four (the K of one MFMA); wave w of the
// workgroup handles groups w, w + 4, w + 8, ... of its split, U groups per
// step, with the next step's loads in flight during the current step.
template <int DT, int DE, int NSET, int U>
__global__ __launch_bounds__(kThreads) void av_pass1_mfma(Pass1Args a) {
    constexpr int ES = esize<DT>();
    constexpr int NB = DE * ES;                      // V bytes per lane and row
    constexpr int NREG = NSET * DE * 4;              // accumulator floats per lane
    constexpr int TO = NREG * 64;                    // outputs of the tile (= 16 * NSET * D)
    __shared__ float red[kWaves * TO];

    const Tile T = decode_tile(a, 16 * NSET);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int k = lane >> 4;                         // row inside a group of four
    const int n = lane & 15;                         // D-chunk / head index inside a set

    const int64_t cb = static_cast<int64_t>(T.s) * a.rows_per_split;
    const int64_t ce = min(a.C, cb + a.rows_per_split);
    const size_t vrow = static_cast<size_t>(a.Hkv) * a.D * ES;
    const uint8_t* vbase = a.V + (static_cast<size_t>(T.b) * a.v_seq_rows * a.Hkv + T.kv) * a.D * ES
                               + static_cast<size_t>(n) * NB;
    // Lane n of set s reads head q_first + 16 s + n. Heads past the tile's nq
    // read the tile's last head instead (a valid address): their A-operand row
    // only feeds output rows past nq, which are never written. Every load is
    // unconditional and no loaded value is touched before the MFMA, so the
    // compiler's wait counts stay exact and the next step's loads overlap the
    // current step's MFMAs.
    const float* abase = a.attn + static_cast<size_t>(T.b) * a.C * a.Hq + T.q_first;
    int woff[NSET];
#pragma unroll
    for (int s = 0; s < NSET; ++s) woff[s] = min(n + 16 * s, T.nq - 1);

    f32x4 acc[NSET][DE];
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int e = 0; e < DE; ++e) acc[s][e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    constexpr int RSTEP = 4 * kWaves * U;            // rows per workgroup step
    const int64_t nsteps = ce > cb ? (ce - cb + RSTEP - 1) / RSTEP : 0;

    // Row of group u of the step starting at c0, for this lane.
    auto row_of = [&](int64_t c0, int u) -> int64_t { return c0 + 4 * (u * kWaves + wave) + k; };
    auto load = [&](Raw<NB> (&rv)[U], float (&rw)[U][NSET], int64_t c0) {
        if (c0 + RSTEP <= ce) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = row_of(c0, u);
                rv[u] = load_raw<NB>(vbase + static_cast<size_t>(c) * vrow);
#pragma unroll
                for (int s = 0; s < NSET; ++s) rw[u][s] = abase[c * a.Hq + woff[s]];
            }
        } else {
            // Last, partial step: rows past ce read row ce - 1 and are zeroed.
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = row_of(c0, u);
                const bool in = c < ce;
                const int64_t cc = in ? c : ce - 1;
                const Raw<NB> raw = load_raw<NB>(vbase + static_cast<size_t>(cc) * vrow);
#pragma unroll
                for (int i = 0; i < (NB >= 4 ? NB / 4 : 1); ++i) rv[u].w[i] = in ? raw.w[i] : 0u;
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    const float w = abase[cc * a.Hq + woff[s]];
                    rw[u][s] = in ? w : 0.0f;
                }
            }
        }
    };
    auto compute = [&](const Raw<NB> (&rv)[U], const float (&rw)[U][NSET]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[DE];
            widen<DT, NB>(rv[u], f);
#pragma unroll
            for (int s = 0; s < NSET; ++s)
#pragma unroll
                for (int e = 0; e < DE; ++e)
                    acc[s][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(rw[u][s], f[e], acc[s][e], 0, 0, 0);
        }
    };

    Raw<NB> vA[U], vB[U];
    float wA[U][NSET], wB[U][NSET];
    int64_t st = 0;
    if (nsteps > 0) load(vA, wA, cb);
    for (; st + 1 < nsteps; st += 2) {
        const int64_t c1 = cb + (st + 1) * RSTEP;
        load(vB, wB, c1);
        compute(vA, wA);
        if (st + 2 < nsteps) load(vA, wA, c1 + RSTEP);
        compute(vB, wB);
    }
    if (st < nsteps) compute(vA, wA);

    // Add the four waves' 16 x D tiles. Register i of acc[s][e] in lane l is
    // head 16 s + 4 (l / 16) + i, element d = (l % 16) * DE + e; as a tile
    // output index: ((s * DE + e) * 4 + i) * 64 + l.
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int e = 0; e < DE; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave * TO + ((s * DE + e) * 4 + i) * 64 + lane] = acc[s][e][i];
    __syncthreads();
    float* const plane = a.nsplit > 1 ? a.part + static_cast<size_t>(T.s) * a.B * a.Hq * a.D : a.out;
    auto out_index = [&](int idx, size_t* o) -> bool {
        const int l = idx & 63, reg = idx >> 6;
        const int i = reg & 3, se = reg >> 2;
        const int e = se % DE, s = se / DE;
        const int g = 16 * s + 4 * (l >> 4) + i;
        *o = (static_cast<size_t>(T.b) * a.Hq + T.q_first + g) * a.D + (l & 15) * DE + e;
        return g < T.nq;
    };
    for (int idx = threadIdx.x; idx < TO; idx += kThreads) {
        float sum = red[idx];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) sum += red[w * TO + idx];
        size_t o;
        if (out_index(idx, &o)) plane[o] = sum;
    }
}

// ---- pass 1: bf16 matrix-core engine ----------------------------------------

// For bf16 V the fp32 matrix instruction above is the bottleneck at large G:
// a 16-head set costs 2 * 16 * D flops per V row at the fp32 matrix rate,
// which at 8 TB/s of V keeps every SIMD about 80 % busy. This engine uses
// v_mfma_f32_16x16x32_bf16 instead (eight times the fp32 matrix rate per
// instruction slot) and keeps the products exact:
//  * each fp32 weight w is split into three bf16 terms by truncation,
//    hi = trunc(w), mid = trunc(w - hi), lo = w - hi - mid. Both subtractions
//    are exact (Sterbenz) and lo has at most 8 significant bits, so
//    w = hi + mid + lo exactly for every normal w down to 2^-103; each
//    product V * term is exact in fp32 (8-bit by 8-bit significands);
//  * one 16 x 16 output tile takes three instructions per 32 context rows,
//    so the matrix core is about 15 % busy at 8 TB/s.
// Operand layout (K = 32 context rows): lane 16 g + m holds, in its eight
// 16-bit slots j = 0..7, A[head m][row 8 g + j] and B[row 8 g + j][column m].
// B needs eight rows of one column per lane while a V row is contiguous along
// D, so each wave writes its 32 rows to a private LDS region as loaded
// (16-byte lane stores) and reads the columns back as 16-bit loads. 16-byte
// pieces of a row are XOR-swizzled by its row group (row / 8) so the four
// lane groups of a column read hit different banks.
//
// PR = D / 8 16-byte pieces per row (8, 16 or 32); NSET sets of 16 heads; U
// chunks of 32 rows per wave and buffer, two buffers in flight; NW waves per
// workgroup (4 or 8); HT adjacent KV heads per workgroup (1, 2 or 4; 8 with
// eight waves, not in fused attention), each streamed by NW / HT waves, so the
// workgroup reads HT * 2 D contiguous bytes of every row.
//
// SM: fused softmax (see av_pass1_valu). A wave keeps one running maximum per
// head for its rows: the four lane groups holding a head's weights of a chunk
// agree on the chunk's maximum through two lane exchanges, so every product
// summed into one accumulator uses the same maximum. The waves of a KV head
// are brought to their common maximum before they are added.
//
// VDT: V's element type, kBF16 or kFP8. fp8 V (OCP E4M3) is loaded as 8-byte
// pieces of 8 values and widened in registers to the same 16-byte bf16 pieces
// before the LDS store -- exactly: every E4M3 value is a bfloat16 value -- so
// everything after the store is the bf16 path; each output is then multiplied
// by its KV head's scale.
//
// PG: paged V (see av_pass1_valu): the split's page list in LDS, each lane's
// row addresses from it, rows past the sequence's length reading the split's
// last valid row with weight 0.
//
// QK: fused decode attention (with SM, dense bf16 or fp8 K and V). Each chunk's K rows
// go through the same LDS region as its V rows; S = Q K^T for the tile's 16
// heads and the chunk's 32 rows comes from v_mfma_f32_16x16x32_bf16 with the
// queries as the A operand, split exactly into three bf16 terms, and the K
// rows as the B operand (16 bytes of one row per lane, read straight from the
// swizzled region); S times qk_scale then passes through the region once more
// to reach the weights' layout, and the fused softmax runs on it as on scores
// read from memory.
template <int PR, int NSET, int U, int HT, bool SM = false, int VDT = kBF16, bool PG = false, bool QK = false,
          int NW = kWaves>
__global__ __launch_bounds__(64 * NW) void av_pass1_mfma_bf16(Pass1Args a) {
    constexpr int NTH = 64 * NW;                     // threads of the workgroup
    static_assert(!QK || SM, "fused attention runs the fused softmax");
    static_assert(PR == 8 || PR == 16 || PR == 32, "D must be 64, 128 or 256");
    static_assert(VDT == kBF16 || VDT == kFP8, "bf16 or fp8 V");
    constexpr bool FP8 = VDT == kFP8;
    constexpr int VES = FP8 ? 1 : 2;                 // bytes of one V element in memory
    constexpr int PB = 8 * VES;                      // bytes of one 8-value piece in memory
    static_assert((HT == 1 || HT == 2 || HT == 4 || (HT == 8 && !QK)) && NW % HT == 0,
                  "KV heads per tile must divide the waves (eight: not fused attention, a wave per KV head)");
    constexpr int D = PR * 8;
    constexpr int RB = PR * 16;                      // bytes of one D-row
    constexpr int NT = D / 16;                       // 16-column output tiles
    constexpr int LPI = PR / 2;                      // 16-byte loads per lane and chunk
    constexpr int RPI = 64 / PR;                     // rows one 64-lane load covers
    constexpr int WPH = NW / HT;                     // waves per KV head
    constexpr int STAGE = NW * 32 * RB;              // bytes: one 32-row region per wave
    constexpr int GH = 16 * NSET;                    // heads of a KV head's tile
    constexpr int RP = D + 4;                        // floats per row of the final sum (padded)
    constexpr int RED = NW * GH * RP * 4;            // bytes: the final cross-wave sum
    __shared__ __align__(16) uint8_t smem[STAGE > RED ? STAGE : RED];

    const Tile T = decode_tile(a, 16 * NSET);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;                         // K group: rows 8 g .. 8 g + 7 of a chunk
    const int m = lane & 15;                         // head (A) / column (B) inside a tile
    const int kvl = wave / WPH;                      // which KV head of the tile
    const int wh = wave % WPH;                       // which of that head's waves

    // The split bounds are workgroup-uniform; keep them in scalar registers.
    // Interleaved splits (dense V; see av_pass1_valu): cb = 0, ce = C, and the
    // workgroup takes the steps s, s + nsplit, ... of the sequence.
    const bool il = !PG && !QK && a.interleave;
    const int64_t cb = il ? 0 : uniform64(static_cast<int64_t>(T.s) * a.rows_per_split);
    int64_t ce_ = il ? a.C : min(a.C, cb + a.rows_per_split);
    if constexpr (PG) {
        const int64_t len = a.seq_lens[T.b];
        ce_ = min(ce_, len < 0 ? int64_t{0} : min(len, a.C));
    }
    const int64_t ce = uniform64(ce_);
    // > 0 for dense V (splits never start past C); paged V may give 0
    const int nrows = ce > cb ? static_cast<int>(ce - cb) : 0;
    const int vrow = a.Hkv * D * VES;                // bytes between consecutive rows of V

    // Both operands are read through buffer resources that end with the
    // split's last row: a row at or past ce reads as zero, so a partial last
    // step needs no clamping or masking, and a step wholly past ce (the
    // pipeline's unconditional reload) touches no memory. The plan keeps a
    // split's V span under 2 GB so 32-bit offsets suffice.
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.V) + (PG ? 0 : ((static_cast<size_t>(T.b) * a.v_seq_rows + cb) * a.Hkv + T.kv) * D * VES), 0,
        PG || nrows == 0 ? 0 : (nrows - 1) * vrow + HT * D * VES, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.attn) + (static_cast<size_t>(T.b) * a.C + cb) * a.Hq + T.q_first, 0,
        nrows == 0 ? 0 : ((nrows - 1) * a.Hq + (HT - 1) * a.G + T.nq) * 4, kRawBufferFlags);
    // PG: the split's pages, from the block table into LDS.
    __shared__ int32_t s_pages[PG ? kMaxSplitPages : 1];
    const int64_t pg0 = PG ? (cb >> a.page_shift) : 0;
    const int npg = PG && nrows > 0 ? static_cast<int>(((cb + nrows - 1) >> a.page_shift) - pg0 + 1) : 0;
    if constexpr (PG) {
        const int32_t* const btr = a.block_table + static_cast<size_t>(T.b) * a.max_pages + pg0;
        for (int i = threadIdx.x; i < npg; i += NTH) {
            const int32_t pg = btr[i];
            s_pages[i] = pg < 0 ? 0 : (pg >= a.num_pages ? static_cast<int32_t>(a.num_pages - 1) : pg);
        }
        __syncthreads();
    }
    const int64_t pmask = PG ? (int64_t{1} << a.page_shift) - 1 : 0;
    // This lane's pieces of a chunk: load i covers rows RPI i .. RPI i + RPI - 1.
    const int prow = lane / PR, ppiece = lane % PR;
    const int vlane = prow * vrow + kvl * D * VES + ppiece * PB;
    // PG with pages of at least RPI rows and a split that starts at a multiple
    // of RPI (automatic plans; chunks start at multiples of 32): the RPI rows
    // of one load start at a multiple of RPI and so lie in one page, whose
    // base is then uniform over the wave. (And a page's bytes must fit the
    // resource's 32-bit range.) Used for fp8, whose 8-byte lane loads pay the
    // per-lane page arithmetic twice per byte: measured on MI355X with 16-row
    // pages, paged fp8 attention at B = 64, C = 8192, Hkv = 8, G = 8 takes
    // 225 us against 252 per lane; for bf16 the per-lane form is faster (the
    // fused softmax product at that size: 191 us against 210).
    const bool page_uniform = PG && FP8 && (int64_t{1} << a.page_shift) >= RPI && (cb & (RPI - 1)) == 0 &&
                              (int64_t{1} << a.page_shift) * vrow <= INT32_MAX;
    // Heads past the tile's nq read the tile's last head (in range); their A
    // rows only feed output rows that are never written.
    int wlane[NSET];
#pragma unroll
    for (int s = 0; s < NSET; ++s) wlane[s] = (8 * g * a.Hq + kvl * a.G + min(m + 16 * s, T.nq - 1)) * 4;
    // QK: K through a resource like V's, and this lane's query operand: head
    // m + 16 s of the wave's KV head (heads past the tile read its last head),
    // d = 32 kk + 8 g .. + 7, as three exact bf16 terms.
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(QK ? a.K : a.V) + (PG ? 0 : ((static_cast<size_t>(T.b) * a.C + cb) * a.Hkv + T.kv) * D * VES),
        0, QK && !PG && nrows > 0 ? (nrows - 1) * vrow + HT * D * VES : 0, kRawBufferFlags);
    constexpr int NKK = QK ? D / 32 : 1;             // 32-wide d blocks of a score
    // Dense bf16 K loads straight into the B operand's layout (KD): load i of
    // a chunk is rows 16 t2 + n (t2 = i / NKK), piece 4 kk + g (kk = i % NKK),
    // so lane 16 g + n already holds what the score MFMAs take and K skips
    // LDS. Measured on MI355X (B = 64, C = 8192, Hkv = 8, G = 8): bf16
    // attention 319.4 -> 312.8 us, G = 2 88.7 -> 85.1; fp8 the other way
    // (193.0 -> 262.7: each 8-byte load then touches 16 rows' cache lines
    // instead of 4), so fp8 and paged K keep the row-major loads through LDS.
    constexpr bool KD = QK && !PG && !FP8;
    static_assert(!QK || LPI == 2 * NKK, "one K load per B operand");
    const int klane = (lane & 15) * vrow + kvl * D * VES + (lane >> 4) * PB;
    u32x4 qa[3][NSET][NKK];
    if constexpr (QK) {
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            const float* qrow = a.q + (static_cast<size_t>(T.b) * a.Hq + T.q_first + kvl * a.G +
                                       min(m + 16 * s, T.nq - 1)) * D + 8 * g;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t th[2], tm[2], tl[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) split_bf16x3(qrow[32 * kk + 2 * p + e], th[e], tm[e], tl[e]);
                    qa[0][s][kk][p] = (th[0] >> 16) | th[1];
                    qa[1][s][kk][p] = (tm[0] >> 16) | tm[1];
                    qa[2][s][kk][p] = (tl[0] >> 16) | tl[1];
                }
        }
    }

    // LDS region of this wave: 32 rows of RB bytes, each row cut into 32-byte
    // column pairs (16 columns) whose order is XORed with swz(row) so that
    // both the row stores and the transposing reads spread over the banks.
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    typedef __attribute__((address_space(3))) short4v lds_s4;
    lds_u8* const region = (lds_u8*)(smem) + wave * 32 * RB;
    auto swz = [](int row) {
        return PR == 8 ? (((row & 3) ^ (row >> 3)) & 3) : (((row & 3) | ((row >> 3) << 2)) & (PR / 2 - 1));
    };
    // Load i's 16-byte piece of row RPI i + prow ...
    auto st_off = [&](int i) {
        const int row = RPI * i + prow;
        return row * RB + 32 * ((ppiece >> 1) ^ swz(row)) + 16 * (ppiece & 1);
    };
    // ... and the transposing read of rows 8 g + 4 h .. 8 g + 4 h + 3 for
    // column tile t: source lane 4 k + q of a 16-lane group points at row
    // 8 g + 4 h + k, columns 16 t + 4 q .. 16 t + 4 q + 3; ds_read_b64_tr_b16
    // then hands lane m of the group the column 16 t + m of those four rows.
    auto tr_off = [&](int t, int h) {
        const int row = 8 * g + 4 * h + ((lane & 15) >> 2);
        return row * RB + 32 * (t ^ swz(row)) + 8 * (lane & 3);
    };

    f32x4 acc[NSET][NT];
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[s][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float mx[NSET], lsum[NSET];                      // SM: head m + 16 s, this lane's rows (maximum score, weight sum)
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        mx[s] = -INFINITY;
        lsum[s] = 0.0f;
    }

    constexpr int RSTEP = 32 * WPH * U;             // rows per workgroup step
    const int nblk = (nrows + RSTEP - 1) / RSTEP;   // steps of the rows [cb, ce)
    const int nsteps = il ? (nblk > T.s ? (nblk - T.s + a.nsplit - 1) / a.nsplit : 0) : nblk;
    // First row (from cb) of this workgroup's step st.
    auto step_row = [&](int st) { return (il ? st * a.nsplit + T.s : st) * RSTEP; };

    typedef typename std::conditional<FP8, u32x2, u32x4>::type Piece;
    struct Buf {
        Piece v[U][LPI];
        Piece k[QK ? U : 1][QK ? LPI : 1];           // QK: the chunk's K pieces
        float w[U][NSET][QK ? 1 : 8];                // weights or scores read from memory (not with QK)
    };
    // Chunk u of step st starts at split row step_row(st) + 32 (u WPH + wh).
    // UNI: PG with pages of at least RPI rows (see page_uniform).
    auto load = [&](Buf& bf, int st, auto uni) {
        constexpr bool UNI = decltype(uni)::value;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r0 = step_row(st) + 32 * (u * WPH + wh);
            // UNI: the chunk's page-list entries, all read before the first
            // is used (one wait for the lot).
            int pl[UNI ? LPI : 1];
            if constexpr (UNI) {
#pragma unroll
                for (int i = 0; i < LPI; ++i)
                    pl[i] = s_pages[min(static_cast<int>(((cb + r0 + RPI * i) >> a.page_shift) - pg0), npg - 1)];
            }
#pragma unroll
            for (int i = 0; i < LPI; ++i) {
                if constexpr (UNI) {
                    // The load's page through a buffer resource that ends with
                    // the split's last row in that page: rows past it read as
                    // zero (their weight is 0), and a load wholly past the split
                    // touches no memory. QK: K from its pool at the same offsets.
                    const int64_t r = cb + r0 + RPI * i;            // the load's first row
                    const int64_t pstart = r & ~pmask;
                    const int pix = __builtin_amdgcn_readfirstlane(pl[i]);
                    const int64_t vr = min(pmask + 1, cb + nrows - pstart);   // valid rows of the page
                    const size_t pbase = (static_cast<size_t>(pix) << a.page_shift) * vrow + T.kv * D * VES;
                    const int nrec = vr > 0 ? static_cast<int>(vr * vrow - T.kv * D * VES) : 0;
                    const int off = vlane + static_cast<int>(r & pmask) * vrow;
                    const __amdgpu_buffer_rsrc_t pv = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<uint8_t*>(a.V) + pbase, 0, nrec, kRawBufferFlags);
                    if constexpr (FP8) bf.v[u][i] = __builtin_amdgcn_raw_buffer_load_b64(pv, off, 0, kCachePolicyNt);
                    else bf.v[u][i] = __builtin_amdgcn_raw_buffer_load_b128(pv, off, 0, kCachePolicyNt);
                    if constexpr (QK) {
                        const __amdgpu_buffer_rsrc_t pk = __builtin_amdgcn_make_buffer_rsrc(
                            const_cast<uint8_t*>(a.K) + pbase, 0, nrec, kRawBufferFlags);
                        if constexpr (FP8) bf.k[u][i] = __builtin_amdgcn_raw_buffer_load_b64(pk, off, 0, kCachePolicyNt);
                        else bf.k[u][i] = __builtin_amdgcn_raw_buffer_load_b128(pk, off, 0, kCachePolicyNt);
                    }
                } else if constexpr (PG) {
                    // Rows past the split read its last row (their weight is 0).
                    // QK: K rows come from K's page pool at the same offsets.
                    const int64_t c = cb + min(r0 + RPI * i + prow, nrows - 1);
                    const int64_t page = s_pages[(c >> a.page_shift) - pg0];
                    const size_t off = static_cast<size_t>(((page << a.page_shift) + (c & pmask)) * vrow +
                                                           (T.kv + kvl) * D * VES + ppiece * PB);
                    bf.v[u][i] = __builtin_nontemporal_load(reinterpret_cast<const Piece*>(a.V + off));
                    if constexpr (QK)
                        bf.k[u][i] = __builtin_nontemporal_load(reinterpret_cast<const Piece*>(a.K + off));
                } else if constexpr (FP8) {
                    bf.v[u][i] = __builtin_amdgcn_raw_buffer_load_b64(vres, vlane, (r0 + RPI * i) * vrow, kCachePolicyNt);
                    if constexpr (KD)
                        bf.k[u][i] = __builtin_amdgcn_raw_buffer_load_b64(
                            kres, klane, (r0 + 16 * (i / NKK)) * vrow + 4 * (i % NKK) * PB, kCachePolicyNt);
                    else if constexpr (QK)
                        bf.k[u][i] = __builtin_amdgcn_raw_buffer_load_b64(kres, vlane, (r0 + RPI * i) * vrow,
                                                                          kCachePolicyNt);
                } else {
                    bf.v[u][i] = __builtin_amdgcn_raw_buffer_load_b128(vres, vlane, (r0 + RPI * i) * vrow,
                                                                       kCachePolicyNt);
                    if constexpr (KD)
                        bf.k[u][i] = __builtin_amdgcn_raw_buffer_load_b128(
                            kres, klane, (r0 + 16 * (i / NKK)) * vrow + 4 * (i % NKK) * PB, kCachePolicyNt);
                    else if constexpr (QK)
                        bf.k[u][i] = __builtin_amdgcn_raw_buffer_load_b128(kres, vlane, (r0 + RPI * i) * vrow,
                                                                           kCachePolicyNt);
                }
            }
            if constexpr (!QK) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int s = 0; s < NSET; ++s)
                        bf.w[u][s][j] = __uint_as_float(
                            __builtin_amdgcn_raw_buffer_load_b32(wres, wlane[s], (r0 + j) * a.Hq * 4, 0));
            }
        }
    };
    // A memory piece as 8 bfloat16 values: bf16 as it is; fp8 widened by
    // gfx950's packed conversion with scale 1, which is exact (bf16 holds
    // every E4M3 value; checked on MI355X against the fp32 conversion for all
    // 256 bytes) and takes one instruction per two values.
    auto to_bf16 = [](const Piece& pc) -> u32x4 {
        if constexpr (FP8) {
            u32x4 piece;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                piece[2 * h] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(pc[h]), 1.0f, false));
                piece[2 * h + 1] = __builtin_bit_cast(
                    uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(pc[h]), 1.0f, true));
            }
            return piece;
        } else {
            return pc;
        }
    };
    // QK: the factor on a score: the score scale, times the KV head's fp8 key scale.
    const float s_mul = QK ? a.qk_scale * (FP8 && a.k_scale ? a.k_scale[T.kv + kvl] : 1.0f) : 0.0f;
    auto consume = [&](const Buf& bf, int st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // The region's previous contents have been read (in program
            // order; LDS executes one wave's operations in order).
            asm volatile("" ::: "memory");
            // QK: the chunk's scores, in the weights' layout (head m + 16 s, rows 8 g .. 8 g + 7).
            float sc[QK ? NSET : 1][QK ? 8 : 1];
            if constexpr (QK) {
                if constexpr (!KD) {
#pragma unroll
                    for (int i = 0; i < LPI; ++i)
                        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(region + st_off(i)) =
                            to_bf16(bf.k[u][i]);
                    asm volatile("" ::: "memory");
                }
                // B operand: lane 16 g + n holds row 16 t2 + n, d = 32 kk + 8 g .. + 7 (piece 4 kk + g).
                f32x4 sacc[NSET][2];
#pragma unroll
                for (int s = 0; s < NSET; ++s)
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) sacc[s][t2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        const int row = 16 * t2 + m, piece = 4 * kk + g;
                        u32x4 kb;
                        if constexpr (KD)
                            kb = to_bf16(bf.k[u][t2 * NKK + kk]);
                        else
                            kb = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                                region + row * RB + 32 * ((piece >> 1) ^ swz(row)) + 16 * (piece & 1));
#pragma unroll
                        for (int k = 0; k < 3; ++k)
#pragma unroll
                            for (int s = 0; s < NSET; ++s)
                                sacc[s][t2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    __builtin_bit_cast(bf16x8, qa[k][s][kk]), __builtin_bit_cast(bf16x8, kb),
                                    sacc[s][t2], 0, 0, 0);
                    }
                asm volatile("" ::: "memory");
                // Register i of sacc[s][t2] in lane 16 g' + n' is head 16 s + 4 g' + i, row 16 t2 + n';
                // through the region as [head][32 rows] floats to head m + 16 s, rows 8 g .. 8 g + 7.
                typedef __attribute__((address_space(3))) float lds_f;
                lds_f* const sreg = reinterpret_cast<lds_f*>(region);
#pragma unroll
                for (int s = 0; s < NSET; ++s)
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            sreg[(16 * s + 4 * g + i) * 32 + 16 * t2 + m] = sacc[s][t2][i] * s_mul;
                asm volatile("" ::: "memory");
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    typedef __attribute__((address_space(3))) f32x4 lds_f4;
                    const f32x4 lo = *reinterpret_cast<const lds_f4*>(sreg + (16 * s + m) * 32 + 8 * g);
                    const f32x4 hi = *reinterpret_cast<const lds_f4*>(sreg + (16 * s + m) * 32 + 8 * g + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        sc[s][j] = lo[j];
                        sc[s][4 + j] = hi[j];
                    }
                }
                asm volatile("" ::: "memory");
            }
#pragma unroll
            for (int i = 0; i < LPI; ++i)
                *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(region + st_off(i)) = to_bf16(bf.v[u][i]);
            asm volatile("" ::: "memory");
            float wt[NSET][8];
            if constexpr (SM) {
                // Scores of rows 8 g .. 8 g + 7 of the chunk; rows past the
                // split read as zero and must not count.
                const int rb = step_row(st) + 32 * (u * WPH + wh) + 8 * g;
                float nm[NSET];
                bool up = false;
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    float t = -INFINITY;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        float x;
                        if constexpr (QK) x = sc[s][j];
                        else x = bf.w[u][s][j];
                        wt[s][j] = rb + j < nrows ? x : -INFINITY;
                        t = fmaxf(t, wt[s][j]);
                    }
                    t = fmaxf(t, __shfl_xor(t, 16));
                    t = fmaxf(t, __shfl_xor(t, 32));
                    nm[s] = fmaxf(mx[s], t);
                    up |= nm[s] > mx[s];
                }
                if (__any(up)) {
#pragma unroll
                    for (int s = 0; s < NSET; ++s) {
                        const float al = nm[s] > mx[s] ? __builtin_amdgcn_exp2f((mx[s] - nm[s]) * kLog2e) : 1.0f;
                        lsum[s] *= al;
                        mx[s] = nm[s];
                        // Register i of acc[s][t] belongs to head 16 s + 4 (lane / 16) + i,
                        // whose factor lane 4 (lane / 16) + i holds.
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float ai = __shfl(al, 4 * (lane >> 4) + i);
#pragma unroll
                            for (int t = 0; t < NT; ++t) acc[s][t][i] *= ai;
                        }
                    }
                }
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    const float ref = mx[s] == -INFINITY ? 0.0f : mx[s];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        wt[s][j] = __builtin_amdgcn_exp2f((wt[s][j] - ref) * kLog2e);
                        lsum[s] += wt[s][j];
                    }
                }
            } else {
#pragma unroll
                for (int s = 0; s < NSET; ++s)
#pragma unroll
                    for (int j = 0; j < 8; ++j) wt[s][j] = bf.w[u][s][j];
            }
            // Split the weights: three bf16x8 A operands per head set.
            u32x4 aw[3][NSET];
#pragma unroll
            for (int s = 0; s < NSET; ++s) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t th[2], tm[2], tl[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) split_bf16x3(wt[s][2 * p + e], th[e], tm[e], tl[e]);
                    aw[0][s][p] = (th[0] >> 16) | th[1];
                    aw[1][s][p] = (tm[0] >> 16) | tm[1];
                    aw[2][s][p] = (tl[0] >> 16) | tl[1];
                }
            }
            // B operands of all column tiles, then the MFMAs with the tiles
            // innermost so consecutive instructions never share an accumulator.
            u32x4 bv[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s4*>(region + tr_off(t, 0)));
                const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s4*>(region + tr_off(t, 1)));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                bv[t] = u32x4{l2.x, l2.y, h2.x, h2.y};
            }
#pragma unroll
            for (int k = 0; k < 3; ++k)
#pragma unroll
                for (int s = 0; s < NSET; ++s)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, aw[k][s]), __builtin_bit_cast(bf16x8, bv[t]), acc[s][t], 0, 0, 0);
        }
    };

    // Two buffers in flight; the reload of bA is unconditional (past ce it
    // reads zeros): a conditional load would leave the compiler unsure whether
    // it is outstanding, and it would then wait for every load before
    // consuming bB.
    // Keep each step's loads ahead of the other buffer's work (see av_pass1_valu).
    // Not in dense fused attention: the barrier keeps both buffers' K and V
    // pieces live across the score MFMAs, which takes its fp8 kernel (and the
    // bf16 one at D = 64 with 32-head sets) past 256 registers, to one wave per
    // SIMD where the plan runs two workgroups per CU (fp8 at B = 64, C = 8192,
    // Hkv = 8, G = 8: 209 us against 178).
    auto fence = [] {
        if constexpr (PG || !QK) __builtin_amdgcn_sched_barrier(0);
    };
    // The pipeline, once per load kind, so that each loop holds one kind of
    // load (with both in one loop the compiler waits for loads it need not).
    auto run = [&](auto uni) {
        Buf bA, bB;
        int st = 0;
        if (nsteps > 0) load(bA, 0, uni);
        for (; st + 1 < nsteps; st += 2) {
            load(bB, st + 1, uni);
            fence();
            consume(bA, st);
            load(bA, st + 2, uni);
            fence();
            consume(bB, st + 1);
        }
        if (st < nsteps) consume(bA, st);
    };
    if constexpr (PG && FP8) {
        if (page_uniform) run(std::true_type{});
        else run(std::false_type{});
    } else {
        run(std::false_type{});
    }

    // SM: each wave's maximum and weight sum per head (lane group 0 holds head
    // m + 16 s after the sum over the four lane groups).
    __shared__ float s_wm[NW][GH], s_wl[NW][GH], s_tm[HT][GH], s_tl[HT][GH];
    if constexpr (SM) {
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            lsum[s] += __shfl_xor(lsum[s], 16);
            lsum[s] += __shfl_xor(lsum[s], 32);
            if (g == 0) {
                s_wm[wave][m + 16 * s] = mx[s];
                s_wl[wave][m + 16 * s] = lsum[s];
            }
        }
    }

    // Add the tiles of each KV head's waves. Register i of acc[s][t] in lane
    // l is head 16 s + 4 (l / 16) + i, column 16 t + l % 16. Each wave puts
    // its tile into LDS as [head][column] rows of RP floats (the padding puts
    // the four lane groups of one store on different banks); a thread then
    // adds four consecutive columns of one head over the KV head's waves, in
    // wave order, and writes them with one 16-byte store.
    __syncthreads();                                 // every wave is done with its region
    if constexpr (SM) {
        // Bring this wave's tile to the maximum of its KV head's waves.
#pragma unroll
        for (int s = 0; s < NSET; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int hh = 16 * s + 4 * (lane >> 4) + i;
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < WPH; ++w) M = fmaxf(M, s_wm[kvl * WPH + w][hh]);
                const float mw = s_wm[wave][hh];
                const float al = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mw - M) * kLog2e);
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[s][t][i] *= al;
            }
        // The tile's maximum and weight sum per (KV head, head).
        if (threadIdx.x < HT * GH) {
            const int k = threadIdx.x / GH, hh = threadIdx.x % GH;
            float M = -INFINITY, L = 0.0f;
#pragma unroll
            for (int w = 0; w < WPH; ++w) M = fmaxf(M, s_wm[k * WPH + w][hh]);
#pragma unroll
            for (int w = 0; w < WPH; ++w) {
                const float mw = s_wm[k * WPH + w][hh];
                L += mw == -INFINITY ? 0.0f : s_wl[k * WPH + w][hh] * __builtin_amdgcn_exp2f((mw - M) * kLog2e);
            }
            // PG: a sequence of length 0 (its first split is empty) hands the
            // combine maximum 0 and weight sum 1 beside zero partials, so its
            // outputs come out as zeros rather than 0 / 0.
            const bool empty = PG && T.s == 0 && nrows == 0;
            s_tm[k][hh] = empty ? 0.0f : M;
            s_tl[k][hh] = empty ? 1.0f : L;
        }
    }
    float* const red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[(wave * GH + 16 * s + 4 * (lane >> 4) + i) * RP + 16 * t + (lane & 15)] = acc[s][t][i];
    __syncthreads();
    float* const plane = a.nsplit > 1 ? a.part + static_cast<size_t>(T.s) * a.B * a.Hq * D : a.out;
    // `out` need only be 4-byte aligned; the split planes are 16-byte aligned.
    const bool vec_store = (reinterpret_cast<uintptr_t>(plane) & 15u) == 0;
    constexpr int Q4 = D / 4;                        // column quads of a head's row
    typedef __attribute__((address_space(3))) f32x4 lds_f4;
    for (int qi = threadIdx.x; qi < HT * GH * Q4; qi += NTH) {
        const int k = qi / (GH * Q4), hh = (qi / Q4) % GH, c4 = qi % Q4;
        typedef __attribute__((address_space(3))) float lds_fl;
        const lds_f4* const r0 = (const lds_f4*)((lds_fl*)(smem) + (k * WPH * GH + hh) * RP + 4 * c4);
        f32x4 sum = r0[0];
#pragma unroll
        for (int w = 1; w < WPH; ++w) sum += r0[w * GH * RP / 4];
        if constexpr (SM) {
            // One split: normalise here; several: the combine does.
            if (a.nsplit == 1) sum = nrows > 0 ? sum / s_tl[k][hh] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        if constexpr (FP8) {
            if (a.v_scale) sum *= a.v_scale[T.kv + k];   // the tile's k-th KV head
        }
        if (hh < T.nq) {
            float* const o = plane + (static_cast<size_t>(T.b) * a.Hq + T.q_first + k * a.G + hh) * D + 4 * c4;
            if (vec_store) {
                *reinterpret_cast<f32x4*>(o) = sum;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = sum[c];
            }
        }
    }
    if constexpr (SM) {
        if (a.nsplit > 1 && threadIdx.x < HT * GH) {
            const int k = threadIdx.x / GH, hh = threadIdx.x % GH;
            if (hh < T.nq) {
                float* const stp =
                    a.stats + ((static_cast<size_t>(T.s) * a.B + T.b) * a.Hq + T.q_first + k * a.G + hh) * 2;
                stp[0] = s_tm[k][hh];
                stp[1] = s_tl[k][hh];
            }
        }
    }
}

}  // namespace gqa_av
