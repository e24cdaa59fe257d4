// Device code of the GQA decode score step on gfx950 (MI355X).
//
//   scores[b, c, q_h] = scale * sum_d q[b, q_h, d] * K[b, c, kv_h, d],  kv_h = q_h / G
//
// It is the step before the attention-times-V product of ExecuTorch PR #21063,
// "...GEMV" (that page covers the product only): its output, after a softmax
// over c, is that product's attn input and has the same [B][C][Hq] layout. The
// page's idea carries over unchanged -- the G query heads of a group share one
// K row, so a workgroup per KV head reads each K row once for all G of them.
//
// Every score depends on a single K row, so the context needs no split and no
// combine: a workgroup owns a tile (b, HT adjacent KV heads, head set) and a
// block of context rows; 4 / HT of its waves stream each KV head, so the
// workgroup reads an HT * D-wide contiguous slice of every row. The contraction over d is a skinny matrix product, done on the matrix
// cores with the K rows as the A operand (16 rows x 32 d), which is K's own
// row-major layout, and the query heads as the B operand (32 d x 16 heads):
//  * bf16 K: v_mfma_f32_16x16x32_bf16, with each fp32 q value split once per
//    workgroup into three bf16 terms (split_bf16x3, exact), so every product is
//    exact and only the fp32 sums round;
//  * fp16 K: v_mfma_f32_16x16x32_f16 with K as it is. Each query head's q
//    values are scaled by a power of two 2^e that brings their largest
//    magnitude into [2^14, 2^15) and split into three fp16 terms by rounding
//    (each remainder is exact); every product of fp16 values is exact in fp32,
//    and what the split drops is below 2^-33 of that head's largest q value
//    (2^-38 of it near fp16's subnormal range), far under the fp32 rounding of
//    the sums. The head's result column is multiplied by scale * 2^-e;
//  * fp32 K: K as fp32 and v_mfma_f32_16x16x4_f32;
//  * fp8 K (OCP FP8 E4M3, a float32 scale per KV head): every E4M3 value is a
//    bfloat16 value, so each 16-byte piece of 16 fp8 values is widened exactly
//    (v_cvt_pk_f32_fp8, then the upper half of each fp32) into two bf16
//    pieces on its way into LDS, and the bf16 path runs from there; the KV
//    head's scale joins the score scale on the head's result column.
// The A operand wants lane 16 g + m to hold row m's d-range
// [32 blk + 8 g, 32 blk + 8 g + 8). Loaded that way, one 64-lane load would
// touch 16 rows at 64 bytes each, a pattern that streams 25 % slower on
// MI355X than whole rows. So each wave loads its 16-row block as consecutive
// 16-byte pieces (whole rows, several per load), stores them to a private LDS
// region with rows padded by 16 bytes (so the 16 rows of an operand read fall
// in different banks), and reads each lane's operand back with one 16-byte
// LDS load per block of 32 d (two for fp32). Lane 16 g + n holds head n's q
// values for the same d-range. The result of a 16-row block comes back as lane
// 16 g + n holding rows 4 g + i, head n.
#pragma once

#include "av_kernels.hpp"

#ifndef GQA_QK_BLOCKS
#define GQA_QK_BLOCKS 1   // 16-row blocks per wave and buffer (two buffers in flight); 2 and 4 measured slower
#endif
#ifndef GQA_QK_BLOCKS_FP8
#define GQA_QK_BLOCKS_FP8 2   // fp8 K: half the bytes per block, so twice the blocks per step
#endif

namespace gqa_av {

struct QkArgs {
    const float* q;          // [B][Hq][D]
    const uint8_t* K;        // [B][C][Hkv][D] of KDT
    float* scores;           // [B][C][Hq]
    float scale;
    int64_t C;
    int32_t rows_per_block;  // context rows per workgroup, a multiple of 64
    int32_t nchunk;          // ceil(C / rows_per_block)
    int32_t B, Hq, Hkv, G;
    int32_t per_head;        // 0: tiles of up to 16 * NSET heads of one group; 1: one head per tile
    int32_t nsg;             // head sub-groups per KV head (reuse)
    int32_t ht;              // adjacent KV heads per tile (reuse; 1 for per-head)
    int32_t vec4;            // 1: every tile's score run is whole rows of 16-byte groups, 16-byte aligned
    const float* k_scale;    // fp8 K: [Hkv] scales, or NULL for 1
    // Paged K (block_table != NULL): K points at pages [num_pages][2^page_shift][Hkv][D];
    // row c of sequence b is row c % P of page block_table[b][c / P]; rows c >= seq_lens[b] get no score.
    const int32_t* block_table;
    const int32_t* seq_lens;
    int64_t num_pages;
    int32_t page_shift;
    int32_t max_pages;
    uint32_t nblocks;
};

// Four OCP FP8 E4M3 values (one word, byte 0 first) as four bfloat16 values in
// two words (low half first). Exact: an E4M3 value has at most 4 significant
// bits, so its fp32 form ends in 16 zero bits.
__device__ inline void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    // gfx950's packed conversion, scale 1: exact (bf16 holds every E4M3 value;
    // checked on MI355X against the fp32 conversion for all 256 bytes).
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, true));
}

// KDT: element type of K; NBLK = D / 32; NSET sets of 16 heads per tile; HT
// adjacent KV heads per tile (1, 2 or 4); PG: paged K. A paged workgroup
// copies the block-table entries of its rows into LDS (clamped into the
// cache), takes each lane's row address from them (rows past the sequence's
// length read its last row), and its score resource ends at that length, so
// rows past it are not written.
template <int KDT, int NBLK, int NSET, int HT, bool PG = false>
__global__ __launch_bounds__(kThreads) void qk_scores(QkArgs a) {
    static_assert(HT == 1 || HT == 2 || HT == 4, "KV heads per tile must divide the waves");
    constexpr int WPH = kWaves / HT;                 // waves per KV head
    constexpr bool FP8 = KDT == kFP8;
    constexpr int ES = esize<KDT>();                 // bytes of a K element in memory
    constexpr int ESL = FP8 ? 2 : ES;                // and in LDS (fp8 widened to bf16)
    constexpr int D = 32 * NBLK;
    constexpr int PIECES = KDT == kF32 ? 2 : 1;      // 16-byte operand pieces per lane and block of 32 d
    constexpr bool BF16 = KDT == kBF16 || FP8;
    constexpr bool F16 = KDT == kF16;
    constexpr bool SPLIT = BF16 || F16;              // three 16-bit q terms on the 16x16x32 instruction
    constexpr int NP = D * ES / 16;                  // 16-byte pieces per row in memory
    static_assert(NP % 4 == 0, "whole 64-lane loads per 16-row block");
    constexpr int NLD = NP / 4;                      // 64-lane loads per 16-row block
    constexpr int RBP = D * ESL + 16;                // padded LDS row
    __shared__ __align__(16) uint8_t stage[kWaves * 16 * RBP];

    // Logical tile order, fastest first: head sub-group (or the head's place in
    // its group for the per-head baseline), KV head, context chunk, batch. The
    // KV heads of one (b, chunk) then run on one XCD: they share the lines of
    // each score row they write.
    uint32_t t = xcd_remap(blockIdx.x, a.nblocks);
    const int nminor = a.per_head ? a.G : a.nsg;
    const int minor = t % nminor; t /= nminor;
    const int nkvt = a.Hkv / HT;
    const int kv0 = static_cast<int>(t % nkvt) * HT; t /= nkvt;   // first KV head of the tile
    const int chunk = t % a.nchunk; t /= a.nchunk;
    const int b = static_cast<int>(t);
    const int64_t r0 = uniform64(static_cast<int64_t>(chunk) * a.rows_per_block);
    int64_t end = min(r0 + a.rows_per_block, a.C);
    if constexpr (PG) {
        const int64_t len = a.seq_lens[b];
        end = min(end, len < 0 ? int64_t{0} : min(len, a.C));
    }
    const int nrows = static_cast<int>(uniform64(end > r0 ? end - r0 : 0));
    if (PG && nrows == 0) return;                    // the whole chunk is past the length (uniform)

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15;                         // row (A) / head (B, result) inside a tile
    const int g = lane >> 4;                         // d-group of 8 inside a block of 32
    const int kvl = wave / WPH;                      // this wave's KV head inside the tile
    const int wh = wave % WPH;                       // and its place among that head's waves
    const int kv = kv0 + kvl;
    const int q_first = a.per_head ? kv * a.G + minor : kv * a.G + minor * 16 * NSET;
    const int nq = a.per_head ? 1 : min(16 * NSET, a.G - minor * 16 * NSET);

    // K through a buffer resource ending at the chunk's last row: rows past it
    // read as zero (their scores are never stored).
    const int krow = a.Hkv * D * ES;
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.K) + (PG ? 0 : ((static_cast<size_t>(b) * a.C + r0) * a.Hkv + kv0) * D * ES), 0,
        PG ? 0 : (nrows - 1) * krow + HT * D * ES, kRawBufferFlags);
    // PG: the chunk's pages, from the block table into LDS.
    __shared__ int32_t s_pages[PG ? kMaxSplitPages : 1];
    const int64_t pg0 = PG ? (r0 >> a.page_shift) : 0;
    if constexpr (PG) {
        const int npg = static_cast<int>(((r0 + nrows - 1) >> a.page_shift) - pg0 + 1);
        const int32_t* const btr = a.block_table + static_cast<size_t>(b) * a.max_pages + pg0;
        for (int i = threadIdx.x; i < npg; i += kThreads) {
            const int32_t pg = btr[i];
            s_pages[i] = pg < 0 ? 0 : (pg >= a.num_pages ? static_cast<int32_t>(a.num_pages - 1) : pg);
        }
        __syncthreads();
    }
    const int64_t pmask = PG ? (int64_t{1} << a.page_shift) - 1 : 0;
    // Load i of a block: lane l takes piece f = 64 i + l, i.e. row f / NP,
    // piece f % NP (whole rows, consecutive in memory within each row).
    int koff[NLD], soff[NLD], prow[NLD], pcol[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int f = 64 * i + lane;
        koff[i] = (f / NP) * krow + kvl * D * ES + (f % NP) * 16;
        prow[i] = f / NP;                            // PG: this lane's row inside a 16-row block ...
        pcol[i] = (f % NP) * 16;                     // ... and its piece of that row's KV-head slice
        soff[i] = (f / NP) * RBP + (f % NP) * 16 * (ESL / ES);
    }
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    lds_u8* const region = (lds_u8*)stage + wave * 16 * RBP;

    // Scores: each step's results of all waves are gathered in an LDS tile of
    // R rows (the step's 16-row blocks) by W = HT nq columns (the tile's heads,
    // KV head by KV head) and written out by the whole workgroup: row r of the
    // tile goes to wave r % 4, whose lanes store consecutive heads of the row
    // (one contiguous run per row when nsg = 1), VE of them per lane: 4 (16-byte
    // stores) when every run is 16-byte aligned (a.vec4, set by the host),
    // else 1. Masked MI355X stores are not free, so a step issues only the
    // rounds that hold entries: (R / 4) W / (64 VE) rounded up.
    // Rows past the chunk fall outside the score resource, which ends after the
    // chunk's last row of the tile's heads; lanes past the tile get an offset
    // beyond it. Every offset, plus the step's row offset, stays below 2^30
    // (the plan keeps a chunk's scores under it).
    constexpr int UB = FP8 ? GQA_QK_BLOCKS_FP8 : GQA_QK_BLOCKS;   // 16-row blocks per wave and buffer
    constexpr int R = 16 * WPH * UB;                 // rows per step
    constexpr int WMAX = HT * 16 * NSET;             // tile columns at most
    constexpr int OP = WMAX + 4;                     // LDS tile pitch in floats (4 spare columns)
    constexpr int NSR = R / kWaves * WMAX / 64;      // 4-byte store rounds per wave and step at most
    __shared__ __align__(16) float otile[2][R * OP];
    const int q_tile = kv0 * a.G + (a.per_head ? minor : minor * 16 * NSET);   // first head of the tile
    const int W = HT * nq;
    const int VE = a.vec4 ? 4 : 1;
    const int WQ = W / VE;                           // lanes per tile row
    const int nsr = (R / kWaves * W + 64 * VE - 1) / (64 * VE);   // store rounds per step (<= NSR)
    const int srow = a.Hq * 4;
    const __amdgpu_buffer_rsrc_t sres = __builtin_amdgcn_make_buffer_rsrc(
        a.scores + (static_cast<size_t>(b) * a.C + r0) * a.Hq + q_tile, 0,
        (nrows - 1) * srow + 4 * ((HT - 1) * a.G + nq), kRawBufferFlags);
    int st_lds[NSR], st_off[NSR];
#pragma unroll
    for (int k = 0; k < NSR; ++k) {
        const int e = 64 * k + lane;
        const int rq = e / WQ, c = (e - rq * WQ) * VE;
        const int r = kWaves * rq + wave;            // tile row
        const int kc = c / nq;                       // KV head of column c inside the tile
        const bool ok = r < R;
        st_lds[k] = ok ? r * OP + c : 0;
        st_off[k] = ok ? r * srow + 4 * (kc * a.G + c - kc * nq) : kOutOfRange;
    }
    // This lane's tile column for head m + 16 s (a spare column past the
    // tile's heads when m + 16 s >= nq).
    int o_col[NSET];
#pragma unroll
    for (int s = 0; s < NSET; ++s) o_col[s] = m + 16 * s < nq ? kvl * nq + m + 16 * s : WMAX + (m & 3);

    // q operand, once per wave. Heads past nq read the tile's last head (a
    // valid address); their result columns are never stored.
    u32x4 qb[SPLIT ? 3 : 1][NSET][NBLK];
    float qf[SPLIT ? 1 : NSET][SPLIT ? 1 : NBLK][8];
    float qv[NSET][NBLK][8];
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        const float* qrow = a.q + (static_cast<size_t>(b) * a.Hq + q_first + min(m + 16 * s, nq - 1)) * D + 8 * g;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[s][blk][j] = qrow[32 * blk + j];
    }
    // fp16 K: each head's power-of-two scale (see above). Head m + 16 s's q
    // values sit in lanes m, m + 16, m + 32 and m + 48; its result column in
    // the same lanes.
    float out_scale[NSET];
    const float kv_scale = FP8 && a.k_scale ? a.k_scale[kv] : 1.0f;
#pragma unroll
    for (int s = 0; s < NSET; ++s) out_scale[s] = a.scale * kv_scale;
    if constexpr (F16) {
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            float mx = 0.0f;
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
                for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(qv[s][blk][j]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            int ex = 0;
            (void)frexpf(mx, &ex);                   // mx in [2^(ex-1), 2^ex)
            const int e = mx > 0.0f ? 15 - ex : 0;
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
                for (int j = 0; j < 8; ++j) qv[s][blk][j] = ldexpf(qv[s][blk][j], e);
            out_scale[s] = ldexpf(a.scale, -e);
        }
    }
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
            const float* v = qv[s][blk];
            if constexpr (F16) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t t[3][2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const _Float16 h1 = static_cast<_Float16>(v[2 * p + e]);
                        const float r1 = v[2 * p + e] - static_cast<float>(h1);
                        const _Float16 h2 = static_cast<_Float16>(r1);
                        const float r2 = r1 - static_cast<float>(h2);
                        const _Float16 h3 = static_cast<_Float16>(r2);
                        t[0][e] = __builtin_bit_cast(uint16_t, h1);
                        t[1][e] = __builtin_bit_cast(uint16_t, h2);
                        t[2][e] = __builtin_bit_cast(uint16_t, h3);
                    }
#pragma unroll
                    for (int k = 0; k < 3; ++k) qb[k][s][blk][p] = t[k][0] | (t[k][1] << 16);
                }
            } else if constexpr (BF16) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    uint32_t th[2], tm[2], tl[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) split_bf16x3(v[2 * p + e], th[e], tm[e], tl[e]);
                    qb[0][s][blk][p] = (th[0] >> 16) | th[1];
                    qb[1][s][blk][p] = (tm[0] >> 16) | tm[1];
                    qb[2][s][blk][p] = (tl[0] >> 16) | tl[1];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) qf[s][blk][j] = v[j];
            }
        }
    }

    struct Buf {
        u32x4 raw[UB][NLD];
    };
    // Step st of the head's wave wh covers row blocks j = (st UB + u) WPH + wh,
    // u < UB, each of 16 rows.
    auto block_of = [&](int st, int u) { return (st * UB + u) * WPH + wh; };
    auto load = [&](Buf& bf, int st) {
#pragma unroll
        for (int u = 0; u < UB; ++u)
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                if constexpr (PG) {
                    // Rows past the chunk read its last row (their scores are not stored).
                    const int64_t c = r0 + min(16 * block_of(st, u) + prow[i], nrows - 1);
                    const int64_t page = s_pages[(c >> a.page_shift) - pg0];
                    const uint8_t* const p =
                        a.K + (((page << a.page_shift) + (c & pmask)) * a.Hkv + kv) * D * ES + pcol[i];
                    bf.raw[u][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
                } else {
                    bf.raw[u][i] = __builtin_amdgcn_raw_buffer_load_b128(kres, koff[i], 16 * block_of(st, u) * krow,
                                                                         kCachePolicyNt);
                }
            }
    };
    auto compute_store = [&](const u32x4 (&bfin)[NLD], int j, int st, int tb) {
        // Re-layout through the wave's LDS region (in program order: one
        // wave's LDS operations execute in order).
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            typedef __attribute__((address_space(3))) u32x4 lds_u4;
            if constexpr (FP8) {
                uint32_t w[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) fp8x4_to_bf16x4(bfin[i][k], w[2 * k], w[2 * k + 1]);
                *reinterpret_cast<lds_u4*>(region + soff[i]) = u32x4{w[0], w[1], w[2], w[3]};
                *reinterpret_cast<lds_u4*>(region + soff[i] + 16) = u32x4{w[4], w[5], w[6], w[7]};
            } else {
                *reinterpret_cast<lds_u4*>(region + soff[i]) = bfin[i];
            }
        }
        asm volatile("" ::: "memory");
        struct {
            u32x4 raw[NBLK][PIECES];
        } bf;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
            for (int p = 0; p < PIECES; ++p)
                bf.raw[blk][p] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                    region + m * RBP + (32 * blk + 8 * g) * ESL + 16 * p);
        asm volatile("" ::: "memory");
        // Independent accumulators keep consecutive MFMAs off one dependency chain.
        constexpr int NACC = SPLIT ? 3 : 4;
        f32x4 acc[NACC][NSET];
#pragma unroll
        for (int k = 0; k < NACC; ++k)
#pragma unroll
            for (int s = 0; s < NSET; ++s) acc[k][s] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
            if constexpr (BF16) {
                const bf16x8 ka = __builtin_bit_cast(bf16x8, bf.raw[blk][0]);
#pragma unroll
                for (int k = 0; k < 3; ++k)
#pragma unroll
                    for (int s = 0; s < NSET; ++s)
                        acc[k][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            ka, __builtin_bit_cast(bf16x8, qb[k][s][blk]), acc[k][s], 0, 0, 0);
            } else if constexpr (F16) {
                const half8 ka = __builtin_bit_cast(half8, bf.raw[blk][0]);
#pragma unroll
                for (int k = 0; k < 3; ++k)
#pragma unroll
                    for (int s = 0; s < NSET; ++s)
                        acc[k][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            ka, __builtin_bit_cast(half8, qb[k][s][blk]), acc[k][s], 0, 0, 0);
            } else {
                float kf[8];
#pragma unroll
                for (int p = 0; p < 2; ++p)
#pragma unroll
                    for (int e = 0; e < 4; ++e) kf[4 * p + e] = __uint_as_float(bf.raw[blk][p][e]);
#pragma unroll
                for (int st = 0; st < 8; ++st)
#pragma unroll
                    for (int s = 0; s < NSET; ++s)
                        acc[st & 3][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[st], qf[s][blk][st], acc[st & 3][s],
                                                                            0, 0, 0);
            }
        }
        // Into the step's LDS tile: row 16 (j - first block of the step) + 4 g + i.
        float* const tile = otile[tb] + (16 * (j - st * UB * WPH) + 4 * g) * OP;
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            f32x4 sum = acc[0][s];
#pragma unroll
            for (int k = 1; k < NACC; ++k) sum += acc[k][s];
#pragma unroll
            for (int i = 0; i < 4; ++i) tile[i * OP + o_col[s]] = sum[i] * out_scale[s];
        }
    };

    // Two buffers in flight; the reload is unconditional (blocks past the
    // chunk read zeros and store nothing).
    const int nrb = (nrows + 15) / 16;
    const int nsteps = (nrb + WPH * UB - 1) / (WPH * UB);
    // Step st fills tile tb = st & 1; the barrier of step st + 1 comes after
    // every wave's reads of tile tb, so step st + 2 may overwrite it.
    auto consume = [&](const Buf& bf, int st, int tb) {
#pragma unroll
        for (int u = 0; u < UB; ++u) compute_store(bf.raw[u], block_of(st, u), st, tb);
        __syncthreads();
        if (a.vec4) {
#pragma unroll
            for (int k = 0; k < NSR; ++k)
                if (k < nsr)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4*>(&otile[tb][st_lds[k]])), sres,
                        st_off[k], st * R * srow, 0);
        } else {
#pragma unroll
            for (int k = 0; k < NSR; ++k)
                if (k < nsr)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(otile[tb][st_lds[k]]), sres, st_off[k],
                                                          st * R * srow, 0);
        }
    };
    // PG: keep each step's loads ahead of the other buffer's work (the page
    // lookups would otherwise let the scheduler sink them).
    auto fence = [] {
        if constexpr (PG) __builtin_amdgcn_sched_barrier(0);
    };
    Buf bA, bB;
    int st = 0;
    if (nsteps > 0) load(bA, 0);
    for (; st + 1 < nsteps; st += 2) {
        load(bB, st + 1);
        fence();
        consume(bA, st, 0);
        load(bA, st + 2);
        fence();
        consume(bB, st + 1, 1);
    }
    if (st < nsteps) consume(bA, st, 0);
}

}  // namespace gqa_av
