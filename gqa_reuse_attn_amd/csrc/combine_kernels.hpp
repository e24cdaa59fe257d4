// Second-kernel split combines of the AV path (plain and fused softmax).
// Included by the host translation unit only: these kernels are launched there.
#pragma once

#include "av_kernels.hpp"

namespace gqa_av {

// ---- pass 2: split-C combine -------------------------------------------------

// out[i] = sum over s of part[s][i] for the `plane` outputs, in a fixed order.
// A workgroup covers kThreads / S quads (4 consecutive outputs) with S split
// groups each: group g of a quad sums the contiguous split range
// [nsplit * g / S, nsplit * (g + 1) / S) in increasing s, and the S group sums
// are then added in increasing g (S = 1: one thread sums every split of its
// quad and stores it, no LDS). S (a power of two, 1 to 64) is chosen by the
// host so that a group holds at most four splits when it can: a thread's
// loads of a batch of four are issued together (addresses clamped into its
// range, values masked afterwards), so the kernel costs about one memory
// round trip.
constexpr int kCombineLoads = 4;     // loads a thread issues together
template <int S>
__global__ __launch_bounds__(kThreads) void av_pass2_combine(const float* __restrict__ part,
                                                             float* __restrict__ out,
                                                             int64_t plane, int32_t nsplit) {
    static_assert(S >= 1 && S <= kThreads && (S & (S - 1)) == 0, "split groups: a power of two");
    constexpr int Q = kThreads / S;
    __shared__ f32x4 red[kThreads];
    const int q = threadIdx.x % Q;
    const int g = threadIdx.x / Q;
    const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * Q + q) * 4;
    const int s0 = static_cast<int>((static_cast<int64_t>(nsplit) * g) / S);
    const int s1 = static_cast<int>((static_cast<int64_t>(nsplit) * (g + 1)) / S);
    // Whole float4 loads need a plane of whole quads; the store needs `out` 16-byte aligned.
    const bool quads = (plane & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0;
    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    if (quads && i0 + 3 < plane) {
        for (int sb = s0; sb < s1; sb += kCombineLoads) {
            f32x4 v[kCombineLoads];
#pragma unroll
            for (int k = 0; k < kCombineLoads; ++k)
                v[k] = *reinterpret_cast<const f32x4*>(part + static_cast<size_t>(min(sb + k, s1 - 1)) * plane + i0);
#pragma unroll
            for (int k = 0; k < kCombineLoads; ++k)
                if (sb + k < s1) sum += v[k];
        }
    } else {
        for (int s = s0; s < s1; ++s)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (i0 + c < plane) sum[c] += part[static_cast<size_t>(s) * plane + i0 + c];
    }
    if constexpr (S == 1) {
        if (quads && i0 + 3 < plane) {
            *reinterpret_cast<f32x4*>(out + i0) = sum;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (i0 + c < plane) out[i0 + c] = sum[c];
        }
        return;
    }
    red[g * Q + q] = sum;
    __syncthreads();
    if (g == 0) {
        f32x4 t = red[q];
#pragma unroll
        for (int k = 1; k < S; ++k) t += red[k * Q + q];
        if (quads && i0 + 3 < plane) {
            *reinterpret_cast<f32x4*>(out + i0) = t;
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (i0 + c < plane) out[i0 + c] = t[c];
        }
    }
}

// Split groups of av_pass2_combine for nsplit splits over `plane` outputs:
// the smallest power of two, at most 64, that leaves each group at most four
// splits, starting from 8 (more threads for small outputs), or from 1 when
// one thread per quad already makes at least 512 workgroups (the large batch
// with two splits: 512 workgroups of single threads adding two quads, where
// eight groups left six of every eight threads idle).
inline int combine_groups(int nsplit, int64_t plane) {
    int S = plane >= int64_t{512} * kThreads * 4 ? 1 : 8;
    while (S < 64 && S * 4 < nsplit) S *= 2;
    return S;
}

// Fused softmax, several splits: split s left the unnormalised sum
// part[s][b][q][d] = sum_c exp(s_c - m_s) V[c][d] over its rows and stats[s][b][q] =
// (m_s, l_s), its maximum score and weight sum. With M = max_s m_s and
// f_s = exp(m_s - M) (computed as exp2((m_s - M) log2 e)),
//   out[b][q][d] = sum_s f_s part[s][b][q][d] / sum_s f_s l_s.
// A split with m_s = -inf (all of its scores -inf) adds nothing; a row whose
// scores are all -inf gives 0 / 0. Two kernels, each summing in a fixed order:
//  * few splits (nsplit <= kCombineBatch): one thread per 4 outputs of a row,
//    every split loaded at once, summed in increasing s;
//  * more: one workgroup per (b, q), 8 split groups x 32 quad lanes, each group
//    summing its contiguous split range in increasing order, then the groups in
//    order (the association of av_pass2_combine). A group's loads run in
//    batches of kCombineBatch independent splits; the first batch is in flight
//    while the workgroup finds M.
constexpr int kCombineBatch = 8;

// Outputs d .. d + 3 of a D-long row (zeros past D). The address is clamped
// into the row and the value masked afterwards, so the load never sits behind
// a branch (a branch around each load makes the compiler wait for every load
// before the next). QUADS: D % 4 == 0 and the row 16-byte aligned.
template <bool QUADS>
__device__ inline f32x4 load_quad(const float* row, int d, int D) {
    f32x4 v;
    if constexpr (QUADS) {
        v = *reinterpret_cast<const f32x4*>(row + min(d, D - 4));
        if (d >= D) v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = row[min(d + c, D - 1)];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if (d + c >= D) v[c] = 0.0f;
    }
    return v;
}

__device__ inline float combine_factor(float ms, float M) {
    return ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((ms - M) * kLog2e);
}

// Splits sb .. sb + kCombineBatch - 1 (those below s1) of row bq at d, loaded
// all at once: statistics as (m, l) pairs and partial quads. Splits at or past
// s1 read split s1 - 1 and are masked to (-inf, 0) and zeros.
template <bool QUADS>
__device__ inline void load_batch(const float2* st2, const float* part, int64_t nbq, int64_t bq, int D, int sb,
                                  int s1, int d, float2 (&ml)[kCombineBatch], f32x4 (&pv)[kCombineBatch]) {
    const int64_t pstride = nbq * D;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
        const int s = min(sb + k, s1 - 1);
        ml[k] = st2[s * nbq + bq];
        pv[k] = load_quad<QUADS>(part + s * pstride + bq * D, d, D);
    }
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k)
        if (sb + k >= s1) {
            ml[k] = float2{-INFINITY, 0.0f};
            pv[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
}

template <bool QUADS>
__global__ __launch_bounds__(kThreads) void av_pass2_softmax_combine_few(const float* __restrict__ part,
                                                                         const float* __restrict__ stats,
                                                                         float* __restrict__ out, int32_t D,
                                                                         int64_t nbq, int32_t nsplit) {
    const int qpr = (D + 3) / 4;                     // quads per row
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (gid >= nbq * qpr) return;
    const int64_t bq = gid / qpr;
    const int d = static_cast<int>(gid - bq * qpr) * 4;
    float2 ml[kCombineBatch];
    f32x4 pv[kCombineBatch];
    load_batch<QUADS>(reinterpret_cast<const float2*>(stats), part, nbq, bq, D, 0, nsplit, d, ml, pv);
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) M = fmaxf(M, ml[k].x);
    f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
        const float f = combine_factor(ml[k].x, M);
        den += f * ml[k].y;
        num += f * pv[k];
    }
    float* const ob = out + bq * D;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (d + c < D) ob[d + c] = num[c] / den;
}

template <bool QUADS>
__global__ __launch_bounds__(kThreads) void av_pass2_softmax_combine(const float* __restrict__ part,
                                                                     const float* __restrict__ stats,
                                                                     float* __restrict__ out, int32_t D,
                                                                     int64_t nbq, int32_t nsplit) {
    constexpr int kQL = kThreads / kSplitGroups;     // quad lanes per split group
    constexpr int kB = kCombineBatch;
    __shared__ float s_max[kWaves];
    __shared__ float s_den[kSplitGroups];
    __shared__ f32x4 s_num[kSplitGroups][kQL];
    const int64_t bq = blockIdx.x;
    const int tid = threadIdx.x;
    const float2* const st2 = reinterpret_cast<const float2*>(stats);
    const int sg = tid / kQL, ql = tid % kQL;
    // nsplit > kCombineBatch >= ... so every group holds at least one split.
    const int s0 = static_cast<int>((static_cast<int64_t>(nsplit) * sg) / kSplitGroups);
    const int s1 = static_cast<int>((static_cast<int64_t>(nsplit) * (sg + 1)) / kSplitGroups);
    // This group's first batch at d = 4 ql: in flight while M is found.
    float2 ml[kB];
    f32x4 pv[kB];
    load_batch<QUADS>(st2, part, nbq, bq, D, s0, s1, 4 * ql, ml, pv);
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kB; ++k) m = fmaxf(m, ml[k].x);
    for (int s = s0 + kB; s < s1; ++s) m = fmaxf(m, st2[s * nbq + bq].x);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) s_max[tid >> 6] = m;
    __syncthreads();
    float M = s_max[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_max[w]);
    float* const ob = out + bq * D;
    for (int d0 = 0; d0 < D; d0 += 4 * kQL) {       // uniform trip count: barriers inside
        const int d = d0 + 4 * ql;
        f32x4 num = {0.0f, 0.0f, 0.0f, 0.0f};
        float den = 0.0f;
        for (int sb = s0; sb < s1; sb += kB) {
            if (d0 > 0 || sb > s0) load_batch<QUADS>(st2, part, nbq, bq, D, sb, s1, d, ml, pv);
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                const float f = combine_factor(ml[k].x, M);
                den += f * ml[k].y;
                num += f * pv[k];
            }
        }
        s_num[sg][ql] = num;
        if (ql == 0) s_den[sg] = den;
        __syncthreads();
        if (sg == 0) {
            f32x4 t = s_num[0][ql];
            float dn = s_den[0];
#pragma unroll
            for (int k = 1; k < kSplitGroups; ++k) {
                t += s_num[k][ql];
                dn += s_den[k];
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (d + c < D) ob[d + c] = t[c] / dn;
        }
        __syncthreads();
    }
}

}  // namespace gqa_av
