// Top-k selection and softmax of one token's router logits by one wavefront.
//
// ZeroModels GPT-OSS page, "Mixture-of-experts feed-forward": the router selects the top
// num_experts_per_tok experts and their softmax weights combine the expert outputs. Order:
// larger logit first; equal logits -> lower expert index first. The softmax runs over the
// k selected logits.
#pragma once

#include <math.h>

#include "device_common.h"

namespace moe {

constexpr int kTopkC = kMaxE / kWave;   // candidates per lane: expert e = lane + 64c
constexpr int kTopkScratch = kMaxE + 8; // LDS words (8 bytes) of scratch per wavefront

// Selection key of expert e with logit v: a 64-bit unsigned integer that orders by logit
// (larger first) and, among equal logits, by expert index (lower first). The upper 56 bits
// are the order-preserving image of the double (sign flipped for positives, all bits
// inverted for negatives; -0 and +0 coincide), the low 8 bits hold 255 - e. Logits that
// differ only in their 8 lowest mantissa bits (below 2^-44 relative, under the error of an
// fp64 dot product of this length) therefore count as equal and go to the lower index.
// Keys are distinct for distinct experts and nonzero.
__device__ __forceinline__ uint64_t select_key(double v, int e) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v + 0.0));   // -0 + 0 = +0
    const uint64_t ord = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
    return (ord & ~0xffull) | static_cast<uint64_t>(255 - e);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane));
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffffu), lane));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Rank of each candidate e = lane + 64c (NC candidates per lane in use): the number of
// experts whose key is larger. Keys are read from LDS eight at a time (four 16-byte reads
// in flight); entries past E are zero and never count.
template <int NC>
__device__ __forceinline__ void rank_keys(const uint64_t *s_key, const uint64_t (&key)[kTopkC], int E,
                                          int (&rank)[kTopkC]) {
    for (int f0 = 0; f0 < E; f0 += 8) {
        const ulonglong2 q0 = *reinterpret_cast<const ulonglong2 *>(s_key + f0);
        const ulonglong2 q1 = *reinterpret_cast<const ulonglong2 *>(s_key + f0 + 2);
        const ulonglong2 q2 = *reinterpret_cast<const ulonglong2 *>(s_key + f0 + 4);
        const ulonglong2 q3 = *reinterpret_cast<const ulonglong2 *>(s_key + f0 + 6);
        const uint64_t kf[8] = {q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int c = 0; c < NC; ++c) rank[c] += kf[j] > key[c] ? 1 : 0;
    }
}

// Top-k + softmax of one token. v[c] is the logit of expert e = lane + 64c (ignored for
// e >= E). Every candidate's rank on select_key (logit descending, index ascending) is
// counted against all E keys; the candidate of rank j < k is slot j. The slot's weight
// exp(l_j - l_max) / sum_i exp(l_i - l_max) is summed in slot order, one exp per selected
// candidate. Slot j goes to idx_out[j] / w_out[j] and, when given, idx_out2[j] / w_out2[j].
// k <= 8. scratch: kTopkScratch eight-byte LDS words private to the wavefront, 16-byte
// aligned. Called by all 64 lanes of the wavefront. C = ceil(E / 64) candidate slots per lane
// (a compile-time count, so that no work is spent on the unused ones).
template <int C>
__device__ inline void topk_softmax_nc(const double (&v)[kTopkC], int E, int k, int lane,
                                       int32_t *idx_out, float *w_out, int32_t *idx_out2,
                                       float *w_out2, uint64_t *scratch) {
    const int epad = (E + 7) & ~7;              // the rank loop reads keys up to here
    uint64_t key[kTopkC];
    int rank[kTopkC];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = lane + kWave * c;
        key[c] = e < E ? select_key(v[c], e) : 0ull;
        rank[c] = 0;
        if (e < epad) scratch[e] = key[c];
    }
    __builtin_amdgcn_wave_barrier();
    rank_keys<C>(scratch, key, E, rank);
    // the largest logit: the candidate of rank 0
    double lmax = 0.0;
#pragma unroll
    for (int c = C - 1; c >= 0; --c) {
        const uint64_t m = __ballot(lane + kWave * c < E && rank[c] == 0);
        if (m) lmax = readlane_f64(v[c], __ffsll(static_cast<long long>(m)) - 1);
    }
    double *s_ex = reinterpret_cast<double *>(scratch + kMaxE);
    double ex[kTopkC];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const bool sel = lane + kWave * c < E && rank[c] < k;
        ex[c] = sel ? exp(v[c] - lmax) : 0.0;
        if (sel) s_ex[rank[c]] = ex[c];
    }
    __builtin_amdgcn_wave_barrier();
    const double2 d0 = *reinterpret_cast<const double2 *>(s_ex);
    const double2 d1 = *reinterpret_cast<const double2 *>(s_ex + 2);
    const double2 d2 = *reinterpret_cast<const double2 *>(s_ex + 4);
    const double2 d3 = *reinterpret_cast<const double2 *>(s_ex + 6);
    const double exs[8] = {d0.x, d0.y, d1.x, d1.y, d2.x, d2.y, d3.x, d3.y};
    double den = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < k) den += exs[j];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = lane + kWave * c;
        if (e < E && rank[c] < k) {
            const int j = rank[c];
            const float wj = static_cast<float>(ex[c] / den);
            idx_out[j] = e;
            w_out[j] = wj;
            if (idx_out2) {
                idx_out2[j] = e;
                w_out2[j] = wj;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
}

__device__ inline void topk_softmax_values(const double (&v)[kTopkC], int E, int k, int lane,
                                           int32_t *idx_out, float *w_out, int32_t *idx_out2,
                                           float *w_out2, uint64_t *scratch) {
    switch ((E + kWave - 1) / kWave) {
        case 1: topk_softmax_nc<1>(v, E, k, lane, idx_out, w_out, idx_out2, w_out2, scratch); break;
        case 2: topk_softmax_nc<2>(v, E, k, lane, idx_out, w_out, idx_out2, w_out2, scratch); break;
        case 3: topk_softmax_nc<3>(v, E, k, lane, idx_out, w_out, idx_out2, w_out2, scratch); break;
        default: topk_softmax_nc<4>(v, E, k, lane, idx_out, w_out, idx_out2, w_out2, scratch); break;
    }
}

// The same for logits lg[0..E) in memory (LDS or global); logits_out (optional) receives
// every logit rounded to fp32.
__device__ inline void topk_softmax_wave(const double *lg, int E, int k, int lane, int32_t *idx_out,
                                         float *w_out, int32_t *idx_out2, float *w_out2,
                                         float *logits_out, uint64_t *scratch) {
    double v[kTopkC];
#pragma unroll
    for (int c = 0; c < kTopkC; ++c) {
        const int e = lane + kWave * c;
        v[c] = e < E ? lg[e] : 0.0;
        if (logits_out && e < E) logits_out[e] = static_cast<float>(v[c]);
    }
    topk_softmax_values(v, E, k, lane, idx_out, w_out, idx_out2, w_out2, scratch);
}

}  // namespace moe
