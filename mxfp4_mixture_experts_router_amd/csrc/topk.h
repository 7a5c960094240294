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

// lg[0..E) (double, in LDS: every lane reads all E of them):
// each lane ranks its candidates e = lane + 64c against all logits on the key (logit
// descending, index ascending); the candidate of rank j < k is slot j. The slot's softmax
// weight exp(l_j - l_max) / sum_i exp(l_i - l_max) is summed in slot order. Lane-parallel:
// one exp per selected candidate. s_ex: 8 doubles of scratch visible to the wavefront (LDS).
// Slot j goes to idx_out[j] / w_out[j] and, when given, idx_out2[j] / w_out2[j]; logits_out
// (optional) receives every logit rounded to fp32.
__device__ inline void topk_softmax_wave(const double *lg, int E, int k, int lane, int32_t *idx_out,
                                         float *w_out, int32_t *idx_out2, float *w_out2,
                                         float *logits_out, double *s_ex) {
    double v[kMaxE / kWave];
    int rank[kMaxE / kWave];
#pragma unroll
    for (int c = 0; c < kMaxE / kWave; ++c) {
        const int e = lane + kWave * c;
        v[c] = e < E ? lg[e] : 0.0;
        rank[c] = 0;
        if (logits_out && e < E) logits_out[e] = static_cast<float>(v[c]);
    }
    for (int f = 0; f < E; ++f) {
        const double lf = lg[f];
#pragma unroll
        for (int c = 0; c < kMaxE / kWave; ++c) {
            const int e = lane + kWave * c;
            rank[c] += (lf > v[c] || (lf == v[c] && f < e)) ? 1 : 0;
        }
    }
    // the largest logit (rank 0) is owned by exactly one lane
    double lmax = 0.0;
#pragma unroll
    for (int c = 0; c < kMaxE / kWave; ++c)
        if (lane + kWave * c < E && rank[c] == 0) s_ex[0] = v[c];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    lmax = s_ex[0];
    __builtin_amdgcn_wave_barrier();
    double ex[kMaxE / kWave];
#pragma unroll
    for (int c = 0; c < kMaxE / kWave; ++c) {
        const bool sel = lane + kWave * c < E && rank[c] < k;
        ex[c] = sel ? exp(v[c] - lmax) : 0.0;
        if (sel) s_ex[rank[c]] = ex[c];
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += s_ex[j];
#pragma unroll
    for (int c = 0; c < kMaxE / kWave; ++c) {
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

}  // namespace moe
