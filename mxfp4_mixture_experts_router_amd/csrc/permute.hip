// Expert-sorted permutation of the routed (token, slot) pairs: histogram over experts,
// exclusive scan, stable scatter. The grouped GEMMs then see each expert's rows as one
// contiguous range (ZeroModels GPT-OSS page, "MXFP4 experts": only routed experts are
// evaluated; each expert's packed weights are streamed once per tile of its rows).
//
// One workgroup of 1024 threads. Integer work only, so the result is exact and
// deterministic: the position of pair n = t*k + j inside its expert's range is the number
// of earlier pairs (smaller n) routed to the same expert.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

// Exclusive scan of cnt[0..E) by one wavefront (E <= 256: four entries per lane).
__device__ void wave_exclusive_scan(const int *cnt, int *out, int E, int lane) {
    int v[4];
    int local = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int e = 4 * lane + c;
        v[c] = e < E ? cnt[e] : 0;
        local += v[c];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    int run = incl - local;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int e = 4 * lane + c;
        if (e < E) out[e] = run;
        run += v[c];
    }
    if (lane == kWave - 1) out[E] = incl;   // total
}

__global__ __launch_bounds__(kThreads) void k_permute(
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w, int32_t N, int E,
    int k, int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_token,
    float *__restrict__ sorted_w, int32_t *__restrict__ slot_row) {
    __shared__ int cnt[kMaxE];
    __shared__ int cursor[kMaxE + 1];
    __shared__ int wcnt[kWaves][kMaxE];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;

    for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
    __syncthreads();
    for (int n = tid; n < N; n += kThreads) {
        const int e = topk_idx[n];
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (wave == 0) wave_exclusive_scan(cnt, cursor, E, lane);
    __syncthreads();
    for (int e = tid; e <= E; e += kThreads) offsets[e] = cursor[e];

    for (int base = 0; base < N; base += kThreads) {
        for (int i = tid; i < kWaves * kMaxE; i += kThreads) (&wcnt[0][0])[i] = 0;
        const int n = base + tid;
        const int e = n < N ? topk_idx[n] : -1;
        const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
        __syncthreads();
        // group the wavefront's lanes by expert: peers = lanes holding the same expert
        uint64_t peers = 0;
        uint64_t rest = __ballot(valid);
        while (rest) {
            const int leader = __ffsll(static_cast<unsigned long long>(rest)) - 1;
            const int le = __shfl(e, leader);
            const uint64_t m = __ballot(valid && e == le);
            if (valid && e == le) peers = m;
            rest &= ~m;
        }
        const int rank = __popcll(peers & lanemask_lt());
        if (valid && rank == 0) wcnt[wave][e] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int pos = cursor[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
            sorted_token[pos] = n / k;
            sorted_w[pos] = topk_w[n];
            slot_row[n] = pos;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += kThreads) {
            int add = 0;
            for (int w = 0; w < kWaves; ++w) add += wcnt[w][ee];
            cursor[ee] += add;
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_permute(const Dims &d, const int32_t *topk_idx, const float *topk_w,
                          int32_t *offsets, int32_t *sorted_token, float *sorted_w,
                          int32_t *slot_row, hipStream_t s) {
    const int32_t N = static_cast<int32_t>(d.T * d.k);
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(kThreads), 0, s, topk_idx, topk_w, N, d.E, d.k,
                       offsets, sorted_token, sorted_w, slot_row);
    return hipGetLastError();
}

}  // namespace moe
