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
#include "routing.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBatch = 16;   // rounds of 64 pairs whose loads are issued together
constexpr int kStageCap = 16384;   // pairs whose sorted rows fit the LDS staging area

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

// Wavefront w owns the contiguous pairs [w * per, (w + 1) * per) and walks them 64 at a
// time twice: first counting its pairs per expert, then, after the block has turned the
// counts into each wavefront's starting position per expert, scattering them. Within a
// round the pairs of one expert are ranked by lane (ballot match over the BITS bits an
// expert index can have), so the order is by pair index throughout.
template <int BITS>
__global__ __launch_bounds__(kThreads) void k_permute(
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w, int32_t N, int E,
    int k, int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_token,
    float *__restrict__ sorted_w, int32_t *__restrict__ slot_row) {
    __shared__ int wcnt[kWaves][kMaxE];   // per-wavefront counts, then starting positions
    __shared__ int32_t st_tok[kStageCap];  // sorted rows staged in LDS (N <= kStageCap), so that
    __shared__ float st_w[kStageCap];      // the scattered writes stay on chip
    __shared__ int cnt[kMaxE];
    __shared__ int cursor[kMaxE + 1];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int per = ((N + kWaves - 1) / kWaves + kWave - 1) & ~(kWave - 1);
    const bool staged = N <= kStageCap;
    const int n_begin = wave * per;
    const int n_end = min(N, n_begin + per);

    for (int e = lane; e < E; e += kWave) wcnt[wave][e] = 0;
    __builtin_amdgcn_wave_barrier();
    // the expert indices of up to kBatch rounds are loaded at once (their latency overlaps)
    for (int nb = n_begin; nb < n_end; nb += kBatch * kWave) {
        int eb[kBatch];
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
            const int n = nb + r * kWave + lane;
            eb[r] = n < n_end ? topk_idx[n] : -1;
        }
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
            const int e = eb[r];
            const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
            const uint64_t peers = same_expert_lanes<BITS>(e, valid);
            if (valid && (peers & lanemask_lt()) == 0) wcnt[wave][e] += __popcll(peers);
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads) {
        int total = 0;
        for (int w = 0; w < kWaves; ++w) total += wcnt[w][e];
        cnt[e] = total;
    }
    __syncthreads();
    if (wave == 0) wave_exclusive_scan(cnt, cursor, E, lane);
    __syncthreads();
    for (int e = tid; e <= E; e += kThreads) offsets[e] = cursor[e];
    for (int e = tid; e < E; e += kThreads) {
        int run = cursor[e];
        for (int w = 0; w < kWaves; ++w) {
            const int c = wcnt[w][e];
            wcnt[w][e] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int nb = n_begin; nb < n_end; nb += kBatch * kWave) {
        int eb[kBatch];
        float wb[kBatch];
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
            const int n = nb + r * kWave + lane;
            eb[r] = n < n_end ? topk_idx[n] : -1;
            wb[r] = n < n_end ? topk_w[n] : 0.f;
        }
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
            const int n = nb + r * kWave + lane;
            const int e = eb[r];
            const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
            const uint64_t peers = same_expert_lanes<BITS>(e, valid);
            const int base = valid ? wcnt[wave][e] : 0;
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                const int pos = base + __popcll(peers & lanemask_lt());
                if (staged) {
                    st_tok[pos] = n / k;
                    st_w[pos] = wb[r];
                } else {
                    sorted_token[pos] = n / k;
                    sorted_w[pos] = wb[r];
                }
                slot_row[n] = pos;
                if ((peers & lanemask_lt()) == 0) wcnt[wave][e] = base + __popcll(peers);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    if (staged) {
        __syncthreads();
        for (int i = tid; i < N; i += kThreads) {
            sorted_token[i] = st_tok[i];
            sorted_w[i] = st_w[i];
        }
    }
}

// The same permutation by many workgroups, for the forward passes (which have workspace for
// the per-block histograms). Block b owns pairs [b P, (b + 1) P), one per thread.
// k_permute_count writes hist(e, b), the number of block b's pairs routed to expert e.
// k_permute_scatter then gives pair n (expert e, block b, wavefront w, lane l) the position
//   offsets[e] + sum_{b' < b} hist(e, b') + (pairs of e in wavefronts < w of block b)
//              + (pairs of e in lanes < l of wavefront w),
// the count of earlier pairs routed to e: the same stable order as k_permute.
// Up to kPermuteDirectBlocks blocks the histogram is block-major (hist[b][e]) and every
// scatter block sums it itself (nblk E reads per block, so the total grows with nblk^2);
// above that it is expert-major (hist[e][b]), k_permute_scan first turns each expert's row
// into its exclusive prefix sums and its total, and a scatter block reads only the E entries
// of its own column.
constexpr int kPT = 256;   // threads (and pairs) per block
constexpr int kPW = kPT / kWave;

template <int BITS>
__global__ __launch_bounds__(kPT) void k_permute_count(const int32_t *__restrict__ topk_idx, int32_t N, int E,
                                                       int32_t *__restrict__ hist) {
    __shared__ int cnt[kMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kPT) cnt[e] = 0;
    __syncthreads();
    const int n = blockIdx.x * kPT + tid;
    const int e = n < N ? topk_idx[n] : -1;
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    const uint64_t peers = same_expert_lanes<BITS>(e, valid);
    if (valid && (peers & lanemask_lt()) == 0) atomicAdd(&cnt[e], __popcll(peers));
    __syncthreads();
    // expert-major for the scan pass; block-major otherwise, so that the direct sums' adjacent
    // lanes add into different experts' LDS counters
    const bool by_expert = gridDim.x > kPermuteDirectBlocks;
    for (int e2 = tid; e2 < E; e2 += kPT)
        hist[by_expert ? static_cast<int64_t>(e2) * gridDim.x + blockIdx.x
                       : static_cast<int64_t>(blockIdx.x) * E + e2] = cnt[e2];
}

// One workgroup per expert e: hist[e][b] becomes sum_{b' < b} hist[e][b'] (in place) and
// tot[e] the row's total, scanning kScanT entries at a time.
constexpr int kScanT = 1024;
__global__ __launch_bounds__(kScanT) void k_permute_scan(int32_t *__restrict__ hist, int nblk,
                                                         int32_t *__restrict__ tot) {
    __shared__ int wsum[kScanT / kWave];
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    int32_t *row = hist + static_cast<int64_t>(blockIdx.x) * nblk;
    int carry = 0;
    for (int base = 0; base < nblk; base += kScanT) {
        const int i = base + tid;
        const int v = i < nblk ? row[i] : 0;
        int incl = v;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        if (lane == kWave - 1) wsum[wave] = incl;
        __syncthreads();
        int before = 0, chunk = 0;
#pragma unroll
        for (int w = 0; w < kScanT / kWave; ++w) {
            const int c = wsum[w];
            before += w < wave ? c : 0;
            chunk += c;
        }
        if (i < nblk) row[i] = carry + before + incl - v;
        carry += chunk;
        __syncthreads();   // wsum is rewritten by the next chunk
    }
    if (tid == 0) tot[blockIdx.x] = carry;
}

template <int BITS, bool SCANNED>
__global__ __launch_bounds__(kPT) void k_permute_scatter(
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w, int32_t N, int E, int k,
    int nblk, const int32_t *__restrict__ hist, const int32_t *__restrict__ hist_tot, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_token, float *__restrict__ sorted_w, int32_t *__restrict__ slot_row) {
    __shared__ int tot[kMaxE];        // pairs per expert, all blocks
    __shared__ int before[kMaxE];     // pairs per expert in blocks < this one
    __shared__ int start[kMaxE + 1];  // exclusive scan of tot
    __shared__ int wc[kPW][kMaxE];    // pairs per expert in each wavefront of this block
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int b = blockIdx.x;
    for (int e = tid; e < E; e += kPT) {
        if (SCANNED) {
            tot[e] = hist_tot[e];
            before[e] = hist[static_cast<int64_t>(e) * nblk + b];
        } else {
            tot[e] = 0;
            before[e] = 0;
        }
    }
#pragma unroll
    for (int w = 0; w < kPW; ++w)
        for (int e = tid; e < E; e += kPT) wc[w][e] = 0;
    const int n = b * kPT + tid;
    const int e = n < N ? topk_idx[n] : -1;
    const float wt = n < N ? topk_w[n] : 0.f;
    __syncthreads();
    if (!SCANNED) {
        // column sums of hist[b][e] (integers: the order of the LDS atomics does not matter)
        const int total = nblk * E;
#pragma unroll 8
        for (int q = tid; q < total; q += kPT) {
            const int c = hist[q];
            const int i = q / E, ee = q - i * E;
            atomicAdd(&tot[ee], c);
            if (i < b) atomicAdd(&before[ee], c);
        }
    }
    const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
    const uint64_t peers = same_expert_lanes<BITS>(e, valid);
    if (valid && (peers & lanemask_lt()) == 0) wc[wave][e] = __popcll(peers);
    __syncthreads();
    if (wave == 0) wave_exclusive_scan(tot, start, E, lane);
    __syncthreads();
    if (b == 0)
        for (int e2 = tid; e2 <= E; e2 += kPT) offsets[e2] = start[e2];
    if (valid) {
        int pos = start[e] + before[e] + __popcll(peers & lanemask_lt());
        for (int w = 0; w < wave; ++w) pos += wc[w][e];
        sorted_token[pos] = n / k;
        sorted_w[pos] = wt;
        slot_row[n] = pos;
    }
}

}  // namespace

int64_t permute_hist_ints(int64_t N, int E) {
    const int64_t nblk = (N + kPT - 1) / kPT;
    return N > 0 ? (nblk + 1) * E : 0;
}

hipError_t launch_permute(const Dims &d, const int32_t *topk_idx, const float *topk_w,
                          int32_t *offsets, int32_t *sorted_token, float *sorted_w,
                          int32_t *slot_row, hipStream_t s, int32_t *hist) {
    const int32_t N = static_cast<int32_t>(d.T * d.k);
    const int nblk = static_cast<int>((static_cast<int64_t>(N) + kPT - 1) / kPT);
    if (hist != nullptr && N > 0) {
        // one stage, two or three launches: the count kernel records the stage's start event,
        // the scatter kernel its stop event
        int32_t *tot = hist + static_cast<int64_t>(nblk) * d.E;
        const LaunchEvents ev = launch_events();
#define MOE_PERMUTE_MB(B)                                                                                 \
    do {                                                                                                  \
        launch_events() = LaunchEvents{ev.start, nullptr};                                                \
        MOE_LAUNCH(k_permute_count<B>, dim3(nblk), dim3(kPT), 0, s, topk_idx, N, d.E, hist);              \
        launch_events() = LaunchEvents{};                                                                 \
        if (nblk > kPermuteDirectBlocks) {                                                                \
            MOE_LAUNCH(k_permute_scan, dim3(d.E), dim3(kScanT), 0, s, hist, nblk, tot);                   \
            launch_events() = LaunchEvents{nullptr, ev.stop};                                             \
            MOE_LAUNCH((k_permute_scatter<B, true>), dim3(nblk), dim3(kPT), 0, s, topk_idx, topk_w, N,    \
                       d.E, d.k, nblk, hist, tot, offsets, sorted_token, sorted_w, slot_row);             \
        } else {                                                                                          \
            launch_events() = LaunchEvents{nullptr, ev.stop};                                             \
            MOE_LAUNCH((k_permute_scatter<B, false>), dim3(nblk), dim3(kPT), 0, s, topk_idx, topk_w, N,   \
                       d.E, d.k, nblk, hist, tot, offsets, sorted_token, sorted_w, slot_row);             \
        }                                                                                                 \
        launch_events() = ev;                                                                             \
    } while (0)
        if (d.E <= 32) MOE_PERMUTE_MB(5);
        else if (d.E <= 64) MOE_PERMUTE_MB(6);
        else if (d.E <= 128) MOE_PERMUTE_MB(7);
        else MOE_PERMUTE_MB(8);
#undef MOE_PERMUTE_MB
        return hipGetLastError();
    }
#define MOE_PERMUTE(B) MOE_LAUNCH(k_permute<B>, dim3(1), dim3(kThreads), 0, s, topk_idx, topk_w, N, d.E, d.k, \
                                   offsets, sorted_token, sorted_w, slot_row)
    if (d.E <= 32) MOE_PERMUTE(5);
    else if (d.E <= 64) MOE_PERMUTE(6);
    else if (d.E <= 128) MOE_PERMUTE(7);
    else MOE_PERMUTE(8);
#undef MOE_PERMUTE
    return hipGetLastError();
}

}  // namespace moe
