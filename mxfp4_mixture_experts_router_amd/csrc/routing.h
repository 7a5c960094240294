// Routing lookups shared by the few-token kernels: which expert a block's slot stands for,
// and which routed (token, slot) pairs went to it.
#pragma once
#include "device_common.h"

namespace moe {

constexpr int kMaxRows = 64;          // pairs of one expert at most: an expert is chosen at most once per token

// The slot-th routed expert in increasing index order (-1 if fewer), computed by every
// thread from the bitmap.
__device__ inline int expert_of_slot(const uint32_t *bitmap, int slot) {
    int rem = slot;
#pragma unroll
    for (int w = 0; w < kMaxE / 32; ++w) {
        uint32_t bits = bitmap[w];
        const int c = __popc(bits);
        if (rem < c) {
            for (int q = 0; q < rem; ++q) bits &= bits - 1u;
            return 32 * w + __ffs(bits) - 1;
        }
        rem -= c;
    }
    return -1;
}

// Routed pairs n = t*k + j of expert e in increasing n, by one wavefront (caller syncs);
// returns their number (the same in every lane).
__device__ inline int rows_of_expert(const int *s_idx, int N, int e, int *s_rows, int *s_nrows) {
    const int lane = threadIdx.x % kWave;
    int cnt = 0;
    for (int base = 0; base < N; base += kWave) {
        const int n = base + lane;
        const bool hit = n < N && s_idx[n] == e;
        const uint64_t m = __ballot(hit);
        const int pos = cnt + __popcll(m & lanemask_lt());
        if (hit && pos < kMaxRows) s_rows[pos] = n;
        cnt += __popcll(m);
    }
    if (lane == 0) *s_nrows = cnt < kMaxRows ? cnt : kMaxRows;
    return cnt < kMaxRows ? cnt : kMaxRows;
}

// Lanes of the wavefront whose expert equals this lane's, for experts below 2^BITS (one
// ballot per bit; E <= 256 needs at most eight).
template <int BITS = 8>
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool valid) {
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

}  // namespace moe
