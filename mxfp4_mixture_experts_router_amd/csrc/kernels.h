// Host-side launchers of the gfx950 kernels (internal to libmoe_mxfp4.so).
// Each returns hipSuccess or the launch error; none synchronises.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Events that the next kernel launch of this thread records around the kernel itself (start
// and end of its execution, from the dispatch); both null outside the timed forward call.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
inline LaunchEvents &launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}

// Every launcher launches through this macro (one kernel per launcher call).
#define MOE_LAUNCH(kernel, grid, block, shmem, stream, ...)                                   \
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ::moe::launch_events().start,   \
                          ::moe::launch_events().stop, 0, __VA_ARGS__)

// Token count up to which the forward pass takes the decode path (per-expert work found
// inside the expert kernels, no sorted permutation in memory).
constexpr int64_t kDecodeMaxT = 64;
// Largest H and I the decode kernels take (their scale rows are staged in LDS, 128 bytes per
// row); larger shapes take the grouped path at any token count.
constexpr int kDecodeMaxK = 4096;

inline bool use_decode_path(int64_t T, int H, int I) {
    return T <= kDecodeMaxT && H <= kDecodeMaxK && I <= kDecodeMaxK;
}

struct Dims {
    int64_t T;
    int H, I, E, k;
    float alpha, limit;
};

// Router logits only (double [T, E]); for few tokens, where the top-k runs in the
// up-projection. Needs H <= 6144. Also writes x as an mx8 matrix (T rows of H, mx_mfma.h).
// With gamma != nullptr the router and the mx8 rows take the RMSNorm of x (rms.h) instead.
hipError_t launch_logits(const Dims &d, const uint16_t *x, const uint16_t *gamma, double eps,
                         const uint16_t *router_w, const uint16_t *router_b, double *logits, uint8_t *x8,
                         hipStream_t s);

// Whether launch_route can normalize the token rows itself (gamma != nullptr): the
// one-workgroup-per-token router (T <= kDecodeMaxT, H <= 3584).
inline bool route_normalizes(const Dims &d) { return d.T <= kDecodeMaxT && d.H <= 3584; }

// Router, top-k and softmax; with x8 != nullptr (T <= kDecodeMaxT) also writes x as an mx8
// matrix. With gamma != nullptr (only where route_normalizes) both take the RMSNorm of x.
// Above kDecodeMaxT tokens, when there are fewer 16-token groups than kRouteSplitCUs and
// E >= 64, the router sums slices of H in route_split(d) blocks per group into `part`
// (route_part_doubles(d) doubles of workspace), then a second kernel adds the slices, the bias
// and selects; otherwise (and then `part` may be null) one kernel does everything.
constexpr int kRouteSplitCUs = 256;
int route_split(const Dims &d);
int64_t route_part_doubles(const Dims &d);
hipError_t launch_route(const Dims &d, const uint16_t *x, const uint16_t *gamma, double eps,
                        const uint16_t *router_w, const uint16_t *router_b, int32_t *topk_idx, float *topk_w,
                        float *logits, uint8_t *x8, hipStream_t s, double *part = nullptr);

// hist (optional): workspace of permute_hist_ints(T k, E) ints; with it the permutation runs
// on many workgroups (a histogram pass, above kPermuteDirectBlocks blocks of 256 pairs a scan
// pass, then a scatter pass), without it on one. All give the same result.
constexpr int kPermuteDirectBlocks = 64;
int64_t permute_hist_ints(int64_t N, int E);
hipError_t launch_permute(const Dims &d, const int32_t *topk_idx, const float *topk_w,
                          int32_t *offsets, int32_t *sorted_token, float *sorted_w,
                          int32_t *slot_row, hipStream_t s, int32_t *hist = nullptr);

// up (prefill): h[r] = swiglu(x[sorted_token[r]] . Wgu[e]^T + bgu[e]) for the sorted rows r of
// every expert e, from the mx8 matrix x8 (T rows of H) into the mx8 matrix h8 (T k rows of I).
hipError_t launch_up_grouped(const Dims &d, const uint8_t *x8, const uint8_t *gu_blocks,
                             const uint8_t *gu_scales, const uint16_t *gu_bias,
                             const int32_t *offsets, const int32_t *sorted_token,
                             uint8_t *h8, hipStream_t s);

// down (prefill): o[r] = sorted_w[r] * (h[r] . Wdn[e]^T + bdn[e]) (fp32 [T k, H]) from h8.
hipError_t launch_down_grouped(const Dims &d, const uint8_t *h8, const uint8_t *dn_blocks,
                               const uint8_t *dn_scales, const uint16_t *dn_bias,
                               const int32_t *offsets, const float *sorted_w, float *o,
                               hipStream_t s);

// combine (prefill): y[t, :] = bf16(sum_j o[slot_row[t*k + j], :] (+ residual[t, :])), slot order.
hipError_t launch_combine(const Dims &d, const float *o, const int32_t *slot_row,
                          const uint16_t *residual, uint16_t *y, hipStream_t s);

// Decode path (T <= kDecodeMaxT). Below kStreamMinT tokens: router logits (launch_logits),
// then an up-projection that also takes the top-k, then a down-projection that also adds
// the k slots; from kStreamMinT tokens: launch_route, the weight-streaming projections and
// a combine.
constexpr int64_t kStreamMinT = 4;

// up (T < kStreamMinT): h[t*k + j, :] = w[t, j] * swiglu(x[t] . Wgu[e_tj]^T + bgu[e_tj]) as the
// mx8 matrix h8 of 2 T k rows of I (row 2n + half: one 16-value half of every MX block of
// h[n], zeros in the other), from the mx8 matrix x8 (T rows of H). Every block computes the
// top-k + softmax of `logits` (double [T, E]) itself; block 0 writes it to topk_idx / topk_w.
hipError_t launch_up_decode(const Dims &d, const uint8_t *x8, const uint8_t *gu_blocks,
                            const uint8_t *gu_scales, const uint16_t *gu_bias, const double *logits,
                            int32_t *topk_idx, float *topk_w, uint8_t *h8, hipStream_t s);
// down (T < kStreamMinT): y[t, :] = bf16(sum_j h[t*k + j] . Wdn[e_tj]^T + w[t, j] * bdn[e_tj]
// (+ residual[t, :])).
hipError_t launch_down_decode(const Dims &d, const uint8_t *h8, const uint8_t *dn_blocks,
                              const uint8_t *dn_scales, const uint16_t *dn_bias, int32_t *topk_idx,
                              float *topk_w, const uint16_t *residual, uint16_t *y, hipStream_t s);
// y[t, :] = bf16(sum_{j < k} part[t*k + j, :] (+ residual[t, :])), slot order.
hipError_t launch_combine_decode(const Dims &d, const float *part, const uint16_t *residual, uint16_t *y,
                                 hipStream_t s);

// Batched decode (kStreamMinT <= T <= kDecodeMaxT): the routed experts' weights streamed
// once, routing (topk_idx / topk_w) from launch_route.
// up: h[n, :] = swiglu(x[t] . Wgu[e_n]^T + bgu[e_n]) for every pair n = t*k + j, as the plain
// mx8 matrix h8 of T k rows of I.
hipError_t launch_up_stream(const Dims &d, const uint8_t *x8, const uint8_t *gu_blocks, const uint8_t *gu_scales,
                            const uint16_t *gu_bias, const int32_t *topk_idx, uint8_t *h8, hipStream_t s);
// down: part[n, :] = w[n] * (h[n] . Wdn[e_n]^T + bdn[e_n]) (fp32 [T k, H]); launch_combine_decode
// then forms y.
hipError_t launch_down_stream(const Dims &d, const uint8_t *h8, const uint8_t *dn_blocks, const uint8_t *dn_scales,
                              const uint16_t *dn_bias, const int32_t *topk_idx, const float *topk_w, float *part,
                              hipStream_t s);

// The expert GEMMs on a bf16 bank (launch_dequant of the packed bank), grouped over the
// sorted rows of launch_permute, on the bf16 MFMA.
// up: h[r, :] = bf16(swiglu(x[tok(r)] . Wgu[e]^T + bgu[e])) (bf16 [T k, I]); gu_w [E, 2I, H].
hipError_t launch_up_bank(const Dims &d, const uint16_t *x, const uint16_t *gu_w, const uint16_t *gu_bias,
                          const int32_t *offsets, const int32_t *sorted_token, uint16_t *h, hipStream_t s);
// down: o[r, :] = sorted_w[r] * (h[r] . Wdn[e]^T + bdn[e]) (fp32 [T k, H]); dn_w [E, H, I].
hipError_t launch_down_bank(const Dims &d, const uint16_t *h, const uint16_t *dn_w, const uint16_t *dn_bias,
                            const int32_t *offsets, const float *sorted_w, float *o, hipStream_t s);

// Pre-LN RMSNorm: xn[t, :] = bf16(x[t, :] * gamma / sqrt(mean_h x[t, h]^2 + eps)), in double,
// one rounding (nearest, ties to even). One workgroup per token; H a multiple of 8.
hipError_t launch_rmsnorm(const Dims &d, const uint16_t *x, const uint16_t *gamma, double eps, uint16_t *xn,
                          hipStream_t s);

// bf16 [rows, cols] -> mx8 matrix, or with h8 the grouped down GEMM's h8 layout (group-major
// scales; both in mx_mfma.h).
hipError_t launch_quantize(const uint16_t *x, int64_t rows, int cols, uint8_t *q8, bool h8, hipStream_t s);

hipError_t launch_dequant(const uint8_t *blocks, const uint8_t *scales, int64_t rows, int cols,
                          uint16_t *out, hipStream_t s);

// Shader-clock probe (benchmark context): workgroup b writes its shader cycles and its 100 MHz
// ticks over a fixed ALU chain to out[2b], out[2b + 1].
hipError_t launch_clock_probe(uint64_t *out, int blocks, int iters, hipStream_t s);

}  // namespace moe
