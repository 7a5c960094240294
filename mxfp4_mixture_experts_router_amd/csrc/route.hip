// Router: logits, top-k selection and softmax over the selected logits.
//
// ZeroModels GPT-OSS page, "Mixture-of-experts feed-forward": a top-num_experts_per_tok
// router selects experts whose softmax weights combine the per-expert outputs.
//
// Logits are accumulated in double precision. Every product of two bf16 values is exact
// in double, so the only error is the summation's (about 1e-13 relative for H = 2880);
// the integer decision (which k experts) therefore matches exact arithmetic unless two
// logits are closer than that, and equal logits (e.g. duplicated router rows, which take
// the identical summation sequence here) resolve to the lower expert index.
#include "device_common.h"
#include "kernels.h"
#include "mx_mfma.h"
#include "topk.h"

#include <math.h>

namespace moe {
namespace {


// Sum of the 8 exact bf16 x bf16 products held in two uint4 vectors, added to acc in order.
__device__ __forceinline__ double dot8(uint4 xv, uint4 wv, double acc) {
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
    const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc = fma(static_cast<double>(__uint_as_float(xs[q] << 16)),
                  static_cast<double>(__uint_as_float(ws[q] << 16)), acc);
        acc = fma(static_cast<double>(__uint_as_float(xs[q] & 0xffff0000u)),
                  static_cast<double>(__uint_as_float(ws[q] & 0xffff0000u)), acc);
    }
    return acc;
}

// Latency-oriented router for few tokens: one block (8 wavefronts) per token. The token
// row and the wave's four router rows are loaded with every load in flight at once (lane l
// covers h = 8l + 512i, i < NI, NI = ceil(H / 512)); wavefront w handles experts
// 4w .. 4w+3, then 32 + 4w .. and so on.
template <int NI>
__global__ __launch_bounds__(512) void k_route_token(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const uint16_t *__restrict__ br, int H, int E, int k, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, float *__restrict__ logits_out, uint8_t *__restrict__ x8, int T) {
    constexpr int kEPW = 4;
    __shared__ double lg[kMaxE];
    __shared__ __attribute__((aligned(16))) uint64_t s_tk[kTopkScratch];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t t = blockIdx.x;
    const uint16_t *xr = x + t * H;
    uint4 xv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int h = 8 * lane + 8 * kWave * i;
        xv[i] = h < H ? *reinterpret_cast<const uint4 *>(xr + h) : zero4();
    }
    for (int e0 = kEPW * wave; e0 < E; e0 += kEPW * 8) {
        uint4 a[kEPW][NI];
#pragma unroll
        for (int q = 0; q < kEPW; ++q) {
            const int e = e0 + q < E ? e0 + q : e0;
            const uint16_t *wrow = wr + static_cast<int64_t>(e) * H;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int h = 8 * lane + 8 * kWave * i;
                a[q][i] = h < H ? *reinterpret_cast<const uint4 *>(wrow + h) : zero4();
            }
        }
        double acc[kEPW];
#pragma unroll
        for (int q = 0; q < kEPW; ++q) {
            acc[q] = 0.0;
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[q] = dot8(xv[i], a[q][i], acc[q]);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
            for (int q = 0; q < kEPW; ++q) acc[q] += __shfl_xor(acc[q], off);
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < kEPW; ++q)
                if (e0 + q < E) lg[e0 + q] = acc[q] + static_cast<double>(bf16_to_f32(br[e0 + q]));
        }
    }
    __syncthreads();
    if (wave == 0)
        topk_softmax_wave(lg, E, k, lane, topk_idx + t * k, topk_w + t * k, nullptr, nullptr,
                          logits_out ? logits_out + t * E : nullptr, s_tk);
    if (x8 != nullptr) write_mx8_row(xr, H, x8, T, t);
}

// Logits only, for few tokens (the top-k then runs in the up-projection's prologue): block
// (expert pair, token); its 4 wavefronts split H (lane l of wavefront w covers
// h = 8l + 512(w + 4i)) and their partial sums are added in wavefront order.
//   logits[t, e] = sum_h x[t, h] * Wr[e, h] + br[e]     (double)
// One extra block per token (the last in x) writes the token as an mx8 row of x8 (T rows)
// for the expert GEMMs.
template <int NIQ>
__global__ __launch_bounds__(256) void k_logits(const uint16_t *__restrict__ x,
                                                const uint16_t *__restrict__ wr,
                                                const uint16_t *__restrict__ br, int H, int E,
                                                double *__restrict__ logits, uint8_t *__restrict__ x8, int T) {
    __shared__ double part[4][2];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t t = blockIdx.y;
    if (blockIdx.x == gridDim.x - 1) {   // the extra block: token t as an mx8 row
        write_mx8_row(x + t * H, H, x8, T, t);
        return;
    }
    const int e0 = 2 * blockIdx.x;
    const bool has2 = e0 + 1 < E;
    const uint16_t *xr = x + t * H;
    const uint16_t *w0 = wr + static_cast<int64_t>(e0) * H;
    const uint16_t *w1 = wr + static_cast<int64_t>(has2 ? e0 + 1 : e0) * H;
    uint4 xv[NIQ], a[NIQ], b[NIQ];
#pragma unroll
    for (int i = 0; i < NIQ; ++i) {
        const int h = 8 * lane + 8 * kWave * (wave + 4 * i);
        const bool ok = h < H;
        xv[i] = ok ? *reinterpret_cast<const uint4 *>(xr + h) : zero4();
        a[i] = ok ? *reinterpret_cast<const uint4 *>(w0 + h) : zero4();
        b[i] = ok ? *reinterpret_cast<const uint4 *>(w1 + h) : zero4();
    }
    double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
    for (int i = 0; i < NIQ; ++i) {
        acc0 = dot8(xv[i], a[i], acc0);
        acc1 = dot8(xv[i], b[i], acc1);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        acc0 += __shfl_xor(acc0, off);
        acc1 += __shfl_xor(acc1, off);
    }
    if (lane == 0) {
        part[wave][0] = acc0;
        part[wave][1] = acc1;
    }
    __syncthreads();
    if (threadIdx.x < 2 && (threadIdx.x == 0 || has2)) {
        const int q = threadIdx.x;
        const double v = ((part[0][q] + part[1][q]) + part[2][q]) + part[3][q];
        logits[t * E + e0 + q] = v + static_cast<double>(bf16_to_f32(br[e0 + q]));
    }
}

// Throughput router for many tokens: block = NW wavefronts handling TPB consecutive
// tokens; (token, expert-pair) work items are spread over the wavefronts.
template <int NW, int TPB>
__global__ __launch_bounds__(NW * 64) void k_route(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const uint16_t *__restrict__ br, int64_t T, int H, int E, int k,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ logits_out,
    uint8_t *__restrict__ x8) {
    __shared__ double lg[TPB][kMaxE];
    __shared__ __attribute__((aligned(16))) uint64_t s_tk[NW][kTopkScratch];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * TPB;
    const int egroups = (E + 1) / 2;

    for (int p = wave; p < TPB * egroups; p += NW) {
        const int tt = p / egroups;
        const int e0 = 2 * (p % egroups);
        const int64_t t = t0 + tt;
        if (t >= T) continue;
        const bool has2 = (e0 + 1) < E;
        const uint16_t *xr = x + t * H;
        const uint16_t *w0 = wr + static_cast<int64_t>(e0) * H;
        const uint16_t *w1 = wr + static_cast<int64_t>(has2 ? e0 + 1 : e0) * H;
        double acc0 = 0.0, acc1 = 0.0;
        for (int h = lane * 8; h < H; h += 8 * kWave) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xr + h);
            acc0 = dot8(xv, *reinterpret_cast<const uint4 *>(w0 + h), acc0);
            acc1 = dot8(xv, *reinterpret_cast<const uint4 *>(w1 + h), acc1);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            acc0 += __shfl_xor(acc0, off);
            acc1 += __shfl_xor(acc1, off);
        }
        if (lane == 0) {
            lg[tt][e0] = acc0 + static_cast<double>(bf16_to_f32(br[e0]));
            if (has2) lg[tt][e0 + 1] = acc1 + static_cast<double>(bf16_to_f32(br[e0 + 1]));
        }
    }
    __syncthreads();
    for (int tt = wave; tt < TPB; tt += NW) {
        const int64_t t = t0 + tt;
        if (t >= T) continue;
        topk_softmax_wave(lg[tt], E, k, lane, topk_idx + t * k, topk_w + t * k, nullptr, nullptr,
                          logits_out ? logits_out + t * E : nullptr, s_tk[wave]);
    }
    if (x8 != nullptr)
        for (int tt = 0; tt < TPB && t0 + tt < T; ++tt) write_mx8_row(x + (t0 + tt) * H, H, x8, T, t0 + tt);
}

template <int NI>
void launch_token(const Dims &d, const uint16_t *x, const uint16_t *w, const uint16_t *b,
                  int32_t *idx, float *wt, float *logits, uint8_t *x8, hipStream_t s) {
    hipLaunchKernelGGL((k_route_token<NI>), dim3(static_cast<unsigned>(d.T)), dim3(512), 0, s, x, w,
                       b, d.H, d.E, d.k, idx, wt, logits, x8, static_cast<int>(d.T));
}

}  // namespace

hipError_t launch_logits(const Dims &d, const uint16_t *x, const uint16_t *router_w,
                         const uint16_t *router_b, double *logits, uint8_t *x8, hipStream_t s) {
    if (d.T <= 0) return hipSuccess;
    const int niq = (d.H + 2047) / 2048;
    const dim3 grid(static_cast<unsigned>((d.E + 1) / 2 + 1), static_cast<unsigned>(d.T));
    switch (niq) {
        case 1: hipLaunchKernelGGL((k_logits<1>), grid, dim3(256), 0, s, x, router_w, router_b, d.H, d.E, logits, x8, static_cast<int>(d.T)); break;
        case 2: hipLaunchKernelGGL((k_logits<2>), grid, dim3(256), 0, s, x, router_w, router_b, d.H, d.E, logits, x8, static_cast<int>(d.T)); break;
        case 3: hipLaunchKernelGGL((k_logits<3>), grid, dim3(256), 0, s, x, router_w, router_b, d.H, d.E, logits, x8, static_cast<int>(d.T)); break;
        default: return hipErrorInvalidValue;   // H > 6144: the caller uses launch_route
    }
    return hipGetLastError();
}

hipError_t launch_route(const Dims &d, const uint16_t *x, const uint16_t *router_w,
                        const uint16_t *router_b, int32_t *topk_idx, float *topk_w,
                        float *logits, uint8_t *x8, hipStream_t s) {
    if (d.T <= 0) return hipSuccess;
    const int ni = (d.H + 511) / 512;
    if (d.T <= kDecodeMaxT && ni <= 7) {
        switch (ni) {
            case 1: launch_token<1>(d, x, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 2: launch_token<2>(d, x, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 3: launch_token<3>(d, x, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 4: launch_token<4>(d, x, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 5: launch_token<5>(d, x, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 6: launch_token<6>(d, x, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            default: launch_token<7>(d, x, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
        }
    } else {
        const int64_t blocks = (d.T + 3) / 4;
        hipLaunchKernelGGL((k_route<4, 4>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           x, router_w, router_b, d.T, d.H, d.E, d.k, topk_idx, topk_w, logits, x8);
    }
    return hipGetLastError();
}

}  // namespace moe
