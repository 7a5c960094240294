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

#include <math.h>

namespace moe {
namespace {

constexpr int kMaxE = 256;

// Block = NW wavefronts handling TPB consecutive tokens. (token, expert-pair) work items
// are spread over the wavefronts; each lane sums h = 8*lane + 512*i .. +8, then the wave
// reduces with a fixed butterfly.
template <int NW, int TPB>
__global__ __launch_bounds__(NW * 64) void k_route(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const uint16_t *__restrict__ br, int64_t T, int H, int E, int k,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ logits_out) {
    __shared__ double lg[TPB][kMaxE];
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
            const uint4 av = *reinterpret_cast<const uint4 *>(w0 + h);
            const uint4 bv = *reinterpret_cast<const uint4 *>(w1 + h);
            const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
            const uint32_t as[4] = {av.x, av.y, av.z, av.w};
            const uint32_t bs[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double xl = __uint_as_float(xs[q] << 16), xh = __uint_as_float(xs[q] & 0xffff0000u);
                const double al = __uint_as_float(as[q] << 16), ah = __uint_as_float(as[q] & 0xffff0000u);
                const double bl = __uint_as_float(bs[q] << 16), bh = __uint_as_float(bs[q] & 0xffff0000u);
                acc0 = fma(xl, al, acc0);
                acc0 = fma(xh, ah, acc0);
                acc1 = fma(xl, bl, acc1);
                acc1 = fma(xh, bh, acc1);
            }
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

    // Top-k: one wavefront per token. Each lane holds candidates e = lane + 64*c; k rounds
    // of a wave-wide arg-max on the key (logit descending, index ascending).
    for (int tt = wave; tt < TPB; tt += NW) {
        const int64_t t = t0 + tt;
        if (t >= T) continue;
        double v[kMaxE / kWave];
        bool taken[kMaxE / kWave];
#pragma unroll
        for (int c = 0; c < kMaxE / kWave; ++c) {
            const int e = lane + kWave * c;
            v[c] = e < E ? lg[tt][e] : -INFINITY;
            taken[c] = e >= E;
            if (logits_out && e < E) logits_out[t * E + e] = static_cast<float>(v[c]);
        }
        double sv[8];
        int se[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sv[j] = -INFINITY;
            se[j] = 0;
            if (j < k) {
                double bv = -INFINITY;
                int be = 0x7fffffff;
#pragma unroll
                for (int c = 0; c < kMaxE / kWave; ++c) {
                    const int e = lane + kWave * c;
                    if (!taken[c] && (be == 0x7fffffff || v[c] > bv || (v[c] == bv && e < be))) {
                        bv = v[c];
                        be = e;
                    }
                }
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) {
                    const double ov = __shfl_xor(bv, off);
                    const int oe = __shfl_xor(be, off);
                    if (oe != 0x7fffffff && (be == 0x7fffffff || ov > bv || (ov == bv && oe < be))) {
                        bv = ov;
                        be = oe;
                    }
                }
                sv[j] = bv;
                se[j] = be;
#pragma unroll
                for (int c = 0; c < kMaxE / kWave; ++c)
                    if (be == lane + kWave * c) taken[c] = true;
            }
        }
        // softmax over the k selected logits (sv[0] is the largest), in selection order
        double den = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (j < k) den += exp(sv[j] - sv[0]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < k && lane == j) {
                topk_idx[t * k + j] = se[j];
                topk_w[t * k + j] = static_cast<float>(exp(sv[j] - sv[0]) / den);
            }
        }
    }
}

}  // namespace

hipError_t launch_route(const Dims &d, const uint16_t *x, const uint16_t *router_w,
                        const uint16_t *router_b, int32_t *topk_idx, float *topk_w,
                        float *logits, hipStream_t s) {
    if (d.T <= 0) return hipSuccess;
    if (d.T <= 16) {
        // latency path: one token per block, 16 wavefronts share its E dot products
        hipLaunchKernelGGL((k_route<16, 1>), dim3(static_cast<unsigned>(d.T)), dim3(16 * 64), 0, s,
                           x, router_w, router_b, d.T, d.H, d.E, d.k, topk_idx, topk_w, logits);
    } else {
        const int64_t blocks = (d.T + 3) / 4;
        hipLaunchKernelGGL((k_route<4, 4>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                           x, router_w, router_b, d.T, d.H, d.E, d.k, topk_idx, topk_w, logits);
    }
    return hipGetLastError();
}

}  // namespace moe
