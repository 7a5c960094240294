// Pre-LN RMSNorm of the layer input ("GPT-OSS MLX Implementation" README, "Architecture
// Details": RMSNorm with Pre-LN placement; ZeroModels GPT-OSS page, "API" table: norm_eps).
//   xn[t, h] = bf16(x[t, h] * r * gamma[h]),  r = 1 / sqrt(sum_h x[t, h]^2 / H + eps)
// in double (products left to right), rounded once to bf16 (nearest, ties to even). The
// squares of bf16 values are exact in double, so the sum carries only its own rounding.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// The bf16 nearest to v (ties to even): v keeps 8 significant bits, so with 2^(e-1) the
// leading bit of |v|, the result is rint(v * 2^(8 - e)) * 2^(e - 8), exact in float.
__device__ __forceinline__ uint16_t bf16_nearest(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int e;
    frexp(v, &e);
    const float f = static_cast<float>(ldexp(rint(ldexp(v, 8 - e)), e - 8));
    return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// One workgroup per token row; thread i takes the 8-element groups i, i + 256, ...
__global__ __launch_bounds__(kThreads) void k_rmsnorm(const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ gamma, int H, double eps,
                                                      uint16_t *__restrict__ xn) {
    __shared__ double s_part[kThreads / kWave];
    __shared__ double s_r;
    const int64_t t = blockIdx.x;
    const uint16_t *xr = x + t * H;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    double ss = 0.0;
    for (int h = 8 * tid; h < H; h += 8 * kThreads) {
        const uint4 u = *reinterpret_cast<const uint4 *>(xr + h);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double a = __uint_as_float(w[q] << 16), b = __uint_as_float(w[q] & 0xffff0000u);
            ss += a * a;
            ss += b * b;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) s_part[wave] = ss;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int w = 0; w < kThreads / kWave; ++w) tot += s_part[w];
        s_r = 1.0 / sqrt(tot / H + eps);
    }
    __syncthreads();
    const double r = s_r;
    uint16_t *out = xn + t * H;
    for (int h = 8 * tid; h < H; h += 8 * kThreads) {
        const uint4 u = *reinterpret_cast<const uint4 *>(xr + h);
        const uint4 gv = *reinterpret_cast<const uint4 *>(gamma + h);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double a = static_cast<double>(__uint_as_float(w[q] << 16)) * r *
                             static_cast<double>(__uint_as_float(gw[q] << 16));
            const double b = static_cast<double>(__uint_as_float(w[q] & 0xffff0000u)) * r *
                             static_cast<double>(__uint_as_float(gw[q] & 0xffff0000u));
            o[q] = bf16_nearest(a) | (static_cast<uint32_t>(bf16_nearest(b)) << 16);
        }
        *reinterpret_cast<uint4 *>(out + h) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace

hipError_t launch_rmsnorm(const Dims &d, const uint16_t *x, const uint16_t *gamma, double eps, uint16_t *xn,
                          hipStream_t s) {
    if (d.T <= 0) return hipSuccess;
    MOE_LAUNCH(k_rmsnorm, dim3(static_cast<unsigned>(d.T)), dim3(kThreads), 0, s, x, gamma, d.H, eps, xn);
    return hipGetLastError();
}

}  // namespace moe
