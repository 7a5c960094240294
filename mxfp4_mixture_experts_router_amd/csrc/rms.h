// Pieces of the Pre-LN RMSNorm ("GPT-OSS MLX Implementation" README, "Architecture Details";
// ZeroModels GPT-OSS page, "API" table: norm_eps), shared by the standalone normalization
// kernel and the decode routers that normalize the token row they load anyway:
//   xn[h] = bf16(x[h] * r * gamma[h]),  r = 1 / sqrt(sum_h x[h]^2 / H + eps)
// in double, products left to right, one rounding to bf16 (nearest, ties to even).
#pragma once

#include <math.h>

#include "device_common.h"

namespace moe {

// The bf16 nearest to v (ties to even): with 2^(e-1) the leading bit of |v|, the bf16 keeps
// the bits down to 2^(e-8), so the result is rint(v * 2^(8 - e)) * 2^(e - 8), exact in float.
__device__ __forceinline__ uint16_t bf16_nearest(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int e;
    frexp(v, &e);
    const float f = static_cast<float>(ldexp(rint(ldexp(v, 8 - e)), e - 8));
    return static_cast<uint16_t>(__float_as_uint(f) >> 16);
}

// ss + the squares of the 8 bf16 values in u, added in element order (each square is exact).
__device__ __forceinline__ double sumsq8(const uint4 &u, double ss) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const double a = __uint_as_float(w[q] << 16), b = __uint_as_float(w[q] & 0xffff0000u);
        ss += a * a;
        ss += b * b;
    }
    return ss;
}

// Sum over the 64 lanes of a wavefront; every lane receives the same bits.
__device__ __forceinline__ double wave_sum(double v) { return wave_sum_f64(v); }

__device__ __forceinline__ double rms_scale(double ss, int H, double eps) { return 1.0 / sqrt(ss / H + eps); }

// bf16(x * r * gamma) for the 8 values of xv with their weights gv.
__device__ __forceinline__ uint4 rms_apply8(const uint4 &xv, const uint4 &gv, double r) {
    const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w}, g[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const double a = static_cast<double>(__uint_as_float(w[q] << 16)) * r *
                         static_cast<double>(__uint_as_float(g[q] << 16));
        const double b = static_cast<double>(__uint_as_float(w[q] & 0xffff0000u)) * r *
                         static_cast<double>(__uint_as_float(g[q] & 0xffff0000u));
        o[q] = bf16_nearest(a) | (static_cast<uint32_t>(bf16_nearest(b)) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace moe
