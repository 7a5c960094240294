// Pre-LN RMSNorm of the layer input as a kernel of its own (the prefill sequence and the
// moe_mxfp4_rmsnorm entry point; the decode routers normalize in their own prologue).
#include "device_common.h"
#include "kernels.h"
#include "rms.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// One workgroup per token row; thread i takes the 8-element groups i, i + 256, ...; the
// per-thread sums are added across each wavefront, then the wavefronts' sums in order.
__global__ __launch_bounds__(kThreads) void k_rmsnorm(const uint16_t *__restrict__ x,
                                                      const uint16_t *__restrict__ gamma, int H, double eps,
                                                      uint16_t *__restrict__ xn) {
    __shared__ double s_part[kThreads / kWave];
    const int64_t t = blockIdx.x;
    const uint16_t *xr = x + t * H;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    double ss = 0.0;
    for (int h = 8 * tid; h < H; h += 8 * kThreads) ss = sumsq8(*reinterpret_cast<const uint4 *>(xr + h), ss);
    ss = wave_sum(ss);
    if (lane == 0) s_part[wave] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) tot += s_part[w];
    const double r = rms_scale(tot, H, eps);
    uint16_t *out = xn + t * H;
    for (int h = 8 * tid; h < H; h += 8 * kThreads)
        *reinterpret_cast<uint4 *>(out + h) = rms_apply8(*reinterpret_cast<const uint4 *>(xr + h),
                                                         *reinterpret_cast<const uint4 *>(gamma + h), r);
}

}  // namespace

hipError_t launch_rmsnorm(const Dims &d, const uint16_t *x, const uint16_t *gamma, double eps, uint16_t *xn,
                          hipStream_t s) {
    if (d.T <= 0) return hipSuccess;
    MOE_LAUNCH(k_rmsnorm, dim3(static_cast<unsigned>(d.T)), dim3(kThreads), 0, s, x, gamma, d.H, eps, xn);
    return hipGetLastError();
}

}  // namespace moe
