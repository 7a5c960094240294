// Shader-clock probe for the benchmark's context: the rooflines divide by peak rates quoted at
// the chip's 2.4 GHz peak clock, and this measures the clock the CUs actually run at under a
// full-chip ALU load. Every workgroup times a fixed chain of dependent multiply-adds with the
// shader cycle counter (s_memtime) and the constant 100 MHz counter (s_memrealtime); the ratio
// of the sums over the grid, times 100 MHz, is the clock.
#include "kernels.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void k_clock(uint64_t *__restrict__ out, int iters) {
    float a = static_cast<float>(threadIdx.x) * 1e-3f;
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) a = fmaf(a, 0.999f, 0.25f);
    asm volatile("" ::"v"(a));   // the chain is complete before the second reading
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = c1 - c0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace

hipError_t launch_clock_probe(uint64_t *out, int blocks, int iters, hipStream_t s) {
    MOE_LAUNCH(k_clock, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, out, iters);
    return hipGetLastError();
}

}  // namespace moe
