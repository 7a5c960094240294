// Direct global -> LDS loads and the waits around them, for kernels that stage operands
// in LDS without the compiler's knowledge.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// global_load_lds (saddr form): lane l's 16 (or 4) bytes at base + voff land at LDS byte
// address lds + 16 l (4 l). base and lds are wavefront-uniform. M0 is set in the same
// statement; nothing else in these kernels keeps a value in M0.
__device__ __forceinline__ void dma16(const uint8_t *base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t *base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) (N <= 63), other counters untouched; the empty asm statements keep the
// compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}
// s_waitcnt lgkmcnt(0) only (LDS writes done; vector memory loads may stay in flight).
__device__ __forceinline__ void wait_lgkm0() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    asm volatile("" ::: "memory");
}
// s_waitcnt vmcnt(S * n) for a run-time n <= MAXN (vmcnt needs an immediate).
template <int S, int MAXN>
__device__ __forceinline__ void wait_vm_times(int n) {
    if constexpr (MAXN > 0) {
        if (n >= MAXN) {
            wait_vm<S * MAXN>();
            return;
        }
        wait_vm_times<S, MAXN - 1>(n);
    } else {
        wait_vm<0>();
    }
}
__device__ __forceinline__ void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace moe
