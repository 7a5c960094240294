// Device helpers shared by the gfx950 kernels of the MXFP4 mixture-of-experts layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxE = 256;       // most experts the kernels handle (one bit each in a 256-bit mask)

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// s += the four bf16 values at r (8-byte aligned): the residual branch of a pre-norm block.
__device__ __forceinline__ void add_residual4(float4 &s, const uint16_t *r) {
    const uint2 u = *reinterpret_cast<const uint2 *>(r);
    s.x += __uint_as_float(u.x << 16);
    s.y += __uint_as_float(u.x & 0xffff0000u);
    s.z += __uint_as_float(u.y << 16);
    s.w += __uint_as_float(u.y & 0xffff0000u);
}

// E8M0 scale byte -> the fp32 power of two 2^(s - 127) (valid for s in 1..254, which
// covers the supported 2..252).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) { return __uint_as_float(s << 23); }

// One packed 32-bit word = 8 FP4 E2M1 codes (byte j: low nibble = element 2j, high
// nibble = element 2j+1) -> 8 bf16 values scaled by `scale`. gfx950 converts a byte to
// two scaled bf16 values in one instruction (v_cvt_scalef32_pk_bf16_fp4).
__device__ __forceinline__ bf16x8 mxfp4_word_to_bf16x8(uint32_t word, float scale) {
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16) on one wavefront.
// Lane l supplies A row (l % 16) and B column (l % 16), 8 consecutive entries of the
// contraction each, for contraction group (l / 16); D lane l holds column (l % 16), rows
// 4 * (l / 16) + 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// sigmoid-gated clamped SwiGLU of the GPT-OSS experts: (clamp(up) + 1) * g * sigmoid(alpha*g)
// with g = min(gate, limit) and up clamped to [-limit, limit]. The sigmoid takes the hardware
// reciprocal (1 ulp): every caller rounds h to 8 significant bits afterwards.
__device__ __forceinline__ float swiglu(float gate, float up, float alpha, float limit) {
    float g = fminf(gate, limit);
    float u = fminf(fmaxf(up, -limit), limit);
    float sig = __builtin_amdgcn_rcpf(1.0f + __expf(-alpha * g));
    return (u + 1.0f) * g * sig;
}

// v of lane ^ 1 and of lane ^ 2, by DPP quad permutations (no LDS round trip, unlike
// __shfl_xor).
__device__ __forceinline__ float lane_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
}

// v + (the double from another lane by DPP control CTRL; 0 where ROW_MASK disables the row)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double add_dpp_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(b & 0xffffffffll), CTRL, ROW_MASK, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, ROW_MASK, 0xf, false);
    return v + __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

// Sum of v over the 64 lanes of a wavefront, the same bits in every lane: pairs, quads,
// 8- and 16-lane groups by DPP within each row, then the rows by broadcasts into lane 63,
// whose value every lane reads. A fixed order, no LDS round trips.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = add_dpp_f64<0xB1, 0xf>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    v = add_dpp_f64<0x4E, 0xf>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    v = add_dpp_f64<0x141, 0xf>(v);   // row_half_mirror: the other quad of the 8
    v = add_dpp_f64<0x140, 0xf>(v);   // row_mirror: the other 8 of the row
    v = add_dpp_f64<0x142, 0xa>(v);   // row_bcast15 into rows 1 and 3
    v = add_dpp_f64<0x143, 0xc>(v);   // row_bcast31 into rows 2 and 3
    const long long b = __double_as_longlong(v);
    const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffffll), 63));
    const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63));
    return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (1ull << __lane_id()) - 1ull;
}

}  // namespace moe
