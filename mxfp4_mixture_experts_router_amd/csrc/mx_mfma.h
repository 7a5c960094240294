// Block-scaled MFMA helpers: MXFP4 weights as the raw B operand of gfx950's
// v_mfma_scale_f32_16x16x128_f8f6f4, activations as exact fp8 (e4m3) hi/lo pairs.
//
// OCP Microscaling Formats (MX) v1.0 (cited by the ZeroModels GPT-OSS page, "MXFP4
// experts"): an MX block is 32 elements sharing one E8M0 scale 2^(s-127). The weights
// arrive in that form (E2M1 elements). Activations are brought into the same form with
// E4M3 elements: a block with largest magnitude m gets the exponent eb = floor(log2 m) - 7
// (so every x / 2^eb lies below 256, inside E4M3's range), hi = E4M3(x / 2^eb) rounded to
// nearest even, and the remainder x / 2^eb - hi (at most half an E4M3 step, hence at most
// 4 significant bits) is stored as lo = E4M3(16 (x / 2^eb - hi)) with exponent eb - 4. For a
// bf16 x (8 significant bits) hi + lo reproduces x exactly unless lo falls below E4M3's
// normal range (elements some 2^14 below the block's largest); an fp32 x keeps 8 bits.
//
// The two parts become two rows of the A operand (hi in row 2s, lo in row 2s + 1, each with
// its own scale), so one MFMA yields both partial products and the result of activation
// row s is D[2s] + D[2s + 1].
//
// Operand layouts of the 16x16x128 instruction (lane l, g = l / 16):
//  B (E2M1): lane (n = l % 16, g) holds the 32 elements of contraction block g of column n,
//            16 bytes, low nibble first: one packed MXFP4 block as stored; scale_b = its E8M0.
//  A (E4M3): lane (m = l % 16, g) holds 32 bytes of row m: bytes 0-15 are contraction entries
//            16g .. 16g + 15 and bytes 16-31 entries 64 + 16g .. 64 + 16g + 15; scale_a is
//            the E8M0 of row m's contraction block g.
//  D:        lane (n = l % 16, g) holds column n, rows 4g .. 4g + 3.
// The 128 contraction entries of one instruction may be any four 32-blocks ("virtual block"
// v = 0..3 -> actual block ab[v]) as long as A, B and both scales agree on the mapping.
#pragma once

#include "device_common.h"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_mx(const i32x8 &a, const i32x8 &b, f32x4 c, uint32_t scale_a,
                                         uint32_t scale_b) {
    // A format E4M3 (cbsz 0), B format E2M1 (blgp 4); scales in byte 0 of each register
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, static_cast<int>(scale_a), 0,
                                                            static_cast<int>(scale_b));
}

// B operand from one packed 16-byte MXFP4 block (the upper half of the register tuple is
// not read for E2M1).
__device__ __forceinline__ i32x8 mx_b_operand(const uint4 &blk) {
    i32x8 b;
    b[0] = static_cast<int>(blk.x); b[1] = static_cast<int>(blk.y);
    b[2] = static_cast<int>(blk.z); b[3] = static_cast<int>(blk.w);
    b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
    return b;
}

__device__ __forceinline__ i32x8 mx_a_operand(const uint4 &first, const uint4 &second) {
    i32x8 a;
    a[0] = static_cast<int>(first.x); a[1] = static_cast<int>(first.y);
    a[2] = static_cast<int>(first.z); a[3] = static_cast<int>(first.w);
    a[4] = static_cast<int>(second.x); a[5] = static_cast<int>(second.y);
    a[6] = static_cast<int>(second.z); a[7] = static_cast<int>(second.w);
    return a;
}

// Exponent eb of an activation block with largest magnitude m (see above); clamped so that
// both E8M0 scales 127 + eb and 123 + eb stay in [0, 254].
__device__ __forceinline__ int mx8_block_exponent(float m) {
    const int ex = static_cast<int>((__float_as_uint(m) >> 23) & 0xffu) - 127;   // floor(log2 m), m normal
    return m > 0.f ? max(ex - 7, -123) : 0;
}

// hi/lo E4M3 bytes of four values (already divided by 2^eb): one 32-bit word each.
__device__ __forceinline__ void mx8_split4(float a, float b, float c, float d, uint32_t &hi, uint32_t &lo) {
    int h = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    h = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, h, true);
    const float ra = (a - __builtin_amdgcn_cvt_f32_fp8(h, 0)) * 16.f;
    const float rb = (b - __builtin_amdgcn_cvt_f32_fp8(h, 1)) * 16.f;
    const float rc = (c - __builtin_amdgcn_cvt_f32_fp8(h, 2)) * 16.f;
    const float rd = (d - __builtin_amdgcn_cvt_f32_fp8(h, 3)) * 16.f;
    int l = __builtin_amdgcn_cvt_pk_fp8_f32(ra, rb, 0, false);
    l = __builtin_amdgcn_cvt_pk_fp8_f32(rc, rd, l, true);
    hi = static_cast<uint32_t>(h);
    lo = static_cast<uint32_t>(l);
}

// One 32-element block x[0..31] -> 32 hi bytes, 32 lo bytes (8 words each) and the two E8M0
// scales (127 + eb for hi, 123 + eb for lo).
__device__ __forceinline__ void mx8_split_block(const float (&x)[32], uint32_t (&hi)[8], uint32_t (&lo)[8],
                                                uint32_t &s_hi, uint32_t &s_lo) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(x[i]));
    const int eb = mx8_block_exponent(m);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        mx8_split4(ldexpf(x[4 * j], -eb), ldexpf(x[4 * j + 1], -eb), ldexpf(x[4 * j + 2], -eb),
                   ldexpf(x[4 * j + 3], -eb), hi[j], lo[j]);
    s_hi = static_cast<uint32_t>(127 + eb);
    s_lo = static_cast<uint32_t>(123 + eb);
}

// E4M3 activation matrices ("mx8"): for R activation rows of K elements, 2R byte rows of K
// (row 2r = hi, row 2r + 1 = lo of activation row r), followed by 2R scale rows of
// mx8_scale_stride(K) bytes (K / 32 E8M0 bytes, padded to a multiple of 16). A lo row's
// scale is always its hi row's minus 4 (every writer below); readers may rely on it.
__host__ __device__ inline int mx8_scale_stride(int K) { return ((K / 32) + 15) & ~15; }
__host__ __device__ inline size_t mx8_bytes(int64_t rows, int K) {
    return static_cast<size_t>(2 * rows) * (static_cast<size_t>(K) + static_cast<size_t>(mx8_scale_stride(K)));
}

// Writes the hi/lo split of one 32-element block v into rows 2n and 2n + 1 of an mx8 matrix
// (row stride K bytes; scales at qs with stride ss) at block b.
__device__ __forceinline__ void store_mx8_block(const float (&v)[32], uint8_t *q8, uint8_t *qs, int64_t n, int K,
                                                int ss, int b) {
    uint32_t hi[8], lo[8], sh, sl;
    mx8_split_block(v, hi, lo, sh, sl);
    uint4 *dh = reinterpret_cast<uint4 *>(q8 + (2 * n) * K + 32 * b);
    uint4 *dl = reinterpret_cast<uint4 *>(q8 + (2 * n + 1) * K + 32 * b);
    dh[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    dh[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    dl[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    dl[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
    qs[(2 * n) * ss + b] = static_cast<uint8_t>(sh);
    qs[(2 * n + 1) * ss + b] = static_cast<uint8_t>(sl);
}

// The expert intermediate h ("h8": written by the grouped gate_up GEMM, read by the grouped
// down GEMM) uses the same data rows with group-major scales: for R rows, group j of sixteen
// scale blocks (16j .. 16j + 15, four GEMM stages of 128 elements) is R 16-byte words, word n
// holding row n's hi scales of those blocks (byte b % 16); a lo scale is its hi scale minus 4
// and is not stored. The windows of consecutive rows are then contiguous. 16 R ceil(K / 512)
// scale bytes: half of the row-major layout's 2 R S.
__host__ __device__ inline size_t h8_scale_offset(int64_t R, int64_t n, int b) {
    return static_cast<size_t>(16 * (static_cast<int64_t>(b >> 4) * R + n) + (b & 15));
}

// Writes one 32-element block v of row n as store_mx8_block does, into an h8 matrix of R
// rows (group-major scales at qs).
__device__ __forceinline__ void store_h8_block(const float (&v)[32], uint8_t *q8, uint8_t *qs, int64_t n, int K,
                                               int64_t R, int b) {
    uint32_t hi[8], lo[8], sh, sl;
    mx8_split_block(v, hi, lo, sh, sl);
    uint4 *dh = reinterpret_cast<uint4 *>(q8 + (2 * n) * K + 32 * b);
    uint4 *dl = reinterpret_cast<uint4 *>(q8 + (2 * n + 1) * K + 32 * b);
    dh[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    dh[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    dl[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    dl[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
    qs[h8_scale_offset(R, n, b)] = static_cast<uint8_t>(sh);
}

// The mx8 rows of bf16 activation row `xrow` (K elements) as row r of the mx8 matrix q8
// holding R rows; the calling block's threads from `first` on share the K / 32 blocks
// (threads below `first` do nothing).
__device__ __forceinline__ void write_mx8_row(const uint16_t *xrow, int K, uint8_t *q8, int64_t R, int64_t r,
                                              int first = 0) {
    uint8_t *qs = q8 + static_cast<size_t>(2 * R) * K;
    if (static_cast<int>(threadIdx.x) < first) return;
    for (int b = static_cast<int>(threadIdx.x) - first; b < K / 32; b += static_cast<int>(blockDim.x) - first) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 u = *reinterpret_cast<const uint4 *>(xrow + 32 * b + 8 * j);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[8 * j + 2 * i] = __uint_as_float(w[i] << 16);
                v[8 * j + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
        store_mx8_block(v, q8, qs, r, K, mx8_scale_stride(K), b);
    }
}

}  // namespace moe
