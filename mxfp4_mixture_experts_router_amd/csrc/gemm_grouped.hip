// Grouped expert GEMMs over expert-sorted rows (prefill path), MXFP4 weights dequantized
// in the LDS -> register staging, bf16 MFMA with fp32 accumulation.
//
//  up  : h[r, i] = swiglu(x[tok(r)] . Wgu[e, 2i] + bgu[e, 2i], x[tok(r)] . Wgu[e, 2i+1] + bgu[e, 2i+1])
//        (ZeroModels GPT-OSS page, "Mixture-of-experts feed-forward"; gate/up interleave:
//        MaxText PR "Checkpoint conversion utility ...", "1 Support many-to-one transform";
//        orientation [E, 2I, H]: Megatron-Bridge gpt_oss_bridge page)
//  down: o[r, d] = w[r] * (h[r] . Wdn[e, d] + bdn[e, d])    (orientation [E, H, I], same page)
//
// Work list: every expert's rows [offsets[e], offsets[e+1]) are cut into BM-row tiles; the
// (m-tile, n-tile) pairs of all experts form one flattened list that a persistent grid walks.
// Consecutive list entries share an m-tile (activation reuse in L2) and consecutive m-tiles
// of one expert share its weights.
//
// Contraction mapping: see the decode kernels. Per 128-wide chunk, lane group g = lane/16
// takes the chunk's scale block g, and MFMA step s takes entries 8s..8s+7 of that block.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBK = 128;                 // contraction chunk (4 scale blocks)
constexpr int kAStride = kBK + 8;        // bf16 elements per LDS activation row (padded)
constexpr int kBStride = kBK / 2 + 16;   // bytes per LDS packed weight row (padded)

template <bool UP, int BM, int BN>
__global__ __launch_bounds__(256) void k_grouped(
    const uint16_t *__restrict__ act,          // up: x [T, K]; down: h [T*k, K]
    const int32_t *__restrict__ sorted_token,  // up only
    const float *__restrict__ sorted_w,        // down only
    const uint8_t *__restrict__ wblocks, const uint8_t *__restrict__ wscales,
    const uint16_t *__restrict__ wbias, const int32_t *__restrict__ offsets, int E,
    int K, int Nrows, float alpha, float limit,
    uint16_t *__restrict__ h_out,              // up
    float *__restrict__ o_out) {               // down
    static_assert(BM == 128 && BN == 128, "wave tiling below assumes 128 x 128 tiles");
    __shared__ int s_off[kMaxE + 1];
    __shared__ int s_mcum[kMaxE + 1];
    __shared__ __attribute__((aligned(16))) uint16_t sA[BM * kAStride];
    __shared__ __attribute__((aligned(16))) uint8_t sB[BN * kBStride];
    __shared__ __attribute__((aligned(16))) uint8_t sS[BN * 4];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;
    const int wm = wave >> 1, wn = wave & 1;

    for (int e = tid; e <= E; e += 256) s_off[e] = offsets[e];
    __syncthreads();
    if (wave == 0) {
        // m-tile prefix over experts (E <= 256: four per lane)
        int v[4], local = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * lane + c;
            v[c] = e < E ? (s_off[e + 1] - s_off[e] + BM - 1) / BM : 0;
            local += v[c];
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
        }
        int run = incl - local;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * lane + c;
            if (e < E) s_mcum[e] = run;
            run += v[c];
        }
        if (lane == kWave - 1) s_mcum[E] = incl;
    }
    __syncthreads();

    const int ntn = (Nrows + BN - 1) / BN;
    const int total = s_mcum[E] * ntn;
    const int kb_total = K / 32;
    const int nchunks = (kb_total + 3) / 4;
    const int kbytes = K / 2, kscales = K / 32;

    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        const int mg = tile / ntn, nt = tile % ntn;
        int lo = 0, hi = E - 1;                       // last e with s_mcum[e] <= mg
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_mcum[mid] <= mg) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int row0 = s_off[e] + (mg - s_mcum[e]) * BM;
        const int rows = min(BM, s_off[e + 1] - row0);
        const int n0 = nt * BN;

        // per-thread global source rows for the staged loads
        const uint16_t *arow[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = (tid + 256 * i) >> 4;
            if (r < rows) {
                const int64_t src = UP ? sorted_token[row0 + r] : row0 + r;
                arow[i] = act + src * K;
            } else {
                arow[i] = nullptr;
            }
        }
        const uint8_t *brow[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = (tid + 256 * i) >> 2;
            brow[i] = (n0 + r < Nrows) ? wblocks + (static_cast<int64_t>(e) * Nrows + n0 + r) * kbytes : nullptr;
        }
        const uint8_t *srow = (tid < BN && n0 + tid < Nrows)
                                  ? wscales + (static_cast<int64_t>(e) * Nrows + n0 + tid) * kscales
                                  : nullptr;

        f32x4 acc[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

        uint4 ra[8], rb[2];
        uint32_t rs = 0;
        auto fetch = [&](int c) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int q = (tid + 256 * i) & 15;          // 16-byte piece within the row chunk
                const int kk = c * kBK + q * 8;
                ra[i] = (arow[i] != nullptr && kk < K) ? *reinterpret_cast<const uint4 *>(arow[i] + kk) : zero4();
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int q = (tid + 256 * i) & 3;
                const int kb = 4 * c + q;
                rb[i] = (brow[i] != nullptr && kb < kb_total) ? *reinterpret_cast<const uint4 *>(brow[i] + kb * 16) : zero4();
            }
            rs = 0;
            if (srow != nullptr) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int kb = 4 * c + q;
                    if (kb < kb_total) rs |= static_cast<uint32_t>(srow[kb]) << (8 * q);
                }
            }
        };
        auto stash = [&]() {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int idx = tid + 256 * i;
                *reinterpret_cast<uint4 *>(&sA[(idx >> 4) * kAStride + (idx & 15) * 8]) = ra[i];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int idx = tid + 256 * i;
                *reinterpret_cast<uint4 *>(&sB[(idx >> 2) * kBStride + (idx & 3) * 16]) = rb[i];
            }
            if (tid < BN) *reinterpret_cast<uint32_t *>(&sS[tid * 4]) = rs;
        };

        fetch(0);
        for (int c = 0; c < nchunks; ++c) {
            __syncthreads();                 // previous chunk's LDS reads are done
            stash();
            __syncthreads();
            if (c + 1 < nchunks) fetch(c + 1);

            // B fragments: 4 weight rows per wave, decoded for all 4 steps of the chunk
            bf16x8 bw[4][4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                int lr;
                if (UP) lr = wn * 64 + 2 * (16 * (f >> 1) + col) + (f & 1);   // f: (pair block, gate/up)
                else lr = wn * 64 + 16 * f + col;
                const uint4 p = *reinterpret_cast<const uint4 *>(&sB[lr * kBStride + 16 * g]);
                const float sc = e8m0_to_f32(sS[lr * 4 + g]);
                bw[f][0] = mxfp4_word_to_bf16x8(p.x, sc);
                bw[f][1] = mxfp4_word_to_bf16x8(p.y, sc);
                bw[f][2] = mxfp4_word_to_bf16x8(p.z, sc);
                bw[f][3] = mxfp4_word_to_bf16x8(p.w, sc);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int ar = wm * 64 + 16 * mt + col;
                    const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4 *>(&sA[ar * kAStride + 32 * g + 8 * s]));
#pragma unroll
                    for (int f = 0; f < 4; ++f) acc[mt][f] = mfma16(av, bw[f][s], acc[mt][f]);
                }
            }
        }

        // epilogue
        if (UP) {
#pragma unroll
            for (int pb = 0; pb < 2; ++pb) {
                const int i = n0 / 2 + wn * 32 + 16 * pb + col;
                if (2 * i >= Nrows) continue;
                const float bgate = bf16_to_f32(wbias[static_cast<int64_t>(e) * Nrows + 2 * i]);
                const float bup = bf16_to_f32(wbias[static_cast<int64_t>(e) * Nrows + 2 * i + 1]);
                const int Iw = Nrows / 2;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int lr = wm * 64 + 16 * mt + 4 * g + r;
                        if (lr >= rows) continue;
                        const float hv = swiglu(acc[mt][2 * pb][r] + bgate, acc[mt][2 * pb + 1][r] + bup, alpha, limit);
                        h_out[static_cast<int64_t>(row0 + lr) * Iw + i] = f32_to_bf16(hv);
                    }
            }
        } else {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int d = n0 + wn * 64 + 16 * f + col;
                if (d >= Nrows) continue;
                const float bd = bf16_to_f32(wbias[static_cast<int64_t>(e) * Nrows + d]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int lr = wm * 64 + 16 * mt + 4 * g + r;
                        if (lr >= rows) continue;
                        o_out[static_cast<int64_t>(row0 + lr) * Nrows + d] = (acc[mt][f][r] + bd) * sorted_w[row0 + lr];
                    }
            }
        }
    }
}

// y[t, d] = sum_j o[slot_row[t*k + j], d] in slot order, rounded to bf16. Thread = 4 columns
// per grid-stride step.
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ o,
                                                 const int32_t *__restrict__ slot_row, int64_t T,
                                                 int H, int k, uint16_t *__restrict__ y) {
    const int per_row = H / 4;
    const int64_t total = T * per_row;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < total;
         q += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t t = q / per_row;
        const int d = static_cast<int>(q % per_row) * 4;
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const float4 v = *reinterpret_cast<const float4 *>(o + static_cast<int64_t>(slot_row[t * k + j]) * H + d);
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        const uint32_t lo = f32_to_bf16(s.x) | (static_cast<uint32_t>(f32_to_bf16(s.y)) << 16);
        const uint32_t hi = f32_to_bf16(s.z) | (static_cast<uint32_t>(f32_to_bf16(s.w)) << 16);
        *reinterpret_cast<uint2 *>(y + t * H + d) = make_uint2(lo, hi);
    }
}

// Standalone dequantization: one thread per 32-element scale block (16 packed bytes) per
// grid-stride step.
__global__ __launch_bounds__(256) void k_dequant(const uint8_t *__restrict__ blocks,
                                                 const uint8_t *__restrict__ scales, int64_t nblk,
                                                 uint16_t *__restrict__ out) {
    for (int64_t b = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; b < nblk;
         b += static_cast<int64_t>(gridDim.x) * 256) {
        const uint4 p = *reinterpret_cast<const uint4 *>(blocks + b * 16);
        const float sc = e8m0_to_f32(scales[b]);
        uint4 *dst = reinterpret_cast<uint4 *>(out + b * 32);
        dst[0] = __builtin_bit_cast(uint4, mxfp4_word_to_bf16x8(p.x, sc));
        dst[1] = __builtin_bit_cast(uint4, mxfp4_word_to_bf16x8(p.y, sc));
        dst[2] = __builtin_bit_cast(uint4, mxfp4_word_to_bf16x8(p.z, sc));
        dst[3] = __builtin_bit_cast(uint4, mxfp4_word_to_bf16x8(p.w, sc));
    }
}

unsigned grid_for(int64_t items) {
    const int64_t blocks = (items + 255) / 256;
    return static_cast<unsigned>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

int persistent_blocks(int64_t rows_upper, int E, int Nrows, int BM, int BN) {
    const int64_t mtiles = (rows_upper + BM - 1) / BM + (rows_upper < E ? rows_upper : E);
    const int64_t tiles = mtiles * ((Nrows + BN - 1) / BN);
    const int64_t cap = 256 * 4;
    return static_cast<int>(tiles < cap ? (tiles > 0 ? tiles : 1) : cap);
}

}  // namespace

hipError_t launch_up_grouped(const Dims &d, const uint16_t *x, const uint8_t *gu_blocks,
                             const uint8_t *gu_scales, const uint16_t *gu_bias,
                             const int32_t *offsets, const int32_t *sorted_token,
                             uint16_t *h, hipStream_t s) {
    const int Nrows = 2 * d.I;
    const int blocks = persistent_blocks(d.T * d.k, d.E, Nrows, 128, 128);
    hipLaunchKernelGGL((k_grouped<true, 128, 128>), dim3(blocks), dim3(256), 0, s, x, sorted_token,
                       nullptr, gu_blocks, gu_scales, gu_bias, offsets, d.E, d.H, Nrows, d.alpha,
                       d.limit, h, nullptr);
    return hipGetLastError();
}

hipError_t launch_down_grouped(const Dims &d, const uint16_t *h, const uint8_t *dn_blocks,
                               const uint8_t *dn_scales, const uint16_t *dn_bias,
                               const int32_t *offsets, const float *sorted_w, float *o,
                               hipStream_t s) {
    const int blocks = persistent_blocks(d.T * d.k, d.E, d.H, 128, 128);
    hipLaunchKernelGGL((k_grouped<false, 128, 128>), dim3(blocks), dim3(256), 0, s, h, nullptr,
                       sorted_w, dn_blocks, dn_scales, dn_bias, offsets, d.E, d.I, d.H, d.alpha,
                       d.limit, nullptr, o);
    return hipGetLastError();
}

hipError_t launch_combine(const Dims &d, const float *o, const int32_t *slot_row, uint16_t *y,
                          hipStream_t s) {
    hipLaunchKernelGGL(k_combine, dim3(grid_for(d.T * (d.H / 4))), dim3(256), 0, s, o, slot_row,
                       d.T, d.H, d.k, y);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *blocks, const uint8_t *scales, int64_t rows, int cols,
                          uint16_t *out, hipStream_t s) {
    const int64_t nblk = rows * (cols / 32);
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL(k_dequant, dim3(grid_for(nblk)), dim3(256), 0, s, blocks, scales,
                       nblk, out);
    return hipGetLastError();
}

}  // namespace moe
