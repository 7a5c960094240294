// Grouped expert GEMMs over expert-sorted rows (prefill path) on gfx950's block-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4): the packed MXFP4 weight blocks are the B operand as
// stored, the activations are E4M3 hi/lo pairs (mx8 matrices, see mx_mfma.h) as A rows.
//
//  up  : h[r, i] = swiglu(x[tok(r)] . Wgu[e, 2i] + bgu[e, 2i], x[tok(r)] . Wgu[e, 2i+1] + bgu[e, 2i+1])
//        (ZeroModels GPT-OSS page, "Mixture-of-experts feed-forward"; gate/up interleave:
//        MaxText PR "Checkpoint conversion utility ...", "1 Support many-to-one transform";
//        orientation [E, 2I, H]: Megatron-Bridge gpt_oss_bridge page), written as the mx8
//        matrix h8 (T k rows of I, sorted-row order)
//  down: o[r, d] = w[r] * (h[r] . Wdn[e, d] + bdn[e, d])    (orientation [E, H, I], same page)
//
// Work list: every expert's rows [offsets[e], offsets[e+1]) are cut into BM-row tiles; the
// (m-tile, n-tile) pairs of all experts form one flattened list. The grid is persistent and
// XCD-aware: the blocks of one XCD (block b runs on XCD b % 8) take the m-tiles mg with
// mg % 8 == XCD, walking all n-tiles of one m-tile before the next, so an m-tile's
// activations are fetched into one XCD's L2 and reused across its n-tiles.
//
// Block tile: BM = 128 activation rows (256 A rows: hi, lo) x BN = 192 output columns, BK =
// 128 (one MFMA step) per LDS stage, two LDS stages (the next stage's global loads are in
// flight while the current one is multiplied). 8 wavefronts stacked along M; each owns 32 A
// rows x 192 columns = 2 x 12 MFMA tiles (96 accumulator registers; 192 columns = 96 gate/up
// pairs = 3 whole MX blocks of h). Within a stage lane group g takes scale block g.
#include "device_common.h"
#include "kernels.h"
#include "mx_mfma.h"

namespace moe {
namespace {

constexpr int kBM = 128;                 // activation rows per tile (2 A rows each)
constexpr int kBN = 192;                 // output columns (weight rows) per tile
constexpr int kBK = 128;                 // contraction per stage (4 scale blocks)
constexpr int kAStride = kBK + 16;       // bytes per LDS A row (padded)
constexpr int kBStride = kBK / 2 + 16;   // bytes per LDS packed weight row (padded)

template <bool UP>
__global__ __launch_bounds__(512) void k_gemm_mx(
    const uint8_t *__restrict__ a8, int64_t a_rows,  // mx8 activations: up x8 (T rows), down h8 (T k rows)
    const int32_t *__restrict__ sorted_token,        // up only
    const float *__restrict__ sorted_w,              // down only
    const uint8_t *__restrict__ wblocks, const uint8_t *__restrict__ wscales,
    const uint16_t *__restrict__ wbias, const int32_t *__restrict__ offsets, int E,
    int K, int Nrows, float alpha, float limit,
    uint8_t *__restrict__ h8, int64_t h_rows,        // up: mx8 output (T k rows of Nrows / 2)
    float *__restrict__ o_out) {                     // down
    __shared__ int s_off[kMaxE + 1];
    __shared__ int s_mcum[kMaxE + 1];
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][2 * kBM * kAStride];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][kBN * kBStride];
    __shared__ __attribute__((aligned(16))) uint32_t sAS[2][2 * kBM];   // 4 E8M0 bytes per A row
    __shared__ __attribute__((aligned(16))) uint32_t sBS[2][kBN];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;

    for (int e = tid; e <= E; e += 512) s_off[e] = offsets[e];
    __syncthreads();
    if (wave == 0) {
        // m-tile prefix over experts (E <= 256: four per lane)
        int v[4], local = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * lane + c;
            v[c] = e < E ? (s_off[e + 1] - s_off[e] + kBM - 1) / kBM : 0;
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

    const int ntn = (Nrows + kBN - 1) / kBN;
    const int mtiles = s_mcum[E];
    const int nkb = K / 32;                      // scale blocks per row
    const int kt_total = (nkb + 3) / 4;
    const int kbytes = K / 2;
    const int ass = mx8_scale_stride(K);
    const uint8_t *a_sc = a8 + static_cast<size_t>(2 * a_rows) * K;
    // XCD-aware walk: this block's XCD owns m-tiles mg = xcd + 8j
    const int xcd = blockIdx.x & 7, lb = blockIdx.x >> 3, nb = gridDim.x >> 3;
    const int my_m = mtiles > xcd ? (mtiles - xcd + 7) / 8 : 0;
    const int my_tiles = my_m * ntn;

    for (int it = lb; it < my_tiles; it += nb) {
        const int mg = xcd + 8 * (it / ntn), nt = it % ntn;
        int lo = 0, hi = E - 1;                       // last e with s_mcum[e] <= mg
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_mcum[mid] <= mg) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int row0 = s_off[e] + (mg - s_mcum[e]) * kBM;
        const int rows = min(kBM, s_off[e + 1] - row0);
        const int n0 = nt * kBN;

        // this thread's staged pieces: A rows (tid + 512 i) / 8, 16-byte piece tid % 8;
        // B rows (tid + 512 i) / 4 (i = 1 only for tid < 256), piece tid % 4; scales of A row
        // tid (< 256) and B row tid (< 192).
        int arow[4];      // A byte row (2 src + part) of the staged pieces, -1 past the tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid + 512 * i) >> 3;       // A row: activation row r / 2, part r % 2
            arow[i] = -1;
            if ((r >> 1) < rows) arow[i] = 2 * (UP ? sorted_token[row0 + (r >> 1)] : row0 + (r >> 1)) + (r & 1);
        }
        int ascr = -1;    // A scale row of thread tid < 256
        if (tid < 2 * kBM && (tid >> 1) < rows) ascr = 2 * (UP ? sorted_token[row0 + (tid >> 1)] : row0 + (tid >> 1)) + (tid & 1);
        const uint8_t *wbase = wblocks + static_cast<int64_t>(e) * Nrows * kbytes;   // uniform
        const uint8_t *sbase = wscales + static_cast<int64_t>(e) * Nrows * nkb;
        int brow[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) brow[i] = min(n0 + ((tid + 512 * i) >> 2), Nrows - 1);
        const int bscr = min(n0 + tid, Nrows - 1);

        // raw staged values; the scale bytes are assembled at stash time so that issuing a
        // stage's loads never waits for them
        uint4 ra[4], rb[2];
        uint32_t rsa = 0x7f7f7f7fu, rsb[4] = {127u, 127u, 127u, 127u};
        auto fetch = [&](int kt) {
            const int pa = tid & 7;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = kt * kBK + 16 * pa;
                ra[i] = (arow[i] >= 0 && kk < K)
                            ? *reinterpret_cast<const uint4 *>(a8 + static_cast<int64_t>(arow[i]) * K + kk)
                            : zero4();
            }
            const int pb = tid & 3;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int kb = 4 * kt + pb;
                rb[i] = (kb < nkb && tid + 512 * i < 4 * kBN)
                            ? *reinterpret_cast<const uint4 *>(wbase + static_cast<int64_t>(brow[i]) * kbytes + 16 * kb)
                            : zero4();
            }
            // A scale rows are padded to 16 bytes: the 4 bytes of this stage are in bounds
            if (ascr >= 0) rsa = *reinterpret_cast<const uint32_t *>(a_sc + static_cast<int64_t>(ascr) * ass + 4 * kt);
            if (tid < kBN) {
                const uint8_t *bs = sbase + static_cast<int64_t>(bscr) * nkb;
#pragma unroll
                for (int q = 0; q < 4; ++q) rsb[q] = 4 * kt + q < nkb ? bs[4 * kt + q] : 127u;
            }
        };
        auto stash = [&](int buf, int kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int idx = tid + 512 * i;
                *reinterpret_cast<uint4 *>(&sA[buf][(idx >> 3) * kAStride + (idx & 7) * 16]) = ra[i];
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int idx = tid + 512 * i;
                if (idx < 4 * kBN) *reinterpret_cast<uint4 *>(&sB[buf][(idx >> 2) * kBStride + (idx & 3) * 16]) = rb[i];
            }
            if (tid < 2 * kBM) {
                // bytes past the row's nkb blocks (never written) become 127 (their data is 0)
                uint32_t v = ascr >= 0 ? rsa : 0x7f7f7f7fu;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (4 * kt + q >= nkb) v = (v & ~(0xffu << (8 * q))) | (127u << (8 * q));
                sAS[buf][tid] = v;
            }
            if (tid < kBN) sBS[buf][tid] = rsb[0] | (rsb[1] << 8) | (rsb[2] << 16) | (rsb[3] << 24);
        };

        f32x4 acc[2][12];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 12; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

        __syncthreads();   // the previous tile's last stage is no longer read
        fetch(0);
        stash(0, 0);
        __syncthreads();
        for (int kt = 0; kt < kt_total; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < kt_total) fetch(kt + 1);
            // A fragments of this wave's 2 m-tiles, B fragments of its 12 n-tiles
            i32x8 af[2];
            uint32_t sa[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int ar = wave * 32 + 16 * mt + col;
                const uint8_t *p = &sA[buf][ar * kAStride];
                af[mt] = mx_a_operand(*reinterpret_cast<const uint4 *>(p + 16 * g),
                                      *reinterpret_cast<const uint4 *>(p + 64 + 16 * g));
                sa[mt] = (sAS[buf][ar] >> (8 * g)) & 0xffu;
            }
#pragma unroll
            for (int nt2 = 0; nt2 < 12; ++nt2) {
                const int br = 16 * nt2 + col;
                const i32x8 bop = mx_b_operand(*reinterpret_cast<const uint4 *>(&sB[buf][br * kBStride + 16 * g]));
                const uint32_t sb = (sBS[buf][br] >> (8 * g)) & 0xffu;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) acc[mt][nt2] = mfma_mx(af[mt], bop, acc[mt][nt2], sa[mt], sb);
            }
            if (kt + 1 < kt_total) stash(buf ^ 1, kt + 1);
            __syncthreads();
        }

        // epilogue. D rows 16 mt + 4g + r of the wave's A rows: activation row
        // 16 wave + 8 mt + 2g + r/2 (part r % 2) -> value = D[.., 2j] + D[.., 2j + 1].
        if (UP) {
            // h of the tile's 128 rows x 96 pairs (fp32) into LDS,
            // then one thread per (row, MX block of 32 pairs) quantizes it into h8
            constexpr int kHS = kBN / 2 + 1;                   // padded row of pairs
            float *s_h = reinterpret_cast<float *>(&sA[0][0]);
            __syncthreads();
#pragma unroll
            for (int nt2 = 0; nt2 < 12; ++nt2) {
                const int wr = n0 + 16 * nt2 + col;
                const float bias = wr < Nrows ? bf16_to_f32(wbias[static_cast<int64_t>(e) * Nrows + wr]) : 0.f;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int lr = wave * 16 + 8 * mt + 2 * g + j;
                        const float v = acc[mt][nt2][2 * j] + acc[mt][nt2][2 * j + 1] + bias;
                        const float other = __shfl_xor(v, 1);
                        if ((col & 1) == 0) s_h[lr * kHS + 8 * nt2 + col / 2] = swiglu(v, other, alpha, limit);
                    }
            }
            __syncthreads();
            const int Iw = Nrows / 2;
            const int is8 = mx8_scale_stride(Iw);
            uint8_t *h_sc = h8 + static_cast<size_t>(2 * h_rows) * Iw;
            for (int item = tid; item < kBM * (kBN / 64); item += 512) {
                const int r = item / (kBN / 64), q = item % (kBN / 64);
                const int ib = n0 / 64 + q;                       // MX block of i
                if (r >= rows || 64 * ib >= Nrows) continue;
                float v[32];
#pragma unroll
                for (int i = 0; i < 32; ++i) v[i] = s_h[r * kHS + 32 * q + i];
                store_mx8_block(v, h8, h_sc, static_cast<int64_t>(row0 + r), Iw, is8, ib);
            }
        } else {
#pragma unroll
            for (int nt2 = 0; nt2 < 12; ++nt2) {
                const int d = n0 + 16 * nt2 + col;
                if (d >= Nrows) continue;
                const float bd = bf16_to_f32(wbias[static_cast<int64_t>(e) * Nrows + d]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int lr = wave * 16 + 8 * mt + 2 * g + j;
                        if (lr >= rows) continue;
                        const float v = acc[mt][nt2][2 * j] + acc[mt][nt2][2 * j + 1];
                        o_out[static_cast<int64_t>(row0 + lr) * Nrows + d] = (v + bd) * sorted_w[row0 + lr];
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

// bf16 rows -> mx8 matrix: one thread per 32-element block per grid-stride step.
__global__ __launch_bounds__(256) void k_quantize(const uint16_t *__restrict__ x, int64_t rows, int cols,
                                                  uint8_t *__restrict__ q8) {
    const int nb = cols / 32;
    const int ss = mx8_scale_stride(cols);
    uint8_t *qs = q8 + static_cast<size_t>(2 * rows) * cols;
    const int64_t total = rows * nb;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < total;
         q += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t r = q / nb;
        const int b = static_cast<int>(q % nb);
        const uint16_t *src = x + r * cols + 32 * b;
        float v[32];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 u = *reinterpret_cast<const uint4 *>(src + 8 * j);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[8 * j + 2 * i] = __uint_as_float(w[i] << 16);
                v[8 * j + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        }
        store_mx8_block(v, q8, qs, r, cols, ss, b);
    }
}

unsigned grid_for(int64_t items) {
    const int64_t blocks = (items + 255) / 256;
    return static_cast<unsigned>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

// One block per CU (the LDS stages take most of a CU's LDS), a multiple of 8 (XCDs).
int persistent_blocks() { return 256; }

}  // namespace

hipError_t launch_up_grouped(const Dims &d, const uint8_t *x8, const uint8_t *gu_blocks,
                             const uint8_t *gu_scales, const uint16_t *gu_bias,
                             const int32_t *offsets, const int32_t *sorted_token,
                             uint8_t *h8, hipStream_t s) {
    hipLaunchKernelGGL((k_gemm_mx<true>), dim3(persistent_blocks()), dim3(512), 0, s, x8, d.T, sorted_token,
                       nullptr, gu_blocks, gu_scales, gu_bias, offsets, d.E, d.H, 2 * d.I, d.alpha, d.limit,
                       h8, d.T * d.k, nullptr);
    return hipGetLastError();
}

hipError_t launch_down_grouped(const Dims &d, const uint8_t *h8, const uint8_t *dn_blocks,
                               const uint8_t *dn_scales, const uint16_t *dn_bias,
                               const int32_t *offsets, const float *sorted_w, float *o,
                               hipStream_t s) {
    hipLaunchKernelGGL((k_gemm_mx<false>), dim3(persistent_blocks()), dim3(512), 0, s, h8, d.T * d.k, nullptr,
                       sorted_w, dn_blocks, dn_scales, dn_bias, offsets, d.E, d.I, d.H, d.alpha, d.limit,
                       nullptr, 0, o);
    return hipGetLastError();
}

hipError_t launch_combine(const Dims &d, const float *o, const int32_t *slot_row, uint16_t *y,
                          hipStream_t s) {
    hipLaunchKernelGGL(k_combine, dim3(grid_for(d.T * (d.H / 4))), dim3(256), 0, s, o, slot_row,
                       d.T, d.H, d.k, y);
    return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t *x, int64_t rows, int cols, uint8_t *q8, hipStream_t s) {
    const int64_t nblk = rows * (cols / 32);
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL(k_quantize, dim3(grid_for(nblk)), dim3(256), 0, s, x, rows, cols, q8);
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
