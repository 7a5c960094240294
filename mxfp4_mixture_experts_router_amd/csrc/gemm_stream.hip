// Weight-streaming expert projections for a few tokens (batched decode) on gfx950's
// block-scaled MFMA.
//
// ZeroModels GPT-OSS page, "MXFP4 experts": on decode only the routed experts' packed
// weights are touched, and the layer's time is the time to read them once from HBM. The
// work is cut into items (routed expert e, tile of 64 weight rows, group of up to 8 of e's
// routed pairs):
//   up:   h[n, 32 tile + i] = swiglu(x[t] . Wgu[e, 64 tile + 2i] + b, x[t] . Wgu[e, 64 tile + 2i + 1] + b)
//   down: part[n, 64 tile + d] = w[n] * (h[n] . Wdn[e, 64 tile + d] + bdn[e, 64 tile + d])
// for the group's pairs n = t*k + j (increasing n). The weights stay packed: each 16-byte
// MXFP4 block, as stored, is the B operand of v_mfma_scale_f32_16x16x128_f8f6f4
// (mx_mfma.h); the activations are exact E4M3 hi/lo pairs (16 A rows for 8 pairs).
//
// Persistent workgroups of four wavefronts walk the items; the items of one weight tile
// (its pair groups) are consecutive and run at the same time on one XCD, so the tile is
// read from HBM once and shared through that XCD's L2. Per item, every wavefront first
// copies its share of the group's activation rows (all of the contraction, straight into
// LDS with global_load_lds), then requests its 16 weight rows, up to 12 chunks of 256
// contraction entries ahead (whole 128-byte lines per load instruction). Memory requests
// are served roughly in issue order, so the activations land first; the wavefront waits for
// them alone (vmcnt), one barrier publishes them, and the contraction then runs without
// barriers, each chunk waiting only for its own weight registers.
//
// The up-projection writes h as a plain mx8 matrix of T k rows (64 weight rows = 32 values
// of h = one MX block per pair and tile); the down-projection writes fp32 partial rows that
// a combine kernel adds in slot order.
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "mx_mfma.h"
#include "routing.h"
#include "weight_tiles.h"

namespace moe {
namespace {

constexpr int kWaves = 4;                     // wavefronts per workgroup, 16 weight rows each
constexpr int kThreads = kWaves * kWave;
constexpr int kRowsW = 16 * kWaves;           // weight rows per item
constexpr int kPairs = 8;                     // routed pairs per item (16 A rows)
constexpr int kUB = 12;                       // weight chunks in flight per wavefront
constexpr int kMaxN = kMaxRows * 8;           // routed pairs: T <= 64, k <= 8
constexpr int kHP = 33;                       // up epilogue: padded row of 32 fp32 values
constexpr int kBlocksPerXcd = 64;             // persistent workgroups: 2 per CU
constexpr int kGrid = 8 * kBlocksPerXcd;

// LDS bytes of the dynamic area for contraction length K.
inline size_t stream_lds_bytes(int K) {
    const int nblocks = K / 32, nchunks = (nblocks + 7) / 8;
    return static_cast<size_t>(nchunks) * 4096 + 2048 + kWaves * static_cast<size_t>((16 * nblocks + 15) & ~15);
}

// A layout in LDS, per chunk c (4 KB): step h (2 KB) holds the 16 A rows' pieces of the
// blocks 8c + h + 2v, v = 0..3 (the weight lane group g holds block 8c + 2g + h); per A row
// R (128 bytes), 16-byte piece j = half j % 2 of block 8c + h + 2 (j / 2), stored at position
// j ^ (R & 7) (conflict-free operand reads). A row R is part R % 2 (hi, lo) of pair R / 2.
template <bool UP>
__global__ __launch_bounds__(kThreads) void k_stream(
    const uint8_t *__restrict__ a8, int64_t a_rows,   // mx8 activations: up x8 (T rows), down h8 (T k rows)
    // (the weight pointers are deliberately not __restrict__: their loads must stay on their
    // side of the copies' wait, which counts them)
    const uint8_t *wblocks, const uint8_t *wscales, const uint16_t *wbias, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ topk_w, int T, int E, int k, int K, int Nrows, float alpha, float limit,
    uint8_t *h8, float *part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    __shared__ int s_idx[kMaxN];
    __shared__ float s_w[kMaxN];
    __shared__ int s_pairs[kMaxN];        // pairs sorted by expert, increasing n within one
    __shared__ int s_cnt[kMaxE];          // pairs per expert, then the running placement count
    __shared__ int s_off[kMaxE + 1];      // first sorted pair of expert e
    __shared__ int s_icum[kMaxE + 1];     // first item of expert e
    __shared__ float s_h[kPairs * kHP];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int m = lane & 15, g = lane >> 4;
    const int N = T * k;
    const int nblocks = K / 32, nchunks = (nblocks + 7) / 8;
    const int kbytes = K / 2;
    const int ass = mx8_scale_stride(K);
    const int ntiles = (Nrows + kRowsW - 1) / kRowsW;
    uint8_t *s_a = dyn;                                   // [nchunks][2][16][128]
    uint8_t *s_asc = dyn + nchunks * 4096;                // [16][ass] (2 KB: ass <= 128)
    uint8_t *s_wsc = s_asc + 2048;                        // [kWaves][16 rows x nblocks]
    uint8_t *my_sc = s_wsc + wave * ((16 * nblocks + 15) & ~15);

    // --- routing, once per workgroup: pairs counted and stably sorted by expert; expert e
    // has ntiles * ceil(cnt / kPairs) items, tile-major, pair group fastest
    for (int e = tid; e < E; e += kThreads) s_cnt[e] = 0;
    __syncthreads();
    for (int n = tid; n < N; n += kThreads) {
        const int e = topk_idx[n];
        s_idx[n] = e;
        s_w[n] = topk_w != nullptr ? topk_w[n] : 0.f;
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    if (wave == 0) {
        // exclusive scans of the pair counts and of the item counts (E <= 256: 4 per lane)
        int pc[4], ic[4], lp = 0, li = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * lane + c;
            pc[c] = e < E ? s_cnt[e] : 0;
            ic[c] = ntiles * ((pc[c] + kPairs - 1) / kPairs);
            lp += pc[c];
            li += ic[c];
        }
        int ip = lp, ii = li;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int a = __shfl_up(ip, off), b = __shfl_up(ii, off);
            if (lane >= off) {
                ip += a;
                ii += b;
            }
        }
        int rp = ip - lp, ri = ii - li;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * lane + c;
            if (e < E) {
                s_off[e] = rp;
                s_icum[e] = ri;
                s_cnt[e] = 0;
            }
            rp += pc[c];
            ri += ic[c];
        }
        if (lane == kWave - 1) {
            s_off[E] = ip;
            s_icum[E] = ii;
        }
        __builtin_amdgcn_wave_barrier();
        // stable placement, 64 pairs at a time in order of n
        for (int n0 = 0; n0 < N; n0 += kWave) {
            const int n = n0 + lane;
            const int e = n < N ? s_idx[n] : -1;
            const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
            const uint64_t peers = same_expert_lanes(e, valid);
            const int base = valid ? s_cnt[e] : 0;
            __builtin_amdgcn_wave_barrier();
            if (valid) {
                s_pairs[s_off[e] + base + __popcll(peers & lanemask_lt())] = n;
                if ((peers & lanemask_lt()) == 0) s_cnt[e] = base + __popcll(peers);
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
    const int items = s_icum[E];

    // per-lane constants of the activation copies: 1 KB copy q = 4c + 2h + i fills A rows
    // 8i + lane/8 of step (c, h) at piece position lane%8, i.e. source piece
    // j = (lane%8) ^ (row & 7)
    const int j = (lane & 7) ^ ((lane >> 3) & 7);
    const uint32_t pj = 64 * (j >> 1) + 16 * (j & 1);    // byte of piece j within the step
    const int bj = 2 * (j >> 1);                          // its block, relative to 8c + h
    const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)s_a;
    const uint32_t lasc = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)s_asc;
    const uint8_t *a_sc = a8 + static_cast<size_t>(2 * a_rows) * K;
    const int ncopies = 4 * nchunks;
    const int per = ass / 16;                 // 16-byte pieces per A scale row
    const int sc_pieces = 16 * per;           // of all 16 rows (<= 128: wavefronts 0 and 1)

    // XCD-aware walk: chunk c8 of kBlocksPerXcd consecutive items runs on XCD c8 % 8, item
    // c8 kBlocksPerXcd + lb on that XCD's lb-th workgroup
    const int xcd = blockIdx.x & 7, lb = blockIdx.x >> 3;
    for (int c8 = xcd; c8 * kBlocksPerXcd < items; c8 += 8) {
        const int item = c8 * kBlocksPerXcd + lb;
        if (item >= items) continue;   // uniform
        int lo = 0, hi = E - 1;                           // last e with s_icum[e] <= item
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_icum[mid] <= item) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int cnt = s_off[e + 1] - s_off[e];
        const int ng = (cnt + kPairs - 1) / kPairs;
        const int local = item - s_icum[e];
        const int tile = local / ng, grp = local % ng;
        const int p0 = s_off[e] + kPairs * grp;                     // first sorted pair
        const int ne = min(kPairs, cnt - kPairs * grp);              // pairs of this item

        // this wavefront's 16 weight rows (a wavefront past the matrix's last row repeats
        // the last 16 rows and stores nothing)
        const int wr0 = tile * kRowsW + 16 * wave;
        const bool wvalid = wr0 < Nrows;
        const int wrb = wvalid ? wr0 : Nrows - 16;
        const int64_t grow = static_cast<int64_t>(e) * Nrows + wrb;
        const uint8_t *wrows = wblocks + grow * kbytes;

        // 1. the activation rows: copies q = wave, wave + 4, ...; then the A scales
        // (wavefronts 0 and 1, 64 pieces each; the tail repeats the last piece)
        auto src_row = [&](int R) -> uint32_t {
            const int n = s_pairs[p0 + ((R >> 1) < ne ? (R >> 1) : 0)];
            return static_cast<uint32_t>(2 * (UP ? n / k : n) + (R & 1));
        };
        {
            const uint32_t rsrc0 = src_row(lane >> 3) * static_cast<uint32_t>(K);
            const uint32_t rsrc1 = src_row(8 + (lane >> 3)) * static_cast<uint32_t>(K);
            for (int q = wave; q < ncopies; q += kWaves) {
                const int c = q >> 2, h = (q >> 1) & 1;
                // pieces past K re-read the row's first piece (finite data the multiply zeroes)
                const uint32_t off = 8 * c + h + bj < nblocks ? 32 * (8 * c + h) + pj : 0u;
                dma16(a8, ((q & 1) ? rsrc1 : rsrc0) + off, la + 1024 * q);
            }
            if (wave < 2) {
                const int pp = min(64 * wave + lane, sc_pieces - 1);
                dma16(a_sc, src_row(pp / per) * static_cast<uint32_t>(ass) + 16 * (pp % per), lasc + 1024 * wave);
            }
        }
        // 2. the weight rows' scales (dwords), the bias, the first kUB weight chunks: exactly
        // 9 + 2 kUB load instructions (indices are clamped, not tested, and made opaque so
        // that repeated addresses are not merged)
        uint32_t scw[8];
        const uint32_t *srow = reinterpret_cast<const uint32_t *>(wscales + grow * nblocks);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            int i = min(lane + kWave * q, 4 * nblocks - 1);
            asm volatile("" : "+v"(i));
            scw[q] = srow[i];
        }
        const uint16_t bias_raw = wbias[grow + m];
        uint4 wf[kUB], ws[kUB];
#pragma unroll
        for (int u = 0; u < kUB; ++u) {
            int cu = min(u, nchunks - 1);
            asm volatile("" : "+s"(cu));
            load_tile_chunk(wrows, kbytes, cu, nblocks, lane, wf[u], ws[u]);
        }
        // 3. this wavefront's copies have landed once at most the 9 + 2 kUB younger loads
        // are pending; one barrier then publishes every wavefront's copies
        wait_vm<9 + 2 * kUB>();
        wait_lgkm0();
        barrier_only();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int i = lane + kWave * q;
            if (i < 4 * nblocks) reinterpret_cast<uint32_t *>(my_sc)[i] = scw[q];
        }

        // 4. the contraction
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < nchunks; c0 += kUB) {
#pragma unroll
            for (int u = 0; u < kUB; ++u) {
                const int c = c0 + u;
                if (c < nchunks) {   // uniform
                uint4 blo, bhi;
                tile_chunk_to_mfma(wf[u], ws[u], lane, blo, bhi);
                if (c + kUB < nchunks) load_tile_chunk(wrows, kbytes, c + kUB, nblocks, lane, wf[u], ws[u]);
                const bool last = 8 * c + 8 > nblocks;   // uniform: blocks past K in this chunk
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint8_t *base = s_a + (2 * c + h) * 2048;
                    uint4 f = *reinterpret_cast<const uint4 *>(base + m * 128 + 16 * (g ^ (m & 7)));
                    uint4 sc = *reinterpret_cast<const uint4 *>(base + m * 128 + 16 * ((g + 4) ^ (m & 7)));
                    uint32_t sa = s_asc[m * ass + 8 * c + 2 * g + h];
                    const uint32_t sb = my_sc[m * nblocks + min(8 * c + 2 * g + h, nblocks - 1)];
                    if (last) {
                        // lane group g: pieces of blocks 8c + h + 2(g/2) and + 4; scale of 8c + 2g + h
                        if (8 * c + h + 2 * (g >> 1) >= nblocks) f = zero4();
                        if (8 * c + h + 4 + 2 * (g >> 1) >= nblocks) sc = zero4();
                        if (8 * c + 2 * g + h >= nblocks) sa = 127u;
                    }
                    acc = mfma_mx(mx_a_operand(f, sc), mx_b_operand(h ? bhi : blo), acc, sa, sb);
                }
                }
            }
        }

        // 5. epilogue. Lane (m, g) holds weight row m of the wavefront and A rows 4g + r:
        // pair 2g + r/2, part r % 2; value = D[hi] + D[lo].
        const float bias = bf16_to_f32(bias_raw);
        if (UP) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int s = 2 * g + jj;
                const float v = acc[2 * jj] + acc[2 * jj + 1] + bias;
                const float other = __shfl_xor(v, 1);   // even row m: gate, odd: up
                if ((m & 1) == 0 && s < ne) s_h[s * kHP + 8 * wave + (m >> 1)] = swiglu(v, other, alpha, limit);
            }
            __syncthreads();
            // each pair's 32 values (one MX block of its h8 rows) on eight lanes of wavefront 0,
            // four values each: the block maximum by three lane exchanges, then each lane splits
            // and stores its own four hi and four lo bytes (the same bytes store_mx8_block writes)
            if (wave == 0) {
                const int sl = lane >> 3, j = lane & 7;
                float v[4] = {0.f, 0.f, 0.f, 0.f};
                if (sl < ne)
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = s_h[sl * kHP + 4 * j + i];
                float mx = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
                mx = fmaxf(mx, lane_xor1(mx));
                mx = fmaxf(mx, lane_xor2(mx));
                mx = fmaxf(mx, __shfl_xor(mx, 4));
                if (sl < ne) {
                    const int eb = mx8_block_exponent(mx);
                    uint32_t hi, lo;
                    mx8_split4(ldexpf(v[0], -eb), ldexpf(v[1], -eb), ldexpf(v[2], -eb), ldexpf(v[3], -eb), hi, lo);
                    const int Iw = Nrows / 2, ss = mx8_scale_stride(Iw);
                    uint8_t *h_sc = h8 + static_cast<size_t>(2 * N) * Iw;
                    const int64_t n = s_pairs[p0 + sl];
                    reinterpret_cast<uint32_t *>(h8 + (2 * n) * Iw + 32 * tile)[j] = hi;
                    reinterpret_cast<uint32_t *>(h8 + (2 * n + 1) * Iw + 32 * tile)[j] = lo;
                    if (j == 0) {
                        h_sc[(2 * n) * ss + tile] = static_cast<uint8_t>(127 + eb);
                        h_sc[(2 * n + 1) * ss + tile] = static_cast<uint8_t>(123 + eb);
                    }
                }
            }
        } else if (wvalid) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int s = 2 * g + jj;
                if (s < ne) {
                    const int n = s_pairs[p0 + s];
                    part[static_cast<int64_t>(n) * Nrows + wr0 + m] = (acc[2 * jj] + acc[2 * jj + 1] + bias) * s_w[n];
                }
            }
        }
        __syncthreads();   // the activation and epilogue buffers are free for the next item
    }
}

template <bool UP>
hipError_t stream(const Dims &d, const uint8_t *a8, int64_t a_rows, const uint8_t *blocks, const uint8_t *scales,
                  const uint16_t *bias, const int32_t *idx, const float *w, int K, int Nrows, uint8_t *h8,
                  float *part, hipStream_t s) {
    const size_t lds = stream_lds_bytes(K);
    if (lds > 65536) {   // long contractions: allow more than the default 64 KB
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_stream<UP>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (err != hipSuccess) return err;
    }
    MOE_LAUNCH((k_stream<UP>), dim3(kGrid), dim3(kThreads), lds, s, a8, a_rows, blocks, scales,
               bias, idx, w, static_cast<int>(d.T), d.E, d.k, K, Nrows, d.alpha, d.limit, h8, part);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_up_stream(const Dims &d, const uint8_t *x8, const uint8_t *gu_blocks, const uint8_t *gu_scales,
                            const uint16_t *gu_bias, const int32_t *topk_idx, uint8_t *h8, hipStream_t s) {
    return stream<true>(d, x8, d.T, gu_blocks, gu_scales, gu_bias, topk_idx, nullptr, d.H, 2 * d.I, h8, nullptr, s);
}

hipError_t launch_down_stream(const Dims &d, const uint8_t *h8, const uint8_t *dn_blocks, const uint8_t *dn_scales,
                              const uint16_t *dn_bias, const int32_t *topk_idx, const float *topk_w, float *part,
                              hipStream_t s) {
    return stream<false>(d, h8, d.T * d.k, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, d.I, d.H, nullptr,
                         part, s);
}

}  // namespace moe
