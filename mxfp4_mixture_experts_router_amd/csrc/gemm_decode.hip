// Decode path (T <= 64): weight-streaming expert GEMMs on gfx950's block-scaled MFMA.
//
// ZeroModels GPT-OSS page, "MXFP4 experts": on decode only the routed experts' packed
// weights are touched and the bank stays packed. Here the packed MXFP4 blocks are not
// dequantized at all: each 16-byte block, as stored, is the B operand of
// v_mfma_scale_f32_16x16x128_f8f6f4 with its E8M0 byte as the B scale (see mx_mfma.h). The
// activations enter as exact E4M3 hi/lo pairs (two A rows per activation row), written once
// per call by their producer: the router kernel for x, the up-projection's epilogue for the
// SwiGLU output h. Each packed weight byte is read from HBM exactly once per call.
//
// Streaming a few MB per call at HBM speed needs every workgroup's share of the packed
// weights in flight at once: each wavefront issues all (or a large batch) of its 16-byte
// weight loads before its first MFMA, and the activation rows (a few KB) are staged in LDS
// while those loads are outstanding. Each load instruction covers 8 rows x 128 contiguous
// bytes (whole cache lines); one lane exchange then gives every lane two blocks of one row
// (load_tile_chunk / tile_chunk_to_mfma).
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "mx_mfma.h"
#include "routing.h"
#include "weight_tiles.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kDownScaleLds = 16384;  // LDS bytes for the routed experts' scale rows (few tokens)
constexpr int kStageLds = 24 * 1024;  // LDS bytes for staged E4M3 activation rows

// Routing of all T tokens into LDS: s_idx / s_w [T*k]. With `logits` (double [T, E]) the
// top-k + softmax is computed here by every block (wavefront w < 4 handles tokens w, w+4, ...)
// and block 0 also writes it to topk_idx / topk_w; otherwise it is read from them.
// The first routing loads are issued before `stage()` (the caller's routing-independent
// loads), so both latencies overlap. Then bitmap = the set of routed experts. Ends with a
// block barrier.
template <bool WITH_LOGITS, typename Stage>
__device__ __forceinline__ void load_routing(const double *logits, int32_t *topk_idx, float *topk_w, int T, int E,
                                             int k, int *s_idx, float *s_w, uint32_t *bitmap, Stage &&stage) {
    constexpr int kPre = 2;                 // routing entries per thread loaded up front
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    // the wavefront's routing role: tokens wr, wr + 4, ..; rotated with the workgroup so that
    // the workgroups sharing a CU run their top-k on different SIMDs
    const int wr = (wave + static_cast<int>(blockIdx.x)) & 3;
    const int N = T * k;
    if (tid < kMaxE / 32) bitmap[tid] = 0u;
    double lg0[kMaxE / kWave];
    int32_t pi[kPre];
    float pw[kPre];
    if (WITH_LOGITS && logits) {
#pragma unroll
        for (int c = 0; c < kMaxE / kWave; ++c) {
            const int e = lane + kWave * c;
            lg0[c] = (wave < 4 && wr < T && e < E) ? logits[static_cast<int64_t>(wr) * E + e] : 0.0;
        }
    } else {
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int n = tid + q * static_cast<int>(blockDim.x);
            pi[q] = n < N ? topk_idx[n] : 0;
            pw[q] = n < N ? topk_w[n] : 0.f;
        }
    }
    stage();
    if constexpr (WITH_LOGITS) {
        __shared__ __attribute__((aligned(16))) uint64_t s_tk[4][kTopkScratch];
        if (logits && wave < 4) {
            const bool writer = blockIdx.x == 0;
            for (int t = wr; t < T; t += 4) {
                if (t != wr) {
#pragma unroll
                    for (int c = 0; c < kMaxE / kWave; ++c) {
                        const int e = lane + kWave * c;
                        lg0[c] = e < E ? logits[static_cast<int64_t>(t) * E + e] : 0.0;
                    }
                }
                topk_softmax_values(lg0, E, k, lane, s_idx + t * k, s_w + t * k,
                                    writer ? topk_idx + t * k : nullptr, writer ? topk_w + t * k : nullptr,
                                    s_tk[wave]);
            }
        }
    }
    if (!WITH_LOGITS || !logits) {
#pragma unroll
        for (int q = 0; q < kPre; ++q) {
            const int n = tid + q * static_cast<int>(blockDim.x);
            if (n < N) {
                s_idx[n] = pi[q];
                s_w[n] = pw[q];
            }
        }
        for (int n = tid + kPre * static_cast<int>(blockDim.x); n < N; n += blockDim.x) {
            s_idx[n] = topk_idx[n];
            s_w[n] = topk_w[n];
        }
    }
    __syncthreads();
    for (int n = tid; n < N; n += blockDim.x) {
        const int e = s_idx[n];
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicOr(&bitmap[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
}

// Copy `bytes` contiguous bytes (a multiple of 16) into LDS; each thread issues up to 4
// loads before its first LDS store (clamped slots reload and rewrite the last piece).
__device__ __forceinline__ void stage_bytes(uint8_t *dst, const uint8_t *src, int bytes) {
    const int total = bytes / 16;
    const int nt = blockDim.x;
    auto ld = [&](int q) { return *reinterpret_cast<const uint4 *>(src + 16 * static_cast<int64_t>(q)); };
    auto st = [&](int q, uint4 v) { *reinterpret_cast<uint4 *>(dst + 16 * q) = v; };
    for (int base = threadIdx.x; base < total; base += 4 * nt) {
        const int q0 = base, q1 = min(base + nt, total - 1), q2 = min(base + 2 * nt, total - 1),
                  q3 = min(base + 3 * nt, total - 1);
        const uint4 v0 = ld(q0), v1 = ld(q1), v2 = ld(q2), v3 = ld(q3);
        st(q0, v0);
        st(q1, v1);
        st(q2, v2);
        st(q3, v3);
    }
}

// One block-scaled MFMA over the blocks 8c + 2v + h (v = 0..3) of chunk c, h = 0 or 1: B is
// the lane's block 8c + 2g + h (from tile_chunk_to_mfma) with scale sb. arow: E4M3 row of the
// lane's A row m, asc: its scale row; with !valid (a zero row) they point at any real row.
// Blocks past nblocks contribute 0. The reads are unconditional (indices clamped into the
// row) and the zeroing is by selects, so a step has no divergent branches.
__device__ __forceinline__ f32x4 mx_step(f32x4 acc, const uint8_t *arow, const uint8_t *asc, bool valid,
                                         const i32x8 &bop, uint32_t sb, int c, int h, int g, int nblocks) {
    const int b0 = 8 * c + 2 * (g >> 1) + h;    // A bytes 0-15: virtual block g/2
    const int b1 = b0 + 4;                      // A bytes 16-31: virtual block 2 + g/2
    const int kb = 8 * c + 2 * g + h;           // the lane group's own (virtual g) block
    const int last = nblocks - 1;
    uint4 f = *reinterpret_cast<const uint4 *>(arow + min(b0, last) * 32 + 16 * (g & 1));
    uint4 s = *reinterpret_cast<const uint4 *>(arow + min(b1, last) * 32 + 16 * (g & 1));
    const uint32_t sa = asc[min(kb, last)];
    const uint32_t m0 = valid && b0 <= last ? ~0u : 0u, m1 = valid && b1 <= last ? ~0u : 0u;
    f = make_uint4(f.x & m0, f.y & m0, f.z & m0, f.w & m0);
    s = make_uint4(s.x & m1, s.y & m1, s.z & m1, s.w & m1);
    return mfma_mx(mx_a_operand(f, s), bop, acc, valid && kb <= last ? sa : 127u, sb);
}

// ---------------------------------------------------------------------------------------
// Up-projection. Block = (routing slot, 16 gate/up pairs = 32 interleaved rows = two 16-row
// tiles); wavefront w takes tile w % 2 and every other 256-wide chunk of H (parity w / 2);
// the two halves are added through LDS.
//   h[n, i] = w[n] * swiglu(x[t] . Wgu[e, 2i] + bgu[e, 2i], x[t] . Wgu[e, 2i+1] + bgu[e, 2i+1])
// for every pair n = t*k + j routed to expert e (the slot-th routed expert). Column c of
// tile q is row 16q + c of the block: pair 8q + c/2, gate for even c, up for odd.
// h is written as an mx8 matrix of 2 T k rows: row 2n + half holds the block's 16 values
// (half = (i0 / 16) % 2 of MX block i0 / 32) and zeros in the other half, so every 16
// values get their own exponent and a block never needs its neighbour's values; the down
// projection reads 4 A rows (h8 rows 4n .. 4n + 3) per pair.
// A rows: 2 per routed pair (hi, lo of x8 row 2t, 2t + 1); block y takes the expert's pairs
// 8 NMT y .. 8 NMT (y + 1) - 1 in NMT 16-row m-tiles; UB chunks per wavefront per load batch
// (two loads each). With LDS_A the E4M3 token rows are staged in LDS; the token scales
// always are. With `logits` the routing (top-k + softmax) is computed in the prologue, see
// load_routing.
template <int NMT, int UB, bool LDS_A, bool WITH_LOGITS>
__global__ __launch_bounds__(256) void k_up_mx(
    const uint8_t *__restrict__ x8, const uint8_t *__restrict__ xs8, const uint8_t *__restrict__ gu_blocks,
    const uint8_t *__restrict__ gu_scales, const uint16_t *__restrict__ gu_bias,
    const double *__restrict__ logits, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int T, int H, int I, int E, int k, float alpha, float limit, uint8_t *__restrict__ h8,
    uint8_t *__restrict__ hs8) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    __shared__ uint32_t bitmap[kMaxE / 32];
    __shared__ int s_idx[kMaxRows * 8];
    __shared__ float s_w[kMaxRows * 8];
    __shared__ int s_rows[kMaxRows];
    __shared__ int s_nrows;
    // chunk-half partial sums, later the slots' SwiGLU outputs [slot][17]
    constexpr int kRed = 2 * NMT * 4 * kWave > kMaxRows * 17 ? 2 * NMT * 4 * kWave : kMaxRows * 17;
    __shared__ float s_red[kRed];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;
    const int tiles_i = I / 16;
    const int N = T * k;
    const int hs = H / 32, sxs = mx8_scale_stride(H);
    uint8_t *xs_lds = dyn + (LDS_A ? 2 * T * H : 0);
    // the token rows (E4M3) and their scales into LDS, overlapped with the routing loads
    load_routing<WITH_LOGITS>(logits, topk_idx, topk_w, T, E, k, s_idx, s_w, bitmap, [&] {
        if (LDS_A) stage_bytes(dyn, x8, 2 * T * H);
        stage_bytes(xs_lds, xs8, 2 * T * sxs);
    });
    const int e = expert_of_slot(bitmap, blockIdx.x / tiles_i);
    if (e < 0) return;  // fewer routed experts than slots (uniform over the block)
    const int i0 = (blockIdx.x % tiles_i) * 16;

    const int64_t row0 = static_cast<int64_t>(e) * 2 * I + 2 * i0;   // first of the 32 rows
    const int hb = H / 2;
    const int nblocks = hs;
    const int nchunks = (nblocks + 7) / 8;
    const int q = wave & 1, p = wave >> 1;
    // each chunk's two scale bytes per lane (row 16q + col, blocks 8c + 2g and 8c + 2g + 1)
    // are requested just ahead of its weights, so a chunk is usable as soon as it arrives
    const uint8_t *wrows = gu_blocks + (row0 + 16 * q) * hb;
    const uint8_t *srow = gu_scales + (row0 + 16 * q + col) * hs;
    uint4 wf[UB], ws[UB];
    uint32_t sclo[UB], schi[UB];
    auto load_batch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int cu = min(c0 + 2 * u, nchunks - 1);
            sclo[u] = srow[min(8 * cu + 2 * g, nblocks - 1)];
            schi[u] = srow[min(8 * cu + 2 * g + 1, nblocks - 1)];
            load_tile_chunk(wrows, hb, cu, nblocks, lane, wf[u], ws[u]);
        }
    };
    load_batch(p);
    const float bias = bf16_to_f32(gu_bias[row0 + 16 * q + col]);

    if (wave == 0) rows_of_expert(s_idx, N, e, s_rows, &s_nrows);
    // LDS writes done; the weight loads stay in flight across the barrier (a full
    // __syncthreads would wait for them), so the contraction starts with the first chunk
    wait_lgkm0();
    barrier_only();
    const int s0 = 8 * NMT * blockIdx.y;       // first slot (routed pair of e) of this block
    const int nrows = s_nrows - s0;            // slots of this block (may exceed 8 NMT)
    if (nrows <= 0) return;                    // uniform
    // A row r = 16 mt + col: slot s0 + r / 2, part r % 2 (hi, lo) -> x8 row 2 t + part
    const uint8_t *arow[NMT];
    const uint8_t *asc[NMT];
    bool avalid[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const int r = 16 * mt + col;
        arow[mt] = LDS_A ? dyn : x8;     // a real row; zeroed by !avalid
        asc[mt] = xs_lds;
        avalid[mt] = false;
        if ((r >> 1) < nrows) {
            const int xr = 2 * (s_rows[s0 + (r >> 1)] / k) + (r & 1);
            arow[mt] = (LDS_A ? dyn : x8) + static_cast<int64_t>(xr) * H;
            asc[mt] = xs_lds + xr * sxs;
            avalid[mt] = true;
        }
    }

    f32x4 acc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = p; c0 < nchunks; c0 += 2 * UB) {
        if (c0 != p) load_batch(c0);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int c = c0 + 2 * u;
            if (c >= nchunks) break;   // uniform
            uint4 lo, hi;
            tile_chunk_to_mfma(wf[u], ws[u], lane, lo, hi);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t sb = h ? schi[u] : sclo[u];
                const i32x8 bop = mx_b_operand(h ? hi : lo);
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt)
                    if (16 * mt < 2 * nrows) acc[mt] = mx_step(acc[mt], arow[mt], asc[mt], avalid[mt], bop, sb, c, h, g, nblocks);
            }
        }
    }

    // the second chunk half hands its sums to the first
    float(*red)[NMT * 4][kWave] = reinterpret_cast<float(*)[NMT * 4][kWave]>(s_red);   // [2] tiles
    if (p == 1)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[q][mt * 4 + r][lane] = acc[mt][r];
    __syncthreads();
    if (p == 0)
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[mt][r] += red[q][mt * 4 + r][lane];
    __syncthreads();   // s_red is reused for the SwiGLU outputs below
    float(*s_h)[17] = reinterpret_cast<float(*)[17]>(s_red);
    if (p == 0) {
        // D rows 16mt + 4g + r: slot 8mt + 2g + r/2, part r % 2
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int s = 8 * mt + 2 * g + j;   // local slot
                const float v = acc[mt][2 * j] + acc[mt][2 * j + 1] + bias;
                const float other = lane_xor1(v);
                if ((col & 1) == 0 && s < nrows)
                    s_h[s][8 * q + col / 2] = swiglu(v, other, alpha, limit) * s_w[s_rows[s0 + s]];
            }
    }
    __syncthreads();
    // each slot's 16 outputs: one half of MX block i0 / 32 of h8 row 2n + half, the other
    // half zero. 8 threads per slot: thread j < 4 converts values 4j .. 4j + 3, threads
    // j >= 4 write the zero words; the block exponent comes from the max over the group.
    {
        const int half = (i0 / 16) & 1;
        const int sl = tid >> 3, j = tid & 7;
        const bool live = sl < nrows && sl < 8 * NMT;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (live && j < 4)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = s_h[sl][4 * j + i];
        float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        m = fmaxf(m, lane_xor1(m));
        m = fmaxf(m, lane_xor2(m));
        m = fmaxf(m, __shfl_xor(m, 4));
        if (live) {
            const int eb = mx8_block_exponent(m);
            uint32_t hi = 0u, lo = 0u;
            if (j < 4) mx8_split4(ldexpf(v[0], -eb), ldexpf(v[1], -eb), ldexpf(v[2], -eb), ldexpf(v[3], -eb), hi, lo);
            const int64_t r = 2 * (2 * static_cast<int64_t>(s_rows[s0 + sl]) + half);   // hi byte row
            const int b = i0 / 32;
            // word w of the 32-byte block: values in words 4 half .. 4 half + 3
            const int w = j < 4 ? 4 * half + j : 4 * (1 - half) + (j - 4);
            reinterpret_cast<uint32_t *>(h8 + r * I + 32 * b)[w] = hi;
            reinterpret_cast<uint32_t *>(h8 + (r + 1) * I + 32 * b)[w] = lo;
            if (j == 0) {
                const int ss = mx8_scale_stride(I);
                hs8[r * ss + b] = static_cast<uint8_t>(127 + eb);
                hs8[(r + 1) * ss + b] = static_cast<uint8_t>(123 + eb);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// Down-projection with the combine folded in (few tokens). Block = one 16-row tile of output
// features d for every token; NW wavefronts share the (routed expert, 256-wide chunk of I)
// work units. For routed expert e the A rows of token t are the four h8 rows 4n .. 4n + 3
// (hi/lo of both halves, see k_up_mx) when pair n = t*k + j has idx[t, j] == e, else zero,
// so all experts accumulate into the same per-token tile:
//   y[t, d] = bf16( sum_{e, i} h_e[t, i] * Wdn[e, d, i]  +  sum_j w[t, j] * bdn[e_tj, d] ).
// (h already carries the routing weight.) The wavefronts' partial tiles are reduced through
// LDS in wavefront order. A rows 4t + sub, NMT = ceil(T / 4) m-tiles. With LDS_A the h8 rows
// are staged in LDS; their scales always are. With SC_LDS the weight scale rows of all
// routed experts are staged in LDS up front (they must fit kDownScaleLds bytes); otherwise
// each unit loads its scale bytes along with its weights.
template <int NMT, int NW, int UB, bool LDS_A, bool SC_LDS>
__global__ __launch_bounds__(NW * 64) void k_down_mx_tokens(
    const uint8_t *__restrict__ h8, const uint8_t *__restrict__ hs8, const uint8_t *__restrict__ dn_blocks,
    const uint8_t *__restrict__ dn_scales, const uint16_t *__restrict__ dn_bias,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int T, int H, int I, int E, int k,
    const uint16_t *__restrict__ res, uint16_t *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
    __shared__ uint32_t bitmap[kMaxE / 32];
    __shared__ int s_idx[16 * 8];
    __shared__ float s_w[16 * 8];
    __shared__ int s_experts[kMaxE];
    __shared__ int s_rowof[16 * 8][16];     // [routed expert slot][token] -> pair n, or -1
    __shared__ int s_na;
    __shared__ float red[NW][NMT * 4][kWave];
    __shared__ float s_bprod[16 * 8][16];   // [pair n][feature] w[n] * bdn[e_n, d0 + feature]
    __shared__ __attribute__((aligned(16))) uint8_t s_sc[SC_LDS ? kDownScaleLds : 16];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;
    const int d0 = blockIdx.x * 16;
    const int N = T * k;        // T <= 16 here
    const int shs = mx8_scale_stride(I);
    uint8_t *hs_lds = dyn + (LDS_A ? 4 * N * I : 0);
    // the h rows (E4M3) and their scales into LDS, overlapped with the routing loads
    load_routing<false>(nullptr, topk_idx, topk_w, T, E, k, s_idx, s_w, bitmap, [&] {
        if (LDS_A) stage_bytes(dyn, h8, 4 * N * I);
        stage_bytes(hs_lds, hs8, 4 * N * shs);
    });
    if (tid < kMaxE / 32) {
        int before = 0;
        for (int w = 0; w < tid; ++w) before += __popc(bitmap[w]);
        uint32_t bits = bitmap[tid];
        while (bits) {
            s_experts[before++] = 32 * tid + __ffs(bits) - 1;
            bits &= bits - 1u;
        }
        if (tid == kMaxE / 32 - 1) s_na = before;
    }
    __syncthreads();
    const int na = s_na;
    for (int qq = tid; qq < na * 16; qq += NW * 64) {
        const int a = qq / 16, t = qq % 16;
        int n = -1;
        if (t < T)
            for (int j = 0; j < k; ++j)
                if (s_idx[t * k + j] == s_experts[a]) n = t * k + j;
        s_rowof[a][t] = n;
    }
    const int nblocks = I / 32;
    const int nchunks = (nblocks + 7) / 8;
    const int nunits = na * nchunks;
    const int is = I / 32;

    // the 16 rows of scales of every routed expert (I/2 contiguous bytes each), loaded before
    // the weight stream
    const int nsc = SC_LDS ? na * (I / 32) : 0;     // 16-byte pieces
    uint4 scv[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        const int idx = tid + NW * 64 * qq;
        scv[qq] = zero4();
        if (SC_LDS && idx < nsc) {
            const int a = idx / (I / 32), piece = idx % (I / 32);
            scv[qq] = *reinterpret_cast<const uint4 *>(dn_scales + (static_cast<int64_t>(s_experts[a]) * H + d0) * is + 16 * piece);
        }
    }
    constexpr int kBiasPer = (16 * 8 * 16 + NW * 64 - 1) / (NW * 64);
    uint16_t bias_v[kBiasPer];
#pragma unroll
    for (int qq = 0; qq < kBiasPer; ++qq) {
        const int idx = tid + NW * 64 * qq;
        bias_v[qq] = idx < N * 16 ? dn_bias[static_cast<int64_t>(s_idx[idx / 16]) * H + d0 + idx % 16] : 0;
    }
    // this wavefront's first batch of packed-weight loads
    uint4 wf[UB], ws[UB];
    uint32_t sclo[UB], schi[UB];
    int ua[UB], uaa[UB], ucc[UB];
    auto load_batch = [&](int u0) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            // unconditional loads at clamped indices; units past the end read a real tile and
            // are neutralised by zero activation rows
            const int unit = u0 + NW * u;
            const int uc = min(unit, nunits - 1);
            const int a = uc / nchunks, c = uc % nchunks;
            const int64_t row0 = static_cast<int64_t>(s_experts[a]) * H + d0;
            load_tile_chunk(dn_blocks + row0 * (I / 2), I / 2, c, nblocks, lane, wf[u], ws[u]);
            if (!SC_LDS) {
                const uint8_t *srow = dn_scales + (row0 + col) * is;
                sclo[u] = srow[min(8 * c + 2 * g, nblocks - 1)];
                schi[u] = srow[min(8 * c + 2 * g + 1, nblocks - 1)];
            }
            ua[u] = unit < nunits ? a : -1;
            uaa[u] = a;
            ucc[u] = c;
        }
    };
    load_batch(wave);
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
        const int idx = tid + NW * 64 * qq;
        if (SC_LDS && idx < nsc) *reinterpret_cast<uint4 *>(s_sc + 16 * idx) = scv[qq];
    }
    // bias products w[n] * bdn[e_n, d] of every pair n and feature d of the tile (loads issued
    // before the weight batch, so consuming them does not wait for it)
#pragma unroll
    for (int qq = 0; qq < kBiasPer; ++qq) {
        const int idx = tid + NW * 64 * qq;
        if (idx < N * 16) s_bprod[idx / 16][idx % 16] = s_w[idx / 16] * bf16_to_f32(bias_v[qq]);
    }
    wait_lgkm0();     // LDS writes done; the weight batch stays in flight across the barrier
    barrier_only();

    f32x4 acc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int u0 = wave; u0 < nunits; u0 += NW * UB) {
        if (u0 != wave) load_batch(u0);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            // A row r = 16 mt + col: token 4 mt + col / 4, h8 row 4n + col % 4
            const uint8_t *arow[NMT];
            const uint8_t *asc[NMT];
            bool avalid[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                const int n = ua[u] >= 0 ? s_rowof[ua[u]][4 * mt + (col >> 2)] : -1;
                const int hr = 4 * n + (col & 3);
                arow[mt] = (LDS_A ? dyn : h8) + static_cast<int64_t>(n >= 0 ? hr : 0) * I;
                asc[mt] = hs_lds + (n >= 0 ? hr : 0) * shs;
                avalid[mt] = n >= 0;
            }
            uint4 lo, hi;
            tile_chunk_to_mfma(wf[u], ws[u], lane, lo, hi);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t sb = SC_LDS ? s_sc[(uaa[u] * 16 + col) * is + min(8 * ucc[u] + 2 * g + h, nblocks - 1)]
                                           : (h ? schi[u] : sclo[u]);
                const i32x8 bop = mx_b_operand(h ? hi : lo);
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt)
                    acc[mt] = mx_step(acc[mt], arow[mt], asc[mt], avalid[mt], bop, sb, ucc[u], h, g, nblocks);
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mt * 4 + r][lane] = acc[mt][r];
    __syncthreads();
    if (wave != 0) return;
    const int64_t drow = d0 + col;
    // D rows 16mt + 4g + r: token 4mt + g, its four A rows r
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const int t = 4 * mt + g;
        if (t < T) {
            float v = 0.f;
            for (int w = 0; w < NW; ++w)
                v += (red[w][mt * 4][lane] + red[w][mt * 4 + 1][lane]) + (red[w][mt * 4 + 2][lane] + red[w][mt * 4 + 3][lane]);
            float bterm = 0.f;
            for (int jj = 0; jj < k; ++jj) bterm += s_bprod[t * k + jj][col];
            float out = v + bterm;
            if (res) out += bf16_to_f32(res[static_cast<int64_t>(t) * H + drow]);
            y[static_cast<int64_t>(t) * H + drow] = f32_to_bf16(out);
        }
    }
}

// y[t, d] = bf16(sum_{j < K} part[t*K + j, d] (+ res[t, d])) in slot order. Thread = 4
// features; its K row reads are issued together.
template <int K>
__global__ __launch_bounds__(256) void k_combine_slots(const float *__restrict__ part, int T, int H,
                                                       const uint16_t *__restrict__ res,
                                                       uint16_t *__restrict__ y) {
    const int per_row = H / 4;
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q >= T * per_row) return;
    const int t = q / per_row, d = (q % per_row) * 4;
    float4 v[K];
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = *reinterpret_cast<const float4 *>(part + static_cast<int64_t>(t * K + j) * H + d);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < K; ++j) {
        s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
    }
    if (res) add_residual4(s, res + static_cast<int64_t>(t) * H + d);
    const uint32_t lo = f32_to_bf16(s.x) | (static_cast<uint32_t>(f32_to_bf16(s.y)) << 16);
    const uint32_t hi = f32_to_bf16(s.z) | (static_cast<uint32_t>(f32_to_bf16(s.w)) << 16);
    *reinterpret_cast<uint2 *>(y + static_cast<int64_t>(t) * H + d) = make_uint2(lo, hi);
}

int slots_of(const Dims &d) { return static_cast<int>(d.T * d.k < d.E ? d.T * d.k : d.E); }

template <int NMT, int UB, bool LDS_A, bool WITH_LOGITS>
hipError_t up_n(const Dims &d, const uint8_t *x8, const uint8_t *xs8, const uint8_t *gb, const uint8_t *gs,
                const uint16_t *gbias, const double *logits, int32_t *idx, float *w, uint8_t *h8, uint8_t *hs8,
                hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>(slots_of(d) * (d.I / 16));
    const unsigned groups = static_cast<unsigned>((d.T + 8 * NMT - 1) / (8 * NMT));   // an expert has <= T pairs
    const size_t lds = (LDS_A ? static_cast<size_t>(2 * d.T) * d.H : 0) +
                       static_cast<size_t>(2 * d.T) * mx8_scale_stride(d.H);
    MOE_LAUNCH((k_up_mx<NMT, UB, LDS_A, WITH_LOGITS>), dim3(blocks, groups), dim3(256), lds, s, x8, xs8, gb, gs, gbias,
                       logits, idx, w, static_cast<int>(d.T), d.H, d.I, d.E, d.k, d.alpha, d.limit, h8, hs8);
    return hipGetLastError();
}

template <int NMT, int NW, int UB, bool LDS_A, bool SC_LDS>
hipError_t down_tokens_n(const Dims &d, const uint8_t *h8, const uint8_t *hs8, const uint8_t *db, const uint8_t *ds,
                         const uint16_t *dbias, int32_t *idx, float *w, const uint16_t *res, uint16_t *y,
                         hipStream_t s) {
    const int64_t N = d.T * d.k;
    const size_t lds = (LDS_A ? static_cast<size_t>(4 * N) * d.I : 0) +
                       static_cast<size_t>(4 * N) * mx8_scale_stride(d.I);
    MOE_LAUNCH((k_down_mx_tokens<NMT, NW, UB, LDS_A, SC_LDS>), dim3(static_cast<unsigned>(d.H / 16)),
                       dim3(NW * 64), lds, s, h8, hs8, db, ds, dbias, idx, w, static_cast<int>(d.T), d.H, d.I, d.E,
                       d.k, res, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_decode(const Dims &d, const float *part, const uint16_t *residual, uint16_t *y,
                                 hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>((d.T * (d.H / 4) + 255) / 256);
#define MOE_COMBINE(K) MOE_LAUNCH((k_combine_slots<K>), dim3(blocks), dim3(256), 0, s, part, \
                                   static_cast<int>(d.T), d.H, residual, y)
    switch (d.k) {
        case 1: MOE_COMBINE(1); break;
        case 2: MOE_COMBINE(2); break;
        case 3: MOE_COMBINE(3); break;
        case 4: MOE_COMBINE(4); break;
        case 5: MOE_COMBINE(5); break;
        case 6: MOE_COMBINE(6); break;
        case 7: MOE_COMBINE(7); break;
        default: MOE_COMBINE(8); break;
    }
#undef MOE_COMBINE
    return hipGetLastError();
}

hipError_t launch_up_decode(const Dims &d, const uint8_t *x8, const uint8_t *gu_blocks,
                            const uint8_t *gu_scales, const uint16_t *gu_bias, const double *logits,
                            int32_t *topk_idx, float *topk_w, uint8_t *h8, hipStream_t s) {
    if (d.T >= kStreamMinT || logits == nullptr) return hipErrorInvalidValue;
    const uint8_t *xs8 = x8 + static_cast<size_t>(2 * d.T) * d.H;
    uint8_t *hs8 = h8 + static_cast<size_t>(4 * d.T * d.k) * d.I;   // h8: mx8 matrix of 2 T k rows
    // the token rows (2T of H bytes) are staged in LDS when they fit
    if (mx8_bytes(d.T, d.H) <= static_cast<size_t>(kStageLds))
        return up_n<1, 6, true, true>(d, x8, xs8, gu_blocks, gu_scales, gu_bias, logits, topk_idx, topk_w, h8, hs8, s);
    return up_n<1, 6, false, true>(d, x8, xs8, gu_blocks, gu_scales, gu_bias, logits, topk_idx, topk_w, h8, hs8, s);
}

hipError_t launch_down_decode(const Dims &d, const uint8_t *h8, const uint8_t *dn_blocks,
                              const uint8_t *dn_scales, const uint16_t *dn_bias, int32_t *topk_idx,
                              float *topk_w, const uint16_t *residual, uint16_t *y, hipStream_t s) {
    if (d.T >= kStreamMinT) return hipErrorInvalidValue;
    const int64_t N = d.T * d.k;
    const uint8_t *hs8 = h8 + static_cast<size_t>(4 * N) * d.I;   // h8: mx8 matrix of 2N rows
    // weight scale rows of every routed expert: at most min(T*k, E) experts x 16 rows x I/32 bytes
    const bool sc_lds = static_cast<int64_t>(slots_of(d)) * (d.I / 2) <= kDownScaleLds;
    const bool lds_a = mx8_bytes(2 * N, d.I) <= static_cast<size_t>(kStageLds);
    if (lds_a && sc_lds)
        return down_tokens_n<1, 16, 3, true, true>(d, h8, hs8, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, residual, y, s);
    if (sc_lds)
        return down_tokens_n<1, 16, 3, false, true>(d, h8, hs8, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, residual, y, s);
    return down_tokens_n<1, 16, 3, false, false>(d, h8, hs8, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, residual, y, s);
}

}  // namespace moe
