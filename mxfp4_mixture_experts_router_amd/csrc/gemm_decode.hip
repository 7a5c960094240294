// Decode path (T <= 64): weight-streaming expert GEMMs with the MXFP4 dequantization
// fused into the register staging.
//
// ZeroModels GPT-OSS page, "MXFP4 experts": on decode only the routed experts' packed
// weights are touched (the bank stays packed; dequantization happens on the fly). Each
// packed byte is read from HBM exactly once per call, decoded to bf16 in registers by
// v_cvt_scalef32_pk_bf16_fp4 (E2M1 code times the block's E8M0 power of two) and fed to
// bf16 MFMA with fp32 accumulation.
//
// Streaming a few MB per call at HBM speed needs every workgroup's share of the packed
// weights in flight at once: each wavefront issues all (or a large batch) of its 16-byte
// weight loads before its first MFMA, and the activation rows (a few KB) are staged in LDS
// while those loads are outstanding.
//
// Contraction mapping. A 16x16x32 MFMA step consumes, per lane, 8 consecutive contraction
// entries; lane group g = lane / 16 is free to take any 8 entries as long as the A and B
// operands agree. Here one 16-byte load of a weight row = one 32-wide scale block; the four
// lane groups take four consecutive blocks (a 128-wide chunk), and step s of the chunk uses
// entries 8s..8s+7 of each group's block. Activations are read to match.
#include "device_common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kMaxRows = 64;          // = kDecodeMaxT: an expert is chosen at most once per token
constexpr int kDownScaleLds = 16384;   // LDS bytes for the routed experts' scale rows (few tokens)

// Routing of all T tokens into LDS: s_idx / s_w [T*k]. With `logits` (double [T, E]) the
// top-k + softmax is computed here by every block (wavefront w handles tokens w, w+NW, ...)
// and block 0 also writes it to topk_idx / topk_w; otherwise it is read from them.
// Then bitmap = the set of routed experts. Ends with a block barrier.
__device__ void load_routing(const double *logits, int32_t *topk_idx, float *topk_w, int T, int E,
                             int k, int *s_idx, float *s_w, uint32_t *bitmap) {
    __shared__ double s_lg[4][kMaxE];
    __shared__ double s_ex[4][8];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int nw = blockDim.x / kWave;
    const int N = T * k;
    if (tid < kMaxE / 32) bitmap[tid] = 0u;
    if (logits) {
        const bool writer = blockIdx.x == 0;
        for (int t = wave; t < T; t += nw) {
            if (wave < 4) {
                for (int e = lane; e < E; e += kWave) s_lg[wave][e] = logits[static_cast<int64_t>(t) * E + e];
                __builtin_amdgcn_wave_barrier();
                topk_softmax_wave(s_lg[wave], E, k, lane, s_idx + t * k, s_w + t * k,
                                  writer ? topk_idx + t * k : nullptr, writer ? topk_w + t * k : nullptr,
                                  nullptr, s_ex[wave]);
            }
        }
    } else {
        for (int n = tid; n < N; n += blockDim.x) {
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

// The slot-th routed expert in increasing index order (-1 if fewer), computed by every
// thread from the bitmap.
__device__ int expert_of_slot(const uint32_t *bitmap, int slot) {
    int rem = slot;
#pragma unroll
    for (int w = 0; w < kMaxE / 32; ++w) {
        uint32_t bits = bitmap[w];
        const int c = __popc(bits);
        if (rem < c) {
            for (int q = 0; q < rem; ++q) bits &= bits - 1u;
            return 32 * w + __ffs(bits) - 1;
        }
        rem -= c;
    }
    return -1;
}

// Routed pairs n = t*k + j of expert e in increasing n, by wavefront 0 (caller syncs).
__device__ void rows_of_expert(const int *s_idx, int N, int e, int *s_rows, int *s_nrows) {
    const int lane = threadIdx.x % kWave;
    int cnt = 0;
    for (int base = 0; base < N; base += kWave) {
        const int n = base + lane;
        const bool hit = n < N && s_idx[n] == e;
        const uint64_t m = __ballot(hit);
        const int pos = cnt + __popcll(m & lanemask_lt());
        if (hit && pos < kMaxRows) s_rows[pos] = n;
        cnt += __popcll(m);
    }
    if (lane == 0) *s_nrows = cnt < kMaxRows ? cnt : kMaxRows;
}

// Copy `nrows` rows (row r = src + row_of(r) * K) into LDS rows of K elements.
template <typename RowOf>
__device__ void stage_rows(uint16_t *dst, const uint16_t *src, int nrows, int K, RowOf row_of) {
    const int per_row = K / 8;
    for (int q = threadIdx.x; q < nrows * per_row; q += blockDim.x) {
        const int r = q / per_row, c = q % per_row;
        *reinterpret_cast<uint4 *>(dst + r * K + 8 * c) =
            *reinterpret_cast<const uint4 *>(src + static_cast<int64_t>(row_of(r)) * K + 8 * c);
    }
}

// ---------------------------------------------------------------------------------------
// Up-projection. Block = (routing slot, 16 gate/up pairs); 4 wavefronts split the
// contraction (H) in 128-wide chunks and are reduced through LDS in a fixed order.
//   hw[n, i] = bf16(w[n] * swiglu(x[t] . Wgu[e, 2i] + bgu[e, 2i], x[t] . Wgu[e, 2i+1] + bgu[e, 2i+1]))
// for every pair n = t*k + j routed to expert e (the slot-th routed expert).
// NMT = 16-row m-subtiles (>= rows / 16); UB = chunks per load batch per wavefront; with
// LDS_A the activation rows are staged in dynamic LDS (rows * H bf16). With `logits` the
// routing (top-k + softmax) is computed in the prologue, see load_routing.
template <int NMT, int UB, bool LDS_A>
__global__ __launch_bounds__(256) void k_up_small(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ gu_blocks,
    const uint8_t *__restrict__ gu_scales, const uint16_t *__restrict__ gu_bias,
    const double *__restrict__ logits, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    int T, int H, int I, int E, int k, float alpha, float limit, uint16_t *__restrict__ hw) {
    extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
    __shared__ uint32_t bitmap[kMaxE / 32];
    __shared__ int s_idx[kMaxRows * 8];
    __shared__ float s_w[kMaxRows * 8];
    __shared__ int s_rows[kMaxRows];
    __shared__ int s_nrows;
    __shared__ float red[4][NMT * 8][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t s_sc[32 * kMaxScaleCols];   // 32 rows x H/32

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;
    const int tiles_i = I / 16;
    const int N = T * k;
    // every token row into LDS first (independent of the routing, so its latency overlaps it)
    if (LDS_A) stage_rows(xs, x, T, H, [](int r) { return r; });
    load_routing(logits, topk_idx, topk_w, T, E, k, s_idx, s_w, bitmap);
    const int e = expert_of_slot(bitmap, blockIdx.x / tiles_i);
    if (e < 0) return;  // fewer routed experts than slots (uniform over the block)
    const int i0 = (blockIdx.x % tiles_i) * 16;

    // all packed-weight loads of the first batch; scale bytes stay raw until use so that no
    // wait is needed before the whole batch is in flight
    const int64_t grow = static_cast<int64_t>(e) * 2 * I + 2 * (i0 + col);   // gate row
    const int hb = H / 2, hs = H / 32;
    const uint8_t *gate_b = gu_blocks + grow * hb;
    const uint8_t *up_b = gate_b + hb;
    const int nblocks = H / 32;
    const int nchunks = (nblocks + 3) / 4;
    // the block's 32 rows of scales are H contiguous bytes: one 16-byte load per thread,
    // issued before the weight stream so that waiting for it never waits for the stream
    const uint8_t *sc_src = gu_scales + (static_cast<int64_t>(e) * 2 * I + 2 * i0) * hs;
    uint4 scv[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + 256 * q;
        scv[q] = idx < H / 16 ? *reinterpret_cast<const uint4 *>(sc_src + 16 * idx) : zero4();
    }
    uint4 bg[UB], bu[UB];
    // loads are unconditional (block index clamped into the row) so that the whole batch is
    // issued without branches; chunks past the end are neutralised on the activation side
    auto load_batch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int kb = min(4 * (c0 + 4 * u) + g, nblocks - 1);
            bg[u] = *reinterpret_cast<const uint4 *>(gate_b + kb * 16);
            bu[u] = *reinterpret_cast<const uint4 *>(up_b + kb * 16);
        }
    };
    load_batch(wave);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + 256 * q;
        if (idx < H / 16) *reinterpret_cast<uint4 *>(s_sc + 16 * idx) = scv[q];
    }
    const uint32_t bias_pair = *reinterpret_cast<const uint32_t *>(gu_bias + grow);   // gate, up

    if (wave == 0) rows_of_expert(s_idx, N, e, s_rows, &s_nrows);
    __syncthreads();
    const int nrows = s_nrows;
    const uint16_t *arow[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const int r = 16 * mt + col;
        arow[mt] = r < nrows ? (LDS_A ? xs : x) + static_cast<int64_t>(s_rows[r] / k) * H : nullptr;
    }

    f32x4 accg[NMT], accu[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        accg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int c0 = wave; c0 < nchunks; c0 += 4 * UB) {
        if (c0 != wave) load_batch(c0);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int kb = 4 * (c0 + 4 * u) + g;
            const bool ok = c0 + 4 * u < nchunks && kb < nblocks;
            uint4 a[NMT][4];
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    a[mt][s] = (ok && arow[mt] != nullptr)
                                   ? *reinterpret_cast<const uint4 *>(arow[mt] + kb * 32 + 8 * s)
                                   : zero4();
            const uint32_t gw[4] = {bg[u].x, bg[u].y, bg[u].z, bg[u].w};
            const uint32_t uw[4] = {bu[u].x, bu[u].y, bu[u].z, bu[u].w};
            const int kbc = min(kb, nblocks - 1);
            const float scg = e8m0_to_f32(s_sc[(2 * col) * hs + kbc]);
            const float scu = e8m0_to_f32(s_sc[(2 * col + 1) * hs + kbc]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 wg = mxfp4_word_to_bf16x8(gw[s], scg);
                const bf16x8 wu = mxfp4_word_to_bf16x8(uw[s], scu);
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) {
                    if (16 * mt < nrows) {
                        accg[mt] = mfma16(as_bf16x8(a[mt][s]), wg, accg[mt]);
                        accu[mt] = mfma16(as_bf16x8(a[mt][s]), wu, accu[mt]);
                    }
                }
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            red[wave][mt * 8 + r][lane] = accg[mt][r];
            red[wave][mt * 8 + 4 + r][lane] = accu[mt][r];
        }
    __syncthreads();
    if (wave != 0) return;
    const int i = i0 + col;
    const float bgate = bf16_to_f32(static_cast<uint16_t>(bias_pair & 0xffffu));
    const float bup = bf16_to_f32(static_cast<uint16_t>(bias_pair >> 16));
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * g + r;
            if (row >= nrows) continue;
            float gsum = 0.f, usum = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                gsum += red[w][mt * 8 + r][lane];
                usum += red[w][mt * 8 + 4 + r][lane];
            }
            const int n = s_rows[row];
            const float hval = swiglu(gsum + bgate, usum + bup, alpha, limit) * s_w[n];
            hw[static_cast<int64_t>(n) * I + i] = f32_to_bf16(hval);
        }
}

// ---------------------------------------------------------------------------------------
// Down-projection with the combine folded in (few tokens). Block = 16 output features d
// for every token; NW wavefronts share the (routed expert, 128-wide chunk of I) work units.
// For routed expert e the A operand row of token t is hw[t*k + j] when idx[t, j] == e, else
// zero, so all experts accumulate into the same per-token tile:
//   y[t, d] = bf16( sum_{e, i} A_e[t, i] * Wdn[e, d, i]  +  sum_j w[t, j] * bdn[e_tj, d] ).
// Each wavefront alternates two accumulators (shorter MFMA dependency chains); the partial
// tiles are reduced through LDS in (wavefront, accumulator) order. With SC_LDS the scale
// rows of all routed experts are staged in LDS up front (they must fit kDownScaleLds bytes);
// otherwise each weight load brings its scale byte along.
template <int UB, int NW, bool LDS_A, bool SC_LDS>
__global__ __launch_bounds__(NW * 64) void k_down_tokens(
    const uint16_t *__restrict__ hw, const uint8_t *__restrict__ dn_blocks,
    const uint8_t *__restrict__ dn_scales, const uint16_t *__restrict__ dn_bias,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int T, int H, int I, int E, int k,
    uint16_t *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) uint16_t hs_lds[];
    __shared__ uint32_t bitmap[kMaxE / 32];
    __shared__ int s_idx[16 * 8];
    __shared__ float s_w[16 * 8];
    __shared__ int s_experts[kMaxE];
    __shared__ int s_rowof[16 * 8][16];     // [routed expert slot][token] -> pair n, or -1
    __shared__ int s_na;
    __shared__ float red[NW * 2][4][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t s_sc[SC_LDS ? kDownScaleLds : 16];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;
    const int d0 = blockIdx.x * 16;
    const int N = T * k;        // T <= 16 here
    // every (token, slot) row of hw into LDS first (independent of the routing)
    if (LDS_A) stage_rows(hs_lds, hw, N, I, [](int r) { return r; });
    load_routing(nullptr, topk_idx, topk_w, T, E, k, s_idx, s_w, bitmap);
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
    for (int q = tid; q < na * 16; q += NW * 64) {
        const int a = q / 16, t = q % 16;
        int n = -1;
        if (t < T)
            for (int j = 0; j < k; ++j)
                if (s_idx[t * k + j] == s_experts[a]) n = t * k + j;
        s_rowof[a][t] = n;
    }
    const int nblocks = I / 32;
    const int nchunks = (nblocks + 3) / 4;
    const int nunits = na * nchunks;
    const int64_t drow = d0 + col;

    // the 16 rows of scales of every routed expert (I/2 contiguous bytes each), loaded before
    // the weight stream
    const int is = I / 32;
    const int nsc = SC_LDS ? na * (I / 32) : 0;     // 16-byte pieces
    uint4 scv[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + NW * 64 * q;
        scv[q] = zero4();
        if (SC_LDS && idx < nsc) {
            const int a = idx / (I / 32), piece = idx % (I / 32);
            scv[q] = *reinterpret_cast<const uint4 *>(dn_scales + (static_cast<int64_t>(s_experts[a]) * H + d0) * is + 16 * piece);
        }
    }
    // this wavefront's first batch of packed-weight loads
    uint4 b[UB];
    uint32_t sc[UB];
    int ua[UB], uaa[UB], ukb[UB];
    auto load_batch = [&](int u0) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            // unconditional loads at clamped indices; units past the end read a real block and
            // are neutralised by a zero activation row
            const int unit = u0 + NW * u;
            const int uc = min(unit, nunits - 1);
            const int a = uc / nchunks;
            const int kb = min(4 * (uc % nchunks) + g, nblocks - 1);
            const bool ok = unit < nunits && 4 * (uc % nchunks) + g < nblocks;
            const int64_t row = static_cast<int64_t>(s_experts[a]) * H + drow;
            b[u] = *reinterpret_cast<const uint4 *>(dn_blocks + row * (I / 2) + kb * 16);
            if (!SC_LDS) sc[u] = dn_scales[row * is + kb];
            ua[u] = ok ? a : -1;
            uaa[u] = a;
            ukb[u] = kb;
        }
    };
    load_batch(wave);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int idx = tid + NW * 64 * q;
        if (SC_LDS && idx < nsc) *reinterpret_cast<uint4 *>(s_sc + 16 * idx) = scv[q];
    }
    // bias term of the epilogue rows (wavefront 0): sum_j w[t, j] * bdn[e_tj, d], t = 4g + r
    float bterm[4] = {0.f, 0.f, 0.f, 0.f};
    if (wave == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            if (t < T)
                for (int j = 0; j < k; ++j)
                    bterm[r] += s_w[t * k + j] * bf16_to_f32(dn_bias[static_cast<int64_t>(s_idx[t * k + j]) * H + drow]);
        }
    }
    __syncthreads();

    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int u0 = wave; u0 < nunits; u0 += NW * UB) {
        if (u0 != wave) load_batch(u0);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int n = ua[u] >= 0 ? s_rowof[ua[u]][col] : -1;
            const uint16_t *src = (LDS_A ? hs_lds : hw) + static_cast<int64_t>(n) * I + ukb[u] * 32;
            const uint32_t ww[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
            const float scf = e8m0_to_f32(SC_LDS ? s_sc[(uaa[u] * 16 + col) * is + ukb[u]] : sc[u]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 av = n >= 0 ? *reinterpret_cast<const uint4 *>(src + 8 * s) : zero4();
                acc[u & 1] = mfma16(as_bf16x8(av), mxfp4_word_to_bf16x8(ww[s], scf), acc[u & 1]);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        red[2 * wave][r][lane] = acc[0][r];
        red[2 * wave + 1][r][lane] = acc[1][r];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = 4 * g + r;
        if (t >= T) continue;
        float v = 0.f;
        for (int w = 0; w < 2 * NW; ++w) v += red[w][r][lane];
        y[static_cast<int64_t>(t) * H + drow] = f32_to_bf16(v + bterm[r]);
    }
}

// ---------------------------------------------------------------------------------------
// Down-projection for more tokens: block = (routing slot, 16 output features); 4 wavefronts
// split the contraction. part[n, d] = hw[n] . Wdn[e, d] + w[n] * bdn[e, d] for the pairs n
// routed to e; a separate combine sums part over the k slots of each token.
template <int NMT, int UB>
__global__ __launch_bounds__(256) void k_down_slots(
    const uint16_t *__restrict__ hw, const uint8_t *__restrict__ dn_blocks,
    const uint8_t *__restrict__ dn_scales, const uint16_t *__restrict__ dn_bias,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int T, int H, int I,
    int E, int k, float *__restrict__ part) {
    __shared__ uint32_t bitmap[kMaxE / 32];
    __shared__ int s_idx[kMaxRows * 8];
    __shared__ float s_w[kMaxRows * 8];
    __shared__ int s_rows[kMaxRows];
    __shared__ int s_nrows;
    __shared__ float red[4][NMT * 4][kWave];
    __shared__ __attribute__((aligned(16))) uint8_t s_sc[16 * kMaxScaleCols];   // 16 rows x I/32

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;
    const int tiles_d = H / 16;
    const int N = T * k;
    load_routing(nullptr, topk_idx, topk_w, T, E, k, s_idx, s_w, bitmap);
    const int e = expert_of_slot(bitmap, blockIdx.x / tiles_d);
    if (e < 0) return;
    const int d = (blockIdx.x % tiles_d) * 16 + col;
    const int64_t wrow = static_cast<int64_t>(e) * H + d;
    const uint8_t *wb = dn_blocks + wrow * (I / 2);
    const int is = I / 32;
    const int nblocks = I / 32;
    const int nchunks = (nblocks + 3) / 4;
    // the block's 16 rows of scales: I/2 contiguous bytes, loaded before the weight stream
    const uint8_t *sc_src = dn_scales + (static_cast<int64_t>(e) * H + (blockIdx.x % tiles_d) * 16) * is;
    uint4 scv = tid < I / 32 ? *reinterpret_cast<const uint4 *>(sc_src + 16 * tid) : zero4();
    uint4 b[UB];
    auto load_batch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int kb = min(4 * (c0 + 4 * u) + g, nblocks - 1);   // unconditional, clamped
            b[u] = *reinterpret_cast<const uint4 *>(wb + kb * 16);
        }
    };
    load_batch(wave);
    if (tid < I / 32) *reinterpret_cast<uint4 *>(s_sc + 16 * tid) = scv;
    const float bd = bf16_to_f32(dn_bias[wrow]);
    if (wave == 0) rows_of_expert(s_idx, N, e, s_rows, &s_nrows);
    __syncthreads();
    const int nrows = s_nrows;
    const uint16_t *arow[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const int r = 16 * mt + col;
        arow[mt] = r < nrows ? hw + static_cast<int64_t>(s_rows[r]) * I : nullptr;
    }
    f32x4 acc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = wave; c0 < nchunks; c0 += 4 * UB) {
        if (c0 != wave) load_batch(c0);
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int kb = 4 * (c0 + 4 * u) + g;
            const bool ok = c0 + 4 * u < nchunks && kb < nblocks;
            const uint32_t ww[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
            const float scf = e8m0_to_f32(s_sc[col * is + min(kb, nblocks - 1)]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 wv = mxfp4_word_to_bf16x8(ww[s], scf);
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) {
                    if (16 * mt < nrows) {
                        const uint4 av = (ok && arow[mt] != nullptr)
                                             ? *reinterpret_cast<const uint4 *>(arow[mt] + kb * 32 + 8 * s)
                                             : zero4();
                        acc[mt] = mfma16(as_bf16x8(av), wv, acc[mt]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mt * 4 + r][lane] = acc[mt][r];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * g + r;
            if (row >= nrows) continue;
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) v += red[w][mt * 4 + r][lane];
            const int n = s_rows[row];
            part[static_cast<int64_t>(n) * H + d] = v + s_w[n] * bd;
        }
}

// y[t, d] = bf16(sum_{j < k} part[t*k + j, d]) in slot order. Thread = 4 features.
__global__ __launch_bounds__(256) void k_combine_slots(const float *__restrict__ part, int T, int H,
                                                       int k, uint16_t *__restrict__ y) {
    const int per_row = H / 4;
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q >= T * per_row) return;
    const int t = q / per_row, d = (q % per_row) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        const float4 v = *reinterpret_cast<const float4 *>(part + static_cast<int64_t>(t * k + j) * H + d);
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const uint32_t lo = f32_to_bf16(s.x) | (static_cast<uint32_t>(f32_to_bf16(s.y)) << 16);
    const uint32_t hi = f32_to_bf16(s.z) | (static_cast<uint32_t>(f32_to_bf16(s.w)) << 16);
    *reinterpret_cast<uint2 *>(y + static_cast<int64_t>(t) * H + d) = make_uint2(lo, hi);
}

int slots_of(const Dims &d) { return static_cast<int>(d.T * d.k < d.E ? d.T * d.k : d.E); }

// LDS staging of activation rows when they fit next to other resident blocks.
bool lds_fits(int64_t rows, int K) { return rows * K * 2 <= 48 * 1024; }

template <int NMT, int UB, bool LDS_A>
hipError_t up_n(const Dims &d, const uint16_t *x, const uint8_t *gb, const uint8_t *gs,
                const uint16_t *gbias, const double *logits, int32_t *idx, float *w, uint16_t *hw,
                hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>(slots_of(d) * (d.I / 16));
    const size_t lds = LDS_A ? static_cast<size_t>(d.T) * d.H * 2 : 0;   // every token row
    hipLaunchKernelGGL((k_up_small<NMT, UB, LDS_A>), dim3(blocks), dim3(256), lds, s, x, gb, gs, gbias,
                       logits, idx, w, static_cast<int>(d.T), d.H, d.I, d.E, d.k, d.alpha, d.limit, hw);
    return hipGetLastError();
}

template <int NMT, int UB>
hipError_t down_slots_n(const Dims &d, const uint16_t *hw, const uint8_t *db, const uint8_t *ds,
                        const uint16_t *dbias, int32_t *idx, float *w, float *part, hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>(slots_of(d) * (d.H / 16));
    hipLaunchKernelGGL((k_down_slots<NMT, UB>), dim3(blocks), dim3(256), 0, s, hw, db, ds, dbias, idx, w,
                       static_cast<int>(d.T), d.H, d.I, d.E, d.k, part);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_decode(const Dims &d, const float *part, uint16_t *y, hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>((d.T * (d.H / 4) + 255) / 256);
    hipLaunchKernelGGL(k_combine_slots, dim3(blocks), dim3(256), 0, s, part, static_cast<int>(d.T), d.H,
                       d.k, y);
    return hipGetLastError();
}

hipError_t launch_up_decode(const Dims &d, const uint16_t *x, const uint8_t *gu_blocks,
                            const uint8_t *gu_scales, const uint16_t *gu_bias, const double *logits,
                            int32_t *topk_idx, float *topk_w, uint16_t *hw, hipStream_t s) {
    const int nmt = static_cast<int>((d.T + 15) / 16);
    switch (nmt) {
        case 1:
            return lds_fits(d.T, d.H)
                       ? up_n<1, 6, true>(d, x, gu_blocks, gu_scales, gu_bias, logits, topk_idx, topk_w, hw, s)
                       : up_n<1, 3, false>(d, x, gu_blocks, gu_scales, gu_bias, logits, topk_idx, topk_w, hw, s);
        case 2: return up_n<2, 3, false>(d, x, gu_blocks, gu_scales, gu_bias, logits, topk_idx, topk_w, hw, s);
        case 3: return up_n<3, 2, false>(d, x, gu_blocks, gu_scales, gu_bias, logits, topk_idx, topk_w, hw, s);
        default: return up_n<4, 2, false>(d, x, gu_blocks, gu_scales, gu_bias, logits, topk_idx, topk_w, hw, s);
    }
}

hipError_t launch_down_decode(const Dims &d, const uint16_t *hw, const uint8_t *dn_blocks,
                              const uint8_t *dn_scales, const uint16_t *dn_bias, int32_t *topk_idx,
                              float *topk_w, float *part, uint16_t *y, hipStream_t s) {
    if (d.T <= kDownTokensMaxT) {
        constexpr int NW = 16;
        const unsigned blocks = static_cast<unsigned>(d.H / 16);
        // scale rows of every routed expert: at most min(T*k, E) experts x 16 rows x I/32 bytes
        const bool sc_lds = static_cast<int64_t>(slots_of(d)) * (d.I / 2) <= kDownScaleLds;
        if (lds_fits(d.T * d.k, d.I)) {
            const size_t lds = static_cast<size_t>(d.T) * d.k * d.I * 2;
            if (sc_lds)
                hipLaunchKernelGGL((k_down_tokens<6, NW, true, true>), dim3(blocks), dim3(NW * 64), lds, s, hw,
                                   dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, static_cast<int>(d.T),
                                   d.H, d.I, d.E, d.k, y);
            else
                hipLaunchKernelGGL((k_down_tokens<6, NW, true, false>), dim3(blocks), dim3(NW * 64), lds, s, hw,
                                   dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, static_cast<int>(d.T),
                                   d.H, d.I, d.E, d.k, y);
        } else {
            hipLaunchKernelGGL((k_down_tokens<4, NW, false, false>), dim3(blocks), dim3(NW * 64), 0, s, hw,
                               dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, static_cast<int>(d.T), d.H,
                               d.I, d.E, d.k, y);
        }
        return hipGetLastError();
    }
    const int nmt = static_cast<int>((d.T + 15) / 16);
    switch (nmt) {
        case 2: return down_slots_n<2, 3>(d, hw, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, part, s);
        case 3: return down_slots_n<3, 3>(d, hw, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, part, s);
        default: return down_slots_n<4, 2>(d, hw, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, part, s);
    }
}

}  // namespace moe
