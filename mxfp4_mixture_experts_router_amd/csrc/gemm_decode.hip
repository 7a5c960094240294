// Decode path (T <= 64): weight-streaming expert GEMMs with the MXFP4 dequantization
// fused into the register staging.
//
// ZeroModels GPT-OSS page, "MXFP4 experts": on decode only the routed experts' packed
// weights are touched (the bank stays packed; dequantization happens on the fly). Each
// packed byte is read from HBM exactly once per call, decoded to bf16 in registers by
// v_cvt_scalef32_pk_bf16_fp4 (E2M1 code times the block's E8M0 power of two) and fed to
// bf16 MFMA with fp32 accumulation.
//
// Contraction mapping. A 16x16x32 MFMA step consumes, per lane, 8 consecutive contraction
// entries; lane group g = lane / 16 is free to take any 8 entries as long as the A and B
// operands agree. Here one 16-byte load of a weight row = one 32-wide scale block; the four
// lane groups take four consecutive blocks (a 128-wide chunk), and step s of the chunk uses
// entries 8s..8s+7 of each group's block. Activations are loaded to match.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kMaxE = 256;
constexpr int kMaxRows = 64;          // = kDecodeMaxT: an expert is chosen at most once per token

// Bitmap of the experts named in topk_idx[0..N) -> in LDS. Returns nothing; caller syncs.
__device__ __forceinline__ void mark_experts(const int32_t *topk_idx, int N, int E,
                                             uint32_t *bitmap, int tid, int nthreads) {
    for (int n = tid; n < N; n += nthreads) {
        const int e = topk_idx[n];
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicOr(&bitmap[e >> 5], 1u << (e & 31));
    }
}

// ---------------------------------------------------------------------------------------
// Up-projection. Block = (expert slot a, 16 gate/up pairs); 4 wavefronts split the
// contraction (H) in 128-wide chunks and are reduced through LDS in fixed order.
//   hw[n, i] = bf16(w[n] * swiglu(x[t] . Wgu[e, 2i] + bgu[e, 2i], x[t] . Wgu[e, 2i+1] + bgu[e, 2i+1]))
// for every pair n = t*k + j routed to expert e (the slot-th distinct routed expert).
template <int NMT, int UB>
__global__ __launch_bounds__(256) void k_up_decode(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ gu_blocks,
    const uint8_t *__restrict__ gu_scales, const uint16_t *__restrict__ gu_bias,
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w, int T, int H, int I,
    int E, int k, float alpha, float limit, uint16_t *__restrict__ hw) {
    __shared__ uint32_t bitmap[kMaxE / 32];
    __shared__ int s_expert;
    __shared__ int s_nrows;
    __shared__ int s_rows[kMaxRows];
    __shared__ float red[4][NMT * 8][kWave];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;
    const int tiles_i = I / 16;
    const int slot = blockIdx.x / tiles_i;
    const int i0 = (blockIdx.x % tiles_i) * 16;
    const int N = T * k;

    if (tid < kMaxE / 32) bitmap[tid] = 0u;
    __syncthreads();
    mark_experts(topk_idx, N, E, bitmap, tid, 256);
    __syncthreads();
    if (tid == 0) {
        int rem = slot, ex = -1;
        for (int w = 0; w < kMaxE / 32 && ex < 0; ++w) {
            uint32_t bits = bitmap[w];
            const int c = __popc(bits);
            if (rem < c) {
                for (int q = 0; q < rem; ++q) bits &= bits - 1u;
                ex = 32 * w + __ffs(bits) - 1;
            } else {
                rem -= c;
            }
        }
        s_expert = ex;
    }
    __syncthreads();
    const int e = s_expert;
    if (e < 0) return;  // fewer distinct experts than slots: nothing to do (uniform)
    if (wave == 0) {
        int cnt = 0;
        for (int base = 0; base < N; base += kWave) {
            const int n = base + lane;
            const bool hit = n < N && topk_idx[n] == e;
            const uint64_t m = __ballot(hit);
            const int pos = cnt + __popcll(m & lanemask_lt());
            if (hit && pos < kMaxRows) s_rows[pos] = n;
            cnt += __popcll(m);
        }
        if (lane == 0) s_nrows = cnt < kMaxRows ? cnt : kMaxRows;
    }
    __syncthreads();
    const int nrows = s_nrows;

    // per-lane activation rows: row r = 16*mt + col of this expert
    const uint16_t *xrow[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        const int r = 16 * mt + col;
        xrow[mt] = r < nrows ? x + static_cast<int64_t>(s_rows[r] / k) * H : nullptr;
    }

    const int64_t grow = static_cast<int64_t>(e) * 2 * I + 2 * (i0 + col);   // gate row
    const int hb = H / 2, hs = H / 32;
    const uint8_t *gate_b = gu_blocks + grow * hb;
    const uint8_t *up_b = gate_b + hb;
    const uint8_t *gate_s = gu_scales + grow * hs;
    const uint8_t *up_s = gate_s + hs;
    const int nblocks = H / 32;
    const int nchunks = (nblocks + 3) / 4;

    f32x4 accg[NMT], accu[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
        accg[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int c0 = wave; c0 < nchunks; c0 += 4 * UB) {
        uint4 bg[UB], bu[UB];
        float sg[UB], su[UB];
        uint4 a[UB][NMT][4];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int c = c0 + 4 * u;
            const int kb = 4 * c + g;
            const bool ok = c < nchunks && kb < nblocks;
            bg[u] = ok ? *reinterpret_cast<const uint4 *>(gate_b + kb * 16) : zero4();
            bu[u] = ok ? *reinterpret_cast<const uint4 *>(up_b + kb * 16) : zero4();
            sg[u] = ok ? e8m0_to_f32(gate_s[kb]) : 0.f;
            su[u] = ok ? e8m0_to_f32(up_s[kb]) : 0.f;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                const bool ao = ok && xrow[mt] != nullptr;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    a[u][mt][s] = ao ? *reinterpret_cast<const uint4 *>(xrow[mt] + kb * 32 + 8 * s) : zero4();
            }
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const uint32_t gw[4] = {bg[u].x, bg[u].y, bg[u].z, bg[u].w};
            const uint32_t uw[4] = {bu[u].x, bu[u].y, bu[u].z, bu[u].w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 wg = mxfp4_word_to_bf16x8(gw[s], sg[u]);
                const bf16x8 wu = mxfp4_word_to_bf16x8(uw[s], su[u]);
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) {
                    if (16 * mt < nrows) {
                        accg[mt] = mfma16(as_bf16x8(a[u][mt][s]), wg, accg[mt]);
                        accu[mt] = mfma16(as_bf16x8(a[u][mt][s]), wu, accu[mt]);
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
    const float bgate = bf16_to_f32(gu_bias[static_cast<int64_t>(e) * 2 * I + 2 * i]);
    const float bup = bf16_to_f32(gu_bias[static_cast<int64_t>(e) * 2 * I + 2 * i + 1]);
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
            const float hval = swiglu(gsum + bgate, usum + bup, alpha, limit) * topk_w[n];
            hw[static_cast<int64_t>(n) * I + i] = f32_to_bf16(hval);
        }
}

// ---------------------------------------------------------------------------------------
// Down-projection with the combine folded in. Block = 16 output columns d for every token;
// NW wavefronts share the (routed expert, 128-wide chunk of I) work units. For routed
// expert e the A operand row of token t is hw[t*k + j] when idx[t, j] == e, else zero, so
// all experts accumulate into the same per-token tile:
//   y[t, d] = bf16( sum_{e, i} A_e[t, i] * Wdn[e, d, i]  +  sum_j w[t, j] * bdn[e_tj, d] ).
template <int NMT, int UB, int NW>
__global__ __launch_bounds__(NW * 64) void k_down_decode(
    const uint16_t *__restrict__ hw, const uint8_t *__restrict__ dn_blocks,
    const uint8_t *__restrict__ dn_scales, const uint16_t *__restrict__ dn_bias,
    const int32_t *__restrict__ topk_idx, const float *__restrict__ topk_w, int T, int H, int I,
    int E, int k, uint16_t *__restrict__ y) {
    __shared__ uint32_t bitmap[kMaxE / 32];
    __shared__ int s_experts[kMaxE];
    __shared__ int s_na;
    __shared__ int s_idx[kMaxRows * 8];
    __shared__ float red[NW][NMT * 4][kWave];

    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int col = lane & 15, g = lane >> 4;
    const int d0 = blockIdx.x * 16;
    const int N = T * k;

    if (tid < kMaxE / 32) bitmap[tid] = 0u;
    for (int n = tid; n < N; n += NW * 64) s_idx[n] = topk_idx[n];
    __syncthreads();
    mark_experts(topk_idx, N, E, bitmap, tid, NW * 64);
    __syncthreads();
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

    const int ib = I / 2, is = I / 32;
    const int nblocks = I / 32;
    const int nchunks = (nblocks + 3) / 4;
    const int nunits = na * nchunks;
    const int64_t drow = d0 + col;

    f32x4 acc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int u0 = wave; u0 < nunits; u0 += NW * UB) {
        uint4 b[UB];
        float sc[UB];
        uint4 a[UB][NMT][4];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const int unit = u0 + NW * u;
            const bool uok = unit < nunits;
            const int aidx = uok ? unit / nchunks : 0;
            const int c = uok ? unit % nchunks : 0;
            const int e = s_experts[aidx];
            const int kb = 4 * c + g;
            const bool ok = uok && kb < nblocks;
            const int64_t row = static_cast<int64_t>(e) * H + drow;
            b[u] = ok ? *reinterpret_cast<const uint4 *>(dn_blocks + row * ib + kb * 16) : zero4();
            sc[u] = ok ? e8m0_to_f32(dn_scales[row * is + kb]) : 0.f;
#pragma unroll
            for (int mt = 0; mt < NMT; ++mt) {
                const int t = 16 * mt + col;
                int n = -1;
                if (ok && t < T)
                    for (int j = 0; j < k; ++j)
                        if (s_idx[t * k + j] == e) n = t * k + j;
                const uint16_t *src = hw + static_cast<int64_t>(n) * I + kb * 32;
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    a[u][mt][s] = n >= 0 ? *reinterpret_cast<const uint4 *>(src + 8 * s) : zero4();
            }
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const uint32_t ww[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 wv = mxfp4_word_to_bf16x8(ww[s], sc[u]);
#pragma unroll
                for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma16(as_bf16x8(a[u][mt][s]), wv, acc[mt]);
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
            const int t = 16 * mt + 4 * g + r;
            if (t >= T) continue;
            float v = 0.f;
            for (int w = 0; w < NW; ++w) v += red[w][mt * 4 + r][lane];
            for (int j = 0; j < k; ++j) {
                const int e = s_idx[t * k + j];
                v += topk_w[t * k + j] * bf16_to_f32(dn_bias[static_cast<int64_t>(e) * H + drow]);
            }
            y[static_cast<int64_t>(t) * H + drow] = f32_to_bf16(v);
        }
}

template <int NMT, int UB>
hipError_t up_decode_n(const Dims &d, const uint16_t *x, const uint8_t *gb, const uint8_t *gs,
                       const uint16_t *gbias, const int32_t *idx, const float *w, uint16_t *hw,
                       hipStream_t s) {
    const int slots = static_cast<int>(d.T * d.k < d.E ? d.T * d.k : d.E);
    const unsigned blocks = static_cast<unsigned>(slots * (d.I / 16));
    hipLaunchKernelGGL((k_up_decode<NMT, UB>), dim3(blocks), dim3(256), 0, s, x, gb, gs, gbias, idx, w,
                       static_cast<int>(d.T), d.H, d.I, d.E, d.k, d.alpha, d.limit, hw);
    return hipGetLastError();
}

template <int NMT, int UB>
hipError_t down_decode_n(const Dims &d, const uint16_t *hw, const uint8_t *db, const uint8_t *ds,
                         const uint16_t *dbias, const int32_t *idx, const float *w, uint16_t *y,
                         hipStream_t s) {
    constexpr int NW = 16;
    hipLaunchKernelGGL((k_down_decode<NMT, UB, NW>), dim3(static_cast<unsigned>(d.H / 16)), dim3(NW * 64),
                       0, s, hw, db, ds, dbias, idx, w, static_cast<int>(d.T), d.H, d.I, d.E, d.k, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_up_decode(const Dims &d, const uint16_t *x, const uint8_t *gu_blocks,
                            const uint8_t *gu_scales, const uint16_t *gu_bias,
                            const int32_t *topk_idx, const float *topk_w, uint16_t *hw,
                            hipStream_t s) {
    const int nmt = static_cast<int>((d.T + 15) / 16);
    switch (nmt) {
        case 1: return up_decode_n<1, 6>(d, x, gu_blocks, gu_scales, gu_bias, topk_idx, topk_w, hw, s);
        case 2: return up_decode_n<2, 3>(d, x, gu_blocks, gu_scales, gu_bias, topk_idx, topk_w, hw, s);
        case 3: return up_decode_n<3, 2>(d, x, gu_blocks, gu_scales, gu_bias, topk_idx, topk_w, hw, s);
        default: return up_decode_n<4, 2>(d, x, gu_blocks, gu_scales, gu_bias, topk_idx, topk_w, hw, s);
    }
}

hipError_t launch_down_decode(const Dims &d, const uint16_t *hw, const uint8_t *dn_blocks,
                              const uint8_t *dn_scales, const uint16_t *dn_bias,
                              const int32_t *topk_idx, const float *topk_w, uint16_t *y,
                              hipStream_t s) {
    const int nmt = static_cast<int>((d.T + 15) / 16);
    switch (nmt) {
        case 1: return down_decode_n<1, 4>(d, hw, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, y, s);
        case 2: return down_decode_n<2, 2>(d, hw, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, y, s);
        case 3: return down_decode_n<3, 2>(d, hw, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, y, s);
        default: return down_decode_n<4, 1>(d, hw, dn_blocks, dn_scales, dn_bias, topk_idx, topk_w, y, s);
    }
}

}  // namespace moe
