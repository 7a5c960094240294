// Router: logits, top-k selection and softmax over the selected logits.
//
// ZeroModels GPT-OSS page, "Mixture-of-experts feed-forward": a top-num_experts_per_tok
// router selects experts whose softmax weights combine the per-expert outputs.
//
// Logits are accumulated in double precision. Every product of two bf16 values is exact
// in double, so the only error is the summation's (about 1e-13 relative for H = 2880);
// the integer decision (which k experts) therefore matches exact arithmetic unless two
// logits are closer than that, and equal logits (e.g. duplicated router rows, which take
// the identical summation sequence here) resolve to the lower expert index.
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "mx_mfma.h"
#include "rms.h"
#include "topk.h"

#include <math.h>

namespace moe {
namespace {


// Sum of the 8 exact bf16 x bf16 products held in two uint4 vectors, added to acc in order.
__device__ __forceinline__ double dot8(uint4 xv, uint4 wv, double acc) {
    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
    const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc = fma(static_cast<double>(__uint_as_float(xs[q] << 16)),
                  static_cast<double>(__uint_as_float(ws[q] << 16)), acc);
        acc = fma(static_cast<double>(__uint_as_float(xs[q] & 0xffff0000u)),
                  static_cast<double>(__uint_as_float(ws[q] & 0xffff0000u)), acc);
    }
    return acc;
}

// Latency-oriented router for few tokens: one block (8 wavefronts) per token. The token
// row and the wave's four router rows are loaded with every load in flight at once (lane l
// covers h = 8l + 512i, i < NI, NI = ceil(H / 512)); wavefront w handles experts
// 4w .. 4w+3, then 32 + 4w .. and so on.
// With gamma (the pre-norm block), the token row is first normalized (rms.h): every
// wavefront holds the whole row, so each sums its squares itself, in the same order; wavefront
// w normalizes the 512-element chunk w into LDS, and every wavefront reads the normalized row
// back. The first router rows are requested before all this and stay in flight.
template <int NI>
__global__ __launch_bounds__(512) void k_route_token(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma, double eps, const uint16_t *__restrict__ wr,
    const uint16_t *__restrict__ br, int H, int E, int k, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, float *__restrict__ logits_out, uint8_t *__restrict__ x8, int T) {
    constexpr int kEPW = 4;
    __shared__ double lg[kMaxE];
    __shared__ __attribute__((aligned(16))) uint64_t s_tk[kTopkScratch];
    __shared__ __attribute__((aligned(16))) uint16_t s_xn[NI * 8 * kWave];   // the normalized row
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t t = blockIdx.x;
    const uint16_t *xr = x + t * H;
    uint4 xv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int h = 8 * lane + 8 * kWave * i;
        xv[i] = h < H ? *reinterpret_cast<const uint4 *>(xr + h) : zero4();
    }
    const int hw = 8 * lane + 8 * kWave * wave;        // this wavefront's chunk to normalize
    const uint4 gv = gamma && wave < NI && hw < H ? *reinterpret_cast<const uint4 *>(gamma + hw) : zero4();
    uint4 a[kEPW][NI];
    auto load_rows = [&](int e0) {
#pragma unroll
        for (int q = 0; q < kEPW; ++q) {
            const int e = e0 + q < E ? e0 + q : e0;
            const uint16_t *wrow = wr + static_cast<int64_t>(e) * H;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int h = 8 * lane + 8 * kWave * i;
                a[q][i] = h < H ? *reinterpret_cast<const uint4 *>(wrow + h) : zero4();
            }
        }
    };
    if (kEPW * wave < E) load_rows(kEPW * wave);
    if (gamma) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < NI; ++i) ss = sumsq8(xv[i], ss);
        const double r = rms_scale(wave_sum(ss), H, eps);
        uint4 mine = xv[0];
#pragma unroll
        for (int i = 1; i < NI; ++i)
            if (i == wave) mine = xv[i];
        if (wave < NI && hw < H) *reinterpret_cast<uint4 *>(s_xn + hw) = rms_apply8(mine, gv, r);
        wait_lgkm0();
        barrier_only();
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int h = 8 * lane + 8 * kWave * i;
            xv[i] = h < H ? *reinterpret_cast<const uint4 *>(s_xn + h) : zero4();
        }
    }
    for (int e0 = kEPW * wave; e0 < E; e0 += kEPW * 8) {
        if (e0 != kEPW * wave) load_rows(e0);
        double acc[kEPW];
#pragma unroll
        for (int q = 0; q < kEPW; ++q) {
            acc[q] = 0.0;
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[q] = dot8(xv[i], a[q][i], acc[q]);
        }
#pragma unroll
        for (int q = 0; q < kEPW; ++q) acc[q] = wave_sum_f64(acc[q]);
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < kEPW; ++q)
                if (e0 + q < E) lg[e0 + q] = acc[q] + static_cast<double>(bf16_to_f32(br[e0 + q]));
        }
    }
    __syncthreads();
    if (wave == 0)
        topk_softmax_wave(lg, E, k, lane, topk_idx + t * k, topk_w + t * k, nullptr, nullptr,
                          logits_out ? logits_out + t * E : nullptr, s_tk);
    // wavefront 0 runs the top-k; the others write the mx8 row meanwhile (s_xn: written before
    // the barrier)
    if (x8 != nullptr && wave > 0) write_mx8_row(gamma ? s_xn : xr, H, x8, T, t, kWave);
}

// Logits only, for few tokens (the top-k then runs in the up-projection's prologue): block
// (expert pair, token); its 4 wavefronts split H (lane l of wavefront w covers
// h = 8l + 512(w + 4i)) and their partial sums are added in wavefront order.
//   logits[t, e] = sum_h x[t, h] * Wr[e, h] + br[e]     (double)
// One extra block per token (the last in x) writes the token as an mx8 row of x8 (T rows)
// for the expert GEMMs. With gamma (the pre-norm block) every block first normalizes the
// token row (rms.h); all blocks sum the squares in the same order (per lane, across each
// wavefront, then the wavefronts in order), so they agree on every normalized value.
template <int NIQ>
__global__ __launch_bounds__(256) void k_logits(const uint16_t *__restrict__ x, const uint16_t *__restrict__ gamma,
                                                double eps, const uint16_t *__restrict__ wr,
                                                const uint16_t *__restrict__ br, int H, int E,
                                                double *__restrict__ logits, uint8_t *__restrict__ x8, int T) {
    __shared__ double part[4][2];
    __shared__ double s_ss[4];
    __shared__ __attribute__((aligned(16))) uint16_t s_xn[NIQ * 4 * 8 * kWave];   // the normalized row
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t t = blockIdx.y;
    const bool extra = blockIdx.x == gridDim.x - 1;
    if (extra && gamma == nullptr) {   // the extra block: token t as an mx8 row
        write_mx8_row(x + t * H, H, x8, T, t);
        return;
    }
    const int e0 = 2 * blockIdx.x;
    const bool has2 = e0 + 1 < E;
    const uint16_t *xr = x + t * H;
    const int ea = extra ? 0 : e0;                      // the extra block loads no router rows
    const int eb = extra || !has2 ? ea : e0 + 1;
    const uint16_t *w0 = wr + static_cast<int64_t>(ea) * H;
    const uint16_t *w1 = wr + static_cast<int64_t>(eb) * H;
    uint4 xv[NIQ], a[NIQ], b[NIQ];
#pragma unroll
    for (int i = 0; i < NIQ; ++i) {
        const int h = 8 * lane + 8 * kWave * (wave + 4 * i);
        const bool ok = h < H;
        xv[i] = ok ? *reinterpret_cast<const uint4 *>(xr + h) : zero4();
        a[i] = ok && !extra ? *reinterpret_cast<const uint4 *>(w0 + h) : zero4();
        b[i] = ok && !extra ? *reinterpret_cast<const uint4 *>(w1 + h) : zero4();
    }
    if (gamma) {
        uint4 gv[NIQ];
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < NIQ; ++i) {
            const int h = 8 * lane + 8 * kWave * (wave + 4 * i);
            gv[i] = h < H ? *reinterpret_cast<const uint4 *>(gamma + h) : zero4();
            ss = sumsq8(xv[i], ss);
        }
        ss = wave_sum(ss);
        if (lane == 0) s_ss[wave] = ss;
        __syncthreads();
        const double r = rms_scale(((s_ss[0] + s_ss[1]) + s_ss[2]) + s_ss[3], H, eps);
#pragma unroll
        for (int i = 0; i < NIQ; ++i) xv[i] = rms_apply8(xv[i], gv[i], r);
        if (extra) {
#pragma unroll
            for (int i = 0; i < NIQ; ++i) {
                const int h = 8 * lane + 8 * kWave * (wave + 4 * i);
                if (h < H) *reinterpret_cast<uint4 *>(s_xn + h) = xv[i];
            }
            __syncthreads();
            write_mx8_row(s_xn, H, x8, T, t);
            return;
        }
    }
    double acc0 = 0.0, acc1 = 0.0;
#pragma unroll
    for (int i = 0; i < NIQ; ++i) {
        acc0 = dot8(xv[i], a[i], acc0);
        acc1 = dot8(xv[i], b[i], acc1);
    }
    acc0 = wave_sum_f64(acc0);
    acc1 = wave_sum_f64(acc1);
    if (lane == 0) {
        part[wave][0] = acc0;
        part[wave][1] = acc1;
    }
    __syncthreads();
    if (threadIdx.x < 2 && (threadIdx.x == 0 || has2)) {
        const int q = threadIdx.x;
        const double v = ((part[0][q] + part[1][q]) + part[2][q]) + part[3][q];
        logits[t * E + e0 + q] = v + static_cast<double>(bf16_to_f32(br[e0 + q]));
    }
}

// Throughput router for many tokens on the fp64 MFMA (16 x 16 x 4 per instruction): block =
// THREADS / 64 wavefronts (8; 16 for E <= 32, where the registers allow four wavefronts per SIMD to
// hide more load latency) and 16 consecutive tokens, 16 NT experts. Wavefront w takes the 32-element
// chunks c = w, w + NW, .. of H (up to three chunks' loads in flight at a time). For chunk c, lane (m, g) (m = lane % 16, g = lane / 16)
// loads elements 32c + 8g .. 32c + 8g + 7 of token m and of experts 16 nt + m; MFMA step j
// (0..7) multiplies element j of every lane, so that lane group g supplies contraction index
// g of the step and A and B agree on the element. Products of bf16 values are exact in
// double, so the partial sums carry only the accumulation's rounding. The wavefronts'
// partial logits are then added in wavefront order in LDS. The same chunk loads write the
// tokens as mx8 rows (a 32-element block = lanes m, m + 16, m + 32, m + 48).
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kRT = 16;             // tokens per block
constexpr int kRouteThreads = 512;  // 8 wavefronts split H (16 for E <= 32: 1024 threads)

// Eight bf16 values (one uint4) as doubles.
__device__ __forceinline__ void bf16x8_to_f64(const uint4 &u, double (&d)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        d[2 * q] = static_cast<double>(__uint_as_float(w[q] << 16));
        d[2 * q + 1] = static_cast<double>(__uint_as_float(w[q] & 0xffff0000u));
    }
}

// Elements h .. h + 7 of mx8 row t (of R rows, K columns): this lane's quarter of a
// 32-element block whose other quarters are in lanes lane ^ 16, lane ^ 32, lane ^ 48 (all
// four active together); the lane with g == 0 writes the two scales.
__device__ __forceinline__ void mx8_store_quarter(const uint4 &u, uint8_t *q8, int64_t R, int K, int64_t t,
                                                  int h, bool first) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float v[8];
    float m = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
        m = fmaxf(m, fmaxf(fabsf(v[2 * q]), fabsf(v[2 * q + 1])));
    }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const int eb = mx8_block_exponent(m);
    uint32_t hi0, lo0, hi1, lo1;
    mx8_split4(ldexpf(v[0], -eb), ldexpf(v[1], -eb), ldexpf(v[2], -eb), ldexpf(v[3], -eb), hi0, lo0);
    mx8_split4(ldexpf(v[4], -eb), ldexpf(v[5], -eb), ldexpf(v[6], -eb), ldexpf(v[7], -eb), hi1, lo1);
    *reinterpret_cast<uint2 *>(q8 + (2 * t) * K + h) = make_uint2(hi0, hi1);
    *reinterpret_cast<uint2 *>(q8 + (2 * t + 1) * K + h) = make_uint2(lo0, lo1);
    if (first) {
        const int ss = mx8_scale_stride(K);
        uint8_t *qs = q8 + static_cast<size_t>(2 * R) * K;
        qs[(2 * t) * ss + h / 32] = static_cast<uint8_t>(127 + eb);
        qs[(2 * t + 1) * ss + h / 32] = static_cast<uint8_t>(123 + eb);
    }
}

// With SPLIT, block (g, s) = (blockIdx.x / S, blockIdx.x % S) of a grid of S blocks per
// 16-token group sums only the chunks of slice s of H (slices of ceil(nch / S) chunks) and
// writes those partial logits, without bias, to part[s][t][e]; k_route_topk then adds the S
// slices in order, adds the bias and selects. For few token groups (fewer than the CUs), so
// that the fp64 MFMA work of the whole chip is used.
template <int NT, bool SPLIT, int THREADS = kRouteThreads>
__global__ __launch_bounds__(THREADS) void k_route(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wr,
    const uint16_t *__restrict__ br, int64_t T, int H, int E, int k,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, float *__restrict__ logits_out,
    uint8_t *__restrict__ x8, double *__restrict__ part, int S) {
    constexpr int NW = THREADS / kWave;
    constexpr int kAhead = NT >= 16 ? 1 : (NT >= 8 ? 2 : 3);   // chunks loaded together (registers)
    constexpr int LS = 16 * NT + 1;   // LDS row of one token's logits (padded)
    __shared__ double lg[kRT * LS];
    __shared__ __attribute__((aligned(16))) uint64_t s_tk[NW][kTopkScratch];
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int m = lane & 15, g = lane >> 4;
    const int grp = SPLIT ? static_cast<int>(blockIdx.x) / S : static_cast<int>(blockIdx.x);
    const int slice = SPLIT ? static_cast<int>(blockIdx.x) % S : 0;
    const int64_t t0 = static_cast<int64_t>(grp) * kRT;
    const int64_t tm = t0 + m;
    const uint16_t *xrow = x + min(tm, T - 1) * H;      // past T: a duplicate row
    const uint16_t *wrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) wrow[nt] = wr + static_cast<int64_t>(min(16 * nt + m, E - 1)) * H;
    const bool quant = x8 != nullptr && tm < T;
    const int nch_all = H / 32;
    const int per = SPLIT ? (nch_all + S - 1) / S : nch_all;
    const int c_lo = slice * per;                       // this block's chunks [c_lo, nch)
    const int nch = min(nch_all, c_lo + per);

    f64x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f64x4{0.0, 0.0, 0.0, 0.0};
    // chunks c = wave + NW i, loaded kAhead at a time so that their latencies overlap
    for (int c0 = c_lo + wave; c0 < nch; c0 += kAhead * NW) {
        uint4 xv[kAhead], wv[kAhead][NT];
#pragma unroll
        for (int a = 0; a < kAhead; ++a) {
            const int c = min(c0 + a * NW, nch - 1);      // past the end: reloads the last chunk
            const int h = 32 * c + 8 * g;
            xv[a] = *reinterpret_cast<const uint4 *>(xrow + h);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) wv[a][nt] = *reinterpret_cast<const uint4 *>(wrow[nt] + h);
        }
#pragma unroll
        for (int a = 0; a < kAhead; ++a) {
            const int c = c0 + a * NW;
            if (c >= nch) break;
            if (quant) mx8_store_quarter(xv[a], x8, T, H, tm, 32 * c + 8 * g, g == 0);
            double xd[8];
            bf16x8_to_f64(xv[a], xd);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                double wd[8];
                bf16x8_to_f64(wv[a][nt], wd);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd[j], wd[j], acc[nt], 0, 0, 0);
            }
        }
    }
    // lane (n, g) holds D[g + 4i][n] of each expert tile: token g + 4i, expert 16 nt + n;
    // the wavefronts' partial sums are added in wavefront order
    for (int w = 0; w < NW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    double *dst = &lg[(g + 4 * i) * LS + 16 * nt + m];
                    *dst = w == 0 ? acc[nt][i] : *dst + acc[nt][i];
                }
        }
        __syncthreads();
    }
    if (SPLIT) {
        for (int i = threadIdx.x; i < kRT * E; i += THREADS) {
            const int j = i / E, e = i % E;
            if (t0 + j < T) part[(static_cast<int64_t>(slice) * T + t0 + j) * E + e] = lg[j * LS + e];
        }
        return;
    }
    for (int i = threadIdx.x; i < kRT * E; i += THREADS) {
        const int j = i / E, e = i % E;
        lg[j * LS + e] += static_cast<double>(bf16_to_f32(br[e]));
    }
    __syncthreads();
    for (int j = wave; j < kRT; j += NW) {
        const int64_t t = t0 + j;
        if (t < T)
            topk_softmax_wave(&lg[j * LS], E, k, lane, topk_idx + t * k, topk_w + t * k, nullptr, nullptr,
                              logits_out ? logits_out + t * E : nullptr, s_tk[wave]);
    }
}

// Logits from S slices of partial sums (added in slice order) plus the bias, then the top-k
// and softmax of the token: one wavefront per token.
__global__ __launch_bounds__(512) void k_route_topk(const double *__restrict__ part, int S,
                                                    const uint16_t *__restrict__ br, int64_t T, int E, int k,
                                                    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
                                                    float *__restrict__ logits_out) {
    __shared__ __attribute__((aligned(16))) uint64_t s_tk[8][kTopkScratch];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 8 + wave;
    if (t >= T) return;
    double v[kTopkC];
#pragma unroll
    for (int c = 0; c < kTopkC; ++c) {
        const int e = lane + kWave * c;
        double l = 0.0;
        if (e < E) {
            l = part[t * E + e];
            for (int q = 1; q < S; ++q) l += part[(static_cast<int64_t>(q) * T + t) * E + e];
            l += static_cast<double>(bf16_to_f32(br[e]));
            if (logits_out) logits_out[t * E + e] = static_cast<float>(l);
        }
        v[c] = l;
    }
    topk_softmax_values(v, E, k, lane, topk_idx + t * k, topk_w + t * k, nullptr, nullptr, s_tk[wave]);
}

template <int NI>
void launch_token(const Dims &d, const uint16_t *x, const uint16_t *gamma, double eps, const uint16_t *w,
                  const uint16_t *b, int32_t *idx, float *wt, float *logits, uint8_t *x8, hipStream_t s) {
    MOE_LAUNCH((k_route_token<NI>), dim3(static_cast<unsigned>(d.T)), dim3(512), 0, s, x, gamma, eps, w,
                       b, d.H, d.E, d.k, idx, wt, logits, x8, static_cast<int>(d.T));
}

}  // namespace

hipError_t launch_logits(const Dims &d, const uint16_t *x, const uint16_t *gamma, double eps,
                         const uint16_t *router_w, const uint16_t *router_b, double *logits, uint8_t *x8,
                         hipStream_t s) {
    if (d.T <= 0) return hipSuccess;
    const int niq = (d.H + 2047) / 2048;
    const dim3 grid(static_cast<unsigned>((d.E + 1) / 2 + 1), static_cast<unsigned>(d.T));
    switch (niq) {
        case 1: MOE_LAUNCH((k_logits<1>), grid, dim3(256), 0, s, x, gamma, eps, router_w, router_b, d.H, d.E, logits, x8, static_cast<int>(d.T)); break;
        case 2: MOE_LAUNCH((k_logits<2>), grid, dim3(256), 0, s, x, gamma, eps, router_w, router_b, d.H, d.E, logits, x8, static_cast<int>(d.T)); break;
        case 3: MOE_LAUNCH((k_logits<3>), grid, dim3(256), 0, s, x, gamma, eps, router_w, router_b, d.H, d.E, logits, x8, static_cast<int>(d.T)); break;
        default: return hipErrorInvalidValue;   // H > 6144: the caller uses launch_route
    }
    return hipGetLastError();
}

int route_split(const Dims &d) {
    if (d.T <= kDecodeMaxT) return 1;
    const int64_t groups = (d.T + kRT - 1) / kRT;
    if (d.E < 64 || groups >= kRouteSplitCUs) return 1;       // enough 16-token groups (or little work per group)
    return groups * 2 >= kRouteSplitCUs ? 2 : 4;
}

int64_t route_part_doubles(const Dims &d) {
    const int S = route_split(d);
    return S > 1 ? static_cast<int64_t>(S) * d.T * d.E : 0;
}

hipError_t launch_route(const Dims &d, const uint16_t *x, const uint16_t *gamma, double eps,
                        const uint16_t *router_w, const uint16_t *router_b, int32_t *topk_idx, float *topk_w,
                        float *logits, uint8_t *x8, hipStream_t s, double *part) {
    if (d.T <= 0) return hipSuccess;
    const int ni = (d.H + 511) / 512;
    if (gamma != nullptr && !route_normalizes(d)) return hipErrorInvalidValue;
    if (d.T <= kDecodeMaxT && ni <= 7) {
        switch (ni) {
            case 1: launch_token<1>(d, x, gamma, eps, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 2: launch_token<2>(d, x, gamma, eps, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 3: launch_token<3>(d, x, gamma, eps, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 4: launch_token<4>(d, x, gamma, eps, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 5: launch_token<5>(d, x, gamma, eps, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            case 6: launch_token<6>(d, x, gamma, eps, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
            default: launch_token<7>(d, x, gamma, eps, router_w, router_b, topk_idx, topk_w, logits, x8, s); break;
        }
    } else {
        const int64_t groups = (d.T + kRT - 1) / kRT;
        const int S = part != nullptr ? route_split(d) : 1;
        const dim3 grid(static_cast<unsigned>(groups * S));
        // with S > 1: one stage, two launches (the partial-logit kernel records the stage's start
        // event, the top-k kernel its stop event)
        const LaunchEvents ev = launch_events();
        if (S > 1) launch_events() = LaunchEvents{ev.start, nullptr};
#define MOE_ROUTE(NT) do { if (S > 1) MOE_LAUNCH((k_route<NT, true>), grid, dim3(kRouteThreads), 0, s, x, router_w, \
                                         router_b, d.T, d.H, d.E, d.k, topk_idx, topk_w, logits, x8, part, S); \
                           else MOE_LAUNCH((k_route<NT, false>), grid, dim3(kRouteThreads), 0, s, x, router_w, \
                                         router_b, d.T, d.H, d.E, d.k, topk_idx, topk_w, logits, x8, part, 1); } while (0)
#define MOE_ROUTE_WIDE(NT) do { if (S > 1) MOE_LAUNCH((k_route<NT, true, 1024>), grid, dim3(1024), 0, s, x, router_w, \
                                         router_b, d.T, d.H, d.E, d.k, topk_idx, topk_w, logits, x8, part, S); \
                           else MOE_LAUNCH((k_route<NT, false, 1024>), grid, dim3(1024), 0, s, x, router_w, \
                                         router_b, d.T, d.H, d.E, d.k, topk_idx, topk_w, logits, x8, part, 1); } while (0)
        if (d.E <= 16) MOE_ROUTE_WIDE(1);
        else if (d.E <= 32) MOE_ROUTE_WIDE(2);
        else if (d.E <= 64) MOE_ROUTE(4);
        else if (d.E <= 128) MOE_ROUTE(8);
        else MOE_ROUTE(16);
#undef MOE_ROUTE
#undef MOE_ROUTE_WIDE
        if (S > 1) {
            const hipError_t e1 = hipGetLastError();
            if (e1 != hipSuccess) {
                launch_events() = ev;
                return e1;
            }
            launch_events() = LaunchEvents{nullptr, ev.stop};
            MOE_LAUNCH(k_route_topk, dim3(static_cast<unsigned>((d.T + 7) / 8)), dim3(512), 0, s, part, S, router_b,
                       d.T, d.E, d.k, topk_idx, topk_w, logits);
            launch_events() = ev;
        }
    }
    return hipGetLastError();
}

}  // namespace moe
