// The layer's expert GEMMs on a bank dequantized once to bf16 (ZeroModels GPT-OSS page, "MXFP4
// experts": longer prefills dequantize the whole bank once, and both paths give identical
// results). Grouped over the expert-sorted rows of launch_permute, on the bf16 MFMA:
//   up  : h[r, i] = bf16(swiglu(x[tok(r)] . Wgu[e, 2i] + bgu[e, 2i], x[tok(r)] . Wgu[e, 2i+1] + bgu[e, 2i+1]))
//   down: o[r, n] = sorted_w[r] * (h[r] . Wdn[e, n] + bdn[e, n])          (fp32)
// with e the expert of sorted row r. The packed path (gemm_grouped.hip) never expands the
// weights; this one exists to measure what expanding them costs on this chip.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kBM = 128;                      // rows per tile
constexpr int kBN = 128;                      // output columns (weight rows) per tile
constexpr int kBK = 64;                       // contraction per stage
constexpr int kThreads = 256;                 // 4 wavefronts, 2 x 2 over the tile
constexpr int kRowB = kBK * 2;                // bytes of a tile row per stage
constexpr int kTileB = kBM * kRowB;           // 16 KB (A and B alike)
constexpr int kStageB = 2 * kTileB;           // A then B
constexpr int kLds = 2 * kStageB;             // two stages
constexpr int kBlocksPerXcd = 64;             // two workgroups per CU
constexpr int kGrid = 8 * kBlocksPerXcd;

static_assert(kBM == kBN, "A and B tiles share the load mapping");

// Byte offset of 16-byte slot s of tile row r: slots XOR-swizzled by the row so that the
// MFMA operand reads (16 rows, one slot each) hit 8 distinct slots per 8 lanes.
__device__ __forceinline__ uint32_t slot_at(int r, int s) { return r * kRowB + ((s ^ (r & 7)) << 4); }

template <bool UP>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_bf16(
    const uint16_t *a,                               // up: x [T, K]; down: h [T k, K] (sorted rows)
    const int32_t *__restrict__ sorted_token,        // up only
    const float *__restrict__ sorted_w,              // down only
    const uint16_t *w, const uint16_t *__restrict__ wbias,   // [E, Nrows, K], [E, Nrows]
    const int32_t *__restrict__ offsets, int E, int K, int Nrows, float alpha, float limit,
    uint16_t *__restrict__ h,                        // up: [T k, Nrows / 2]
    float *__restrict__ o) {                         // down: [T k, Nrows]
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int s_off[kMaxE + 1];
    __shared__ int s_icum[kMaxE + 1];                // item prefix over experts

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int m = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int ntn = (Nrows + kBN - 1) / kBN;
    for (int e = tid; e <= E; e += kThreads) s_off[e] = offsets[e];
    __syncthreads();
    if (wave == 0) {
        // expert e has ceil(rows / BM) row tiles x ntn column tiles (E <= 256: four per lane)
        int v[4], local = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * lane + c;
            v[c] = e < E ? ntn * ((s_off[e + 1] - s_off[e] + kBM - 1) / kBM) : 0;
            local += v[c];
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int u = __shfl_up(incl, off);
            if (lane >= off) incl += u;
        }
        int run = incl - local;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * lane + c;
            if (e < E) s_icum[e] = run;
            run += v[c];
        }
        if (lane == kWave - 1) s_icum[E] = incl;
    }
    __syncthreads();
    const int items = s_icum[E];
    const int nk = (K + kBK - 1) / kBK;
    // this thread's share of a stage's loads: tile rows lr0 + 32 q (q < 4), 16-byte slot ls
    const int lr0 = tid >> 3, ls = tid & 7;
    const int xcd = blockIdx.x & 7, lb = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;

    // XCD-aware walk: chunk c of per_xcd consecutive items runs on XCD c % 8, so that the
    // row tiles of one weight tile (consecutive items) share that XCD's L2
    for (int c = xcd; c * per_xcd < items; c += 8) {
        const int item = c * per_xcd + lb;
        if (item >= items) continue;
        int lo = 0, hi = E - 1;                      // last e with s_icum[e] <= item
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_icum[mid] <= item) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int mt_e = (s_off[e + 1] - s_off[e] + kBM - 1) / kBM;
        const int local_item = item - s_icum[e];
        const int n0 = (local_item / mt_e) * kBN;
        const int row0 = s_off[e] + (local_item % mt_e) * kBM;
        const int rows = min(kBM, s_off[e + 1] - row0);

        const uint16_t *arow[4], *brow[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = lr0 + 32 * q;
            arow[q] = nullptr;
            if (r < rows) {
                const int64_t src = UP ? sorted_token[row0 + r] : row0 + r;
                arow[q] = a + src * K;
            }
            brow[q] = n0 + r < Nrows ? w + (static_cast<int64_t>(e) * Nrows + n0 + r) * K : nullptr;
        }
        uint4 ra[4], rb[4];
        auto load_stage = [&](int kt) {
            const int k = kBK * kt + 8 * ls;
            const bool kin = k < K;                  // K is a multiple of 32: whole slots
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                ra[q] = kin && arow[q] ? *reinterpret_cast<const uint4 *>(arow[q] + k) : zero4();
                rb[q] = kin && brow[q] ? *reinterpret_cast<const uint4 *>(brow[q] + k) : zero4();
            }
        };
        auto store_stage = [&](int buf) {
            uint8_t *sa = lds + buf * kStageB;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t off = slot_at(lr0 + 32 * q, ls);
                *reinterpret_cast<uint4 *>(sa + off) = ra[q];
                *reinterpret_cast<uint4 *>(sa + kTileB + off) = rb[q];
            }
        };

        f32x4 acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        load_stage(0);
        store_stage(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more) load_stage(kt + 1);
            const uint8_t *sa = lds + (kt & 1) * kStageB;
            const uint8_t *sb = sa + kTileB;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                uint4 af[4], bf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    af[i] = *reinterpret_cast<const uint4 *>(sa + slot_at(64 * wm + 16 * i + m, 4 * ks + g));
                    bf[i] = *reinterpret_cast<const uint4 *>(sb + slot_at(64 * wn + 16 * i + m, 4 * ks + g));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = mfma16(as_bf16x8(af[i]), as_bf16x8(bf[j]), acc[i][j]);
            }
            if (more) store_stage((kt + 1) & 1);
            __syncthreads();
        }

        // epilogue. D lane (m, g) of tile (i, j) holds column 64 wn + 16 j + m, rows
        // 64 wm + 16 i + 4 g + 0..3.
        if (UP) {
            // gate (even column) and up (odd column) sit in neighbouring lanes; the even lane
            // forms h for its four rows into LDS ([128 rows][64 h columns] bf16), then the tile
            // leaves as 16-byte row segments
            uint16_t *s_h = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + 64 * wn + 16 * j + m;
                const float b = col < Nrows ? bf16_to_f32(wbias[static_cast<int64_t>(e) * Nrows + col]) : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float v = acc[i][j][r] + b;
                        const float up = lane_xor1(v);
                        if ((m & 1) == 0) {
                            const int lr = 64 * wm + 16 * i + 4 * g + r;
                            s_h[lr * 64 + 32 * wn + 8 * j + (m >> 1)] = f32_to_bf16(swiglu(v, up, alpha, limit));
                        }
                    }
            }
            __syncthreads();
            const int I = Nrows / 2, h0 = n0 / 2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int lr = lr0 + 32 * q;
                if (lr < rows && h0 + 8 * ls < I)
                    *reinterpret_cast<uint4 *>(h + static_cast<int64_t>(row0 + lr) * I + h0 + 8 * ls) =
                        *reinterpret_cast<const uint4 *>(s_h + lr * 64 + 8 * ls);
            }
            __syncthreads();     // s_h is the next item's first stage
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = n0 + 64 * wn + 16 * j + m;
                if (col >= Nrows) continue;
                const float b = bf16_to_f32(wbias[static_cast<int64_t>(e) * Nrows + col]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int lr = 64 * wm + 16 * i + 4 * g + r;
                        if (lr < rows)
                            o[static_cast<int64_t>(row0 + lr) * Nrows + col] = (acc[i][j][r] + b) * sorted_w[row0 + lr];
                    }
            }
        }
    }
}

template <bool UP>
hipError_t launch_bank(const uint16_t *a, const int32_t *sorted_token, const float *sorted_w, const uint16_t *w,
                       const uint16_t *bias, const int32_t *offsets, const Dims &d, int K, int Nrows, uint16_t *h,
                       float *o, hipStream_t s) {
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void *>(&k_gemm_bf16<UP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (attr != hipSuccess) return attr;
    // an upper bound on the items (sum over experts of row tiles x column tiles)
    const int64_t items = ((d.T * d.k + kBM - 1) / kBM + d.E) * ((Nrows + kBN - 1) / kBN);
    const unsigned grid = static_cast<unsigned>(items < kGrid ? ((items + 7) / 8) * 8 : kGrid);
    MOE_LAUNCH((k_gemm_bf16<UP>), dim3(grid), dim3(kThreads), kLds, s, a, sorted_token, sorted_w, w, bias, offsets,
               d.E, K, Nrows, d.alpha, d.limit, h, o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_up_bank(const Dims &d, const uint16_t *x, const uint16_t *gu_w, const uint16_t *gu_bias,
                          const int32_t *offsets, const int32_t *sorted_token, uint16_t *h, hipStream_t s) {
    return launch_bank<true>(x, sorted_token, nullptr, gu_w, gu_bias, offsets, d, d.H, 2 * d.I, h, nullptr, s);
}

hipError_t launch_down_bank(const Dims &d, const uint16_t *h, const uint16_t *dn_w, const uint16_t *dn_bias,
                            const int32_t *offsets, const float *sorted_w, float *o, hipStream_t s) {
    return launch_bank<false>(h, nullptr, sorted_w, dn_w, dn_bias, offsets, d, d.I, d.H, nullptr, o, s);
}

}  // namespace moe
