// Grouped expert GEMMs over expert-sorted rows (prefill path) on gfx950's block-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4): the packed MXFP4 weight blocks are the B operand as
// stored, the activations are E4M3 hi/lo pairs (mx8 matrices, see mx_mfma.h) as A rows.
//
//  up  : h[r, i] = swiglu(x[tok(r)] . Wgu[e, 2i] + bgu[e, 2i], x[tok(r)] . Wgu[e, 2i+1] + bgu[e, 2i+1])
//        (ZeroModels GPT-OSS page, "Mixture-of-experts feed-forward"; gate/up interleave:
//        MaxText PR "Checkpoint conversion utility ...", "1 Support many-to-one transform";
//        orientation [E, 2I, H]: Megatron-Bridge gpt_oss_bridge page), written as the h8
//        matrix (mx8 data rows with group-major scales, mx_mfma.h; T k rows of I, sorted-row
//        order)
//  down: o[r, d] = w[r] * (h[r] . Wdn[e, d] + bdn[e, d])    (orientation [E, H, I], same page)
//
// Work list: every expert's rows [offsets[e], offsets[e+1]) are cut into BM-row tiles; each
// expert's (n-tile, m-tile) pairs, m-tile innermost, form one flattened list over all
// experts. The grid is persistent (one block per CU) and XCD-aware: chunk c of 32
// consecutive items runs on XCD c % 8 (block b runs on XCD b % 8), one item per block, so
// that the blocks running together on an XCD share an expert's weight tiles (read from HBM
// once, then from that XCD's L2) and its activation tiles.
//
// Block tile: BM = 128 activation rows (256 A rows: hi, lo) x BN = 256 output columns; the
// contraction advances BK = 128 (one MFMA step = four scale blocks) per stage. Eight
// wavefronts, two per SIMD, in a 4 x 2 arrangement: wavefront (wm, wn) owns the 16-row A
// tiles 4 i + wm (i < 4; interleaved so that the rows of a partly filled tile are shared
// evenly, and tiles past the expert's rows are skipped) and columns 128 wn .. 128 wn + 127,
// i.e. 4 x 8 MFMA tiles (128 accumulators). The two wavefronts of a SIMD (wn = 0 and 1) run
// one phase apart (ping-pong): while one multiplies from registers, the other reads its
// next operands from LDS and issues global loads, and barriers separate the phases.
// Operands go from global memory straight into LDS (global_load_lds: each
// lane's 16 or 4 bytes land at the instruction's LDS base + lane * size) into a ring of
// three stage buffers; a stage's loads are issued two stages before it is multiplied. The
// loads are issued from inline assembly: the compiler then neither knows of them nor
// inserts its own (all-draining) waits before LDS reads; the kernel waits for exactly the
// stage it needs with vmcnt and publishes it with a barrier.
//
// Scale loads fetch a few bytes from each of many rows, so they touch far more cache lines
// than their size suggests; they are kept few. Only the hi rows' A scales are loaded (an
// mx8 lo row's scale is always its hi row's minus 4) in aligned 16-byte windows that serve
// four stages, and the weight scales in 16-byte windows that serve three stages. The up GEMM
// writes h with group-major scales (mx_mfma.h), so that the down GEMM's A-scale windows of 128
// rows are 2 KB of contiguous bytes.
//
// Stage buffer layout (bytes):
//   A   [256 rows][128]: row R = 2 * (tile row) + part; its eight 16-byte chunks c are stored
//       at slot c ^ (R & 7).
//   B   [256 rows][64]: the stage's four packed MXFP4 blocks of weight row n, block c at
//       slot c ^ ((n >> 1) & 3).
//   (In a 16-byte operand read the eight lanes m .. m + 7 of a lane group hit eight different
//   slots of a 128-byte bank row. Orders that also keep lanes m and m + 8 apart over 256 bytes
//   measured slower, so the hardware serves these reads as the first layout assumes. Where
//   the bank conflicts its counters report arise is not separated by measurement; the
//   single-byte scale reads and the epilogue's staging are the remaining candidates.)
// Then two weight-scale group buffers (group j = stages 3j .. 3j + 2, buffer j % 2):
//   BSG [256 rows] 16 bytes: the four 4-byte-aligned dwords of weight scale row n that hold
//       the group's twelve scale bytes (weight scale rows are K / 32 bytes long, not
//       4-aligned); a dword past the tensor's end holds no valid byte and reads the last
//       dword instead.
// Then two A-scale group buffers (group j = stages 4j .. 4j + 3, buffer j % 2):
//   ASG [128 tile rows] 16 bytes: the E8M0 scales of the hi row's blocks 16j .. 16j + 15.
#include "device_common.h"
#include "kernels.h"
#include "lds_dma.h"
#include "mx_mfma.h"



namespace moe {
namespace {

template <int N> struct IntC { static constexpr int value = N; };

// f(IntC<0>{}), ..., f(IntC<N - 1>{}): compile-time indices (instruction operand selects).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(IntC<I>{});
        static_for<N, I + 1>(f);
    }
}

constexpr int kBN = 256;                       // output columns (weight rows) per tile
constexpr int kBK = 128;                       // contraction per stage
constexpr int kThreads = 512;                  // 8 wavefronts: 4 row groups x 2 column halves
constexpr int kChunk = 32;                     // items per XCD chunk (= blocks per XCD)
constexpr int kHS = 67;                        // up epilogue: padded row of 64 fp32 pairs
constexpr int kOS = 132;                       // down epilogue: padded row of 128 fp32 outputs
constexpr int kGA = 4;                         // stages per A-scale group (16 blocks)
constexpr int kASG = 128 * 16;                 // one A-scale group buffer

// The two tile configurations (LDS byte offsets).
//   Full tiles (SMALL = false): 128 activation rows; each stage buffer holds the stage's A
//   rows and its 256 weight rows' 64 bytes (half of a 128-byte line); weight scales in
//   16-byte windows per three stages (group ring of two).
//   Small groups (SMALL = true, experts of at most about 96 rows): 96 activation rows; the
//   stage buffers hold A only; the weights come as whole 128-byte lines that serve two
//   stages, into a ring of two such pair slots per column half (each half is read only by
//   the wavefronts of its column half, which also load it), with their scale windows per pair.
//   Both: the hi rows' A scales in 16-byte windows per four stages (group ring of two).
// Global-to-LDS instructions per wavefront: full: 4 A, 2 B per stage, 2 weight-scale dwords
// every third stage; small: 3 A per stage, and with every even stage 4 B and 2 weight-scale
// dwords; both: 1 A-scale window every fourth stage (wavefronts 0-1).
template <bool SMALL> struct GemmCfg;
template <> struct GemmCfg<false> {
    static constexpr int BM = 128, NA = 4;
    static constexpr int OFF_B = 2 * BM * kBK;                 // 32768
    static constexpr int STAGE = OFF_B + kBN * kBK / 2;        // 49152
    static constexpr int GS = 3;                               // stages per weight-scale group
    static constexpr int OFF_BSG = 3 * STAGE;                  // 147456
    static constexpr int BSG = kBN * 16;                       // one group buffer
    static constexpr int OFF_ASG = OFF_BSG + 2 * BSG;          // 155648
    static constexpr int TOTAL = OFF_ASG + 2 * kASG;           // 159744
};
template <> struct GemmCfg<true> {
    static constexpr int BM = 96, NA = 3;
    static constexpr int STAGE = 2 * BM * kBK;                 // 24576
    static constexpr int OFF_BP = 3 * STAGE;                   // 73728: pair slots [half][2]
    static constexpr int BP = 128 * 128;                       // one slot: 128 rows x 128 bytes
    static constexpr int OFF_BSG = OFF_BP + 4 * BP;            // 139264: scale slots [half][2]
    static constexpr int BSG = 128 * 16;
    static constexpr int OFF_ASG = OFF_BSG + 4 * BSG;          // 147456
    static constexpr int TOTAL = OFF_ASG + 2 * kASG;           // 151552
    static constexpr int OFF_B = 0, GS = 2;                    // (weights and their scales per pair)
};

__shared__ __attribute__((aligned(16))) uint8_t g_stages[GemmCfg<false>::TOTAL];
static_assert(GemmCfg<true>::TOTAL <= GemmCfg<false>::TOTAL, "one LDS array serves both configurations");
static_assert(8 * 32 * kOS * 4 <= GemmCfg<true>::OFF_ASG && 8 * 32 * kOS * 4 <= GemmCfg<false>::OFF_ASG,
              "the epilogue's staging fits both configurations below the A-scale groups");

template <bool UP, bool SMALL>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mx(
    const uint8_t *__restrict__ a8, int64_t a_rows,  // mx8 activations: up x8 (T rows), down h8 (T k rows)
    const int32_t *__restrict__ sorted_token,        // up only
    const float *__restrict__ sorted_w,              // down only
    const uint8_t *__restrict__ wblocks, const uint8_t *__restrict__ wscales,
    const uint16_t *__restrict__ wbias, const int32_t *__restrict__ offsets, int E,
    int K, int Nrows, float alpha, float limit,
    uint8_t *__restrict__ h8, int64_t h_rows,        // up: mx8 output (T k rows of Nrows / 2)
    float *__restrict__ o_out) {                     // down
    __shared__ int s_off[kMaxE + 1];
    __shared__ int s_icum[kMaxE + 1];               // item prefix over experts
    __shared__ uint16_t s_bias[kBN];                // the tile's biases (bf16)
    using C = GemmCfg<SMALL>;
    constexpr int kBM = C::BM;
    // up: the next tile's token indices ([2][128]); down: the tile rows' routing weights
    __shared__ int s_tok_rw[256];
    float *s_rw = reinterpret_cast<float *>(s_tok_rw);

    const int ntn = (Nrows + kBN - 1) / kBN;
    const int tid0 = threadIdx.x;
    for (int e = tid0; e <= E; e += kThreads) s_off[e] = offsets[e];
    __syncthreads();
    if (tid0 < kWave) {
        const int lane = tid0;
        // item prefix: expert e has ceil(rows / BM) m-tiles x ntn n-tiles (E <= 256: four
        // per lane)
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
            const int o = __shfl_up(incl, off);
            if (lane >= off) incl += o;
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
    const int nkb = K / 32;                      // scale blocks per row
    const int kt_total = (nkb + 3) / 4;
    const int kt_last = kt_total - 1;
    const int kbytes = K / 2;
    const int ass = mx8_scale_stride(K);
    const uint8_t *a_sc = a8 + static_cast<size_t>(2 * a_rows) * K;
    // XCD-aware walk over chunks of kChunk consecutive items: chunk c runs on XCD c % 8,
    // item c kChunk + j on that XCD's j-th block
    const int xcd = blockIdx.x & 7, lb = blockIdx.x >> 3;

    // Global addresses of one item's stage loads: a uniform base plus a 32-bit per-lane offset
    // (the host keeps every operand below 4 GiB).
    struct Addr {
        int e, row0, rows, n0;
        uint32_t a_off[C::NA], as_off, b_off[SMALL ? 4 : 2], bs_off[2], last4;
        const uint8_t *wblk, *wsc;
    };
    // the tile rows' token indices: tok (LDS, the tile's rows in order) or, with nullptr, the
    // global sorted_token
    auto addr_of = [&](int item, const int *tok) {
        Addr A;
        int lo = 0, hi = E - 1;                       // last e with s_icum[e] <= item
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_icum[mid] <= item) lo = mid; else hi = mid - 1;
        }
        A.e = lo;
        const int mt_e = (s_off[A.e + 1] - s_off[A.e] + kBM - 1) / kBM;
        const int local_item = item - s_icum[A.e];
        A.row0 = s_off[A.e] + (local_item % mt_e) * kBM;
        A.rows = min(kBM, s_off[A.e + 1] - A.row0);
        A.n0 = (local_item / mt_e) * kBN;
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
        // source byte row of tile A row R (activation row R / 2, part R % 2); rows past the
        // tile read the tile's first row (finite data, results never stored)
        auto a_src = [&](int R) -> uint32_t {
            const int ar = (R >> 1) < A.rows ? (R >> 1) : 0;
            const int src = UP ? (tok ? tok[ar] : sorted_token[A.row0 + ar]) : A.row0 + ar;
            return static_cast<uint32_t>(2 * src + (R & 1));
        };
        // A: instruction i of wavefront w fills A rows 8 (NA w + i) + lane / 8
#pragma unroll
        for (int i = 0; i < C::NA; ++i)
            A.a_off[i] = a_src(8 * (C::NA * wave + i) + (lane >> 3)) * static_cast<uint32_t>(K);
        // A-scale windows of the hi rows: wavefront w < 2 fills tile rows 64 w + lane (up:
        // window j of x8's row-major scale row, at byte 16 j; down: row r's 16 bytes of h8's
        // group j, at 16 (j rows + r))
        const uint32_t asrc = a_src(2 * (64 * (wave & 1) + lane));
        A.as_off = UP ? asrc * static_cast<uint32_t>(ass) : (asrc >> 1) * 16u;
        A.wblk = wblocks + static_cast<int64_t>(A.e) * Nrows * kbytes;
        if constexpr (SMALL) {
            // B pairs: instruction i of wavefront w fills rows 32 (w % 4) + 8 i + lane / 8 of
            // column half w / 4 (clamped to the matrix), a whole 128-byte line each
#pragma unroll
            for (int i = 0; i < 4; ++i)
                A.b_off[i] = min(A.n0 + 128 * (wave >> 2) + 32 * (wave & 3) + 8 * i + (lane >> 3), Nrows - 1) * kbytes;
        } else {
            // B: instruction i fills weight rows 32 w + 16 i + lane / 4 (clamped to the matrix)
#pragma unroll
            for (int i = 0; i < 2; ++i) A.b_off[i] = min(A.n0 + 32 * wave + 16 * i + (lane >> 2), Nrows - 1) * kbytes;
        }
        // weight scales, read as aligned dwords: for group j the four dwords from
        // ((n K/32 + 12 j) & ~3) hold the group's bytes; instruction i of wavefront w fills
        // rows 32 w + 16 i + lane / 4, dword lane % 4
        A.wsc = wscales + static_cast<int64_t>(A.e) * Nrows * nkb;
        const int64_t sc_len = static_cast<int64_t>(E - A.e) * Nrows * nkb;   // to the tensor's end
        A.last4 = static_cast<uint32_t>(min<int64_t>(sc_len, 0x7fffffff) - 4);
        // (small groups: rows 32 (w % 4) + 16 i + lane / 4 of column half w / 4, per pair)
        const int bs_row0 = SMALL ? 128 * (wave >> 2) + 32 * (wave & 3) : 32 * wave;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            A.bs_off[i] = (min(A.n0 + bs_row0 + 16 * i + (lane >> 2), Nrows - 1) * nkb & ~3) + 4 * (lane & 3);
        return A;
    };

    // up: the next tile's token indices, loaded into LDS while the current tile runs, so that
    // its stage addresses need no dependent global load when it starts
    int (*s_ntok)[128] = reinterpret_cast<int (*)[128]>(s_tok_rw);
    int ntile = 0;  // tiles this workgroup has started
    for (int c = xcd; c * kChunk < items; c += 8, ++ntile) {
        const int item = c * kChunk + lb;
        if (item >= items) continue;
        const bool pre = UP && ntile > 0;     // the previous tile loaded this one's tokens
        const Addr A = addr_of(item, pre ? s_ntok[ntile & 1] : nullptr);
        const int e = A.e, row0 = A.row0, rows = A.rows, n0 = A.n0;

        // Per-lane values are derived from an opaque copy of the thread index in every tile,
        // so that the compiler recomputes them here instead of keeping them live (spilled)
        // across the whole loop.
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
        const int m = lane & 15, g = lane >> 4;
        const int wm = wave & 3, wn = wave >> 2;

        // A chunk or block past K (last stage only) loads chunk / block 0 instead: finite data
        // whose contribution the multiply zeroes.
        const int a_c = (lane & 7) ^ ((lane >> 3) & 7);
        const int b_c = (lane & 3) ^ ((lane >> 3) & 3);
        const int a_vc = (K - kBK * kt_last) / 16;   // valid chunks in the last stage (2..8)
        const int b_vb = nkb - 4 * kt_last;          // valid blocks in the last stage (1..4)
        const uint32_t a_ch = 16 * a_c, a_ch_last = a_c < a_vc ? 16 * a_c : 0;
        const uint32_t b_ch = 16 * b_c, b_ch_last = b_c < b_vb ? 16 * b_c : 0;

        const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)g_stages;
        // a B pair's 16-byte chunk past the row (last pair only) loads the pair's chunk 0
        const int kbp = (kbytes - 128 * (kt_total / 2 + (kt_total & 1) - 1)) / 16;   // valid chunks of the last pair
        const uint32_t bp_ch = 16 * a_c, bp_ch_last = a_c < kbp ? 16 * a_c : 0;
        // the wavefront's share of stage kt's loads into buffer buf (A rows and the hi rows'
        // scales; the weight rows and their scales as the configuration takes them)
        auto issue_of = [&](const Addr &S, int buf, int kt) {
            const uint32_t lbuf = lds0 + buf * C::STAGE;
            const uint32_t ach = kt == kt_last ? a_ch_last : a_ch;
            const uint8_t *a_k = a8 + kBK * kt;          // uniform bases
#pragma unroll
            for (int i = 0; i < C::NA; ++i) dma16(a_k, S.a_off[i] + ach, lbuf + (C::NA * wave + i) * 1024);
            if (kt % kGA == 0 && wave < 2)
                dma16(UP ? a_sc + 4 * kt : a_sc + static_cast<size_t>(4 * kt) * a_rows, S.as_off,
                      lds0 + C::OFF_ASG + ((kt / kGA) & 1) * kASG + 1024 * wave);
            if constexpr (SMALL) {
                if ((kt & 1) == 0) {
                    const int q = kt >> 1;                  // pair q: stages 2q, 2q + 1
                    const bool last = 2 * q + 2 >= kt_total;
                    const uint32_t slot = static_cast<uint32_t>(2 * (wave >> 2) + (q & 1));
                    const uint32_t pb = lds0 + C::OFF_BP + slot * C::BP + 4096 * (wave & 3);
                    const uint8_t *b_k = S.wblk + 128 * q;
#pragma unroll
                    for (int i = 0; i < 4; ++i) dma16(b_k, S.b_off[i] + (last ? bp_ch_last : bp_ch), pb + 1024 * i);
                    const uint32_t gb = lds0 + C::OFF_BSG + slot * C::BSG + 512 * (wave & 3);
#pragma unroll
                    for (int i = 0; i < 2; ++i) dma4(S.wsc, min(S.bs_off[i] + 8 * q, S.last4), gb + 256 * i);
                }
            } else {
                const uint32_t bch = kt == kt_last ? b_ch_last : b_ch;
                const uint8_t *b_k = S.wblk + 64 * kt;
#pragma unroll
                for (int i = 0; i < 2; ++i) dma16(b_k, S.b_off[i] + bch, lbuf + C::OFF_B + (2 * wave + i) * 1024);
                if (kt % C::GS == 0) {
                    const int j = kt / C::GS;
                    const uint32_t gbuf = lds0 + C::OFF_BSG + (j & 1) * C::BSG + 512 * wave;
#pragma unroll
                    for (int i = 0; i < 2; ++i) dma4(S.wsc, min(S.bs_off[i] + 12 * j, S.last4), gbuf + 256 * i);
                }
            }
        };
        auto issue = [&](int buf, int kt) { issue_of(A, buf, kt); };

        // The tile body, for NL = the wavefront's row tiles that hold valid rows (0 to 4; a
        // compile-time constant, so that skipped tiles cost no branches and the accumulators
        // stay in their registers).
        auto tile_body = [&](auto nl_tag) {
        constexpr int NL = decltype(nl_tag)::value;
        f32x4 acc[4][8];
#pragma unroll
        for (int a = 0; a < NL; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

        // --- multiply: an 8-wavefront ping-pong. The wavefronts 0-3 (one per SIMD) and 4-7 (the
        // other one per SIMD) alternate between a memory phase and a matrix phase, one phase
        // apart, separated by workgroup barriers: while one wavefront of a SIMD multiplies
        // from registers, the other reads its next stage's operands from LDS and issues its
        // share of a later stage's global loads, so the matrix unit is fed from both.
        //   phase 2s:     wavefronts 0-3 read stage s;       4-7 multiply stage s - 1
        //   phase 2s + 1: wavefronts 0-3 multiply stage s;   4-7 read stage s
        // In its memory phase for stage s a wavefront also issues its loads of stage s + 2
        // into the buffer stage s - 1 used (both groups have read it by then). Before phase 2s
        // every wavefront waits for its loads of stage s (only stage s + 1's stay in flight),
        // and the barrier then publishes the stage; a memory phase ends with its LDS reads
        // complete, so the buffer is free for the refill that follows.
        //
        // Operand reads: B fragments and scales of the wavefront's eight column tiles, then
        // the A fragments of its row tiles. LDS addresses are one per-lane base per operand
        // plus constants. The scales are read as single bytes: the hi row of A row R's block
        // g (minus 4 for a lo row), and weight row n's block g of group stage s at byte
        // (n K/32) % 4 + 4 s + g of its 16-byte window (the same offset for all eight column
        // tiles: they are 16 rows apart). Small groups: the B fragment of stage s is chunk
        // 4 (s % 2) + g of the pair's 128-byte row, stored at slot chunk ^ (row % 8).
        const uint32_t lb_b = SMALL ? 128 * m + 16 * (g ^ (m & 7))
                                    : C::OFF_B + 8192 * wn + 64 * m + 16 * (g ^ ((m >> 1) & 3));
        const uint32_t lb_bs = C::OFF_BSG + 16 * ((SMALL ? 0 : 128 * wn) + m) + (((n0 + 128 * wn + m) * nkb) & 3) + g;
        const uint32_t lb_a = 2048 * wm + 128 * m + 16 * (g ^ (m & 7));
        const uint32_t lb_as = 16 * (8 * wm + (m >> 1)) + g;
        const uint32_t lo_row = 4u * (m & 1);
        // the wavefront's row tiles are the tile's 16-row tiles 4 mt + wm (interleaved, so
        // that a partly filled tile splits its rows evenly); only the first NL are multiplied
        uint4 bq[8], alo[4], ahi[4];
        // scale bytes packed four to a register (column tiles 4i .. 4i + 3 in sbp[i], row
        // tiles in sap); the instruction's operand select picks the byte
        uint32_t sbp[2], sap;
        // In the last stage of a contraction whose block count is not a multiple of 4
        // (vb < 4, a uniform branch), blocks past K get zero A data and unit scales, so they
        // add exactly 0.
        auto read_stage = [&](int kt) {
            const int buf = kt % 3;
            const uint8_t *base = g_stages + buf * C::STAGE;
            const uint8_t *bsrc, *gsc;
            uint32_t lbb = lb_b;
            int bstride;
            if constexpr (SMALL) {
                const int slot = 2 * wn + ((kt >> 1) & 1);
                bsrc = g_stages + C::OFF_BP + slot * C::BP;
                lbb ^= (kt & 1) ? 64u : 0u;          // chunk g + 4 for the pair's second stage
                bstride = 2048;                      // 16 rows of 128 bytes
                gsc = g_stages + slot * C::BSG + 4 * (kt & 1);
            } else {
                bsrc = base;
                bstride = 1024;
                gsc = g_stages + ((kt / C::GS) & 1) * C::BSG + 4 * (kt % C::GS);
            }
            const int vb = nkb - 4 * kt;
            const uint8_t *asg = g_stages + C::OFF_ASG + ((kt / kGA) & 1) * kASG + 4 * (kt % kGA);
            uint32_t sb[8], sa[4];
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                bq[nt] = *reinterpret_cast<const uint4 *>(bsrc + lbb + bstride * nt);
                sb[nt] = gsc[lb_bs + 256 * nt];
            }
#pragma unroll
            for (int mt = 0; mt < NL; ++mt) {
                alo[mt] = *reinterpret_cast<const uint4 *>(base + lb_a + 8192 * mt);
                ahi[mt] = *reinterpret_cast<const uint4 *>(base + (lb_a ^ 64u) + 8192 * mt);   // chunk g + 4
                sa[mt] = asg[lb_as + 512 * mt] - lo_row;
            }
#pragma unroll
            for (int mt = NL; mt < 4; ++mt) sa[mt] = 127u;
            if (vb < 4) {
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) sb[nt] = g < vb ? sb[nt] : 127u;
#pragma unroll
                for (int mt = 0; mt < NL; ++mt) {
                    // lane group g carries blocks g / 2 (low half) and 2 + g / 2 (high half)
                    if ((g >> 1) >= vb) alo[mt] = zero4();
                    if (2 + (g >> 1) >= vb) ahi[mt] = zero4();
                    if (g >= vb) sa[mt] = 127u;
                }
            }
            sbp[0] = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
            sbp[1] = sb[4] | (sb[5] << 8) | (sb[6] << 16) | (sb[7] << 24);
            sap = sa[0] | (sa[1] << 8) | (sa[2] << 16) | (sa[3] << 24);
        };
        auto multiply = [&]() {
            static_for<NL>([&](auto mt_c) {
                constexpr int mt = decltype(mt_c)::value;
                const i32x8 af = mx_a_operand(alo[mt], ahi[mt]);
                static_for<8>([&](auto nt_c) {
                    constexpr int nt = decltype(nt_c)::value;
                    acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        af, mx_b_operand(bq[nt]), acc[mt][nt], 0, 4, mt, static_cast<int>(sap), nt & 3,
                        static_cast<int>(sbp[nt >> 2]));
                });
            });
        };
        // every wavefront's loads of stage s have landed (stage s + 1's, if any, stay in flight)
        auto wait_stage = [&](int s) {
            if (s + 1 < kt_total) {
                // this wavefront's loads of stage s + 1
                const int nas = wave < 2 && (s + 1) % kGA == 0 ? 1 : 0;
                const int n = SMALL ? 3 + nas + (((s + 1) & 1) == 0 ? 6 : 0)
                                    : 6 + nas + ((s + 1) % C::GS == 0 ? 2 : 0);
                switch (n) {
                    case 3: wait_vm<3>(); break;
                    case 4: wait_vm<4>(); break;
                    case 6: wait_vm<6>(); break;
                    case 7: wait_vm<7>(); break;
                    case 8: wait_vm<8>(); break;
                    case 9: wait_vm<9>(); break;
                    default: wait_vm<10>(); break;
                }
            } else {
                wait_vm<0>();
            }
        };
        auto phase_end = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            barrier_only();
            __builtin_amdgcn_sched_barrier(0);
        };

        // the epilogue's bias and routing-weight loads go out now (their latency hides behind
        // the contraction) and land in LDS after it
        const int bcol = min(n0 + tid, Nrows - 1);
        const uint16_t bias_v = tid < kBN ? wbias[static_cast<int64_t>(e) * Nrows + bcol] : 0;
        const float rw_v = !UP && tid < kBM ? sorted_w[row0 + min(tid, rows - 1)] : 0.f;
        wait_lgkm0();      // the previous tile's epilogue is done with LDS (loads may stay in flight)
        barrier_only();
        const int cn = c + 8, nitem = cn * kChunk + lb;
        const bool has_next = UP && cn * kChunk < items && nitem < items;
        if (has_next && wave < 2) {
            // the next tile's 128 token indices (rows past its end repeat its last row)
            int lo2 = 0, hi2 = E - 1;
            while (lo2 < hi2) {
                const int mid = (lo2 + hi2 + 1) >> 1;
                if (s_icum[mid] <= nitem) lo2 = mid; else hi2 = mid - 1;
            }
            const int mt2 = (s_off[lo2 + 1] - s_off[lo2] + kBM - 1) / kBM;
            const int r0 = __builtin_amdgcn_readfirstlane(s_off[lo2] + ((nitem - s_icum[lo2]) % mt2) * kBM);
            const int nr = min(kBM, s_off[lo2 + 1] - r0);
            const uint32_t ldst = __builtin_amdgcn_readfirstlane(
                (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int *)&s_ntok[(ntile + 1) & 1][64 * wave]);
            dma4(reinterpret_cast<const uint8_t *>(sorted_token + r0),
                 4u * static_cast<uint32_t>(min(64 * wave + lane, nr - 1)), ldst);
        }
        issue(0, 0);
        if (kt_total > 1) issue(1, 1);
        wait_stage(0);
        phase_end();
        // the memory phase for stage kt: stage kt's operands into registers and stage kt + 2's
        // loads out (into the buffer of stage kt - 1, read by both groups two phases ago). The
        // small-group tiles issue the loads first, so that they have the operand reads' time
        // more to land before the wait that publishes them (120B gate_up 410 -> 405 us, down
        // 210 -> 202 us); the full tiles read first (no gain there, and issuing first keeps one
        // more address live across the reads: a spill in the full-tile gate_up GEMM).
        auto mem_phase = [&](int kt) {
            if constexpr (SMALL) {
                if (kt + 2 < kt_total) issue((kt + 2) % 3, kt + 2);
                read_stage(kt);
            } else {
                read_stage(kt);
                if (kt + 2 < kt_total) issue((kt + 2) % 3, kt + 2);
            }
            wait_lgkm0();
        };
        if (wave < 4) {
            for (int kt = 0; kt < kt_total; ++kt) {
                mem_phase(kt);                               // phase 2 kt
                phase_end();
                multiply();                                  // phase 2 kt + 1
                if (kt + 1 < kt_total) wait_stage(kt + 1);
                phase_end();
            }
            phase_end();                                     // phase 2 kt_total: idle
        } else {
            phase_end();                                     // phase 0: idle
            for (int kt = 0; kt < kt_total; ++kt) {
                mem_phase(kt);                               // phase 2 kt + 1
                if (kt + 1 < kt_total) wait_stage(kt + 1);
                phase_end();
                multiply();                                  // phase 2 kt + 2
                phase_end();
            }
        }
        if (tid < kBN) s_bias[tid] = bias_v;
        if (!UP && tid < kBM) s_rw[tid] = rw_v;
        __syncthreads();   // every wavefront is done with the stage buffers

        // --- epilogue. Lane (m, g) of MFMA tile (mt, nt) holds column 16 nt + m of the
        // wavefront's A rows 16 mt + 4g + r: its activation row 8 mt + 2g (r = 0, 1: hi, lo)
        // and 8 mt + 2g + 1 (r = 2, 3); value = D[hi] + D[lo]. The wavefront's activation row
        // r is the tile's row 32 (r / 8) + 8 wm + r % 8.
        if (UP) {
            // h of the wavefront's 32 rows x 64 pairs (fp32) into LDS (region `wave` of 32 kHS
            // floats), then each lane quantizes one (row, MX block) item
            float *s_h = reinterpret_cast<float *>(g_stages) + wave * (32 * kHS);
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int wr = n0 + 128 * wn + 16 * nt + m;
                const float bias = wr < Nrows ? bf16_to_f32(s_bias[wr - n0]) : 0.f;
                const int pair = 8 * nt + (m >> 1);
#pragma unroll
                for (int mt = 0; mt < NL; ++mt) {
                    const float v0 = acc[mt][nt][0] + acc[mt][nt][1] + bias;
                    const float v1 = acc[mt][nt][2] + acc[mt][nt][3] + bias;
                    // even lane (gate column) keeps row 8mt + 2g, odd lane (up) row 8mt + 2g + 1
                    const float other = lane_xor1((m & 1) ? v0 : v1);
                    const float gate = (m & 1) ? other : v0;
                    const float up = (m & 1) ? v1 : other;
                    s_h[(8 * mt + 2 * g + (m & 1)) * kHS + pair] = swiglu(gate, up, alpha, limit);
                }
            }
            __syncthreads();
            const int Iw = Nrows / 2;
            uint8_t *h_sc = h8 + static_cast<size_t>(2 * h_rows) * Iw;
            {
                const int r = lane >> 1, blk = lane & 1;
                const int R = 32 * (r >> 3) + 8 * wm + (r & 7);   // tile activation row
                const int ib = (n0 + 128 * wn) / 64 + blk;        // MX block of h
                if (R < rows && 64 * ib < Nrows) {
                    float v[32];
#pragma unroll
                    for (int i = 0; i < 32; ++i) v[i] = s_h[r * kHS + 32 * blk + i];
                    store_h8_block(v, h8, h_sc, static_cast<int64_t>(row0 + R), Iw, h_rows, ib);
                }
            }
        } else {
            // o of the wavefront's 32 rows x 128 columns (bias added, weighted) through LDS
            // (region `wave`, rows of kOS floats), so that each store writes 16 contiguous
            // bytes per lane
            float *s_o = reinterpret_cast<float *>(g_stages) + wave * (32 * kOS);
            float wrow[4][2];
#pragma unroll
            for (int mt = 0; mt < NL; ++mt)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int lr = 32 * mt + 8 * wm + 2 * g + j;
                    wrow[mt][j] = lr < rows ? s_rw[lr] : 0.f;
                }
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                const int d = n0 + 128 * wn + 16 * nt + m;
                if (d >= Nrows) continue;
                const float bd = bf16_to_f32(s_bias[d - n0]);
#pragma unroll
                for (int mt = 0; mt < NL; ++mt)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float v = acc[mt][nt][2 * j] + acc[mt][nt][2 * j + 1];
                        s_o[(8 * mt + 2 * g + j) * kOS + 16 * nt + m] = (v + bd) * wrow[mt][j];
                    }
            }
            __syncthreads();
#pragma unroll 4
            for (int it = 0; it < 16; ++it) {
                const int lrow = 2 * it + (lane >> 5);       // wavefront row
                const int c4 = 4 * (lane & 31);              // first of 4 columns
                const int lr = 32 * (lrow >> 3) + 8 * wm + (lrow & 7);   // tile row
                const int d = n0 + 128 * wn + c4;
                if (lr < rows && d < Nrows)
                    *reinterpret_cast<float4 *>(o_out + static_cast<int64_t>(row0 + lr) * Nrows + d) =
                        *reinterpret_cast<const float4 *>(s_o + lrow * kOS + c4);
            }
        }
        };
        // the wavefront's row tiles holding valid rows (of the (rows + 7) / 8 that do); none
        // when all its 128 columns lie past the matrix (the last column tile of a matrix whose
        // row count is not a multiple of 256), so that the SIMD's other wavefront runs alone
        const int nloc = n0 + 128 * wn >= Nrows ? 0 : ((rows + 7) / 8 - wm + 3) / 4;
        if (nloc > 3) { if constexpr (!SMALL) tile_body(IntC<4>{}); }
        else if (nloc > 2) tile_body(IntC<3>{});
        else if (nloc > 1) tile_body(IntC<2>{});
        else if (nloc > 0) tile_body(IntC<1>{});
        else tile_body(IntC<0>{});
    }
}

// y[t, d] = sum_j o[slot_row[t*K + j], d] in slot order, rounded to bf16. Thread = 4 columns
// per grid-stride step; its K slot indices, then its K rows, are loaded together so that the
// K row reads are in flight at once.
template <int K>
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ o,
                                                 const int32_t *__restrict__ slot_row, int64_t T,
                                                 int H, const uint16_t *__restrict__ res,
                                                 uint16_t *__restrict__ y) {
    const int per_row = H / 4;
    const int64_t total = T * per_row;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < total;
         q += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t t = q / per_row;
        const int d = static_cast<int>(q % per_row) * 4;
        int32_t sr[K];
#pragma unroll
        for (int j = 0; j < K; ++j) sr[j] = slot_row[t * K + j];
        float4 v[K];
#pragma unroll
        for (int j = 0; j < K; ++j) v[j] = *reinterpret_cast<const float4 *>(o + static_cast<int64_t>(sr[j]) * H + d);
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
        }
        if (res) add_residual4(s, res + t * H + d);
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
    // thread q: packed word q (8 values of MX block q / 4) -> 16 output bytes, so that a
    // wavefront's loads and stores are each one contiguous run
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < 4 * nblk;
         q += static_cast<int64_t>(gridDim.x) * 256) {
        const uint32_t word = reinterpret_cast<const uint32_t *>(blocks)[q];
        const float sc = e8m0_to_f32(scales[q >> 2]);
        reinterpret_cast<uint4 *>(out)[q] = __builtin_bit_cast(uint4, mxfp4_word_to_bf16x8(word, sc));
    }
}

// bf16 rows -> mx8 matrix (H8: with the h8 matrix's group-major scales): one thread per
// 32-element block per grid-stride step.
template <bool H8>
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
        if constexpr (H8) store_h8_block(v, q8, qs, r, cols, rows, b);
        else store_mx8_block(v, q8, qs, r, cols, ss, b);
    }
}

unsigned grid_for(int64_t items) {
    const int64_t blocks = (items + 255) / 256;
    return static_cast<unsigned>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

// One block per CU (the LDS stages take most of a CU's LDS), a multiple of 8 (XCDs).
int persistent_blocks() { return 256; }

// The small-group tiles (96 rows, whole-line weight pairs) when the experts average at most
// 96 routed rows: their 128-row tiles would be mostly empty and the weight stream bound.
bool small_groups(const Dims &d) { return d.T * d.k <= static_cast<int64_t>(GemmCfg<true>::BM) * d.E; }

template <bool UP, bool SMALL>
hipError_t launch_gemm(const Dims &d, const uint8_t *a8, int64_t a_rows, const int32_t *sorted_token,
                       const float *sorted_w, const uint8_t *wb, const uint8_t *ws, const uint16_t *wbias,
                       const int32_t *offsets, int K, int Nrows, uint8_t *h8, int64_t h_rows, float *o, hipStream_t s) {
    MOE_LAUNCH((k_gemm_mx<UP, SMALL>), dim3(persistent_blocks()), dim3(kThreads), 0, s, a8, a_rows, sorted_token,
               sorted_w, wb, ws, wbias, offsets, d.E, K, Nrows, d.alpha, d.limit, h8, h_rows, o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_up_grouped(const Dims &d, const uint8_t *x8, const uint8_t *gu_blocks,
                             const uint8_t *gu_scales, const uint16_t *gu_bias,
                             const int32_t *offsets, const int32_t *sorted_token,
                             uint8_t *h8, hipStream_t s) {
    if (small_groups(d))
        return launch_gemm<true, true>(d, x8, d.T, sorted_token, nullptr, gu_blocks, gu_scales, gu_bias, offsets,
                                       d.H, 2 * d.I, h8, d.T * d.k, nullptr, s);
    return launch_gemm<true, false>(d, x8, d.T, sorted_token, nullptr, gu_blocks, gu_scales, gu_bias, offsets,
                                    d.H, 2 * d.I, h8, d.T * d.k, nullptr, s);
}

hipError_t launch_down_grouped(const Dims &d, const uint8_t *h8, const uint8_t *dn_blocks,
                               const uint8_t *dn_scales, const uint16_t *dn_bias,
                               const int32_t *offsets, const float *sorted_w, float *o,
                               hipStream_t s) {
    if (small_groups(d))
        return launch_gemm<false, true>(d, h8, d.T * d.k, nullptr, sorted_w, dn_blocks, dn_scales, dn_bias, offsets,
                                        d.I, d.H, nullptr, 0, o, s);
    return launch_gemm<false, false>(d, h8, d.T * d.k, nullptr, sorted_w, dn_blocks, dn_scales, dn_bias, offsets,
                                     d.I, d.H, nullptr, 0, o, s);
}

hipError_t launch_combine(const Dims &d, const float *o, const int32_t *slot_row, const uint16_t *residual,
                          uint16_t *y, hipStream_t s) {
    const dim3 grid(grid_for(d.T * (d.H / 4)));
#define MOE_COMBINE(K) MOE_LAUNCH((k_combine<K>), grid, dim3(256), 0, s, o, slot_row, d.T, d.H, residual, y)
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

hipError_t launch_quantize(const uint16_t *x, int64_t rows, int cols, uint8_t *q8, bool h8, hipStream_t s) {
    const int64_t nblk = rows * (cols / 32);
    if (nblk == 0) return hipSuccess;
    if (h8) MOE_LAUNCH(k_quantize<true>, dim3(grid_for(nblk)), dim3(256), 0, s, x, rows, cols, q8);
    else MOE_LAUNCH(k_quantize<false>, dim3(grid_for(nblk)), dim3(256), 0, s, x, rows, cols, q8);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *blocks, const uint8_t *scales, int64_t rows, int cols,
                          uint16_t *out, hipStream_t s) {
    const int64_t nblk = rows * (cols / 32);
    if (nblk == 0) return hipSuccess;
    MOE_LAUNCH(k_dequant, dim3(grid_for(4 * nblk)), dim3(256), 0, s, blocks, scales,
                       nblk, out);
    return hipGetLastError();
}

}  // namespace moe
