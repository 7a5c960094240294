/*
 * CPU oracle for the GPT-OSS MXFP4 mixture-of-experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously-correct
 * definition the GPU kernels are checked against. Only the test suite, the
 * package smoke check and the benchmark's CPU-baseline leg may load it; the
 * product path never does. It shares no code, header, table or helper with
 * the HIP library.
 *
 * Arithmetic: every floating-point step is IEEE double. Inputs arrive as bf16
 * bit patterns (exact in double) and packed MXFP4 bytes (exact in double after
 * decoding), so the only rounding is that of the double operations themselves.
 * Loops follow the definitions in the order the pages state them; no blocking,
 * reordering or fusion beyond what the definitions say. Parallelism (OpenMP)
 * is only across independent tokens or independent output elements and never
 * changes the arithmetic of any one result.
 *
 * Sources (web pages, cited by title and section):
 *  [ZM]  ZeroModels "GPT-OSS" documentation page: the intro list items
 *        "Mixture-of-experts feed-forward" and "MXFP4 experts"; the "API"
 *        table (embed_dim, mlp_dim, num_experts, num_experts_per_tok);
 *        "Precision" (bf16 dense weights, 4-bit experts).
 *  [MT]  MaxText pull request "Checkpoint conversion utility: gpt-oss orbax
 *        scan to hf, many-to-one transform, inhomogeneous scan block",
 *        section "1 Support many-to-one transform" (gate = even columns,
 *        up = odd columns of the fused gate_up projection and its bias).
 *  [MB]  NeMo Megatron-Bridge API page "bridge.models.gpt_oss.gpt_oss_bridge":
 *        maybe_modify_loaded_hf_weight (MXFP4-dequantized down_proj is
 *        [E, hidden, intermediate]; gate_up is [E, 2*intermediate, hidden])
 *        and GPTOSSMLPGateUpProjMapping (alternating row interleaving).
 *  [MLX] "GPT-OSS MLX Implementation" README, "Architecture Details":
 *        RMSNorm with Pre-LN placement (the layer's input is normalized, the
 *        block adds the layer's output to its un-normalized input); [ZM] "API"
 *        table: norm_eps 1e-5.
 *  [OCP] OCP Microscaling Formats (MX) v1.0 specification, the FP4 E2M1
 *        element type and the E8M0 shared scale (outside the pages; the pages
 *        name the format only).
 *
 * Readings where the pages are silent (each is listed with its pin in the
 * design notes): low nibble holds the even column; gate is clamped above
 * only and up to [-limit, limit]; the softmax runs over the k selected
 * logits; ties in the top-k go to the lower expert index; every selected
 * expert's output includes its own down bias.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* Threads the token-parallel loops use (OpenMP's current maximum). */
ORACLE_API int oracle_max_threads(void)
{
    return omp_get_max_threads();
}

/* bf16 bit pattern -> double (exact). */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * [OCP] FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no
 * infinities or NaN. Exponent field 0 encodes subnormals 0 and 0.5.
 * [ZM] "MXFP4 experts": the expert weights are nibbles of this type.
 */
ORACLE_API double oracle_e2m1(int code)
{
    int sign = (code >> 3) & 1;
    int exp_field = (code >> 1) & 3;
    int mant = code & 1;
    double magnitude;
    if (exp_field == 0)
        magnitude = 0.5 * mant;                         /* subnormal: m * 2^(1-1) / 2 */
    else
        magnitude = ldexp(1.0 + 0.5 * mant, exp_field - 1);
    return sign ? -magnitude : magnitude;
}

/* [OCP] E8M0 shared scale: 2^(byte - 127); 0xFF is NaN. [ZM] "e8m0 scales". */
ORACLE_API double oracle_e8m0(int byte)
{
    if (byte == 255)
        return NAN;
    return ldexp(1.0, byte - 127);
}

/*
 * One dequantized weight W[row, col] of a packed [rows, cols] matrix
 * ([ZM] "MXFP4 experts"; [MB] orientation: blocks run along the last,
 * contraction axis). Byte col/2 of the row holds columns col & ~1 (low nibble)
 * and col | 1 (high nibble); scale col/32 of the row scales the 32-column block.
 */
static double weight_at(const uint8_t *blocks, const uint8_t *scales,
                        int64_t row, int64_t col, int64_t cols)
{
    uint8_t byte = blocks[row * (cols / 2) + col / 2];
    int code = (col & 1) ? (byte >> 4) : (byte & 0x0F);
    return oracle_e2m1(code) * oracle_e8m0(scales[row * (cols / 32) + col / 32]);
}

/*
 * Dequantize a whole packed [rows, cols] matrix to double: out[r, c] is weight_at(r, c),
 * with the 16 E2M1 codes and the 256 E8M0 bytes decoded once each by the functions above
 * (rows are independent; OpenMP splits them across threads).
 */
ORACLE_API void oracle_dequant(const uint8_t *blocks, const uint8_t *scales,
                               int64_t rows, int64_t cols, double *out)
{
    double value[16], scale[256];
    for (int code = 0; code < 16; ++code)
        value[code] = oracle_e2m1(code);
    for (int byte = 0; byte < 256; ++byte)
        scale[byte] = oracle_e8m0(byte);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            const uint8_t byte = blocks[r * (cols / 2) + c / 2];
            const int code = (c & 1) ? (byte >> 4) : (byte & 0x0F);
            out[r * cols + c] = value[code] * scale[scales[r * (cols / 32) + c / 32]];
        }
}

/*
 * [ZM] "Mixture-of-experts feed-forward": the clamped gated SiLU applied to the
 * de-interleaved gate and up values: (up + 1) * gate * sigmoid(alpha * gate),
 * clamp `limit`. Reading: gate <= limit, -limit <= up <= limit.
 */
ORACLE_API double oracle_swiglu(double gate, double up, double alpha, double limit)
{
    double g = gate < limit ? gate : limit;
    double u = up < -limit ? -limit : (up > limit ? limit : up);
    double sigmoid = 1.0 / (1.0 + exp(-alpha * g));
    return (u + 1.0) * g * sigmoid;
}

/* oracle_swiglu applied element by element: h[i] = swiglu(gate[i], up[i]). */
ORACLE_API void oracle_swiglu_n(const double *gate, const double *up, int64_t n, double alpha, double limit,
                                double *h)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        h[i] = oracle_swiglu(gate[i], up[i], alpha, limit);
}

/*
 * Round a double to the nearest bf16 value, ties to even (finite, normal-range
 * inputs): with q the power of two of v's leading bit, bf16 keeps 8 significant
 * bits, so the value is rint(v / (q / 128)) * (q / 128); rint rounds ties to
 * even in the default rounding mode. Returns the bf16 bit pattern.
 */
static uint16_t bf16_round(double v)
{
    if (v == 0.0)
        return signbit(v) ? 0x8000u : 0u;
    int e;
    frexp(v, &e);                          /* |v| = f 2^e, 0.5 <= f < 1: leading bit 2^(e-1) */
    const double ulp = ldexp(1.0, e - 8);   /* 8 significant bits */
    const double r = rint(v / ulp) * ulp;
    const float f = (float)r;               /* exact: r has 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

ORACLE_API uint16_t oracle_bf16_round(double v)
{
    return bf16_round(v);
}

/*
 * [MLX] Pre-LN RMSNorm of the layer input, [ZM] epsilon: per token,
 *   ms = (sum_h x[t, h]^2) / H,  r = 1 / sqrt(ms + eps),
 *   xn[t, h] = bf16(x[t, h] * r * gamma[h])   (products left to right, one rounding to
 *                                               bf16 at the end, ties to even).
 * The normalized rows are bf16 like every activation the layer takes. `exact`
 * (optional) receives x * r * gamma before that rounding.
 */
ORACLE_API void oracle_rmsnorm(const uint16_t *x, const uint16_t *gamma, int64_t T, int H, double eps,
                               uint16_t *xn, double *exact)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int h = 0; h < H; ++h) {
            const double v = bf16_value(x[t * H + h]);
            ss += v * v;
        }
        const double r = 1.0 / sqrt(ss / H + eps);
        for (int h = 0; h < H; ++h) {
            const double v = bf16_value(x[t * H + h]) * r * bf16_value(gamma[h]);
            xn[t * H + h] = bf16_round(v);
            if (exact)
                exact[t * H + h] = v;
        }
    }
}

/*
 * [ZM] router: logits[t, e] = sum_h x[t, h] * Wr[e, h] + br[e], summed over h in
 * index order. `abs_sum` (optional) receives sum_h |x[t, h] * Wr[e, h]| + |br[e]|,
 * the scale of the rounding error any summation order can make.
 */
ORACLE_API void oracle_router(const uint16_t *x, const uint16_t *router_w,
                              const uint16_t *router_b, int64_t T, int H, int E,
                              double *logits, double *abs_sum)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0, mag = 0.0;
            for (int h = 0; h < H; ++h) {
                double p = bf16_value(x[t * H + h]) * bf16_value(router_w[(int64_t)e * H + h]);
                acc += p;
                mag += fabs(p);
            }
            double b = bf16_value(router_b[e]);
            logits[t * E + e] = acc + b;
            if (abs_sum)
                abs_sum[t * E + e] = mag + fabs(b);
        }
    }
}

/*
 * [ZM] top-k routing with softmax weights over the selected experts. Selection
 * order: larger logit first; equal logits -> lower expert index first.
 * w_j = exp(l_j - l_max) / sum_i exp(l_i - l_max) over the k selected.
 */
ORACLE_API void oracle_topk_softmax(const double *logits, int64_t T, int E, int k,
                                    int32_t *idx, double *w)
{
    for (int64_t t = 0; t < T; ++t) {
        const double *l = logits + t * E;
        int32_t *sel = idx + t * k;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int q = 0; q < j; ++q)
                    taken |= (sel[q] == e);
                if (taken)
                    continue;
                if (best < 0 || l[e] > l[best])   /* strict: an equal later index never wins */
                    best = e;
            }
            sel[j] = best;
        }
        double lmax = l[sel[0]];
        double denom = 0.0;
        for (int j = 0; j < k; ++j)
            denom += exp(l[sel[j]] - lmax);
        for (int j = 0; j < k; ++j)
            w[t * k + j] = exp(l[sel[j]] - lmax) / denom;
    }
}

/*
 * One expert applied to one token (bf16 activation row x[H]):
 *  gu[c] = sum_h x[h] * Wgu[e, c, h] + bgu[e, c]     c < 2I   ([ZM]; [MB] [E, 2I, H])
 *  gate[i] = gu[2i], up[i] = gu[2i + 1]                          ([MT]; [MB] interleave)
 *  h[i] = swiglu(gate[i], up[i])                                 ([ZM])
 *  o[d] = sum_i h[i] * Wdn[e, d, i] + bdn[e, d]      d < H   ([MB] [E, H, I])
 * `h_out` (length I) is optional; `o_out` has length H.
 */
ORACLE_API void oracle_expert(const uint16_t *x_row, int e, int H, int I,
                              const uint8_t *gu_blocks, const uint8_t *gu_scales,
                              const uint16_t *gu_bias, const uint8_t *dn_blocks,
                              const uint8_t *dn_scales, const uint16_t *dn_bias,
                              double alpha, double limit, double *h_out, double *o_out)
{
    const int64_t gu_rows = 2 * (int64_t)I;
    const uint8_t *gb = gu_blocks + (int64_t)e * gu_rows * (H / 2);
    const uint8_t *gs = gu_scales + (int64_t)e * gu_rows * (H / 32);
    const uint8_t *db = dn_blocks + (int64_t)e * H * (I / 2);
    const uint8_t *ds = dn_scales + (int64_t)e * H * (I / 32);
    double *gu = (double *)malloc(sizeof(double) * gu_rows);
    double *h = (double *)malloc(sizeof(double) * I);

    for (int64_t c = 0; c < gu_rows; ++c) {
        double acc = 0.0;
        for (int k = 0; k < H; ++k)
            acc += bf16_value(x_row[k]) * weight_at(gb, gs, c, k, H);
        gu[c] = acc + bf16_value(gu_bias[(int64_t)e * gu_rows + c]);
    }
    for (int i = 0; i < I; ++i)
        h[i] = oracle_swiglu(gu[2 * i], gu[2 * i + 1], alpha, limit);
    for (int d = 0; d < H; ++d) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i)
            acc += h[i] * weight_at(db, ds, d, i, I);
        o_out[d] = acc + bf16_value(dn_bias[(int64_t)e * H + d]);
    }
    if (h_out)
        memcpy(h_out, h, sizeof(double) * I);
    free(gu);
    free(h);
}

/*
 * The whole layer for a list of tokens `tokens[0..n)` (indices into x's T
 * rows), [ZM]: route, then y[t, :] = sum_j w_j * expert_{idx_j}(x[t, :]),
 * summed in slot order j = 0..k-1.
 * Outputs are per listed token (row r describes token tokens[r]):
 *  logits [n, E], abs_sum [n, E] (optional), idx [n, k], w [n, k],
 *  h [n, k, I] (optional), o [n, k, H] (optional), y [n, H].
 */
ORACLE_API void oracle_forward_tokens(
    const int64_t *tokens, int64_t n, int H, int I, int E, int k,
    const uint16_t *x, const uint16_t *router_w, const uint16_t *router_b,
    const uint8_t *gu_blocks, const uint8_t *gu_scales, const uint16_t *gu_bias,
    const uint8_t *dn_blocks, const uint8_t *dn_scales, const uint16_t *dn_bias,
    double alpha, double limit,
    double *logits, double *abs_sum, int32_t *idx, double *w,
    double *h, double *o, double *y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r) {
        const uint16_t *x_row = x + tokens[r] * (int64_t)H;
        oracle_router(x_row, router_w, router_b, 1, H, E, logits + r * E,
                      abs_sum ? abs_sum + r * E : NULL);
        oracle_topk_softmax(logits + r * E, 1, E, k, idx + r * k, w + r * k);
        double *o_tok = (double *)malloc(sizeof(double) * (size_t)k * H);
        for (int j = 0; j < k; ++j)
            oracle_expert(x_row, idx[r * k + j], H, I, gu_blocks, gu_scales, gu_bias,
                          dn_blocks, dn_scales, dn_bias, alpha, limit,
                          h ? h + (r * k + j) * (int64_t)I : NULL, o_tok + (int64_t)j * H);
        for (int d = 0; d < H; ++d) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += w[r * k + j] * o_tok[(int64_t)j * H + d];
            y[r * (int64_t)H + d] = acc;
        }
        if (o)
            memcpy(o + r * (int64_t)k * H, o_tok, sizeof(double) * (size_t)k * H);
        free(o_tok);
    }
}
