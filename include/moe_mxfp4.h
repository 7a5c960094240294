/*
 * moe_mxfp4.h — C ABI of the MI355X (gfx950) GPT-OSS MXFP4 mixture-of-experts layer.
 *
 * The layer (ZeroModels GPT-OSS page, list item "Mixture-of-experts feed-forward"):
 *   1. router logits  l[t, e] = sum_h x[t, h] * Wr[e, h] + br[e]
 *   2. top-k experts per token (larger logit first, equal logits -> lower index),
 *      routing weights w = softmax over the k selected logits
 *   3. for each selected expert e: gu = x[t] . Wgu[e]^T + bgu[e]   (MXFP4 Wgu, dequantized
 *      on the fly: same page, "MXFP4 experts")
 *   4. gate = gu[0::2], up = gu[1::2] (MaxText PR "Checkpoint conversion utility: gpt-oss
 *      orbax scan to hf ...", section "1 Support many-to-one transform"; Megatron-Bridge
 *      gpt_oss_bridge page, GPTOSSMLPGateUpProjMapping: alternating row interleaving),
 *      h = (clamp(up, -limit, limit) + 1) * g * sigmoid(alpha * g), g = min(gate, limit)
 *   5. o = h . Wdn[e]^T + bdn[e]   (MXFP4 Wdn)
 *   6. y[t] = sum_j w[t, j] * o_j
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, owned by the
 *    caller. The library allocates nothing, frees nothing and keeps no state between
 *    calls. Inputs are read-only; outputs are fully overwritten.
 *  - bf16 tensors are passed as uint16_t bit patterns (moe_bf16_t).
 *  - `stream` is a hipStream_t (NULL = the null stream). All work is enqueued on it;
 *    no call synchronises. Calls on different streams with distinct output/workspace
 *    buffers may run concurrently.
 *  - T == 0 (no tokens) returns MOE_OK once the shape is valid, without reading any
 *    pointer argument and without launching anything.
 *  - Validation is host-only and happens before any launch. On error the call returns
 *    a nonzero moe_status_t, launches nothing and writes nothing; moe_mxfp4_last_error()
 *    returns a message (thread-local, valid until the next call on the thread). Launch
 *    failures return MOE_EHIP. Device faults surface at the caller's next synchronisation.
 *  - Determinism: identical inputs give bit-identical outputs (fixed summation orders,
 *    no floating-point atomics).
 *
 * Packed MXFP4 layout (ZeroModels GPT-OSS page, "MXFP4 experts": uint8 nibble blocks plus
 * e8m0 scales; orientation from the Megatron-Bridge gpt_oss_bridge page,
 * maybe_modify_loaded_hf_weight: dequantized gate_up is [E, 2I, H], down is [E, H, I]):
 *  - blocks [E, R, C/2] uint8: byte j of a row holds column 2j (low nibble) and column
 *    2j+1 (high nibble) as FP4 E2M1 codes. (Identical bytes to a [E, R, C/32, 16] view.)
 *  - scales [E, R, C/32] uint8: E8M0, the 32-column block c/32 of a row is multiplied by
 *    2^(s - 127). Supported scale bytes: 2..252 (every dequantized value is then an exact
 *    normal bf16); other bytes give unspecified values.
 *  - gate_up rows are interleaved: row 2i is gate_i, row 2i+1 is up_i (bias likewise).
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MXFP4_ABI_VERSION 6

typedef uint16_t moe_bf16_t;

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,      /* NULL pointer where one is required, T < 0, non-finite alpha/limit */
    MOE_ESHAPE = 2,      /* H or I not a positive multiple of 32, k < 1, k > E, k > 8, E > 256,
                            E < 1, T > 2^24, or the T k activation rows as an mx8 matrix
                            (moe_mxfp4_mx8_bytes(T k, max(H, I))) or one expert's packed
                            gate_up weights reaching 4 GiB (32-bit operand offsets) */
    MOE_EALIGN = 3,      /* a tensor pointer not 16-byte aligned; the two expert scale
                            pointers need 4-byte alignment; biases, router bias: any */
    MOE_EWORKSPACE = 4,  /* workspace NULL or smaller than moe_mxfp4_workspace_bytes() */
    MOE_EHIP = 5         /* a HIP launch failed */
} moe_status_t;

/* Layer shape. T = tokens, H = hidden (embed_dim), I = expert intermediate (mlp_dim),
 * E = experts, k = experts per token. alpha / limit: the SwiGLU constants (GPT-OSS:
 * 1.702 and 7.0, ZeroModels GPT-OSS page, "Mixture-of-experts feed-forward"). */
typedef struct {
    int64_t T;
    int32_t H, I, E, k;
    float swiglu_alpha;
    float swiglu_limit;
} moe_mxfp4_shape_t;

/* ABI version of the loaded library (MOE_MXFP4_ABI_VERSION at build time). */
int moe_mxfp4_abi_version(void);

/* Measurement support, not a step of the layer: the clock the CUs run at under a full-chip
 * ALU load (the published peak rates the benchmark divides by assume 2.4 GHz). Launches
 * `blocks` workgroups of 256 threads, each timing `iters` dependent multiply-adds; workgroup b
 * writes its shader-clock cycles to cycles[2b] and its ticks of the constant 100 MHz counter
 * to cycles[2b + 1] (`cycles`: device memory, 2 * blocks uint64, owned by the caller). Clock in
 * MHz = 100 * sum(cycles[2b]) / sum(cycles[2b + 1]). Asynchronous on `stream`.
 * MOE_EINVAL if cycles is NULL, blocks is outside 1..65536 or iters < 1. */
moe_status_t moe_mxfp4_clock_probe(uint64_t *cycles, int blocks, int iters, void *stream);

/* Message describing the last error on this thread ("" if none). Never NULL. */
const char *moe_mxfp4_last_error(void);

/* Host-only validation of a shape; launches nothing. */
moe_status_t moe_mxfp4_check_shape(const moe_mxfp4_shape_t *shape);

/* Bytes of device workspace moe_mxfp4_forward and moe_mxfp4_forward_prenorm need for
 * `shape` (written to *bytes). Host-only; launches nothing. */
moe_status_t moe_mxfp4_workspace_bytes(const moe_mxfp4_shape_t *shape, size_t *bytes);

/*
 * The whole layer, steps 1-6 above.
 *  x          [T, H]        bf16
 *  router_w   [E, H]        bf16      router_b [E] bf16
 *  gu_blocks  [E, 2I, H/2]  uint8     gu_scales [E, 2I, H/32] uint8   gu_bias [E, 2I] bf16
 *  dn_blocks  [E, H, I/2]   uint8     dn_scales [E, H, I/32]  uint8   dn_bias [E, H]  bf16
 *  y          [T, H]        bf16 (out)
 *  topk_idx   [T, k] int32  (out, or NULL)   selected experts in selection order
 *  topk_w     [T, k] fp32   (out, or NULL)   their softmax weights
 *  workspace  device scratch of at least moe_mxfp4_workspace_bytes() bytes, 256-byte
 *             aligned; its contents on entry are ignored.
 */
moe_status_t moe_mxfp4_forward(const moe_mxfp4_shape_t *shape,
                               const moe_bf16_t *x,
                               const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                               const uint8_t *gu_blocks, const uint8_t *gu_scales,
                               const moe_bf16_t *gu_bias,
                               const uint8_t *dn_blocks, const uint8_t *dn_scales,
                               const moe_bf16_t *dn_bias,
                               moe_bf16_t *y, int32_t *topk_idx, float *topk_w,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * The pre-norm block around the layer (GPT-OSS MLX Implementation README, "Architecture
 * Details": RMSNorm in Pre-LN placement; ZeroModels GPT-OSS page, "API" table: norm_eps,
 * 1e-5 for GPT-OSS):
 *   xn[t, :] = bf16(x[t, :] * norm_w / sqrt(mean_h x[t, h]^2 + norm_eps))
 *   y[t, :]  = bf16(x[t, :] + layer(xn)[t, :])
 * The normalization runs in double and rounds once to bf16 (nearest, ties to even), as
 * moe_mxfp4_rmsnorm; the layer (steps 1-6) then runs on xn, and its last kernel adds the
 * residual x before the one bf16 rounding of y. On the few-token path (T <= 64, H and I <= 4096;
 * H <= 3584 from 4 tokens) the router kernel normalizes the rows it loads, so the block takes
 * as many kernels as the plain layer; otherwise one more kernel writes xn to the workspace
 * first. Arguments as moe_mxfp4_forward, plus
 *  norm_w    [H] bf16, 16-byte aligned (RMSNorm scale; MOE_EINVAL if NULL, MOE_EALIGN if
 *            misaligned)
 *  norm_eps  finite and >= 0 (MOE_EINVAL otherwise)
 * topk_idx / topk_w are the routing of xn. The workspace size is moe_mxfp4_workspace_bytes().
 */
moe_status_t moe_mxfp4_forward_prenorm(const moe_mxfp4_shape_t *shape,
                                       const moe_bf16_t *x,
                                       const moe_bf16_t *norm_w, double norm_eps,
                                       const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                       const uint8_t *gu_blocks, const uint8_t *gu_scales,
                                       const moe_bf16_t *gu_bias,
                                       const uint8_t *dn_blocks, const uint8_t *dn_scales,
                                       const moe_bf16_t *dn_bias,
                                       moe_bf16_t *y, int32_t *topk_idx, float *topk_w,
                                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_mxfp4_forward without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The workspace is a static device array of the library: one copy of
 * moe_mxfp4_noalloc_max_bytes() = 64 MiB per GPU the library runs on, allocated when the
 * library's code object is loaded on that GPU and held until the process ends. The call
 * itself allocates and frees nothing. Every call on one GPU uses that GPU's copy, so calls
 * that overlap on one GPU (on different streams, or from different threads without ordering)
 * race and give undefined results; calls ordered on one stream are safe. Shapes whose
 * moe_mxfp4_workspace_bytes() exceeds the array return MOE_EWORKSPACE (at the GPT-OSS-20B
 * shape: up to 820 tokens, which covers every decode batch). The GPU is the
 * stream's (the current device for the NULL stream). Arguments, results and every other error
 * as moe_mxfp4_forward (same kernels, bit-identical results).
 */
moe_status_t moe_mxfp4_forward_noalloc(const moe_mxfp4_shape_t *shape,
                                       const moe_bf16_t *x,
                                       const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                       const uint8_t *gu_blocks, const uint8_t *gu_scales,
                                       const moe_bf16_t *gu_bias,
                                       const uint8_t *dn_blocks, const uint8_t *dn_scales,
                                       const moe_bf16_t *dn_bias,
                                       moe_bf16_t *y, int32_t *topk_idx, float *topk_w, void *stream);

/* Bytes of the per-GPU static workspace of moe_mxfp4_forward_noalloc. Host-only. */
size_t moe_mxfp4_noalloc_max_bytes(void);

/* Most kernels one moe_mxfp4_forward or moe_mxfp4_forward_prenorm call launches. */
#define MOE_MXFP4_MAX_LAUNCHES 6

/*
 * moe_mxfp4_forward with timing instrumentation for profilers and benchmarks: the same
 * validation, kernels and results, with every kernel launched through hipExtLaunchKernel so
 * that it records two events at the start and at the end of its own execution. `events`
 * holds at least 2 * MOE_MXFP4_MAX_LAUNCHES hipEvent_t handles created by the caller
 * (timing enabled); stage i records events[2i] and events[2i + 1], so that
 * hipEventElapsedTime(events[2i], events[2i + 1]) is that stage's duration. Every stage is one
 * kernel except the permute stage of the grouped sequence (T > 64, or a larger H or I at any T):
 * a histogram pass, above 16384 pairs (64 blocks of 256) a scan pass, and a scatter pass; the
 * first records the start event, the last the end event.
 * *n_launches receives the number of stages. With H <= 4096 and I <= 4096: 3 for
 * T <= 3 (router logits, up-projection with the top-k, down-projection with the combine
 * folded in), 4 for 4 <= T <= 64 (route, up-projection, down-projection, combine); 5 for
 * T > 64 or a larger H or I (route, permute, up-projection, down-projection, combine). MOE_EINVAL if events, an
 * events[i] or n_launches is NULL, or n_events is too small.
 */
moe_status_t moe_mxfp4_forward_timed(const moe_mxfp4_shape_t *shape,
                                     const moe_bf16_t *x,
                                     const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                     const uint8_t *gu_blocks, const uint8_t *gu_scales,
                                     const moe_bf16_t *gu_bias,
                                     const uint8_t *dn_blocks, const uint8_t *dn_scales,
                                     const moe_bf16_t *dn_bias,
                                     moe_bf16_t *y, int32_t *topk_idx, float *topk_w,
                                     void *workspace, size_t workspace_bytes, void *stream,
                                     void *const *events, int n_events, int *n_launches);

/* moe_mxfp4_forward_prenorm with the instrumentation of moe_mxfp4_forward_timed. Launch
 * counts as there, plus the RMSNorm kernel (launch 0) where the router does not normalize. */
moe_status_t moe_mxfp4_forward_prenorm_timed(const moe_mxfp4_shape_t *shape,
                                             const moe_bf16_t *x,
                                             const moe_bf16_t *norm_w, double norm_eps,
                                             const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                             const uint8_t *gu_blocks, const uint8_t *gu_scales,
                                             const moe_bf16_t *gu_bias,
                                             const uint8_t *dn_blocks, const uint8_t *dn_scales,
                                             const moe_bf16_t *dn_bias,
                                             moe_bf16_t *y, int32_t *topk_idx, float *topk_w,
                                             void *workspace, size_t workspace_bytes, void *stream,
                                             void *const *events, int n_events, int *n_launches);

/*
 * The RMSNorm of the pre-norm block alone (GPT-OSS MLX Implementation README, "Architecture
 * Details"): xn[r, :] = bf16(x[r, :] * r_r * norm_w), r_r = 1 / sqrt(sum_c x[r, c]^2 / cols
 * + eps), computed in double (the squares of bf16 values are exact; products left to right)
 * and rounded once to bf16, nearest, ties to even. x, xn [rows, cols] bf16 and norm_w [cols]
 * bf16, all 16-byte aligned (MOE_EALIGN); cols a positive multiple of 8 (MOE_ESHAPE);
 * 0 <= rows <= 2^24; eps finite and >= 0 (MOE_EINVAL). The sum of squares is accumulated in
 * a fixed order (per thread, then across threads); its rounding differs from a sequential
 * sum only in the last bits of a double.
 */
moe_status_t moe_mxfp4_rmsnorm(const moe_bf16_t *x, const moe_bf16_t *norm_w, int64_t rows,
                               int32_t cols, double eps, moe_bf16_t *xn, void *stream);

/*
 * Steps 1-2 only (router, top-k, softmax). Logits are accumulated in double precision
 * from the exact bf16 products, so the selection agrees with exact arithmetic except for
 * logits closer than ~1e-12 relative. Outputs: topk_idx [T, k] int32, topk_w [T, k] fp32
 * (both required), logits [T, E] fp32 (optional, NULL to skip; the double logits
 * rounded to fp32). Only shape->T, H, E, k are used.
 */
moe_status_t moe_mxfp4_route(const moe_mxfp4_shape_t *shape,
                             const moe_bf16_t *x,
                             const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                             int32_t *topk_idx, float *topk_w, float *logits,
                             void *stream);

/*
 * Expert-sorted permutation of the routed (token, slot) pairs, the grouping the grouped
 * GEMMs consume. From topk_idx / topk_w [T, k]:
 *  expert_offsets [E + 1] int32: rows of expert e are [offsets[e], offsets[e+1]).
 *  sorted_token   [T*k]   int32: token of each sorted row; rows of one expert are in
 *                                increasing (token, slot) order (a stable sort).
 *  sorted_weight  [T*k]   fp32 : routing weight of each sorted row.
 *  slot_row       [T*k]   int32: sorted row of pair (t, j), at index t*k + j.
 * Only shape->T, E, k are used. topk_idx entries must lie in [0, E).
 */
moe_status_t moe_mxfp4_permute(const moe_mxfp4_shape_t *shape,
                               const int32_t *topk_idx, const float *topk_w,
                               int32_t *expert_offsets, int32_t *sorted_token,
                               float *sorted_weight, int32_t *slot_row, void *stream);

/*
 * The same permutation on many workgroups: a histogram pass (one workgroup per 256 pairs
 * writes how many of its pairs each expert received), then a scatter pass (each workgroup
 * ranks its own pairs after those of the workgroups before it). Up to 16384 pairs each
 * scatter workgroup sums the earlier histograms itself; above that a scan pass (one workgroup
 * per expert) first turns them into prefix sums, so the work stays linear in T*k. This is the
 * permute every forward call of the grouped sequence runs; the results are identical to
 * moe_mxfp4_permute's, bit for bit. The histograms need moe_mxfp4_permute_workspace_bytes()
 * bytes of device workspace (4-byte aligned; its contents on entry do not matter).
 * MOE_EWORKSPACE if the workspace is NULL or short while T*k > 0; other arguments as
 * moe_mxfp4_permute.
 */
moe_status_t moe_mxfp4_permute_ws(const moe_mxfp4_shape_t *shape,
                                  const int32_t *topk_idx, const float *topk_w,
                                  int32_t *expert_offsets, int32_t *sorted_token,
                                  float *sorted_weight, int32_t *slot_row,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace moe_mxfp4_permute_ws needs: (T*k/256 rounded up, plus 1) times E times
 * 4 bytes (one histogram row per workgroup and the per-expert totals); 0 for T*k = 0. Only
 * shape->T, E, k are used. Host-only. */
moe_status_t moe_mxfp4_permute_workspace_bytes(const moe_mxfp4_shape_t *shape, size_t *bytes);

/*
 * mx8 activation matrix: the expert GEMMs' activation format. gfx950's block-scaled MFMA
 * takes the packed MXFP4 weight blocks as stored (OCP Microscaling Formats v1.0, which the
 * ZeroModels GPT-OSS page's "MXFP4 experts" item refers to: 32-element blocks with one E8M0
 * scale) against OCP E4M3 activations carrying their own E8M0 block scales. An activation
 * row of K values becomes two rows of K bytes: for each 32-element block with largest
 * magnitude m, eb = floor(log2 m) - 7 (0 for an all-zero block), hi = E4M3(x / 2^eb)
 * rounded to nearest even, lo = E4M3(16 * (x / 2^eb - hi)), with scales 127 + eb (hi) and
 * 123 + eb (lo); x = hi * 2^eb + lo * 2^(eb-4), exactly for bf16 x unless lo falls below
 * E4M3's normal range (elements more than about 2^13 below their block's largest).
 * Layout for R rows of K values (K a multiple of 32): 2R rows of K bytes (row 2r = hi,
 * row 2r+1 = lo of row r), then 2R rows of S = roundup(K/32, 16) scale bytes (row-major;
 * bytes past K/32 in a row are unused). Total moe_mxfp4_mx8_bytes(R, K) = 2R (K + S).
 */
size_t moe_mxfp4_mx8_bytes(int64_t rows, int32_t cols);

/*
 * bf16 [rows, cols] -> mx8 (layout above). q8 needs moe_mxfp4_mx8_bytes(rows, cols)
 * bytes, 16-byte aligned. cols must be a positive multiple of 32; rows >= 0.
 */
moe_status_t moe_mxfp4_quantize_act(const moe_bf16_t *x, int64_t rows, int32_t cols,
                                    uint8_t *q8, void *stream);

/*
 * h8 matrix: the format of the expert intermediate h between moe_mxfp4_expert_up and
 * moe_mxfp4_expert_down (step 4's output, step 5's input; ZeroModels GPT-OSS page,
 * "Mixture-of-experts feed-forward"). The same 2R data rows of K bytes and the same hi/lo
 * values and scales as an mx8 matrix, with the scales grouped by sixteen blocks instead of
 * by row: after the data rows come ceil(K/512) groups of R 16-byte words; byte b % 16 of
 * word r of group b / 16 is the hi scale (127 + eb) of row r's block b. Lo scales are not
 * stored (always the hi scale minus 4); bytes for blocks past K/32 are unused. The down GEMM
 * then reads the scales of 128 consecutive rows for four 128-element steps as 2 KB of
 * contiguous bytes. Size: 2RK + 16R ceil(K/512) bytes, less than moe_mxfp4_mx8_bytes(R, K),
 * which callers allocate.
 */

/*
 * bf16 [rows, cols] -> h8 (layout above): the input moe_mxfp4_expert_down takes, for an h
 * computed elsewhere. h8 needs moe_mxfp4_mx8_bytes(rows, cols) bytes, 16-byte aligned; cols a
 * positive multiple of 32; rows >= 0. Errors as moe_mxfp4_quantize_act.
 */
moe_status_t moe_mxfp4_quantize_h(const moe_bf16_t *h, int64_t rows, int32_t cols,
                                  uint8_t *h8, void *stream);

/*
 * Steps 3-4 over the sorted rows (grouped gate_up GEMM on the block-scaled MFMA, bias,
 * clamped SwiGLU): h[r, :] = swiglu(x[sorted_token[r]] . Wgu[e]^T + bgu[e]) for every row r
 * of expert e. x8: x as an mx8 matrix of T rows of H (from moe_mxfp4_quantize_act);
 * h8 (out): h as an h8 matrix (group-major scales, layout above) of T*k rows of I
 * (moe_mxfp4_mx8_bytes(T*k, I) bytes), rows in sorted order. expert_offsets / sorted_token as produced by moe_mxfp4_permute.
 */
moe_status_t moe_mxfp4_expert_up(const moe_mxfp4_shape_t *shape,
                                 const uint8_t *x8,
                                 const uint8_t *gu_blocks, const uint8_t *gu_scales,
                                 const moe_bf16_t *gu_bias,
                                 const int32_t *expert_offsets, const int32_t *sorted_token,
                                 uint8_t *h8, void *stream);

/*
 * Step 5 over the sorted rows (grouped down GEMM on the block-scaled MFMA, bias), scaled
 * by the row's routing weight: o[r, :] = sorted_weight[r] * (h[r] . Wdn[e]^T + bdn[e]).
 * h8: an h8 matrix of T*k rows of I (from moe_mxfp4_expert_up or moe_mxfp4_quantize_h);
 * o [T*k, H] fp32 (out).
 */
moe_status_t moe_mxfp4_expert_down(const moe_mxfp4_shape_t *shape,
                                   const uint8_t *h8,
                                   const uint8_t *dn_blocks, const uint8_t *dn_scales,
                                   const moe_bf16_t *dn_bias,
                                   const int32_t *expert_offsets, const float *sorted_weight,
                                   float *o, void *stream);

/*
 * Step 6 (un-permute and weighted sum; the weights are already applied in o):
 * y[t, :] = sum_{j = 0..k-1} o[slot_row[t*k + j], :], summed in slot order, rounded to bf16.
 */
moe_status_t moe_mxfp4_combine(const moe_mxfp4_shape_t *shape,
                               const float *o, const int32_t *slot_row,
                               moe_bf16_t *y, void *stream);

/*
 * The layer on an expert bank dequantized once to bf16 (ZeroModels GPT-OSS page, "MXFP4
 * experts": longer prefills dequantize the whole bank once instead of on the fly, with results
 * identical to the routed-only path; "Mixture-of-experts feed-forward" for steps 1-6). The
 * caller expands the packed bank once with moe_mxfp4_dequant (rows = E * 2I, cols = H for
 * gate_up; rows = E * H, cols = I for down) and passes the bf16 tensors:
 *  gu_w [E, 2I, H] bf16 (rows interleaved gate/up as in the packed layout), dn_w [E, H, I] bf16;
 *  every other argument as moe_mxfp4_forward.
 * Steps 1-3 and 6 run the same kernels as the packed path at T > 64 (router, permutation,
 * combine); steps 4-5 run grouped GEMMs on the bf16 MFMA with bf16 activations, h stored as
 * bf16 [T k, I] in the workspace. 5 launches at any T. The workspace size is
 * moe_mxfp4_workspace_bytes_dequantized(); gu_w, dn_w 16-byte aligned (MOE_EALIGN).
 * This is the pages' dequantize-once variant, kept to measure it against the packed path,
 * which never expands the weights.
 */
moe_status_t moe_mxfp4_forward_dequantized(const moe_mxfp4_shape_t *shape,
                                           const moe_bf16_t *x,
                                           const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                           const moe_bf16_t *gu_w, const moe_bf16_t *gu_bias,
                                           const moe_bf16_t *dn_w, const moe_bf16_t *dn_bias,
                                           moe_bf16_t *y, int32_t *topk_idx, float *topk_w,
                                           void *workspace, size_t workspace_bytes, void *stream);

/* moe_mxfp4_forward_dequantized with the instrumentation of moe_mxfp4_forward_timed
 * (route, permute, up-projection, down-projection, combine). */
moe_status_t moe_mxfp4_forward_dequantized_timed(const moe_mxfp4_shape_t *shape,
                                                 const moe_bf16_t *x,
                                                 const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                                 const moe_bf16_t *gu_w, const moe_bf16_t *gu_bias,
                                                 const moe_bf16_t *dn_w, const moe_bf16_t *dn_bias,
                                                 moe_bf16_t *y, int32_t *topk_idx, float *topk_w,
                                                 void *workspace, size_t workspace_bytes, void *stream,
                                                 void *const *events, int n_events, int *n_launches);

/* Bytes of device workspace moe_mxfp4_forward_dequantized needs for `shape`. Host-only. */
moe_status_t moe_mxfp4_workspace_bytes_dequantized(const moe_mxfp4_shape_t *shape, size_t *bytes);

/*
 * Standalone MXFP4 -> bf16 dequantization of a packed [rows, cols] matrix
 * (ZeroModels GPT-OSS page, "MXFP4 experts"): out[r, c] = e2m1(nibble) * 2^(scale - 127),
 * exact for scale bytes 2..252. blocks [rows, cols/2], scales [rows, cols/32],
 * out [rows, cols] bf16. cols must be a positive multiple of 32; rows >= 0.
 */
moe_status_t moe_mxfp4_dequant(const uint8_t *blocks, const uint8_t *scales,
                               int64_t rows, int32_t cols, moe_bf16_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
