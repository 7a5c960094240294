// C ABI of the MXFP4 mixture-of-experts layer: host-side validation, workspace layout
// and the launch sequence. No allocation, no synchronisation, no state between calls.
#include "moe_mxfp4.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.h"
#include "mx_mfma.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

moe_status_t ok() {
    g_last_error.clear();
    return MOE_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status_t check_shape(const moe_mxfp4_shape_t *s, bool need_experts) {
    if (!s) return fail(MOE_EINVAL, "shape is NULL");
    if (s->T < 0) return fail(MOE_EINVAL, "T = %lld is negative", static_cast<long long>(s->T));
    if (s->H <= 0 || s->H % 32) return fail(MOE_ESHAPE, "H = %d is not a positive multiple of 32", s->H);
    if (need_experts && (s->I <= 0 || s->I % 32))
        return fail(MOE_ESHAPE, "I = %d is not a positive multiple of 32", s->I);
    if (s->E < 1 || s->E > 256) return fail(MOE_ESHAPE, "E = %d outside 1..256", s->E);
    if (s->k < 1 || s->k > 8 || s->k > s->E)
        return fail(MOE_ESHAPE, "k = %d outside 1..min(E, 8) (E = %d)", s->k, s->E);
    if (s->T > (static_cast<int64_t>(1) << 24))
        return fail(MOE_ESHAPE, "T = %lld exceeds the supported 2^24 tokens per call",
                    static_cast<long long>(s->T));
    if (need_experts) {
        // the grouped GEMMs address their operands with 32-bit offsets
        const int K = s->H > s->I ? s->H : s->I;
        const uint64_t act = moe::mx8_bytes(s->T * s->k, K);
        const uint64_t wgt = static_cast<uint64_t>(2 * s->I) * (s->H / 2);
        if (act >= (static_cast<uint64_t>(1) << 32) || wgt >= (static_cast<uint64_t>(1) << 32))
            return fail(MOE_ESHAPE, "T * k = %lld rows of %d (or one expert's weights) exceed 4 GiB; split the batch",
                        static_cast<long long>(s->T * s->k), K);
    }
    if (need_experts && (!std::isfinite(s->swiglu_alpha) || !std::isfinite(s->swiglu_limit)))
        return fail(MOE_EINVAL, "swiglu_alpha / swiglu_limit must be finite");
    return MOE_OK;
}

moe::Dims dims_of(const moe_mxfp4_shape_t *s) {
    return moe::Dims{s->T, s->H, s->I, s->E, s->k, s->swiglu_alpha, s->swiglu_limit};
}

// Workspace regions (each 256-byte aligned), in order.
struct Layout {
    size_t idx, w, logits, offsets, sorted_token, sorted_w, slot_row, o, part, x8, h8, xn, hist, rpart, total;
};

size_t round_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

Layout layout_of(const moe_mxfp4_shape_t *s) {
    const size_t N = static_cast<size_t>(s->T) * s->k;
    Layout L{};
    size_t p = 0;
    L.idx = p;          p += round_up(N * 4);
    L.w = p;            p += round_up(N * 4);
    // the normalized input of the pre-norm entry points (bf16 [T, H])
    L.xn = p;           p += round_up(static_cast<size_t>(s->T) * s->H * 2);
    L.logits = 0;
    if (moe::use_decode_path(s->T, s->H, s->I)) {
        // activations as E4M3 hi/lo (mx8) matrices: x as T rows of H, h as 2 T k half-block
        // rows of I
        L.x8 = p;       p += round_up(moe::mx8_bytes(s->T, s->H));
        L.h8 = p;       p += round_up(moe::mx8_bytes(2 * static_cast<int64_t>(N), s->I));
        L.part = p;
        if (s->T >= moe::kStreamMinT) p += round_up(N * static_cast<size_t>(s->H) * 4);
        L.logits = p;   p += round_up(static_cast<size_t>(s->T) * s->E * 8);
        L.offsets = L.sorted_token = L.sorted_w = L.slot_row = L.o = L.hist = 0;
    } else {
        L.offsets = p;      p += round_up((static_cast<size_t>(s->E) + 1) * 4);
        L.sorted_token = p; p += round_up(N * 4);
        L.sorted_w = p;     p += round_up(N * 4);
        L.slot_row = p;     p += round_up(N * 4);
        L.hist = p;         p += round_up(static_cast<size_t>(moe::permute_hist_ints(N, s->E)) * 4);
        L.x8 = p;           p += round_up(moe::mx8_bytes(s->T, s->H));
        L.h8 = p;           p += round_up(moe::mx8_bytes(static_cast<int64_t>(N), s->I));
        L.o = p;            p += round_up(N * static_cast<size_t>(s->H) * 4);
        // the router's partial logits over slices of H (few token groups, many experts)
        L.rpart = p;        p += round_up(static_cast<size_t>(moe::route_part_doubles(dims_of(s))) * 8);
        L.part = 0;
    }
    L.total = p;
    return L;
}

// Workspace of the dequantized-bank forward (256-byte aligned regions, in order).
struct BankLayout {
    size_t idx, w, offsets, sorted_token, sorted_w, slot_row, hist, h, o, total;
};

BankLayout bank_layout_of(const moe_mxfp4_shape_t *s) {
    const size_t N = static_cast<size_t>(s->T) * s->k;
    BankLayout L{};
    size_t p = 0;
    L.idx = p;          p += round_up(N * 4);
    L.w = p;            p += round_up(N * 4);
    L.offsets = p;      p += round_up((static_cast<size_t>(s->E) + 1) * 4);
    L.sorted_token = p; p += round_up(N * 4);
    L.sorted_w = p;     p += round_up(N * 4);
    L.slot_row = p;     p += round_up(N * 4);
    L.hist = p;         p += round_up(static_cast<size_t>(moe::permute_hist_ints(N, s->E)) * 4);
    L.h = p;            p += round_up(N * static_cast<size_t>(s->I) * 2);
    L.o = p;            p += round_up(N * static_cast<size_t>(s->H) * 4);
    L.total = p;
    return L;
}

moe_status_t hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

#define REQUIRE(ptr, name)                                                            \
    do {                                                                              \
        if (!(ptr)) return fail(MOE_EINVAL, "%s is NULL", name);                      \
    } while (0)
#define REQUIRE16(ptr, name)                                                          \
    do {                                                                              \
        if (!(ptr)) return fail(MOE_EINVAL, "%s is NULL", name);                      \
        if (!aligned16(ptr)) return fail(MOE_EALIGN, "%s is not 16-byte aligned", name); \
    } while (0)
#define REQUIRE4(ptr, name)                                                           \
    do {                                                                              \
        if (!(ptr)) return fail(MOE_EINVAL, "%s is NULL", name);                      \
        if (reinterpret_cast<uintptr_t>(ptr) & 3u)                                     \
            return fail(MOE_EALIGN, "%s is not 4-byte aligned", name);                \
    } while (0)
#define LAUNCH(call, what)                                                            \
    do {                                                                              \
        moe_status_t st_ = hip_status((call), what);                                  \
        if (st_ != MOE_OK) return st_;                                                \
    } while (0)

}  // namespace

MOE_EXPORT int moe_mxfp4_abi_version(void) { return MOE_MXFP4_ABI_VERSION; }

MOE_EXPORT moe_status_t moe_mxfp4_clock_probe(uint64_t *cycles, int blocks, int iters, void *stream) {
    REQUIRE(cycles, "cycles");
    if (blocks < 1 || blocks > 65536) return fail(MOE_EINVAL, "blocks = %d outside 1..65536", blocks);
    if (iters < 1) return fail(MOE_EINVAL, "iters = %d is not positive", iters);
    LAUNCH(moe::launch_clock_probe(cycles, blocks, iters, static_cast<hipStream_t>(stream)), "clock probe");
    return ok();
}

MOE_EXPORT const char *moe_mxfp4_last_error(void) { return g_last_error.c_str(); }

MOE_EXPORT moe_status_t moe_mxfp4_check_shape(const moe_mxfp4_shape_t *shape) {
    moe_status_t st = check_shape(shape, true);
    return st != MOE_OK ? st : ok();
}

MOE_EXPORT moe_status_t moe_mxfp4_workspace_bytes(const moe_mxfp4_shape_t *shape, size_t *bytes) {
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    REQUIRE(bytes, "bytes");
    *bytes = layout_of(shape).total;
    return ok();
}

namespace {

// Validation + launch sequence shared by moe_mxfp4_forward and moe_mxfp4_forward_timed.
// With `events`, launch i records events[2i] and events[2i + 1] at the start and the end of
// its kernel's execution (hipExtLaunchKernel).
// With norm_w, the pre-norm block y = x + layer(rmsnorm(x)): the normalized rows go to the
// workspace, the layer runs on them and its last kernel adds x.
moe_status_t run_forward(const moe_mxfp4_shape_t *shape, const moe_bf16_t *x,
                         const moe_bf16_t *norm_w, double norm_eps, const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                         const uint8_t *gu_blocks, const uint8_t *gu_scales,
                         const moe_bf16_t *gu_bias, const uint8_t *dn_blocks,
                         const uint8_t *dn_scales, const moe_bf16_t *dn_bias, moe_bf16_t *y,
                         int32_t *topk_idx, float *topk_w, void *workspace, size_t workspace_bytes,
                         void *stream, void *const *events, int n_events, int *n_launches) {
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (events) {
        if (n_events < 2 * MOE_MXFP4_MAX_LAUNCHES)
            return fail(MOE_EINVAL, "n_events = %d, at least %d needed", n_events,
                        2 * MOE_MXFP4_MAX_LAUNCHES);
        for (int i = 0; i < 2 * MOE_MXFP4_MAX_LAUNCHES; ++i)
            if (!events[i]) return fail(MOE_EINVAL, "events[%d] is NULL", i);
        REQUIRE(n_launches, "n_launches");
        *n_launches = 0;
    }
    if (shape->T == 0) return ok();
    REQUIRE16(x, "x");
    if (norm_w) {
        if (!aligned16(norm_w)) return fail(MOE_EALIGN, "norm_w is not 16-byte aligned");
        if (!std::isfinite(norm_eps) || norm_eps < 0.0)
            return fail(MOE_EINVAL, "norm_eps = %g must be finite and >= 0", norm_eps);
    }
    REQUIRE16(router_w, "router_w");
    REQUIRE(router_b, "router_b");
    REQUIRE16(gu_blocks, "gu_blocks");
    REQUIRE4(gu_scales, "gu_scales");
    REQUIRE(gu_bias, "gu_bias");
    REQUIRE16(dn_blocks, "dn_blocks");
    REQUIRE4(dn_scales, "dn_scales");
    REQUIRE(dn_bias, "dn_bias");
    REQUIRE16(y, "y");
    const Layout L = layout_of(shape);
    if (!workspace) return fail(MOE_EWORKSPACE, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(MOE_EALIGN, "workspace is not 256-byte aligned");
    if (workspace_bytes < L.total)
        return fail(MOE_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);

    const moe::Dims d = dims_of(shape);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    int32_t *idx = topk_idx ? topk_idx : reinterpret_cast<int32_t *>(ws + L.idx);
    float *w = topk_w ? topk_w : reinterpret_cast<float *>(ws + L.w);
    int launched = 0;
    // the event pair of the next launch (cleared again however this function returns)
    struct EventGuard {
        ~EventGuard() { moe::launch_events() = moe::LaunchEvents{}; }
    } guard;
    auto arm = [&]() {
        if (events)
            moe::launch_events() = moe::LaunchEvents{static_cast<hipEvent_t>(events[2 * launched]),
                                                     static_cast<hipEvent_t>(events[2 * launched + 1])};
    };
#define STEP(call, what)                                 \
    do {                                                 \
        arm();                                           \
        LAUNCH(call, what);                              \
        ++launched;                                      \
        if (n_launches) *n_launches = launched;          \
    } while (0)

    // pre-norm block: the decode routers normalize the token rows they load; otherwise a
    // kernel of its own writes them to the workspace
    const moe_bf16_t *residual = norm_w ? x : nullptr;
    const moe_bf16_t *gamma = nullptr;
    if (norm_w) {
        const bool fused = moe::use_decode_path(shape->T, shape->H, shape->I) &&
                           (shape->T < moe::kStreamMinT || moe::route_normalizes(d));
        if (fused) {
            gamma = norm_w;
        } else {
            moe_bf16_t *xn = reinterpret_cast<moe_bf16_t *>(ws + L.xn);
            STEP(moe::launch_rmsnorm(d, x, norm_w, norm_eps, xn, s), "rmsnorm");
            x = xn;
        }
    }

    if (moe::use_decode_path(shape->T, shape->H, shape->I)) {
        float *part = reinterpret_cast<float *>(ws + L.part);
        uint8_t *x8 = ws + L.x8, *h8 = ws + L.h8;
        if (shape->T >= moe::kStreamMinT) {
            STEP(moe::launch_route(d, x, gamma, norm_eps, router_w, router_b, idx, w, nullptr, x8, s), "route");
            STEP(moe::launch_up_stream(d, x8, gu_blocks, gu_scales, gu_bias, idx, h8, s), "up (stream)");
            STEP(moe::launch_down_stream(d, h8, dn_blocks, dn_scales, dn_bias, idx, w, part, s), "down (stream)");
            STEP(moe::launch_combine_decode(d, part, residual, y, s), "combine (decode)");
            return ok();
        }
        // few tokens: logits in a multi-block kernel, top-k + softmax inside the up-projection
        double *logits = reinterpret_cast<double *>(ws + L.logits);
        STEP(moe::launch_logits(d, x, gamma, norm_eps, router_w, router_b, logits, x8, s), "router logits");
        STEP(moe::launch_up_decode(d, x8, gu_blocks, gu_scales, gu_bias, logits, idx, w, h8, s), "up (decode)");
        STEP(moe::launch_down_decode(d, h8, dn_blocks, dn_scales, dn_bias, idx, w, residual, y, s), "down (decode)");
        return ok();
    }
    uint8_t *x8 = ws + L.x8, *h8 = ws + L.h8;
    STEP(moe::launch_route(d, x, nullptr, 0.0, router_w, router_b, idx, w, nullptr, x8, s,
                           reinterpret_cast<double *>(ws + L.rpart)), "route");
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    int32_t *sorted_token = reinterpret_cast<int32_t *>(ws + L.sorted_token);
    float *sorted_w = reinterpret_cast<float *>(ws + L.sorted_w);
    int32_t *slot_row = reinterpret_cast<int32_t *>(ws + L.slot_row);
    float *o = reinterpret_cast<float *>(ws + L.o);
    STEP(moe::launch_permute(d, idx, w, offsets, sorted_token, sorted_w, slot_row, s,
                             reinterpret_cast<int32_t *>(ws + L.hist)), "permute");
    STEP(moe::launch_up_grouped(d, x8, gu_blocks, gu_scales, gu_bias, offsets, sorted_token, h8, s), "up");
    STEP(moe::launch_down_grouped(d, h8, dn_blocks, dn_scales, dn_bias, offsets, sorted_w, o, s), "down");
    STEP(moe::launch_combine(d, o, slot_row, residual, y, s), "combine");
#undef STEP
    return ok();
}

}  // namespace

MOE_EXPORT moe_status_t moe_mxfp4_forward(const moe_mxfp4_shape_t *shape, const moe_bf16_t *x,
                                          const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                          const uint8_t *gu_blocks, const uint8_t *gu_scales,
                                          const moe_bf16_t *gu_bias, const uint8_t *dn_blocks,
                                          const uint8_t *dn_scales, const moe_bf16_t *dn_bias,
                                          moe_bf16_t *y, int32_t *topk_idx, float *topk_w,
                                          void *workspace, size_t workspace_bytes, void *stream) {
    return run_forward(shape, x, nullptr, 0.0, router_w, router_b, gu_blocks, gu_scales, gu_bias, dn_blocks,
                       dn_scales, dn_bias, y, topk_idx, topk_w, workspace, workspace_bytes, stream,
                       nullptr, 0, nullptr);
}

MOE_EXPORT moe_status_t moe_mxfp4_forward_prenorm(
    const moe_mxfp4_shape_t *shape, const moe_bf16_t *x, const moe_bf16_t *norm_w, double norm_eps,
    const moe_bf16_t *router_w, const moe_bf16_t *router_b, const uint8_t *gu_blocks,
    const uint8_t *gu_scales, const moe_bf16_t *gu_bias, const uint8_t *dn_blocks,
    const uint8_t *dn_scales, const moe_bf16_t *dn_bias, moe_bf16_t *y, int32_t *topk_idx,
    float *topk_w, void *workspace, size_t workspace_bytes, void *stream) {
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (shape->T > 0) REQUIRE(norm_w, "norm_w");
    return run_forward(shape, x, norm_w, norm_eps, router_w, router_b, gu_blocks, gu_scales, gu_bias,
                       dn_blocks, dn_scales, dn_bias, y, topk_idx, topk_w, workspace, workspace_bytes,
                       stream, nullptr, 0, nullptr);
}

MOE_EXPORT moe_status_t moe_mxfp4_forward_prenorm_timed(
    const moe_mxfp4_shape_t *shape, const moe_bf16_t *x, const moe_bf16_t *norm_w, double norm_eps,
    const moe_bf16_t *router_w, const moe_bf16_t *router_b, const uint8_t *gu_blocks,
    const uint8_t *gu_scales, const moe_bf16_t *gu_bias, const uint8_t *dn_blocks,
    const uint8_t *dn_scales, const moe_bf16_t *dn_bias, moe_bf16_t *y, int32_t *topk_idx,
    float *topk_w, void *workspace, size_t workspace_bytes, void *stream, void *const *events,
    int n_events, int *n_launches) {
    if (!events) return fail(MOE_EINVAL, "events is NULL");
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (shape->T > 0) REQUIRE(norm_w, "norm_w");
    return run_forward(shape, x, norm_w, norm_eps, router_w, router_b, gu_blocks, gu_scales, gu_bias,
                       dn_blocks, dn_scales, dn_bias, y, topk_idx, topk_w, workspace, workspace_bytes,
                       stream, events, n_events, n_launches);
}

MOE_EXPORT moe_status_t moe_mxfp4_forward_timed(
    const moe_mxfp4_shape_t *shape, const moe_bf16_t *x, const moe_bf16_t *router_w,
    const moe_bf16_t *router_b, const uint8_t *gu_blocks, const uint8_t *gu_scales,
    const moe_bf16_t *gu_bias, const uint8_t *dn_blocks, const uint8_t *dn_scales,
    const moe_bf16_t *dn_bias, moe_bf16_t *y, int32_t *topk_idx, float *topk_w, void *workspace,
    size_t workspace_bytes, void *stream, void *const *events, int n_events, int *n_launches) {
    if (!events) return fail(MOE_EINVAL, "events is NULL");
    return run_forward(shape, x, nullptr, 0.0, router_w, router_b, gu_blocks, gu_scales, gu_bias, dn_blocks,
                       dn_scales, dn_bias, y, topk_idx, topk_w, workspace, workspace_bytes, stream,
                       events, n_events, n_launches);
}

// ---------------------------------------------------------------------------------------
// The allocation-free forward: the workspace is a static device array of the library, one
// copy per GPU (allocated by the runtime when the code object is loaded on that GPU, held until
// the process ends). In host code `scratch` names a host-side stand-in, never the device
// memory: the device address is taken once per GPU with hipGetSymbolAddress and only that
// address is passed to kernels.
namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(64) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on `device` (looked up once, with that device current).
moe_status_t scratch_of(int device, void **out) {
    if (device < 0 || device >= kMaxDevices) return fail(MOE_EHIP, "device %d outside 0..%d", device, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[device]) {
        int prev = 0;
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess) return hip_status(e, "hipGetDevice");
        if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return hip_status(e, "hipSetDevice");
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        hipError_t e2 = prev != device ? hipSetDevice(prev) : hipSuccess;
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (e2 != hipSuccess) return hip_status(e2, "hipSetDevice");
        if (!p) return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return MOE_OK;
}

}  // namespace

MOE_EXPORT size_t moe_mxfp4_noalloc_max_bytes(void) { return kScratchBytes; }

MOE_EXPORT moe_status_t moe_mxfp4_forward_noalloc(const moe_mxfp4_shape_t *shape, const moe_bf16_t *x,
                                                  const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                                  const uint8_t *gu_blocks, const uint8_t *gu_scales,
                                                  const moe_bf16_t *gu_bias, const uint8_t *dn_blocks,
                                                  const uint8_t *dn_scales, const moe_bf16_t *dn_bias,
                                                  moe_bf16_t *y, int32_t *topk_idx, float *topk_w, void *stream) {
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    const size_t need = layout_of(shape).total;
    if (need > kScratchBytes)
        return fail(MOE_EWORKSPACE,
                    "this shape needs %zu bytes of workspace; the allocation-free entry point has %zu "
                    "(use moe_mxfp4_forward with a workspace, or split the batch)",
                    need, kScratchBytes);
    int device = 0;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &device) : hipGetDevice(&device);
    if (e != hipSuccess) return hip_status(e, "device of the stream");
    void *ws = nullptr;
    st = scratch_of(device, &ws);
    if (st != MOE_OK) return st;
    return run_forward(shape, x, nullptr, 0.0, router_w, router_b, gu_blocks, gu_scales, gu_bias, dn_blocks,
                       dn_scales, dn_bias, y, topk_idx, topk_w, ws, kScratchBytes, stream, nullptr, 0, nullptr);
}

MOE_EXPORT moe_status_t moe_mxfp4_workspace_bytes_dequantized(const moe_mxfp4_shape_t *shape, size_t *bytes) {
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    REQUIRE(bytes, "bytes");
    *bytes = bank_layout_of(shape).total;
    return ok();
}

namespace {

moe_status_t run_forward_bank(const moe_mxfp4_shape_t *shape, const moe_bf16_t *x, const moe_bf16_t *router_w,
                              const moe_bf16_t *router_b, const moe_bf16_t *gu_w, const moe_bf16_t *gu_bias,
                              const moe_bf16_t *dn_w, const moe_bf16_t *dn_bias, moe_bf16_t *y, int32_t *topk_idx,
                              float *topk_w, void *workspace, size_t workspace_bytes, void *stream,
                              void *const *events, int n_events, int *n_launches) {
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (events) {
        if (n_events < 2 * MOE_MXFP4_MAX_LAUNCHES)
            return fail(MOE_EINVAL, "n_events = %d, at least %d needed", n_events, 2 * MOE_MXFP4_MAX_LAUNCHES);
        for (int i = 0; i < 2 * MOE_MXFP4_MAX_LAUNCHES; ++i)
            if (!events[i]) return fail(MOE_EINVAL, "events[%d] is NULL", i);
        REQUIRE(n_launches, "n_launches");
        *n_launches = 0;
    }
    if (shape->T == 0) return ok();
    REQUIRE16(x, "x");
    REQUIRE16(router_w, "router_w");
    REQUIRE(router_b, "router_b");
    REQUIRE16(gu_w, "gu_w");
    REQUIRE(gu_bias, "gu_bias");
    REQUIRE16(dn_w, "dn_w");
    REQUIRE(dn_bias, "dn_bias");
    REQUIRE16(y, "y");
    const BankLayout L = bank_layout_of(shape);
    if (!workspace) return fail(MOE_EWORKSPACE, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(MOE_EALIGN, "workspace is not 256-byte aligned");
    if (workspace_bytes < L.total)
        return fail(MOE_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, L.total);

    const moe::Dims d = dims_of(shape);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    int32_t *idx = topk_idx ? topk_idx : reinterpret_cast<int32_t *>(ws + L.idx);
    float *w = topk_w ? topk_w : reinterpret_cast<float *>(ws + L.w);
    int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
    int32_t *sorted_token = reinterpret_cast<int32_t *>(ws + L.sorted_token);
    float *sorted_w = reinterpret_cast<float *>(ws + L.sorted_w);
    int32_t *slot_row = reinterpret_cast<int32_t *>(ws + L.slot_row);
    moe_bf16_t *h = reinterpret_cast<moe_bf16_t *>(ws + L.h);
    float *o = reinterpret_cast<float *>(ws + L.o);
    int launched = 0;
    struct EventGuard {
        ~EventGuard() { moe::launch_events() = moe::LaunchEvents{}; }
    } guard;
    auto arm = [&]() {
        if (events)
            moe::launch_events() = moe::LaunchEvents{static_cast<hipEvent_t>(events[2 * launched]),
                                                     static_cast<hipEvent_t>(events[2 * launched + 1])};
    };
#define STEP(call, what)                                 \
    do {                                                 \
        arm();                                           \
        LAUNCH(call, what);                              \
        ++launched;                                      \
        if (n_launches) *n_launches = launched;          \
    } while (0)
    STEP(moe::launch_route(d, x, nullptr, 0.0, router_w, router_b, idx, w, nullptr, nullptr, s), "route");
    STEP(moe::launch_permute(d, idx, w, offsets, sorted_token, sorted_w, slot_row, s,
                             reinterpret_cast<int32_t *>(ws + L.hist)), "permute");
    STEP(moe::launch_up_bank(d, x, gu_w, gu_bias, offsets, sorted_token, h, s), "up (bf16 bank)");
    STEP(moe::launch_down_bank(d, h, dn_w, dn_bias, offsets, sorted_w, o, s), "down (bf16 bank)");
    STEP(moe::launch_combine(d, o, slot_row, nullptr, y, s), "combine");
#undef STEP
    return ok();
}

}  // namespace

MOE_EXPORT moe_status_t moe_mxfp4_forward_dequantized(
    const moe_mxfp4_shape_t *shape, const moe_bf16_t *x, const moe_bf16_t *router_w, const moe_bf16_t *router_b,
    const moe_bf16_t *gu_w, const moe_bf16_t *gu_bias, const moe_bf16_t *dn_w, const moe_bf16_t *dn_bias,
    moe_bf16_t *y, int32_t *topk_idx, float *topk_w, void *workspace, size_t workspace_bytes, void *stream) {
    return run_forward_bank(shape, x, router_w, router_b, gu_w, gu_bias, dn_w, dn_bias, y, topk_idx, topk_w,
                            workspace, workspace_bytes, stream, nullptr, 0, nullptr);
}

MOE_EXPORT moe_status_t moe_mxfp4_forward_dequantized_timed(
    const moe_mxfp4_shape_t *shape, const moe_bf16_t *x, const moe_bf16_t *router_w, const moe_bf16_t *router_b,
    const moe_bf16_t *gu_w, const moe_bf16_t *gu_bias, const moe_bf16_t *dn_w, const moe_bf16_t *dn_bias,
    moe_bf16_t *y, int32_t *topk_idx, float *topk_w, void *workspace, size_t workspace_bytes, void *stream,
    void *const *events, int n_events, int *n_launches) {
    if (!events) return fail(MOE_EINVAL, "events is NULL");
    return run_forward_bank(shape, x, router_w, router_b, gu_w, gu_bias, dn_w, dn_bias, y, topk_idx, topk_w,
                            workspace, workspace_bytes, stream, events, n_events, n_launches);
}

MOE_EXPORT moe_status_t moe_mxfp4_route(const moe_mxfp4_shape_t *shape, const moe_bf16_t *x,
                                        const moe_bf16_t *router_w, const moe_bf16_t *router_b,
                                        int32_t *topk_idx, float *topk_w, float *logits,
                                        void *stream) {
    moe_status_t st = check_shape(shape, false);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    REQUIRE16(x, "x");
    REQUIRE16(router_w, "router_w");
    REQUIRE(router_b, "router_b");
    REQUIRE(topk_idx, "topk_idx");
    REQUIRE(topk_w, "topk_w");
    LAUNCH(moe::launch_route(dims_of(shape), x, nullptr, 0.0, router_w, router_b, topk_idx, topk_w, logits, nullptr,
                             static_cast<hipStream_t>(stream)), "route");
    return ok();
}

MOE_EXPORT moe_status_t moe_mxfp4_permute(const moe_mxfp4_shape_t *shape, const int32_t *topk_idx,
                                          const float *topk_w, int32_t *expert_offsets,
                                          int32_t *sorted_token, float *sorted_weight,
                                          int32_t *slot_row, void *stream) {
    moe_status_t st = check_shape(shape, false);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    REQUIRE(topk_idx, "topk_idx");
    REQUIRE(topk_w, "topk_w");
    REQUIRE(expert_offsets, "expert_offsets");
    REQUIRE(sorted_token, "sorted_token");
    REQUIRE(sorted_weight, "sorted_weight");
    REQUIRE(slot_row, "slot_row");
    LAUNCH(moe::launch_permute(dims_of(shape), topk_idx, topk_w, expert_offsets, sorted_token,
                               sorted_weight, slot_row, static_cast<hipStream_t>(stream)), "permute");
    return ok();
}

MOE_EXPORT moe_status_t moe_mxfp4_permute_workspace_bytes(const moe_mxfp4_shape_t *shape, size_t *bytes) {
    moe_status_t st = check_shape(shape, false);
    if (st != MOE_OK) return st;
    REQUIRE(bytes, "bytes");
    *bytes = static_cast<size_t>(moe::permute_hist_ints(shape->T * shape->k, shape->E)) * 4;
    return ok();
}

MOE_EXPORT moe_status_t moe_mxfp4_permute_ws(const moe_mxfp4_shape_t *shape, const int32_t *topk_idx,
                                             const float *topk_w, int32_t *expert_offsets,
                                             int32_t *sorted_token, float *sorted_weight, int32_t *slot_row,
                                             void *workspace, size_t workspace_bytes, void *stream) {
    moe_status_t st = check_shape(shape, false);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    REQUIRE(topk_idx, "topk_idx");
    REQUIRE(topk_w, "topk_w");
    REQUIRE(expert_offsets, "expert_offsets");
    REQUIRE(sorted_token, "sorted_token");
    REQUIRE(sorted_weight, "sorted_weight");
    REQUIRE(slot_row, "slot_row");
    const size_t need = static_cast<size_t>(moe::permute_hist_ints(shape->T * shape->k, shape->E)) * 4;
    int32_t *hist = nullptr;
    if (need > 0) {
        if (!workspace) return fail(MOE_EWORKSPACE, "workspace is NULL");
        if (reinterpret_cast<uintptr_t>(workspace) & 3u) return fail(MOE_EALIGN, "workspace is not 4-byte aligned");
        if (workspace_bytes < need)
            return fail(MOE_EWORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
        hist = static_cast<int32_t *>(workspace);
    }
    LAUNCH(moe::launch_permute(dims_of(shape), topk_idx, topk_w, expert_offsets, sorted_token, sorted_weight,
                               slot_row, static_cast<hipStream_t>(stream), hist), "permute");
    return ok();
}

MOE_EXPORT moe_status_t moe_mxfp4_rmsnorm(const moe_bf16_t *x, const moe_bf16_t *norm_w, int64_t rows,
                                          int32_t cols, double eps, moe_bf16_t *xn, void *stream) {
    if (rows < 0) return fail(MOE_EINVAL, "rows = %lld is negative", static_cast<long long>(rows));
    if (cols <= 0 || cols % 8) return fail(MOE_ESHAPE, "cols = %d is not a positive multiple of 8", cols);
    if (rows > (static_cast<int64_t>(1) << 24))
        return fail(MOE_ESHAPE, "rows = %lld exceeds 2^24", static_cast<long long>(rows));
    if (!std::isfinite(eps) || eps < 0.0) return fail(MOE_EINVAL, "eps = %g must be finite and >= 0", eps);
    if (rows == 0) return ok();
    REQUIRE16(x, "x");
    REQUIRE16(norm_w, "norm_w");
    REQUIRE16(xn, "xn");
    moe::Dims d{};
    d.T = rows;
    d.H = cols;
    LAUNCH(moe::launch_rmsnorm(d, x, norm_w, eps, xn, static_cast<hipStream_t>(stream)), "rmsnorm");
    return ok();
}

MOE_EXPORT size_t moe_mxfp4_mx8_bytes(int64_t rows, int32_t cols) {
    return rows > 0 && cols > 0 ? moe::mx8_bytes(rows, cols) : 0;
}

namespace {
moe_status_t quantize_rows(const moe_bf16_t *x, int64_t rows, int32_t cols, uint8_t *q8, bool h8, void *stream) {
    if (rows < 0) return fail(MOE_EINVAL, "rows must be >= 0 (got %lld)", static_cast<long long>(rows));
    if (cols <= 0 || cols % 32 != 0) return fail(MOE_ESHAPE, "cols must be a positive multiple of 32 (got %d)", cols);
    if (rows == 0) return ok();
    REQUIRE16(x, "x");
    REQUIRE16(q8, "q8");
    LAUNCH(moe::launch_quantize(x, rows, cols, q8, h8, static_cast<hipStream_t>(stream)), "quantize");
    return ok();
}
}  // namespace

MOE_EXPORT moe_status_t moe_mxfp4_quantize_act(const moe_bf16_t *x, int64_t rows, int32_t cols,
                                               uint8_t *q8, void *stream) {
    return quantize_rows(x, rows, cols, q8, false, stream);
}

MOE_EXPORT moe_status_t moe_mxfp4_quantize_h(const moe_bf16_t *h, int64_t rows, int32_t cols,
                                             uint8_t *h8, void *stream) {
    return quantize_rows(h, rows, cols, h8, true, stream);
}

MOE_EXPORT moe_status_t moe_mxfp4_expert_up(const moe_mxfp4_shape_t *shape, const uint8_t *x8,
                                            const uint8_t *gu_blocks, const uint8_t *gu_scales,
                                            const moe_bf16_t *gu_bias, const int32_t *expert_offsets,
                                            const int32_t *sorted_token, uint8_t *h8, void *stream) {
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    REQUIRE16(x8, "x8");
    REQUIRE16(gu_blocks, "gu_blocks");
    REQUIRE4(gu_scales, "gu_scales");
    REQUIRE(gu_bias, "gu_bias");
    REQUIRE(expert_offsets, "expert_offsets");
    REQUIRE(sorted_token, "sorted_token");
    REQUIRE16(h8, "h8");
    LAUNCH(moe::launch_up_grouped(dims_of(shape), x8, gu_blocks, gu_scales, gu_bias, expert_offsets,
                                  sorted_token, h8, static_cast<hipStream_t>(stream)), "up");
    return ok();
}

MOE_EXPORT moe_status_t moe_mxfp4_expert_down(const moe_mxfp4_shape_t *shape, const uint8_t *h8,
                                              const uint8_t *dn_blocks, const uint8_t *dn_scales,
                                              const moe_bf16_t *dn_bias, const int32_t *expert_offsets,
                                              const float *sorted_weight, float *o, void *stream) {
    moe_status_t st = check_shape(shape, true);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    REQUIRE16(h8, "h8");
    REQUIRE16(dn_blocks, "dn_blocks");
    REQUIRE4(dn_scales, "dn_scales");
    REQUIRE(dn_bias, "dn_bias");
    REQUIRE(expert_offsets, "expert_offsets");
    REQUIRE(sorted_weight, "sorted_weight");
    REQUIRE16(o, "o");
    LAUNCH(moe::launch_down_grouped(dims_of(shape), h8, dn_blocks, dn_scales, dn_bias, expert_offsets,
                                    sorted_weight, o, static_cast<hipStream_t>(stream)), "down");
    return ok();
}

MOE_EXPORT moe_status_t moe_mxfp4_combine(const moe_mxfp4_shape_t *shape, const float *o,
                                          const int32_t *slot_row, moe_bf16_t *y, void *stream) {
    moe_status_t st = check_shape(shape, false);
    if (st != MOE_OK) return st;
    if (shape->T == 0) return ok();
    REQUIRE16(o, "o");
    REQUIRE(slot_row, "slot_row");
    REQUIRE16(y, "y");
    LAUNCH(moe::launch_combine(dims_of(shape), o, slot_row, nullptr, y, static_cast<hipStream_t>(stream)),
           "combine");
    return ok();
}

MOE_EXPORT moe_status_t moe_mxfp4_dequant(const uint8_t *blocks, const uint8_t *scales, int64_t rows,
                                          int32_t cols, moe_bf16_t *out, void *stream) {
    REQUIRE16(blocks, "blocks");
    REQUIRE(scales, "scales");
    REQUIRE16(out, "out");
    if (rows < 0) return fail(MOE_EINVAL, "rows = %lld is negative", static_cast<long long>(rows));
    if (cols <= 0 || cols % 32) return fail(MOE_ESHAPE, "cols = %d is not a positive multiple of 32", cols);
    if (rows * (cols / 32) >= (static_cast<int64_t>(1) << 40))
        return fail(MOE_ESHAPE, "rows * cols too large");
    if (rows == 0) return ok();
    LAUNCH(moe::launch_dequant(blocks, scales, rows, cols, out, static_cast<hipStream_t>(stream)),
           "dequant");
    return ok();
}
