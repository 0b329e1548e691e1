// abi.hip -- the exported C ABI (include/nvfp4moe.h): argument checks that fail closed, then the
// kernel launches. Checks run on the host before anything is enqueued. Metadata gates that "fail
// closed" are the pages' admission rule ("[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency",
// "Guarded production engine result").
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "internal.hpp"

#define NVFP4_API extern "C" __attribute__((visibility("default")))

namespace {

using nvfp4::PlanLayout;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool plan_shape_ok(int32_t M, int32_t topk, int32_t E)
{
    return M >= 0 && topk >= 1 && topk <= nvfp4::MAX_TOPK && E >= 1 && (int64_t)M * topk <= (int64_t(1) << 26);
}

int check_weights(const nvfp4_weights *w)
{
    if (!w || !w->codes || !w->scales || !w->global_scale) return NVFP4_ERR_NULL;
    if (w->groups < 1 || w->rows < 1 || w->k < 16 || w->k % 16 != 0) return NVFP4_ERR_SHAPE;
    if (!aligned(w->codes, 16) || !aligned(w->scales, 8) || !aligned(w->global_scale, 4)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

}  // namespace

NVFP4_API int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

NVFP4_API const char *nvfp4_status_str(int status)
{
    switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED";
    case NVFP4_ERR_LAUNCH: return "NVFP4_ERR_LAUNCH";
    default: return "NVFP4_ERR_UNKNOWN";
    }
}

NVFP4_API size_t nvfp4_moe_plan_bytes(int32_t M, int32_t topk, int32_t E)
{
    if (!plan_shape_ok(M, topk, E)) return 0;
    return (size_t)nvfp4::plan_layout(M, topk, E).words * sizeof(int32_t);
}

NVFP4_API int nvfp4_moe_plan(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, void *plan,
                             size_t plan_bytes, void *stream)
{
    if (!plan_shape_ok(M, topk, E)) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!topk_ids || !plan) return NVFP4_ERR_NULL;
    if (!aligned(topk_ids, 4) || !aligned(plan, 16)) return NVFP4_ERR_ALIGN;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    if (plan_bytes < (size_t)L.words * sizeof(int32_t)) return NVFP4_ERR_WORKSPACE;
    return nvfp4::run_plan(topk_ids, M, topk, E, static_cast<int32_t *>(plan), L, static_cast<hipStream_t>(stream));
}

NVFP4_API int nvfp4_moe_route(const float *logits, int32_t M, int32_t E, int32_t topk, int32_t *topk_ids,
                              float *topk_weights, void *plan, size_t plan_bytes, void *stream)
{
    if (!plan_shape_ok(M, topk, E) || topk > E) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!logits || !topk_ids || !topk_weights || !plan) return NVFP4_ERR_NULL;
    if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) || !aligned(plan, 16))
        return NVFP4_ERR_ALIGN;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    if (plan_bytes < (size_t)L.words * sizeof(int32_t)) return NVFP4_ERR_WORKSPACE;
    return nvfp4::run_route(logits, M, E, topk, topk_ids, topk_weights, static_cast<int32_t *>(plan), L,
                            static_cast<hipStream_t>(stream));
}

NVFP4_API int nvfp4_moe_w13_swiglu(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                                   const nvfp4_weights *w13, int32_t layout, uint16_t *h, void *stream)
{
    if (!plan_shape_ok(M, topk, E)) return NVFP4_ERR_SHAPE;
    if (layout != 0 && layout != 1) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    int st = check_weights(w13);
    if (st != NVFP4_OK) return st;
    if (w13->groups != E || w13->rows % 2 != 0) return NVFP4_ERR_SHAPE;
    const int K = w13->k, I = w13->rows / 2;
    if (K % 128 != 0 || K > nvfp4::MAX_MOE_RED || I % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!plan || !x || !h) return NVFP4_ERR_NULL;
    if (!aligned(plan, 16) || !aligned(x, 16) || !aligned(h, 16)) return NVFP4_ERR_ALIGN;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (nvfp4::use_prefill(M, L.P, E, K, I))
        return nvfp4::run_w13_prefill(nvfp4::plan_view(plan, L), L.A, M, topk, x, *w13, layout, h, s);
    return nvfp4::run_w13(nvfp4::plan_view(plan, L), L.T, topk, x, *w13, layout, h, s);
}

namespace {

// The plan and W13 after every check passed: one launch (the plan built in the W13 launch) for
// small decode batches, else the plan's launches and then the regime's W13 kernel.
// pair_major (the layer call, only where use_pair_major holds): h in pair order, see FusedPlan.
int enqueue_plan_w13(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, int32_t *pl, const uint16_t *x,
                     const nvfp4_weights &w13, int32_t layout, uint16_t *h, hipStream_t s, bool pair_major = false)
{
    const int K = w13.k, I = w13.rows / 2;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    const bool prefill = nvfp4::use_prefill(M, L.P, E, K, I);
    if (!prefill && nvfp4::use_fused_plan(L.P, E)) {
        nvfp4::FusedPlan fp;
        fp.ids = topk_ids;
        fp.plan = pl;
        fp.L = L;
        fp.M = M;
        fp.E = E;
        fp.pair_major = pair_major;
        return nvfp4::run_w13(nvfp4::plan_view(pl, L), L.T, topk, x, w13, layout, h, s, {}, fp);
    }
    int st = nvfp4::run_plan(topk_ids, M, topk, E, pl, L, s);
    if (st != NVFP4_OK) return st;
    if (prefill) return nvfp4::run_w13_prefill(nvfp4::plan_view(pl, L), L.A, M, topk, x, w13, layout, h, s);
    return nvfp4::run_w13(nvfp4::plan_view(pl, L), L.T, topk, x, w13, layout, h, s);
}

// W2 and the reduction after every check passed.
// pair_ids (the layer call's pair-major path): h is in pair order; the token-major kernel reads
// each slot's expert from these ids.
int enqueue_w2(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *h, const nvfp4_weights &w2,
               const float *topk_weights, uint16_t *out, void *ws, hipStream_t s, nvfp4::SharedTerm sh,
               const int32_t *pair_ids = nullptr)
{
    const int K = w2.rows, I = w2.k;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    const nvfp4::PlanView pv = nvfp4::plan_view(plan, L);
    if (nvfp4::use_prefill(M, L.P, E, K, I)) {
        const int st = nvfp4::run_w2_prefill(pv, L.A, L.P, h, w2, static_cast<float *>(ws), s);
        if (st != NVFP4_OK) return st;
        return nvfp4::run_reduce(pv, M, topk, K, topk_weights, static_cast<const float *>(ws), out, s, sh);
    }
    return nvfp4::run_w2(pv, L.T, M, topk, h, w2, topk_weights, out, static_cast<float *>(ws), s, sh, {}, pair_ids);
}

}  // namespace

NVFP4_API int nvfp4_moe_plan_w13_swiglu(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, void *plan,
                                        size_t plan_bytes, const uint16_t *x, const nvfp4_weights *w13,
                                        int32_t layout, uint16_t *h, void *stream)
{
    // Every check of nvfp4_moe_plan and nvfp4_moe_w13_swiglu, before anything is enqueued.
    if (!plan_shape_ok(M, topk, E)) return NVFP4_ERR_SHAPE;
    if (layout != 0 && layout != 1) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    int st = check_weights(w13);
    if (st != NVFP4_OK) return st;
    if (w13->groups != E || w13->rows % 2 != 0) return NVFP4_ERR_SHAPE;
    const int K = w13->k, I = w13->rows / 2;
    if (K % 128 != 0 || K > nvfp4::MAX_MOE_RED || I % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!topk_ids || !plan || !x || !h) return NVFP4_ERR_NULL;
    if (!aligned(topk_ids, 4) || !aligned(plan, 16) || !aligned(x, 16) || !aligned(h, 16)) return NVFP4_ERR_ALIGN;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    if (plan_bytes < (size_t)L.words * sizeof(int32_t)) return NVFP4_ERR_WORKSPACE;
    return enqueue_plan_w13(topk_ids, M, topk, E, static_cast<int32_t *>(plan), x, *w13, layout, h,
                            static_cast<hipStream_t>(stream));
}

NVFP4_API size_t nvfp4_moe_w2_workspace_bytes(int32_t M, int32_t topk, int32_t K)
{
    if (M < 0 || topk < 1 || topk > nvfp4::MAX_TOPK || K < 1) return 0;
    const size_t b = (size_t)M * topk * K * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

namespace {

int w2_reduce(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *h, const nvfp4_weights *w2,
              const float *topk_weights, uint16_t *out, void *ws, size_t ws_bytes, void *stream, nvfp4::SharedTerm sh)
{
    if (!plan_shape_ok(M, topk, E)) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    int st = check_weights(w2);
    if (st != NVFP4_OK) return st;
    if (w2->groups != E) return NVFP4_ERR_SHAPE;
    const int K = w2->rows, I = w2->k;
    if (I % 128 != 0 || I > nvfp4::MAX_MOE_RED || K % 64 != 0) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!plan || !h || !topk_weights || !out || !ws) return NVFP4_ERR_NULL;
    if (!aligned(plan, 16) || !aligned(h, 16) || !aligned(out, 16) || !aligned(ws, 16) || !aligned(topk_weights, 4))
        return NVFP4_ERR_ALIGN;
    if (sh.y && (!aligned(sh.y, 16) || !aligned(sh.sigma, 4))) return NVFP4_ERR_ALIGN;
    if (ws_bytes < nvfp4_moe_w2_workspace_bytes(M, topk, K)) return NVFP4_ERR_WORKSPACE;
    return enqueue_w2(plan, M, topk, E, h, *w2, topk_weights, out, ws, static_cast<hipStream_t>(stream), sh);
}

}  // namespace

NVFP4_API int nvfp4_moe_w2_reduce(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *h,
                                  const nvfp4_weights *w2, const float *topk_weights, uint16_t *out, void *ws,
                                  size_t ws_bytes, void *stream)
{
    return w2_reduce(plan, M, topk, E, h, w2, topk_weights, out, ws, ws_bytes, stream, {});
}

NVFP4_API int nvfp4_moe_w2_reduce_shared(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *h,
                                         const nvfp4_weights *w2, const float *topk_weights, const float *shared_y,
                                         const float *shared_sigma, uint16_t *out, void *ws, size_t ws_bytes,
                                         void *stream)
{
    if (M > 0 && (!shared_y || !shared_sigma)) return NVFP4_ERR_NULL;
    nvfp4::SharedTerm sh;
    sh.y = shared_y;
    sh.sigma = shared_sigma;
    return w2_reduce(plan, M, topk, E, h, w2, topk_weights, out, ws, ws_bytes, stream, sh);
}

namespace {

// Byte offsets of the layer workspace's parts: plan, h, W2 workspace (each a multiple of 256).
struct LayerParts {
    size_t h, w2, total;
};

LayerParts layer_parts(int32_t M, int32_t topk, int32_t E, int32_t K, int32_t I)
{
    LayerParts p;
    p.h = nvfp4_moe_plan_bytes(M, topk, E);
    const size_t hb = (size_t)M * topk * I * 2;
    p.w2 = p.h + ((hb + 255) & ~(size_t)255);
    p.total = p.w2 + nvfp4_moe_w2_workspace_bytes(M, topk, K);
    return p;
}

bool layer_shape_ok(int32_t M, int32_t topk, int32_t E, int32_t K, int32_t I)
{
    return plan_shape_ok(M, topk, E) && K >= 16 && I >= 1;
}

// Every check of nvfp4_moe_plan_w13_swiglu and nvfp4_moe_w2_reduce for the layer call, except the
// workspace size. Returns the status; on OK, *K_out and *I_out are the layer's sizes.
int check_layer(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                const nvfp4_weights *w13, int32_t layout, const nvfp4_weights *w2, const float *topk_weights,
                const uint16_t *out, int32_t *K_out, int32_t *I_out)
{
    if (!plan_shape_ok(M, topk, E) || (layout != 0 && layout != 1)) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    int st = check_weights(w13);
    if (st == NVFP4_OK) st = check_weights(w2);
    if (st != NVFP4_OK) return st;
    if (w13->groups != E || w13->rows % 2 != 0 || w2->groups != E) return NVFP4_ERR_SHAPE;
    const int K = w13->k, I = w13->rows / 2;
    if (w2->rows != K || w2->k != I) return NVFP4_ERR_SHAPE;
    if (K % 128 != 0 || K > nvfp4::MAX_MOE_RED || I % 128 != 0 || I > nvfp4::MAX_MOE_RED)
        return NVFP4_ERR_UNSUPPORTED;
    *K_out = K;
    *I_out = I;
    if (M == 0) return NVFP4_OK;
    if (!topk_ids || !x || !topk_weights || !out) return NVFP4_ERR_NULL;
    if (!aligned(topk_ids, 4) || !aligned(x, 16) || !aligned(topk_weights, 4) || !aligned(out, 16))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// The layer on a workspace that passed every check: plan + W13, then W2 + reduction.
int enqueue_layer(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                  const nvfp4_weights &w13, int32_t layout, const nvfp4_weights &w2, const float *topk_weights,
                  uint16_t *out, uint8_t *ws, hipStream_t s)
{
    const LayerParts parts = layer_parts(M, topk, E, w13.k, w13.rows / 2);
    int32_t *plan = reinterpret_cast<int32_t *>(ws);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + parts.h);
    // Small batches take the pair-major path: W13 reads its rows straight from the ids, h in pair
    // order, and the token-major W2 reads the ids and that h, so no load waits for the plan.
    const bool pm = nvfp4::use_pair_major((int64_t)M * topk, E);
    const int st = enqueue_plan_w13(topk_ids, M, topk, E, plan, x, w13, layout, h, s, pm);
    if (st != NVFP4_OK) return st;
    return enqueue_w2(plan, M, topk, E, h, w2, topk_weights, out, ws + parts.w2, s, {}, pm ? topk_ids : nullptr);
}

}  // namespace

NVFP4_API size_t nvfp4_moe_layer_workspace_bytes(int32_t M, int32_t topk, int32_t E, int32_t K, int32_t I)
{
    if (!layer_shape_ok(M, topk, E, K, I)) return 0;
    return layer_parts(M, topk, E, K, I).total;
}

NVFP4_API int nvfp4_moe_layer(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                              const nvfp4_weights *w13, int32_t layout, const nvfp4_weights *w2,
                              const float *topk_weights, uint16_t *out, void *ws, size_t ws_bytes, void *stream)
{
    int32_t K = 0, I = 0;
    const int st = check_layer(topk_ids, M, topk, E, x, w13, layout, w2, topk_weights, out, &K, &I);
    if (st != NVFP4_OK || M == 0) return st;
    if (!ws) return NVFP4_ERR_NULL;
    if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    if (ws_bytes < layer_parts(M, topk, E, K, I).total) return NVFP4_ERR_WORKSPACE;
    return enqueue_layer(topk_ids, M, topk, E, x, *w13, layout, *w2, topk_weights, out, static_cast<uint8_t *>(ws),
                         static_cast<hipStream_t>(stream));
}

// ---- the layer without allocation (nvfp4_moe_layer_noalloc) ------------------------------------
// For callers that cannot allocate: the layer workspace is this file-scope device array. Each GPU
// holds its own copy at its own address. In host code `scratch` names only a host-side stand-in,
// so it is never passed to a kernel or a copy: the device address comes from hipGetSymbolAddress,
// taken once per device (with that device current) on the first call there, and kept.
static __device__ __align__(256) uint8_t scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::atomic<uint8_t *> scratch_dev[MAX_DEVICES];
std::mutex scratch_mu;

// Device address of the current device's scratch array, or nullptr (status in *st) if the runtime
// cannot give it.
uint8_t *scratch_ptr(int *st)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        *st = NVFP4_ERR_LAUNCH;
        return nullptr;
    }
    uint8_t *p = scratch_dev[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
            *st = NVFP4_ERR_LAUNCH;
            return nullptr;
        }
        p = static_cast<uint8_t *>(addr);
        scratch_dev[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

NVFP4_API int nvfp4_moe_layer_noalloc(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                                      const nvfp4_weights *w13, int32_t layout, const nvfp4_weights *w2,
                                      const float *topk_weights, uint16_t *out, void *stream)
{
    int32_t K = 0, I = 0;
    int st = check_layer(topk_ids, M, topk, E, x, w13, layout, w2, topk_weights, out, &K, &I);
    if (st != NVFP4_OK || M == 0) return st;
    if (layer_parts(M, topk, E, K, I).total > NVFP4_NOALLOC_SCRATCH_BYTES) return NVFP4_ERR_WORKSPACE;
    uint8_t *ws = scratch_ptr(&st);
    if (!ws) return st;
    return enqueue_layer(topk_ids, M, topk, E, x, *w13, layout, *w2, topk_weights, out, ws,
                         static_cast<hipStream_t>(stream));
}

NVFP4_API int nvfp4_moe_shared_expert(const uint16_t *x, int32_t M, const nvfp4_weights *w13, int32_t layout,
                                      const nvfp4_weights *w2, const uint16_t *gate, uint16_t *h, float *shared_y,
                                      float *shared_sigma, void *stream)
{
    if (M < 0 || (layout != 0 && layout != 1)) return NVFP4_ERR_SHAPE;
    int st = check_weights(w13);
    if (st == NVFP4_OK) st = check_weights(w2);
    if (st != NVFP4_OK) return st;
    const int K = w13->k, I = w13->rows / 2;
    if (w13->groups != 1 || w2->groups != 1 || w13->rows % 2 != 0 || w2->rows != K || w2->k != I)
        return NVFP4_ERR_SHAPE;
    if (K % 128 != 0 || K > nvfp4::MAX_LINEAR_SWIGLU_K || I % 128 != 0 || I > nvfp4::MAX_LINEAR_K)
        return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!x || !gate || !h || !shared_y || !shared_sigma) return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(h, 16) || !aligned(shared_y, 16) || !aligned(gate, 2) || !aligned(shared_sigma, 4))
        return NVFP4_ERR_ALIGN;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = nvfp4::linear_prepare();
    if (st == NVFP4_OK) st = nvfp4::run_linear_swiglu(x, M, *w13, layout, h, s);
    if (st == NVFP4_OK) st = nvfp4::run_linear_f32(h, M, *w2, shared_y, s);
    if (st == NVFP4_OK) st = nvfp4::run_shared_gate(x, M, K, gate, shared_sigma, s);
    return st;
}

NVFP4_API int nvfp4_moe_w13_swiglu_with_shared(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *x,
                                               const nvfp4_weights *w13, int32_t layout, uint16_t *h,
                                               const nvfp4_weights *shared_w13, const uint16_t *gate, uint16_t *shared_h,
                                               float *shared_sigma, void *stream)
{
    if (!plan_shape_ok(M, topk, E) || (layout != 0 && layout != 1)) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    int st = check_weights(w13);
    if (st == NVFP4_OK) st = check_weights(shared_w13);
    if (st != NVFP4_OK) return st;
    if (w13->groups != E || w13->rows % 2 != 0 || shared_w13->groups != 1 || shared_w13->rows % 2 != 0 ||
        shared_w13->k != w13->k)
        return NVFP4_ERR_SHAPE;
    const int K = w13->k, I = w13->rows / 2, Is = shared_w13->rows / 2;
    if (K % 128 != 0 || K > nvfp4::MAX_MOE_RED || I % 16 != 0 || Is % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!plan || !x || !h || !gate || !shared_h || !shared_sigma) return NVFP4_ERR_NULL;
    if (!aligned(plan, 16) || !aligned(x, 16) || !aligned(h, 16) || !aligned(shared_h, 16) || !aligned(gate, 2) ||
        !aligned(shared_sigma, 4))
        return NVFP4_ERR_ALIGN;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const nvfp4::PlanView pv = nvfp4::plan_view(plan, L);
    if (!nvfp4::use_prefill(M, L.P, E, K, I) && Is == I && aligned(gate, 16)) {
        nvfp4::SharedW13 shx;
        shx.codes = shared_w13->codes;
        shx.scales = shared_w13->scales;
        shx.gscale = shared_w13->global_scale;
        shx.h = shared_h;
        shx.gate = gate;
        shx.sigma = shared_sigma;
        shx.M = M;
        return nvfp4::run_w13(pv, L.T, topk, x, *w13, layout, h, s, shx);
    }
    // Separate launches: the routed regime's W13, then the shared expert's gate/up and its gate.
    st = nvfp4::linear_prepare();
    if (st != NVFP4_OK) return st;
    st = nvfp4::use_prefill(M, L.P, E, K, I) ? nvfp4::run_w13_prefill(pv, L.A, M, topk, x, *w13, layout, h, s)
                                              : nvfp4::run_w13(pv, L.T, topk, x, *w13, layout, h, s);
    if (st == NVFP4_OK) st = nvfp4::run_linear_swiglu(x, M, *shared_w13, layout, shared_h, s);
    if (st == NVFP4_OK) st = nvfp4::run_shared_gate(x, M, K, gate, shared_sigma, s);
    return st;
}

NVFP4_API int nvfp4_moe_plan_w13_swiglu_with_shared(const int32_t *topk_ids, int32_t M, int32_t topk, int32_t E,
                                                    void *plan, size_t plan_bytes, const uint16_t *x,
                                                    const nvfp4_weights *w13, int32_t layout, uint16_t *h,
                                                    const nvfp4_weights *shared_w13, const uint16_t *gate,
                                                    uint16_t *shared_h, float *shared_sigma, void *stream)
{
    // Every check of nvfp4_moe_plan and nvfp4_moe_w13_swiglu_with_shared, before anything is enqueued.
    if (!plan_shape_ok(M, topk, E) || (layout != 0 && layout != 1)) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    int st = check_weights(w13);
    if (st == NVFP4_OK) st = check_weights(shared_w13);
    if (st != NVFP4_OK) return st;
    if (w13->groups != E || w13->rows % 2 != 0 || shared_w13->groups != 1 || shared_w13->rows % 2 != 0 ||
        shared_w13->k != w13->k)
        return NVFP4_ERR_SHAPE;
    const int K = w13->k, I = w13->rows / 2, Is = shared_w13->rows / 2;
    if (K % 128 != 0 || K > nvfp4::MAX_MOE_RED || I % 16 != 0 || Is % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!topk_ids || !plan || !x || !h || !gate || !shared_h || !shared_sigma) return NVFP4_ERR_NULL;
    if (!aligned(topk_ids, 4) || !aligned(plan, 16) || !aligned(x, 16) || !aligned(h, 16) ||
        !aligned(shared_h, 16) || !aligned(gate, 2) || !aligned(shared_sigma, 4))
        return NVFP4_ERR_ALIGN;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    if (plan_bytes < (size_t)L.words * sizeof(int32_t)) return NVFP4_ERR_WORKSPACE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (!nvfp4::use_prefill(M, L.P, E, K, I) && Is == I && aligned(gate, 16) && nvfp4::use_fused_plan(L.P, E)) {
        nvfp4::SharedW13 shx;
        shx.codes = shared_w13->codes;
        shx.scales = shared_w13->scales;
        shx.gscale = shared_w13->global_scale;
        shx.h = shared_h;
        shx.gate = gate;
        shx.sigma = shared_sigma;
        shx.M = M;
        nvfp4::FusedPlan fp;
        fp.ids = topk_ids;
        fp.plan = static_cast<int32_t *>(plan);
        fp.L = L;
        fp.M = M;
        fp.E = E;
        return nvfp4::run_w13(nvfp4::plan_view(plan, L), L.T, topk, x, *w13, layout, h, s, shx, fp);
    }
    st = nvfp4::linear_prepare();  // the call below may run the shared expert's own launches
    if (st == NVFP4_OK) st = nvfp4::run_plan(topk_ids, M, topk, E, static_cast<int32_t *>(plan), L, s);
    if (st != NVFP4_OK) return st;
    return nvfp4_moe_w13_swiglu_with_shared(plan, M, topk, E, x, w13, layout, h, shared_w13, gate, shared_h,
                                            shared_sigma, stream);
}

NVFP4_API int nvfp4_moe_w2_reduce_with_shared(const void *plan, int32_t M, int32_t topk, int32_t E, const uint16_t *h,
                                              const nvfp4_weights *w2, const float *topk_weights,
                                              const uint16_t *shared_h, const nvfp4_weights *shared_w2,
                                              const float *shared_sigma, float *shared_y, uint16_t *out, void *ws,
                                              size_t ws_bytes, void *stream)
{
    if (!plan_shape_ok(M, topk, E)) return NVFP4_ERR_SHAPE;
    if (E > nvfp4::MAX_EXPERTS) return NVFP4_ERR_UNSUPPORTED;
    int st = check_weights(w2);
    if (st == NVFP4_OK) st = check_weights(shared_w2);
    if (st != NVFP4_OK) return st;
    if (w2->groups != E || shared_w2->groups != 1 || shared_w2->rows != w2->rows) return NVFP4_ERR_SHAPE;
    const int K = w2->rows, I = w2->k, Is = shared_w2->k;
    if (I % 128 != 0 || I > nvfp4::MAX_MOE_RED || K % 64 != 0 || Is % 128 != 0 || Is > nvfp4::MAX_LINEAR_K)
        return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!plan || !h || !topk_weights || !out || !ws || !shared_h || !shared_sigma || !shared_y) return NVFP4_ERR_NULL;
    if (!aligned(plan, 16) || !aligned(h, 16) || !aligned(out, 16) || !aligned(ws, 16) || !aligned(topk_weights, 4) ||
        !aligned(shared_h, 16) || !aligned(shared_sigma, 4) || !aligned(shared_y, 16))
        return NVFP4_ERR_ALIGN;
    if (ws_bytes < nvfp4_moe_w2_workspace_bytes(M, topk, K)) return NVFP4_ERR_WORKSPACE;
    const PlanLayout L = nvfp4::plan_layout(M, topk, E);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const nvfp4::PlanView pv = nvfp4::plan_view(plan, L);
    if (!nvfp4::use_prefill(M, L.P, E, K, I) && Is == I) {
        nvfp4::SharedW2 shw;
        shw.codes = shared_w2->codes;
        shw.scales = shared_w2->scales;
        shw.gscale = shared_w2->global_scale;
        shw.h = shared_h;
        shw.y = shared_y;
        shw.sigma = shared_sigma;
        shw.M = M;
        return nvfp4::run_w2(pv, L.T, M, topk, h, *w2, topk_weights, out, static_cast<float *>(ws), s, {}, shw);
    }
    // Separate launches: the shared expert's down projection, then W2 + reduction with its term.
    st = nvfp4::linear_prepare();
    if (st == NVFP4_OK) st = nvfp4::run_linear_f32(shared_h, M, *shared_w2, shared_y, s);
    if (st != NVFP4_OK) return st;
    nvfp4::SharedTerm sh;
    sh.y = shared_y;
    sh.sigma = shared_sigma;
    return w2_reduce(plan, M, topk, E, h, w2, topk_weights, out, ws, ws_bytes, stream, sh);
}

NVFP4_API int nvfp4_linear(const uint16_t *x, int32_t M, const nvfp4_weights *w, uint16_t *y, void *stream)
{
    if (M < 0) return NVFP4_ERR_SHAPE;
    int st = check_weights(w);
    if (st != NVFP4_OK) return st;
    if (w->groups != 1) return NVFP4_ERR_SHAPE;
    if (w->k % 128 != 0 || w->k > nvfp4::MAX_LINEAR_K || w->rows % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!x || !y) return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16)) return NVFP4_ERR_ALIGN;
    return nvfp4::run_linear(x, M, *w, y, static_cast<hipStream_t>(stream));
}

NVFP4_API int nvfp4_linear_swiglu(const uint16_t *x, int32_t M, const nvfp4_weights *w13, int32_t layout, uint16_t *h,
                                  void *stream)
{
    if (M < 0 || (layout != 0 && layout != 1)) return NVFP4_ERR_SHAPE;
    int st = check_weights(w13);
    if (st != NVFP4_OK) return st;
    if (w13->groups != 1 || w13->rows % 2 != 0) return NVFP4_ERR_SHAPE;
    if (w13->k % 128 != 0 || w13->k > nvfp4::MAX_LINEAR_SWIGLU_K || (w13->rows / 2) % 16 != 0)
        return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!x || !h) return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(h, 16)) return NVFP4_ERR_ALIGN;
    return nvfp4::run_linear_swiglu(x, M, *w13, layout, h, static_cast<hipStream_t>(stream));
}

NVFP4_API size_t nvfp4_linear_ws_bytes(int32_t M, int32_t N, int32_t K)
{
    if (M < 0 || N < 1 || K < 1) return 0;
    return nvfp4::linear_ws_bytes(M, N, K);
}

// The split-K calls: the same checks as the one-launch calls, then the workspace's.
static int split_ws_ok(int32_t M, const nvfp4_weights *w, const void *ws, size_t ws_bytes)
{
    if (!ws) return NVFP4_ERR_NULL;
    if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    if (ws_bytes < nvfp4::linear_ws_bytes(M, w->rows, w->k)) return NVFP4_ERR_WORKSPACE;
    // the fold launch takes four outputs per thread, 64 threads per block
    if ((int64_t)M * w->rows / 256 >= (int64_t)INT32_MAX) return NVFP4_ERR_UNSUPPORTED;
    return NVFP4_OK;
}

NVFP4_API int nvfp4_linear_ws(const uint16_t *x, int32_t M, const nvfp4_weights *w, uint16_t *y, void *ws,
                              size_t ws_bytes, void *stream)
{
    if (M < 0) return NVFP4_ERR_SHAPE;
    int st = check_weights(w);
    if (st != NVFP4_OK) return st;
    if (w->groups != 1) return NVFP4_ERR_SHAPE;
    if (w->k % 128 != 0 || w->k > nvfp4::MAX_LINEAR_K || w->rows % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!x || !y) return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16)) return NVFP4_ERR_ALIGN;
    if ((st = split_ws_ok(M, w, ws, ws_bytes)) != NVFP4_OK) return st;
    return nvfp4::run_linear_split(x, M, *w, y, ws, static_cast<hipStream_t>(stream));
}

NVFP4_API int nvfp4_linear_swiglu_ws(const uint16_t *x, int32_t M, const nvfp4_weights *w13, int32_t layout,
                                     uint16_t *h, void *ws, size_t ws_bytes, void *stream)
{
    if (M < 0 || (layout != 0 && layout != 1)) return NVFP4_ERR_SHAPE;
    int st = check_weights(w13);
    if (st != NVFP4_OK) return st;
    if (w13->groups != 1 || w13->rows % 2 != 0) return NVFP4_ERR_SHAPE;
    if (w13->k % 128 != 0 || w13->k > nvfp4::MAX_LINEAR_SWIGLU_K || (w13->rows / 2) % 16 != 0)
        return NVFP4_ERR_UNSUPPORTED;
    if (M == 0) return NVFP4_OK;
    if (!x || !h) return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(h, 16)) return NVFP4_ERR_ALIGN;
    if ((st = split_ws_ok(M, w13, ws, ws_bytes)) != NVFP4_OK) return st;
    return nvfp4::run_linear_swiglu_split(x, M, *w13, layout, h, ws, static_cast<hipStream_t>(stream));
}

NVFP4_API int nvfp4_linear_fp8(const uint16_t *x, int32_t M, const fp8_channel_weights *w, uint16_t *y, void *stream)
{
    if (M < 0) return NVFP4_ERR_SHAPE;
    if (!w || !w->codes || !w->channel_scale) return NVFP4_ERR_NULL;
    if (w->rows < 1 || w->k < 16) return NVFP4_ERR_SHAPE;
    if (w->k % 128 != 0 || w->k > nvfp4::MAX_LINEAR_FP8_K || w->rows % 16 != 0) return NVFP4_ERR_UNSUPPORTED;
    if (!aligned(w->codes, 16) || !aligned(w->channel_scale, 4)) return NVFP4_ERR_ALIGN;
    if (M == 0) return NVFP4_OK;
    if (!x || !y) return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16)) return NVFP4_ERR_ALIGN;
    return nvfp4::run_linear_fp8(x, M, *w, y, static_cast<hipStream_t>(stream));
}
