// internal.hpp -- declarations shared by the host ABI (abi.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <tuple>
#include <type_traits>
#include <utility>

#include "../../include/nvfp4moe.h"

namespace nvfp4 {

// Word offsets of the routing plan's arrays inside the caller's plan buffer; the layout is the one
// documented with nvfp4_moe_plan in nvfp4moe.h. P = M*topk pairs, A = min(E, P) active-expert
// bound, T = A + ceil(P/16) row-tile bound. Plans with P > SMALL_PLAN_PAIRS also carry scratch:
// per-chunk expert histograms hist[E][G] (G = ceil(P/PLAN_CHUNK)), per-chunk bad-id counts and
// each expert's first row-tile index.
constexpr int PLAN_HDR_WORDS = 16;
constexpr int PLAN_TILE_ROWS = 16;
constexpr int SMALL_PLAN_PAIRS = 1024;
constexpr int PLAN_CHUNK = 256;
constexpr int MAX_EXPERTS = 4096;
constexpr int MAX_TOPK = 32;
// Largest reduction lengths with a kernel: the MoE kernels split at most four 512-element chunks
// over a block's waves; the dense kernel keeps one LDS partial tile per chunk.
constexpr int MAX_MOE_RED = 2048;
// The dense kernels keep one FP32 partial tile per (chunk, row tile, weight tile) in LDS:
// S * 2 * NW * 16 * 20 * 4 bytes for S = K/512 chunks and NW weight tiles per wave, within the
// 160 KiB of a gfx950 CU. Two weight tiles per wave therefore fit up to K = 16384 and one up to
// K = 32768; the plain projection takes one tile per wave beyond 16384.
constexpr int MAX_LINEAR_K = 32768;
constexpr int MAX_LINEAR_SWIGLU_K = 16384;  // always two weight tiles per wave (gate and up)
constexpr int MAX_LINEAR_FP8_K = 16384;     // two weight tiles per wave always fit
constexpr size_t MAX_LDS_BYTES = 160 * 1024;
constexpr size_t linear_lds_bytes(int k, int nw) { return (size_t)((k + 511) / 512) * 2 * nw * 16 * 20 * 4; }
// Most weight tiles per wave of the plain dense kernels: two wherever their partial tiles fit in
// LDS, else one. A block then owns up to 16 output columns per tile.
constexpr int linear_max_tiles(int k) { return linear_lds_bytes(k, 2) <= MAX_LDS_BYTES ? 2 : 1; }

// CU count of the current device, queried from the runtime once per device and cached.
inline int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

struct PlanLayout {
    int64_t P, A, T, G;
    int64_t hdr, counts, offsets, active, tile_expert, tile_row0, tile_base, tile_rows, tile_pair, sorted_pair,
        pos_of_pair, pair_expert, hist, badc, tile_first, words;
};

inline PlanLayout plan_layout(int32_t M, int32_t topk, int32_t E)
{
    PlanLayout L{};
    L.P = (int64_t)M * topk;
    L.A = L.P < E ? L.P : E;
    L.T = L.A + (L.P + PLAN_TILE_ROWS - 1) / PLAN_TILE_ROWS;
    L.G = L.P > SMALL_PLAN_PAIRS ? (L.P + PLAN_CHUNK - 1) / PLAN_CHUNK : 0;
    int64_t o = 0;
    L.hdr = o;         o += PLAN_HDR_WORDS;
    L.counts = o;      o += E;
    L.offsets = o;     o += E + 1;
    L.active = o;      o += L.A;
    L.tile_expert = o; o += L.T;
    L.tile_row0 = o;   o += L.T;
    L.tile_base = o;   o += L.T;
    L.tile_rows = o;   o += L.T;
    L.tile_pair = o;    o += L.T * PLAN_TILE_ROWS;
    L.sorted_pair = o; o += L.P;
    L.pos_of_pair = o; o += L.P;
    L.pair_expert = o; o += L.P;
    L.hist = o;        o += (int64_t)E * L.G;
    L.badc = o;        o += L.G;
    L.tile_first = o;  o += L.G > 0 ? E : 0;
    L.words = (o + 63) & ~(int64_t)63;  // whole 256-byte lines
    return L;
}

// Read-only device view of a built plan.
struct PlanView {
    const int32_t *hdr, *counts, *offsets, *active, *tile_expert, *tile_row0, *tile_base, *tile_rows, *tile_pair,
        *sorted_pair, *pos_of_pair, *pair_expert;
};

inline PlanView plan_view(const void *plan, const PlanLayout &L)
{
    const int32_t *p = static_cast<const int32_t *>(plan);
    return PlanView{p + L.hdr,       p + L.counts,    p + L.offsets,   p + L.active,
                    p + L.tile_expert, p + L.tile_row0, p + L.tile_base, p + L.tile_rows,
                    p + L.tile_pair,  p + L.sorted_pair, p + L.pos_of_pair, p + L.pair_expert};
}

// Launch `kernel` through hipLaunchKernel, so a rejected launch is reported as a status instead
// of being left in the runtime's sticky last-error slot.
template <typename... KArgs, typename... Args>
inline int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t s, Args &&...args)
{
    std::tuple<KArgs...> held(std::forward<Args>(args)...);
    void *argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    std::apply([&](auto &...a) {
        int i = 0;
        ((argv[i++] = static_cast<void *>(&a)), ...);
    }, held);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, shmem, s);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

// Kernel launchers, one per translation unit. Arguments are validated by the caller (abi.hip).
int run_plan(const int32_t *ids, int32_t M, int32_t topk, int32_t E, int32_t *plan, const PlanLayout &L,
             hipStream_t s);
int run_route(const float *logits, int32_t M, int32_t E, int32_t topk, int32_t *ids, float *weights, int32_t *plan,
              const PlanLayout &L, hipStream_t s);
// The shared expert as extra tiles of the routed W13 stream launch (M = 0: none). Its tiles come
// before the plan's: tile t covers tokens 16t .. 16t+15. Its weights have the routed I and layout.
// Besides its h, the launch computes each token's gate sigma = 1 / (1 + e^-(x . gate)).
struct SharedW13 {
    const uint8_t *codes = nullptr, *scales = nullptr;  // one group: [2I][K/2], [2I][K/16]
    const float *gscale = nullptr;
    uint16_t *h = nullptr;           // [M][I] fp16
    const uint16_t *gate = nullptr;  // [K], 16-byte aligned
    float *sigma = nullptr;          // [M]
    int32_t M = 0;
};
// The plan built inside the W13 launch (ids == nullptr: read pv): block 0 writes it to `plan`.
constexpr int FUSED_PLAN_PAIRS = 256;     // one pair per thread of a W13 block
constexpr int FUSED_PLAN_EXPERTS = 1024;  // four experts per thread in the scans
// pair_major: W13 takes its rows straight from the ids, one pair per row tile (the pair-major
// small-batch path of the layer call); h is then written in pair order (row p = t*topk + k) and
// block 0 only builds and writes the plan.
struct FusedPlan {
    const int32_t *ids = nullptr;  // [M*topk]
    int32_t *plan = nullptr;
    PlanLayout L{};
    int32_t M = 0, E = 0;
    bool pair_major = false;
};
inline bool use_fused_plan(int64_t P, int32_t E) { return P <= FUSED_PLAN_PAIRS && E <= FUSED_PLAN_EXPERTS; }
int run_w13(const PlanView &pv, int64_t t_max, int32_t topk, const uint16_t *x, const nvfp4_weights &w,
            int32_t layout, uint16_t *h, hipStream_t s, SharedW13 shx = {}, FusedPlan fp = {});
// The shared expert's contribution to the MoE output (both pointers NULL: none): FP32 y [M][K] and
// the per-token gate sigma [M], added after the routed slots as one more fmaf.
struct SharedTerm {
    const float *y = nullptr;
    const float *sigma = nullptr;
};
// The shared expert as extra tiles of the routed W2 launch (M = 0: none): in the expert-major
// regime its tiles (first, as in SharedW13) write y, which the reduction adds with sigma; in the
// token-major regime it is one more slot, after the routed ones, with weight sigma.
struct SharedW2 {
    const uint8_t *codes = nullptr, *scales = nullptr;  // one group: [K][I/2], [K][I/16]
    const float *gscale = nullptr;
    const uint16_t *h = nullptr;  // [M][I] fp16
    float *y = nullptr;           // [M][K] FP32
    const float *sigma = nullptr; // [M]
    int32_t M = 0;
};

int run_w2(const PlanView &pv, int64_t t_max, int32_t M, int32_t topk, const uint16_t *h, const nvfp4_weights &w,
           const float *topk_weights, uint16_t *out, float *ws, hipStream_t s, SharedTerm sh = {},
           SharedW2 shw = {}, const int32_t *pair_ids = nullptr);
// Lets the dense kernels use the CU's whole LDS; idempotent, cheap after the first call on a device.
// Entry points that enqueue several launches call it before the first one.
int linear_prepare();
int run_linear(const uint16_t *x, int32_t M, const nvfp4_weights &w, uint16_t *y, hipStream_t s);
int run_linear_fp8(const uint16_t *x, int32_t M, const fp8_channel_weights &w, uint16_t *y, hipStream_t s);
int run_linear_swiglu(const uint16_t *x, int32_t M, const nvfp4_weights &w, int32_t layout, uint16_t *h,
                      hipStream_t s);
int run_w13_prefill(const PlanView &pv, int64_t a_max, int32_t M, int32_t topk, const uint16_t *x,
                    const nvfp4_weights &w, int32_t layout, uint16_t *h, hipStream_t s);
int run_w2_prefill(const PlanView &pv, int64_t a_max, int64_t P, const uint16_t *h, const nvfp4_weights &w, float *ws,
                   hipStream_t s);
// The prefill kernels address x, h and one expert's weights with 32-bit byte offsets.
bool prefill_offsets_fit(int64_t M, int64_t P, int32_t K, int32_t I);
int run_reduce(const PlanView &pv, int32_t M, int32_t topk, int32_t K, const float *topk_weights, const float *ws,
               uint16_t *out, hipStream_t s, SharedTerm sh = {});
int run_linear_f32(const uint16_t *x, int32_t M, const nvfp4_weights &w, float *y, hipStream_t s);
// Split-K forms with a workspace of linear_ws_bytes(M, w.rows, w.k) bytes (16-byte aligned).
size_t linear_ws_bytes(int32_t M, int32_t N, int32_t K);
int run_linear_split(const uint16_t *x, int32_t M, const nvfp4_weights &w, uint16_t *y, void *ws, hipStream_t s);
int run_linear_swiglu_split(const uint16_t *x, int32_t M, const nvfp4_weights &w, int32_t layout, uint16_t *h,
                            void *ws, hipStream_t s);
int run_shared_gate(const uint16_t *x, int32_t M, int32_t K, const uint16_t *g, float *sigma, hipStream_t s);

// Regime switch (performance only: every kernel uses the same reduction order, so results are
// bitwise identical either way). The MFMA-tiled prefill kernels pay off once experts average at
// least 16 pairs, i.e. M*topk >= 16*E; below that the streaming kernels win. They also need every
// byte offset to fit in 31 bits; larger problems stay on the streaming kernels.
// Small batches run W2 token-major with the slot reduction fused (one block per token and 16
// output rows). Each pair then reads its expert's rows itself, so this pays while pairs rarely
// share an expert. Measured on MI355X at E=512, top-10 (W2 + reduce, µs, token-major vs
// expert-major): M=2 8.3 vs 14.6, M=8 19.2 vs 22.0, M=12 22.8 vs 26.4, M=16 30.2 vs 28.8; hence
// P <= E/4.
#ifndef NVFP4_TOKEN_W2_DIV
#define NVFP4_TOKEN_W2_DIV 4
#endif
inline bool use_token_w2(int64_t P, int32_t E) { return NVFP4_TOKEN_W2_DIV * P <= (int64_t)E; }
// The layer call's pair-major path: W13 one pair per row tile straight from the ids, h in pair
// order, token-major W2 reading the ids and that h (no plan lookup on the critical path). Needs the
// token-major regime and a plan that one W13 block can build.
inline bool use_pair_major(int64_t P, int32_t E) { return use_token_w2(P, E) && use_fused_plan(P, E); }

inline bool use_prefill(int64_t M, int64_t P, int32_t E, int32_t K, int32_t I)
{
    return P >= 16 * (int64_t)E && prefill_offsets_fit(M, P, K, I);
}

}  // namespace nvfp4
