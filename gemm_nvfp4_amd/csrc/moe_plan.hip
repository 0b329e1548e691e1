// moe_plan.hip -- routing plan: top-k id histogram, prefix-sum expert bucketing and a stable
// scatter into bucket order. W13 and W2 both reuse this integer plan, so planning happens once per
// layer (the grouped W2 takes W13's plan instead of planning again: "[Kernel][SM70] Improve Qwen3.8
// no-MTP concurrency", "Scope and related PRs").
//
// The plan is a stable counting sort of the valid (token, slot) pairs by expert; ties keep
// ascending pair index p = t*topk + k. That makes it unique, and every path below produces it
// bit-exactly.
//   - Small path, P <= 1024 pairs (the decode regime): one 1024-thread block builds everything
//     in LDS in one launch. A pair takes a ticket in its expert's group while counting; once the
//     offsets are known, the group's pairs are listed and each pair's stable rank is the number
//     of group members with a smaller index.
//   - Large path (prefill): pairs are cut into chunks of 256, each with its own expert histogram.
//     A per-expert scan over chunks gives every (expert, chunk) its start. Within a chunk a
//     pair's rank counts the earlier pairs of the same expert, so the scatter is stable with no
//     atomics on positions. Four launches, none of which is serial over the pairs.
//
// The router (top-k selection and softmax weights from router logits) runs one wave per token. At
// decode sizes it shares the small path's block, so routing and planning are one launch.
#include "internal.hpp"
#include "plan_device.hpp"

namespace nvfp4 {
namespace {

// Exclusive scan of one int per thread over a block of nwaves*64 threads. `wsum` is LDS scratch
// of at least nwaves ints. Ends with a barrier, so `wsum` can be reused at once.
__device__ __forceinline__ int block_excl_scan(int v, int *wsum, int nwaves, int *total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int pre = 0, tot = 0;
    for (int w = 0; w < nwaves; ++w) {
        const int s = wsum[w];
        pre += (w < wid) ? s : 0;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return pre + incl - v;
}

// Stable rank of this thread's pair among the block's earlier pairs: how many of ids4[0 .. tid)
// equal `id` (id >= 0). ids4 holds the block's ids, four per int4, padded to the wave's end with
// values that match no id. The loop bound is uniform per wave and eight 16-byte LDS reads are in
// flight at a time (every lane reads the same address: a broadcast).
__device__ __forceinline__ int stable_rank(const int4 *ids4, int tid, int id)
{
    const int n4 = ((tid | 63) + 1) >> 2;
    int rank = 0;
#pragma unroll 8
    for (int j4 = 0; j4 < n4; ++j4) {
        const int4 v = ids4[j4];
        const int j = 4 * j4;
        rank += (v.x == id && j < tid) + (v.y == id && j + 1 < tid) + (v.z == id && j + 2 < tid) +
                (v.w == id && j + 3 < tid);
    }
    return rank;
}

// Writes counts, offsets, the active list, the row-tile lists (expert, first row, first bucket row,
// row count) and header words 0,1,3 from per-expert counts `cnt` (LDS or global). Also leaves offsets in `off_lds` (E+1 ints of LDS) and
// each expert's first tile index in `tile_first` (E ints, LDS or global) for the caller. Runs on a
// 1024-thread block; E <= 4096, so each thread owns up to 4 consecutive experts.
__device__ void build_lists(const int *cnt, int E, int32_t *plan, const PlanLayout &L, int *off_lds, int *tile_first,
                            int *wsum)
{
    const int ept = (E + 1023) / 1024;
    const int e0 = threadIdx.x * ept;
    int c[4];
    int3 sums{0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = e0 + i;
        c[i] = (i < ept && e < E) ? cnt[e] : 0;
        sums.x += c[i];
        sums.y += c[i] > 0;
        sums.z += (c[i] + PLAN_TILE_ROWS - 1) / PLAN_TILE_ROWS;
    }
    int3 tot;
    const int3 pre = block_excl_scan3<16>(sums, wsum, &tot);
    write_expert_lists(plan, L, e0, min(ept, E - e0), c, pre.x, pre.y, pre.z, off_lds, tile_first);
    if (threadIdx.x == 0) {
        write_totals(plan, L, E, tot);
        off_lds[E] = tot.x;
    }
}

// ---- small path: P <= 1024, one block -----------------------------------------------------------
// The whole plan from one 1024-thread block; thread p holds pair p's raw id (-1 past P).
__device__ void plan_small_body(int raw, int M, int topk, int E, int32_t *__restrict__ plan, const PlanLayout &L)
{
    __shared__ int cnt[MAX_EXPERTS];
    __shared__ int off[MAX_EXPERTS + 1];
    __shared__ int first[MAX_EXPERTS];
    __shared__ int slot[SMALL_PLAN_PAIRS];
    __shared__ int wsum[48];
    __shared__ int bad;
    const int tid = threadIdx.x;
    const int P = (int)L.P;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    // Count, and take a ticket inside the expert's group (arrival order, not yet stable).
    int id = -1, ticket = 0;
    if (tid < P) {
        if (raw >= 0 && raw < E) {
            id = raw;
            ticket = atomicAdd(&cnt[raw], 1);
        } else if (raw != -1) {
            atomicAdd(&bad, 1);
        }
    }
    __syncthreads();
    build_lists(cnt, E, plan, L, off, first, wsum);
    __syncthreads();
    if (id >= 0) slot[off[id] + ticket] = tid;  // the group's pairs, in arrival order
    __syncthreads();
    if (tid < P) {
        if (id >= 0) {
            // Stable rank: pairs of the same group with a smaller index (groups are small at decode).
            const int o = off[id], n = cnt[id];
            int rank = 0;
            for (int i = 0; i < n; ++i) rank += slot[o + i] < tid;
            place_pair(plan, L, tid, id, o + rank, rank, first[id]);
        } else {
            plan[L.pos_of_pair + tid] = -1;
            plan[L.pair_expert + tid] = -1;
        }
    }
    if (tid == 0) write_header_tail(plan, L, bad, M, topk, E);
}

__global__ __launch_bounds__(1024) void plan_small_kernel(const int32_t *__restrict__ ids, int M, int topk, int E,
                                                          int32_t *__restrict__ plan, PlanLayout L)
{
    const int raw = (int)threadIdx.x < L.P ? ids[threadIdx.x] : -1;  // issued first: the only load of the kernel
    plan_small_body(raw, M, topk, E, plan, L);
}

// ---- router ---------------------------------------------------------------------------------------
// Top-k routing from FP32 router logits (the "router" that the "[Kernel][SM70] Improve Qwen3.8
// no-MTP concurrency" page lists among the fused MoE parts, "Scope and related PRs"; the pages give
// no formula, and this is the plain reading): a token takes the experts of its topk largest
// logits, largest first; equal logits (+0 and -0 are equal) go in ascending expert order; NaN
// ranks below every number. The slot weights are the softmax of the selected logits,
// exp(l_k - l_0) / sum_j exp(l_j - l_0) in FP32, l_0 the largest selected logit.
//
// One wave per token. Each logit becomes a unique 64-bit key: an order-preserving 32-bit image of
// the value (NaN lowest) above the complemented expert id, so equal values put the lower expert
// higher. Round r takes the wave's largest key below round r-1's winner: nothing is ever removed
// and every round is one pass over the lane's registers plus a six-step butterfly.
__device__ __forceinline__ uint64_t route_key(float x, int e)
{
    const uint32_t b = __float_as_uint(x == 0.0f ? 0.0f : x);  // -0 and +0 get one image
    uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);   // ascending with the value
    if (x != x) k = 0;                                          // NaN below -inf
    return ((uint64_t)k << 32) | (uint64_t)(~(uint32_t)e);
}

// Wave-wide reductions on the DPP crossbar (no LDS round trips): pairs, quads, half rows and rows
// combine with quad_perm / row mirrors, then row broadcasts 15 and 31 carry rows 0-1 and 0-2 up,
// so lane 63 ends with the whole wave's result. Lanes a step leaves without a source take the
// identity. The combining tree is fixed, so a floating-point sum is reproducible.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t identity)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROWS, 0xf, false);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t max_step(uint64_t v)
{
    const uint64_t o = ((uint64_t)dpp_u32<CTRL, ROWS>((uint32_t)(v >> 32), 0u) << 32) | dpp_u32<CTRL, ROWS>((uint32_t)v, 0u);
    return o > v ? o : v;
}

template <int CTRL, int ROWS>
__device__ __forceinline__ float add_step(float v)
{
    return v + __uint_as_float(dpp_u32<CTRL, ROWS>(__float_as_uint(v), 0u));
}

// Largest 64-bit key of the wave, in every lane (0 is the identity: below every real key).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    v = max_step<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]
    v = max_step<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]
    v = max_step<0x141, 0xf>(v);  // row_half_mirror
    v = max_step<0x140, 0xf>(v);  // row_mirror: every lane holds its row's maximum
    v = max_step<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = max_step<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63), hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Sum over the wave in a fixed order, in every lane.
__device__ __forceinline__ float wave_sum_f32(float v)
{
    v = add_step<0xB1, 0xf>(v);
    v = add_step<0x4E, 0xf>(v);
    v = add_step<0x141, 0xf>(v);
    v = add_step<0x140, 0xf>(v);
    v = add_step<0x142, 0xa>(v);
    v = add_step<0x143, 0xc>(v);
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// Routes token row `lg` (E <= 64*NPL logits, 1 <= topk <= min(E, 32)). Lane k < topk ends with
// the expert and weight of slot k.
template <int NPL>
__device__ __forceinline__ void route_token(const float *__restrict__ lg, int E, int topk, int &id, float &w)
{
    const int lane = threadIdx.x & 63;
    uint64_t c[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        c[i] = e < E ? route_key(lg[e], e) : 0;  // 0 is below every real key
    }
    uint64_t thr = ~0ull, mine = 0;
    for (int r = 0; r < topk; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < NPL; ++i) best = (c[i] < thr && c[i] > best) ? c[i] : best;
        thr = wave_max_u64(best);
        if (lane == r) mine = thr;
    }
    // The slot's expert and logit come back from its key: the low word is the complemented
    // expert; the high word inverts to the value (+0 for either zero, NaN for key 0), which gives
    // the same exponentials as the logit itself.
    id = (int)~(uint32_t)mine;
    const uint32_t k = (uint32_t)(mine >> 32);
    const float x = k == 0 ? __uint_as_float(0x7fc00000u) : __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
    const float l0 = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 0));
    const float ev = lane < topk ? expf(x - l0) : 0.0f;
    w = ev / wave_sum_f32(ev);  // one sum for every slot
}

// Many tokens: one wave per token, four per block.
template <int NPL>
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int M, int E, int topk,
                                                    int32_t *__restrict__ ids, float *__restrict__ weights)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (t >= M) return;  // wave-uniform
    int id;
    float w;
    route_token<NPL>(logits + (size_t)t * E, E, topk, id, w);
    if (lane < topk) {
        ids[(size_t)t * topk + lane] = id;
        weights[(size_t)t * topk + lane] = w;
    }
}

// Decode sizes (M*topk <= 1024, E <= 1024): the sixteen waves route the tokens, the ids meet in
// LDS, and the same block builds the plan.
template <int NPL>
__global__ __launch_bounds__(1024) void route_plan_small_kernel(const float *__restrict__ logits, int M, int E,
                                                                int topk, int32_t *__restrict__ ids,
                                                                float *__restrict__ weights,
                                                                int32_t *__restrict__ plan, PlanLayout L)
{
    __shared__ int s_ids[SMALL_PLAN_PAIRS];
    const int lane = threadIdx.x & 63;
    for (int t = threadIdx.x >> 6; t < M; t += 16) {  // wave-uniform loop
        int id;
        float w;
        route_token<NPL>(logits + (size_t)t * E, E, topk, id, w);
        if (lane < topk) {
            ids[t * topk + lane] = id;
            weights[t * topk + lane] = w;
            s_ids[t * topk + lane] = id;
        }
    }
    __syncthreads();
    plan_small_body((int)threadIdx.x < L.P ? s_ids[threadIdx.x] : -1, M, topk, E, plan, L);
}

// ---- large path ---------------------------------------------------------------------------------
// 1) per-chunk histograms hist[e][g] and bad-id counts badc[g].
__global__ __launch_bounds__(PLAN_CHUNK) void plan_hist_kernel(const int32_t *__restrict__ ids, int E,
                                                               int32_t *__restrict__ plan, PlanLayout L)
{
    __shared__ int cnt[MAX_EXPERTS];
    __shared__ int bad;
    const int g = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < E; e += PLAN_CHUNK) cnt[e] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    const int64_t p = (int64_t)g * PLAN_CHUNK + tid;
    if (p < L.P) {
        const int raw = ids[p];
        if (raw >= 0 && raw < E) atomicAdd(&cnt[raw], 1);
        else if (raw != -1) atomicAdd(&bad, 1);
    }
    __syncthreads();
    int32_t *hist = plan + L.hist;
    for (int e = tid; e < E; e += PLAN_CHUNK) hist[(int64_t)e * L.G + g] = cnt[e];
    if (tid == 0) plan[L.badc + g] = bad;
}

// 2) one wave per expert: hist[e][g] becomes the exclusive prefix over chunks; counts[e] = total.
__global__ __launch_bounds__(256) void plan_scan_chunks_kernel(int E, int32_t *__restrict__ plan, PlanLayout L)
{
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (e >= E) return;
    int32_t *row = plan + L.hist + (int64_t)e * L.G;
    int running = 0;
    for (int64_t g0 = 0; g0 < L.G; g0 += 64) {
        const bool in = g0 + lane < L.G;
        const int v = in ? row[g0 + lane] : 0;
        const int incl = wave_incl_scan(v);
        if (in) row[g0 + lane] = running + incl - v;
        running += __shfl(incl, 63, 64);
    }
    if (lane == 0) plan[L.counts + e] = running;
}

// 3) one block: offsets, active list, tiles and the header. The same words as build_lists, but the
//    row tiles (thousands at prefill sizes) are written tile-parallel: tile t finds its expert by
//    binary search over the tile starts, so a wave's stores are contiguous.
__global__ __launch_bounds__(1024) void plan_lists_kernel(int M, int topk, int E, int32_t *__restrict__ plan, PlanLayout L)
{
    __shared__ int off[MAX_EXPERTS + 1];
    __shared__ int tfirst[MAX_EXPERTS + 1];
    __shared__ int wsum[48];
    __shared__ int cnt[MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += 1024) cnt[e] = plan[L.counts + e];
    int bad = 0;
    for (int64_t g = threadIdx.x; g < L.G; g += 1024) bad += plan[L.badc + g];
    __syncthreads();
    const int ept = (E + 1023) / 1024, e0 = threadIdx.x * ept, ne = min(ept, E - e0);
    int c[4];
    int3 sums{0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c[i] = i < ne ? cnt[e0 + i] : 0;
        sums.x += c[i];
        sums.y += c[i] > 0;
        sums.z += (c[i] + PLAN_TILE_ROWS - 1) / PLAN_TILE_ROWS;
    }
    int3 tot;
    const int3 pre = block_excl_scan3<16>(sums, wsum, &tot);
    {
        int cpre = pre.x, apre = pre.y, tpre = pre.z;
        int32_t *counts = plan + L.counts, *offsets = plan + L.offsets, *active = plan + L.active;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= ne) continue;
            const int e = e0 + i;
            counts[e] = c[i];
            offsets[e] = cpre;
            off[e] = cpre;
            plan[L.tile_first + e] = tpre;
            tfirst[e] = tpre;
            if (c[i] > 0) active[apre++] = e;
            cpre += c[i];
            tpre += (c[i] + PLAN_TILE_ROWS - 1) / PLAN_TILE_ROWS;
        }
    }
    if (threadIdx.x == 0) {
        write_totals(plan, L, E, tot);
        off[E] = tot.x;
        tfirst[E] = tot.z;
    }
    __syncthreads();
    int32_t *tile_e = plan + L.tile_expert, *tile_r = plan + L.tile_row0, *tile_b = plan + L.tile_base;
    int32_t *tile_n = plan + L.tile_rows;
    for (int t = threadIdx.x; t < tot.z; t += 1024) {
        // the last expert whose first tile is <= t: experts without tiles have empty ranges
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tfirst[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int r = (t - tfirst[lo]) * PLAN_TILE_ROWS;
        tile_e[t] = lo;
        tile_r[t] = r;
        tile_b[t] = off[lo] + r;
        tile_n[t] = min(PLAN_TILE_ROWS, cnt[lo] - r);
    }
    int total_bad;
    block_excl_scan(bad, wsum, 16, &total_bad);
    if (threadIdx.x == 0) write_header_tail(plan, L, total_bad, M, topk, E);
}

// 4) stable scatter: position = offsets[e] + chunk prefix[e][g] + rank among the chunk's earlier
//    pairs of expert e.
__global__ __launch_bounds__(PLAN_CHUNK) void plan_scatter_kernel(const int32_t *__restrict__ ids, int E,
                                                                  int32_t *__restrict__ plan, PlanLayout L)
{
    __shared__ __attribute__((aligned(16))) int id_s[PLAN_CHUNK];
    const int g = blockIdx.x, tid = threadIdx.x;
    const int64_t p = (int64_t)g * PLAN_CHUNK + tid;
    int id = -1;
    if (p < L.P) {
        const int raw = ids[p];
        id = (raw >= 0 && raw < E) ? raw : -1;
    }
    id_s[tid] = id;
    __syncthreads();
    if (p >= L.P) return;
    if (id < 0) {
        plan[L.pos_of_pair + p] = -1;
        plan[L.pair_expert + p] = -1;
        return;
    }
    const int rank = stable_rank(reinterpret_cast<const int4 *>(id_s), tid, id);
    const int before = plan[L.hist + (int64_t)id * L.G + g] + rank;  // earlier pairs of expert id
    place_pair(plan, L, p, id, plan[L.offsets + id] + before, before, plan[L.tile_first + id]);
}

int route_npl(int E)
{
    int npl = 1;
    while (64 * npl < E) npl *= 2;
    return npl;
}

}  // namespace

int run_route(const float *logits, int32_t M, int32_t E, int32_t topk, int32_t *ids, float *weights, int32_t *plan,
              const PlanLayout &L, hipStream_t s)
{
    const int npl = route_npl(E);
    if (L.P <= SMALL_PLAN_PAIRS && npl <= 16) {  // the block's 128 registers per lane hold 16 keys per lane
#define NVFP4_ROUTE_SMALL(N) \
    case N: return launch(route_plan_small_kernel<N>, dim3(1), dim3(1024), 0, s, logits, M, E, topk, ids, weights, plan, L);
        switch (npl) {
            NVFP4_ROUTE_SMALL(1) NVFP4_ROUTE_SMALL(2) NVFP4_ROUTE_SMALL(4) NVFP4_ROUTE_SMALL(8)
            NVFP4_ROUTE_SMALL(16)
        default: return NVFP4_ERR_UNSUPPORTED;
        }
#undef NVFP4_ROUTE_SMALL
    }
    const dim3 grid((unsigned)(((int64_t)M + 3) / 4)), block(256);
    int st;
#define NVFP4_ROUTE(N) \
    case N: st = launch(route_kernel<N>, grid, block, 0, s, logits, M, E, topk, ids, weights); break;
    switch (npl) {
        NVFP4_ROUTE(1) NVFP4_ROUTE(2) NVFP4_ROUTE(4) NVFP4_ROUTE(8) NVFP4_ROUTE(16) NVFP4_ROUTE(32) NVFP4_ROUTE(64)
    default: return NVFP4_ERR_UNSUPPORTED;
    }
#undef NVFP4_ROUTE
    if (st != NVFP4_OK) return st;
    return run_plan(ids, M, topk, E, plan, L, s);
}

int run_plan(const int32_t *ids, int32_t M, int32_t topk, int32_t E, int32_t *plan, const PlanLayout &L, hipStream_t s)
{
    if (L.P <= SMALL_PLAN_PAIRS)
        return launch(plan_small_kernel, dim3(1), dim3(1024), 0, s, ids, M, topk, E, plan, L);
    const unsigned G = (unsigned)L.G;
    int st = launch(plan_hist_kernel, dim3(G), dim3(PLAN_CHUNK), 0, s, ids, E, plan, L);
    if (st == NVFP4_OK) st = launch(plan_scan_chunks_kernel, dim3((E + 3) / 4), dim3(256), 0, s, E, plan, L);
    if (st == NVFP4_OK) st = launch(plan_lists_kernel, dim3(1), dim3(1024), 0, s, M, topk, E, plan, L);
    if (st == NVFP4_OK) st = launch(plan_scatter_kernel, dim3(G), dim3(PLAN_CHUNK), 0, s, ids, E, plan, L);
    return st;
}

}  // namespace nvfp4
