// plan_device.hpp -- device-side pieces of the routing plan shared by the plan kernels
// (moe_plan.hip) and the W13 launch that builds its own plan (moe_gemm.hip): block scans and
// the writers of the plan's documented arrays (layout: PlanLayout in internal.hpp).
//
// The plan is a stable counting sort of the valid (token, slot) pairs by expert, ties by
// ascending pair index p = t*topk + k: the one integer plan that W13 and the grouped W2 share
// ("[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency", "Scope and related PRs"). Every writer
// below produces the same words, so every path gives the same plan bit for bit.
#pragma once

#include "internal.hpp"

namespace nvfp4 {

// Inclusive scan of one int across a wave64.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
    }
    return v;
}

// Three exclusive scans at once over a block of NW waves (one pair of barriers). `wsum` is LDS
// scratch of at least 3*NW ints.
template <int NW>
__device__ __forceinline__ int3 block_excl_scan3(int3 v, int *wsum, int3 *total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int ix = wave_incl_scan(v.x), iy = wave_incl_scan(v.y), iz = wave_incl_scan(v.z);
    if (lane == 63) {
        wsum[wid] = ix;
        wsum[NW + wid] = iy;
        wsum[2 * NW + wid] = iz;
    }
    __syncthreads();
    int3 pre{0, 0, 0}, tot{0, 0, 0};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int sx = wsum[w], sy = wsum[NW + w], sz = wsum[2 * NW + w];
        if (w < wid) {
            pre.x += sx;
            pre.y += sy;
            pre.z += sz;
        }
        tot.x += sx;
        tot.y += sy;
        tot.z += sz;
    }
    __syncthreads();
    *total = tot;
    return int3{pre.x + ix - v.x, pre.y + iy - v.y, pre.z + iz - v.z};
}

// Per-expert lists for a thread's consecutive experts e0 .. e0+n-1 with counts c[]: counts,
// offsets, the active list and the row tiles (expert, first row, first bucket row, row count).
// cpre/apre/tpre are the exclusive prefix sums of counts, active flags and tile counts at e0.
// Also records each expert's offset and first tile in off_out / tile_first (LDS or global).
template <int N>
__device__ __forceinline__ void write_expert_lists(int32_t *plan, const PlanLayout &L, int e0, int n, const int (&c)[N],
                                                   int cpre, int apre, int tpre, int *off_out, int *tile_first)
{
    int32_t *counts = plan + L.counts, *offsets = plan + L.offsets, *active = plan + L.active;
    int32_t *tile_e = plan + L.tile_expert, *tile_r = plan + L.tile_row0, *tile_b = plan + L.tile_base;
    int32_t *tile_n = plan + L.tile_rows;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i >= n) continue;
        const int e = e0 + i;
        counts[e] = c[i];
        offsets[e] = cpre;
        off_out[e] = cpre;
        tile_first[e] = tpre;
        if (c[i] > 0) {
            active[apre++] = e;
            for (int r = 0; r < c[i]; r += PLAN_TILE_ROWS) {
                tile_e[tpre] = e;
                tile_r[tpre] = r;
                tile_b[tpre] = cpre + r;
                tile_n[tpre] = min(PLAN_TILE_ROWS, c[i] - r);
                ++tpre;
            }
        }
        cpre += c[i];
    }
}

// Header words 0, 1, 3 (valid pairs, active experts, row tiles) and the offsets' end.
__device__ __forceinline__ void write_totals(int32_t *plan, const PlanLayout &L, int E, int3 tot)
{
    plan[L.offsets + E] = tot.x;
    int32_t *hdr = plan + L.hdr;
    hdr[0] = tot.x;
    hdr[1] = tot.y;
    hdr[3] = tot.z;
}

// Records a valid pair's place: sorted_pair, pos_of_pair, its expert and its row in its tile's pair
// list.
__device__ __forceinline__ void place_pair(int32_t *plan, const PlanLayout &L, int64_t p, int e, int pos,
                                           int row_in_expert, int first_tile)
{
    plan[L.sorted_pair + pos] = (int32_t)p;
    plan[L.pos_of_pair + p] = pos;
    plan[L.pair_expert + p] = e;
    const int64_t t = first_tile + row_in_expert / PLAN_TILE_ROWS;
    plan[L.tile_pair + t * PLAN_TILE_ROWS + row_in_expert % PLAN_TILE_ROWS] = (int32_t)p;
}

__device__ __forceinline__ void write_header_tail(int32_t *plan, const PlanLayout &L, int n_bad, int M, int topk, int E)
{
    int32_t *hdr = plan + L.hdr;
    hdr[2] = n_bad;
    hdr[4] = M;
    hdr[5] = topk;
    hdr[6] = E;
    hdr[7] = PLAN_TILE_ROWS;
}

}  // namespace nvfp4
