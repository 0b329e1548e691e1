// stream_schedule.hpp -- how the streaming MoE kernels (moe_gemm.hip) deal their work units to a
// persistent grid. Plain functions of the unit count, the grid size and the block index, so that
// the kernels and a host-side checker (tests/stream_schedule_check.cpp) run the same code.
//
// A work unit is (row tile of the plan, a group of 16-row weight tiles); units are numbered
// tile-major, upt units per row tile. Each block takes one contiguous unit range and stages the
// row tiles it touches in LDS (at most MAX_RANGE_TILES of them).
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define NVFP4_SCHED_FN __host__ __device__ __forceinline__
#else
#define NVFP4_SCHED_FN inline
#endif

// The first `first` blocks are the first resident block of each CU. With two blocks per CU, the
// second block's first loads queue behind the first block's first unit and its prefetch, so it
// runs about 1.7 units behind for the whole kernel (measured on MI355X at 16 tokens: first units
// done at 7.5 vs 12.2 us, ends at 27.7 vs 34.0 us). First blocks therefore take weight FIRST_W and
// second ones SECOND_W (13 : 7 was the fastest of 11 : 9 to 14 : 6 for W13 at 16 tokens: 36.8 vs
// 38.1 us with an equal split). Only while there are at most two blocks per CU and more units than
// blocks; otherwise the split is equal (with U <= G every block has at most one unit anyway).
#ifndef NVFP4_FIRST_W
#define NVFP4_FIRST_W 13
#endif
#ifndef NVFP4_SECOND_W
#define NVFP4_SECOND_W 7
#endif

namespace nvfp4 {
namespace sched {

constexpr int MAX_RANGE_TILES = 16;  // row tiles a block's unit range may touch
constexpr int FIRST_W = NVFP4_FIRST_W, SECOND_W = NVFP4_SECOND_W;

// Contiguous unit range [u0, u1) of block b of G out of U units; returns false if it is empty.
// The hardware deals block ids to the 8 XCDs round-robin. Within each group of blocks (first,
// second) the ranges are laid out XCD-major (the blocks of one XCD get consecutive ranges), so
// that the rounding of U / G to whole units does not fall on the same XCDs every time (an equal
// split at U/G = 8.5 gave every odd XCD 9 units per block and every even one 8).
NVFP4_SCHED_FN bool unit_range(int64_t U, int first, int G, int b, int64_t &u0, int64_t &u1)
{
    const int nA = first < G ? first : G, nB = G - nA;
    const bool weighted = nB > 0 && nB <= nA && U > G;
    const int wa = weighted ? FIRST_W : 1, wb = weighted ? SECOND_W : 1;
    const bool in_a = b < nA;
    const int n = in_a ? nA : nB, i = in_a ? b : b - nA, w = in_a ? wa : wb;
    const int L = (n & 7) == 0 ? (i & 7) * (n >> 3) + (i >> 3) : i;
    const int64_t W0 = (in_a ? 0 : (int64_t)nA * wa) + (int64_t)L * w;
    const int64_t Wt = (int64_t)nA * wa + (int64_t)nB * wb;
    u0 = U * W0 / Wt;
    u1 = U * (W0 + w) / Wt;
    return u0 < u1;
}

// First row tile of a non-empty range and the number of row tiles it touches.
NVFP4_SCHED_FN int range_first_tile(int64_t u0, int upt) { return (int)(u0 / upt); }
NVFP4_SCHED_FN int range_tiles(int64_t u0, int64_t u1, int upt) { return (int)((u1 - 1) / upt) - (int)(u0 / upt) + 1; }

// Persistent grid: `occ` 256-thread blocks per CU, never more blocks than units, and enough
// blocks that no block's range touches more than MAX_RANGE_TILES row tiles. With the weighted
// split (only while G <= 2 * first) a block gets at most 2*13/20 U/G + 1 units, i.e. at most
// 1.3 t_max/G + 3 row tiles, so G >= t_max / 10 keeps that within 16 (the host-side checker
// sweeps t_max up to 60000, 1..32 units per tile, 8..304 CUs and both occupancies).
NVFP4_SCHED_FN int grid_blocks(int occ, int cus, int64_t units_max, int64_t t_max)
{
    static_assert(MAX_RANGE_TILES == 16, "the bound above assumes 16 staged row tiles");
    int64_t g = occ * (int64_t)cus;
    const int64_t g_min = (t_max + 9) / 10;
    if (g < g_min) g = g_min;
    if (g > units_max) g = units_max;
    return (int)(g > 0 ? g : 1);
}

// The number of blocks that come first on their CU, given the grid.
NVFP4_SCHED_FN int first_blocks(int occ, int cus, int G) { return occ > 1 ? cus : G; }

}  // namespace sched
}  // namespace nvfp4
