// Host-side check of the streaming kernels' work split (gemm_nvfp4_amd/csrc/stream_schedule.hpp),
// built with g++ and run by test_stream_schedule.py. The kernels include the same header. Over a
// sweep of CU counts (8..304), blocks per CU (1, 2), units per row tile (1..32), row-tile counts
// up to 60000, and tile counts below what the grid was sized for (the device-side count is only
// bounded on the host), and for the pair-major W13 launch's unit blocks as well, it checks:
//   * the grid has at least one block and never more blocks than units;
//   * the blocks' ranges are disjoint and cover every unit of [0, U) exactly once;
//   * every range touches at most MAX_RANGE_TILES row tiles, so each unit's staged slot
//     (its tile minus the range's first tile) stays inside the LDS staging arrays.
// Prints "ok <launches> <blocks>" and exits 0, or prints the first failure and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "stream_schedule.hpp"

using namespace nvfp4::sched;

namespace {

int fail(const char *what, int64_t a, int64_t b, int64_t c)
{
    std::printf("FAIL %s (%lld %lld %lld)\n", what, (long long)a, (long long)b, (long long)c);
    std::exit(1);
}

int64_t launches = 0, blocks_seen = 0;

// One launch: G blocks over U = T * upt units; with `cover`, every unit is also marked.
void check_launch(int64_t T, int upt, int G, int first, bool cover)
{
    ++launches;
    const int64_t U = T * upt;
    int64_t total = 0;
    std::vector<uint8_t> seen(cover ? (size_t)U : 0, 0);
    for (int b = 0; b < G; ++b) {
        ++blocks_seen;
        int64_t u0 = 0, u1 = 0;
        if (!unit_range(U, first, G, b, u0, u1)) continue;
        if (u0 < 0 || u1 > U || u0 >= u1) fail("range outside [0, U)", u0, u1, U);
        const int t0 = range_first_tile(u0, upt), nt = range_tiles(u0, u1, upt);
        if (nt < 1 || nt > MAX_RANGE_TILES) fail("range touches too many row tiles", nt, T, G);
        if ((int)((u1 - 1) / upt) - t0 >= MAX_RANGE_TILES) fail("slot outside the staging", u1, t0, upt);
        if (cover)
            for (int64_t u = u0; u < u1; ++u)
                if (seen[(size_t)u]++) fail("unit in two ranges", u, U, G);
        total += u1 - u0;
    }
    if (total != U) fail("ranges do not add up to U", total, U, G);
    if (cover)
        for (int64_t u = 0; u < U; ++u)
            if (seen[(size_t)u] != 1) fail("unit in no range", u, U, G);
}

}  // namespace

int main()
{
    const int cus_list[] = {8, 80, 136, 256, 304};
    for (int cus : cus_list)
        for (int occ = 1; occ <= 2; ++occ)
            for (int upt : {1, 2, 3, 5, 8, 13, 16, 24, 31, 32})
                for (int64_t t_max = 1; t_max <= 60000; t_max += (t_max < 400 ? 1 : 173)) {
                    const int G = grid_blocks(occ, cus, t_max * upt, t_max);
                    if (G < 1 || G > t_max * upt) fail("grid size", G, t_max * upt, cus);
                    const int first = first_blocks(occ, cus, G);
                    const bool cover = t_max * upt <= 20000;
                    check_launch(t_max, upt, G, first, cover);
                    // the pair-major W13 launch: block 0 builds the plan, one unit block fewer
                    // when that keeps every block resident
                    int Gp = G;
                    if (Gp == occ * cus && Gp > 1 && Gp - 1 >= (t_max + 9) / 10) --Gp;
                    check_launch(t_max, upt, Gp, first_blocks(occ, cus, Gp + 1), cover);
                    // the device-side tile count below the bound the grid was sized for
                    if (t_max > 1) check_launch((t_max * 3) / 4, upt, G, first, cover);
                    if (t_max > 2) check_launch(1, upt, G, first, cover);
                }
    std::printf("ok %lld %lld\n", (long long)launches, (long long)blocks_seen);
    return 0;
}
