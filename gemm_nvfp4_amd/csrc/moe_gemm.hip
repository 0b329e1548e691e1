// moe_gemm.hip -- grouped expert GEMMs of the MoE layer, decode (streaming) regime.
//   W13 with fused SwiGLU (an expert-grouped W13 over several rows with SiLU in its epilogue and
//   the reduction axis split inside a block), then W2 with the top-k-weighted reduction fused in
//   (W2 reads the plan W13 used), as listed on the "[Kernel][SM70] Improve Qwen3.8 no-MTP
//   concurrency" page, "Scope and related PRs".
//
// At small M the layer reads every active expert's packed weights once and does little math on
// them. It is bound by HBM bandwidth, so the design goal is many bytes in flight per CU. On
// MI355X that works best with many resident waves each holding one unit's loads (measured: deeper
// per-wave prefetch lowers the achieved read rate). gfx950 design:
//   * Work unit: (row tile of the plan, a group of 16-row weight tiles). A row tile has at most
//     16 bucket rows (pairs) of one expert. Units are numbered tile-major and cut into contiguous
//     ranges, one per persistent block (W13: two 256-thread blocks per CU; W2: one), weighted so
//     that blocks that start late get fewer units (stream_schedule.hpp). Blocks past the
//     device-side unit count leave at once, so no device-to-host read is ever needed.
//   * Block start: the block stages its range's tile descriptors from the plan (expert, rows, first
//     bucket row, activation row of each row) in LDS: one load after the tile count.
//   * Inside a block the four waves split the reduction axis into its 512-element chunks
//     (intra-block split-K) when there are several. Otherwise each takes its own tiles. A wave
//     always owns two 16-row weight tiles: W13's gate and up rows of one 16-wide i slice, or two
//     W2 output tiles. Per unit it loads its packed weights (per row and lane: four 16-byte code
//     loads and one 8-byte scale load), decodes them to fp16 and runs the MFMA chain against A
//     fragments held in registers. The A fragments (its chunk of the tile's rows of x for W13, or
//     of h for W2) are read from global memory, where they are L2-resident, only when the tile
//     changes.
//   * Chunk partials meet in LDS and are added in chunk order: the library-wide reduction order
//     of nvfp4_device.hpp. The epilogue applies the FP32 global scale, then SwiGLU (W13) or
//     stores per-pair FP32 results (W2).
//   * A last pass sums each token's slots in slot order with fmaf and rounds to fp16 once.
#include "internal.hpp"
#include "nvfp4_device.hpp"
#include "plan_device.hpp"
#include "stream_schedule.hpp"

namespace nvfp4 {
namespace {

constexpr int LDS_ROW = 20;  // padded row of 16 floats: rows 4 apart land on different banks
using sched::MAX_RANGE_TILES;

// Per-block staging of the row tiles its unit range touches: expert id, row count, first bucket
// row, the activation row index of each row (token for W13, bucket row for W2) and, for W2, each
// row's pair index (where its result goes).
struct TileStage {
    int e[MAX_RANGE_TILES];
    int cnt[MAX_RANGE_TILES];
    int base[MAX_RANGE_TILES];
    int arow[MAX_RANGE_TILES][16];
    int pair[MAX_RANGE_TILES][16];
};

// This block's contiguous unit range out of U units (sched::unit_range); false if empty.
__device__ __forceinline__ bool unit_range(int64_t U, int first, int64_t &u0, int64_t &u1)
{
    return sched::unit_range(U, first, (int)gridDim.x, (int)blockIdx.x, u0, u1);
}

// Stage tiles [t_lo, t_lo + ntl) from the plan's tile descriptors: expert id, row count, first
// bucket row, each row's pair, and its activation row: the pair's token when topk > 0 (W13), else
// the bucket row itself (W2). All of it is one dependent load away from the tile index.
// The first Ts tiles are the shared expert's (Ts = 0: none): expert id -1, tokens 16t .. 16t+15 of
// Ms as rows (first row 16t of its own h or y; activation row: the token, or its shared h row).
template <bool SH = false>
__device__ __forceinline__ void stage_tiles(const PlanView &pv, TileStage &st, int t_lo, int ntl, int topk, int Ts = 0,
                                            int Ms = 0)
{
    if constexpr (!SH) Ts = 0;
    if ((int)threadIdx.x < ntl) {
        const int tg = t_lo + threadIdx.x, t = tg - Ts;
        const bool shr = SH && tg < Ts;
        st.e[threadIdx.x] = shr ? -1 : pv.tile_expert[t];
        st.cnt[threadIdx.x] = shr ? min(16, Ms - 16 * tg) : pv.tile_rows[t];
        st.base[threadIdx.x] = shr ? 16 * tg : pv.tile_base[t];
    }
    if ((int)threadIdx.x < ntl * 16) {
        const int i = threadIdx.x >> 4, r = threadIdx.x & 15, tg = t_lo + i, t = tg - Ts;
        if (SH && tg < Ts) {
            const int n = min(16, Ms - 16 * tg);
            st.pair[i][r] = 0;
            st.arow[i][r] = 16 * tg + (r < n ? r : 0);
        } else {
            const int n = pv.tile_rows[t];
            const int p = r < n ? pv.tile_pair[(int64_t)t * 16 + r] : 0;  // padding rows: pair 0, never stored
            st.pair[i][r] = p;
            st.arow[i][r] = topk > 0 ? p / topk : pv.tile_base[t] + (r < n ? r : 0);
        }
    }
    __syncthreads();
}

// ---- the routing plan inside the W13 launch (nvfp4_moe_plan_w13_swiglu) ----------------------------
// For small batches the plan's own launch is a large share of the layer, so every W13 block builds
// the plan of the ids in LDS (one pair per thread) and stages its row tiles from there; block 0
// also writes the plan buffer, word for word what nvfp4_moe_plan writes, for W2 and the caller.
// The steps are those of the one-block plan kernel: a ticket per pair while counting, scans over
// the experts, the group's pairs listed in ticket order, and each pair's stable rank as the number
// of group members with a smaller index.
struct PlanLds {
    int cnt[FUSED_PLAN_EXPERTS];
    int off[FUSED_PLAN_EXPERTS + 1];
    int tfirst[FUSED_PLAN_EXPERTS];
    int slot[FUSED_PLAN_PAIRS];
    int wsum[12];
    int bad;
};

// Builds the plan of fp.ids (P <= 256 pairs, E <= 1024 experts) in LDS on a 256-thread block, and
// in fp.plan if this is block 0. Returns the row-tile count. id and rank: this thread's pair's
// expert (-1 for none) and its rank among the expert's pairs.
__device__ int fused_plan(const FusedPlan &fp, PlanLds &pl, int topk, int &id, int &rank)
{
    const int tid = threadIdx.x, P = (int)fp.L.P, E = fp.E;
    const bool writer = blockIdx.x == 0;  // (in the pair-major launch, block 0 does nothing else)
    const int raw = tid < P ? fp.ids[tid] : -1;
    for (int e = tid; e < E; e += 256) pl.cnt[e] = 0;
    if (tid == 0) pl.bad = 0;
    __syncthreads();
    id = -1;
    int ticket = 0;
    if (tid < P) {
        if (raw >= 0 && raw < E) {
            id = raw;
            ticket = atomicAdd(&pl.cnt[raw], 1);
        } else if (raw != -1) {
            atomicAdd(&pl.bad, 1);
        }
    }
    __syncthreads();
    constexpr int EPT = FUSED_PLAN_EXPERTS / 256;
    const int ept = (E + 255) / 256, e0 = tid * ept, ne = min(ept, E - e0);
    int c[EPT];
    int3 sums{0, 0, 0};
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        c[i] = i < ne ? pl.cnt[e0 + i] : 0;
        sums.x += c[i];
        sums.y += c[i] > 0;
        sums.z += (c[i] + PLAN_TILE_ROWS - 1) / PLAN_TILE_ROWS;
    }
    int3 tot;
    const int3 pre = block_excl_scan3<4>(sums, pl.wsum, &tot);
    if (writer) {
        write_expert_lists(fp.plan, fp.L, e0, ne, c, pre.x, pre.y, pre.z, pl.off, pl.tfirst);
    } else {
        int cpre = pre.x, tpre = pre.z;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            if (i >= ne) continue;
            pl.off[e0 + i] = cpre;
            pl.tfirst[e0 + i] = tpre;
            cpre += c[i];
            tpre += (c[i] + PLAN_TILE_ROWS - 1) / PLAN_TILE_ROWS;
        }
    }
    if (tid == 0) {
        pl.off[E] = tot.x;
        if (writer) write_totals(fp.plan, fp.L, E, tot);
    }
    __syncthreads();
    if (id >= 0) pl.slot[pl.off[id] + ticket] = tid;  // the group's pairs, in ticket order
    __syncthreads();
    rank = 0;
    if (id >= 0) {
        const int o = pl.off[id], n = pl.cnt[id];
        for (int i = 0; i < n; ++i) rank += pl.slot[o + i] < tid;
        if (writer) place_pair(fp.plan, fp.L, tid, id, o + rank, rank, pl.tfirst[id]);
    } else if (writer && tid < P) {
        fp.plan[fp.L.pos_of_pair + tid] = -1;
        fp.plan[fp.L.pair_expert + tid] = -1;
    }
    if (writer && tid == 0) write_header_tail(fp.plan, fp.L, pl.bad, fp.M, topk, E);
    return tot.z;
}

// stage_tiles from the LDS plan: rows default to pair 0 / token 0 (padding), then every pair of a
// staged tile writes its row and the first pair of each tile the tile's expert, rows and base.
// The first Ts tiles are the shared expert's, staged as stage_tiles stages them (tokens 16t ..
// 16t+15 of Ms).
__device__ void stage_tiles_fused(const PlanLds &pl, TileStage &st, int t_lo, int ntl, int topk, int id, int rank,
                                  int Ts = 0, int Ms = 0)
{
    for (int i = threadIdx.x; i < ntl * 16; i += 256) {
        const int tg = t_lo + (i >> 4), r = i & 15;
        st.pair[i >> 4][r] = 0;
        st.arow[i >> 4][r] = tg < Ts ? 16 * tg + (r < Ms - 16 * tg ? r : 0) : 0;
    }
    if ((int)threadIdx.x < ntl) {
        const int tg = t_lo + threadIdx.x;
        if (tg < Ts) {
            st.e[threadIdx.x] = -1;
            st.cnt[threadIdx.x] = min(16, Ms - 16 * tg);
            st.base[threadIdx.x] = 16 * tg;
        }
    }
    __syncthreads();
    if (id >= 0) {
        const int t = Ts + pl.tfirst[id] + rank / PLAN_TILE_ROWS - t_lo, r = rank % PLAN_TILE_ROWS;
        if (t >= 0 && t < ntl) {
            st.pair[t][r] = threadIdx.x;
            st.arow[t][r] = threadIdx.x / topk;
            if (r == 0) {
                st.e[t] = id;
                st.cnt[t] = min(PLAN_TILE_ROWS, pl.cnt[id] - rank);
                st.base[t] = pl.off[id] + rank;
            }
        }
    }
    __syncthreads();
}

// Stage tiles [t_lo, t_lo + ntl) of the pair-major W13 launch: tile p is pair p alone (expert
// ids[p], or -1 when the id is outside [0, E): the pair is skipped), activation row p / topk, h row
// p (pair order).
__device__ __forceinline__ void stage_tiles_pairs(const int32_t *__restrict__ ids, int E, TileStage &st, int t_lo,
                                                  int ntl, int topk)
{
    if ((int)threadIdx.x < ntl) {
        const int p = t_lo + threadIdx.x, id = ids[p];
        const bool ok = id >= 0 && id < E;
        st.e[threadIdx.x] = ok ? id : -1;
        st.cnt[threadIdx.x] = ok ? 1 : 0;
        st.base[threadIdx.x] = p;
    }
    if ((int)threadIdx.x < ntl * 16) {
        const int i = threadIdx.x >> 4, r = threadIdx.x & 15;
        st.arow[i][r] = (t_lo + i) / topk;  // rows past the first are padding, never loaded
        st.pair[i][r] = t_lo + i;
    }
    __syncthreads();
}

// Tuning of the streaming kernels: TP 16-row weight-tile pairs per wave per unit, *_OCC resident
// 256-thread blocks per CU.
#ifndef NVFP4_W13_TP
#define NVFP4_W13_TP 1
#endif
#ifndef NVFP4_W2_TP
#define NVFP4_W2_TP 1
#endif
#ifndef NVFP4_W13_OCC
#define NVFP4_W13_OCC 2
#endif
#ifndef NVFP4_W2_OCC
#define NVFP4_W2_OCC 1
#endif
#ifndef NVFP4_W2T_OCC
#define NVFP4_W2T_OCC 3
#endif
constexpr int W2T_OCC = NVFP4_W2T_OCC;
constexpr int W13_TP = NVFP4_W13_TP;
constexpr int W2_TP = NVFP4_W2_TP;
constexpr int W13_OCC = NVFP4_W13_OCC;
constexpr int W2_OCC = NVFP4_W2_OCC;

// A unit's place in a block's range: index among the block's staged row tiles, unit within the
// tile. The stream kernels step it by one per unit instead of dividing a 64-bit unit index.
struct UnitPos {
    int ti, j;
};
__device__ __forceinline__ UnitPos next_pos(UnitPos p, int upt)
{
    return p.j + 1 < upt ? UnitPos{p.ti, p.j + 1} : UnitPos{p.ti + 1, 0};
}

// A block's n units (from position pa) with two weight buffers: step(pos, next, last, w, wn)
// computes the unit at pos from w and loads the next unit (next) into wn, or a dummy when last.
// The loop runs pairs of steps with the trip count fixed on entry, then the odd unit: an exit
// between the two steps would become (after the compiler makes the loop single-exit) a path back
// to the top on which the first step's prefetch looks still in flight when its buffer is next
// written, and the compiler would then wait for every load before issuing the next unit's.
template <typename Buf, typename Load, typename Step>
__device__ __forceinline__ void run_units(UnitPos pa, int n, int upt, Buf &wa, Buf &wb, Load load_unit, Step step)
{
    load_unit(pa, wa, false);
    int left = n;
    for (; left >= 2; left -= 2) {
        const UnitPos pb = next_pos(pa, upt), pc = next_pos(pb, upt);
        step(pa, pb, false, wa, wb);
        step(pb, pc, left == 2, wb, wa);
        pa = pc;
    }
    if (left) step(pa, pa, true, wa, wb);
}

// Geometry shared by both kernels: SPLIT waves per wave group (parallel chunks), 4/SPLIT wave
// groups per unit; `red` is the reduction length.
template <int SPLIT>
struct Geo {
    static constexpr int GROUPS = 4 / SPLIT;
    int lane, wave, n, q, sub, c, S, kb, kb_ld, q_ld;
    bool chunk, qv;  // this wave has a chunk; this lane group has data in it
    __device__ Geo(int red)
    {
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: unit bases stay scalar
        n = lane & 15;
        q = lane >> 4;
        sub = wave / SPLIT;
        c = wave % SPLIT;
        S = num_chunks(red);
        chunk = c < S;
        kb = c * KCHUNK;
        kb_ld = (chunk ? c : S - 1) * KCHUNK;  // idle waves read a valid chunk they never use
        const int groups = min(KCHUNK, red - kb_ld) >> 7;  // 128-element lane groups with data
        qv = chunk && q < groups;
        q_ld = q < groups ? q : groups - 1;
    }
};

// A fragments of this lane's activation row (zero when the row or the lane group is empty) for
// the whole chunk: 16 steps, kept in registers while the tile does not change.
__device__ __forceinline__ void load_a_chunk(f16x8 af[4][4], const f16 *row, bool valid, int kb, int q)
{
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int s = 0; s < 4; ++s) af[b][s] = valid ? a_frag(row, kb, q, b, s) : zero8();
}

// One chunk of NW weight rows (tiles) against the resident A fragments. A lane group past the
// chunk end (qv false) takes zero block scales: its finite E2M1 codes then decode to zeros, one
// select per scale pair instead of one per fragment.
template <int NW>
__device__ __forceinline__ void mma_chunk(const RawChunk (&w)[NW], const f16x8 af[4][4], bool qv, f32x4 (&acc)[NW])
{
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f16x2 sc[NW];
#pragma unroll
        for (int t = 0; t < NW; ++t) sc[t] = qv ? chunk_scales(w[t], b) : f16x2{0, 0};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < NW; ++t) acc[t] = mfma_step(af[b][s], decode8(w[t].codes[b][s], sc[t][s >> 1]), acc[t]);
    }
}

// ---- W13 + SwiGLU ---------------------------------------------------------------------------------
// Unit = (row tile, GROUPS*TP consecutive 16-wide i slices); wave (sub, c) owns the gate and up rows
// of slices (GROUPS*unit_index + sub)*TP .. +TP-1 for chunk c. A wave loads unit u+1's weights
// while unit u computes; barriers order LDS only, so they do not wait for those loads.
//
// SH: the shared expert's tiles come first (SharedW13); without it the kernel has none of their code.
//
// FP: the launch builds the plan itself from fp.ids (fused_plan) instead of reading pv.
//
// PM (pair-major, small batches of the layer call): row tile p is pair p alone, taken straight
// from fp.ids, and h is written in pair order; block 0 builds and writes the plan (for the caller)
// and computes nothing, blocks 1.. share the units. No unit waits for the plan.
template <int SPLIT, int TP, bool SH, bool FP = false, bool PM = false, bool PK = false>
__global__ __launch_bounds__(256, W13_OCC) void w13_swiglu_stream_kernel(PlanView pv, int topk, const f16 *__restrict__ x,
                                                                             const uint8_t *__restrict__ codes,
                                                                             const uint8_t *__restrict__ scales,
                                                                             const float *__restrict__ gscale, int K, int I,
                                                                             int layout, f16 *__restrict__ h, int first,
                                                                             SharedW13 shx, FusedPlan fp)
{
    static_assert(!PM || (!SH && !FP), "the pair-major launch has neither shared tiles nor staged plan rows");
    static_assert(!PK || (PM && TP == 1), "packed gate/up tiles are a pair-major, one-pair-per-wave form");
    using G = Geo<SPLIT>;
    constexpr int SL = G::GROUPS * TP;  // i slices per unit
    __shared__ float part[4][2 * TP][16][LDS_ROW];
    __shared__ TileStage st;
    // PK: a 16-row weight tile holds 8 gate rows and the same 8 up rows (lanes n < 8: gate i,
    // n >= 8: up i), so a unit covers 8 columns of h and a launch has twice the units. Every
    // output's MFMA chain is the same as with separate tiles, so h is bitwise the same.
    constexpr int IS = PK ? 8 : 16;  // h columns per i slice
    const int itiles = I / IS;
    const int upt = (itiles + SL - 1) / SL;  // units per row tile
    const int Ts = SH ? (shx.M + 15) >> 4 : 0;  // shared expert tiles, before the plan's
    int64_t u0, u1;
    __shared__ std::conditional_t<FP || PM, PlanLds, int> pl;
    int fid = -1, frank = 0;
    int T;
    bool has_units;
    if constexpr (PM) {
        if (blockIdx.x == 0) {  // the plan, for the caller; nothing downstream waits for it
            fused_plan(fp, pl, topk, fid, frank);
            return;
        }
        T = (int)fp.L.P;
        has_units = sched::unit_range((int64_t)T * upt, first, (int)gridDim.x - 1, (int)blockIdx.x - 1, u0, u1);
    } else {
        if constexpr (FP) T = fused_plan(fp, pl, topk, fid, frank);
        else T = pv.hdr[3];
        has_units = unit_range((int64_t)(Ts + T) * upt, first, u0, u1);
    }
    // Shared expert: block b computes the gates of tokens b, b + G, ... (wave 0). The first one's
    // loads go out after the tile staging (whose barrier would otherwise wait for them) and its sum
    // at the block's end, so neither delays the block's first weight loads (16-token layer with a
    // 512-wide shared expert, one launch each for W13 and W2: 68.2 -> 67.6 us on MI355X).
    const f16 *gv = reinterpret_cast<const f16 *>(shx.gate);
    const bool gate0 = SH && (int)blockIdx.x < shx.M && threadIdx.x < 64;
    WaveDotRegs gr;
    if constexpr (SH) {
        if (has_units) {
            const int tl = sched::range_first_tile(u0, upt), nl = sched::range_tiles(u0, u1, upt);
            if constexpr (FP) stage_tiles_fused(pl, st, tl, nl, topk, fid, frank, Ts, shx.M);
            else stage_tiles<SH>(pv, st, tl, nl, topk, Ts, shx.M);
        }
        if (gate0) wave_dot_load(gr, x + (size_t)blockIdx.x * K, gv, K);
    }
    auto finish_gates = [&]() {
        if constexpr (SH) {
            if (gate0) {
                const float z = wave_dot_sum(gr, K);
                if (threadIdx.x == 0) shx.sigma[blockIdx.x] = 1.0f / (1.0f + expf(-z));
                for (int r = blockIdx.x + gridDim.x; r < shx.M; r += gridDim.x) {
                    const float zr = wave_dot_f16(x + (size_t)r * K, gv, K);
                    if (threadIdx.x == 0) shx.sigma[r] = 1.0f / (1.0f + expf(-zr));
                }
            }
        }
    };
    if (!has_units) {  // block-uniform
        finish_gates();
        return;
    }
    const int t_lo = sched::range_first_tile(u0, upt);
    const G g(K);
    const size_t crow = (size_t)K >> 1, srow = (size_t)K >> 4;
    if constexpr (PM) {
        stage_tiles_pairs(fp.ids, fp.E, st, t_lo, sched::range_tiles(u0, u1, upt), topk);
    } else if constexpr (!SH) {
        if constexpr (FP) stage_tiles_fused(pl, st, t_lo, sched::range_tiles(u0, u1, upt), topk, fid, frank);
        else stage_tiles<SH>(pv, st, t_lo, sched::range_tiles(u0, u1, upt), topk);
    }

    int cur = -1;
    f16x8 af[4][4];
    // Packed weights of unit u into w. Loads are unconditional (idle waves and missing slices
    // re-read valid rows), so no branch separates them from the waits.
    // dummy (block-uniform): the "next unit" of the last unit, whose registers are never used; every
    // lane then reads the same 64 bytes of row 0 (one cache line per load), so the block's last
    // unit costs no second copy of its bytes through the CU's memory path.
    // A unit's rows are a wave-uniform base (expert, slice; scalar arithmetic) plus this lane's
    // fixed offsets (its row among the slice's 16 and its lane group's bytes in the chunk, at most
    // 31 rows of at most 1 KiB of codes).
    const int rstep = layout ? 2 : 1;  // row distance between consecutive i
    const size_t up_rows = layout ? 1 : (size_t)I;  // an up row relative to its gate row
    const uint32_t lrow = PK ? (uint32_t)(rstep * (g.n & 7)) + (g.n >= 8 ? (uint32_t)up_rows : 0u) : (uint32_t)(rstep * g.n);
    const uint32_t lane_c = lrow * (uint32_t)crow + (uint32_t)(g.kb_ld >> 1) + 64u * (uint32_t)g.q_ld;
    const uint32_t lane_s = lrow * (uint32_t)srow + (uint32_t)(g.kb_ld >> 4) + 8u * (uint32_t)g.q_ld;
    auto load_unit = [&](UnitPos pu, RawChunk (&w)[2 * TP], bool dummy) {
        const int it0 = pu.j * SL + g.sub * TP;
        const int e = __builtin_amdgcn_readfirstlane(st.e[pu.ti]);
        if constexpr (PM) dummy = dummy || e < 0;  // a skipped pair: nothing of it is read
        const bool own = !SH || e >= 0;
        const uint8_t *cb = own ? codes : shx.codes, *sb = own ? scales : shx.scales;
        const size_t eb = own ? (size_t)e * 2 * I : 0;
        const uint32_t lc = dummy ? 0u : lane_c, ls = dummy ? 0u : lane_s;
#pragma unroll
        for (int p = 0; p < TP; ++p) {
            const size_t rg = dummy ? 0 : eb + (size_t)rstep * (size_t)(min(it0 + p, itiles - 1) * IS);
            if constexpr (PK) {
                w[p] = load_chunk_at(cb + rg * crow, lc, sb + rg * srow, ls);
            } else {
                const size_t ru = dummy ? 0 : rg + up_rows;
                w[2 * p] = load_chunk_at(cb + rg * crow, lc, sb + rg * srow, ls);
                w[2 * p + 1] = load_chunk_at(cb + ru * crow, lc, sb + ru * srow, ls);
            }
        }
    };
    // One unit: math on `w` (already loading) and the next unit's weights into `wn`, or the dummy
    // when last. The two buffers alternate, so no register copy ever waits on a load in flight.
    auto step = [&](UnitPos pu, UnitPos pn, bool last, RawChunk (&w)[2 * TP], RawChunk (&wn)[2 * TP]) {
        const int ti = pu.ti;
        const int it0 = pu.j * SL + g.sub * TP;
        const int e = __builtin_amdgcn_readfirstlane(st.e[ti]), cnt = st.cnt[ti], base = st.base[ti];
        if (ti != cur) {  // A of this tile's rows, reused by every unit of the tile
            cur = ti;
            load_a_chunk(af, x + (size_t)st.arow[ti][g.n] * K, g.qv && g.n < cnt, g.kb, g.q);
        }
        load_unit(last ? pu : pn, wn, last);  // next unit's weights (after the last: a dummy)
        // The global scale (a scalar load) is read here, after the LDS reads that address the loads
        // above: scalar loads and LDS share one wait counter, so an earlier read would hold those
        // loads back, and here its latency overlaps the MFMA chain. (A skipped pair of the
        // pair-major launch has no scale and stores nothing: its tile has no rows.)
        const float gs = SH ? (e >= 0 ? gscale[e] : shx.gscale[0]) : gscale[PM && e < 0 ? 0 : e];
        __builtin_amdgcn_sched_barrier(0);      // keep those loads ahead of this unit's math
        f32x4 acc[2 * TP];
#pragma unroll
        for (int t = 0; t < 2 * TP; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        constexpr int NA = PK ? TP : 2 * TP;  // accumulator tiles
        mma_chunk<NA>(reinterpret_cast<const RawChunk(&)[NA]>(w), af, g.qv, reinterpret_cast<f32x4(&)[NA]>(acc));
        if (!(g.chunk && it0 < itiles)) {
#pragma unroll
            for (int t = 0; t < NA; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int t = 0; t < NA; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) part[g.wave][t][4 * g.q + j][g.n] = acc[t][j];
        lds_barrier();
        f16 *hb = !SH || e >= 0 ? h : reinterpret_cast<f16 *>(shx.h);
        const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
#pragma unroll
        for (int gp = 0; gp < G::GROUPS; ++gp)
#pragma unroll
            for (int p = 0; p < TP; ++p) {
                const int itx = pu.j * SL + gp * TP + p;
                const int tg = PK ? p : 2 * p, tu = PK ? p : 2 * p + 1, cu = PK ? col + 8 : col;
                if (itx < itiles && row < cnt && (!PK || col < 8)) {
                    float Gs = part[gp * SPLIT][tg][row][col];
                    float Us = part[gp * SPLIT][tu][row][cu];
                    for (int cc = 1; cc < g.S; ++cc) {
                        Gs += part[gp * SPLIT + cc][tg][row][col];
                        Us += part[gp * SPLIT + cc][tu][row][cu];
                    }
                    hb[(size_t)(base + row) * I + itx * IS + col] = f16_of_f32(swiglu(Gs * gs, Us * gs));
                }
            }
        lds_barrier();
    };
    RawChunk wa[2 * TP], wb[2 * TP];
    // The range starts in staged tile 0.
    run_units(UnitPos{0, (int)(u0 - (int64_t)t_lo * upt)}, (int)(u1 - u0), upt, wa, wb, load_unit, step);
    finish_gates();
}

// ---- W2: per-pair FP32 results y[p][n] = global * sum_i dq(W2)[n][i] * h[j][i], stored in pair order -----
// Unit = (row tile, 2*GROUPS*TP consecutive 16-row output tiles); wave (sub, c) owns output tiles
// 2*TP*(GROUPS*unit_index + sub) .. +2*TP-1 for chunk c. With one chunk (I <= 512) the waves never
// meet. As in W13, unit u+1's weights load while unit u computes.
//
// SH: the shared expert's tiles come first (SharedW2); without it the kernel has none of their code.
template <int SPLIT, int TP, bool SH>
__global__ __launch_bounds__(256, W2_OCC) void w2_stream_kernel(PlanView pv, const f16 *__restrict__ hin,
                                                                 const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 const float *__restrict__ gscale, int K, int I,
                                                                 float *__restrict__ ws, int first, SharedW2 shw)
{
    using G = Geo<SPLIT>;
    constexpr int NT = 2 * TP;            // output tiles per wave
    constexpr int UT = G::GROUPS * NT;    // output tiles per unit
    __shared__ float part[SPLIT > 1 ? 4 : 1][NT][16][LDS_ROW];
    __shared__ TileStage st;
    const int ntiles = K >> 4;
    const int upt = (ntiles + UT - 1) / UT;
    const int Ts = SH ? (shw.M + 15) >> 4 : 0;  // shared expert tiles, before the plan's
    int64_t u0, u1;
    if (!unit_range((int64_t)(Ts + pv.hdr[3]) * upt, first, u0, u1)) return;
    const int t_lo = sched::range_first_tile(u0, upt);
    const G g(I);
    const size_t crow = (size_t)I >> 1, srow = (size_t)I >> 4;
    stage_tiles<SH>(pv, st, t_lo, sched::range_tiles(u0, u1, upt), 0, Ts, SH ? shw.M : 0);

    int cur = -1;
    f16x8 af[4][4];
    // Packed weights of unit u into w; unconditional (idle waves re-read valid rows).
    // dummy: as in the W13 kernel, the never-used "next unit" of the last unit reads one line.
    // Wave-uniform row base plus this lane's fixed offsets, as in the W13 kernel.
    const uint32_t lane_c = (uint32_t)g.n * (uint32_t)crow + (uint32_t)(g.kb_ld >> 1) + 64u * (uint32_t)g.q_ld;
    const uint32_t lane_s = (uint32_t)g.n * (uint32_t)srow + (uint32_t)(g.kb_ld >> 4) + 8u * (uint32_t)g.q_ld;
    auto load_unit = [&](UnitPos pu, RawChunk (&w)[NT], bool dummy) {
        const int nt0 = pu.j * UT + g.sub * NT;
        const int e = __builtin_amdgcn_readfirstlane(st.e[pu.ti]);
        const bool own = !SH || e >= 0;
        const uint8_t *cb = own ? codes : shw.codes, *sb = own ? scales : shw.scales;
        const size_t eb = own ? (size_t)e * K : 0;
        const uint32_t lc = dummy ? 0u : lane_c, ls = dummy ? 0u : lane_s;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const size_t r = dummy ? 0 : eb + (size_t)(min(nt0 + t, ntiles - 1) * 16);
            w[t] = load_chunk_at(cb + r * crow, lc, sb + r * srow, ls);
        }
    };
    // One unit: math on `w`, next unit's weights into `wn` (the buffers alternate).
    auto step = [&](UnitPos pu, UnitPos pn, bool last, RawChunk (&w)[NT], RawChunk (&wn)[NT]) {
        const int ti = pu.ti;
        const int nt0 = pu.j * UT + g.sub * NT;
        const int e = __builtin_amdgcn_readfirstlane(st.e[ti]), cnt = st.cnt[ti], base = st.base[ti];
        const bool working = g.chunk && nt0 < ntiles;
        if (ti != cur) {
            cur = ti;
            const f16 *ha = !SH || e >= 0 ? hin : reinterpret_cast<const f16 *>(shw.h);
            load_a_chunk(af, ha + (size_t)st.arow[ti][g.n] * I, g.qv && g.n < cnt, g.kb, g.q);
        }
        // Row `row`'s output: its pair's row of ws, or for the shared expert the token's row of y.
        auto out_row = [&](int row) {
            return !SH || e >= 0 ? ws + (size_t)st.pair[ti][row] * K : shw.y + (size_t)(base + row) * K;
        };
        load_unit(last ? pu : pn, wn, last);  // after the last unit: a dummy
        // The global scale: a scalar load, read after the LDS reads that address the loads above
        // (scalar loads and LDS share one wait counter), so its latency overlaps the MFMA chain.
        const float gs = SH ? (e >= 0 ? gscale[e] : shw.gscale[0]) : gscale[e];
        __builtin_amdgcn_sched_barrier(0);      // keep those loads ahead of this unit's math
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        mma_chunk<NT>(w, af, g.qv, acc);
        if constexpr (SPLIT == 1) {
            if (working) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 4 * g.q + j;
                    if (row < cnt) {
                        float *y = out_row(row) + nt0 * 16 + g.n;
#pragma unroll
                        for (int t = 0; t < NT; ++t)
                            if (nt0 + t < ntiles) y[16 * t] = acc[t][j] * gs;
                    }
                }
            }
        } else {
            if (!working) {
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) part[g.wave][t][4 * g.q + j][g.n] = acc[t][j];
            lds_barrier();
            const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
#pragma unroll
            for (int gp = 0; gp < G::GROUPS; ++gp)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int ntx = pu.j * UT + gp * NT + t;
                    if (ntx < ntiles && row < cnt) {
                        float Y = part[gp * SPLIT][t][row][col];
                        for (int cc = 1; cc < g.S; ++cc) Y += part[gp * SPLIT + cc][t][row][col];
                        out_row(row)[ntx * 16 + col] = Y * gs;
                    }
                }
            lds_barrier();
        }
    };
    RawChunk wa[NT], wb[NT];
    run_units(UnitPos{0, (int)(u0 - (int64_t)t_lo * upt)}, (int)(u1 - u0), upt, wa, wb, load_unit, step);
}

// ---- slot-order weighted reduction: out[t][n] = fp16( fmaf chain over valid slots ) -----------------
// ws holds y in pair order (row p = t*topk + k), so the y loads do not wait for the plan; a slot
// is valid when the plan placed its pair (pos_of_pair >= 0). Rows of invalid pairs are never
// written and never used. Each thread owns 4 consecutive columns of one token.
__global__ __launch_bounds__(256) void reduce_kernel(const int32_t *__restrict__ pos_of_pair, const float *__restrict__ tw,
                                                     const float *__restrict__ ws, int topk, int K, int blocks_per_token,
                                                     SharedTerm sh, f16 *__restrict__ out)
{
    const int t = blockIdx.x / blocks_per_token;
    const int nb = blockIdx.x - t * blocks_per_token;
    const int n = (nb * (int)blockDim.x + (int)threadIdx.x) * 4;
    if (n >= K) return;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    // Slots go in batches of 16: a batch's rows are all loaded before the first fmaf, so their
    // latencies overlap, then folded in slot order. Each y row is read exactly once, so the loads
    // are non-temporal (no cache allocation): at 8192 tokens (671 MB of y) 153 -> 115 us on MI355X.
    constexpr int BATCH = 16;
    for (int k0 = 0; k0 < topk; k0 += BATCH) {
        f32x4 y[BATCH];
        float wk[BATCH];
        int pos[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            if (k0 + i < topk) {
                const size_t p = (size_t)t * topk + k0 + i;
                y[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(ws + p * K + n));
                pos[i] = pos_of_pair[p];
                wk[i] = tw[p];
            }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            if (k0 + i < topk && pos[i] >= 0) {
                const float w = wk[i];
                s0 = fmaf(w, y[i][0], s0);
                s1 = fmaf(w, y[i][1], s1);
                s2 = fmaf(w, y[i][2], s2);
                s3 = fmaf(w, y[i][3], s3);
            }
        }
    }
    if (sh.y) {  // the shared expert, after the routed slots
        const float g = sh.sigma[t];
        const float4 v = *reinterpret_cast<const float4 *>(sh.y + (size_t)t * K + n);
        s0 = fmaf(g, v.x, s0);
        s1 = fmaf(g, v.y, s1);
        s2 = fmaf(g, v.z, s2);
        s3 = fmaf(g, v.w, s3);
    }
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<f16x4 *>(out + (size_t)t * K + n) = f16x4{f16_of_f32(s0), f16_of_f32(s1), f16_of_f32(s2), f16_of_f32(s3)};
}

// One float read on the vector memory path (a buffer load over n floats; an index past them reads
// 0). A scalar load would share its wait counter with LDS accesses, so every LDS wait after it
// would also wait for this often cold read; a vector load can be issued beside the weight loads.
__device__ __forceinline__ float vector_load_f32(const float *base, int index, int n)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, n * 4, 0x00020000);
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, index * 4, 0, 0));
}

// Stage the valid slots' h rows (pieces of 8 fp16, 16 bytes) into LDS for the token-major W2
// kernels: in rounds of up to four pieces per thread, each thread first issues the round's loads,
// then stores them, so their latencies overlap instead of one round trip per piece. (Four per
// round: batching eight makes the kernels spill.) One round covers 16 slots of 512 columns.
template <int NT = 256, typename RowOf, typename ValidOf>
__device__ __forceinline__ void stage_slot_rows(f16 (*s_h)[KCHUNK], int nslot, int pieces, RowOf row_of, ValidOf valid)
{
    constexpr int MAXP = 4;
    const int total = nslot * pieces;
    for (int base = 0; base < total; base += MAXP * NT) {
        u32x4 v[MAXP];
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int idx = base + (int)threadIdx.x + NT * i;
            const int k = idx / pieces, pc = idx - k * pieces;
            if (idx < total && valid(k)) v[i] = *reinterpret_cast<const u32x4 *>(row_of(k) + 8 * pc);
        }
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int idx = base + (int)threadIdx.x + NT * i;
            const int k = idx / pieces, pc = idx - k * pieces;
            if (idx < total && valid(k)) *reinterpret_cast<u32x4 *>(&s_h[k][8 * pc]) = v[i];
        }
    }
}

// The slot-order fold of one output column of the token-major kernels: acc = fmaf(w_k, y_k, acc)
// over the valid slots k < nslot in order, from +0 (the reduce kernel's chain). The slot data are
// read from LDS eight slots at a time, all reads before the fmafs, so the chain does not wait for
// one LDS round trip per slot.
__device__ __forceinline__ float slot_fold(const int *s_e, const float *s_w, const float *yk, int nslot, int col)
{
    float acc = 0.f;
    for (int k0 = 0; k0 < nslot; k0 += 8) {
        int e[8];
        float w[8], y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int k = k0 + i < nslot ? k0 + i : k0;
            e[i] = s_e[k];
            w[i] = s_w[k];
            y[i] = yk[k * 16 + col];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (k0 + i < nslot && e[i] >= 0) acc = fmaf(w[i], y[i], acc);
    }
    return acc;
}

// ---- W2 + reduction, token-major (small batches) -----------------------------------------------------
// One block per (token t, 16 output rows n-tile); its four waves take the token's slots k = w,
// w+4, ... For each valid slot the wave runs the same MFMA chain as w2_stream_kernel on a
// one-row A (the pair's h row) and that slot's expert rows, so y[p][n] is bitwise the streaming
// kernel's value. The slot results meet in LDS and one fmaf chain per column, in slot order, gives
// out[t][n] directly: no FP32 workspace round trip and no second launch. Each pair's expert rows
// are read once per pair instead of once per expert, which costs little when pairs rarely share
// an expert (P << E); blocks of one n-tile are numbered consecutively per XCD so that shared rows
// meet in its L2.
//
// Pair mode (ids != NULL: the layer call's pair-major path): h is in pair order and each slot's
// expert is its id (skipped when outside [0, E)), so no load waits for the plan.
template <int NW>  // waves per block: 4 (three slots per wave) or 12 (one)
__global__ __launch_bounds__(64 * NW, NW == 4 ? W2T_OCC : 1) void w2_token_kernel(PlanView pv, int M, int topk, const f16 *__restrict__ hin,
                                                          const uint8_t *__restrict__ codes,
                                                          const uint8_t *__restrict__ scales,
                                                          const float *__restrict__ gscale, int K, int I,
                                                          const float *__restrict__ tw, SharedTerm sh,
                                                          f16 *__restrict__ out, const int32_t *__restrict__ ids,
                                                          int E)
{
    __shared__ float yk[MAX_TOPK][16];
    __shared__ int s_row[MAX_TOPK], s_e[MAX_TOPK];
    __shared__ float s_w[MAX_TOPK];
    __shared__ __attribute__((aligned(16))) f16 s_h[MAX_TOPK][KCHUNK];  // the slots' h rows (one-chunk case)
    const int ntiles = K >> 4;
    const int G = M * ntiles;
    const int per = (G + 7) >> 3;
    const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);  // XCD-aware numbering
    if (item >= G) return;
    const int nt = item / M, t = item - nt * M;
    const int S = num_chunks(I);
    const bool slot_thread = (int)threadIdx.x < topk;
    int row_r = 0, e_r = -1;
    float w_r = 0.f;
    if (slot_thread) {  // the loads first; the LDS writes wait for them after the h staging below
        const int p = t * topk + threadIdx.x;
        w_r = tw[p];
        if (ids) {
            row_r = p;
            e_r = ids[p];
        } else {
            row_r = pv.pos_of_pair[p];
            e_r = pv.pair_expert[p];  // -1 for a skipped pair: loaded beside pos_of_pair, not after it
        }
    }
    // Pair mode with one chunk: h rows are in pair order, so every slot's row is staged now, beside
    // the id loads (a skipped pair's row holds no result and is never used).
    if (ids && S == 1)
        stage_slot_rows<64 * NW>(s_h, topk, I >> 3, [&](int k) { return hin + ((size_t)t * topk + k) * I; },
                        [&](int) { return true; });
    if (slot_thread) {
        s_row[threadIdx.x] = row_r;
        s_e[threadIdx.x] = ids ? (e_r >= 0 && e_r < E ? e_r : -1) : e_r;
        s_w[threadIdx.x] = w_r;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, q = lane >> 4;
    const size_t crow = (size_t)I >> 1, srow = (size_t)I >> 4;
    if (S == 1) {
        // One chunk (I <= 512). Each wave issues the packed rows and global scales of its SPW slots
        // (12 / NW: three or one) at once; then the block stages the valid slots' h rows in LDS while those loads are
        // in flight, so the weight round trip never waits for the h round trip.
        const int pieces = I >> 3;
        const int groups = I >> 7;
        const bool qv = q < groups;
        const int q_ld = qv ? q : groups - 1;
        constexpr int SPW = 12 / NW;
        const int ngroups = (topk + 11) / 12;  // block-uniform trip count (the loop holds a barrier)
        for (int gi = 0; gi < ngroups; ++gi) {
            const int k0 = wave + 12 * gi;
            RawChunk w[SPW];
            int eg[SPW], se[SPW];
            float gsk[SPW];
#pragma unroll
            for (int g = 0; g < SPW; ++g) se[g] = k0 + NW * g < topk ? s_e[k0 + NW * g] : -1;  // LDS reads together
#pragma unroll
            for (int g = 0; g < SPW; ++g) {
                const int k = k0 + NW * g;
                const bool live = se[g] >= 0;
                eg[g] = __builtin_amdgcn_readfirstlane(live ? se[g] : 0);
                // An idle slot's registers are never used: all its lanes read one line of row 0.
                const size_t wr = live ? (size_t)eg[g] * K + nt * 16 + n : 0;
                w[g] = load_chunk(codes + wr * crow, scales + wr * srow, 0, live ? q_ld : 0);
                gsk[g] = vector_load_f32(gscale, eg[g], E);  // beside the weights: one round trip
            }
            if (gi == 0 && !ids)  // plan mode: the rows come from the plan, loaded above
                stage_slot_rows<64 * NW>(s_h, topk, pieces, [&](int k) { return hin + (size_t)s_row[k] * I; },
                                [&](int k) { return s_e[k] >= 0; });
            if (gi == 0) __syncthreads();  // s_h staged; it is not written again
#pragma unroll
            for (int g = 0; g < SPW; ++g) {
                const int k = k0 + NW * g;
                if (se[g] < 0) continue;  // wave-uniform (also past topk)
                f16x8 af[4][4];
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                    for (int ss = 0; ss < 4; ++ss) {
                        const f16x8 v = *reinterpret_cast<const f16x8 *>(&s_h[k][128 * q_ld + 32 * bb + 8 * ss]);
                        af[bb][ss] = (n == 0 && qv) ? v : zero8();  // row 0 of the tile is the pair
                    }
                f32x4 ca[1] = {{0.f, 0.f, 0.f, 0.f}};
                mma_chunk<1>(reinterpret_cast<const RawChunk(&)[1]>(w[g]), af, qv, ca);
                if (q == 0) yk[k][n] = ca[0][0] * gsk[g];
            }
        }
    } else {
        for (int k = wave; k < topk; k += NW) {
            const int e = s_e[k];
            if (e < 0) continue;  // wave-uniform
            const size_t wr = (size_t)e * K + nt * 16 + n;
            const f16 *hr = hin + (size_t)s_row[k] * I;
            f32x4 tot = {-0.f, -0.f, -0.f, -0.f};  // -0 + x == x: chunk 0 needs no special case
            for (int c = 0; c < S; ++c) {
                const int kb = c * KCHUNK;
                const int groups = min(KCHUNK, I - kb) >> 7;
                const bool qv = q < groups;
                const RawChunk w = load_chunk(codes + wr * crow, scales + wr * srow, kb, qv ? q : groups - 1);
                f16x8 af[4][4];
                load_a_chunk(af, hr, n == 0 && qv, kb, q);  // the pair's h row in row 0 of the tile
                f32x4 ca[1] = {{0.f, 0.f, 0.f, 0.f}};
                mma_chunk<1>(reinterpret_cast<const RawChunk(&)[1]>(w), af, qv, ca);
                tot += ca[0];
            }
            if (q == 0) yk[k][n] = tot[0] * gscale[e];  // row 0 of the tile: lanes 0..15, register 0
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < 16) {
        float acc = slot_fold(s_e, s_w, &yk[0][0], topk, threadIdx.x);
        if (sh.y) acc = fmaf(sh.sigma[t], sh.y[(size_t)t * K + nt * 16 + threadIdx.x], acc);  // shared expert last
        out[(size_t)t * K + nt * 16 + threadIdx.x] = f16_of_f32(acc);
    }
}

//
// w2_token_shared_kernel: w2_token_kernel with slot topk the shared expert (SharedW2): row t of its
// h, its own weights, weight sigma, added after the routed slots. The routed-only kernel is kept
// separate so that it carries none of this.
template <int NW>  // waves per block, as in w2_token_kernel
__global__ __launch_bounds__(64 * NW, NW == 4 ? W2T_OCC : 1) void w2_token_shared_kernel(PlanView pv, int M, int topk, const f16 *__restrict__ hin,
                                                          const uint8_t *__restrict__ codes,
                                                          const uint8_t *__restrict__ scales,
                                                          const float *__restrict__ gscale, int K, int I,
                                                          const float *__restrict__ tw, SharedW2 shw,
                                                          f16 *__restrict__ out)
{
    constexpr int NS = MAX_TOPK + 1;
    __shared__ float yk[NS][16];
    __shared__ int s_row[NS], s_e[NS];
    __shared__ float s_w[NS];
    __shared__ __attribute__((aligned(16))) f16 s_h[NS][KCHUNK];  // the slots' h rows (one-chunk case)
    const int ntiles = K >> 4;
    const int G = M * ntiles;
    const int per = (G + 7) >> 3;
    const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);  // XCD-aware numbering
    if (item >= G) return;
    const int nt = item / M, t = item - nt * M;
    const int nslot = topk + 1;  // slot topk: the shared expert
    if ((int)threadIdx.x < topk) {
        const int p = t * topk + threadIdx.x;
        const int j = pv.pos_of_pair[p];
        s_row[threadIdx.x] = j;
        s_e[threadIdx.x] = pv.pair_expert[p];  // -1 for a skipped pair: loaded beside pos_of_pair, not after it
        s_w[threadIdx.x] = tw[p];
    } else if ((int)threadIdx.x == topk) {
        s_row[topk] = t;
        s_e[topk] = 0;
        s_w[topk] = shw.sigma[t];
    }
    __syncthreads();
    auto slot_h = [&](int k) { return k < topk ? hin : reinterpret_cast<const f16 *>(shw.h); };
    auto slot_codes = [&](int k) { return k < topk ? codes : shw.codes; };
    auto slot_scales = [&](int k) { return k < topk ? scales : shw.scales; };
    auto slot_gs = [&](int k) { return k < topk ? gscale[s_e[k]] : shw.gscale[0]; };
    auto slot_row0 = [&](int k, int e) { return (k < topk ? (size_t)e * K : 0) + nt * 16; };
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, q = lane >> 4;
    const int S = num_chunks(I);
    const size_t crow = (size_t)I >> 1, srow = (size_t)I >> 4;
    if (S == 1) {
        // One chunk (I <= 512), as in w2_token_kernel: weights and global scales first, then the
        // h rows staged in LDS while they are in flight.
        const int pieces = I >> 3;
        const int groups = I >> 7;
        const bool qv = q < groups;
        const int q_ld = qv ? q : groups - 1;
        constexpr int SPW = 12 / NW;
        const int ngroups = (nslot + 11) / 12;  // block-uniform trip count (the loop holds a barrier)
        for (int gi = 0; gi < ngroups; ++gi) {
            const int k0 = wave + 12 * gi;
            RawChunk w[SPW];
            int eg[SPW], kg[SPW];
            float gsk[SPW];
#pragma unroll
            for (int g = 0; g < SPW; ++g) {
                const int k = k0 + NW * g;
                const bool live = k < nslot && s_e[k] >= 0;
                eg[g] = __builtin_amdgcn_readfirstlane(live ? s_e[k] : 0);
                kg[g] = k < nslot ? k : 0;
                const size_t wr = live ? slot_row0(kg[g], eg[g]) + n : 0;  // idle slot: one line of row 0
                w[g] = load_chunk(slot_codes(kg[g]) + wr * crow, slot_scales(kg[g]) + wr * srow, 0, live ? q_ld : 0);
            }
            if (gi == 0)
                stage_slot_rows<64 * NW>(s_h, nslot, pieces, [&](int k) { return slot_h(k) + (size_t)s_row[k] * I; },
                                [&](int k) { return s_e[k] >= 0; });
#pragma unroll
            for (int g = 0; g < SPW; ++g) gsk[g] = kg[g] < topk ? gscale[eg[g]] : shw.gscale[0];  // after the LDS reads
            if (gi == 0) __syncthreads();  // s_h staged; it is not written again
#pragma unroll
            for (int g = 0; g < SPW; ++g) {
                const int k = k0 + NW * g;
                if (k >= nslot || s_e[k] < 0) continue;  // wave-uniform
                f16x8 af[4][4];
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                    for (int ss = 0; ss < 4; ++ss) {
                        const f16x8 v = *reinterpret_cast<const f16x8 *>(&s_h[k][128 * q_ld + 32 * bb + 8 * ss]);
                        af[bb][ss] = (n == 0 && qv) ? v : zero8();  // row 0 of the tile is the pair
                    }
                f32x4 ca[1] = {{0.f, 0.f, 0.f, 0.f}};
                mma_chunk<1>(reinterpret_cast<const RawChunk(&)[1]>(w[g]), af, qv, ca);
                if (q == 0) yk[k][n] = ca[0][0] * gsk[g];
            }
        }
    } else {
        for (int k = wave; k < nslot; k += NW) {
            const int e = s_e[k];
            if (e < 0) continue;  // wave-uniform
            const size_t wr = slot_row0(k, e) + n;
            const uint8_t *cb = slot_codes(k), *sb = slot_scales(k);
            const f16 *hr = slot_h(k) + (size_t)s_row[k] * I;
            f32x4 tot = {-0.f, -0.f, -0.f, -0.f};  // -0 + x == x: chunk 0 needs no special case
            for (int c = 0; c < S; ++c) {
                const int kb = c * KCHUNK;
                const int groups = min(KCHUNK, I - kb) >> 7;
                const bool qv = q < groups;
                const RawChunk w = load_chunk(cb + wr * crow, sb + wr * srow, kb, qv ? q : groups - 1);
                f16x8 af[4][4];
                load_a_chunk(af, hr, n == 0 && qv, kb, q);  // the pair's h row in row 0 of the tile
                f32x4 ca[1] = {{0.f, 0.f, 0.f, 0.f}};
                mma_chunk<1>(reinterpret_cast<const RawChunk(&)[1]>(w), af, qv, ca);
                tot += ca[0];
            }
            if (q == 0) yk[k][n] = tot[0] * slot_gs(k);  // row 0 of the tile: lanes 0..15, register 0
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < 16) {
        float acc = slot_fold(s_e, s_w, &yk[0][0], topk, threadIdx.x);
        acc = fmaf(s_w[topk], yk[topk][threadIdx.x], acc);  // the shared expert last
        out[(size_t)t * K + nt * 16 + threadIdx.x] = f16_of_f32(acc);
    }
}

int split_for(int k)
{
    const int s = num_chunks(k);
    return s <= 1 ? 1 : (s <= 2 ? 2 : 4);
}

// Persistent grid (sched::grid_blocks). *cus_out: the device's CU count.
unsigned stream_grid(int occ, int64_t units_max, int64_t t_max, int *cus_out)
{
    const int cus = device_cus();
    *cus_out = cus;
    return (unsigned)sched::grid_blocks(occ, cus, units_max, t_max);
}

}  // namespace

int run_w13(const PlanView &pv, int64_t t_max, int32_t topk, const uint16_t *x, const nvfp4_weights &w, int32_t layout,
            uint16_t *h, hipStream_t s, SharedW13 shx, FusedPlan fp)
{
    const int K = w.k, I = w.rows / 2;
    const int split = split_for(K);
    const int sl = (4 / split) * W13_TP;
    const int upt = (I / 16 + sl - 1) / sl;
    t_max += (shx.M + 15) / 16;  // the shared expert's tiles
    int cus = 0;
    const dim3 grid(stream_grid(W13_OCC, t_max * upt, t_max, &cus)), block(256);
    const int first = sched::first_blocks(W13_OCC, cus, (int)grid.x);
    const f16 *xp = reinterpret_cast<const f16 *>(x);
    f16 *hp = reinterpret_cast<f16 *>(h);
    if (fp.ids && fp.pair_major) {  // block 0: the plan; blocks 1..: one pair per row tile
        // Packed gate/up tiles (8 h columns per unit) while there are at most ten 16-column units
        // per CU: twice the units, so the last ones spread more evenly over the CUs. Measured on
        // MI355X (512 experts, top-10, K = 2048, I = 512; layer call): 14.1 -> 13.5 us at one
        // token, 17.1 -> 16.6 at two, 24.8 -> 23.9 at four, 38.5 -> 38.3 at eight; at twelve
        // tokens (15 units per CU) 50.6 -> 51.5, so larger batches keep 16-column units.
        constexpr bool PKF = W13_TP == 1;  // the packed form exists for one tile pair per wave
        const bool pk = PKF && fp.L.P * upt <= 10 * (int64_t)cus;
        const int64_t U = fp.L.P * (pk ? (I / 8 + sl - 1) / sl : upt);
        // Unit blocks as for any streaming launch (at least P / 10, so a range stays within the
        // staging), less one when that keeps block 0 and every unit block resident at once.
        int ub = sched::grid_blocks(W13_OCC, cus, U, fp.L.P);
        if (ub == W13_OCC * cus && ub > 1 && ub - 1 >= (fp.L.P + 9) / 10) --ub;
        const dim3 gp((unsigned)(ub + 1));
        // Block 0 takes a first slot but finishes early, so the unit block that shares its CU counts
        // as a first block: the weighted split stays on (cus first against cus - 1 second blocks).
        const int fpm = sched::first_blocks(W13_OCC, cus, ub + 1);
        auto go = [&](auto kern) {
            return launch(kern, gp, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp, fpm, shx, fp);
        };
        switch (split) {
        case 1: return pk ? go(w13_swiglu_stream_kernel<1, W13_TP, false, false, true, PKF>) : go(w13_swiglu_stream_kernel<1, W13_TP, false, false, true>);
        case 2: return pk ? go(w13_swiglu_stream_kernel<2, W13_TP, false, false, true, PKF>) : go(w13_swiglu_stream_kernel<2, W13_TP, false, false, true>);
        default: return pk ? go(w13_swiglu_stream_kernel<4, W13_TP, false, false, true, PKF>) : go(w13_swiglu_stream_kernel<4, W13_TP, false, false, true>);
        }
    }
    if (fp.ids) {  // the plan built in the launch
        switch (split) {
        case 1: return launch(shx.M > 0 ? w13_swiglu_stream_kernel<1, W13_TP, true, true> : w13_swiglu_stream_kernel<1, W13_TP, false, true>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp, first, shx, fp);
        case 2: return launch(shx.M > 0 ? w13_swiglu_stream_kernel<2, W13_TP, true, true> : w13_swiglu_stream_kernel<2, W13_TP, false, true>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp, first, shx, fp);
        default: return launch(shx.M > 0 ? w13_swiglu_stream_kernel<4, W13_TP, true, true> : w13_swiglu_stream_kernel<4, W13_TP, false, true>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp, first, shx, fp);
        }
    }
    switch (split) {
    case 1: return launch(shx.M > 0 ? w13_swiglu_stream_kernel<1, W13_TP, true> : w13_swiglu_stream_kernel<1, W13_TP, false>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp, first, shx, fp);
    case 2: return launch(shx.M > 0 ? w13_swiglu_stream_kernel<2, W13_TP, true> : w13_swiglu_stream_kernel<2, W13_TP, false>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp, first, shx, fp);
    default: return launch(shx.M > 0 ? w13_swiglu_stream_kernel<4, W13_TP, true> : w13_swiglu_stream_kernel<4, W13_TP, false>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp, first, shx, fp);
    }
}

int run_w2(const PlanView &pv, int64_t t_max, int32_t M, int32_t topk, const uint16_t *h, const nvfp4_weights &w,
           const float *topk_weights, uint16_t *out, float *ws, hipStream_t s, SharedTerm sh, SharedW2 shw,
           const int32_t *pair_ids)
{
    const int K = w.rows, I = w.k;
    if (pair_ids && (!use_token_w2((int64_t)M * topk, w.groups) || shw.M > 0)) return NVFP4_ERR_UNSUPPORTED;
    if (use_token_w2((int64_t)M * topk, w.groups)) {
        const int64_t G = (int64_t)M * (K / 16);
        // Waves per block: with at most one block per CU, a block's slots are spread over 12 waves
        // (one slot chain per wave instead of three in a row). Measured on MI355X (512 experts,
        // top-10, K = 2048, I = 512; layer call): 15.3 -> 14.1 us at one token, 18.3 -> 17.3 at
        // two; six waves at two blocks per CU were slower (25.0 -> 26.9 us at four tokens).
        const int64_t nb = (G + 7) / 8 * 8, cus = device_cus();
        const dim3 grid((unsigned)nb);
        if (shw.M > 0) {
            auto go_sh = [&](auto kern, int threads) {
                return launch(kern, grid, dim3((unsigned)threads), 0, s, pv, M, topk, reinterpret_cast<const f16 *>(h),
                              w.codes, w.scales, w.global_scale, K, I, topk_weights, shw, reinterpret_cast<f16 *>(out));
            };
            return nb <= cus ? go_sh(w2_token_shared_kernel<12>, 768) : go_sh(w2_token_shared_kernel<4>, 256);
        }
        auto go = [&](auto kern, int threads) {
            return launch(kern, grid, dim3((unsigned)threads), 0, s, pv, M, topk, reinterpret_cast<const f16 *>(h), w.codes,
                          w.scales, w.global_scale, K, I, topk_weights, sh, reinterpret_cast<f16 *>(out), pair_ids,
                          w.groups);
        };
        if (nb <= cus) return go(w2_token_kernel<12>, 768);
        return go(w2_token_kernel<4>, 256);
    }
    if (shw.M > 0) {  // the shared tiles write y; the reduction adds sigma * y after the routed slots
        sh.y = shw.y;
        sh.sigma = shw.sigma;
    }
    const int split = split_for(I);
    const int ut = (4 / split) * 2 * W2_TP;
    const int upt = (K / 16 + ut - 1) / ut;
    t_max += (shw.M + 15) / 16;
    int cus = 0;
    const dim3 grid(stream_grid(W2_OCC, t_max * upt, t_max, &cus)), block(256);
    const int first = sched::first_blocks(W2_OCC, cus, (int)grid.x);
    const f16 *hp = reinterpret_cast<const f16 *>(h);
    int st;
    switch (split) {
    case 1: st = launch(shw.M > 0 ? w2_stream_kernel<1, W2_TP, true> : w2_stream_kernel<1, W2_TP, false>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, ws, first, shw); break;
    case 2: st = launch(shw.M > 0 ? w2_stream_kernel<2, W2_TP, true> : w2_stream_kernel<2, W2_TP, false>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, ws, first, shw); break;
    default: st = launch(shw.M > 0 ? w2_stream_kernel<4, W2_TP, true> : w2_stream_kernel<4, W2_TP, false>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, ws, first, shw); break;
    }
    if (st != NVFP4_OK) return st;
    return run_reduce(pv, M, topk, K, topk_weights, ws, out, s, sh);
}

int run_reduce(const PlanView &pv, int32_t M, int32_t topk, int32_t K, const float *topk_weights, const float *ws,
               uint16_t *out, hipStream_t s, SharedTerm sh)
{
    // Each CU's load throughput bounds this pass, so a small batch runs 64-thread blocks: its rows
    // spread over four times as many CUs (at 16 tokens and K = 2048: 128 blocks instead of 32).
    const int threads = (int64_t)M * ((K / 4 + 255) / 256) < 2 * (int64_t)device_cus() ? 64 : 256;
    const int bpt = (K / 4 + threads - 1) / threads;
    return launch(reduce_kernel, dim3((unsigned)((int64_t)M * bpt)), dim3((unsigned)threads), 0, s, pv.pos_of_pair,
                  topk_weights, ws, topk, K, bpt, sh, reinterpret_cast<f16 *>(out));
}

}  // namespace nvfp4
