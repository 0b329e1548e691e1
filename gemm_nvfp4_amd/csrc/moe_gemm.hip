// moe_gemm.hip -- grouped expert GEMMs of the MoE layer, decode (streaming) regime.
//   W13 with fused SwiGLU ("expert-grouped multi-row W13/SiLU with intra-CTA Split-K"), then W2
//   with the top-k-weighted reduction ("grouped W2 reusing the same integer plan", "W2/reduction
//   fusion"), from the "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page, "Scope and
//   related PRs".
//
// At small M the layer reads every active expert's packed weights once and does little math on
// them. It is bound by HBM bandwidth, so the design goal is many bytes in flight per CU. On
// MI355X that works best with many resident waves each holding one unit's loads (measured: deeper
// per-wave prefetch lowers the achieved read rate). gfx950 design:
//   * Work unit: (row tile of the plan, a group of 16-row weight tiles). A row tile has at most
//     16 bucket rows (pairs) of one expert. Units are numbered tile-major and cut into equal
//     contiguous ranges, one per persistent block (three 256-thread blocks per CU, at most 168
//     VGPRs per lane, so 12 waves per CU). Blocks past the device-side unit count leave at once,
//     so no device-to-host read is ever needed.
//   * Block start: the block stages its range's tile metadata (expert, rows, first bucket row,
//     activation-row index of each row) in LDS. That is one dependent-load chain per block.
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

namespace nvfp4 {
namespace {

constexpr int LDS_ROW = 20;  // padded row of 16 floats: rows 4 apart land on different banks
constexpr int MAX_RANGE_TILES = 16;

// Per-block staging of the row tiles its unit range touches: expert id, row count, first bucket
// row and the activation row index of each row (token for W13, bucket row for W2).
struct TileStage {
    int e[MAX_RANGE_TILES];
    int cnt[MAX_RANGE_TILES];
    int base[MAX_RANGE_TILES];
    int arow[MAX_RANGE_TILES][16];
};

// Contiguous unit range of this block out of U units; returns false if empty.
__device__ __forceinline__ bool unit_range(int64_t U, int64_t &u0, int64_t &u1)
{
    u0 = U * blockIdx.x / gridDim.x;
    u1 = U * (blockIdx.x + 1) / gridDim.x;
    return u0 < u1;
}

// Stage tiles [t_lo, t_lo + ntl): expert ids, row counts, first bucket rows, then each row's
// activation row: the token (pair / topk) when topk > 0, else the bucket row itself.
__device__ __forceinline__ void stage_tiles(const PlanView &pv, TileStage &st, int t_lo, int ntl, int topk)
{
    if ((int)threadIdx.x < ntl) {
        const int e = pv.tile_expert[t_lo + threadIdx.x];
        const int r0 = pv.tile_row0[t_lo + threadIdx.x];
        st.e[threadIdx.x] = e;
        st.cnt[threadIdx.x] = min(16, pv.counts[e] - r0);
        st.base[threadIdx.x] = pv.offsets[e] + r0;
    }
    __syncthreads();
    if ((int)threadIdx.x < ntl * 16) {
        const int i = threadIdx.x >> 4, r = threadIdx.x & 15;
        const int j = st.base[i] + r;
        st.arow[i][r] = r < st.cnt[i] ? (topk > 0 ? pv.sorted_pair[j] / topk : j) : 0;
    }
    __syncthreads();
}

// Geometry shared by both kernels: SPLIT waves per tile pair (parallel chunks), 4/SPLIT tile pairs
// per unit; `red` is the reduction length.
template <int SPLIT>
struct Geo {
    static constexpr int PAIRS = 4 / SPLIT;
    int lane, wave, n, q, sub, c, S, kb, kb_ld, q_ld;
    bool chunk, qv;  // this wave has a chunk; this lane group has data in it
    __device__ Geo(int red)
    {
        lane = threadIdx.x & 63;
        wave = threadIdx.x >> 6;
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

// One chunk of two weight rows (tiles) against the resident A fragments.
__device__ __forceinline__ void mma_chunk2(const RawChunk &w0, const RawChunk &w1, const f16x8 af[4][4], bool qv,
                                           f32x4 &acc0, f32x4 &acc1)
{
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const f16x2 sc0 = chunk_scales(w0, b), sc1 = chunk_scales(w1, b);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            acc0 = mfma_step(af[b][s], b_frag(w0, sc0, b, s, qv), acc0);
            acc1 = mfma_step(af[b][s], b_frag(w1, sc1, b, s, qv), acc1);
        }
    }
}

// ---- W13 + SwiGLU ---------------------------------------------------------------------------------
// Unit = (row tile, PAIRS consecutive 16-wide i slices); wave (sub, c) owns the gate and up rows of
// slice PAIRS*unit_index + sub for chunk c.
template <int SPLIT>
__global__ __launch_bounds__(256, 3) void w13_swiglu_stream_kernel(PlanView pv, int topk, const f16 *__restrict__ x,
                                                                    const uint8_t *__restrict__ codes,
                                                                    const uint8_t *__restrict__ scales,
                                                                    const float *__restrict__ gscale, int K, int I,
                                                                    int layout, f16 *__restrict__ h)
{
    using G = Geo<SPLIT>;
    __shared__ float part[4][2][16][LDS_ROW];
    __shared__ TileStage st;
    const int itiles = I >> 4;
    const int upt = (itiles + G::PAIRS - 1) / G::PAIRS;  // units per row tile
    int64_t u0, u1;
    if (!unit_range((int64_t)pv.hdr[3] * upt, u0, u1)) return;  // block-uniform
    const int t_lo = (int)(u0 / upt);
    const G g(K);
    const size_t crow = (size_t)K >> 1, srow = (size_t)K >> 4;
    stage_tiles(pv, st, t_lo, (int)((u1 - 1) / upt) - t_lo + 1, topk);

    int cur = -1;
    f16x8 af[4][4];
    for (int64_t u = u0; u < u1; ++u) {
        const int ti = (int)(u / upt) - t_lo;
        const int it = (int)(u % upt) * G::PAIRS + g.sub;
        const int e = st.e[ti], cnt = st.cnt[ti], base = st.base[ti];
        f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
        if (g.chunk && it < itiles) {
            const int i_row = it * 16 + g.n;
            const int rg = layout ? 2 * i_row : i_row;
            const int ru = layout ? 2 * i_row + 1 : I + i_row;
            const size_t eb = (size_t)e * 2 * I;
            const RawChunk wg = load_chunk(codes + (eb + rg) * crow, scales + (eb + rg) * srow, g.kb_ld, g.q_ld);
            const RawChunk wu = load_chunk(codes + (eb + ru) * crow, scales + (eb + ru) * srow, g.kb_ld, g.q_ld);
            if (ti != cur) {  // A of this tile's rows, reused by every unit of the tile
                cur = ti;
                load_a_chunk(af, x + (size_t)st.arow[ti][g.n] * K, g.qv && g.n < cnt, g.kb, g.q);
            }
            mma_chunk2(wg, wu, af, g.qv, accg, accu);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            part[g.wave][0][4 * g.q + j][g.n] = accg[j];
            part[g.wave][1][4 * g.q + j][g.n] = accu[j];
        }
        __syncthreads();
        const float gs = gscale[e];
        const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
#pragma unroll
        for (int p = 0; p < G::PAIRS; ++p) {
            const int itx = (int)(u % upt) * G::PAIRS + p;
            if (itx < itiles && row < cnt) {
                float Gs = part[p * SPLIT][0][row][col];
                float Us = part[p * SPLIT][1][row][col];
                for (int cc = 1; cc < g.S; ++cc) {
                    Gs += part[p * SPLIT + cc][0][row][col];
                    Us += part[p * SPLIT + cc][1][row][col];
                }
                h[(size_t)(base + row) * I + itx * 16 + col] = (f16)swiglu(Gs * gs, Us * gs);
            }
        }
        __syncthreads();
    }
}

// ---- W2: per-pair FP32 results y[j][n] = global * sum_i dq(W2)[n][i] * h[j][i] -------------------------
// Unit = (row tile, 2*PAIRS consecutive 16-row output tiles); wave (sub, c) owns output tiles
// 2*(PAIRS*unit_index + sub) and +1 for chunk c. With one chunk (I <= 512) the waves never meet.
template <int SPLIT>
__global__ __launch_bounds__(256, 3) void w2_stream_kernel(PlanView pv, const f16 *__restrict__ hin,
                                                            const uint8_t *__restrict__ codes,
                                                            const uint8_t *__restrict__ scales,
                                                            const float *__restrict__ gscale, int K, int I,
                                                            float *__restrict__ ws)
{
    using G = Geo<SPLIT>;
    __shared__ float part[SPLIT > 1 ? 4 : 1][2][16][LDS_ROW];
    __shared__ TileStage st;
    const int npairs = K >> 5;  // K is a multiple of 64 (host check)
    const int upt = (npairs + G::PAIRS - 1) / G::PAIRS;
    int64_t u0, u1;
    if (!unit_range((int64_t)pv.hdr[3] * upt, u0, u1)) return;
    const int t_lo = (int)(u0 / upt);
    const G g(I);
    const size_t crow = (size_t)I >> 1, srow = (size_t)I >> 4;
    stage_tiles(pv, st, t_lo, (int)((u1 - 1) / upt) - t_lo + 1, 0);

    int cur = -1;
    f16x8 af[4][4];
    for (int64_t u = u0; u < u1; ++u) {
        const int ti = (int)(u / upt) - t_lo;
        const int tp = (int)(u % upt) * G::PAIRS + g.sub;
        const int e = st.e[ti], cnt = st.cnt[ti], base = st.base[ti];
        const bool working = g.chunk && tp < npairs;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        if (working) {
            const size_t r0 = (size_t)e * K + tp * 32 + g.n, r1 = r0 + 16;
            const RawChunk w0 = load_chunk(codes + r0 * crow, scales + r0 * srow, g.kb_ld, g.q_ld);
            const RawChunk w1 = load_chunk(codes + r1 * crow, scales + r1 * srow, g.kb_ld, g.q_ld);
            if (ti != cur) {
                cur = ti;
                load_a_chunk(af, hin + (size_t)st.arow[ti][g.n] * I, g.qv && g.n < cnt, g.kb, g.q);
            }
            mma_chunk2(w0, w1, af, g.qv, acc0, acc1);
        }
        const float gs = gscale[e];
        if constexpr (SPLIT == 1) {
            if (working) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 4 * g.q + j;
                    if (row < cnt) {
                        float *y = ws + (size_t)(base + row) * K + tp * 32 + g.n;
                        y[0] = acc0[j] * gs;
                        y[16] = acc1[j] * gs;
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                part[g.wave][0][4 * g.q + j][g.n] = acc0[j];
                part[g.wave][1][4 * g.q + j][g.n] = acc1[j];
            }
            __syncthreads();
            const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
#pragma unroll
            for (int p = 0; p < G::PAIRS; ++p) {
                const int tpx = (int)(u % upt) * G::PAIRS + p;
                if (tpx < npairs && row < cnt) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        float Y = part[p * SPLIT][t][row][col];
                        for (int cc = 1; cc < g.S; ++cc) Y += part[p * SPLIT + cc][t][row][col];
                        ws[(size_t)(base + row) * K + tpx * 32 + 16 * t + col] = Y * gs;
                    }
                }
            }
            __syncthreads();
        }
    }
}

// ---- slot-order weighted reduction: out[t][n] = fp16( fmaf chain over valid slots ) -----------------
// Each thread owns 4 consecutive columns of one token.
__global__ __launch_bounds__(256) void reduce_kernel(const int32_t *__restrict__ pos_of_pair, const float *__restrict__ tw,
                                                     const float *__restrict__ ws, int topk, int K, int blocks_per_token,
                                                     f16 *__restrict__ out)
{
    const int t = blockIdx.x / blocks_per_token;
    const int nb = blockIdx.x - t * blocks_per_token;
    const int n = (nb * 256 + threadIdx.x) * 4;
    if (n >= K) return;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    for (int k = 0; k < topk; ++k) {
        const int j = pos_of_pair[(size_t)t * topk + k];
        if (j < 0) continue;
        const float w = tw[(size_t)t * topk + k];
        const float4 y = *reinterpret_cast<const float4 *>(ws + (size_t)j * K + n);
        s0 = fmaf(w, y.x, s0);
        s1 = fmaf(w, y.y, s1);
        s2 = fmaf(w, y.z, s2);
        s3 = fmaf(w, y.w, s3);
    }
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<f16x4 *>(out + (size_t)t * K + n) = f16x4{(f16)s0, (f16)s1, (f16)s2, (f16)s3};
}

int split_for(int k)
{
    const int s = num_chunks(k);
    return s <= 1 ? 1 : (s <= 2 ? 2 : 4);
}

// Persistent grid: three 256-thread blocks per CU, never more blocks than units, and enough blocks
// that no block's unit range spans more than MAX_RANGE_TILES row tiles (range <= t_max/G + 2).
unsigned stream_grid(int64_t units_max, int64_t t_max)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    int64_t g = 3 * (int64_t)cus;
    const int64_t g_min = (t_max + MAX_RANGE_TILES - 3) / (MAX_RANGE_TILES - 2);
    if (g < g_min) g = g_min;
    if (g > units_max) g = units_max;
    return (unsigned)(g > 0 ? g : 1);
}

}  // namespace

int run_w13(const PlanView &pv, int64_t t_max, int32_t topk, const uint16_t *x, const nvfp4_weights &w, int32_t layout,
            uint16_t *h, hipStream_t s)
{
    const int K = w.k, I = w.rows / 2;
    const int split = split_for(K);
    const int pairs = 4 / split;
    const int upt = (I / 16 + pairs - 1) / pairs;
    const dim3 grid(stream_grid(t_max * upt, t_max)), block(256);
    const f16 *xp = reinterpret_cast<const f16 *>(x);
    f16 *hp = reinterpret_cast<f16 *>(h);
    switch (split) {
    case 1: return launch(w13_swiglu_stream_kernel<1>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp);
    case 2: return launch(w13_swiglu_stream_kernel<2>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp);
    default: return launch(w13_swiglu_stream_kernel<4>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, hp);
    }
}

int run_w2(const PlanView &pv, int64_t t_max, int32_t M, int32_t topk, const uint16_t *h, const nvfp4_weights &w,
           const float *topk_weights, uint16_t *out, float *ws, hipStream_t s)
{
    const int K = w.rows, I = w.k;
    const int split = split_for(I);
    const int pairs = 4 / split;
    const int upt = (K / 32 + pairs - 1) / pairs;
    const dim3 grid(stream_grid(t_max * upt, t_max)), block(256);
    const f16 *hp = reinterpret_cast<const f16 *>(h);
    int st;
    switch (split) {
    case 1: st = launch(w2_stream_kernel<1>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, ws); break;
    case 2: st = launch(w2_stream_kernel<2>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, ws); break;
    default: st = launch(w2_stream_kernel<4>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, ws); break;
    }
    if (st != NVFP4_OK) return st;
    return run_reduce(pv, M, topk, K, topk_weights, ws, out, s);
}

int run_reduce(const PlanView &pv, int32_t M, int32_t topk, int32_t K, const float *topk_weights, const float *ws,
               uint16_t *out, hipStream_t s)
{
    const int bpt = (K / 4 + 255) / 256;
    return launch(reduce_kernel, dim3((unsigned)((int64_t)M * bpt)), dim3(256), 0, s, pv.pos_of_pair, topk_weights,
                  ws, topk, K, bpt, reinterpret_cast<f16 *>(out));
}

}  // namespace nvfp4
