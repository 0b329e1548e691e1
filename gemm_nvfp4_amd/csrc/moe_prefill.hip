// moe_prefill.hip -- grouped expert GEMMs of the MoE layer, prefill (MFMA-bound) regime: the
// 8192-token, top-10 W13/W2 route of the "[Perf][SM70] Optimize Qwen3.8 Flash Next prefill" page
// ("SM70 QSA indexer hotspot update": default W13/W2 at 8192 tokens / top-10).
//
// With hundreds of pairs per expert the layer is a dense contraction (about 570 FLOP per weight
// byte), so the design goal is MFMA throughput. gfx950 design:
//   * A block owns one active expert and a slice of its output columns: 64 i values (gate and up
//     rows) for W13, or 128 output rows for W2. It walks the expert's bucket rows in passes of 96.
//     Blocks of one expert are numbered consecutively and mapped to the same XCD, so they share
//     the expert's activation rows in that XCD's L2.
//   * Each wave owns two 16-wide weight tiles (W13: gate and up of one i slice; W2: two output
//     tiles) and 6 row tiles. Per 512-element chunk it decodes its weights once (gfx950 fp4/fp8
//     converts plus one exact fp16 multiply) and reuses each B fragment for all 6 row tiles.
//   * Activation rows are staged in LDS a quarter chunk at a time: lane group q's 32 elements
//     for step group b, for every row. Staging is double-buffered, so the global loads of the next
//     quarter overlap the MFMAs of the current one.
//   * The reduction order is the library-wide one of nvfp4_device.hpp: 512-element chunks, each
//     a chain of 16 MFMA steps from +0, chunk results added in order, global scale last. Results
//     are bitwise identical to the streaming (decode) kernels, so batch invariance holds across
//     regimes.
//   * W13's epilogue runs straight from registers: gate and up of one (row, i) sit in the same
//     lane. It applies SwiGLU and stores fp16 h. W2's epilogue stores per-pair FP32 results for
//     the slot-order reduction.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int PF_R = 6;                 // row tiles per wave
constexpr int PF_ROWS = 16 * PF_R;      // bucket rows per pass
constexpr int AQ = 32;                  // elements of one lane group per step group (4 steps x 8)
constexpr int A_ROW = 4 * AQ + 8;       // staged halves per row: 4 lane groups + 16 bytes of bank padding
constexpr int STAGE_PIECES = PF_ROWS * 16;  // 16-byte pieces per staged quarter chunk
constexpr int PIECES_PER_THREAD = (STAGE_PIECES + 255) / 256;

struct PrefillShared {
    f16 a[2][PF_ROWS][A_ROW];  // double-buffered activation quarter chunks
    int arow[PF_ROWS];         // activation row (token or bucket row) of each pass row
};

// Logical block index with blocks of one expert kept on one XCD: the hardware deals block ids to
// the 8 XCDs round-robin, so logical = xcd * ceil(G/8) + slot puts consecutive logical blocks on the
// same XCD. Returns -1 for the padding ids of the last XCD.
__device__ __forceinline__ int xcd_logical_block(int G)
{
    const int per = (G + 7) >> 3;
    const int logical = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
    return logical < G ? logical : -1;
}

// Global loads of one quarter chunk (step group b of chunk kb) for `rows` rows into registers:
// piece = row * 16 + q * 4 + p covers elements [kb + 128q + 32b + 8p, +8) of the row.
struct StageRegs {
    u32x4 v[PIECES_PER_THREAD];
};

__device__ __forceinline__ void stage_load(StageRegs &s, const f16 *src, int L, const int *arow, int rows, int kb,
                                           int b, int groups)
{
#pragma unroll
    for (int i = 0; i < PIECES_PER_THREAD; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int r = idx >> 4, q = (idx >> 2) & 3, p = idx & 3;
        if (r < rows && q < groups)
            s.v[i] = *reinterpret_cast<const u32x4 *>(src + (size_t)arow[r] * L + kb + 128 * q + AQ * b + 8 * p);
    }
}

__device__ __forceinline__ void stage_store(const StageRegs &s, f16 (*a)[A_ROW], int rows, int groups)
{
#pragma unroll
    for (int i = 0; i < PIECES_PER_THREAD; ++i) {
        const int idx = threadIdx.x + 256 * i;
        const int r = idx >> 4, q = (idx >> 2) & 3, p = idx & 3;
        if (r < rows && q < groups) *reinterpret_cast<u32x4 *>(&a[r][AQ * q + 8 * p]) = s.v[i];
    }
}

// One chunk of two weight rows against the pass's staged activation rows.
// acc[r][t]: row tile r, weight tile t. Staging of quarter b+1 overlaps the MFMAs of quarter b.
__device__ __forceinline__ void chunk_pass(PrefillShared &sh, const f16 *src, int L, int rows, int kb, int groups,
                                           const RawChunk &w0, const RawChunk &w1, bool working, int n, int q,
                                           f32x4 acc[PF_R][2])
{
    const bool qv = q < groups;
    StageRegs st;
    stage_load(st, src, L, sh.arow, rows, kb, 0, groups);
    stage_store(st, sh.a[0], rows, groups);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if (b < 3) stage_load(st, src, L, sh.arow, rows, kb, b + 1, groups);
        if (working) {
            const f16x2 sc0 = chunk_scales(w0, b), sc1 = chunk_scales(w1, b);
            f16x8 b0[4], b1[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                b0[s] = b_frag(w0, sc0, b, s, qv);
                b1[s] = b_frag(w1, sc1, b, s, qv);
            }
            const f16(*a)[A_ROW] = sh.a[b & 1];
#pragma unroll
            for (int r = 0; r < PF_R; ++r) {
                if (16 * r >= rows) break;
                const int row = 16 * r + n;
                const bool rv = row < rows && qv;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f16x8 av = rv ? *reinterpret_cast<const f16x8 *>(&a[row][AQ * q + 8 * s]) : zero8();
                    acc[r][0] = mfma_step(av, b0[s], acc[r][0]);
                    acc[r][1] = mfma_step(av, b1[s], acc[r][1]);
                }
            }
        }
        if (b < 3) stage_store(st, sh.a[(b + 1) & 1], rows, groups);
        __syncthreads();
    }
}

// ---- W13 + SwiGLU ---------------------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void w13_swiglu_prefill_kernel(PlanView pv, int topk, const f16 *__restrict__ x,
                                                                     const uint8_t *__restrict__ codes,
                                                                     const uint8_t *__restrict__ scales,
                                                                     const float *__restrict__ gscale, int K, int I,
                                                                     int layout, f16 *__restrict__ h, int a_max)
{
    __shared__ PrefillShared sh;
    const int itiles = I >> 4;
    const int nblk = (itiles + 3) >> 2;  // 4 i slices (one per wave) per block
    const int lb = xcd_logical_block(a_max * nblk);
    if (lb < 0) return;
    const int a = lb / nblk, nb = lb - a * nblk;
    if (a >= pv.hdr[1]) return;  // block-uniform
    const int e = pv.active[a], cnt = pv.counts[e], base = pv.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, q = lane >> 4;
    const int it = nb * 4 + wave;
    const bool working = it < itiles;
    const int itc = working ? it : itiles - 1;
    const int i_row = itc * 16 + n;
    const size_t eb = (size_t)e * 2 * I, crow = (size_t)K >> 1, srow = (size_t)K >> 4;
    const size_t rg = eb + (layout ? 2 * i_row : i_row), ru = eb + (layout ? 2 * i_row + 1 : I + i_row);
    const float gs = gscale[e];
    const int S = num_chunks(K);

    for (int rp = 0; rp < cnt; rp += PF_ROWS) {
        const int rows = min(PF_ROWS, cnt - rp);
        __syncthreads();  // the previous pass is done with sh.arow
        for (int r = threadIdx.x; r < rows; r += 256) sh.arow[r] = pv.sorted_pair[base + rp + r] / topk;
        __syncthreads();
        f32x4 tot[PF_R][2];
        for (int c = 0; c < S; ++c) {
            const int kb = c * KCHUNK;
            const int groups = min(KCHUNK, K - kb) >> 7;
            const int q_ld = q < groups ? q : groups - 1;
            const RawChunk wg = load_chunk(codes + rg * crow, scales + rg * srow, kb, q_ld);
            const RawChunk wu = load_chunk(codes + ru * crow, scales + ru * srow, kb, q_ld);
            f32x4 ca[PF_R][2];
#pragma unroll
            for (int r = 0; r < PF_R; ++r) ca[r][0] = ca[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            chunk_pass(sh, x, K, rows, kb, groups, wg, wu, working, n, q, ca);
#pragma unroll
            for (int r = 0; r < PF_R; ++r)
#pragma unroll
                for (int t = 0; t < 2; ++t) tot[r][t] = c == 0 ? ca[r][t] : tot[r][t] + ca[r][t];
        }
        if (working) {
#pragma unroll
            for (int r = 0; r < PF_R; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * r + 4 * q + j;
                    if (row < rows)
                        h[(size_t)(base + rp + row) * I + it * 16 + n] = (f16)swiglu(tot[r][0][j] * gs, tot[r][1][j] * gs);
                }
        }
    }
}

// ---- W2: per-pair FP32 results -----------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void w2_prefill_kernel(PlanView pv, const f16 *__restrict__ hin,
                                                             const uint8_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ scales,
                                                             const float *__restrict__ gscale, int K, int I,
                                                             float *__restrict__ ws, int a_max)
{
    __shared__ PrefillShared sh;
    const int npairs = K >> 5;             // pairs of 16-row output tiles
    const int nblk = (npairs + 3) >> 2;    // 4 tile pairs (one per wave) per block
    const int lb = xcd_logical_block(a_max * nblk);
    if (lb < 0) return;
    const int a = lb / nblk, nb = lb - a * nblk;
    if (a >= pv.hdr[1]) return;
    const int e = pv.active[a], cnt = pv.counts[e], base = pv.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, q = lane >> 4;
    const int tp = nb * 4 + wave;
    const bool working = tp < npairs;
    const int tpc = working ? tp : npairs - 1;
    const size_t r0 = (size_t)e * K + tpc * 32 + n, r1 = r0 + 16;
    const size_t crow = (size_t)I >> 1, srow = (size_t)I >> 4;
    const float gs = gscale[e];
    const int S = num_chunks(I);

    for (int rp = 0; rp < cnt; rp += PF_ROWS) {
        const int rows = min(PF_ROWS, cnt - rp);
        __syncthreads();
        for (int r = threadIdx.x; r < rows; r += 256) sh.arow[r] = base + rp + r;
        __syncthreads();
        f32x4 tot[PF_R][2];
        for (int c = 0; c < S; ++c) {
            const int kb = c * KCHUNK;
            const int groups = min(KCHUNK, I - kb) >> 7;
            const int q_ld = q < groups ? q : groups - 1;
            const RawChunk w0 = load_chunk(codes + r0 * crow, scales + r0 * srow, kb, q_ld);
            const RawChunk w1 = load_chunk(codes + r1 * crow, scales + r1 * srow, kb, q_ld);
            f32x4 ca[PF_R][2];
#pragma unroll
            for (int r = 0; r < PF_R; ++r) ca[r][0] = ca[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            chunk_pass(sh, hin, I, rows, kb, groups, w0, w1, working, n, q, ca);
#pragma unroll
            for (int r = 0; r < PF_R; ++r)
#pragma unroll
                for (int t = 0; t < 2; ++t) tot[r][t] = c == 0 ? ca[r][t] : tot[r][t] + ca[r][t];
        }
        if (working) {
#pragma unroll
            for (int r = 0; r < PF_R; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * r + 4 * q + j;
                    if (row < rows) {
                        float *y = ws + (size_t)(base + rp + row) * K + tp * 32 + n;
                        y[0] = tot[r][0][j] * gs;
                        y[16] = tot[r][1][j] * gs;
                    }
                }
        }
    }
}

}  // namespace

int run_w13_prefill(const PlanView &pv, int64_t a_max, int32_t topk, const uint16_t *x, const nvfp4_weights &w,
                    int32_t layout, uint16_t *h, hipStream_t s)
{
    const int K = w.k, I = w.rows / 2;
    const int nblk = (I / 16 + 3) / 4;
    const int64_t G = a_max * nblk;
    const unsigned grid = (unsigned)((G + 7) / 8 * 8);
    return launch(w13_swiglu_prefill_kernel, dim3(grid), dim3(256), 0, s, pv, topk, reinterpret_cast<const f16 *>(x),
                  w.codes, w.scales, w.global_scale, K, I, layout, reinterpret_cast<f16 *>(h), (int)a_max);
}

int run_w2_prefill(const PlanView &pv, int64_t a_max, const uint16_t *h, const nvfp4_weights &w, float *ws,
                   hipStream_t s)
{
    const int K = w.rows, I = w.k;
    const int nblk = (K / 32 + 3) / 4;
    const int64_t G = a_max * nblk;
    const unsigned grid = (unsigned)((G + 7) / 8 * 8);
    return launch(w2_prefill_kernel, dim3(grid), dim3(256), 0, s, pv, reinterpret_cast<const f16 *>(h), w.codes,
                  w.scales, w.global_scale, K, I, ws, (int)a_max);
}

}  // namespace nvfp4
