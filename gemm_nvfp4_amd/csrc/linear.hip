// linear.hip -- dense NVFP4 projection y = fp16(global * x W^T), the "QPN" projection of the
// "[SM70][Draft] Extend Qwen3.8 DFlash2 concurrency paths" page ("Purpose": independent row tiles
// admitted through M <= 32; "TP4-only NVFP4 verifier follow-up": two-row-tile CTAs that reuse the
// loaded packed weights while keeping the split-K / FP32 reduction order), and its gated form for
// the packed gate/up projection of a dense MLP (same page and section: the gate/up and down
// projections of the packed MLP weights): h = fp16(silu(g) * u) with g and u the projections on
// the gate and up rows.
//
// gfx950 design: one block per R consecutive output columns (weight rows; gate and up rows of R h
// columns in the gated form), R chosen so that the blocks cover every CU with an equal share of the
// weight bytes (each CU's load path, not HBM, limits a small launch: at 4352 rows, 17 columns on
// 256 blocks instead of 32 on 136 took the one-token projection from 8.9 to 8.5 us). Its waves share
// the reduction axis, one 512-element chunk each (intra-block split-K). A wave decodes its chunk into
// MFMA B fragments in registers and applies them to every 16-row tile of x, so at small M the weight
// bytes are read from HBM exactly once. Chunk
// partials meet in LDS and are added in chunk order, which is the same reduction order as every
// other GEMM here; the gated epilogue is the MoE W13 epilogue (global scale, then SwiGLU). A batch
// of any size is therefore bitwise equal to single-row calls, and the gated form equals the
// grouped W13 of a one-expert MoE bitwise.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int LDS_ROW = 20;
// Waves per block: one per 512-element chunk up to ten (K = 5120), so every chunk's weights are
// requested in the first round of loads; longer reductions take further chunks in turn. Ten waves
// leave 168 registers per wave, which the row-tile loop below stays within by not being unrolled
// (unrolled, the compiler keeps one row tile's decoded weights live for the next: 222 registers).
constexpr int MAX_WAVES = 10;

constexpr int ROW_GROUP = 2;    // 16-row tiles of x handled per pass over the weights

// Small batches stage each wave's activation chunk in LDS: one 16-byte direct-to-LDS load per lane
// and row (gfx950 global_load_lds_dwordx4: lane i's bytes land at the row's base + 16 i) brings a
// whole 1 KB chunk row in with one instruction, where the fragment loads take sixteen per row tile
// whatever the number of rows (at one token, 60% of a CU's load instructions, with 4 of 64 lanes
// active each; a CU's load issue, not HBM, bounds these launches). Row pitch 1040 bytes: the
// fragment reads of 16 rows and two lane groups hit distinct 16-byte bank slots.
constexpr int XS_ROWS = 8;       // batches up to this many rows stage (M * 1040 bytes per wave)
constexpr int XS_PITCH = 1040;

// Rows [0, M) of the activation chunk starting at element kb into this wave's LDS rows. Lanes past
// K load the row's first 16 bytes into the tail of the row's slot, which no fragment reads (lane
// groups past the chunk end feed zeros).
__device__ __forceinline__ void stage_x_chunk(const f16 *x, int M, int K, int kb, unsigned char *xw, int lane)
{
    const int k = kb + 8 * lane;
    for (int r = 0; r < M; ++r) {
        const f16 *src = x + (size_t)r * K + (k < K ? k : 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                         (__attribute__((address_space(3))) void *)(xw + r * XS_PITCH), 16, 0, 0);
    }
}

// An empty asm that the compiler must treat as changing the weight registers: placed inside the
// row-tile loop, it keeps the decode there. Hoisted out of the loop, the decoded fragments would hold
// 128 registers across it (spills) and the decode would wait for the weights before the A loads of
// the first row tile are issued. No instruction is emitted.
__device__ __forceinline__ void keep_in_loop(RawChunk &w)
{
#pragma unroll
    for (int b = 0; b < 4; ++b) asm volatile("" : "+v"(w.codes[b]));
    asm volatile("" : "+v"(w.scales[0]), "+v"(w.scales[1]));
}

// Where a kernel's A fragments come from.
enum AFrom { A_GLOBAL, A_BUFFER, A_STAGED };

// The A fragments of one 16-row tile, row m of the pass's M rows (xg: the pass's first row): from
// this wave's staged LDS rows (A_STAGED: the pass is rows 0..M-1 of x), or from x by loads that only
// valid lanes issue (A_GLOBAL) or by buffer loads that all lanes issue, at an out-of-range offset for
// the others (A_BUFFER: no branch, so no wait for the earlier loads at the merge; measured faster
// for the channel-FP8 kernel, slower for the NVFP4 one). Rows at or past M, and lane groups past the
// chunk end, are zeros.
template <AFrom AF>
__device__ __forceinline__ void load_a_tile(f16x8 (&af)[4][4], const f16 *xg, rsrc_t xr, const unsigned char *xw,
                                            int m, int M, int K, int kb, int q, bool qv)
{
    const bool v = m < M && qv;
    if constexpr (AF == A_STAGED) {
        // The compiler does not order LDS reads after the direct-to-LDS loads that fill them: wait
        // for every load of this wave (vmcnt(0); expcnt and lgkmcnt left at their maxima).
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // an LDS-typed pointer, so that the reads are ds_read_b128 and not flat loads
        typedef const __attribute__((address_space(3))) f16x8 lds_f16x8;
        lds_f16x8 *p = (lds_f16x8 *)(xw + (v ? m : 0) * XS_PITCH + 256 * q);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s) af[b][s] = v ? p[4 * b + s] : zero8();
    } else if constexpr (AF == A_BUFFER) {
        const uint32_t o = v ? (uint32_t)(m * K + kb + 128 * q) * 2u : BUF_OOB;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s) af[b][s] = __builtin_bit_cast(f16x8, bload16(xr, o + 64 * b + 16 * s, 0));
    } else {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s) af[b][s] = zero8();
        if (v) {
            const f16 *xp = xg + (size_t)m * K;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) af[b][s] = a_frag(xp, kb, q, b, s);
        }
    }
}

// Each wave holds NW 16-row weight tiles. Block nt owns output columns nt*R .. nt*R + R - 1 (R at
// most 16*NW plain, 16 gated). Plain (GATED false): lane n of tile t takes column nt*R + 16t + n.
// Gated: tile 0 holds the gate rows and tile 1 the up rows of h columns nt*R + n (layout 0: rows i
// and I + i; layout 1: rows 2i and 2i + 1). Lanes of columns outside the block's range read zero
// weights; an MFMA column depends only on its own operands, so a column's result is the same
// whatever R is.
// OUT is the output type: fp16 (rounded once), or FP32 for a result that is summed further (the
// shared expert's down projection, added into the MoE output before its one rounding).
template <int NW, bool GATED, typename OUT, bool XS>
__global__ __launch_bounds__(MAX_WAVES * 64) void linear_kernel(const f16 *__restrict__ x, int M,
                                                                 const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 const float *__restrict__ gscale, int N, int K,
                                                                 int layout, OUT *__restrict__ y, int R)
{
    extern __shared__ float part[];  // [S][ROW_GROUP][NW][16][LDS_ROW], then with XS the staged rows
    const int nt = blockIdx.x;
    const int col0 = nt * R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int S = num_chunks(K);
    const int row_tiles = (M + 15) >> 4;
    const uint8_t *cr[NW], *sr[NW];
    bool cv[NW];  // this lane's column of tile t lies in the block's range
#pragma unroll
    for (int t = 0; t < NW; ++t) {
        const int lc = GATED ? n : 16 * t + n;  // column within the block
        cv[t] = lc < R && col0 + lc < N;
        const int col = cv[t] ? col0 + lc : 0;
        const size_t wrow = GATED ? (size_t)(layout ? 2 * col + t : t * N + col) : (size_t)col;
        cr[t] = codes + wrow * ((size_t)K >> 1);
        sr[t] = scales + wrow * ((size_t)K >> 4);
    }
    const float gs = gscale[0];
    unsigned char *xw = reinterpret_cast<unsigned char *>(part + (size_t)S * ROW_GROUP * NW * 16 * LDS_ROW) +
                        (size_t)wave * M * XS_PITCH;

    for (int rt0 = 0; rt0 < row_tiles; rt0 += ROW_GROUP) {
        // x rows of this pass (offsets relative to its first row stay within 32 bits)
        const int gm = min(M - 16 * rt0, 16 * ROW_GROUP);
        const f16 *xg = x + (size_t)16 * rt0 * K;
        const rsrc_t xr = make_rsrc(xg, (uint32_t)gm * (uint32_t)K * 2u);
        for (int c = wave; c < S; c += nwaves) {
            const int kb = c * KCHUNK;
            const int groups = min(KCHUNK, K - kb) >> 7;  // 128-element lane groups with data
            const bool qv = q < groups;
            // Lanes outside the block's columns or past the chunk end load nothing (masked lanes cost
            // the address unit nothing; a buffer load at an out-of-range offset would) and keep the
            // zero codes and scales, which decode to exact zeros.
            RawChunk w[NW];
#pragma unroll
            for (int t = 0; t < NW; ++t) {
                w[t] = RawChunk{};
                if (cv[t] && qv) w[t] = load_chunk(cr[t], sr[t], kb, q);
            }
            if constexpr (XS) stage_x_chunk(x, M, K, kb, xw, lane);
#pragma unroll 1
            for (int r = 0; r < ROW_GROUP; ++r) {
                const int rt = rt0 + r;
                if (rt >= row_tiles) break;
                // All 16 A fragments are read before the chain, back to back, so their latencies
                // overlap.
                f16x8 af[4][4];
                load_a_tile<XS ? A_STAGED : A_GLOBAL>(af, xg, xr, xw, r * 16 + n, gm, K, kb, q, qv);
                __builtin_amdgcn_sched_barrier(0);  // every load (weights, then A) is issued before the math
#pragma unroll
                for (int t = 0; t < NW; ++t) keep_in_loop(w[t]);
                f32x4 acc[NW];
#pragma unroll
                for (int t = 0; t < NW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    f16x2 sc[NW];
#pragma unroll
                    for (int t = 0; t < NW; ++t) sc[t] = chunk_scales(w[t], b);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int t = 0; t < NW; ++t) acc[t] = mfma_step(af[b][s], decode8(w[t].codes[b][s], sc[t][s >> 1]), acc[t]);
                }
#pragma unroll
                for (int t = 0; t < NW; ++t) {
                    float *pc = part + (((size_t)c * ROW_GROUP + r) * NW + t) * 16 * LDS_ROW;
#pragma unroll
                    for (int j = 0; j < 4; ++j) pc[(4 * q + j) * LDS_ROW + n] = acc[t][j];
                }
            }
        }
        __syncthreads();
        for (int o = threadIdx.x; o < ROW_GROUP * 256; o += blockDim.x) {
            const int r = o >> 8, row = (o >> 4) & 15, cl = o & 15;
            const int m = (rt0 + r) * 16 + row;
            if (rt0 + r < row_tiles && m < M) {
                float tot[NW];
#pragma unroll
                for (int t = 0; t < NW; ++t) {
                    tot[t] = part[(((size_t)0 * ROW_GROUP + r) * NW + t) * 16 * LDS_ROW + row * LDS_ROW + cl];
                    for (int c = 1; c < S; ++c)
                        tot[t] += part[(((size_t)c * ROW_GROUP + r) * NW + t) * 16 * LDS_ROW + row * LDS_ROW + cl];
                }
                if constexpr (GATED) {
                    if (cl < R && col0 + cl < N) y[(size_t)m * N + col0 + cl] = f16_of_f32(swiglu(tot[0] * gs, tot[1] * gs));
                } else {
#pragma unroll
                    for (int t = 0; t < NW; ++t) {
                        const int lc = 16 * t + cl;
                        if (lc < R && col0 + lc < N) y[(size_t)m * N + col0 + lc] = to_out<OUT>(tot[t] * gs);
                    }
                }
            }
        }
        __syncthreads();
    }
}

// ---- channel-FP8 ("QPN8") weights ----------------------------------------------------------------
// The channel-FP8 projection of the same page ("Follow-up: exact channel-FP8 QPN8 concurrency
// paths and endpoint evidence"): E4M3FN weight bytes with one FP32 scale per output channel. An
// E4M3 byte converts to fp16 exactly (one gfx950 convert per pair, no block scale), the MFMA chain
// and the chunk order are the library's, and the channel scale multiplies the FP32 sum in the
// epilogue, where it is exact arithmetic on the definition (the pages apply it before the MMA).

// One lane's bytes of one weight row for one chunk: lane group q's 128 elements, eight 16-byte loads.
struct Fp8Chunk {
    u32x4 codes[8];  // codes[j] = elements [kb + 128q + 16j, +16)
};

// B fragment of step (b, s): elements [128q + 32b + 8s, +8), i.e. half of load 2b + s/2.
__device__ __forceinline__ f16x8 b_frag8(const Fp8Chunk &r, int b, int s)
{
    const u32x4 v = r.codes[2 * b + (s >> 1)];
    const uint32_t d0 = v[2 * (s & 1)], d1 = v[2 * (s & 1) + 1];
    const f16x2 p0 = e4m3_pair<false>(d0), p1 = e4m3_pair<true>(d0), p2 = e4m3_pair<false>(d1), p3 = e4m3_pair<true>(d1);
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Up to two 16-row weight tiles per wave, block nt owning output columns nt*R .. +R-1, as the
// NVFP4 kernel.
// Eight waves: the channel-FP8 chunk holds twice the packed bytes of an NVFP4 one (two weight tiles
// take 64 registers), so ten waves would spill; at K = 5120 two waves take a second chunk.
constexpr int FP8_WAVES = 8;
template <int NW, bool XS>
__global__ __launch_bounds__(FP8_WAVES * 64) void linear_fp8_kernel(const f16 *__restrict__ x, int M,
                                                          const uint8_t *__restrict__ codes,
                                                          const float *__restrict__ chscale, int N, int K,
                                                          f16 *__restrict__ y, int R)
{
    extern __shared__ float part[];  // [S][ROW_GROUP][NW][16][LDS_ROW], then with XS the staged rows
    const int nt = blockIdx.x;
    const int col0 = nt * R;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int S = num_chunks(K);
    const int row_tiles = (M + 15) >> 4;
    const uint8_t *cr[NW];
    bool cv[NW];
#pragma unroll
    for (int t = 0; t < NW; ++t) {
        cv[t] = 16 * t + n < R && col0 + 16 * t + n < N;
        cr[t] = codes + (size_t)(cv[t] ? col0 + 16 * t + n : 0) * K;
    }
    unsigned char *xw = reinterpret_cast<unsigned char *>(part + (size_t)S * ROW_GROUP * NW * 16 * LDS_ROW) +
                        (size_t)wave * M * XS_PITCH;

    for (int rt0 = 0; rt0 < row_tiles; rt0 += ROW_GROUP) {
        // x rows of this pass (offsets relative to its first row stay within 32 bits)
        const int gm = min(M - 16 * rt0, 16 * ROW_GROUP);
        const f16 *xg = x + (size_t)16 * rt0 * K;
        const rsrc_t xr = make_rsrc(xg, (uint32_t)gm * (uint32_t)K * 2u);
        for (int c = wave; c < S; c += nwaves) {
            const int kb = c * KCHUNK;
            const int groups = min(KCHUNK, K - kb) >> 7;
            const bool qv = q < groups;
            Fp8Chunk w[NW];  // as in linear_kernel: masked lanes keep zero bytes, exact zero weights
#pragma unroll
            for (int t = 0; t < NW; ++t) {
                w[t] = Fp8Chunk{};
                if (cv[t] && qv) {
                    const uint8_t *c = cr[t] + kb + 128 * q;
#pragma unroll
                    for (int j = 0; j < 8; ++j) w[t].codes[j] = *reinterpret_cast<const u32x4 *>(c + 16 * j);
                }
            }
            if constexpr (XS) stage_x_chunk(x, M, K, kb, xw, lane);
#pragma unroll
            for (int r = 0; r < ROW_GROUP; ++r) {
                const int rt = rt0 + r;
                if (rt >= row_tiles) break;
                f16x8 af[4][4];
                load_a_tile<XS ? A_STAGED : A_BUFFER>(af, xg, xr, xw, r * 16 + n, gm, K, kb, q, qv);
                __builtin_amdgcn_sched_barrier(0);  // every load (weights, then A) is issued before the math
                f32x4 acc[NW];
#pragma unroll
                for (int t = 0; t < NW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int t = 0; t < NW; ++t) acc[t] = mfma_step(af[b][s], b_frag8(w[t], b, s), acc[t]);
#pragma unroll
                for (int t = 0; t < NW; ++t) {
                    float *pc = part + (((size_t)c * ROW_GROUP + r) * NW + t) * 16 * LDS_ROW;
#pragma unroll
                    for (int j = 0; j < 4; ++j) pc[(4 * q + j) * LDS_ROW + n] = acc[t][j];
                }
            }
        }
        __syncthreads();
        for (int o = threadIdx.x; o < ROW_GROUP * 256; o += blockDim.x) {
            const int r = o >> 8, row = (o >> 4) & 15, cl = o & 15;
            const int m = (rt0 + r) * 16 + row;
            if (rt0 + r < row_tiles && m < M) {
#pragma unroll
                for (int t = 0; t < NW; ++t) {
                    float tot = part[(((size_t)0 * ROW_GROUP + r) * NW + t) * 16 * LDS_ROW + row * LDS_ROW + cl];
                    for (int c = 1; c < S; ++c)
                        tot += part[(((size_t)c * ROW_GROUP + r) * NW + t) * 16 * LDS_ROW + row * LDS_ROW + cl];
                    const int colx = col0 + 16 * t + cl;
                    if (16 * t + cl < R && colx < N) y[(size_t)m * N + colx] = f16_of_f32(tot * chscale[colx]);
                }
            }
        }
        __syncthreads();
    }
}

// ---- split-K form (workspace) ---------------------------------------------------------------------
// The same products with the reduction split across blocks and a second launch that adds the chunk
// partials. In the one-launch kernel every block reads all of x (M * K * 2 bytes; 327 KB per CU at
// 32 rows of 5120), which bounds it once M grows. Here block b takes chunk c = b % S and T
// consecutive 16-row weight tiles, one per wave, so a CU reads one chunk of x (M KB) and T tiles of
// that chunk's weights. Each wave's FP32 chain result for (chunk c, rows, its 16 weight rows) is
// stored to part[c][m][n]; the fold launch adds part[0..S-1] in chunk order and applies the same
// epilogue as the one-launch kernel, so the outputs are bitwise those of nvfp4_linear and
// nvfp4_linear_swiglu.
constexpr int SPLIT_ROWS = 32;  // activation rows staged in LDS per pass
constexpr int SPLIT_WAVES = 12;  // three waves per SIMD: room for the decoded fragments (168 registers)

__global__ __launch_bounds__(SPLIT_WAVES * 64) void linear_partials_kernel(const f16 *__restrict__ x, int M,
                                                                           const uint8_t *__restrict__ codes,
                                                                           const uint8_t *__restrict__ scales, int N,
                                                                           int K, float *__restrict__ part)
{
    __shared__ __attribute__((aligned(16))) unsigned char xs[SPLIT_ROWS * XS_PITCH];
    const int S = num_chunks(K);
    const int c = blockIdx.x % S;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int t = (blockIdx.x / S) * nwaves + wave;  // this wave's weight tile
    const bool tv = t < (N >> 4);                    // wave-uniform
    const int kb = c * KCHUNK;
    const bool qv = q < (min(KCHUNK, K - kb) >> 7);
    // The weights first, so that they are in flight while the activations are staged.
    RawChunk w = RawChunk{};
    if (tv && qv) {
        const size_t row = (size_t)t * 16 + n;
        w = load_chunk(codes + row * ((size_t)K >> 1), scales + row * ((size_t)K >> 4), kb, q);
    }
    const int k = kb + 8 * lane;
    for (int m0 = 0; m0 < M; m0 += SPLIT_ROWS) {
        const int gm = min(M - m0, SPLIT_ROWS);
        if (m0 > 0) lds_barrier();  // the previous pass's fragment reads are done
        for (int r = wave; r < gm; r += nwaves) {
            const f16 *src = x + (size_t)(m0 + r) * K + (k < K ? k : 0);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(xs + r * XS_PITCH), 16, 0, 0);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's direct-to-LDS loads (and weights) are done
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        lds_barrier();                       // and every other wave's
        if (!tv) continue;
        // One tile per wave leaves room to keep the decoded B fragments for every row tile.
        f16x8 bf[4][4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const f16x2 sc = chunk_scales(w, b);
#pragma unroll
            for (int s = 0; s < 4; ++s) bf[b][s] = decode8(w.codes[b][s], sc[s >> 1]);
        }
#pragma unroll 1
        for (int rt = 0; rt * 16 < gm; ++rt) {
            f16x8 af[4][4];
            load_a_tile<A_STAGED>(af, x, make_rsrc(x, 0), xs, rt * 16 + n, gm, K, kb, q, qv);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mfma_step(af[b][s], bf[b][s], acc);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int m = m0 + rt * 16 + 4 * q + j;
                if (m < M) part[((size_t)c * M + m) * N + (size_t)t * 16 + n] = acc[j];
            }
        }
    }
}

// y = epilogue(sum over c of part[c]) for 4 consecutive output columns per thread. Plain: the N
// weight rows are the N columns of y (fp16, or FP32 for OUT = float). Gated: y has N/2 columns, h
// column i from weight rows g(i) and u(i) of the layout, as the one-launch kernel.
constexpr int FOLD_THREADS = 64;  // small blocks: the fold's few threads spread over many CUs

template <bool GATED, typename OUT>
__global__ __launch_bounds__(FOLD_THREADS) void linear_fold_kernel(const float *__restrict__ part, int S, int M, int N,
                                                          const float *__restrict__ gscale, int layout,
                                                          OUT *__restrict__ y)
{
    const int Ny = GATED ? N >> 1 : N;
    const size_t i = ((size_t)blockIdx.x * FOLD_THREADS + threadIdx.x) * 4;
    if (i >= (size_t)M * Ny) return;
    const int m = (int)(i / Ny), col = (int)(i % Ny);
    const size_t plane = (size_t)M * N;
    const float *p = part + (size_t)m * N;
    const float gs = gscale[0];
    // Sums of the chunk partials of weight rows ra .. ra + 3 and (GATED) rb .. rb + 3, each in chunk
    // order, with the loads of up to FB chunks of both issued before their adds.
    constexpr int FB = GATED ? 8 : 16;
    auto chunk_sums = [&](int ra, int rb, float4 &ta, float4 &tb) {
        ta = *reinterpret_cast<const float4 *>(p + ra);
        if (GATED) tb = *reinterpret_cast<const float4 *>(p + rb);
        for (int c0 = 1; c0 < S; c0 += FB) {
            float4 va[FB], vb[FB];
#pragma unroll
            for (int e = 0; e < FB; ++e)
                if (c0 + e < S) {
                    va[e] = *reinterpret_cast<const float4 *>(p + (size_t)(c0 + e) * plane + ra);
                    if (GATED) vb[e] = *reinterpret_cast<const float4 *>(p + (size_t)(c0 + e) * plane + rb);
                }
#pragma unroll
            for (int e = 0; e < FB; ++e)
                if (c0 + e < S) {
                    ta.x += va[e].x, ta.y += va[e].y, ta.z += va[e].z, ta.w += va[e].w;
                    if (GATED) tb.x += vb[e].x, tb.y += vb[e].y, tb.z += vb[e].z, tb.w += vb[e].w;
                }
        }
    };
    OUT *yo = y + (size_t)m * Ny + col;
    if constexpr (GATED) {
        float g[4], u[4];
        float4 a, b;
        if (layout) {  // gate and up rows interleaved: rows 2i, 2i + 1
            chunk_sums(2 * col, 2 * col + 4, a, b);
            g[0] = a.x, u[0] = a.y, g[1] = a.z, u[1] = a.w, g[2] = b.x, u[2] = b.y, g[3] = b.z, u[3] = b.w;
        } else {
            chunk_sums(col, Ny + col, a, b);
            g[0] = a.x, g[1] = a.y, g[2] = a.z, g[3] = a.w, u[0] = b.x, u[1] = b.y, u[2] = b.z, u[3] = b.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) yo[e] = f16_of_f32(swiglu(g[e] * gs, u[e] * gs));
    } else {
        float4 a, b;
        chunk_sums(col, col, a, b);
        yo[0] = to_out<OUT>(a.x * gs);
        yo[1] = to_out<OUT>(a.y * gs);
        yo[2] = to_out<OUT>(a.z * gs);
        yo[3] = to_out<OUT>(a.w * gs);
    }
}

template <typename KernelT>
hipError_t allow_lds(KernelT *kernel)
{
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)MAX_LDS_BYTES);
}

}  // namespace

// Opt every dense kernel into the CU's whole LDS (beyond the 64 KiB default), once per device.
int linear_prepare()
{
    static std::atomic<int> done[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return NVFP4_ERR_LAUNCH;
    if (dev < 64 && done[dev].load(std::memory_order_acquire)) return NVFP4_OK;
    hipError_t e = hipSuccess;
    for (int xs = 0; xs < 2 && e == hipSuccess; ++xs) {
        e = allow_lds(xs ? linear_kernel<1, false, f16, true> : linear_kernel<1, false, f16, false>);
        if (e == hipSuccess) e = allow_lds(xs ? linear_kernel<2, false, f16, true> : linear_kernel<2, false, f16, false>);
        if (e == hipSuccess)
            e = allow_lds(xs ? linear_kernel<1, false, float, true> : linear_kernel<1, false, float, false>);
        if (e == hipSuccess)
            e = allow_lds(xs ? linear_kernel<2, false, float, true> : linear_kernel<2, false, float, false>);
        if (e == hipSuccess) e = allow_lds(xs ? linear_kernel<2, true, f16, true> : linear_kernel<2, true, f16, false>);
        if (e == hipSuccess) e = allow_lds(xs ? linear_fp8_kernel<1, true> : linear_fp8_kernel<1, false>);
        if (e == hipSuccess) e = allow_lds(xs ? linear_fp8_kernel<2, true> : linear_fp8_kernel<2, false>);
    }
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
    if (dev < 64) done[dev].store(1, std::memory_order_release);
    return NVFP4_OK;
}

namespace {

// Whether the activations stage in LDS: small batches whose staged rows fit beside the partial tiles.
bool stage_rows(int M, int waves, size_t part_bytes)
{
    return M >= 1 && M <= XS_ROWS && part_bytes + (size_t)waves * M * XS_PITCH <= MAX_LDS_BYTES;
}

// Output columns per block: the N columns spread over every CU of the device, at most max_cols.
int cols_per_block(int n, int max_cols)
{
    const int cus = device_cus();
    const int r = (n + cus - 1) / cus;
    return r < 1 ? 1 : (r > max_cols ? max_cols : r);
}

template <int NW>
int launch_linear_fp8(const uint16_t *x, int32_t M, const fp8_channel_weights &w, int R, uint16_t *y, hipStream_t s)
{
    const int N = w.rows, K = w.k;
    const int S = num_chunks(K);
    const int waves = S < FP8_WAVES ? S : FP8_WAVES;
    const size_t shmem = (size_t)S * ROW_GROUP * NW * 16 * LDS_ROW * sizeof(float);
    if (shmem > MAX_LDS_BYTES) return NVFP4_ERR_UNSUPPORTED;  // the entry point admits no such K
    const bool xs = stage_rows(M, waves, shmem);
    const int st = linear_prepare();
    if (st != NVFP4_OK) return st;
    return launch(xs ? linear_fp8_kernel<NW, true> : linear_fp8_kernel<NW, false>, dim3((unsigned)((N + R - 1) / R)),
                  dim3((unsigned)(waves * 64)), shmem + (xs ? (size_t)waves * M * XS_PITCH : 0), s,
                  reinterpret_cast<const f16 *>(x), M, w.codes, w.channel_scale, N, K, reinterpret_cast<f16 *>(y), R);
}

template <int NW, bool GATED, typename OUT = f16>
int launch_linear(const uint16_t *x, int32_t M, const nvfp4_weights &w, int N, int layout, int R, void *y,
                  hipStream_t s)
{
    const int K = w.k;
    const int S = num_chunks(K);
    const int waves = S < MAX_WAVES ? S : MAX_WAVES;
    const size_t shmem = (size_t)S * ROW_GROUP * NW * 16 * LDS_ROW * sizeof(float);
    static_assert(ROW_GROUP == 2 && LDS_ROW == 20, "linear_lds_bytes assumes this partial-tile layout");
    if (shmem != linear_lds_bytes(K, NW) || shmem > MAX_LDS_BYTES) return NVFP4_ERR_UNSUPPORTED;
    const bool xs = stage_rows(M, waves, shmem);
    const int st = linear_prepare();
    if (st != NVFP4_OK) return st;
    const int blocks = (N + R - 1) / R;
    return launch(xs ? linear_kernel<NW, GATED, OUT, true> : linear_kernel<NW, GATED, OUT, false>, dim3((unsigned)blocks),
                  dim3((unsigned)(waves * 64)), shmem + (xs ? (size_t)waves * M * XS_PITCH : 0), s,
                  reinterpret_cast<const f16 *>(x), M, w.codes, w.scales, w.global_scale, N, K, layout,
                  static_cast<OUT *>(y), R);
}

}  // namespace

int run_linear(const uint16_t *x, int32_t M, const nvfp4_weights &w, uint16_t *y, hipStream_t s)
{
    const int R = cols_per_block(w.rows, 16 * linear_max_tiles(w.k));
    if (R > 16) return launch_linear<2, false>(x, M, w, w.rows, 0, R, y, s);
    return launch_linear<1, false>(x, M, w, w.rows, 0, R, y, s);
}

int run_linear_f32(const uint16_t *x, int32_t M, const nvfp4_weights &w, float *y, hipStream_t s)
{
    const int R = cols_per_block(w.rows, 16 * linear_max_tiles(w.k));
    if (R > 16) return launch_linear<2, false, float>(x, M, w, w.rows, 0, R, y, s);
    return launch_linear<1, false, float>(x, M, w, w.rows, 0, R, y, s);
}

size_t linear_ws_bytes(int32_t M, int32_t N, int32_t K)
{
    return (size_t)num_chunks(K) * (size_t)M * (size_t)N * sizeof(float);
}

// Split-K form: the partials launch, then the fold. N = weight rows (2I for the gated form).
namespace {
int launch_split(const uint16_t *x, int32_t M, const nvfp4_weights &w, float *part, hipStream_t s)
{
    const int N = w.rows, K = w.k, S = num_chunks(K), NT = N / 16;
    const int cus = device_cus();
    int T = (int)(((int64_t)NT * S + cus - 1) / cus);  // tiles per block: about one block per CU
    T = T < 1 ? 1 : (T > SPLIT_WAVES ? SPLIT_WAVES : T);
    const int64_t blocks = (int64_t)S * ((NT + T - 1) / T);
    return launch(linear_partials_kernel, dim3((unsigned)blocks), dim3((unsigned)(T * 64)), 0, s,
                  reinterpret_cast<const f16 *>(x), M, w.codes, w.scales, N, K, part);
}

template <bool GATED>
int launch_fold(const float *part, int32_t M, const nvfp4_weights &w, int layout, uint16_t *y, hipStream_t s)
{
    const int N = w.rows, S = num_chunks(w.k);
    const int64_t quads = (int64_t)M * (GATED ? N / 2 : N) / 4;
    return launch(linear_fold_kernel<GATED, f16>, dim3((unsigned)((quads + FOLD_THREADS - 1) / FOLD_THREADS)),
                  dim3(FOLD_THREADS), 0, s, part, S, M, N, w.global_scale, layout, reinterpret_cast<f16 *>(y));
}
}  // namespace

// The split form pays once the copy of x that every one-launch block reads (M * K * 2 bytes) is
// large: past 8 rows and 96 KiB. Measured on MI355X, 4352x5120: 7.3 vs 8.6 us at one row, 8.2 vs
// 9.2 at eight (one-launch faster), 9.3 vs 10.7 at twelve, 12.1 vs 16.1 at 32; the 5120x2176 down
// projection of the gated MLP: 7.5 vs 8.0 at 16 rows (70 KB of x), 9.6 vs 10.7 at 32. Below that the
// split-K calls run the one-launch kernel (the same results bitwise; ws is then not touched).
bool split_pays(int32_t M, int32_t K) { return M > 8 && (int64_t)M * K * 2 > 96 * 1024; }

int run_linear_split(const uint16_t *x, int32_t M, const nvfp4_weights &w, uint16_t *y, void *ws, hipStream_t s)
{
    if (!split_pays(M, w.k)) return run_linear(x, M, w, y, s);
    float *part = static_cast<float *>(ws);
    const int st = launch_split(x, M, w, part, s);
    return st != NVFP4_OK ? st : launch_fold<false>(part, M, w, 0, y, s);
}

int run_linear_swiglu_split(const uint16_t *x, int32_t M, const nvfp4_weights &w, int32_t layout, uint16_t *h,
                            void *ws, hipStream_t s)
{
    if (!split_pays(M, w.k)) return run_linear_swiglu(x, M, w, layout, h, s);
    float *part = static_cast<float *>(ws);
    const int st = launch_split(x, M, w, part, s);
    return st != NVFP4_OK ? st : launch_fold<true>(part, M, w, layout, h, s);
}

// ---- shared-expert gate ---------------------------------------------------------------------------
// sigma[m] = 1 / (1 + e^-z), z = sum_k x[m][k] g[k] (the "shared gate" of the "[Kernel][SM70] Improve
// Qwen3.8 no-MTP concurrency" page, "Scope and related PRs"). One wave per token: each lane sums
// its strided elements in FP32 in ascending order, then a fixed butterfly over the lanes, read
// from lane 0, so the value never depends on the batch.
// VEC (g 16-byte aligned; x rows always are, K % 128 == 0): wave_dot_f16, 16-byte loads with four
// pieces in flight at once (the order the fused shared-expert launch uses too). Otherwise one element
// per lane and step. Either way a token's sum has one fixed order, whatever M.
template <bool VEC>
__global__ __launch_bounds__(256) void shared_gate_kernel(const f16 *__restrict__ x, int M, int K,
                                                          const f16 *__restrict__ g, float *__restrict__ sigma)
{
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (m >= M) return;  // wave-uniform
    const f16 *xr = x + (size_t)m * K;
    float z;
    if (VEC) {
        z = wave_dot_f16(xr, g, K);
    } else {
        z = 0.0f;
        for (int k = lane; k < K; k += 64) z = fmaf((float)xr[k], (float)g[k], z);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
        z = __shfl(z, 0, 64);
    }
    if (lane == 0) sigma[m] = 1.0f / (1.0f + expf(-z));
}

int run_shared_gate(const uint16_t *x, int32_t M, int32_t K, const uint16_t *g, float *sigma, hipStream_t s)
{
    const dim3 grid((unsigned)(((int64_t)M + 3) / 4));
    const f16 *xp = reinterpret_cast<const f16 *>(x), *gp = reinterpret_cast<const f16 *>(g);
    if ((reinterpret_cast<uintptr_t>(g) & 15) == 0 && K % 8 == 0)
        return launch(shared_gate_kernel<true>, grid, dim3(256), 0, s, xp, M, K, gp, sigma);
    return launch(shared_gate_kernel<false>, grid, dim3(256), 0, s, xp, M, K, gp, sigma);
}

int run_linear_fp8(const uint16_t *x, int32_t M, const fp8_channel_weights &w, uint16_t *y, hipStream_t s)
{
    const int R = cols_per_block(w.rows, 16 * linear_max_tiles(w.k));
    if (R > 16) return launch_linear_fp8<2>(x, M, w, R, y, s);
    return launch_linear_fp8<1>(x, M, w, R, y, s);
}

int run_linear_swiglu(const uint16_t *x, int32_t M, const nvfp4_weights &w, int32_t layout, uint16_t *h,
                      hipStream_t s)
{
    return launch_linear<2, true>(x, M, w, w.rows / 2, layout, cols_per_block(w.rows / 2, 16), h, s);
}

}  // namespace nvfp4
