// linear.hip -- dense NVFP4 projection y = fp16(global * x W^T), the "QPN" projection of the
// "[SM70][Draft] Extend Qwen3.8 DFlash2 concurrency paths" page ("Purpose": independent row tiles
// admitted through M <= 32; "TP4-only NVFP4 verifier follow-up": two-row-tile CTAs that reuse the
// loaded packed weights while keeping the split-K / FP32 reduction order), and its gated form for
// the packed gate/up projection of a dense MLP (same page and section: the gate/up and down
// projections of the packed MLP weights): h = fp16(silu(g) * u) with g and u the projections on
// the gate and up rows.
//
// gfx950 design: one block per 16 output columns (weight rows; gate and up rows of 16 h columns in
// the gated form). Its waves share the reduction axis, one 512-element chunk each (intra-block
// split-K). A wave decodes its chunk once into MFMA B fragments in registers and applies them to
// every 16-row tile of x, so at small M the weight bytes are read from HBM exactly once. Chunk
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

// Each wave holds NW 16-row weight tiles. Plain (GATED false): tile t covers output columns
// (nt*NW + t)*16 .. +15. Gated: tile 0 holds the gate rows and tile 1 the up rows of h columns
// nt*16 .. +15 (layout 0: rows i and I + i; layout 1: rows 2i and 2i + 1).
// OUT is the output type: fp16 (rounded once), or FP32 for a result that is summed further (the
// shared expert's down projection, added into the MoE output before its one rounding).
template <int NW, bool GATED, typename OUT = f16>
__global__ __launch_bounds__(MAX_WAVES * 64) void linear_kernel(const f16 *__restrict__ x, int M,
                                                                 const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 const float *__restrict__ gscale, int N, int K,
                                                                 int layout, OUT *__restrict__ y)
{
    extern __shared__ float part[];  // [S][ROW_GROUP][NW][16][LDS_ROW]
    const int nt = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int S = num_chunks(K);
    const int row_tiles = (M + 15) >> 4;
    const int col = nt * 16 + n;  // gated: h column of this lane's weight rows
    const uint8_t *cr[NW], *sr[NW];
#pragma unroll
    for (int t = 0; t < NW; ++t) {
        const size_t wrow = GATED ? (size_t)(layout ? 2 * col + t : t * N + col) : (size_t)((nt * NW + t) * 16 + n);
        cr[t] = codes + wrow * ((size_t)K >> 1);
        sr[t] = scales + wrow * ((size_t)K >> 4);
    }
    const float gs = gscale[0];

    for (int rt0 = 0; rt0 < row_tiles; rt0 += ROW_GROUP) {
        for (int c = wave; c < S; c += nwaves) {
            const int kb = c * KCHUNK;
            const int groups = min(KCHUNK, K - kb) >> 7;  // 128-element lane groups with data
            const bool qv = q < groups;
            RawChunk w[NW];
#pragma unroll
            for (int t = 0; t < NW; ++t) w[t] = load_chunk(cr[t], sr[t], kb, qv ? q : groups - 1);
#pragma unroll 1
            for (int r = 0; r < ROW_GROUP; ++r) {
                const int rt = rt0 + r;
                if (rt >= row_tiles) break;
                const int m = rt * 16 + n;
                const bool rv = m < M && qv;
                // All 16 A fragments are loaded before the chain, back to back, so their latencies
                // overlap. Only lanes of rows below M (and lane groups inside K) load: padding rows
                // are zeros without a load, so a small batch does not pull duplicate activation
                // bytes through the CU (each CU's load throughput is the limit here).
                const f16 *xr = x + (size_t)(rv ? m : 0) * K;
                f16x8 af[4][4];
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int s = 0; s < 4; ++s) af[b][s] = zero8();
                if (rv) {
#pragma unroll
                    for (int b = 0; b < 4; ++b)
#pragma unroll
                        for (int s = 0; s < 4; ++s) af[b][s] = a_frag(xr, kb, q, b, s);
                }
                __builtin_amdgcn_sched_barrier(0);  // every load (weights, then A) is issued before the math
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
                        for (int t = 0; t < NW; ++t) acc[t] = mfma_step(af[b][s], b_frag(w[t], sc[t], b, s, qv), acc[t]);
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
                    y[(size_t)m * N + nt * 16 + cl] = f16_of_f32(swiglu(tot[0] * gs, tot[1] * gs));
                } else {
#pragma unroll
                    for (int t = 0; t < NW; ++t) y[(size_t)m * N + (nt * NW + t) * 16 + cl] = to_out<OUT>(tot[t] * gs);
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

__device__ __forceinline__ Fp8Chunk load_chunk8(const uint8_t *row, int kb, int q_ld)
{
    Fp8Chunk r;
    const uint8_t *c = row + kb + 128 * q_ld;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.codes[j] = *reinterpret_cast<const u32x4 *>(c + 16 * j);
    return r;
}

// B fragment of step (b, s): elements [128q + 32b + 8s, +8), i.e. half of load 2b + s/2.
__device__ __forceinline__ f16x8 b_frag8(const Fp8Chunk &r, int b, int s, bool qv)
{
    const u32x4 v = r.codes[2 * b + (s >> 1)];
    const uint32_t d0 = v[2 * (s & 1)], d1 = v[2 * (s & 1) + 1];
    const f16x2 p0 = e4m3_pair<false>(d0), p1 = e4m3_pair<true>(d0), p2 = e4m3_pair<false>(d1), p3 = e4m3_pair<true>(d1);
    const f16x8 w = f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    return qv ? w : zero8();
}

// Two 16-row weight tiles per wave (output columns (nt*2 + t)*16 .. +15), as the NVFP4 kernel.
// Eight waves: the channel-FP8 chunk holds twice the packed bytes of an NVFP4 one (two weight tiles
// take 64 registers), so ten waves would spill; at K = 5120 two waves take a second chunk.
constexpr int FP8_WAVES = 8;
template <int NW>
__global__ __launch_bounds__(FP8_WAVES * 64) void linear_fp8_kernel(const f16 *__restrict__ x, int M,
                                                          const uint8_t *__restrict__ codes,
                                                          const float *__restrict__ chscale, int N, int K,
                                                          f16 *__restrict__ y)
{
    extern __shared__ float part[];  // [S][ROW_GROUP][NW][16][LDS_ROW]
    const int nt = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int S = num_chunks(K);
    const int row_tiles = (M + 15) >> 4;
    const uint8_t *cr[NW];
#pragma unroll
    for (int t = 0; t < NW; ++t) cr[t] = codes + (size_t)((nt * NW + t) * 16 + n) * K;

    for (int rt0 = 0; rt0 < row_tiles; rt0 += ROW_GROUP) {
        for (int c = wave; c < S; c += nwaves) {
            const int kb = c * KCHUNK;
            const int groups = min(KCHUNK, K - kb) >> 7;
            const bool qv = q < groups;
            Fp8Chunk w[NW];
#pragma unroll
            for (int t = 0; t < NW; ++t) w[t] = load_chunk8(cr[t], kb, qv ? q : groups - 1);
#pragma unroll
            for (int r = 0; r < ROW_GROUP; ++r) {
                const int rt = rt0 + r;
                if (rt >= row_tiles) break;
                const int m = rt * 16 + n;
                const bool rv = m < M && qv;
                // As in linear_kernel: only valid rows load their A fragments.
                const f16 *xr = x + (size_t)(rv ? m : 0) * K;
                f16x8 af[4][4];
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int s = 0; s < 4; ++s) af[b][s] = zero8();
                if (rv) {
#pragma unroll
                    for (int b = 0; b < 4; ++b)
#pragma unroll
                        for (int s = 0; s < 4; ++s) af[b][s] = a_frag(xr, kb, q, b, s);
                }
                __builtin_amdgcn_sched_barrier(0);  // every load (weights, then A) is issued before the math
                f32x4 acc[NW];
#pragma unroll
                for (int t = 0; t < NW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int t = 0; t < NW; ++t) acc[t] = mfma_step(af[b][s], b_frag8(w[t], b, s, qv), acc[t]);
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
                    const int colx = (nt * NW + t) * 16 + cl;
                    y[(size_t)m * N + colx] = f16_of_f32(tot * chscale[colx]);
                }
            }
        }
        __syncthreads();
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
    hipError_t e = allow_lds(linear_kernel<1, false, f16>);
    if (e == hipSuccess) e = allow_lds(linear_kernel<2, false, f16>);
    if (e == hipSuccess) e = allow_lds(linear_kernel<1, false, float>);
    if (e == hipSuccess) e = allow_lds(linear_kernel<2, false, float>);
    if (e == hipSuccess) e = allow_lds(linear_kernel<2, true, f16>);
    if (e == hipSuccess) e = allow_lds(linear_fp8_kernel<1>);
    if (e == hipSuccess) e = allow_lds(linear_fp8_kernel<2>);
    if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
    if (dev < 64) done[dev].store(1, std::memory_order_release);
    return NVFP4_OK;
}

namespace {

template <int NW>
int launch_linear_fp8(const uint16_t *x, int32_t M, const fp8_channel_weights &w, uint16_t *y, hipStream_t s)
{
    const int N = w.rows, K = w.k;
    const int S = num_chunks(K);
    const int waves = S < FP8_WAVES ? S : FP8_WAVES;
    const size_t shmem = (size_t)S * ROW_GROUP * NW * 16 * LDS_ROW * sizeof(float);
    if (shmem > MAX_LDS_BYTES) return NVFP4_ERR_UNSUPPORTED;  // the entry point admits no such K
    const int st = linear_prepare();
    if (st != NVFP4_OK) return st;
    return launch(linear_fp8_kernel<NW>, dim3((unsigned)(N / (16 * NW))), dim3((unsigned)(waves * 64)), shmem, s,
                  reinterpret_cast<const f16 *>(x), M, w.codes, w.channel_scale, N, K, reinterpret_cast<f16 *>(y));
}

template <int NW, bool GATED, typename OUT = f16>
int launch_linear(const uint16_t *x, int32_t M, const nvfp4_weights &w, int N, int layout, void *y, hipStream_t s)
{
    const int K = w.k;
    const int S = num_chunks(K);
    const int waves = S < MAX_WAVES ? S : MAX_WAVES;
    const size_t shmem = (size_t)S * ROW_GROUP * NW * 16 * LDS_ROW * sizeof(float);
    static_assert(ROW_GROUP == 2 && LDS_ROW == 20, "linear_lds_bytes assumes this partial-tile layout");
    if (shmem != linear_lds_bytes(K, NW) || shmem > MAX_LDS_BYTES) return NVFP4_ERR_UNSUPPORTED;
    const int st = linear_prepare();
    if (st != NVFP4_OK) return st;
    const int blocks = GATED ? N / 16 : N / (16 * NW);
    return launch(linear_kernel<NW, GATED, OUT>, dim3((unsigned)blocks), dim3((unsigned)(waves * 64)), shmem, s,
                  reinterpret_cast<const f16 *>(x), M, w.codes, w.scales, w.global_scale, N, K, layout,
                  static_cast<OUT *>(y));
}

}  // namespace

int run_linear(const uint16_t *x, int32_t M, const nvfp4_weights &w, uint16_t *y, hipStream_t s)
{
    if (linear_tiles(w.rows, w.k) == 2) return launch_linear<2, false>(x, M, w, w.rows, 0, y, s);
    return launch_linear<1, false>(x, M, w, w.rows, 0, y, s);
}

int run_linear_f32(const uint16_t *x, int32_t M, const nvfp4_weights &w, float *y, hipStream_t s)
{
    if (linear_tiles(w.rows, w.k) == 2) return launch_linear<2, false, float>(x, M, w, w.rows, 0, y, s);
    return launch_linear<1, false, float>(x, M, w, w.rows, 0, y, s);
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
    if (w.rows % 32 == 0) return launch_linear_fp8<2>(x, M, w, y, s);
    return launch_linear_fp8<1>(x, M, w, y, s);
}

int run_linear_swiglu(const uint16_t *x, int32_t M, const nvfp4_weights &w, int32_t layout, uint16_t *h,
                      hipStream_t s)
{
    return launch_linear<2, true>(x, M, w, w.rows / 2, layout, h, s);
}

}  // namespace nvfp4
