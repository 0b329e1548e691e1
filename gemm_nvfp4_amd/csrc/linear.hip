// linear.hip -- dense NVFP4 projection y = fp16(global * x W^T), the "QPN" projection of the
// "[SM70][Draft] Extend Qwen3.8 DFlash2 concurrency paths" page ("Purpose": independent row tiles
// admitted through M <= 32; "TP4-only NVFP4 verifier follow-up": two-row-tile CTAs that reuse the
// loaded packed weights while keeping the split-K / FP32 reduction order).
//
// gfx950 design: one block per 16 output columns (weight rows). Its waves share the reduction
// axis, one 512-element chunk each (intra-block split-K). A wave decodes its chunk once into MFMA
// B fragments in registers and applies them to every 16-row tile of x, so at small M the weight
// bytes are read from HBM exactly once. Chunk partials meet in LDS and are added in chunk order,
// which is the same reduction order as every other GEMM here. A batch of any size is therefore
// bitwise equal to single-row calls.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int LDS_ROW = 20;
constexpr int MAX_WAVES = 10;   // waves per block; chunks beyond are taken in turn
constexpr int ROW_GROUP = 2;    // 16-row tiles of x handled per pass over the weights

__global__ __launch_bounds__(MAX_WAVES * 64) void linear_kernel(const f16 *__restrict__ x, int M,
                                                                 const uint8_t *__restrict__ codes,
                                                                 const uint8_t *__restrict__ scales,
                                                                 const float *__restrict__ gscale, int N, int K,
                                                                 f16 *__restrict__ y)
{
    extern __shared__ float part[];  // [S][ROW_GROUP][16][LDS_ROW]
    const int nt = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int S = num_chunks(K);
    const int row_tiles = (M + 15) >> 4;
    const size_t wrow = (size_t)nt * 16 + n;
    const uint8_t *cr = codes + wrow * ((size_t)K >> 1);
    const uint8_t *sr = scales + wrow * ((size_t)K >> 4);
    const float gs = gscale[0];

    for (int rt0 = 0; rt0 < row_tiles; rt0 += ROW_GROUP) {
        for (int c = wave; c < S; c += nwaves) {
            const int kb = c * KCHUNK;
            const int groups = min(KCHUNK, K - kb) >> 7;  // 128-element lane groups with data
            const bool qv = q < groups;
            const RawChunk w = load_chunk(cr, sr, kb, qv ? q : groups - 1);
#pragma unroll
            for (int r = 0; r < ROW_GROUP; ++r) {
                const int rt = rt0 + r;
                if (rt >= row_tiles) break;
                const int m = rt * 16 + n;
                const bool rv = m < M && qv;
                // All 16 A fragments are loaded before the chain, unconditionally (rows past M and
                // lane groups past K re-read valid data of row 0 / lane group 0, then become zeros),
                // so their latencies overlap instead of adding up.
                const f16 *xr = x + (size_t)(m < M ? m : 0) * K;
                const int qa = qv ? q : 0;
                f16x8 af[4][4];
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int s = 0; s < 4; ++s) af[b][s] = a_frag(xr, kb, qa, b, s);
                __builtin_amdgcn_sched_barrier(0);  // every load (weights, then A) is issued before the math
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        if (!rv) af[b][s] = zero8();
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const f16x2 sc = chunk_scales(w, b);
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = mfma_step(af[b][s], b_frag(w, sc, b, s, qv), acc);
                }
                float *pc = part + ((size_t)c * ROW_GROUP + r) * 16 * LDS_ROW;
#pragma unroll
                for (int j = 0; j < 4; ++j) pc[(4 * q + j) * LDS_ROW + n] = acc[j];
            }
        }
        __syncthreads();
        for (int o = threadIdx.x; o < ROW_GROUP * 256; o += blockDim.x) {
            const int r = o >> 8, row = (o >> 4) & 15, col = o & 15;
            const int m = (rt0 + r) * 16 + row;
            if (rt0 + r < row_tiles && m < M) {
                float tot = part[((size_t)0 * ROW_GROUP + r) * 16 * LDS_ROW + row * LDS_ROW + col];
                for (int c = 1; c < S; ++c) tot += part[((size_t)c * ROW_GROUP + r) * 16 * LDS_ROW + row * LDS_ROW + col];
                y[(size_t)m * N + nt * 16 + col] = (f16)(tot * gs);
            }
        }
        __syncthreads();
    }
}

}  // namespace

int run_linear(const uint16_t *x, int32_t M, const nvfp4_weights &w, uint16_t *y, hipStream_t s)
{
    const int N = w.rows, K = w.k;
    const int S = num_chunks(K);
    const int waves = S < MAX_WAVES ? S : MAX_WAVES;
    const size_t shmem = (size_t)S * ROW_GROUP * 16 * LDS_ROW * sizeof(float);
    if (shmem > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(linear_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
        if (e != hipSuccess) return NVFP4_ERR_LAUNCH;
    }
    return launch(linear_kernel, dim3((unsigned)(N / 16)), dim3((unsigned)(waves * 64)), shmem, s,
                  reinterpret_cast<const f16 *>(x), M, w.codes, w.scales, w.global_scale, N, K,
                  reinterpret_cast<f16 *>(y));
}

}  // namespace nvfp4
