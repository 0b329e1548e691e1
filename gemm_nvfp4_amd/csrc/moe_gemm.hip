// moe_gemm.hip -- grouped expert GEMMs of the MoE layer:
//   W13 with fused SwiGLU ("expert-grouped multi-row W13/SiLU with intra-CTA Split-K"), then W2
//   with the top-k-weighted reduction ("grouped W2 reusing the same integer plan", "W2/reduction
//   fusion"), from the "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page, "Scope and
//   related PRs".
//
// Work decomposition (gfx950, wave64):
//   * A block serves one active expert (plan.active[a]) and a few 16-column output tiles. Blocks
//     past the device-side n_active exit at once, so the grid is sized from host-known bounds
//     and no device-to-host read is ever needed.
//   * Inside a block, the four waves split the reduction axis into its 512-element chunks
//     (intra-block split-K) when there are several. Otherwise each wave takes its own output
//     tile.
//   * A wave loads its chunk of packed weights once, with one 16-byte load per lane per
//     superblock, and decodes it into MFMA B fragments held in registers. It then loops over
//     all of the expert's 16-row tiles of bucket-ordered pairs. So every expert's weights are
//     read from HBM once, whether the expert has one pair or hundreds.
//   * Chunk partials meet in LDS and are added in chunk order. The epilogue applies the FP32
//     global scale, then SwiGLU (W13) or the store of per-pair FP32 results (W2).
//   * A separate pass sums each token's slots in slot order with fmaf and rounds to fp16 once.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace {

constexpr int LDS_ROW = 20;  // padded row of 16 floats: rows 4 apart land on different banks

// ---- W13 + SwiGLU ---------------------------------------------------------------------------------
// SPLIT = waves per output tile, i.e. chunks computed in parallel (1, 2 or 4; >= num_chunks(K)).
template <int SPLIT>
__global__ __launch_bounds__(256) void w13_swiglu_kernel(PlanView pv, int topk, const f16 *__restrict__ x,
                                                         const uint8_t *__restrict__ codes,
                                                         const uint8_t *__restrict__ scales,
                                                         const float *__restrict__ gscale, int K, int I, int layout,
                                                         int blocks_per_expert, f16 *__restrict__ h)
{
    constexpr int TPB = 4 / SPLIT;  // 16-wide i tiles per block
    __shared__ float part[4][2][16][LDS_ROW];

    const int a = blockIdx.x / blocks_per_expert;
    const int ib = blockIdx.x - a * blocks_per_expert;
    if (a >= pv.hdr[1]) return;  // block-uniform, before any barrier
    const int e = pv.active[a];
    const int cnt = pv.counts[e];
    const int base = pv.offsets[e];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int sub = wave / SPLIT, c = wave % SPLIT;
    const int it = ib * TPB + sub;
    const int itiles = I >> 4;
    const int S = num_chunks(K);
    const bool working = it < itiles && c < S;
    const int kb = c * KCHUNK;
    const int nsb = working ? min(KCHUNK / KSB, (K - kb) / KSB) : 0;

    f16x8 bg[4][4], bu[4][4];
    if (working) {
        const int i_row = it * 16 + n;
        const int rg = layout ? 2 * i_row : i_row;
        const int ru = layout ? 2 * i_row + 1 : I + i_row;
        const size_t crow = (size_t)K >> 1, srow = (size_t)K >> 4;
        const size_t eb = (size_t)e * 2 * I;
        const uint8_t *cg = codes + (eb + rg) * crow, *cu = codes + (eb + ru) * crow;
        const uint8_t *sg = scales + (eb + rg) * srow, *su = scales + (eb + ru) * srow;
        RawSB rgw[4], ruw[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (b < nsb) {
                rgw[b] = load_sb(cg, sg, kb + KSB * b, q);
                ruw[b] = load_sb(cu, su, kb + KSB * b, q);
            }
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (b < nsb) {
                decode_sb(rgw[b], bg[b]);
                decode_sb(ruw[b], bu[b]);
            }
    }
    const float gs = gscale[e];

    for (int r0 = 0; r0 < cnt; r0 += 16) {
        f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
        if (working) {
            const bool rv = r0 + n < cnt;  // this lane's A row is r0 + (lane % 16)
            const int t = rv ? pv.sorted_pair[base + r0 + n] / topk : 0;
            const f16 *xr = x + (size_t)t * K;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (b < nsb) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const f16x8 av = rv ? load_a(xr, kb + KSB * b, q, s) : zero8();
                        accg = mfma_step(av, bg[b][s], accg);
                        accu = mfma_step(av, bu[b][s], accu);
                    }
                }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            part[wave][0][4 * q + j][n] = accg[j];
            part[wave][1][4 * q + j][n] = accu[j];
        }
        __syncthreads();
        const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
#pragma unroll
        for (int sb = 0; sb < TPB; ++sb) {
            const int itx = ib * TPB + sb;
            if (itx < itiles && r0 + row < cnt) {
                float G = part[sb * SPLIT][0][row][col];
                float U = part[sb * SPLIT][1][row][col];
                for (int cc = 1; cc < S; ++cc) {
                    G += part[sb * SPLIT + cc][0][row][col];
                    U += part[sb * SPLIT + cc][1][row][col];
                }
                const float hv = swiglu(G * gs, U * gs);
                h[(size_t)(base + r0 + row) * I + itx * 16 + col] = (f16)hv;
            }
        }
        __syncthreads();
    }
}

// ---- W2: per-pair FP32 results y[j][n] = global * sum_i dq(W2)[n][i] * h[j][i] ------------------------
template <int SPLIT>
__global__ __launch_bounds__(256) void w2_kernel(PlanView pv, const f16 *__restrict__ hin, const uint8_t *__restrict__ codes,
                                                 const uint8_t *__restrict__ scales, const float *__restrict__ gscale,
                                                 int K, int I, int blocks_per_expert, float *__restrict__ ws)
{
    constexpr int TPB = 4 / SPLIT;  // 16-row output tiles per block
    __shared__ float part[SPLIT > 1 ? 4 : 1][16][LDS_ROW];

    const int a = blockIdx.x / blocks_per_expert;
    const int ib = blockIdx.x - a * blocks_per_expert;
    if (a >= pv.hdr[1]) return;
    const int e = pv.active[a];
    const int cnt = pv.counts[e];
    const int base = pv.offsets[e];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int sub = wave / SPLIT, c = wave % SPLIT;
    const int nt = ib * TPB + sub;
    const int ntiles = K >> 4;
    const int S = num_chunks(I);
    const bool working = nt < ntiles && c < S;
    const int kb = c * KCHUNK;
    const int nsb = working ? min(KCHUNK / KSB, (I - kb) / KSB) : 0;

    f16x8 bw[4][4];
    if (working) {
        const size_t row = (size_t)e * K + nt * 16 + n;
        const uint8_t *cr = codes + row * ((size_t)I >> 1);
        const uint8_t *sr = scales + row * ((size_t)I >> 4);
        RawSB raw[4];
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (b < nsb) raw[b] = load_sb(cr, sr, kb + KSB * b, q);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (b < nsb) decode_sb(raw[b], bw[b]);
    }
    const float gs = gscale[e];

    for (int r0 = 0; r0 < cnt; r0 += 16) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (working) {
            const bool rv = r0 + n < cnt;
            const f16 *hr = hin + (size_t)(base + r0 + (rv ? n : 0)) * I;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (b < nsb) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const f16x8 av = rv ? load_a(hr, kb + KSB * b, q, s) : zero8();
                        acc = mfma_step(av, bw[b][s], acc);
                    }
                }
        }
        if constexpr (SPLIT == 1) {
            if (working) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 4 * q + j;
                    if (r0 + row < cnt) ws[(size_t)(base + r0 + row) * K + nt * 16 + n] = acc[j] * gs;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) part[wave][4 * q + j][n] = acc[j];
            __syncthreads();
            const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
#pragma unroll
            for (int sb = 0; sb < TPB; ++sb) {
                const int ntx = ib * TPB + sb;
                if (ntx < ntiles && r0 + row < cnt) {
                    float Y = part[sb * SPLIT][row][col];
                    for (int cc = 1; cc < S; ++cc) Y += part[sb * SPLIT + cc][row][col];
                    ws[(size_t)(base + r0 + row) * K + ntx * 16 + col] = Y * gs;
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

}  // namespace

int run_w13(const PlanView &pv, int64_t a_max, int32_t topk, const uint16_t *x, const nvfp4_weights &w, int32_t layout,
            uint16_t *h, hipStream_t s)
{
    const int K = w.k, I = w.rows / 2;
    const int split = split_for(K);
    const int tpb = 4 / split;
    const int bpe = (I / 16 + tpb - 1) / tpb;
    const dim3 grid((unsigned)(a_max * bpe)), block(256);
    const f16 *xp = reinterpret_cast<const f16 *>(x);
    f16 *hp = reinterpret_cast<f16 *>(h);
    switch (split) {
    case 1: return launch(w13_swiglu_kernel<1>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, bpe, hp);
    case 2: return launch(w13_swiglu_kernel<2>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, bpe, hp);
    default: return launch(w13_swiglu_kernel<4>, grid, block, 0, s, pv, topk, xp, w.codes, w.scales, w.global_scale, K, I, layout, bpe, hp);
    }
}

int run_w2(const PlanView &pv, int64_t a_max, int32_t M, int32_t topk, const uint16_t *h, const nvfp4_weights &w,
           const float *topk_weights, uint16_t *out, float *ws, hipStream_t s)
{
    const int K = w.rows, I = w.k;
    const int split = split_for(I);
    const int tpb = 4 / split;
    const int bpe = (K / 16 + tpb - 1) / tpb;
    const dim3 grid((unsigned)(a_max * bpe)), block(256);
    const f16 *hp = reinterpret_cast<const f16 *>(h);
    int st;
    switch (split) {
    case 1: st = launch(w2_kernel<1>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, bpe, ws); break;
    case 2: st = launch(w2_kernel<2>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, bpe, ws); break;
    default: st = launch(w2_kernel<4>, grid, block, 0, s, pv, hp, w.codes, w.scales, w.global_scale, K, I, bpe, ws); break;
    }
    if (st != NVFP4_OK) return st;
    const int bpt = (K / 4 + 255) / 256;
    return launch(reduce_kernel, dim3((unsigned)((int64_t)M * bpt)), dim3(256), 0, s, pv.pos_of_pair, topk_weights,
                  (const float *)ws, topk, K, bpt, reinterpret_cast<f16 *>(out));
}

}  // namespace nvfp4
