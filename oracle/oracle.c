/*
 * oracle.c -- plain fp64 CPU oracle for the NVFP4 weight-only MoE path.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load or call this library. The HIP product path never does, and it shares no code, header,
 * table or constant with this file.
 *
 * Sources, all cited by page title and section:
 *  - "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency", sections "Scope and related PRs" and
 *    "Test Plan": weights are native NVFP4 (E2M1 codes with E4M3 block scales) and activations
 *    are FP16. The expert path is W13 with SiLU(gate)*up, then W2 with a top-k-weighted reduction.
 *    One integer plan is shared by W13 and W2. The tests cover E4M3 subnormals, signed zero and
 *    NaN.
 *  - "[Perf][SM70] Optimize Qwen3.8 Flash Next prefill", section "SM70 QSA indexer hotspot
 *    update": the 8192-token top-10 W13/W2 MoE workload.
 *  - The NVFP4 format itself (one E4M3 scale per 16-element K-block plus one FP32 global scale)
 *    and the routing-plan contents are not printed on the pages. The plainest reading, used here,
 *    is the standard NVFP4 layout and a stable counting sort by expert.
 *
 * Everything is computed in IEEE double. Decoded weights are exact in double: an E2M1 value has
 * at most 2 significant bits, an E4M3 value at most 4 and the fp32 global at most 24, so the
 * product has at most 30. Each product x*w (11 + 30 bits) is exact. Sums run in ascending index
 * order.
 *
 * The grouped form (orc_moe_grouped) uses the plan and dequantizes each expert once. The
 * per-token form (orc_moe_token) walks each token's slots and decodes weights row by row. For
 * every pair both perform the same operations in the same order, so their outputs must be
 * bitwise equal in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

int orc_version(void) { return 1; }

/* ---- number formats ---------------------------------------------------------------------- */

/* E2M1 (OCP FP4): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent 0 holds the subnormal m*0.5; otherwise 2^(e-1)*(1+m/2). Magnitudes: 0,0.5,1,1.5,2,3,4,6. */
double orc_e2m1(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN (OCP FP8): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa. There is no
 * infinity; exponent 15 with mantissa 7 is NaN (0x7F, 0xFF). Exponent 0 holds subnormals m*2^-9.
 * The largest finite value is 448 (0x7E). */
double orc_e4m3(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* IEEE binary16 bits -> double. */
double orc_half(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -24);
    else mag = ldexp(1.0 + m / 1024.0, e - 15);
    return s ? -mag : mag;
}

/* double -> IEEE binary16 bits, round to nearest, ties to even; overflow goes to +-inf. */
uint16_t orc_to_half(double v)
{
    if (isnan(v)) return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a >= 65520.0) return sign | 0x7C00; /* 65520 is the tie between 65504 and 2^16 */
    if (a < ldexp(1.0, -14)) {               /* subnormal range: quantum 2^-24 */
        double n = rint(ldexp(a, 24));       /* rint rounds ties to even in the default mode */
        return sign | (uint16_t)n;           /* n == 1024 is the smallest normal, encoded alike */
    }
    int ex;
    frexp(a, &ex);                           /* a = f * 2^ex, f in [0.5, 1) */
    int e = ex - 1;                          /* floor(log2 a) */
    double n = rint(ldexp(a, 10 - e));       /* significand scaled to [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; e += 1; }
    if (e + 15 >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)n - 1024));
}

/* ---- weights ----------------------------------------------------------------------------- */

/* One decoded weight: code nibble (even k in the low nibble) times its block's E4M3 scale times
 * the group's global scale. codes are [G][N][K/2], scales [G][N][K/16]. */
static double weight(const uint8_t *codes, const uint8_t *scales, const float *gscale,
                     int64_t N, int64_t K, int64_t g, int64_t n, int64_t k)
{
    uint8_t byte = codes[(g * N + n) * (K / 2) + k / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 15);
    int sb = scales[(g * N + n) * (K / 16) + k / 16];
    return orc_e2m1(code) * orc_e4m3(sb) * (double)gscale[g];
}

static void weight_row(const uint8_t *codes, const uint8_t *scales, const float *gscale,
                       int64_t N, int64_t K, int64_t g, int64_t n, double *row)
{
    for (int64_t k = 0; k < K; ++k) row[k] = weight(codes, scales, gscale, N, K, g, n, k);
}

/* Full dequantized tensor, out [G][N][K]. For small shapes (tests). */
void orc_dequant(const uint8_t *codes, const uint8_t *scales, const float *gscale,
                 int64_t G, int64_t N, int64_t K, double *out)
{
    for (int64_t g = 0; g < G; ++g)
        for (int64_t n = 0; n < N; ++n) weight_row(codes, scales, gscale, N, K, g, n, out + (g * N + n) * K);
}

static double dot_half_row(const uint16_t *x, const double *w, int64_t K)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += orc_half(x[k]) * w[k];
    return s;
}

/* The same sum with the activation row already decoded to double (xd[k] = orc_half(x[k])): the
 * terms and their order are those of dot_half_row, so the result is bitwise the same. */
static double dot_row(const double *xd, const double *w, int64_t K)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k) s += xd[k] * w[k];
    return s;
}

/* SiLU(g) = g * sigmoid(g) = g / (1 + e^-g). */
double orc_silu(double g) { return g / (1.0 + exp(-g)); }
static double silu(double g) { return orc_silu(g); }

/* ---- dense projection -------------------------------------------------------------------- */

/* y[m][n] = sum_k x[m][k] * W[n][k]  (W has one group). x is fp16 bits [M][K]; y is double [M][N]. */
void orc_linear(const uint16_t *x, int64_t M, int64_t K, const uint8_t *codes, const uint8_t *scales,
                const float *gscale, int64_t N, double *y, int nthreads)
{
#pragma omp parallel num_threads(nthreads)
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            weight_row(codes, scales, gscale, N, K, 0, n, row);
            for (int64_t m = 0; m < M; ++m) y[m * N + n] = dot_half_row(x + m * K, row, K);
        }
        free(row);
    }
}

/* ---- shared expert gate --------------------------------------------------------------------
 * The "shared gate" of the no-MTP page ("Scope and related PRs"; no formula is printed): the
 * shared expert's output enters the MoE output scaled by sigmoid(x . g), g an fp16 vector [K].
 *   sigma[m] = 1 / (1 + exp(-sum_k x[m][k] g[k])),  in double. */
void orc_shared_gate(const uint16_t *x, int64_t M, int64_t K, const uint16_t *g, double *sigma)
{
    for (int64_t m = 0; m < M; ++m) {
        double z = 0.0;
        for (int64_t k = 0; k < K; ++k) z += orc_half(x[m * K + k]) * orc_half(g[k]);
        sigma[m] = 1.0 / (1.0 + exp(-z));
    }
}

/* ---- channel-FP8 dense projection ---------------------------------------------------------
 * The channel-FP8 "QPN8" projection ("[SM70][Draft] Extend Qwen3.8 DFlash2 concurrency paths",
 * "Follow-up: exact channel-FP8 QPN8 concurrency paths and endpoint evidence"): weights are E4M3FN
 * bytes with one FP32 scale per output channel (weight row). The plain definition:
 *   y[m][n] = sum_k x[m][k] * (e4m3(W[n][k]) * s[n]),
 * in double (e4m3 has 4 significant bits and s 24, so each weight is exact). */
void orc_linear_fp8(const uint16_t *x, int64_t M, int64_t K, const uint8_t *codes, const float *chscale,
                    int64_t N, double *y, int nthreads)
{
#pragma omp parallel num_threads(nthreads)
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) row[k] = orc_e4m3(codes[n * K + k]) * (double)chscale[n];
            for (int64_t m = 0; m < M; ++m) y[m * N + n] = dot_half_row(x + m * K, row, K);
        }
        free(row);
    }
}

/* ---- dense gated MLP ----------------------------------------------------------------------
 * The packed gate/up projection with SwiGLU and the down projection of a dense NVFP4 MLP ("[SM70]
 * [Draft] Extend Qwen3.8 DFlash2 concurrency paths", "TP4-only NVFP4 verifier follow-up": gate/up
 * and down projections of the packed MLP weights). For token m:
 *   g_i = sum_k x[m][k] W13[gate_i][k],  u_i likewise on the up row,  h_i = silu(g_i) * u_i,
 *   y_n = sum_i W2[n][i] h_i.
 * W13 is [2I][K] (layout 0: gate rows [0, I), up rows [I, 2I); layout 1: row 2i gate i, row 2i+1
 * up i); W2 is [N][I]. h stays in double (the plain definition). h [M][I] and y [M][N] are double.
 * The sums run in ascending index order, exactly as the MoE oracle's, so a one-expert top-1 MoE
 * with weight 1 gives the same values. */
void orc_gated_mlp(const uint16_t *x, int64_t M, int64_t K, int64_t I,
                   const uint8_t *c13, const uint8_t *s13, const float *g13, int32_t layout,
                   const uint8_t *c2, const uint8_t *s2, const float *g2, int64_t N,
                   double *h, double *y, int nthreads)
{
#pragma omp parallel num_threads(nthreads)
    {
        double *gr = (double *)malloc(sizeof(double) * (size_t)K);
        double *ur = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < I; ++i) {
            weight_row(c13, s13, g13, 2 * I, K, 0, layout ? 2 * i : i, gr);
            weight_row(c13, s13, g13, 2 * I, K, 0, layout ? 2 * i + 1 : I + i, ur);
            for (int64_t m = 0; m < M; ++m) {
                double g = dot_half_row(x + m * K, gr, K);
                double u = dot_half_row(x + m * K, ur, K);
                h[m * I + i] = silu(g) * u;
            }
        }
        free(gr);
        free(ur);
    }
#pragma omp parallel num_threads(nthreads)
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 16)
        for (int64_t n = 0; n < N; ++n) {
            weight_row(c2, s2, g2, N, I, 0, n, row);
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t i = 0; i < I; ++i) acc += row[i] * h[m * I + i];
                y[m * N + n] = acc;
            }
        }
        free(row);
    }
}

/* ---- routing plan ------------------------------------------------------------------------ */

/* Stable counting sort of the (token, slot) pairs by expert id.
 * pair p = t*topk + k; an id is valid when 0 <= id < E; -1 means "no expert"; any other value is
 * also skipped and counted in n_bad.
 *   counts[e]       number of valid pairs routed to e
 *   offsets[e]      exclusive prefix sum of counts (offsets[E] = n_valid)
 *   sorted_pair[j]  pairs in bucket order: by expert, ties by ascending p  (j < n_valid)
 *   pos_of_pair[p]  j such that sorted_pair[j] == p, or -1 for a skipped pair
 *   active[a]       experts with counts > 0, ascending (a < n_active)
 *   tile_expert/tile_row0  row tiles of BM rows per active expert, in (expert, row0) order
 *   summary         {n_valid, n_active, n_bad, n_tiles}                                        */
void orc_plan(const int32_t *ids, int64_t M, int64_t topk, int64_t E, int64_t BM,
              int32_t *counts, int32_t *offsets, int32_t *sorted_pair, int32_t *pos_of_pair,
              int32_t *active, int32_t *tile_expert, int32_t *tile_row0, int32_t *summary)
{
    int64_t P = M * topk, n_bad = 0;
    for (int64_t e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t p = 0; p < P; ++p) {
        int32_t id = ids[p];
        if (id >= 0 && id < E) counts[id]++;
        else if (id != -1) n_bad++;
    }
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int64_t e = 0; e < E; ++e) cursor[e] = offsets[e];
    for (int64_t p = 0; p < P; ++p) {
        int32_t id = ids[p];
        if (id >= 0 && id < E) {
            int32_t j = cursor[id]++;
            sorted_pair[j] = (int32_t)p;
            pos_of_pair[p] = j;
        } else {
            pos_of_pair[p] = -1;
        }
    }
    free(cursor);
    int32_t na = 0, nt = 0;
    for (int64_t e = 0; e < E; ++e) {
        if (counts[e] == 0) continue;
        active[na++] = (int32_t)e;
        for (int32_t r = 0; r < counts[e]; r += (int32_t)BM) {
            tile_expert[nt] = (int32_t)e;
            tile_row0[nt] = r;
            nt++;
        }
    }
    summary[0] = offsets[E];
    summary[1] = na;
    summary[2] = (int32_t)n_bad;
    summary[3] = nt;
}

/* ---- router ------------------------------------------------------------------------------
 * Top-k routing from router logits, the "router" step the no-MTP page lists among the fused MoE
 * parts ("Scope and related PRs"). The pages print no formula; the plainest reading is used:
 *   - token t takes the experts of its topk largest logits, largest first;
 *   - equal logits (+0 and -0 are equal) go in ascending expert order;
 *   - a NaN logit ranks below every number (NaNs among themselves by expert order);
 *   - the slot weights are the softmax of the selected logits,
 *       w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0),  l_0 the first (largest) selected logit,
 *     which equals the full softmax over all experts renormalised over the selection.
 * The selection keeps a sorted list of at most topk experts and inserts each expert in turn; the
 * weights are computed in double from the fp32 logits. */
static int route_before(float a, int32_t ia, float b, int32_t ib)
{
    int an = isnan(a), bn = isnan(b);
    if (an || bn) return (an && bn) ? ia < ib : bn;
    if (a != b) return a > b;
    return ia < ib;
}

void orc_route(const float *logits, int64_t M, int64_t E, int64_t topk, int32_t *ids, double *w)
{
    for (int64_t t = 0; t < M; ++t) {
        const float *x = logits + t * E;
        int32_t *sel = ids + t * topk;
        int64_t n = 0;
        for (int32_t e = 0; e < E; ++e) {
            if (n == topk && !route_before(x[e], e, x[sel[n - 1]], sel[n - 1])) continue;
            int64_t j = n < topk ? n++ : topk - 1;
            while (j > 0 && route_before(x[e], e, x[sel[j - 1]], sel[j - 1])) {
                sel[j] = sel[j - 1];
                --j;
            }
            sel[j] = e;
        }
        double *wt = w + t * topk, l0 = (double)x[sel[0]], s = 0.0;
        for (int64_t k = 0; k < topk; ++k) {
            wt[k] = exp((double)x[sel[k]] - l0);
            s += wt[k];
        }
        for (int64_t k = 0; k < topk; ++k) wt[k] /= s;
    }
}

/* ---- grouped MoE ------------------------------------------------------------------------- */

typedef struct {
    int64_t K, I, E;
    const uint8_t *c13, *s13; const float *g13; int32_t layout;
    const uint8_t *c2, *s2; const float *g2;
} moe_w;

static int64_t gate_row(const moe_w *w, int64_t i) { return w->layout ? 2 * i : i; }
static int64_t up_row(const moe_w *w, int64_t i) { return w->layout ? 2 * i + 1 : w->I + i; }

/* Per-token form. For each listed token t and each slot k in order (skipping ids outside [0,E)):
 *   g_i = sum_k x[t,k] W13[e, gate_i, k],  u_i = sum_k x[t,k] W13[e, up_i, k]
 *   h_i = silu(g_i) * u_i,  y_n = sum_i W2[e, n, i] h_i,  out[t, n] += w[t,k] * y_n
 * out is [n_tokens][K]; h_out (may be NULL) is [n_tokens][topk][I], NaN for skipped slots. */
void orc_moe_token(const uint16_t *x, const int32_t *ids, const float *tw, int64_t M, int64_t topk,
                   int64_t E, int64_t K, int64_t I,
                   const uint8_t *c13, const uint8_t *s13, const float *g13, int32_t layout,
                   const uint8_t *c2, const uint8_t *s2, const float *g2,
                   const int32_t *tokens, int64_t n_tokens, double *out, double *h_out, int nthreads)
{
    moe_w w = {K, I, E, c13, s13, g13, layout, c2, s2, g2};
    (void)M;
#pragma omp parallel num_threads(nthreads)
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)(K > I ? K : I));
        double *h = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n_tokens; ++q) {
            int64_t t = tokens[q];
            const uint16_t *xt = x + t * K;
            double *o = out + q * K;
            for (int64_t n = 0; n < K; ++n) o[n] = 0.0;
            for (int64_t k = 0; k < topk; ++k) {
                int32_t e = ids[t * topk + k];
                if (h_out)
                    for (int64_t i = 0; i < I; ++i) h_out[(q * topk + k) * I + i] = NAN;
                if (e < 0 || e >= E) continue;
                for (int64_t i = 0; i < I; ++i) {
                    weight_row(c13, s13, g13, 2 * I, K, e, gate_row(&w, i), row);
                    double g = dot_half_row(xt, row, K);
                    weight_row(c13, s13, g13, 2 * I, K, e, up_row(&w, i), row);
                    double u = dot_half_row(xt, row, K);
                    h[i] = silu(g) * u;
                    if (h_out) h_out[(q * topk + k) * I + i] = h[i];
                }
                double wk = (double)tw[t * topk + k];
                for (int64_t n = 0; n < K; ++n) {
                    weight_row(c2, s2, g2, K, I, e, n, row);
                    double y = 0.0;
                    for (int64_t i = 0; i < I; ++i) y += row[i] * h[i];
                    o[n] += wk * y;
                }
            }
        }
        free(row);
        free(h);
    }
}

/* Grouped form, driven by the plan of orc_plan. For each active expert e its weights are decoded
 * once, then every pair j in e's bucket gets
 *   h[j][i] = silu(g)*u   (the same sums as above)   and   y[j][n] = sum_i W2[e,n,i] h[j][i].
 * Then out[t][n] = sum over slots k in order of w[t,k] * y[pos_of_pair[t*topk+k]][n].
 * h is [n_valid][I] in bucket order; out is [M][K]; y scratch is allocated here. */
void orc_moe_grouped(const uint16_t *x, const float *tw, int64_t M, int64_t topk, int64_t E,
                     int64_t K, int64_t I,
                     const uint8_t *c13, const uint8_t *s13, const float *g13, int32_t layout,
                     const uint8_t *c2, const uint8_t *s2, const float *g2,
                     const int32_t *offsets, const int32_t *sorted_pair, const int32_t *pos_of_pair,
                     double *h, double *out, int nthreads)
{
    moe_w w = {K, I, E, c13, s13, g13, layout, c2, s2, g2};
    int64_t n_valid = offsets[E];
    double *y = (double *)malloc(sizeof(double) * (size_t)(n_valid > 0 ? n_valid : 1) * (size_t)K);
#pragma omp parallel num_threads(nthreads)
    {
        double *w13 = (double *)malloc(sizeof(double) * (size_t)(2 * I * K));
        double *w2 = (double *)malloc(sizeof(double) * (size_t)(K * I));
        double *xd = (double *)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(dynamic, 1)
        for (int64_t e = 0; e < E; ++e) {
            if (offsets[e + 1] == offsets[e]) continue;
            for (int64_t r = 0; r < 2 * I; ++r) weight_row(c13, s13, g13, 2 * I, K, e, r, w13 + r * K);
            for (int64_t n = 0; n < K; ++n) weight_row(c2, s2, g2, K, I, e, n, w2 + n * I);
            for (int64_t j = offsets[e]; j < offsets[e + 1]; ++j) {
                int64_t t = sorted_pair[j] / topk;
                const uint16_t *xt = x + t * K;
                double *hj = h + j * I;
                for (int64_t k = 0; k < K; ++k) xd[k] = orc_half(xt[k]);  /* decoded once per pair */
                for (int64_t i = 0; i < I; ++i) {
                    double g = dot_row(xd, w13 + gate_row(&w, i) * K, K);
                    double u = dot_row(xd, w13 + up_row(&w, i) * K, K);
                    hj[i] = silu(g) * u;
                }
                for (int64_t n = 0; n < K; ++n) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < I; ++i) acc += w2[n * I + i] * hj[i];
                    y[j * K + n] = acc;
                }
            }
        }
        free(w13);
        free(w2);
        free(xd);
    }
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < M; ++t) {
        for (int64_t n = 0; n < K; ++n) out[t * K + n] = 0.0;
        for (int64_t k = 0; k < topk; ++k) {
            int32_t j = pos_of_pair[t * topk + k];
            if (j < 0) continue;
            double wk = (double)tw[t * topk + k];
            for (int64_t n = 0; n < K; ++n) out[t * K + n] += wk * y[(int64_t)j * K + n];
        }
    }
    free(y);
}

/* W2 and the weighted reduction alone, fed a given fp16 h [n_valid][I] in bucket order (to check
 * the W2 stage in isolation against a device-produced h). out is [M][K]. */
void orc_w2_reduce(const uint16_t *h16, const float *tw, int64_t M, int64_t topk, int64_t E,
                   int64_t K, int64_t I, const uint8_t *c2, const uint8_t *s2, const float *g2,
                   const int32_t *offsets, const int32_t *sorted_pair, const int32_t *pos_of_pair,
                   double *out, int nthreads)
{
    int64_t n_valid = offsets[E];
    double *y = (double *)malloc(sizeof(double) * (size_t)(n_valid > 0 ? n_valid : 1) * (size_t)K);
    (void)sorted_pair;
#pragma omp parallel num_threads(nthreads)
    {
        double *row = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(dynamic, 1)
        for (int64_t e = 0; e < E; ++e) {
            for (int64_t n = 0; n < K && offsets[e + 1] > offsets[e]; ++n) {
                weight_row(c2, s2, g2, K, I, e, n, row);
                for (int64_t j = offsets[e]; j < offsets[e + 1]; ++j) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < I; ++i) acc += row[i] * orc_half(h16[j * I + i]);
                    y[j * K + n] = acc;
                }
            }
        }
        free(row);
    }
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t t = 0; t < M; ++t) {
        for (int64_t n = 0; n < K; ++n) out[t * K + n] = 0.0;
        for (int64_t k = 0; k < topk; ++k) {
            int32_t j = pos_of_pair[t * topk + k];
            if (j < 0) continue;
            double wk = (double)tw[t * topk + k];
            for (int64_t n = 0; n < K; ++n) out[t * K + n] += wk * y[(int64_t)j * K + n];
        }
    }
    free(y);
}
