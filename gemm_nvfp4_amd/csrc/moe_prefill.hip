// moe_prefill.hip -- grouped expert GEMMs of the MoE layer, prefill (MFMA-bound) regime: the
// 8192-token, top-10 W13/W2 route of the "[Perf][SM70] Optimize Qwen3.8 Flash Next prefill" page
// ("SM70 QSA indexer hotspot update": default W13/W2 at 8192 tokens / top-10).
//
// With hundreds of pairs per expert the layer is a dense contraction (about 570 FLOP per weight
// byte), so the design goal is MFMA throughput. gfx950 design:
//   * A block owns one active expert and a slice of its output columns: 128 i values (their gate
//     and up rows) for W13, or 256 output rows for W2. It walks the expert's bucket rows in passes
//     (96 rows for W13, 80 for the multi-chunk W2, 48 for the one-chunk W2). Blocks of one expert
//     are numbered consecutively and mapped to the same XCD, so they share the expert's activation
//     rows in that XCD's L2.
//   * Each wave owns four 16-wide weight tiles (W13: gate and up of two i slices; W2: four output
//     tiles). W13 runs one wave per SIMD (up to 512 registers) with six row tiles: 24 independent
//     accumulator chains keep the matrix pipe busy and each A fragment read from LDS feeds 4
//     MFMAs. The one-chunk W2 runs two blocks per CU with three row tiles, so that one block's
//     latencies hide behind the other's MFMAs.
//   * Per 512-element chunk a wave decodes its weights once (gfx950 fp4/fp8 converts plus one
//     exact fp16 multiply) and reuses each B fragment for all row tiles. Packed weights are loaded
//     one chunk ahead, a quarter at a time, into the registers the current chunk has finished with.
//   * Activation rows are staged in LDS a quarter chunk at a time (lane group q's 32 elements of one
//     step group, for every row), a quarter ahead of their use.
//   * Global memory is read through buffer resources: a uniform base in scalar registers and a
//     32-bit per-lane offset, so a lane keeps one register per stream instead of a 64-bit pointer,
//     and out-of-range reads return zero. The host only picks this regime when every offset fits.
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

constexpr int PF_R = 5;                 // row tiles per wave (and per pass)
constexpr int PF_ROWS = 16 * PF_R;      // bucket rows per pass
constexpr int PF_T = 4;                 // weight tiles per wave
constexpr int AQ = 32;                  // elements of one lane group per quarter chunk (one step group)
constexpr int NBUF = 3;                 // ring of quarter buffers

// Staged activation quarters: [buffer][lane group q][row][AQ elements], each row's four 16-byte
// units swizzled. Measured on MI355X (LDS bank-conflict counters over address patterns), a
// ds_read_b128 is served 32 lanes at a time from 128 four-byte banks, so it is conflict-free when
// each half-wave's 32 addresses fall in 32 different 16-byte slots modulo 512 bytes. The MFMA A
// read of lane (n, q) takes unit s of row 16r + n in plane q: half a wave is rows 0..15 of two
// planes, which no row padding can spread over 32 slots (the old 272-byte pitch left 50% of the
// LDS cycles to conflicts). XOR-ing the unit with bit 3 of the row and bit 0 of q puts rows n and
// n + 8, and planes q and q + 1, on different slots. A row is 64 bytes and every plane's row count
// is a multiple of 16, so planes start at multiples of 512 bytes and a slot depends only on the
// row within its 8-row group, the plane's parity and the unit.
__device__ __forceinline__ int a_unit(int row, int q, int u) { return u ^ ((row >> 3) & 1) ^ ((q & 1) << 1); }

// The 16-byte piece of a staged quarter that thread t loads and stores for each 16-row group:
// unit ps of lane group qs of row srow. Each half-wave stores eight rows of one plane (32
// distinct slots, conflict-free by a_unit), and four consecutive threads read one 64-byte
// segment of a row from global memory.
struct StagePiece {
    int qs, ps, srow;
};
__device__ __forceinline__ StagePiece stage_piece()
{
    const int t = threadIdx.x, hw = (t >> 5) & 7;
    return {hw & 3, t & 3, 8 * (hw >> 2) + ((t >> 2) & 7)};
}
#ifndef NVFP4_W2S1_R
#define NVFP4_W2S1_R 3
#endif
constexpr int W2S1_R = NVFP4_W2S1_R;   // row tiles per pass of the one-chunk W2 kernel (two blocks per CU)

struct __attribute__((aligned(16))) PrefillShared {
    f16 a[NBUF][4][PF_ROWS][AQ];  // activation quarters: [buffer][lane group q][row][32 elements, swizzled]
    int arow[PF_ROWS];            // activation row (token or bucket row) of each pass row
    int pair[PF_ROWS];            // pair index of each pass row (W2: where its result goes)
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

// Eight E2M1 codes (one dword, element order) -> four unscaled fp16 pairs.
__device__ __forceinline__ void e2m1_pairs(f16x2 (&o)[4], uint32_t codes)
{
    o[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
    o[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
    o[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
    o[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
}

// Four unscaled pairs times one block scale -> eight exact fp16 weights: the same products as
// decode8, formed from converts issued earlier.
__device__ __forceinline__ f16x8 scale8(const f16x2 (&p)[4], f16 scale)
{
    const f16x2 s2 = {scale, scale};
    const f16x2 p0 = p[0] * s2, p1 = p[1] * s2, p2 = p[2] * s2, p3 = p[3] * s2;
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// One thread's 16-byte pieces of a staged quarter: one per row tile of the pass.
template <int NR>
struct StageRegs {
    u32x4 v[NR];
};

// Scheduling hints for one MFMA step (row tile outer, weight tile inner): each MFMA is followed by
// up to two VALU ops (the next step's B decode), and each row tile's four MFMAs by the LDS read
// of that row tile's next A fragment, which reuses the fragment's registers.
template <int NR>
__device__ __forceinline__ void interleave_step()
{
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int t = 0; t < PF_T; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
}

// Where one pass reads its operands.
struct PassSrc {
    rsrc_t act;           // activation rows (x for W13, h for W2)
    uint32_t row_bytes;   // bytes per activation row
    rsrc_t codes, scales; // this expert's packed weights
    int red;              // reduction length (K for W13, I for W2)
};

// All chunks of one pass: tot = ((c0 + c1) + c2) + ..., each chunk a chain of 16 MFMA steps
// j = 4b + s from +0, every accumulator seeing its steps in ascending order.
//
// Software pipeline, per wave:
//   * MFMA steps: while step j's NR x 4 MFMAs run, the B fragments of step j + 1 are scaled and
//     the codes of step j + 2 converted (two independent halves of the decode: a convert followed
//     at once by the multiply that reads it stalls the in-order issue, measured at about 1.8 us
//     per 80-row chunk on MI355X), and as soon as a row tile's four MFMAs have issued, its A fragment
//     for step j + 1 is read from LDS. Each B fragment feeds NR MFMAs and each A fragment feeds 4.
//   * Activations move through LDS a quarter chunk at a time (quarter g = 4c + b: lane group q's
//     32 elements of step group b, for every row), in a ring of three buffers. Quarter g + 2 is
//     loaded into registers when quarter g starts and stored to LDS when it ends, so quarter g + 1
//     is in LDS a whole quarter before it is needed and the A reads for its first step are issued
//     during the last step of quarter g. A buffer is rewritten only after the barrier that ends
//     its last reader's quarter.
//   * Weights: packed registers for one chunk. Right after quarter b of chunk c has been decoded
//     for the last time, its registers are refilled with quarter b of chunk c + 1.
// Vector memory ops retire in issue order; every wait is for loads issued at least a quarter
// earlier. Barriers order LDS only, so they never wait for loads in flight.
//
// Loads are unconditional, so they need no branches: rows past `rows` re-read the pass's first row
// and compute results that are never stored (MFMA rows are independent). Lane groups past a
// short chunk's end are staged as exact zeros in A and get zero block scales in B, so their
// products are +-0 and cannot change a sum.
//
// wo[t] is the byte offset of the lane's share of weight tile t inside the expert's codes (row *
// red/2 + 64q); the matching scale offset is wo[t] / 8.
template <int NR, class Epi>
__device__ __forceinline__ void pass_chunks(PrefillShared &sh, const PassSrc &src, int rows, const uint32_t (&wo)[PF_T],
                                            bool working, int n, int q, Epi &&epi)
{
    const int red = src.red, S = num_chunks(red), G = 4 * S;
    const StagePiece sp = stage_piece();
    const int qs = sp.qs, ps = sp.ps, srow = sp.srow;  // staged piece
    uint32_t vo[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int r = srow + 16 * i;
        vo[i] = (uint32_t)sh.arow[r < rows ? r : 0] * src.row_bytes + 256 * qs + 16 * ps;
    }
    auto groups_of = [&](int c) { return min(KCHUNK, red - c * KCHUNK) >> 7; };
    // Lane groups past a short chunk's end stage zeros: their loads get an offset of at least 2^31,
    // out of range of every buffer here (all are smaller than 2^31 bytes), and read as zero.
    auto stage_load = [&](StageRegs<NR> &st, int g) {
        g = g < G ? g : G - 1;  // quarters past the end re-read the last one; they are never used
        const uint32_t so = (uint32_t)((g >> 2) * KCHUNK + AQ * (g & 3)) * 2;
        const uint32_t oob = qs < groups_of(g >> 2) ? 0u : 0x80000000u;
#pragma unroll
        for (int i = 0; i < NR; ++i) st.v[i] = bload16(src.act, vo[i] | oob, so);
    };
    auto stage_store = [&](const StageRegs<NR> &st, int buf) {
#pragma unroll
        for (int i = 0; i < NR; ++i) *reinterpret_cast<u32x4 *>(&sh.a[buf][qs][srow + 16 * i][8 * a_unit(srow, qs, ps)]) = st.v[i];
    };
    RawChunk w[PF_T];
    auto load_quarter = [&](int c, int b) {
        c = c < S ? c : S - 1;  // the last chunk refills itself: cache hits, never used
#pragma unroll
        for (int t = 0; t < PF_T; ++t) {
            w[t].codes[b] = bload16(src.codes, wo[t] + 16 * b, (uint32_t)c * (KCHUNK / 2));
            if (b & 1) w[t].scales[b >> 1] = bload4(src.scales, (wo[t] >> 3) + 4 * (b >> 1), (uint32_t)c * (KCHUNK / 16));
        }
    };
    auto buf_next = [](int x) { return x == NBUF - 1 ? 0 : x + 1; };

    StageRegs<NR> st;
    // Prologue: quarters 0 and 1 in LDS, chunk 0's weights in registers.
    stage_load(st, 0);
    stage_store(st, 0);
    stage_load(st, 1);
#pragma unroll
    for (int b = 0; b < 4; ++b) load_quarter(0, b);
    stage_store(st, 1);
    lds_barrier();

    f32x4 tot[PF_R][PF_T], ca[PF_R][PF_T];
    f16x8 bf[2][PF_T], av[NR];
    f16x2 raw[PF_T][4];
    f16x2 sc[PF_T];
    int cur = 0;  // LDS buffer of the current quarter
    // B decode in two stages, so that no VALU op waits on the one just before it:
    //   cvt_step: E2M1 codes of step (b, s) -> unscaled fp16 pairs in raw (two steps ahead);
    //   mul_step: raw times the block scale -> B fragments of step (b, s) of chunk c in bf[slot]
    //             (one step ahead). Each step runs mul_step before cvt_step overwrites raw.
    auto cvt_step = [&](int b, int s) {
#pragma unroll
        for (int t = 0; t < PF_T; ++t) e2m1_pairs(raw[t], w[t].codes[b][s]);
    };
    auto mul_step = [&](int slot, int c, int b, int s) {
        if (s == 0) {
            const bool qv = q < groups_of(c < S ? c : S - 1);
#pragma unroll
            for (int t = 0; t < PF_T; ++t) sc[t] = qv ? chunk_scales(w[t], b) : f16x2{0, 0};
        }
#pragma unroll
        for (int t = 0; t < PF_T; ++t) bf[slot][t] = scale8(raw[t], sc[t][s >> 1]);
    };
    auto a_read = [&](int r, int s, int buf) {
        return *reinterpret_cast<const f16x8 *>(&sh.a[buf][q][16 * r + n][8 * a_unit(n, q, s)]);
    };
    // The chunk sum starts from -0, the exact identity of addition (-0 + x is x for every x,
    // zeros of both signs included), so no chunk needs a special case.
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < PF_T; ++t) tot[r][t] = f32x4{-0.f, -0.f, -0.f, -0.f};
    cvt_step(0, 0);
    mul_step(0, 0, 0, 0);
    cvt_step(0, 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) av[r] = a_read(r, 0, 0);
    for (int c = 0; c < S; ++c) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int b = j >> 2, s = j & 3, g = 4 * c + b, slot = j & 1;
            if (s == 0) stage_load(st, g + 2);
            // Operands of steps j + 1 (scaled) and j + 2 (converted). Steps past 15 belong to the
            // next chunk: quarter 0 of its codes is already refilled and quarter g + 1 is already
            // in LDS (after the last chunk they are stale or refilled; never used).
            const int sn = (j + 1) & 3, bn = ((j + 1) >> 2) & 3, bufn = s == 3 ? buf_next(cur) : cur;
            mul_step(slot ^ 1, j < 15 ? c : c + 1, bn, sn);
            cvt_step(((j + 2) >> 2) & 3, (j + 2) & 3);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
#pragma unroll
                for (int t = 0; t < PF_T; ++t)
                    ca[r][t] = mfma_step(av[r], bf[slot][t], j == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : ca[r][t]);
                av[r] = a_read(r, sn, bufn);
            }
            interleave_step<NR>();
            __builtin_amdgcn_sched_barrier(0);
            if (s == 3) {
                // Quarter b of this chunk is fully decoded: refill it with the next chunk's bytes.
                load_quarter(c + 1, b);
                stage_store(st, buf_next(buf_next(cur)));
                lds_barrier();
                cur = buf_next(cur);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t = 0; t < PF_T; ++t) tot[r][t] += ca[r][t];
    }
    if (working) epi(tot, NR);
}

// One pass with the row-tile count as a compile-time constant, so the MFMA loops have no
// per-tile branches. Only 1, 3 and 5 row tiles are instantiated (a pass of 2 or 4 tiles runs one
// tile of padding rows): more variants in one kernel made the register allocator spill.
// epi(tot, NR) stores the results; nothing stays live across the switch.
template <class Epi>
__device__ __forceinline__ void pass_dispatch(PrefillShared &sh, const PassSrc &src, int rows, const uint32_t (&wo)[PF_T],
                                              bool working, int n, int q, Epi &&epi)
{
    switch ((rows + 15) >> 4) {
    case 1: pass_chunks<1>(sh, src, rows, wo, working, n, q, epi); break;
    case 2:
    case 3: pass_chunks<3>(sh, src, rows, wo, working, n, q, epi); break;
    default: pass_chunks<5>(sh, src, rows, wo, working, n, q, epi); break;
    }
}

// ---- W13 + SwiGLU ---------------------------------------------------------------------------------
// Wave w of block slice nb owns i slices 8*nb + 2w and +1: tiles {gate0, up0, gate1, up1}.
//
// The block's passes form one stream, as in the one-chunk W2 kernel below: every pass runs five
// row tiles (a short last pass computes padding rows that are never stored), and the next pass
// reuses the same weight rows, so
//   * the activation quarter ring runs on across passes (quarter g of pass p is stream quarter
//     p*4S + g); the last two quarters of a pass stage the next pass's first two;
//   * the weight ring wraps: the last chunk refills its quarters with chunk 0, i.e. the next
//     pass's first chunk;
//   * the next pass's row list is loaded at the start of a pass, stored to LDS before the first
//     quarter's barrier and turned into load offsets after it.
// No pass waits for a prologue, and the SwiGLU epilogue of pass p runs while pass p + 1's first
// loads are in flight. The per-element arithmetic is pass_chunks' (chunk chains from +0, chunk
// sums from -0 in order, global scale last).
#ifndef NVFP4_W13_R
#define NVFP4_W13_R 6
#endif
constexpr int W13_R = NVFP4_W13_R;  // row tiles per W13 pass
constexpr int W13_ROWS = 16 * W13_R;
struct __attribute__((aligned(16))) W13Shared {
    f16 a[NBUF][4][W13_ROWS][AQ];  // activation quarters, as in PrefillShared
    int arow[2][W13_ROWS];         // token of each row of pass p, in arow[p & 1]
};

__global__ __launch_bounds__(256, 1) void w13_swiglu_prefill_kernel(PlanView pv, int topk, const f16 *__restrict__ x,
                                                                     uint32_t x_bytes,
                                                                     const uint8_t *__restrict__ codes,
                                                                     const uint8_t *__restrict__ scales,
                                                                     const float *__restrict__ gscale, int K, int I,
                                                                     int layout, f16 *__restrict__ h, int a_max)
{
    constexpr int NR = W13_R;
    __shared__ W13Shared sh;
    const int itiles = I >> 4;
    const int nblk = (itiles + 7) >> 3;  // 8 i slices per block
    const int lb = xcd_logical_block(a_max * nblk);
    if (lb < 0) return;
    const int a = lb / nblk, nb = lb - a * nblk;
    if (a >= pv.hdr[1]) return;  // block-uniform
    const int e = pv.active[a], cnt = pv.counts[e], base = pv.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, q = lane >> 4;
    const int it0 = nb * 8 + 2 * wave;
    const bool working = it0 < itiles;  // the second slice may be missing (odd itiles): guarded below
    const uint32_t ebytes = (uint32_t)(2 * I) * (uint32_t)(K >> 1);  // one expert's codes
    const rsrc_t act = make_rsrc(x, x_bytes);
    const rsrc_t rc = make_rsrc(codes + (size_t)e * ebytes, ebytes);
    const rsrc_t rs = make_rsrc(scales + (size_t)e * (ebytes >> 3), ebytes >> 3);
    const uint32_t row_bytes = (uint32_t)K * 2;
    uint32_t wo[PF_T];
#pragma unroll
    for (int t = 0; t < PF_T; ++t) {
        const int it = min(it0 + (t >> 1), itiles - 1);
        const int i_row = it * 16 + n;
        const int row = (t & 1) == 0 ? (layout ? 2 * i_row : i_row) : (layout ? 2 * i_row + 1 : I + i_row);
        wo[t] = (uint32_t)row * (uint32_t)(K >> 1) + 64 * q;
    }
    const float gs = gscale[e];
    const int S = num_chunks(K), GQ = 4 * S;  // chunks and quarters per pass
    const int npass = (cnt + W13_ROWS - 1) / W13_ROWS;
    const StagePiece sp = stage_piece();
    const int qs = sp.qs, ps = sp.ps, srow = sp.srow;  // staged piece
    auto groups_of = [&](int c) { return min(KCHUNK, K - c * KCHUNK) >> 7; };
    // Token of row threadIdx.x of pass p (rows past the expert's end and passes past the last read
    // token 0: computed, never stored).
    auto arow_load = [&](int p) {
        const int r = p * W13_ROWS + (int)threadIdx.x;
        return (int)threadIdx.x < W13_ROWS && p < npass && r < cnt ? pv.sorted_pair[base + r] / topk : 0;
    };
    auto offsets_of = [&](int p, uint32_t (&vo)[NR]) {
#pragma unroll
        for (int i = 0; i < NR; ++i) vo[i] = (uint32_t)sh.arow[p & 1][srow + 16 * i] * row_bytes + 256 * qs + 16 * ps;
    };
    // Quarter gl (0 .. 4S-1) of the pass whose row offsets are vo. Lane groups past a short
    // chunk's end stage zeros (offsets of at least 2^31 are out of range and read as zero).
    auto stage_load = [&](StageRegs<NR> &st, int gl, const uint32_t (&vo)[NR]) {
        const uint32_t so = (uint32_t)((gl >> 2) * KCHUNK + AQ * (gl & 3)) * 2;
        const uint32_t oob = qs < groups_of(gl >> 2) ? 0u : 0x80000000u;
#pragma unroll
        for (int i = 0; i < NR; ++i) st.v[i] = bload16(act, vo[i] | oob, so);
    };
    auto stage_store = [&](const StageRegs<NR> &st, int buf) {
#pragma unroll
        for (int i = 0; i < NR; ++i) *reinterpret_cast<u32x4 *>(&sh.a[buf][qs][srow + 16 * i][8 * a_unit(srow, qs, ps)]) = st.v[i];
    };
    RawChunk w[PF_T];
    auto load_quarter = [&](int c, int b) {
#pragma unroll
        for (int t = 0; t < PF_T; ++t) {
            w[t].codes[b] = bload16(rc, wo[t] + 16 * b, (uint32_t)c * (KCHUNK / 2));
            if (b & 1) w[t].scales[b >> 1] = bload4(rs, (wo[t] >> 3) + 4 * (b >> 1), (uint32_t)c * (KCHUNK / 16));
        }
    };
    auto buf_next = [](int v) { return v == NBUF - 1 ? 0 : v + 1; };

    // Prologue: pass 0's rows, its quarters 0 and 1 in LDS, chunk 0's weights in registers.
    {
        const int r0 = arow_load(0);
        if ((int)threadIdx.x < W13_ROWS) sh.arow[0][threadIdx.x] = r0;
    }
    __syncthreads();
    uint32_t vo[NR], vo_next[NR];
    offsets_of(0, vo);
    StageRegs<NR> st;
    stage_load(st, 0, vo);
    stage_store(st, 0);
    stage_load(st, 1 < GQ ? 1 : 0, vo);
#pragma unroll
    for (int b = 0; b < 4; ++b) load_quarter(0, b);
    stage_store(st, 1);
    lds_barrier();

    f32x4 tot[NR][PF_T], ca[NR][PF_T];
    f16x8 bf[2][PF_T], av[NR];
    f16x2 raw[PF_T][4];
    f16x2 sc[PF_T];
    int cur = 0;  // LDS buffer of the current quarter
    auto cvt_step = [&](int b, int s) {
#pragma unroll
        for (int t = 0; t < PF_T; ++t) e2m1_pairs(raw[t], w[t].codes[b][s]);
    };
    auto mul_step = [&](int slot, int c, int b, int s) {
        if (s == 0) {
            const bool qv = q < groups_of(c);
#pragma unroll
            for (int t = 0; t < PF_T; ++t) sc[t] = qv ? chunk_scales(w[t], b) : f16x2{0, 0};
        }
#pragma unroll
        for (int t = 0; t < PF_T; ++t) bf[slot][t] = scale8(raw[t], sc[t][s >> 1]);
    };
    auto a_read = [&](int r, int s, int buf) {
        return *reinterpret_cast<const f16x8 *>(&sh.a[buf][q][16 * r + n][8 * a_unit(n, q, s)]);
    };
    cvt_step(0, 0);
    mul_step(0, 0, 0, 0);
    cvt_step(0, 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) av[r] = a_read(r, 0, 0);
    for (int p = 0; p < npass; ++p) {
        const int rows = min(W13_ROWS, cnt - p * W13_ROWS);
        int pr_next = 0;
        // The chunk sum starts from -0, the exact identity of addition.
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t = 0; t < PF_T; ++t) tot[r][t] = f32x4{-0.f, -0.f, -0.f, -0.f};
        for (int c = 0; c < S; ++c) {
            const int cn = c + 1 < S ? c + 1 : 0;  // the chunk after this one (chunk 0: the next pass)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int b = j >> 2, s = j & 3, slot = j & 1;
                if (s == 0) {
                    // Quarter 4c + b + 2, of this pass or the next one.
                    const int g2 = 4 * c + b + 2;
                    if (g2 < GQ) stage_load(st, g2, vo);
                    else stage_load(st, g2 - GQ, vo_next);
                }
                if (c == 0 && j == 0) pr_next = arow_load(p + 1);
                const int sn = (j + 1) & 3, bn = ((j + 1) >> 2) & 3, bufn = s == 3 ? buf_next(cur) : cur;
                mul_step(slot ^ 1, j < 15 ? c : cn, bn, sn);
                cvt_step(((j + 2) >> 2) & 3, (j + 2) & 3);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
#pragma unroll
                    for (int t = 0; t < PF_T; ++t)
                        ca[r][t] = mfma_step(av[r], bf[slot][t], j == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : ca[r][t]);
                    av[r] = a_read(r, sn, bufn);
                }
                interleave_step<NR>();
                __builtin_amdgcn_sched_barrier(0);
                if (s == 3) {
                    // Quarter b of this chunk is fully decoded: refill it with the next chunk's bytes.
                    load_quarter(cn, b);
                    stage_store(st, buf_next(buf_next(cur)));
                    // sh.arow[(p + 1) & 1] was last read two passes ago (offsets of pass p - 1).
                    if (c == 0 && b == 0 && (int)threadIdx.x < W13_ROWS) sh.arow[(p + 1) & 1][threadIdx.x] = pr_next;
                    lds_barrier();
                    if (c == 0 && b == 0) offsets_of(p + 1, vo_next);
                    cur = buf_next(cur);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int t = 0; t < PF_T; ++t) tot[r][t] += ca[r][t];
        }
        if (working) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * r + 4 * q + j;
                    if (row < rows) {
                        f16 *hr = h + (size_t)(base + p * W13_ROWS + row) * I + it0 * 16 + n;
                        hr[0] = f16_of_f32(swiglu(tot[r][0][j] * gs, tot[r][1][j] * gs));
                        if (it0 + 1 < itiles) hr[16] = f16_of_f32(swiglu(tot[r][2][j] * gs, tot[r][3][j] * gs));
                    }
                }
        }
#pragma unroll
        for (int i = 0; i < NR; ++i) vo[i] = vo_next[i];
    }
}

// ---- W2: per-pair FP32 results, in pair order -----------------------------------------------------------------------
// Wave w of block slice nb owns output tiles 16*nb + 4w .. +3 (64 output rows).
__global__ __launch_bounds__(256, 1) void w2_prefill_kernel(PlanView pv, const f16 *__restrict__ hin, uint32_t h_bytes,
                                                             const uint8_t *__restrict__ codes,
                                                             const uint8_t *__restrict__ scales,
                                                             const float *__restrict__ gscale, int K, int I,
                                                             float *__restrict__ ws, int a_max)
{
    __shared__ PrefillShared sh;
    const int ntiles = K >> 4;
    const int nblk = (ntiles + 15) >> 4;  // 16 output tiles per block
    const int lb = xcd_logical_block(a_max * nblk);
    if (lb < 0) return;
    const int a = lb / nblk, nb = lb - a * nblk;
    if (a >= pv.hdr[1]) return;
    const int e = pv.active[a], cnt = pv.counts[e], base = pv.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, q = lane >> 4;
    const int nt0 = nb * 16 + 4 * wave;
    const bool working = nt0 < ntiles;
    const uint32_t ebytes = (uint32_t)K * (uint32_t)(I >> 1);
    PassSrc src;
    src.act = make_rsrc(hin, h_bytes);
    src.row_bytes = (uint32_t)I * 2;
    src.codes = make_rsrc(codes + (size_t)e * ebytes, ebytes);
    src.scales = make_rsrc(scales + (size_t)e * (ebytes >> 3), ebytes >> 3);
    src.red = I;
    uint32_t wo[PF_T];
#pragma unroll
    for (int t = 0; t < PF_T; ++t) wo[t] = (uint32_t)(min(nt0 + t, ntiles - 1) * 16 + n) * (uint32_t)(I >> 1) + 64 * q;
    const float gs = gscale[e];

    for (int rp = 0; rp < cnt; rp += PF_ROWS) {
        const int rows = min(PF_ROWS, cnt - rp);
        lds_barrier();
        for (int r = threadIdx.x; r < rows; r += 256) {
            sh.arow[r] = base + rp + r;
            sh.pair[r] = pv.sorted_pair[base + rp + r];
        }
        __syncthreads();
        pass_dispatch(sh, src, rows, wo, working, n, q, [&](const f32x4 (&tot)[PF_R][PF_T], int nr) {
#pragma unroll
            for (int r = 0; r < PF_R; ++r) {
                if (r >= nr) break;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * r + 4 * q + j;
                    if (row < rows) {
                        float *y = ws + (size_t)sh.pair[row] * K + nt0 * 16 + n;
#pragma unroll
                        for (int t = 0; t < PF_T; ++t)
                            if (nt0 + t < ntiles) y[16 * t] = tot[r][t][j] * gs;
                    }
                }
            }
        });
    }
}

// ---- W2 with one reduction chunk (I <= 512) ----------------------------------------------------------
// Same block geometry as w2_prefill_kernel (16 output tiles per block, 4 per wave), specialised
// for a single 512-element chunk:
//   * two blocks per CU (at most 256 registers per wave, three row tiles per pass), so one block's
//     weight loads, staging and result stores overlap the other block's MFMAs. One block per CU
//     with five row tiles left each block's start-up and stores exposed (396 vs 324 us at 8192
//     tokens on MI355X, same results bitwise);
//   * the block's packed weights are loaded once and stay in registers for all of its passes;
//     they are decoded again in every pass (the 16 steps' decoded fragments would need 256
//     registers, which only fit at one block per CU);
//   * bucket rows of an expert are contiguous, so the activation quarters of every pass form one
//     stream (quarter g = 4*pass + b) and the next pass's first quarters load while this pass
//     finishes;
//   * each pass's accumulators are its results (one chain from +0, no chunk sum); they are stored
//     in pair order right after the pass's last step.
// Rows past the expert's end re-read its last row and are never stored.
template <int NR>
struct S1Shared {
    f16 a[NBUF][4][16 * NR][AQ];  // as in PrefillShared
    int pair[2][16 * NR];  // pair index of each row of pass p, in pair[p & 1]
};

template <int NR>
__global__ __launch_bounds__(256, 2) void w2_prefill_s1_kernel(PlanView pv, const f16 *__restrict__ hin, uint32_t h_bytes,
                                                               const uint8_t *__restrict__ codes,
                                                               const uint8_t *__restrict__ scales,
                                                               const float *__restrict__ gscale, int K, int I,
                                                               float *__restrict__ ws, int a_max)
{
    constexpr int ROWS = 16 * NR;
    constexpr int PIECES = ROWS * 16 / 256;  // 16-byte pieces of a staged quarter per thread
    __shared__ __attribute__((aligned(16))) S1Shared<NR> sh;
    const int ntiles = K >> 4;
    const int nblk = (ntiles + 15) >> 4;
    const int lb = xcd_logical_block(a_max * nblk);
    if (lb < 0) return;
    const int a = lb / nblk, nb = lb - a * nblk;
    if (a >= pv.hdr[1]) return;
    const int e = pv.active[a], cnt = pv.counts[e], base = pv.offsets[e];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, q = lane >> 4;
    const int nt0 = nb * 16 + 4 * wave;
    const bool working = nt0 < ntiles;
    const uint32_t ebytes = (uint32_t)K * (uint32_t)(I >> 1);
    const rsrc_t act = make_rsrc(hin, h_bytes);
    const rsrc_t rc = make_rsrc(codes + (size_t)e * ebytes, ebytes);
    const rsrc_t rs = make_rsrc(scales + (size_t)e * (ebytes >> 3), ebytes >> 3);
    const int groups = I >> 7;  // 128-element lane groups with data (1..4)
    const bool qv = q < groups;
    const float gs = gscale[e];
    const int npass = (cnt + ROWS - 1) / ROWS, G = 4 * npass;

    // The whole reduction axis of the block's four weight tiles, once.
    RawChunk w[PF_T];
#pragma unroll
    for (int t = 0; t < PF_T; ++t) {
        const uint32_t wo = (uint32_t)(min(nt0 + t, ntiles - 1) * 16 + n) * (uint32_t)(I >> 1) + 64 * (qv ? q : 0);
#pragma unroll
        for (int b = 0; b < 4; ++b) w[t].codes[b] = bload16(rc, wo + 16 * b, 0);
        w[t].scales[0] = bload4(rs, wo >> 3, 0);
        w[t].scales[1] = bload4(rs, (wo >> 3) + 4, 0);
    }

    const StagePiece sp = stage_piece();
    const int qs = sp.qs, ps = sp.ps, srow = sp.srow;
    // Lane groups past the end of a short chunk (I < 512) stage zeros: an offset of at least 2^31
    // is out of range of every buffer here (all are smaller than 2^31 bytes) and reads as zero.
    const uint32_t oob = qs < groups ? 0u : 0x80000000u;
    struct Stage {
        u32x4 v[PIECES];
    };
    auto stage_load = [&](Stage &st, int g) {
        g = g < G ? g : G - 1;
        const int r0 = (g >> 2) * ROWS;
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const int row = base + min(r0 + srow + 16 * i, cnt - 1);
            st.v[i] = bload16(act, ((uint32_t)row * (uint32_t)(I * 2) + 256 * qs + 16 * ps) | oob, AQ * 2 * (g & 3));
        }
    };
    auto stage_store = [&](const Stage &st, int buf) {
#pragma unroll
        for (int i = 0; i < PIECES; ++i) *reinterpret_cast<u32x4 *>(&sh.a[buf][qs][srow + 16 * i][8 * a_unit(srow, qs, ps)]) = st.v[i];
    };
    auto pairs_load = [&](int p) {  // pair indices of pass p's rows, one per thread
        const int r = p * ROWS + (int)threadIdx.x;
        return (int)threadIdx.x < ROWS && p < npass && r < cnt ? pv.sorted_pair[base + r] : 0;
    };
    auto buf_next = [](int x) { return x == NBUF - 1 ? 0 : x + 1; };

    // Prologue: quarters 0 and 1 in LDS, quarter 2 loading; pass 0's pair list in LDS.
    Stage st[2];
    stage_load(st[0], 0);
    stage_load(st[1], 1);
    const int pr0 = pairs_load(0);
    stage_store(st[0], 0);
    stage_store(st[1], 1);
    if ((int)threadIdx.x < ROWS) sh.pair[0][threadIdx.x] = pr0;
    stage_load(st[0], 2);
    __syncthreads();

    f16x2 sc[PF_T][4];  // block scales of every step group, decoded once
#pragma unroll
    for (int t = 0; t < PF_T; ++t)
#pragma unroll
        for (int b = 0; b < 4; ++b) sc[t][b] = qv ? chunk_scales(w[t], b) : f16x2{0, 0};
    f32x4 ca[NR][PF_T];
    f16x8 bf[2][PF_T], av[NR];
    f16x2 raw[PF_T][4];
    // B decode in two stages, as in pass_chunks: converts two steps ahead, scaling one step ahead.
    auto cvt_step = [&](int b, int s) {
#pragma unroll
        for (int t = 0; t < PF_T; ++t) e2m1_pairs(raw[t], w[t].codes[b][s]);
    };
    auto mul_step = [&](int slot, int b, int s) {
#pragma unroll
        for (int t = 0; t < PF_T; ++t) bf[slot][t] = scale8(raw[t], sc[t][b][s >> 1]);
    };
    auto a_read = [&](int r, int s, int buf) {
        return *reinterpret_cast<const f16x8 *>(&sh.a[buf][q][16 * r + n][8 * a_unit(n, q, s)]);
    };
    int cur = 0;
    cvt_step(0, 0);
    mul_step(0, 0, 0);
    cvt_step(0, 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) av[r] = a_read(r, 0, 0);
    for (int p = 0; p < npass; ++p) {
        int pr_next = 0;
        // The packed weights are the same in every pass; this empty asm makes them opaque, so the
        // compiler keeps their decode inside the pass loop instead of holding every decoded
        // fragment in registers across passes.
#pragma unroll
        for (int t = 0; t < PF_T; ++t)
#pragma unroll
            for (int b = 0; b < 4; ++b) asm volatile("" : "+v"(w[t].codes[b]));
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int b = j >> 2, s = j & 3, g = 4 * p + b, slot = j & 1;
            if (s == 0) stage_load(st[(b + 1) & 1], g + 3);
            if (j == 4) pr_next = pairs_load(p + 1);
            const int sn = (j + 1) & 3, bn = ((j + 1) >> 2) & 3, bufn = s == 3 ? buf_next(cur) : cur;
            mul_step(slot ^ 1, bn, sn);  // steps past 15: the next pass, same weights
            cvt_step(((j + 2) >> 2) & 3, (j + 2) & 3);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
#pragma unroll
                for (int t = 0; t < PF_T; ++t)
                    ca[r][t] = mfma_step(av[r], bf[slot][t], j == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : ca[r][t]);
                av[r] = a_read(r, sn, bufn);
            }
            interleave_step<NR>();
            __builtin_amdgcn_sched_barrier(0);
            if (s == 3) {
                stage_store(st[b & 1], buf_next(buf_next(cur)));
                if (j == 15 && (int)threadIdx.x < ROWS) sh.pair[(p + 1) & 1][threadIdx.x] = pr_next;
                lds_barrier();
                cur = buf_next(cur);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // This pass's results. sh.pair[p & 1] was written before the barrier that ended the
        // previous pass (or in the prologue), and is rewritten only after the next pass's barrier.
        if (working) {
            const int rows = min(ROWS, cnt - p * ROWS);
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int row = 16 * r + 4 * q + jj;
                    if (row < rows) {
                        float *y = ws + (size_t)sh.pair[p & 1][row] * K + nt0 * 16 + n;
#pragma unroll
                        for (int t = 0; t < PF_T; ++t)
                            if (nt0 + t < ntiles) y[16 * t] = ca[r][t][jj] * gs;
                    }
                }
        }
    }
}

}  // namespace

bool prefill_offsets_fit(int64_t M, int64_t P, int32_t K, int32_t I)
{
    const int64_t lim = (int64_t)1 << 31;
    return M * K * 2 < lim && P * I * 2 < lim && (int64_t)K * I < lim;
}

int run_w13_prefill(const PlanView &pv, int64_t a_max, int32_t M, int32_t topk, const uint16_t *x,
                    const nvfp4_weights &w, int32_t layout, uint16_t *h, hipStream_t s)
{
    const int K = w.k, I = w.rows / 2;
    const int nblk = (I / 16 + 7) / 8;
    const int64_t G = a_max * nblk;
    const unsigned grid = (unsigned)((G + 7) / 8 * 8);
    return launch(w13_swiglu_prefill_kernel, dim3(grid), dim3(256), 0, s, pv, topk, reinterpret_cast<const f16 *>(x),
                  (uint32_t)((int64_t)M * K * 2), w.codes, w.scales, w.global_scale, K, I, layout,
                  reinterpret_cast<f16 *>(h), (int)a_max);
}

int run_w2_prefill(const PlanView &pv, int64_t a_max, int64_t P, const uint16_t *h, const nvfp4_weights &w, float *ws,
                   hipStream_t s)
{
    const int K = w.rows, I = w.k;
    const int nblk = (K / 16 + 15) / 16;
    const int64_t G = a_max * nblk;
    const unsigned grid = (unsigned)((G + 7) / 8 * 8);
    if (I <= KCHUNK)
        return launch(w2_prefill_s1_kernel<W2S1_R>, dim3(grid), dim3(256), 0, s, pv, reinterpret_cast<const f16 *>(h),
                      (uint32_t)(P * I * 2), w.codes, w.scales, w.global_scale, K, I, ws, (int)a_max);
    return launch(w2_prefill_kernel, dim3(grid), dim3(256), 0, s, pv, reinterpret_cast<const f16 *>(h),
                  (uint32_t)(P * I * 2), w.codes, w.scales, w.global_scale, K, I, ws, (int)a_max);
}

}  // namespace nvfp4
