// nvfp4_device.hpp -- device building blocks shared by every GEMM kernel of the library (gfx950).
//
// NVFP4 decode: weights are E2M1 codes with one E4M3FN scale per 16-element K-block (the native
// NVFP4 weights of the "[Kernel][SM70] Improve Qwen3.8 no-MTP concurrency" page, "Scope and related
// PRs"). The product e2m1 * e4m3 always has at most 6 significant bits and lies in [2^-10, 2688],
// so it is exact in binary16. The kernels form it exactly in fp16 and apply the FP32 global scale
// in the FP32 epilogue.
//   - gfx950 converts E2M1 pairs to fp16 (v_cvt_scalef32_pk_f16_fp4) and E4M3 pairs to fp16
//     (v_cvt_scalef32_pk_f16_fp8). The convert's scale operand only contributes its power of two,
//     so it is always 1.0 here.
//   - The block scale is applied with one exact packed fp16 multiply (v_pk_mul_f16).
//
// Reduction order. Every GEMM in the library uses the same one, so a token's result never depends
// on M, on the other tokens or on the kernel variant. This is the batch invariance of the
// "[SM70][Draft] Extend Qwen3.8 DFlash2 concurrency paths" page, "TP4-only NVFP4 verifier
// follow-up": the M-row output equals the concatenated smaller calls, bitwise.
//   * The reduction axis is cut into chunks of KCHUNK = 512 elements. The last chunk may be
//     shorter, always a multiple of 128.
//   * Each chunk is one chain of v_mfma_f32_16x16x32_f16 steps, starting from +0.
//   * Chunk results are added in FP32, left to right: ((c0 + c1) + c2) + ...
//   * A chunk is a run of 128-element superblocks, each of 4 MFMA steps s = 0..3. In step s, lane
//     group q = lane/16 feeds elements [128*b + 32*q + 8*s, +8) of superblock b. One 16-byte code
//     load per lane per row therefore covers a whole superblock: 32 consecutive elements, one
//     dword per step.
// The MFMA result for one output element depends only on its own A row, B column and C input,
// never on its position inside the 16x16 tile (measured on MI355X). Padding rows never change
// other rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KCHUNK = 512;  // elements per independent MFMA chain
constexpr int KSB = 128;     // elements per superblock (4 MFMA steps)

__host__ __device__ constexpr int num_chunks(int k) { return (k + KCHUNK - 1) / KCHUNK; }

// MFMA operand layout (v_mfma_f32_16x16x32_f16, wave64):
//   A: lane l holds row (l % 16), elements 8*(l/16) .. +7 of the step
//   B: lane l holds column (l % 16), elements 8*(l/16) .. +7 of the step
//   D: lane l, register j holds row 4*(l/16) + j, column l % 16
__device__ __forceinline__ f32x4 mfma_step(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Two E4M3FN bytes -> two exact fp16 values. HI selects bytes 2,3 instead of 0,1.
template <bool HI>
__device__ __forceinline__ f16x2 e4m3_pair(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Eight consecutive E2M1 codes (one dword; the even element in each byte's low nibble) times one
// block scale -> eight exact fp16 weights in element order.
__device__ __forceinline__ f16x8 decode8(uint32_t codes, f16 scale)
{
    const f16x2 s2 = {scale, scale};
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Raw packed data of one weight row for one superblock, as one lane loads it: 16 code bytes
// (32 elements) and the two scale bytes that cover them.
struct RawSB {
    u32x4 codes;
    uint32_t scale2;
};

// Lane's share of superblock `sb` of one weight row. `row_codes` / `row_scales` point at the row's
// first byte; `k0` is the superblock's first element (a multiple of 128); q = lane / 16.
__device__ __forceinline__ RawSB load_sb(const uint8_t *row_codes, const uint8_t *row_scales, int k0, int q)
{
    RawSB r;
    r.codes = *reinterpret_cast<const u32x4 *>(row_codes + (k0 >> 1) + 16 * q);
    r.scale2 = *reinterpret_cast<const uint16_t *>(row_scales + (k0 >> 4) + 2 * q);
    return r;
}

// The four B fragments (steps 0..3) of a loaded superblock. Steps 0,1 use the first scale byte
// (elements 32q..32q+15), steps 2,3 the second.
__device__ __forceinline__ void decode_sb(const RawSB &r, f16x8 out[4])
{
    const f16x2 s = e4m3_pair<false>(r.scale2);
    out[0] = decode8(r.codes[0], s[0]);
    out[1] = decode8(r.codes[1], s[0]);
    out[2] = decode8(r.codes[2], s[1]);
    out[3] = decode8(r.codes[3], s[1]);
}

// A fragment of one activation row for superblock starting at element k0, step s.
__device__ __forceinline__ f16x8 load_a(const f16 *row, int k0, int q, int s)
{
    return *reinterpret_cast<const f16x8 *>(row + k0 + 32 * q + 8 * s);
}

__device__ __forceinline__ f16x8 zero8()
{
    return f16x8{0, 0, 0, 0, 0, 0, 0, 0};
}

// SiLU(g) * u in FP32, as fixed for every regime: g / (1 + e^-g) * u.
__device__ __forceinline__ float swiglu(float g, float u)
{
    return g / (1.0f + expf(-g)) * u;
}

}  // namespace nvfp4
