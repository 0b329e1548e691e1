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
//   * Each chunk is one chain of 16 v_mfma_f32_16x16x32_f16 steps j = 4*b + s (b, s = 0..3),
//     starting from +0.
//   * Chunk results are added in FP32, left to right: ((c0 + c1) + c2) + ...
//   * Lane group q = lane/16 owns the contiguous elements [128q, 128q + 128) of the chunk. In
//     step (b, s) it feeds elements [128q + 32b + 8s, +8). Lane groups past the end of a short
//     chunk feed exact zeros in both operands.
//     Each lane therefore reads 64 contiguous code bytes (four 16-byte loads) and its 8 scale
//     bytes (one 8-byte load) per row per chunk. Measured on MI355X, this beats a layout whose
//     scales need four 2-byte loads.
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

// One lane's packed data of one weight row for one chunk: 64 code bytes (128 elements, four
// 16-byte loads) and the 8 E4M3 scale bytes that cover them (one 8-byte load).
struct RawChunk {
    u32x4 codes[4];     // codes[b].dword[s] = elements [kb + 128q + 32b + 8s, +8)
    uint32_t scales[2]; // byte 2b + (s >> 1) scales step (b, s)
};

// Lane's share of one weight row for the chunk starting at element kb (a multiple of 512).
// `q_ld` is the lane group whose bytes are loaded (clamped into the chunk by the caller).
__device__ __forceinline__ RawChunk load_chunk(const uint8_t *row_codes, const uint8_t *row_scales, int kb, int q_ld)
{
    RawChunk r;
    const uint8_t *c = row_codes + (kb >> 1) + 64 * q_ld;
#pragma unroll
    for (int b = 0; b < 4; ++b) r.codes[b] = *reinterpret_cast<const u32x4 *>(c + 16 * b);
    const uint2 sc = *reinterpret_cast<const uint2 *>(row_scales + (kb >> 4) + 8 * q_ld);
    r.scales[0] = sc.x;
    r.scales[1] = sc.y;
    return r;
}

// load_chunk with the row split into a wave-uniform base and this lane's byte offsets from it
// (codes: its row and lane group within the chunk; scales likewise). Offsets below 2^32 let the
// loads take the base in scalar registers and one 32-bit offset per lane.
__device__ __forceinline__ RawChunk load_chunk_at(const uint8_t *cbase, uint32_t coff, const uint8_t *sbase, uint32_t soff)
{
    RawChunk r;
    const uint8_t *c = cbase + coff;
#pragma unroll
    for (int b = 0; b < 4; ++b) r.codes[b] = *reinterpret_cast<const u32x4 *>(c + 16 * b);
    const uint2 sc = *reinterpret_cast<const uint2 *>(sbase + soff);
    r.scales[0] = sc.x;
    r.scales[1] = sc.y;
    return r;
}

// The two block scales of load b (steps s = 0,1 and s = 2,3), as fp16.
__device__ __forceinline__ f16x2 chunk_scales(const RawChunk &r, int b)
{
    const uint32_t w = r.scales[b >> 1];
    return (b & 1) ? e4m3_pair<true>(w) : e4m3_pair<false>(w);
}

// A fragment of step (b, s) of an activation row, chunk starting at kb.
__device__ __forceinline__ f16x8 a_frag(const f16 *row, int kb, int q, int b, int s)
{
    return *reinterpret_cast<const f16x8 *>(row + kb + 128 * q + 32 * b + 8 * s);
}

__device__ __forceinline__ f16x8 zero8()
{
    return f16x8{0, 0, 0, 0, 0, 0, 0, 0};
}

// ---- buffer loads ----------------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes). Dword 3 = 0x00020000 selects the 32-bit data
// format that gfx9 untyped buffer loads require. Reads at offsets >= bytes return zero, so a lane
// that must feed zeros can load at BUF_OOB instead of branching around its load (a branch around a
// load makes the compiler wait for every earlier load before any later one issues).
constexpr uint32_t BUF_OOB = 0x40000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t voff, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Block barrier that orders LDS only. __syncthreads() also fences global memory, and on gfx9 that
// means s_waitcnt vmcnt(0): it would wait for loads still in flight (a prefetch). Kernels that pass
// no global data between the waves of a block use this instead.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// SiLU(g) * u in FP32, the same in every regime: g * (1 / (1 + e^-g)) * u. e^-g is taken as
// 2^(-g * log2 e) by the hardware base-2 exponential (v_exp_f32) and the reciprocal by v_rcp_f32,
// each within about one FP32 ulp, far below the fp16 rounding of h. Overflow behaves as in the
// plain formula: e^-g = inf gives a signed zero, and g = -inf gives NaN.
__device__ __forceinline__ float swiglu(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// fp16_rne of an FP32 value that is already rounded to FP32: every fp16 output of the library (h,
// the MoE output, the dense projections) is one conversion of an FP32 result. The empty asm keeps
// the compiler from merging the conversion into the multiply or fmaf that produced x (a
// mixed-precision FMA would round the exact result to fp16 once, which differs at ties), so every
// kernel that writes the same output rounds it the same way.
__device__ __forceinline__ f16 f16_of_f32(float x)
{
    asm volatile("" : "+v"(x));
    return (f16)x;
}

// An FP32 result to the output type: fp16 through f16_of_f32, FP32 as is.
template <typename OUT>
__device__ __forceinline__ OUT to_out(float x)
{
    if constexpr (sizeof(OUT) == 2) return f16_of_f32(x);
    else return x;
}

// One wave's dot product x . g over K elements (K % 8 == 0, both 16-byte aligned), in one fixed
// order: lane l sums the 8-element pieces l, l + 64, ... with fmaf, then a butterfly over the 64
// lanes. Every kernel that computes a gate calls this, so they agree bitwise. All lanes get the sum.
__device__ __forceinline__ float wave_dot_f16(const f16 *x, const f16 *g, int K)
{
    const int lane = threadIdx.x & 63, pieces = K >> 3;
    float z = 0.0f;
#pragma unroll 4
    for (int pc = lane; pc < pieces; pc += 64) {
        const f16x8 a = *reinterpret_cast<const f16x8 *>(x + 8 * pc);
        const f16x8 b = *reinterpret_cast<const f16x8 *>(g + 8 * pc);
#pragma unroll
        for (int e = 0; e < 8; ++e) z = fmaf((float)a[e], (float)b[e], z);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
    return __shfl(z, 0, 64);
}

// wave_dot_f16 for K <= 2048 in two halves, the same sum bitwise: wave_dot_load issues the lane's
// (at most four) pieces, wave_dot_sum adds them once they are needed, so other work can hide the
// loads' latency.
struct WaveDotRegs {
    f16x8 a[4], b[4];
};
__device__ __forceinline__ void wave_dot_load(WaveDotRegs &r, const f16 *x, const f16 *g, int K)
{
    const int lane = threadIdx.x & 63, pieces = K >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pc = lane + 64 * i;
        if (pc < pieces) {
            r.a[i] = *reinterpret_cast<const f16x8 *>(x + 8 * pc);
            r.b[i] = *reinterpret_cast<const f16x8 *>(g + 8 * pc);
        }
    }
}
__device__ __forceinline__ float wave_dot_sum(const WaveDotRegs &r, int K)
{
    const int lane = threadIdx.x & 63, pieces = K >> 3;
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < pieces) {
#pragma unroll
            for (int e = 0; e < 8; ++e) z = fmaf((float)r.a[i][e], (float)r.b[i][e], z);
        }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o, 64);
    return __shfl(z, 0, 64);
}

}  // namespace nvfp4
