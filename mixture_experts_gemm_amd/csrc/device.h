// device.h -- gfx950 device helpers shared by the expert-layer kernels:
// bf16 rounding, the MXFP4 -> bf16 expansion on the hardware's scaled
// convert, the bf16 MFMA tile, and deterministic wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float floatx4_t __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest, ties to even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// E8M0 byte -> the fp32 power of two 2^(s-127) (s = 0 gives the fp32
// subnormal 2^-127; s = 255 is NaN in the format and undefined here).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s)
{
    return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Eight FP4 E2M1 codes (one dword, element 2b in the low nibble of byte b)
// times one block scale -> eight bf16 in element order.  The scaled convert
// multiplies by a power of two, so every value is exact in bf16.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t codes, float scale)
{
    bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    bf16x8_t r;
    r[0] = p0[0]; r[1] = p0[1];
    r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1];
    r[6] = p3[0]; r[7] = p3[1];
    return r;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 16x16x32 bf16 MFMA, fp32 accumulate.  Lane l supplies A[m = l%16][8 K
// values of k-group l/16] and B[same 8 K values][n = l%16]; the K order
// inside the instruction is irrelevant as long as A and B agree, which they
// do by construction.  Result: lane l holds C[(l/16)*4 + r][l%16], r = 0..3.
__device__ __forceinline__ floatx4_t mfma16(bf16x8_t a, bf16x8_t b, floatx4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Butterfly sum over the 16 lanes that share l/16 (fixed order, identical
// result in every lane of the group).
__device__ __forceinline__ float sum16(float v)
{
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace moe
