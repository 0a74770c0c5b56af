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
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

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

// ---- the 16-block format: E2M1 codes, one E4M3 scale per 16 values --------
// An E4M3 scale byte b (sign bit 7, exponent bits 6..3 bias 7, mantissa bits
// 2..0; exponent 0 subnormal) as a power of two p and a factor m with
// scale = p * m: p = 2^(E-7), m = 1 + M/8 for E > 0; p = 2^-9, m = M for
// E = 0; the sign goes into m.  The scaled convert applies only the exponent
// of its fp32 scale operand (measured on gfx950), so p goes there and m is
// one packed fp16 multiply.  code * p is an fp16 normal (2^-10 .. 1536) and
// code * p * m has at most 6 significant bits (<= 2880): both exact in fp16.
// Exponent 15 with mantissa 7 (NaN in the format) is undefined input.
struct E4m3Parts {
    float p;
    f16x2_t m;
};
__device__ __forceinline__ E4m3Parts e4m3_parts(uint32_t b)
{
    const uint32_t e = (b >> 3) & 15u, mt = b & 7u;
    E4m3Parts r;
    r.p = __uint_as_float((e ? e + 120u : 118u) << 23);
    float m = e ? 1.0f + 0.125f * (float)mt : (float)mt;
    m = (b & 0x80u) ? -m : m;
    const _Float16 mh = (_Float16)m;  // exact: at most 4 significant bits
    r.m = f16x2_t{mh, mh};
    return r;
}

// Eight codes (one dword, element 2b in the low nibble of byte b) of one
// 16-block -> eight fp16 in element order, code * scale exactly.
__device__ __forceinline__ f16x8_t fp4x8_to_f16(uint32_t codes, const E4m3Parts &s)
{
    const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, s.p, 0) * s.m;
    const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, s.p, 1) * s.m;
    const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, s.p, 2) * s.m;
    const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, s.p, 3) * s.m;
    return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ f16x8_t as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8_t, v); }

// 16x16x32 fp16 MFMA, fp32 accumulate; operand layout as mfma16.
__device__ __forceinline__ floatx4_t mfma16h(f16x8_t a, f16x8_t b, floatx4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---- cross-lane reductions on DPP (no LDS round trips) --------------------
// DPP controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140.  After these four steps every
// lane holds the reduction over its row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float readlane_f(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 16 lanes that share l/16; every lane of the row gets it.
__device__ __forceinline__ float sum16(float v)
{
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return v;
}

// Sum over the wave (rows added in a fixed order); every lane gets it.
__device__ __forceinline__ float wave_sum(float v)
{
    v = sum16(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// Streaming loads of weight bytes: each is read once per layer call, so they
// are marked non-temporal (no reuse expected in the caches).
typedef unsigned int v4u_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void *p)
{
    const v4u_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_nt_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream4(const uint32_t *p) { return __builtin_nontemporal_load(p); }

// Contiguous per-XCD tile ranges (workgroup w runs on XCD w % 8, so
// neighbouring tiles -- same rows, same expert -- share that XCD's L2);
// returns false for surplus workgroups.
__device__ __forceinline__ bool xcd_tile(int total, int &idx)
{
    const int per = (total + 7) >> 3;
    const int local = (int)(blockIdx.x >> 3);
    if (local >= per) return false;
    idx = (int)(blockIdx.x & 7) * per + local;
    return idx < total;
}

// LDS byte offset of a __shared__ object.
__device__ __forceinline__ uint32_t lds_off(const void *p)
{
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// Direct-to-LDS loads.  Issued from inline asm so the compiler does not
// guard later LDS reads with a blanket vmcnt(0) (it cannot tell the ring
// stages apart); every wait on these loads is the explicit one in
// the kernel.  lds (wave-uniform) is the byte offset the lane-0 data lands
// at; lane i's data lands at lds + i*size.  The load takes its LDS base from
// M0, which the compiler reserves: its value is saved in an SGPR and put
// back inside the same statement, so M0 is unchanged across it.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(g) : "memory");
}
__device__ __forceinline__ void dma4(const void *g, uint32_t lds)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "global_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(g) : "memory");
}


// ---- exact split of bf16 into two FP8 E4M3 parts --------------------------
// For a block of 32 bf16 values with largest magnitude M = 2^E * 1.f:
//   hi = RNE_e4m3(v / 2^sh), sh = E - 7 (|v / 2^sh| < 256 <= 448, no clipping)
//   lo = RNE_e4m3((v - hi * 2^sh) / 2^sl), sl = sh - 5
// bf16 keeps 8 significant bits and hi keeps the top 4 (rounded), so the
// residual has at most 4 significant bits: v == hi*2^sh + lo*2^sl exactly
// whenever |v| >= 2^(E-14) (lower values keep an error below 2^(E-22)).
// Scales are returned as E8M0 bytes (exponent + 127).
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

__device__ __forceinline__ void split_e4m3_block(const float *v, uint32_t *hi, uint32_t *lo,
                                                 uint32_t &shi, uint32_t &slo)
{
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int E = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;  // amax == 0 or subnormal: clamp below
    int sh = E - 7;
    if (sh < -120) sh = -120;
    const int sl = sh - 5;
    const float ih = pow2f(-sh), il = pow2f(-sl), fh = pow2f(sh);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        int ph = 0, pl = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const float a = v[4 * w + 2 * half], b = v[4 * w + 2 * half + 1];
            const int h2 = __builtin_amdgcn_cvt_pk_fp8_f32(a * ih, b * ih, 0, false);
            const float ra = a - __builtin_amdgcn_cvt_f32_fp8(h2, 0) * fh;
            const float rb = b - __builtin_amdgcn_cvt_f32_fp8(h2, 1) * fh;
            const int l2 = __builtin_amdgcn_cvt_pk_fp8_f32(ra * il, rb * il, 0, false);
            ph |= (h2 & 0xFFFF) << (16 * half);
            pl |= (l2 & 0xFFFF) << (16 * half);
        }
        hi[w] = (uint32_t)ph;
        lo[w] = (uint32_t)pl;
    }
    shi = (uint32_t)(sh + 127);
    slo = (uint32_t)(sl + 127);
}

// ---- three-part FP6 split of a 32-value block -------------------------------
// Each part is FP6 E2M3 (sign, 2 exponent bits, 3 mantissa bits; magnitudes
// 0 .. 7.5, steps of 1/8 below 2, 1/4 below 4, 1/2 up to 7.5) with its own
// E8M0 scale, taken from the block's largest remaining magnitude R = 2^e*1.f:
//   s = e - 2, or e - 1 when R / 2^(e-2) >= 7.75 (rounding would reach 8);
//   part = RNE_e2m3(r / 2^s), r <- r - part * 2^s.
// No part saturates, and each part's rounding error is at most 2^(s-2), so
// the scales fall by at least 4 per part and the three-part error is at most
// 2^(E-11), E the exponent of the block maximum.  In practice far less: a
// part holds the top 4 significant bits of every value within three binades
// of R, so bf16 values near the block maximum are exact after two parts and
// nearly all after three (largest error seen on Gaussian, heavy-tailed and
// outlier blocks: 2^-15 of the block maximum).  The hardware's scaled conversions do
// the rounding (round to nearest even, verified on gfx950) and the inverse
// (cvt_f32x32_to_e2m3, cvt_e2m3_to_f32x32 below);
// the 2x16 form places element i of its first operand at code 2i and of its
// second at code 2i+1, so the even and odd elements are passed apart to get
// the natural order (code j in bits 6j .. 6j+5, the MFMA operand layout).
typedef int v6i_t __attribute__((__vector_size__(6 * sizeof(int))));
typedef float v16f_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef float v32f_t __attribute__((__vector_size__(32 * sizeof(float))));

// The two conversions are issued from inline asm with early-clobber outputs.
// Through the compiler builtins the register allocator may give the result
// registers an overlap with an input operand; on gfx950 that gave results
// that changed from run to run (measured: about 1e-4 of the third parts of a
// 160 MB split differed between two identical calls).  Here the result
// registers never overlap the inputs.
__device__ __forceinline__ v6i_t cvt_f32x32_to_e2m3(const v16f_t &even, const v16f_t &odd, float scale)
{
    v6i_t r;
    asm volatile("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3"
                 : "=&v"(r) : "v"(even), "v"(odd), "v"(scale));
    return r;
}
__device__ __forceinline__ v32f_t cvt_e2m3_to_f32x32(const v6i_t &codes, float scale)
{
    v32f_t r;
    asm volatile("v_cvt_scalef32_pk32_f32_fp6 %0, %1, %2" : "=&v"(r) : "v"(codes), "v"(scale));
    return r;
}

__device__ __forceinline__ void split_e2m3x3_block(float (&r)[32], uint32_t (&code)[3][6],
                                                   uint32_t (&sc)[3])
{
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(r[i]));
        int s = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 2;
        if (amax >= 7.75f * pow2f(s < -126 ? -126 : s)) ++s;
        s = s < -126 ? -126 : s;  // zero or tiny blocks: the smallest normal scale
        const float scale = pow2f(s);
        v16f_t ev, od;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            ev[i] = r[2 * i];
            od[i] = r[2 * i + 1];
        }
        const v6i_t c = cvt_f32x32_to_e2m3(ev, od, scale);
        const v32f_t q = cvt_e2m3_to_f32x32(c, scale);
#pragma unroll
        for (int i = 0; i < 32; ++i) r[i] -= q[i];
#pragma unroll
        for (int w = 0; w < 6; ++w) code[p][w] = (uint32_t)c[w];
        sc[p] = (uint32_t)(s + 127);
    }
}

// One 32-element bf16 block -> FP8 E4M3 hi and lo parts (32 bytes each) and
// their E8M0 scales (split_e4m3_block).
__device__ __forceinline__ void split_bf16_block(const uint16_t *src, uint8_t *hi, uint8_t *lo,
                                                 uint8_t *shi, uint8_t *slo)
{
    const uint4 *p = reinterpret_cast<const uint4 *>(src);
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 w = p[q];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * q + 2 * i] = __uint_as_float(ws[i] << 16);
            v[8 * q + 2 * i + 1] = __uint_as_float(ws[i] & 0xFFFF0000u);
        }
    }
    uint32_t h[8], l[8], sh, sl;
    split_e4m3_block(v, h, l, sh, sl);
    uint4 *ph = reinterpret_cast<uint4 *>(hi);
    uint4 *pl = reinterpret_cast<uint4 *>(lo);
    ph[0] = make_uint4(h[0], h[1], h[2], h[3]);
    ph[1] = make_uint4(h[4], h[5], h[6], h[7]);
    pl[0] = make_uint4(l[0], l[1], l[2], l[3]);
    pl[1] = make_uint4(l[4], l[5], l[6], l[7]);
    *shi = (uint8_t)sh;
    *slo = (uint8_t)sl;
}

}  // namespace moe
