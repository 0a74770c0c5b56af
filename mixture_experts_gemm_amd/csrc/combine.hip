// combine.hip -- per-expert RMSNorm, router-weighted sum and gated residual.
//
// "Muse Spark Open を段階的に分解する" (animemo.app):
//   section ⑨  every chosen expert's output is normalised, then weighted by
//              the router score and summed (RMSNorm over d, eps inside the
//              square root, no learned gain);
//   section ③  the result is mixed into the residual stream through a gate
//              with per-dimension alpha and beta: s <- alpha*s + beta*y.
//
// One workgroup per (token, 2048-column chunk).  The k slot rows of o are
// either stored in slot order (few-row path) or found through inv (tiled
// path); their sums of squares come from the partials written by the
// down-projection kernel, added in a fixed order.  s_out may be x
// itself: each thread reads its x elements before writing the same elements.
#include "device.h"
#include "internal.h"

namespace moe {

constexpr int kMaxK = 64;          // slots handled per pass over the row
constexpr int kSlotBatch = 8;       // slots per pass when o is in slot order
constexpr int kCombineCols = 2048;  // columns per workgroup (8 per thread)

// SLOT: o and the o^2 partial sums are stored in slot order (row t*k + j is
// slot j of token t); otherwise in the grouped order, found through inv.
// o is read once, by non-temporal loads, so it does not displace the x,
// alpha and beta slices the workgroups share in L2 (prefill combine
// 135.5 -> 124.2 us).
// OUT: kOutGate s_out = bf16(alpha * x + beta * y); kOutBf16 s_out = bf16(y)
// (the latent-width variant widens y before its gate); kOutF32 y_out = y
// (the block variant normalises y before its gate).
enum { kOutGate = 0, kOutBf16 = 1, kOutF32 = 2 };
template <bool SLOT, int OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SLOT ? 1 : 8))) void combine_kernel(
    const uint16_t *x, const float *__restrict__ wts, const int32_t *__restrict__ inv,
    const uint16_t *__restrict__ o, const float *__restrict__ ssq, const float *__restrict__ alpha,
    const float *__restrict__ beta, uint16_t *s_out, float *y_out, int d, int k, int P, float eps)
{
    constexpr bool GATE = OUT == kOutGate;
    constexpr int JB = SLOT ? kSlotBatch : kMaxK;  // slots per pass over the row
    __shared__ float coef[JB];
    __shared__ int32_t row[JB];
    const int t = blockIdx.x;
    const int c0 = blockIdx.y * kCombineCols + threadIdx.x * 8;  // 8 columns per thread
    const bool act = c0 < d;
    // independent loads first
    uint4 xv = make_uint4(0, 0, 0, 0);
    float4 a0 = make_float4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
    if (GATE && act) {
        xv = *reinterpret_cast<const uint4 *>(x + (int64_t)t * d + c0);
        a0 = *reinterpret_cast<const float4 *>(alpha + c0);
        a1 = *reinterpret_cast<const float4 *>(alpha + c0 + 4);
        b0 = *reinterpret_cast<const float4 *>(beta + c0);
        b1 = *reinterpret_cast<const float4 *>(beta + c0 + 4);
    }
    float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto accumulate = [&](const uint4 &ov, float cj) {
        const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[2 * i] = fmaf(cj, __uint_as_float(ow[i] << 16), y[2 * i]);
            y[2 * i + 1] = fmaf(cj, __uint_as_float(ow[i] & 0xFFFF0000u), y[2 * i + 1]);
        }
    };
    if (SLOT && k <= kSlotBatch) {
        // few-row path, one pass: the o rows and every norm partial go out
        // together with x, alpha, beta, so the workgroup waits on memory once
        uint4 ov[kSlotBatch];
#pragma unroll
        for (int j = 0; j < kSlotBatch; ++j)
            ov[j] = act && j < k ? ld_stream16(o + ((int64_t)t * k + j) * d + c0)
                                 : make_uint4(0, 0, 0, 0);
        // 16 lanes per slot; lane l of slot j adds partials l, l+16, ... in
        // that order (loads at a clamped index, masked after, so they are
        // all issued before the first add)
        const int j = threadIdx.x >> 4, l = threadIdx.x & 15;
        const bool js = j < k;
        const float *sp = ssq + ((int64_t)t * k + (js ? j : 0)) * P;
        float ss = 0.f;
        for (int q0 = 0; q0 < P; q0 += 128) {
            float pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pv[i] = sp[min(q0 + 16 * i + l, P - 1)];
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += q0 + 16 * i + l < P ? pv[i] : 0.f;
        }
        ss = sum16(ss);
        if (js && l == 0) coef[j] = wts[(int64_t)t * k + j] * (1.0f / sqrtf(ss / (float)d + eps));
        __syncthreads();
        if (act) {
#pragma unroll
            for (int jj = 0; jj < kSlotBatch; ++jj)
                if (jj < k) accumulate(ov[jj], coef[jj]);
        }
    } else
    for (int j0 = 0; j0 < k; j0 += JB) {
        const int kk = min(JB, k - j0);
        // slot order: the pass's o values go out together with the norms' loads
        uint4 ov[SLOT ? kSlotBatch : 1];
        if constexpr (SLOT) {
#pragma unroll
            for (int j = 0; j < kSlotBatch; ++j)
                ov[j] = act && j < kk ? ld_stream16(o + ((int64_t)t * k + j0 + j) * d + c0)
                                      : make_uint4(0, 0, 0, 0);
        }
        __syncthreads();
        // 16 lanes per slot: 16 slots per pass of the workgroup
        for (int j = (threadIdx.x >> 4); j < kk; j += 16) {
            const int64_t slot = (int64_t)t * k + j0 + j;
            const int p = SLOT ? (int)slot : inv[slot];
            const float wj = wts[slot];  // loaded beside inv, not after the sums
            // lane l adds partials l, l+16, ... in that order; eight loads
            // go out at a time (clamped index, masked after)
            const int l = threadIdx.x & 15;
            float ss = 0.f;
            const float *sp = ssq + (int64_t)p * P;
            for (int q0 = 0; q0 < P; q0 += 128) {
                float pv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) pv[i] = sp[min(q0 + 16 * i + l, P - 1)];
#pragma unroll
                for (int i = 0; i < 8; ++i) ss += q0 + 16 * i + l < P ? pv[i] : 0.f;
            }
            ss = sum16(ss);
            if (l == 0) {
                row[j] = p;
                coef[j] = wj * (1.0f / sqrtf(ss / (float)d + eps));
            }
        }
        __syncthreads();
        if (act) {
            if constexpr (SLOT) {
#pragma unroll
                for (int j = 0; j < kSlotBatch; ++j)
                    if (j < kk) accumulate(ov[j], coef[j]);
            } else {
                for (int j = 0; j < kk; ++j)
                    accumulate(ld_stream16(o + (int64_t)row[j] * d + c0), coef[j]);
            }
        }
    }
    if (OUT == kOutF32 && act) {
        float4 *yo = reinterpret_cast<float4 *>(y_out + (int64_t)t * d + c0);
        yo[0] = make_float4(y[0], y[1], y[2], y[3]);
        yo[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
    if (OUT == kOutBf16 && act) {
        uint32_t ow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ow[i] = (uint32_t)f32_to_bf16(y[2 * i]) | (uint32_t)f32_to_bf16(y[2 * i + 1]) << 16;
        *reinterpret_cast<uint4 *>(s_out + (int64_t)t * d + c0) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
    if (GATE && act) {
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        uint32_t ow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s0 = fmaf(bv[2 * i], y[2 * i], av[2 * i] * __uint_as_float(xw[i] << 16));
            const float s1 = fmaf(bv[2 * i + 1], y[2 * i + 1], av[2 * i + 1] * __uint_as_float(xw[i] & 0xFFFF0000u));
            ow[i] = (uint32_t)f32_to_bf16(s0) | (uint32_t)f32_to_bf16(s1) << 16;
        }
        *reinterpret_cast<uint4 *>(s_out + (int64_t)t * d + c0) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
}

template <int OUT>
static hipError_t combine_launch(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                                 const float *alpha, const float *beta, uint16_t *s_out, float *y_out,
                                 hipStream_t st)
{
    dim3 grid(s.T, (s.d + kCombineCols - 1) / kCombineCols);
    // the few-row down kernel stores in slot order, the tiled ones in the grouped order
    if (p.tiled)
        combine_kernel<false, OUT><<<grid, 256, 0, st>>>(x, ws.wts, ws.inv, ws.o, ws.ssq, alpha, beta,
                                                         s_out, y_out, s.d, s.k, s.d / p.ssq_cols, s.eps);
    else
        combine_kernel<true, OUT><<<grid, 256, 0, st>>>(x, ws.wts, ws.inv, ws.o, ws.ssq, alpha, beta,
                                                        s_out, y_out, s.d, s.k, s.d / p.ssq_cols, s.eps);
    return hipGetLastError();
}

hipError_t launch_combine(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                          const float *alpha, const float *beta, uint16_t *s_out, hipStream_t st)
{
    return combine_launch<kOutGate>(s, p, ws, x, alpha, beta, s_out, nullptr, st);
}

hipError_t launch_combine_sum(const Shape &s, const Plan &p, const Workspace &ws, uint16_t *y,
                              hipStream_t st)
{
    return combine_launch<kOutBf16>(s, p, ws, nullptr, nullptr, nullptr, y, nullptr, st);
}

hipError_t launch_combine_sum_f32(const Shape &s, const Plan &p, const Workspace &ws, float *y,
                                  hipStream_t st)
{
    return combine_launch<kOutF32>(s, p, ws, nullptr, nullptr, nullptr, nullptr, y, st);
}

// ---- the block's stream norms ([MS] section ③) --------------------------------
// One workgroup per token row: the row's sum of squares in a fixed order
// (per-thread partials, wave sums, then the four waves in order), so the
// result does not depend on scheduling.
__device__ __forceinline__ float block_row_sumsq(float part)
{
    __shared__ float wsq[4];
    const float v = wave_sum(part);
    if ((threadIdx.x & 63) == 0) wsq[threadIdx.x >> 6] = v;
    __syncthreads();
    return (wsq[0] + wsq[1]) + (wsq[2] + wsq[3]);
}

// x_n = bf16(x * r * gamma), r = 1 / sqrt(mean(x^2) + eps); 8 columns per
// thread and pass.
__global__ __launch_bounds__(256) void prenorm_kernel(const uint16_t *__restrict__ x,
                                                      const float *__restrict__ gamma,
                                                      uint16_t *__restrict__ xn, int d, float eps)
{
    const int t = blockIdx.x;
    const uint4 *row = reinterpret_cast<const uint4 *>(x + (int64_t)t * d);
    float part = 0.f;
    for (int c = threadIdx.x; c < d / 8; c += 256) {
        const uint4 v = row[c];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = __uint_as_float(w[i] << 16), b = __uint_as_float(w[i] & 0xFFFF0000u);
            part = fmaf(a, a, part);
            part = fmaf(b, b, part);
        }
    }
    const float r = 1.0f / sqrtf(block_row_sumsq(part) / (float)d + eps);
    uint4 *out = reinterpret_cast<uint4 *>(xn + (int64_t)t * d);
    for (int c = threadIdx.x; c < d / 8; c += 256) {
        const uint4 v = row[c];
        const float4 g0 = *reinterpret_cast<const float4 *>(gamma + 8 * c);
        const float4 g1 = *reinterpret_cast<const float4 *>(gamma + 8 * c + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t ow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = __uint_as_float(w[i] << 16) * r * gv[2 * i];
            const float b = __uint_as_float(w[i] & 0xFFFF0000u) * r * gv[2 * i + 1];
            ow[i] = (uint32_t)f32_to_bf16(a) | (uint32_t)f32_to_bf16(b) << 16;
        }
        out[c] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
}

// s_out = bf16(alpha * x + beta * y * r * gamma), r = 1 / sqrt(mean(y^2) + eps).
// s_out may be x: each thread reads its x elements before writing them.
__global__ __launch_bounds__(256) void postnorm_gate_kernel(
    const uint16_t *x, const float *__restrict__ y, const float *__restrict__ gamma,
    const float *__restrict__ alpha, const float *__restrict__ beta, uint16_t *s_out, int d, float eps)
{
    const int t = blockIdx.x;
    const float4 *yr = reinterpret_cast<const float4 *>(y + (int64_t)t * d);
    float part = 0.f;
    for (int c = threadIdx.x; c < d / 4; c += 256) {
        const float4 v = yr[c];
        part = fmaf(v.x, v.x, part);
        part = fmaf(v.y, v.y, part);
        part = fmaf(v.z, v.z, part);
        part = fmaf(v.w, v.w, part);
    }
    const float r = 1.0f / sqrtf(block_row_sumsq(part) / (float)d + eps);
    const uint2 *xr = reinterpret_cast<const uint2 *>(x + (int64_t)t * d);
    uint2 *out = reinterpret_cast<uint2 *>(s_out + (int64_t)t * d);
    for (int c = threadIdx.x; c < d / 4; c += 256) {
        const float4 v = yr[c];
        const uint2 xv = xr[c];
        const float4 g = *reinterpret_cast<const float4 *>(gamma + 4 * c);
        const float4 a = *reinterpret_cast<const float4 *>(alpha + 4 * c);
        const float4 b = *reinterpret_cast<const float4 *>(beta + 4 * c);
        const float s0 = fmaf(b.x, v.x * r * g.x, a.x * __uint_as_float(xv.x << 16));
        const float s1 = fmaf(b.y, v.y * r * g.y, a.y * __uint_as_float(xv.x & 0xFFFF0000u));
        const float s2 = fmaf(b.z, v.z * r * g.z, a.z * __uint_as_float(xv.y << 16));
        const float s3 = fmaf(b.w, v.w * r * g.w, a.w * __uint_as_float(xv.y & 0xFFFF0000u));
        out[c] = make_uint2((uint32_t)f32_to_bf16(s0) | (uint32_t)f32_to_bf16(s1) << 16,
                            (uint32_t)f32_to_bf16(s2) | (uint32_t)f32_to_bf16(s3) << 16);
    }
}

// The block's combine and post-norm in one pass, for rows of at most
// kBlockFusedMaxD columns and at most kBlockFusedMaxK slots: one workgroup
// of NT threads per token row (256 for many rows; 1024 for few, so a row
// of up to 8192 columns is one pass).  Every slot's
// coefficient w / sqrt(mean(o^2) + eps) first (as combine_kernel), then y =
// sum over the slots of coef * o in slot order (the same sums as
// combine_kernel's), kept in registers, 8 columns per thread and pass; the
// row's sum of squares of y in a fixed order (block_row_sumsq); then
// s_out = bf16(alpha * x + beta * y * r * gamma).  s_out may be x: each
// thread reads its x elements before writing them.
constexpr int kBlockPasses = 8;
static_assert(kBlockPasses * 2048 == kBlockFusedMaxD, "a pass of 256 threads is 2048 columns");

// the row's sum of squares over NW waves in a fixed order
template <int NW>
__device__ __forceinline__ float block_row_sumsq_n(float part)
{
    __shared__ float wsq[NW];
    const float v = wave_sum(part);
    if ((threadIdx.x & 63) == 0) wsq[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += wsq[w];
    return s;
}

template <bool SLOT, int NT>
__global__ __launch_bounds__(NT) void combine_postnorm_kernel(
    const uint16_t *x, const float *__restrict__ wts, const int32_t *__restrict__ inv,
    const uint16_t *__restrict__ o, const float *__restrict__ ssq, const float *__restrict__ gamma,
    const float *__restrict__ alpha, const float *__restrict__ beta, uint16_t *s_out, int d, int k, int P,
    float eps)
{
    __shared__ float coef[kBlockFusedMaxK];
    __shared__ int32_t row[kBlockFusedMaxK];
    const int t = blockIdx.x;
    for (int j = threadIdx.x >> 4; j < k; j += NT / 16) {
        const int64_t slot = (int64_t)t * k + j;
        const int p = SLOT ? (int)slot : inv[slot];
        const float wj = wts[slot];
        // lane l adds partials l, l+16, ... in that order, eight loads at a time
        const int l = threadIdx.x & 15;
        float ss = 0.f;
        const float *sp = ssq + (int64_t)p * P;
        for (int q0 = 0; q0 < P; q0 += 128) {
            float pv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pv[i] = sp[min(q0 + 16 * i + l, P - 1)];
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += q0 + 16 * i + l < P ? pv[i] : 0.f;
        }
        ss = sum16(ss);
        if (l == 0) {
            row[j] = p;
            coef[j] = wj * (1.0f / sqrtf(ss / (float)d + eps));
        }
    }
    __syncthreads();
    constexpr int NP = kBlockFusedMaxD / (NT * 8);  // passes
    float y[NP][8];
    float part = 0.f;
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
#pragma unroll
        for (int i = 0; i < 8; ++i) y[ps][i] = 0.f;
        const int c0 = ps * NT * 8 + threadIdx.x * 8;
        if (c0 >= d) continue;
        for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
            // up to kSlotBatch o rows in flight at once (clamped index, masked)
            uint4 ov[kSlotBatch];
#pragma unroll
            for (int jj = 0; jj < kSlotBatch; ++jj)
                ov[jj] = ld_stream16(o + (int64_t)row[min(j0 + jj, k - 1)] * d + c0);
#pragma unroll
            for (int jj = 0; jj < kSlotBatch; ++jj) {
                if (j0 + jj >= k) break;
                const float cj = coef[j0 + jj];
                const uint32_t ow[4] = {ov[jj].x, ov[jj].y, ov[jj].z, ov[jj].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    y[ps][2 * i] = fmaf(cj, __uint_as_float(ow[i] << 16), y[ps][2 * i]);
                    y[ps][2 * i + 1] = fmaf(cj, __uint_as_float(ow[i] & 0xFFFF0000u), y[ps][2 * i + 1]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) part = fmaf(y[ps][i], y[ps][i], part);
    }
    const float r = 1.0f / sqrtf(block_row_sumsq_n<NT / 64>(part) / (float)d + eps);
#pragma unroll
    for (int ps = 0; ps < NP; ++ps) {
        const int c0 = ps * NT * 8 + threadIdx.x * 8;
        if (c0 >= d) continue;
        const uint4 xv = *reinterpret_cast<const uint4 *>(x + (int64_t)t * d + c0);
        const float4 g0 = *reinterpret_cast<const float4 *>(gamma + c0), g1 = *reinterpret_cast<const float4 *>(gamma + c0 + 4);
        const float4 a0 = *reinterpret_cast<const float4 *>(alpha + c0), a1 = *reinterpret_cast<const float4 *>(alpha + c0 + 4);
        const float4 b0 = *reinterpret_cast<const float4 *>(beta + c0), b1 = *reinterpret_cast<const float4 *>(beta + c0 + 4);
        const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
        uint32_t ow[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s0 = fmaf(bv[2 * i], y[ps][2 * i] * r * gv[2 * i], av[2 * i] * __uint_as_float(xw[i] << 16));
            const float s1 = fmaf(bv[2 * i + 1], y[ps][2 * i + 1] * r * gv[2 * i + 1],
                                  av[2 * i + 1] * __uint_as_float(xw[i] & 0xFFFF0000u));
            ow[i] = (uint32_t)f32_to_bf16(s0) | (uint32_t)f32_to_bf16(s1) << 16;
        }
        *reinterpret_cast<uint4 *>(s_out + (int64_t)t * d + c0) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    }
}

hipError_t launch_combine_postnorm(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                                   const float *gamma, const float *alpha, const float *beta,
                                   uint16_t *s_out, hipStream_t st)
{
    if (s.d > kBlockFusedMaxD || s.d % 8 != 0 || s.k > kBlockFusedMaxK) return hipErrorInvalidValue;
    // the few-row down kernel stores in slot order, the tiled ones in the grouped order
    if (p.tiled)
        combine_postnorm_kernel<false, 256><<<s.T, 256, 0, st>>>(x, ws.wts, ws.inv, ws.o, ws.ssq, gamma, alpha,
                                                                 beta, s_out, s.d, s.k, s.d / p.ssq_cols, s.eps);
    else
        combine_postnorm_kernel<true, 1024><<<s.T, 1024, 0, st>>>(x, ws.wts, ws.inv, ws.o, ws.ssq, gamma, alpha,
                                                                  beta, s_out, s.d, s.k, s.d / p.ssq_cols, s.eps);
    return hipGetLastError();
}

hipError_t launch_prenorm(const uint16_t *x, const float *gamma, uint16_t *xn, int T, int d, float eps,
                          hipStream_t st)
{
    prenorm_kernel<<<T, 256, 0, st>>>(x, gamma, xn, d, eps);
    return hipGetLastError();
}

hipError_t launch_postnorm_gate(const uint16_t *x, const float *y, const float *gamma,
                                const float *alpha, const float *beta, uint16_t *s_out, int T, int d,
                                float eps, hipStream_t st)
{
    postnorm_gate_kernel<<<T, 256, 0, st>>>(x, y, gamma, alpha, beta, s_out, d, eps);
    return hipGetLastError();
}

}  // namespace moe
