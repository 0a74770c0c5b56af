// combine.hip -- per-expert RMSNorm, router-weighted sum and gated residual.
//
// "Muse Spark Open を段階的に分解する" (animemo.app):
//   section ⑨  every chosen expert's output is normalised, then weighted by
//              the router score and summed (RMSNorm over d, eps inside the
//              square root, no learned gain);
//   section ③  the result is mixed into the residual stream through a gate
//              with per-dimension alpha and beta: s <- alpha*s + beta*y.
//
// One workgroup per (token, 1024-column chunk).  The k slot rows of o are
// found through inv; their sums of squares come from the partials written by
// the down-projection kernel, added in a fixed order.  s_out may be x
// itself: each thread reads its x elements before writing the same elements.
#include "device.h"
#include "internal.h"

namespace moe {

constexpr int kMaxK = 64;  // slots handled per pass over the row

__global__ __launch_bounds__(256) void combine_kernel(
    const uint16_t *x, const float *__restrict__ wts, const int32_t *__restrict__ inv,
    const uint16_t *__restrict__ o, const float *__restrict__ ssq, const float *__restrict__ alpha,
    const float *__restrict__ beta, uint16_t *s_out, int d, int k, int P, float eps)
{
    __shared__ float coef[kMaxK];
    __shared__ int32_t row[kMaxK];
    const int t = blockIdx.x;
    const int c0 = blockIdx.y * 1024 + threadIdx.x * 4;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const bool act = c0 < d;
    // independent loads first
    uint2 xv = make_uint2(0, 0);
    float4 a = make_float4(0, 0, 0, 0), b = a;
    if (act) {
        xv = *reinterpret_cast<const uint2 *>(x + (int64_t)t * d + c0);
        a = *reinterpret_cast<const float4 *>(alpha + c0);
        b = *reinterpret_cast<const float4 *>(beta + c0);
    }
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += kMaxK) {
        const int kk = min(kMaxK, k - j0);
        __syncthreads();
        // 16 lanes per slot: 16 slots per pass of the workgroup
        for (int j = (threadIdx.x >> 4); j < kk; j += 16) {
            const int64_t slot = (int64_t)t * k + j0 + j;
            const int p = inv[slot];
            float ss = 0.f;
            const float *sp = ssq + (int64_t)p * P;
#pragma unroll 4
            for (int q = (threadIdx.x & 15); q < P; q += 16) ss += sp[q];
            ss = sum16(ss);
            if ((threadIdx.x & 15) == 0) {
                row[j] = p;
                coef[j] = wts[slot] * (1.0f / sqrtf(ss / (float)d + eps));
            }
        }
        __syncthreads();
        if (act) {
            for (int j = 0; j < kk; ++j) {
                const uint2 ov = *reinterpret_cast<const uint2 *>(o + (int64_t)row[j] * d + c0);
                const float cj = coef[j];
                y[0] = fmaf(cj, __uint_as_float(ov.x << 16), y[0]);
                y[1] = fmaf(cj, __uint_as_float(ov.x & 0xFFFF0000u), y[1]);
                y[2] = fmaf(cj, __uint_as_float(ov.y << 16), y[2]);
                y[3] = fmaf(cj, __uint_as_float(ov.y & 0xFFFF0000u), y[3]);
            }
        }
    }
    (void)lane;
    (void)wv;
    if (act) {
        const float s0 = fmaf(b.x, y[0], a.x * __uint_as_float(xv.x << 16));
        const float s1 = fmaf(b.y, y[1], a.y * __uint_as_float(xv.x & 0xFFFF0000u));
        const float s2 = fmaf(b.z, y[2], a.z * __uint_as_float(xv.y << 16));
        const float s3 = fmaf(b.w, y[3], a.w * __uint_as_float(xv.y & 0xFFFF0000u));
        uint2 out;
        out.x = (uint32_t)f32_to_bf16(s0) | (uint32_t)f32_to_bf16(s1) << 16;
        out.y = (uint32_t)f32_to_bf16(s2) | (uint32_t)f32_to_bf16(s3) << 16;
        *reinterpret_cast<uint2 *>(s_out + (int64_t)t * d + c0) = out;
    }
}

hipError_t launch_combine(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                          const float *alpha, const float *beta, uint16_t *s_out, hipStream_t st)
{
    dim3 grid(s.T, (s.d + 1023) / 1024);
    combine_kernel<<<grid, 256, 0, st>>>(x, ws.wts, ws.inv, ws.o, ws.ssq, alpha, beta, s_out, s.d,
                                         s.k, s.d / p.ssq_cols, s.eps);
    return hipGetLastError();
}

}  // namespace moe
