// latent.hip -- the two shared-matrix products and the gate of the
// latent-width variant.
//
// "Muse Spark Open を段階的に分解する" (animemo.app), section ⑨: a matrix
// shared by the chosen experts narrows the token before them, a second one
// widens their weighted sum after them; section ③: the widened sum joins
// the residual through the per-dimension gate s <- alpha*s + beta*(.).
//
// The products are plain dense GEMMs (bf16 operands, fp32 accumulation) and
// run in rocBLAS; the gate is an elementwise pass here.
#include <mutex>

#include <rocblas/rocblas.h>

#include "device.h"
#include "internal.h"

namespace moe {

// One rocBLAS handle per device, created at first use and kept until the
// process ends.  The stream is set under the lock for each call, so calls
// from several threads cannot interleave a stream change with a launch.
static std::mutex g_blas_mu;
static rocblas_handle g_blas[64];

hipError_t launch_dense(const uint16_t *a, const uint16_t *w, void *c, bool c_fp32, int T, int N,
                        int K, hipStream_t st)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_blas_mu);
    if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
        g_blas[dev] = nullptr;
        return hipErrorUnknown;
    }
    rocblas_handle h = g_blas[dev];
    if (rocblas_set_stream(h, st) != rocblas_status_success) return hipErrorUnknown;
    // column-major view: C^T [N][T] = W [N][K] (stored K-major, so op = T) x A^T [K][T]
    const float one = 1.0f, zero = 0.0f;
    const rocblas_datatype ct = c_fp32 ? rocblas_datatype_f32_r : rocblas_datatype_bf16_r;
    const rocblas_status r = rocblas_gemm_ex(
        h, rocblas_operation_transpose, rocblas_operation_none, N, T, K, &one, w,
        rocblas_datatype_bf16_r, K, a, rocblas_datatype_bf16_r, K, &zero, c, ct, N, c, ct, N,
        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    return r == rocblas_status_success ? hipSuccess : hipErrorUnknown;
}

// 8 columns per thread: x (16 B), f (32 B), alpha, beta (32 B each) in,
// 16 B out.
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t *x, const float *__restrict__ f,
                                                   const float *__restrict__ alpha,
                                                   const float *__restrict__ beta, uint16_t *s_out,
                                                   int64_t n8, int D)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= n8) return;
    const int c0 = (int)((q * 8) % D);
    const uint4 xv = reinterpret_cast<const uint4 *>(x)[q];
    const float4 f0 = reinterpret_cast<const float4 *>(f)[2 * q];
    const float4 f1 = reinterpret_cast<const float4 *>(f)[2 * q + 1];
    const float4 a0 = *reinterpret_cast<const float4 *>(alpha + c0);
    const float4 a1 = *reinterpret_cast<const float4 *>(alpha + c0 + 4);
    const float4 b0 = *reinterpret_cast<const float4 *>(beta + c0);
    const float4 b1 = *reinterpret_cast<const float4 *>(beta + c0 + 4);
    const float fv[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
    uint32_t ow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float s0 = fmaf(bv[2 * i], fv[2 * i], av[2 * i] * __uint_as_float(xw[i] << 16));
        const float s1 = fmaf(bv[2 * i + 1], fv[2 * i + 1], av[2 * i + 1] * __uint_as_float(xw[i] & 0xFFFF0000u));
        ow[i] = (uint32_t)f32_to_bf16(s0) | (uint32_t)f32_to_bf16(s1) << 16;
    }
    reinterpret_cast<uint4 *>(s_out)[q] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
}

hipError_t launch_gate(const uint16_t *x, const float *f, const float *alpha, const float *beta,
                       uint16_t *s_out, int64_t T, int D, hipStream_t st)
{
    const int64_t n8 = T * D / 8;
    gate_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(x, f, alpha, beta, s_out, n8, D);
    return hipGetLastError();
}

}  // namespace moe
