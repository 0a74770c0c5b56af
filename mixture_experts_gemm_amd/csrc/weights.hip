// weights.hip -- the expert-weight formats: natural MXFP4 rows -> the packed
// tile layout the layer reads (layout.h), and natural MXFP4 rows -> bf16.
//
// "Muse Spark Open を段階的に分解する" (animemo.app), section ⑪: the expert
// weights are 4-bit values (FP4 E2M1 here) sharing an 8-bit power-of-two
// scale (E8M0) per block of 32, expanded to BF16 for the multiply.
#include "device.h"
#include "internal.h"
#include "layout.h"

namespace moe {

// One thread per 16-byte unit of the packed codes.  The packed codes of an
// expert are linear in units: unit r of W1 is (tile r/1024, row (r%1024)/4,
// slot r%4), and W2 follows W1.  Each unit is one natural 32-element block.
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t *__restrict__ nat,
                                                         uint8_t *__restrict__ out, int64_t total,
                                                         int d, int F)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= total) return;
    const int64_t per_e = (int64_t)3 * d * F / 32;  // units per expert
    const int64_t e = u / per_e, r = u - e * per_e;
    const int64_t w1_units = (int64_t)d * F / 16;
    const int64_t r2 = r < w1_units ? r : r - w1_units;
    const int64_t t = r2 >> 10;
    const int rho = (int)((r2 >> 2) & 255), s = (int)(r2 & 3);
    const int blk = s ^ bswz(rho);
    const uint8_t *src = nat + e * ((int64_t)3 * d * F / 2);
    if (r < w1_units) {
        const int nk = d / kKStep;
        const int nt = (int)(t / nk), kc = (int)(t % nk);
        const int f = nt * 128 + (rho >> 7) * 64 + (rho & 63);
        const int64_t row = ((rho >> 6) & 1) ? (int64_t)F + f : (int64_t)f;
        src += row * (d / 2) + kc * 64 + blk * 16;
    } else {
        const int nk = F / kKStep;
        const int nt = (int)(t / nk), kc = (int)(t % nk);
        const int64_t row = (int64_t)nt * kWRows + rho;
        src += (int64_t)d * F + row * (F / 2) + kc * 64 + blk * 16;
    }
    reinterpret_cast<uint4 *>(out)[u] = *reinterpret_cast<const uint4 *>(src);
}

// One thread per 4-byte unit of the packed scales (the E8M0 bytes of one
// row's 4 blocks of one chunk).
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t *__restrict__ nat,
                                                          uint8_t *__restrict__ out, int64_t total,
                                                          int d, int F)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= total) return;
    const int64_t per_e = (int64_t)3 * d * F / 128;  // dwords per expert
    const int64_t e = u / per_e, r = u - e * per_e;
    const int64_t w1_units = (int64_t)d * F / 64;
    const int64_t r2 = r < w1_units ? r : r - w1_units;
    const int64_t t = r2 >> 8;
    const int rho = (int)(r2 & 255);
    const uint8_t *src = nat + e * ((int64_t)3 * d * F / 32);
    if (r < w1_units) {
        const int nk = d / kKStep;
        const int nt = (int)(t / nk), kc = (int)(t % nk);
        const int f = nt * 128 + (rho >> 7) * 64 + (rho & 63);
        const int64_t row = ((rho >> 6) & 1) ? (int64_t)F + f : (int64_t)f;
        src += row * (d / 32) + kc * 4;
    } else {
        const int nk = F / kKStep;
        const int nt = (int)(t / nk), kc = (int)(t % nk);
        const int64_t row = (int64_t)nt * kWRows + rho;
        src += (int64_t)d * F / 16 + row * (F / 32) + kc * 4;
    }
    reinterpret_cast<uint32_t *>(out)[u] = *reinterpret_cast<const uint32_t *>(src);
}

hipError_t launch_pack(const uint8_t *w, const uint8_t *s, int E, int d, int F, uint8_t *wp,
                       uint8_t *sp, hipStream_t st)
{
    const int64_t nc = (int64_t)E * 3 * d * F / 32, ns = (int64_t)E * 3 * d * F / 128;
    pack_codes_kernel<<<(unsigned)((nc + 255) / 256), 256, 0, st>>>(w, wp, nc, d, F);
    pack_scales_kernel<<<(unsigned)((ns + 255) / 256), 256, 0, st>>>(s, sp, ns, d, F);
    return hipGetLastError();
}

// The 16-block format's scales: one thread per 8-byte unit of the packed
// scale tiles (the E4M3 bytes of one row's eight 16-blocks of one chunk).
// The code bytes are packed by pack_codes_kernel, unchanged.
__global__ __launch_bounds__(256) void pack_scales16_kernel(const uint8_t *__restrict__ nat,
                                                            uint8_t *__restrict__ out, int64_t total,
                                                            int d, int F)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= total) return;
    const int64_t per_e = (int64_t)3 * d * F / 128;  // units per expert
    const int64_t e = u / per_e, r = u - e * per_e;
    const int64_t w1_units = (int64_t)d * F / 64;
    const int64_t r2 = r < w1_units ? r : r - w1_units;
    const int64_t t = r2 >> 8;
    const int rho = (int)(r2 & 255);
    const uint8_t *src = nat + e * ((int64_t)3 * d * F / 16);
    if (r < w1_units) {
        const int nk = d / kKStep;
        const int nt = (int)(t / nk), kc = (int)(t % nk);
        const int f = nt * 128 + (rho >> 7) * 64 + (rho & 63);
        const int64_t row = ((rho >> 6) & 1) ? (int64_t)F + f : (int64_t)f;
        src += row * (d / 16) + kc * 8;
    } else {
        const int nk = F / kKStep;
        const int nt = (int)(t / nk), kc = (int)(t % nk);
        const int64_t row = (int64_t)nt * kWRows + rho;
        src += (int64_t)d * F / 8 + row * (F / 16) + kc * 8;
    }
    reinterpret_cast<uint2 *>(out)[u] = *reinterpret_cast<const uint2 *>(src);
}

hipError_t launch_pack_nv(const uint8_t *w, const uint8_t *s16, int E, int d, int F, uint8_t *wp,
                          uint8_t *sp, hipStream_t st)
{
    const int64_t nc = (int64_t)E * 3 * d * F / 32, ns = (int64_t)E * 3 * d * F / 128;
    pack_codes_kernel<<<(unsigned)((nc + 255) / 256), 256, 0, st>>>(w, wp, nc, d, F);
    pack_scales16_kernel<<<(unsigned)((ns + 255) / 256), 256, 0, st>>>(s16, sp, ns, d, F);
    return hipGetLastError();
}

// MXFP4 rows -> bf16 rows with the conversion the few-row kernels use.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales,
                                                      int64_t n8, int K, uint4 *__restrict__ out)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // group of 8 elements
    if (q >= n8) return;
    const int64_t e = q * 8;
    const int64_t row = e / K, col = e % K;
    const uint32_t c = *reinterpret_cast<const uint32_t *>(codes + row * (K / 2) + col / 2);
    const float scale = e8m0_to_f32(scales[row * (K / 32) + col / 32]);
    out[q] = __builtin_bit_cast(uint4, fp4x8_to_bf16(c, scale));
}

hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int64_t rows, int K,
                          uint16_t *out, hipStream_t st)
{
    const int64_t n8 = rows * K / 8;
    dequant_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(codes, scales, n8, K,
                                                                 reinterpret_cast<uint4 *>(out));
    return hipGetLastError();
}

}  // namespace moe
