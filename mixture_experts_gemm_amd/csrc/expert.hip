// expert.hip -- the grouped expert FFN on MXFP4 weights.
//
// "Muse Spark Open を段階的に分解する" (animemo.app):
//   section ⑨  each expert is a gate, an up and a down matrix; gate decides
//              what passes, up how much, down maps back to the token width
//              (here SwiGLU: h = silu(g) * u, o = h W_down^T);
//   section ⑪  the weights are 4-bit values sharing a small scale per block
//              and are expanded to BF16 for the multiply (here the gfx950
//              scaled convert expands FP4 E2M1 x E8M0 straight into bf16
//              MFMA operands, in registers, once per use);
//   section ⑬  at small token counts an expert's time is its weight read,
//              so these kernels keep many weight bytes in flight per CU.
//
// gemm1: for each tile of <= 16 grouped rows of one expert, h = silu(x Wg^T)
//        * (x Wu^T); the token rows are gathered through perm.
// gemm2: o = h Wd^T, plus per-row partial sums of o^2 over 16 columns (the
//        per-expert RMSNorm needs the whole row, finished in combine).
//
// Each wave owns a 16x16 output block over the whole K range: no LDS and no
// barriers; B (weights) is read once per tile, A (activations) comes from L2.
#include "device.h"
#include "internal.h"

namespace moe {

// K elements per loop step: each lane reads 16 bytes (32 FP4 values, one
// scale block) of one weight row and 64 bytes of one activation row.
constexpr int kKStep = 128;

__global__ __launch_bounds__(256) void gemm1_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ perm,
    const Tile *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    const uint8_t *__restrict__ wpk, const uint8_t *__restrict__ sc, uint16_t *__restrict__ h,
    int d, int F, int k, int groups)
{
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t tile = gw / groups;
    const int grp = (int)(gw % groups);
    if (tile >= *ntiles) return;
    const Tile tl = tiles[tile];
    const int n = lane & 15, g = lane >> 4;
    const int f0 = grp * 8;
    // columns 0..7: gate rows f0..f0+7, columns 8..15: up rows of the same features
    const int wrow = n < 8 ? f0 + n : F + f0 + (n - 8);
    const int64_t ebytes = (int64_t)3 * d * F / 2, escales = (int64_t)3 * d * F / 32;
    const uint8_t *bp = wpk + tl.expert * ebytes + (int64_t)wrow * (d / 2) + g * 16;
    const uint8_t *sp = sc + tl.expert * escales + (int64_t)wrow * (d / 32) + g;
    const bool valid = n < tl.nrows;  // A row m = lane & 15
    const int token = valid ? perm[tl.row0 + n] / k : 0;
    const uint16_t *ap = x + (int64_t)token * d + g * 32;

    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint4 bw = *reinterpret_cast<const uint4 *>(bp);
    uint32_t sb = sp[0];
    for (int k0 = 0; k0 < d; k0 += kKStep) {
        uint4 a[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            a[s] = valid ? *reinterpret_cast<const uint4 *>(ap + k0 + s * 8) : make_uint4(0, 0, 0, 0);
        const uint4 bcur = bw;
        const float scale = e8m0_to_f32(sb);
        if (k0 + kKStep < d) {
            bw = *reinterpret_cast<const uint4 *>(bp + (k0 + kKStep) / 2);
            sb = sp[(k0 + kKStep) / 32];
        }
        acc = mfma16(as_bf16x8(a[0]), fp4x8_to_bf16(bcur.x, scale), acc);
        acc = mfma16(as_bf16x8(a[1]), fp4x8_to_bf16(bcur.y, scale), acc);
        acc = mfma16(as_bf16x8(a[2]), fp4x8_to_bf16(bcur.z, scale), acc);
        acc = mfma16(as_bf16x8(a[3]), fp4x8_to_bf16(bcur.w, scale), acc);
    }
    // lane holds C[g*4 + r][n]; lane ^ 8 holds the up value of the same feature
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float v = acc[r];
        const float u = __shfl_xor(v, 8);
        const int row = g * 4 + r;
        if (n < 8 && row < tl.nrows)
            h[(int64_t)(tl.row0 + row) * F + f0 + n] = f32_to_bf16(silu(v) * u);
    }
}

__global__ __launch_bounds__(256) void gemm2_kernel(
    const uint16_t *__restrict__ h, const Tile *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, const uint8_t *__restrict__ wpk,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ o, float *__restrict__ ssq, int d,
    int F, int blocks)
{
    const int lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t tile = gw / blocks;
    const int blk = (int)(gw % blocks);
    if (tile >= *ntiles) return;
    const Tile tl = tiles[tile];
    const int n = lane & 15, g = lane >> 4;
    const int i0 = blk * 16;
    const int64_t ebytes = (int64_t)3 * d * F / 2, escales = (int64_t)3 * d * F / 32;
    const uint8_t *bp = wpk + tl.expert * ebytes + (int64_t)2 * F * (d / 2) +
                        (int64_t)(i0 + n) * (F / 2) + g * 16;
    const uint8_t *sp = sc + tl.expert * escales + (int64_t)2 * F * (d / 32) +
                        (int64_t)(i0 + n) * (F / 32) + g;
    const bool valid = n < tl.nrows;
    const uint16_t *ap = h + (int64_t)(tl.row0 + (valid ? n : 0)) * F + g * 32;

    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    uint4 bw = *reinterpret_cast<const uint4 *>(bp);
    uint32_t sb = sp[0];
    for (int k0 = 0; k0 < F; k0 += kKStep) {
        uint4 a[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            a[s] = valid ? *reinterpret_cast<const uint4 *>(ap + k0 + s * 8) : make_uint4(0, 0, 0, 0);
        const uint4 bcur = bw;
        const float scale = e8m0_to_f32(sb);
        if (k0 + kKStep < F) {
            bw = *reinterpret_cast<const uint4 *>(bp + (k0 + kKStep) / 2);
            sb = sp[(k0 + kKStep) / 32];
        }
        acc = mfma16(as_bf16x8(a[0]), fp4x8_to_bf16(bcur.x, scale), acc);
        acc = mfma16(as_bf16x8(a[1]), fp4x8_to_bf16(bcur.y, scale), acc);
        acc = mfma16(as_bf16x8(a[2]), fp4x8_to_bf16(bcur.z, scale), acc);
        acc = mfma16(as_bf16x8(a[3]), fp4x8_to_bf16(bcur.w, scale), acc);
    }
    const int P = d / kSsqCols;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float v = acc[r];
        const int row = g * 4 + r;
        const float ss = sum16(v * v);
        if (row < tl.nrows) {
            o[(int64_t)(tl.row0 + row) * d + i0 + n] = f32_to_bf16(v);
            if (n == 0) ssq[(int64_t)(tl.row0 + row) * P + blk] = ss;
        }
    }
}

hipError_t launch_gemm1(const Shape &s, const Workspace &ws, const uint16_t *x,
                        const uint8_t *wpk, const uint8_t *sc, hipStream_t st)
{
    const int groups = s.F / 8;
    const int64_t waves = max_tiles(s) * groups;
    gemm1_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(x, ws.perm, ws.tiles, ws.ntiles, wpk,
                                                              sc, ws.h, s.d, s.F, s.k, groups);
    return hipGetLastError();
}

hipError_t launch_gemm2(const Shape &s, const Workspace &ws, const uint8_t *wpk,
                        const uint8_t *sc, hipStream_t st)
{
    const int blocks = s.d / 16;
    const int64_t waves = max_tiles(s) * blocks;
    gemm2_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(ws.h, ws.tiles, ws.ntiles, wpk, sc,
                                                              ws.o, ws.ssq, s.d, s.F, blocks);
    return hipGetLastError();
}

// MXFP4 rows -> bf16 rows with the conversion the kernels above use.
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
