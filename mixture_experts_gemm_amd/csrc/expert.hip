// expert.hip -- the grouped expert FFN on MXFP4 weights.
//
// "Muse Spark Open を段階的に分解する" (animemo.app):
//   section ⑨  each expert is a gate, an up and a down matrix; gate decides
//              what passes, up how much, down maps back to the token width
//              (here SwiGLU: h = silu(g) * u, o = h W_down^T);
//   section ⑪  the weights are 4-bit values sharing a small scale per block
//              and are expanded to BF16 for the multiply.  Here the few-row
//              kernels expand FP4 E2M1 x E8M0 into bf16 MFMA operands with the
//              gfx950 scaled convert; the streaming and tiled kernels feed the
//              codes and scales unexpanded to the scaled MX MFMA, with the
//              bf16 activations split exactly into FP8 or FP6 parts.  The
//              16-block format (one E4M3 scale per 16 values) is expanded
//              exactly to fp16 and multiplied with fp16 activations
//              (gemm_nv_kernel and the NV forms of the few-row kernels);
//   section ⑬  below ~58 tokens per expert the time is the weight read, above
//              it the multiply: the decode kernels are built to keep weight
//              bytes in flight, the tiled kernels to keep the MFMA pipe busy.
//
// Weights are read in the packed tile layout of layout.h.
//
// bf16 operand layout (mfma 16x16x32 bf16): lane l holds A[m = l%16][k] and
// B[k][n = l%16] for the 8 k of k-group l/16 and step s: k = 32*(l/16) + 8*s
// + [0..8) inside a 128-wide K chunk.  So one 16-byte weight load per lane is
// exactly one 32-element scale block, and four MFMA steps consume it.
#include <hip/hip_ext.h>

#include <type_traits>

#include "device.h"
#include "internal.h"
#include "layout.h"
#include "topk.h"

namespace moe {

constexpr int kDecodeLdsBytes = 32 * 1024;  // LDS for the staged activation rows of the decode kernels
constexpr int kG1StreamU = 4;               // chunks per weight batch of the streaming gate/up kernel
constexpr int kUnroll = 4;  // chunks per weight batch of the decode kernels
constexpr int kDownU = 2;   // the MXFP4 few-row down kernel's (T=1 15.5 -> 14.7 us; T=4 the same as 4)
constexpr size_t kNvFuseLds = 64 * 1024;  // LDS the 16-block down kernel may take for its own h rows

// A tile read from LDS at a workgroup-uniform index, its fields moved to
// scalar registers (the weight addresses then stay scalar, as after a
// scalar load of the global tile list).
__device__ __forceinline__ Tile uniform_tile(const Tile &t)
{
    Tile u;
    u.expert = __builtin_amdgcn_readfirstlane(t.expert);
    u.row0 = __builtin_amdgcn_readfirstlane(t.row0);
    u.nrows = __builtin_amdgcn_readfirstlane(t.nrows);
    u.first = __builtin_amdgcn_readfirstlane(t.first);
    u.count = __builtin_amdgcn_readfirstlane(t.count);
    u.pad[0] = u.pad[1] = u.pad[2] = 0;
    return u;
}

__device__ __forceinline__ floatx4_t mfma_chunk(const uint4 *a, uint4 b, float scale, floatx4_t acc)
{
    acc = mfma16(as_bf16x8(a[0]), fp4x8_to_bf16(b.x, scale), acc);
    acc = mfma16(as_bf16x8(a[1]), fp4x8_to_bf16(b.y, scale), acc);
    acc = mfma16(as_bf16x8(a[2]), fp4x8_to_bf16(b.z, scale), acc);
    acc = mfma16(as_bf16x8(a[3]), fp4x8_to_bf16(b.w, scale), acc);
    return acc;
}

// E4M3 scale byte -> (the scaled convert's fp32 power of two, the fp16
// factor pair) for all 256 bytes, one entry per thread of the first 256.
__device__ __forceinline__ void fill_e4m3_table(uint2 *lut)
{
    if (threadIdx.x < 256) {
        const E4m3Parts e = e4m3_parts(threadIdx.x);
        lut[threadIdx.x] = make_uint2(__float_as_uint(e.p), __builtin_bit_cast(uint32_t, e.m));
    }
}

__device__ __forceinline__ E4m3Parts e4m3_lookup(const uint2 *lut, uint32_t b)
{
    const uint2 v = lut[b];
    return E4m3Parts{__uint_as_float(v.x), __builtin_bit_cast(f16x2_t, v.y)};
}

// The same K chunk with weights in the 16-block format: the lane's 32 codes
// are two 16-blocks (b.x, b.y and b.z, b.w) with the E4M3 scale bytes in
// s2's low and high byte (decoded through the table lut, fill_e4m3_table),
// expanded exactly to fp16; a holds fp16 activations.
__device__ __forceinline__ floatx4_t mfma_chunk_nv(const uint4 *a, uint4 b, uint32_t s2, const uint2 *lut,
                                                   floatx4_t acc)
{
    const E4m3Parts lo = e4m3_lookup(lut, s2 & 0xFFu), hi = e4m3_lookup(lut, (s2 >> 8) & 0xFFu);
    acc = mfma16h(as_f16x8(a[0]), fp4x8_to_f16(b.x, lo), acc);
    acc = mfma16h(as_f16x8(a[1]), fp4x8_to_f16(b.y, lo), acc);
    acc = mfma16h(as_f16x8(a[2]), fp4x8_to_f16(b.z, hi), acc);
    acc = mfma16h(as_f16x8(a[3]), fp4x8_to_f16(b.w, hi), acc);
    return acc;
}

// bf16 rows -> fp16 rows for the 16-block kernels: a row is multiplied by
// 2^q, q chosen so its largest magnitude lands in [2^14, 2^15) (q <= 126),
// and its scale is 2^-q.  Exact for every element down to 2^-32 of the row's
// largest (fp16 keeps 11 significant bits, bf16 has 8); smaller ones round
// to the fp16 subnormal grid.  One row of n 16-byte units by the whole
// workgroup (every thread calls it); dst may be global or LDS; wmax is one
// word of LDS per wave.  Returns the row's scale.
__device__ float f16_row_block(const uint4 *__restrict__ s4, uint4 *d4, int n, uint32_t *wmax)
{
    const int nt = (int)blockDim.x, nw = nt >> 6;
    uint32_t mx = 0;
    for (int i = threadIdx.x; i < n; i += nt) {
        const uint4 v = s4[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mx = max(mx, w[j] & 0x7FFFu);
            mx = max(mx, (w[j] >> 16) & 0x7FFFu);
        }
    }
    // magnitudes of bf16 order as their bit patterns: an integer max
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = wmax[0];
    for (int w = 1; w < nw; ++w) mx = max(mx, wmax[w]);
    const int eb = (int)(mx >> 7);  // biased exponent of the largest magnitude
    int q = mx == 0 ? 0 : (eb == 0 ? 126 : 14 - (eb - 127));
    q = q > 126 ? 126 : q;
    const float f = pow2f(q);
    for (int i = threadIdx.x; i < n; i += nt) {
        const uint4 v = s4[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const _Float16 lo = (_Float16)(bf16_to_f32((uint16_t)(w[j] & 0xFFFFu)) * f);
            const _Float16 hi = (_Float16)(bf16_to_f32((uint16_t)(w[j] >> 16)) * f);
            o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        d4[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    __syncthreads();  // wmax is free again, dst complete
    return pow2f(-q);
}

// One workgroup per row, K a multiple of 8.
__global__ __launch_bounds__(256) void f16_rows_kernel(const uint16_t *__restrict__ src, int K,
                                                       uint16_t *__restrict__ dst,
                                                       float *__restrict__ scale)
{
    __shared__ uint32_t wmax[4];
    const int64_t row = blockIdx.x;
    const float sc = f16_row_block(reinterpret_cast<const uint4 *>(src + row * K),
                                   reinterpret_cast<uint4 *>(dst + row * K), K / 8, wmax);
    if (threadIdx.x == 0) scale[row] = sc;
}

// ---- small device helpers ---------------------------------------------------

// Wait until at most N of this wave's loads are outstanding, then barrier.
template <int N>
__device__ __forceinline__ void chunk_sync()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(N) : "memory");
}

// Wait until at most N of this wave's global loads are outstanding and its LDS
// reads have returned, then barrier.
template <int N>
__device__ __forceinline__ void phase_sync()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its outstanding global loads (which __syncthreads would drain).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// =========================================================================
// Few-row kernels (bf16 MFMA): tiles of <= 16 grouped rows, weights streamed
// once.  The tile's activation rows (usually 1-4 valid rows) are copied once
// into LDS when they fit (rows_fit rows); each lane then reads its A
// fragment from LDS, so the vector-memory path carries almost only weight
// bytes.  Each wave keeps U chunks of weight loads in flight.
// =========================================================================

// gate/up: a workgroup owns 16 features (their gate block and up block); its
// 4 waves take quarters of the K chunks and their partial sums are added in
// LDS in a fixed order.  NV: weights in the 16-block format, x in fp16 with
// per-token scales xs, matrix scales gs [E][3]; else MXFP4 and bf16 x.
template <int U, bool NV>
__global__ __launch_bounds__(256) void gemm1_decode_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ perm,
    const Tile *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    const uint8_t *__restrict__ wpk, const uint8_t *__restrict__ sc, uint16_t *__restrict__ h,
    int d, int F, int k, int groups, int rows_fit, const float *__restrict__ xs,
    const float *__restrict__ gs)
{
    constexpr int NB = 2;  // gate block, up block
    extern __shared__ uint4 arows[];  // [rows_fit][d/8]
    __shared__ floatx4_t red[3][NB][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t tile = blockIdx.x / groups;
    const int grp = (int)(blockIdx.x % groups);
    if (tile >= *ntiles) return;
    const Tile tl = tiles[tile];
    const int n = lane & 15, g = lane >> 4;
    const WView v = NV ? w1_codes(wpk, tl.expert, d, F) : w1_view(wpk, sc, tl.expert, d, F);
    const NvScales vs = w1_nv_scales(sc, tl.expert, d, F);
    const int f = grp * 16 + n, nt = f >> 7;
    const int rho[NB] = {w1_rho(f, false), w1_rho(f, true)};
    const bool valid = n < tl.nrows;
    const bool use_lds = tl.nrows <= rows_fit;
    const int rowq = d / 8;  // 16-byte units per activation row
    const int nc = d / kKStep;
    const int c_begin = wv * nc / 4, c_end = (wv + 1) * nc / 4;
    uint4 b[U][NB];
    uint32_t sw[U][NB];
    auto load_b = [&](int c) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c + u < c_end) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    b[u][nb] = ld_stream16(v.slot(nt, c + u, rho[nb], g));
                    if constexpr (NV)
                        sw[u][nb] = __builtin_nontemporal_load(vs.pair(nt, c + u, rho[nb], g));
                    else
                        sw[u][nb] = ld_stream4(v.scales(nt, c + u, rho[nb]));
                }
            }
    };
    // the first batch of weight loads goes out before the activations are staged
    load_b(c_begin);
    __shared__ uint2 lut[NV ? 256 : 1];
    if constexpr (NV) fill_e4m3_table(lut);
    if (use_lds) {
        for (int q = threadIdx.x; q < tl.nrows * rowq; q += 256) {
            const int r = q / rowq, c = q - r * rowq;
            const int tok = perm[tl.row0 + r] / k;
            arows[q] = *reinterpret_cast<const uint4 *>(x + (int64_t)tok * d + c * 8);
        }
    }
    if (NV || use_lds) __syncthreads();
    const uint16_t *ap = x + (int64_t)(valid ? perm[tl.row0 + n] / k : 0) * d + g * 32;
    const uint4 *al = arows + n * rowq + g * 4;

    floatx4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int c = c_begin; c < c_end; c += U) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c + u < c_end) {
                uint4 a[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (!valid) a[s] = make_uint4(0, 0, 0, 0);
                    else if (use_lds) a[s] = al[(c + u) * (kKStep / 8) + s];
                    else a[s] = *reinterpret_cast<const uint4 *>(ap + (c + u) * kKStep + s * 8);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    if constexpr (NV)
                        acc[nb] = mfma_chunk_nv(a, b[u][nb], sw[u][nb], lut, acc[nb]);
                    else
                        acc[nb] = mfma_chunk(a, b[u][nb], e8m0_to_f32((sw[u][nb] >> (8 * g)) & 0xFFu),
                                             acc[nb]);
                }
            }
        if (c + U < c_end) load_b(c + U);
    }
    if (wv > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) red[wv - 1][nb][lane] = acc[nb];
    }
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        acc[nb] = ((acc[nb] + red[0][nb][lane]) + red[1][nb][lane]) + red[2][nb][lane];
    // lane holds C[g*4 + r][n] of both blocks
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = g * 4 + r;
        if (row < tl.nrows) {
            float gv = acc[0][r], uv = acc[1][r];
            if constexpr (NV) {
                const float xr = xs[perm[tl.row0 + row] / k];
                gv *= xr * gs[3 * tl.expert];
                uv *= xr * gs[3 * tl.expert + 1];
            }
            h[(int64_t)(tl.row0 + row) * F + f] = f32_to_bf16(silu(gv) * uv);
        }
    }
}

// down: a workgroup owns 64 output columns, one 16-column block per wave,
// each wave runs all of K.  The tile's h rows (contiguous in the grouped
// order) are copied to LDS when they fit.  Epilogue: bf16 o and the sum of
// o^2 over the workgroup's 64 columns, both stored in slot order (grouped
// row r goes to slot perm[r]), so the combine step finds a token's k rows at
// slots t*k .. t*k+k-1 without a lookup.
// NV: the 16-block format with fp16 h rows and their scales hs (grouped
// order), as gemm1_decode_kernel; with fuse, h is the bf16 rows and each
// workgroup converts its tile's rows into LDS itself (f16_row_block; every
// tile's rows must fit: rows_fit >= its rows).
// KS = 2: 8 waves, the four column blocks over two K halves each (twice the
// loads in flight a workgroup: the few-row down product waits on load
// latency, not bandwidth); the halves meet in LDS in a fixed order and the
// first half's waves store.
template <int U, bool NV, int KS = 1>
__global__ __launch_bounds__(256 * KS) void gemm2_decode_kernel(
    const uint16_t *__restrict__ h, const int32_t *__restrict__ perm, const Tile *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, const uint8_t *__restrict__ wpk,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ o, float *__restrict__ ssq, int d,
    int F, int wgs_per_tile, int rows_fit, const float *__restrict__ hs, const float *__restrict__ gs,
    bool fuse)
{
    static_assert(KS == 1 || KS == 2, "one or two K parts");
    extern __shared__ uint4 arows[];  // [rows_fit][F/8]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int cw = KS > 1 ? wv & 3 : wv, kh = KS > 1 ? wv >> 2 : 0;
    const int64_t tile = blockIdx.x / wgs_per_tile;
    const int col0 = ((int)(blockIdx.x % wgs_per_tile) * 4 + cw) * 16;
    if (tile >= *ntiles) return;
    const Tile tl = tiles[tile];
    const int n = lane & 15, g = lane >> 4;
    const WView v = NV ? w2_codes(wpk, tl.expert, d, F) : w2_view(wpk, sc, tl.expert, d, F);
    const NvScales vs = w2_nv_scales(sc, tl.expert, d, F);
    const int orow = col0 + n, nt = orow >> 8, rho = orow & 255;
    const bool valid = n < tl.nrows;
    const bool use_lds = tl.nrows <= rows_fit;
    const int rowq = F / 8;
    const int nc = F / kKStep;
    const int c_lo = kh * nc / KS, c_hi = (kh + 1) * nc / KS;  // the wave's chunks
    uint4 b[U];
    uint32_t sw[U];
    auto load_b = [&](int c) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c + u < c_hi) {
                b[u] = ld_stream16(v.slot(nt, c + u, rho, g));
                if constexpr (NV)
                    sw[u] = __builtin_nontemporal_load(vs.pair(nt, c + u, rho, g));
                else
                    sw[u] = ld_stream4(v.scales(nt, c + u, rho));
            }
    };
    load_b(c_lo);
    // destination slots of the lane's 4 output rows and of the row whose
    // o^2 sum this thread stores; in flight with the weights
    int dst[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r] = g * 4 + r < tl.nrows ? perm[tl.row0 + g * 4 + r] : 0;
    const int dst_ss = (int)threadIdx.x < tl.nrows && threadIdx.x < 16 ? perm[tl.row0 + threadIdx.x] : 0;
    __shared__ uint2 lut[NV ? 256 : 1];
    __shared__ uint32_t wmax[4 * KS];
    __shared__ float rsc[16];
    if constexpr (NV) fill_e4m3_table(lut);
    if (NV && fuse) {
        for (int r = 0; r < tl.nrows; ++r) {
            const float sc = f16_row_block(reinterpret_cast<const uint4 *>(h + (int64_t)(tl.row0 + r) * F),
                                           arows + r * rowq, rowq, wmax);
            if (threadIdx.x == 0) rsc[r] = sc;
        }
    } else if (use_lds) {
        const uint4 *src = reinterpret_cast<const uint4 *>(h + (int64_t)tl.row0 * F);
        for (int q = threadIdx.x; q < tl.nrows * rowq; q += 256 * KS) arows[q] = src[q];
    }
    if (NV || use_lds) __syncthreads();
    const uint16_t *ap = h + (int64_t)(tl.row0 + (valid ? n : 0)) * F + g * 32;
    const uint4 *al = arows + n * rowq + g * 4;

    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int c = c_lo; c < c_hi; c += U) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c + u < c_hi) {
                uint4 a[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (!valid) a[s] = make_uint4(0, 0, 0, 0);
                    else if (use_lds) a[s] = al[(c + u) * (kKStep / 8) + s];
                    else a[s] = *reinterpret_cast<const uint4 *>(ap + (c + u) * kKStep + s * 8);
                }
                if constexpr (NV)
                    acc = mfma_chunk_nv(a, b[u], sw[u], lut, acc);
                else
                    acc = mfma_chunk(a, b[u], e8m0_to_f32((sw[u] >> (8 * g)) & 0xFFu), acc);
            }
        if (c + U < c_hi) load_b(c + U);
    }
    if constexpr (KS > 1) {
        __shared__ floatx4_t red[KS - 1][4][64];
        if (kh > 0) red[kh - 1][cw][lane] = acc;
        __syncthreads();
        if (kh == 0) {
#pragma unroll
            for (int j = 0; j < KS - 1; ++j) acc += red[j][cw][lane];
        }
    }
    // sum of o^2 over the workgroup's 64 columns: per wave over its block
    // (DPP within 16-lane rows), then the four waves in LDS in a fixed order
    __shared__ float wsum[4][16];
    const int P = d / 64;
    float gd = 1.0f;
    if constexpr (NV) gd = gs[3 * tl.expert + 2];
    if (kh == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = g * 4 + r;
            float val = acc[r];
            if constexpr (NV) {
                const int rr = row < tl.nrows ? row : 0;
                val *= (fuse ? rsc[rr] : hs[tl.row0 + rr]) * gd;
            }
            if (row < tl.nrows) o[(int64_t)dst[r] * d + col0 + n] = f32_to_bf16(val);
            const float ss = sum16(val * val);
            if (n == 0) wsum[cw][g * 4 + r] = ss;
        }
    }
    __syncthreads();
    if (threadIdx.x < 16 && (int)threadIdx.x < tl.nrows) {
        const int row = threadIdx.x;
        const float t = (wsum[0][row] + wsum[1][row]) + (wsum[2][row] + wsum[3][row]);
        ssq[(int64_t)dst_ss * P + (int)(blockIdx.x % wgs_per_tile)] = t;
    }
}

// =========================================================================
// MX tiled kernels (prefill): tiles of <= 128 grouped rows x 256 weight rows,
// all of K, on the gfx950 scaled MX MFMA (16x16x128, f8f6f4).  The FP4
// weights and their E8M0 scales go into the instruction as they are stored,
// so nothing is expanded in registers.  The bf16 activations arrive split
// into two FP8 E4M3 parts (split_rows_kernel): a = hi*2^sh + lo*2^sl, exact
// for every value above 2^-13 of its 32-block maximum, and every 16x16x128
// block takes two MFMAs (hi, lo).  Accumulation stays fp32.
//
// Operand map of the scaled MFMA (probed on the hardware): lanes l/16 = g.
//   B (FP4, 16 bytes/lane): row n = l%16, the 32 values of weight block g of
//     the chunk, scale_b = that block's E8M0 byte.
//   A (FP8, 32 bytes/lane): row m = l%16, bytes 0-15 = K 16g..16g+15 and
//     bytes 16-31 = K 64+16g..64+16g+15 of the chunk; scale_a of lane group
//     g applies to the A values that meet B block g, i.e. activation block g
//     (K 32g..32g+31), so the activation split uses the natural 32-blocks.
//
// Three-stage LDS ring per 128-wide K chunk, filled by direct-to-LDS loads:
// A hi and lo 128 rows x 128 B each (16-byte slot c of row r at c ^ (r & 7)),
// A scales 128 x (hi word, lo word), and the chunk's weight tile and scale
// tile copied linearly (the packed layout is already the LDS layout).
// 150.5 KB for three stages; chunk kc+2 is in flight while chunk kc is
// multiplied.  Waits are explicit vmcnt counts.
// =========================================================================
constexpr int kTM = 128;  // rows per tile
constexpr int kTN = 256;  // weight rows per tile (one packed weight tile)

typedef int v8i_t __attribute__((__vector_size__(8 * sizeof(int))));

// The rows and N-tile of the item a tiled kernel's workgroup takes.  The
// gate/up kernels take it from the schedule the tile-list code wrote
// (SchedItem, sched_pos), loading the entry and the tile count side by side;
// false past the last item.
struct ItemRows {
    int expert, row0, nrows, ntile;
};
__device__ __forceinline__ bool sched_take(const SchedItem *sched, const int32_t *ntiles, int ntn,
                                           ItemRows &tl)
{
    const SchedItem it = sched[blockIdx.x];
    if (sched_pos((int)blockIdx.x, sched_shape(2 * ntn, *ntiles * ntn)) < 0) return false;
    tl.row0 = it.row0;
    tl.expert = (int)(it.packed & 1023u);
    tl.nrows = (int)((it.packed >> 10) & 255u);
    tl.ntile = (int)(it.packed >> 18);
    return true;
}
// The down kernels take contiguous ranges of the tile list per XCD
// (xcd_tile): expert by expert, N-tile-major inside an expert, so the
// workgroups of an expert's row tiles that read the same weight tile run
// side by side on one XCD and the second read can hit its L2.
__device__ __forceinline__ bool tile_take(const Tile *tiles, const int32_t *ntiles, int ntn,
                                          ItemRows &tl)
{
    int idx;
    if (!xcd_tile(*ntiles * ntn, idx)) return false;
    Tile t = tiles[idx / ntn];
    const int r = idx - t.first * ntn;
    const int nt = r / t.count, mt = t.first + (r - nt * t.count);
    if (mt != idx / ntn) t = tiles[mt];
    tl.expert = t.expert;
    tl.row0 = t.row0;
    tl.nrows = t.nrows;
    tl.ntile = nt;
    return true;
}
__device__ __forceinline__ bool item_take(const SchedItem *sched, const Tile *tiles,
                                          const int32_t *ntiles, int ntn, ItemRows &tl)
{
    return sched ? sched_take(sched, ntiles, ntn, tl) : tile_take(tiles, ntiles, ntn, tl);
}

struct MxArgs {
    const uint8_t *ahi, *alo;     // activation parts [rows][K] (FP8)
    const uint8_t *ashi, *aslo;   // their E8M0 scales [rows][K/32]
    const uint8_t *a6;            // or three-part FP6 records [rows][K/128] (wide kernel)
    const int32_t *perm;
    const Tile *tiles;
    const SchedItem *sched;       // gate/up: the workgroups' items (down: null, tile ranges)
    const int32_t *ntiles;
    const uint8_t *wpk;
    const uint8_t *sc;
    uint16_t *out;                // h or o (bf16)
    float *ssq;
    int d, F, k, ntn;
    uint8_t *h6;                  // gate/up of the wide kernel: h as FP6 records here (else bf16 out)
};

// FP6 E2M3 A (24 bytes/lane: the 32 values of activation block g of the
// chunk, 6 bits each, in K order; probed on the hardware) x FP4 B.  With
// both operands narrower than 8 bits the instruction issues at twice the
// FP8 rate.
__device__ __forceinline__ floatx4_t mfma_mx6(const uint2 &a0, const uint2 &a1, const uint2 &a2,
                                              const uint4 &b, uint32_t sa, uint32_t sb, floatx4_t c)
{
    const v8i_t av = {(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, 0, 0};
    const v8i_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    // format codes: 2 = FP6 E2M3 (A), 4 = FP4 E2M1 (B)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 2, 4, 0, (int)sa, 0, (int)sb);
}

__device__ __forceinline__ floatx4_t mfma_mx(const uint4 &a0, const uint4 &a1, const uint4 &b,
                                             uint32_t sa, uint32_t sb, floatx4_t c)
{
    const v8i_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                      (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const v8i_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    // format codes: 0 = FP8 E4M3 (A), 4 = FP4 E2M1 (B)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 4, 0, (int)sa, 0, (int)sb);
}

template <bool GATE_UP>
__global__ __launch_bounds__(512) void gemm_mx_kernel(const MxArgs pa)
{
    // 8 waves: 4 along M (rows), 2 along N; each wave owns 32 rows x 128 columns
    constexpr int NW = 8, WM = NW / 2, RW = kTM / WM, MB = RW / 16;
    constexpr int AL = kTM * 8 / (64 * NW);  // A-part loads per thread per chunk (each part)
    constexpr int BL = kTN * 4 / (64 * NW);  // weight-tile loads per thread per chunk
    constexpr int NLOADS = 2 * AL + BL + 1;
    __shared__ uint4 Ah0[kTM * 8], Ah1[kTM * 8], Ah2[kTM * 8];
    __shared__ uint4 Al0[kTM * 8], Al1[kTM * 8], Al2[kTM * 8];
    __shared__ uint32_t Ac0[kTM * 2], Ac1[kTM * 2], Ac2[kTM * 2];
    __shared__ uint4 Bs0[kTN * 4], Bs1[kTN * 4], Bs2[kTN * 4];
    __shared__ uint32_t Ss0[kTN], Ss1[kTN], Ss2[kTN];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int d = pa.d, F = pa.F;
    // The item comes from the schedule the tile-list code wrote (longest
    // first, an expert's items together on one XCD, N-tile-major, so the
    // workgroups of an expert's row tiles that read the same weight tile run
    // side by side and the second read can hit the L2).
    ItemRows tl;
    if (!item_take(pa.sched, pa.tiles, pa.ntiles, pa.ntn, tl)) return;
    const int nt = tl.ntile;
    const int K = GATE_UP ? d : F;
    auto src_row = [&](int r) -> int64_t {
        const int rr = r < tl.nrows ? r : 0;  // rows past nrows re-read row 0 (never stored)
        return GATE_UP ? (int64_t)(pa.perm[tl.row0 + rr] / pa.k) : (int64_t)(tl.row0 + rr);
    };

    // ---- load assignment ----------------------------------------------------
    // A parts: load i of this wave fills rows 8*(NW*i + wv) + lane/8, stored slot lane%8
    const uint8_t *ahsrc[AL], *alsrc[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int r = 8 * (NW * i + wv) + (lane >> 3);
        const int slot = (lane & 7) ^ (r & 7);
        const int64_t off = src_row(r) * K + slot * 16;
        ahsrc[i] = pa.ahi + off;
        alsrc[i] = pa.alo + off;
    }
    // weight tile nt of this matrix: load i fills 16-byte unit 64*(NW*i + wv) + lane
    const WView v = GATE_UP ? w1_view(pa.wpk, pa.sc, tl.expert, d, F)
                            : w2_view(pa.wpk, pa.sc, tl.expert, d, F);
    const uint8_t *bsrc = v.tile(nt, 0) + (64 * wv + lane) * 16;
    // scales: A dword q = (row q/2, hi or lo part by q%2); B dword q = row q;
    // waves 0-3 load the A scales, waves 4-7 the B scales.
    const int q = 64 * (wv & 3) + lane;
    const uint8_t *acsrc = ((lane & 1) ? pa.aslo : pa.ashi) + src_row(q >> 1) * (K / 32);
    const uint8_t *ssrc = v.stile(nt, 0) + q * 4;
    const int nk = K / kKStep;

    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int qwu = wvu & 3;
    auto issue = [&](int kc, uint4 *Ah, uint4 *Al, uint32_t *Ac, uint4 *Bs, uint32_t *Ss) {
#pragma unroll
        for (int i = 0; i < AL; ++i) dma16(ahsrc[i] + kc * kKStep, lds_off(Ah + (NW * i + wvu) * 64));
#pragma unroll
        for (int i = 0; i < AL; ++i) dma16(alsrc[i] + kc * kKStep, lds_off(Al + (NW * i + wvu) * 64));
        if (wvu < 4) dma4(acsrc + kc * 4, lds_off(Ac + 64 * qwu));
#pragma unroll
        for (int i = 0; i < BL; ++i)
            dma16(bsrc + (int64_t)kc * kWTileBytes + i * NW * 1024, lds_off(Bs + (NW * i + wvu) * 64));
        if (wvu >= 4) dma4(ssrc + kc * kWTileScaleBytes, lds_off(Ss + 64 * qwu));
    };

    // ---- compute assignment -------------------------------------------------
    const int wm = wv % WM, wn = wv / WM;
    const int n16 = lane & 15, g = lane >> 4;
    int mb_act = (tl.nrows - wm * RW + 15) >> 4;
    mb_act = mb_act < 0 ? 0 : (mb_act > MB ? MB : mb_act);

    floatx4_t acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint4 *Ah, const uint4 *Al, const uint32_t *Ac, const uint4 *Bs,
                       const uint32_t *Ss, auto full) {
        constexpr bool F_ = decltype(full)::value;
        uint4 bw[8];
        uint32_t bsc[8];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
            const int rho = wn * 128 + nb * 16 + n16;
            bw[nb] = Bs[rho * 4 + (g ^ bswz(rho))];
            bsc[nb] = (Ss[rho] >> (8 * g)) & 0xFFu;
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (F_ || mb < mb_act) {
                const int row = wm * RW + mb * 16 + n16;
                const int sw = row & 7;
                const uint4 h0 = Ah[row * 8 + (g ^ sw)], h1 = Ah[row * 8 + ((4 + g) ^ sw)];
                const uint4 l0 = Al[row * 8 + (g ^ sw)], l1 = Al[row * 8 + ((4 + g) ^ sw)];
                const uint32_t sh = (Ac[row * 2] >> (8 * g)) & 0xFFu;
                const uint32_t sl = (Ac[row * 2 + 1] >> (8 * g)) & 0xFFu;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = mfma_mx(h0, h1, bw[nb], sh, bsc[nb], acc[mb][nb]);
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = mfma_mx(l0, l1, bw[nb], sl, bsc[nb], acc[mb][nb]);
            }
        }
    };

    // ---- pipeline --------------------------------------------------------------
    issue(0, Ah0, Al0, Ac0, Bs0, Ss0);
    if (nk > 1) issue(1, Ah1, Al1, Ac1, Bs1, Ss1);
    const bool full = mb_act == MB;
    auto step = [&](int kc, uint4 *Ahc, uint4 *Alc, uint32_t *Acc, uint4 *Bc, uint32_t *Sc,
                    uint4 *Ahn, uint4 *Aln, uint32_t *Acn, uint4 *Bn, uint32_t *Sn) {
        if (kc + 1 < nk) chunk_sync<NLOADS>();
        else chunk_sync<0>();
        if (kc + 2 < nk) issue(kc + 2, Ahn, Aln, Acn, Bn, Sn);
        if (full) compute(Ahc, Alc, Acc, Bc, Sc, std::true_type{});
        else if (mb_act > 0) compute(Ahc, Alc, Acc, Bc, Sc, std::false_type{});
    };
    for (int kc = 0; kc < nk; kc += 3) {
        step(kc, Ah0, Al0, Ac0, Bs0, Ss0, Ah2, Al2, Ac2, Bs2, Ss2);
        if (kc + 1 < nk) step(kc + 1, Ah1, Al1, Ac1, Bs1, Ss1, Ah0, Al0, Ac0, Bs0, Ss0);
        if (kc + 2 < nk) step(kc + 2, Ah2, Al2, Ac2, Bs2, Ss2, Ah1, Al1, Ac1, Bs1, Ss1);
    }

    // ---- epilogue ----------------------------------------------------------------
    // lane holds C[g*4 + r][n16] of every 16x16 block
    if (GATE_UP) {
        // column block nb < 4: gate features wn*64 + 16nb + n16 of N-tile nt; nb + 4: up
        const int fbase = nt * 128 + wn * 64;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = wm * RW + mb * 16 + g * 4 + r;
                    if (row < tl.nrows)
                        pa.out[(int64_t)(tl.row0 + row) * F + fbase + hb * 16 + n16] =
                            f32_to_bf16(silu(acc[mb][hb][r]) * acc[mb][hb + 4][r]);
                }
        }
    } else {
        // bf16 o and the sum of o^2 over each 64-column half of the wave's columns
        const int P = d / 64;
        const int cbase = nt * kTN + wn * 128;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = wm * RW + mb * 16 + g * 4 + r;
                float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) ss0 += acc[mb][nb][r] * acc[mb][nb][r];
#pragma unroll
                for (int nb = 4; nb < 8; ++nb) ss1 += acc[mb][nb][r] * acc[mb][nb][r];
                ss0 = sum16(ss0);
                ss1 = sum16(ss1);
                if (row < tl.nrows) {
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb)
                        pa.out[(int64_t)(tl.row0 + row) * d + cbase + nb * 16 + n16] =
                            f32_to_bf16(acc[mb][nb][r]);
                    if (n16 == 0) {
                        pa.ssq[(int64_t)(tl.row0 + row) * P + cbase / 64] = ss0;
                        pa.ssq[(int64_t)(tl.row0 + row) * P + cbase / 64 + 1] = ss1;
                    }
                }
            }
        }
    }
}

// =========================================================================
// Wide MX tiled kernel (prefill): MR grouped rows x 512 weight rows (two
// packed weight tiles) per workgroup, all of K.  The activations arrive as
// three FP6 E2M3 parts per value (split_e2m3x3_block), so each 16x16x128
// block takes three scaled MFMAs that issue at twice the FP8 rate: 3/4 of
// the matrix-core time of two FP8 parts, for 304 instead of 264 activation
// bytes per row and chunk.  LDS ring filled by direct-to-LDS loads: 128-row
// tiles take two stages of 72 KB (chunk kc+1 in flight while chunk kc is
// multiplied), 64-row tiles three of 53 KB (chunks kc+1 and kc+2 in flight:
// few rows per expert make the multiply short next to the weight loads).
// A row's 304-byte record is copied whole; 304 = 76 dwords puts the 16 rows
// of a row block on distinct LDS banks.  8 waves as 2 (rows) x 4 (columns):
// each wave owns MR/2 rows x 128 columns (MR/32 x 8 blocks of 16x16).  Used
// when the matrix has an even number of 256-row weight tiles.
// =========================================================================
template <bool GATE_UP, int MR>
__global__ __launch_bounds__(512) void gemm_mxw_kernel(const MxArgs pa)
{
    static_assert(MR == 128 || MR == 64, "128-row tiles on two stages, 64-row tiles on three");
    constexpr int NW = 8, MB = MR / 32, RH = MR / 2;  // row blocks per wave, rows per wave row
    constexpr int ST = MR == 128 ? 2 : 3;             // ring stages
    constexpr int AU = MR * kA6Units;                 // 16-byte units of a stage's records
    constexpr int AL = (AU + 64 * NW - 1) / (64 * NW);  // record loads per wave (5 or 3)
    constexpr int BU = 2 * kTN * 4, SU = 2 * kTN / 4;   // weight / scale units of a stage
    // one pool: the stages during the K loop, the fp32 h tile in the epilogue
    __shared__ uint4 pool[ST * (AU + BU + SU)];
    uint4 *const As0 = pool, *const As1 = pool + AU;
    uint4 *const Bs0 = pool + ST * AU, *const Bs1 = Bs0 + BU;
    uint32_t *const Ss0 = reinterpret_cast<uint32_t *>(pool + ST * (AU + BU));
    uint32_t *const Ss1 = Ss0 + 2 * kTN;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int d = pa.d, F = pa.F;
    // the item from the schedule (as gemm_mx_kernel; N-tiles are pairs)
    ItemRows tl;
    if (!item_take(pa.sched, pa.tiles, pa.ntiles, pa.ntn, tl)) return;
    const int np = tl.ntile;
    const int K = GATE_UP ? d : F;
    const int nk = K / kKStep;
    auto src_row = [&](int rw) -> int64_t {
        const int rr = rw < tl.nrows ? rw : 0;  // rows past nrows re-read row 0 (never stored)
        return GATE_UP ? (int64_t)(pa.perm[tl.row0 + rr] / pa.k) : (int64_t)(tl.row0 + rr);
    };

    // ---- load assignment ----------------------------------------------------
    // Records: load i of this wave fills stage unit P = 64*(8i + wv) + lane,
    // unit P % 19 of row P / 19.  Two stages: rows past nrows are not loaded
    // (their LDS rows hold stale data; they only feed output rows that are
    // never stored), and every wait is vmcnt(0), so loads skipped this way
    // cannot upset a count.  Three stages: the waits leave the next chunk's
    // loads in flight by count, so every wave issues a fixed number of
    // whole-wave loads (rows past nrows re-read row 0 and are never stored).
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int na = ST == 2 ? AL : (64 * (NW * (AL - 1) + wvu) < AU ? AL : AL - 1);
    const uint8_t *asrc[AL];
    bool aload[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int P = 64 * (NW * i + wv) + lane;
        const int rw = P / kA6Units, u = P - rw * kA6Units;
        aload[i] = ST == 2 ? (P < AU && rw < tl.nrows) : i < na;
        asrc[i] = pa.a6 + (src_row(aload[i] ? rw : 0) * nk) * kA6Bytes + u * 16;
    }
    // weight tiles 2np and 2np+1: load i fills unit 64*(8i + wv) + lane of the
    // 2048 units (tile i/2); scale dword q = 64*wv + lane of the 512 (tile q/256)
    const WView v = GATE_UP ? w1_view(pa.wpk, pa.sc, tl.expert, d, F)
                            : w2_view(pa.wpk, pa.sc, tl.expert, d, F);
    // loads 2t and 2t+1 read tile t at units 64*wv + lane and 512 + 64*wv + lane
    const uint8_t *bsrc0 = v.tile(2 * np, 0) + (64 * wv + lane) * 16;
    const uint8_t *bsrc1 = v.tile(2 * np + 1, 0) + (64 * wv + lane) * 16;
    const int qb = 64 * wv + lane;
    const uint8_t *ssrc = v.stile(2 * np + (qb >> 8), 0) + (qb & 255) * 4;

    // The loads of a chunk go out in three parts spread over the multiply of
    // the chunk before (part 0 the activation records, parts 1 and 2 the two
    // weight tiles, in the order kPartOrder below), so a wave is not held at
    // the address unit while its MFMAs could be issuing.
    auto issue_part = [&](int part, int kc, uint4 *As, uint4 *Bs, uint32_t *Ss) {
        if (part == 0) {
#pragma unroll
            for (int i = 0; i < AL; ++i)
                if (aload[i]) dma16(asrc[i] + kc * kA6Bytes, lds_off(As + (NW * i + wvu) * 64));
        } else if (part == 1) {
            const int64_t bo = (int64_t)kc * kWTileBytes;
            dma16(bsrc0 + bo, lds_off(Bs + (0 + wvu) * 64));
            dma16(bsrc0 + bo + 8192, lds_off(Bs + (NW + wvu) * 64));
        } else {
            const int64_t bo = (int64_t)kc * kWTileBytes;
            dma16(bsrc1 + bo, lds_off(Bs + (2 * NW + wvu) * 64));
            dma16(bsrc1 + bo + 8192, lds_off(Bs + (3 * NW + wvu) * 64));
            dma4(ssrc + kc * kWTileScaleBytes, lds_off(Ss + 64 * wvu));
        }
    };

    // ---- compute assignment -------------------------------------------------
    // rows RH*wm.., columns 128*wn.. of the 512; waves w and w+4 share a SIMD
    // and own different row halves, so a short tile's MFMAs spread over all four
    const int wm = wv >> 2, wn = wv & 3;
    const int n16 = lane & 15, g = lane >> 4;
    int mb_act = (tl.nrows - wm * RH + 15) >> 4;
    mb_act = mb_act < 0 ? 0 : (mb_act > MB ? MB : mb_act);

    floatx4_t acc[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // multiply the chunk in (As, Bs, Ss); when kn >= 0 the parts of chunk
    // kn's loads (into the other slot) are issued along the way: at its
    // start, after row block 0 and after row block 1.  With two stages the
    // weight tiles (from HBM, the longest latency) go first and the records
    // (shared by an expert's workgroups, mostly L2 hits) last (measured:
    // 128-row tiles 2-4% faster); with three stages the records go first.
    constexpr int kPartOrder[3] = {ST == 2 ? 1 : 0, ST == 2 ? 2 : 1, ST == 2 ? 0 : 2};
    auto compute = [&](const uint4 *As, const uint4 *Bs, const uint32_t *Ss, int kn, uint4 *Asn,
                       uint4 *Bn, uint32_t *Sn) {
        if (kn >= 0) issue_part(kPartOrder[0], kn, Asn, Bn, Sn);
        // LDS reads return in order: row block 0's A fragments first, then the
        // weight fragments, so the first MFMAs wait for few reads
        struct AFr {
            uint2 p[3][3];  // part, 8-byte piece
            uint32_t s[3];
        };
        // A pieces are single 8-byte reads: the compiler barrier between them
        // keeps it from pairing them into ds_read2_b64, which runs at a
        // quarter of the LDS read rate here (ds_read_b64 at the 304-byte row
        // stride is conflict-free, measured)
        auto read_a = [&](int mb) {
            AFr f;
            const int row = wm * RH + mb * 16 + n16;
            const uint2 *rp = reinterpret_cast<const uint2 *>(As + row * kA6Units);
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    f.p[p][j] = rp[12 * p + 3 * g + j];
                    asm volatile("" ::: "memory");
                }
            const uint4 sv = As[row * kA6Units + 18];
            f.s[0] = (sv.x >> (8 * g)) & 0xFFu;
            f.s[1] = (sv.y >> (8 * g)) & 0xFFu;
            f.s[2] = (sv.z >> (8 * g)) & 0xFFu;
            return f;
        };
        uint4 bw[8];
        uint32_t bsc[8];
        auto read_b = [&](int nb) {
            const int rho = wn * 128 + nb * 16 + n16;  // row of the 512; bank swizzle of its tile row
            bw[nb] = Bs[rho * 4 + (g ^ bswz(rho))];
            bsc[nb] = (Ss[rho] >> (8 * g)) & 0xFFu;
        };
        auto mma = [&](int mb, const AFr &f, int p, int nb) {
            acc[mb][nb] = mfma_mx6(f.p[p][0], f.p[p][1], f.p[p][2], bw[nb], f.s[p], bsc[nb], acc[mb][nb]);
        };
        // row block 0: each weight fragment is read two MFMAs before its use
        {
            const AFr f = read_a(0);
            read_b(0);
            read_b(1);
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                __builtin_amdgcn_sched_barrier(0);
                if (nb + 2 < 8) read_b(nb + 2);
                if (mb_act > 0) mma(0, f, 0, nb);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (mb_act > 0) {
#pragma unroll
                for (int p = 1; p < 3; ++p)
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) mma(0, f, p, nb);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kn >= 0) issue_part(kPartOrder[1], kn, Asn, Bn, Sn);
        }
#pragma unroll
        for (int mb = 1; mb < MB; ++mb) {
            // one row block's A fragments at a time (the accumulators take 128 registers)
            __builtin_amdgcn_sched_barrier(0);
            if (mb < mb_act) {
                const AFr f = read_a(mb);
#pragma unroll
                for (int p = 0; p < 3; ++p)
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb) mma(mb, f, p, nb);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (mb == 1 && kn >= 0) issue_part(kPartOrder[2], kn, Asn, Bn, Sn);
        }
    };

    if constexpr (ST == 2) {
        // ---- pipeline: two slots; the barrier before chunk kc also waits for
        // this wave's LDS reads of chunk kc-1, whose slot chunk kc+1 then
        // refills, and for all of this wave's loads of chunk kc -------------
        for (int part = 0; part < 3; ++part) issue_part(part, 0, As0, Bs0, Ss0);
        for (int kc = 0; kc < nk; kc += 2) {
            phase_sync<0>();
            compute(As0, Bs0, Ss0, kc + 1 < nk ? kc + 1 : -1, As1, Bs1, Ss1);
            if (kc + 1 < nk) {
                phase_sync<0>();
                compute(As1, Bs1, Ss1, kc + 2 < nk ? kc + 2 : -1, As0, Bs0, Ss0);
            }
        }
    } else {
        // ---- pipeline: three slots, two chunks ahead.  A wave issues na + 5
        // loads a chunk (records, two weight pairs, the scales), so the wait
        // before chunk kc leaves chunk kc+1's loads in flight and no more;
        // the barrier also waits for every wave's LDS reads of chunk kc-1,
        // whose slot chunk kc+2 then refills --------------------------------
        static_assert(AL == 3, "the waits below count 3 or 2 record loads a wave");
        for (int part = 0; part < 3; ++part) issue_part(part, 0, As0, Bs0, Ss0);
        if (nk > 1)
            for (int part = 0; part < 3; ++part) issue_part(part, 1, As1, Bs1, Ss1);
        int slot = 0;
        for (int kc = 0; kc < nk; ++kc) {
            if (kc + 1 >= nk) phase_sync<0>();
            else if (na == AL) phase_sync<AL + 5>();
            else phase_sync<AL + 4>();
            const int nslot = slot == 0 ? 2 : slot - 1;  // (kc + 2) % 3
            compute(As0 + slot * AU, Bs0 + slot * BU, Ss0 + slot * 2 * kTN, kc + 2 < nk ? kc + 2 : -1,
                    As0 + nslot * AU, Bs0 + nslot * BU, Ss0 + nslot * 2 * kTN);
            slot = slot == 2 ? 0 : slot + 1;
        }
    }

    // ---- epilogue: lane holds C[g*4 + r][n16] of every 16x16 block -----------
    const int nt = 2 * np + (wn >> 1), half = wn & 1;  // weight tile, half of its 256 rows
    if (GATE_UP && pa.h6) {
        // h = silu(gate) * up in fp32 goes through LDS (row r, feature f of
        // the workgroup's 256 at float4 slot (f/4) ^ ((f/32) & 7) of row r, so
        // the block reads below spread over the banks), then one thread per
        // 32-feature block splits it into the down kernel's FP6 records: the
        // workgroup's 256 features are whole chunks 2np and 2np+1 of h.
        constexpr int HS = 260;  // floats per LDS row
        float *hs = reinterpret_cast<float *>(pool);
        __syncthreads();  // every wave is past its last LDS read of the stages
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
                const int f = wn * 64 + hb * 16 + n16, c = f >> 2;
                const int pos = ((c ^ ((c >> 3) & 7)) << 2) | (f & 3);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int row = wm * RH + mb * 16 + g * 4 + rr;
                    hs[row * HS + pos] = silu(acc[mb][hb][rr]) * acc[mb][hb + 4][rr];
                }
            }
        }
        __syncthreads();
        for (int b = tid; b < tl.nrows * 8; b += 64 * NW) {
            const int row = b >> 3, blk = b & 7;
            const float4 *src = reinterpret_cast<const float4 *>(hs + row * HS) + blk * 8;
            float v[32];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 t = src[q ^ blk];
                v[4 * q] = t.x;
                v[4 * q + 1] = t.y;
                v[4 * q + 2] = t.z;
                v[4 * q + 3] = t.w;
            }
            uint32_t code[3][6], sc[3];
            split_e2m3x3_block(v, code, sc);
            uint8_t *rec = pa.h6 + ((int64_t)(tl.row0 + row) * (F / kKStep) + 2 * np + (blk >> 2)) * kA6Bytes;
            const int g4 = blk & 3;
#pragma unroll
            for (int q = 0; q < 3; ++q) {
                uint2 *o = reinterpret_cast<uint2 *>(rec + 96 * q + 24 * g4);
                o[0] = make_uint2(code[q][0], code[q][1]);
                o[1] = make_uint2(code[q][2], code[q][3]);
                o[2] = make_uint2(code[q][4], code[q][5]);
                rec[288 + 4 * q + g4] = (uint8_t)sc[q];
            }
            if (g4 == 0) *reinterpret_cast<uint32_t *>(rec + 300) = 0u;
        }
    } else if (GATE_UP) {
        // column block nb < 4: gate features half*64 + 16nb + n16 of N-tile nt; nb + 4: up
        const int fbase = nt * 128 + half * 64;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int row = wm * RH + mb * 16 + g * 4 + rr;
                    if (row < tl.nrows)
                        pa.out[(int64_t)(tl.row0 + row) * F + fbase + hb * 16 + n16] =
                            f32_to_bf16(silu(acc[mb][hb][rr]) * acc[mb][hb + 4][rr]);
                }
        }
    } else {
        // bf16 o and the sum of o^2 over each 64-column half of the wave's columns
        const int P = d / 64;
        const int cbase = nt * kTN + half * 128;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = wm * RH + mb * 16 + g * 4 + rr;
                float ss0 = 0.f, ss1 = 0.f;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) ss0 += acc[mb][nb][rr] * acc[mb][nb][rr];
#pragma unroll
                for (int nb = 4; nb < 8; ++nb) ss1 += acc[mb][nb][rr] * acc[mb][nb][rr];
                ss0 = sum16(ss0);
                ss1 = sum16(ss1);
                if (row < tl.nrows) {
#pragma unroll
                    for (int nb = 0; nb < 8; ++nb)
                        pa.out[(int64_t)(tl.row0 + row) * d + cbase + nb * 16 + n16] =
                            f32_to_bf16(acc[mb][nb][rr]);
                    if (n16 == 0) {
                        pa.ssq[(int64_t)(tl.row0 + row) * P + cbase / 64] = ss0;
                        pa.ssq[(int64_t)(tl.row0 + row) * P + cbase / 64 + 1] = ss1;
                    }
                }
            }
        }
    }
}

// =========================================================================
// The 16-block format (prefill): tiles of <= 192 grouped rows x
// 256 weight rows, all of K, on the fp16 MFMA (16x16x32).  The scaled MX MFMA takes one
// power-of-two scale per 32 values, so it cannot take these weights; they
// are expanded in registers instead ("Muse Spark Open を段階的に分解する",
// section ⑪: the 4-bit weights are widened for the multiply), exactly, to
// fp16 (fp4x8_to_f16: one convert and one packed multiply per two values).
// The activations are fp16 rows with a power-of-two scale per row
// (f16_rows_kernel), applied with the matrix scale in the epilogue.
//
// LDS ring per 128-wide K chunk, filled by direct-to-LDS loads: A 192 rows x
// 256 bytes (16-byte slot q of row r at q ^ (r & 7)), the chunk's code tile
// and scale tile copied linearly (the packed layout is the LDS layout);
// 66 KB a stage, two stages (192 rows keep one expert's prefill rows in one
// tile, so its weights are loaded and widened once).  8 waves as 2 (rows) x 4 (columns): wave row wm takes the
// 16-row blocks 2j + wm, each wave 64 weight rows (4 column blocks), so a
// wave widens a weight value once per chunk for all the rows it multiplies.
// For gate/up a wave's 64 weight rows are 32 gate features and the same 32
// up features, so SwiGLU is formed in registers.
// =========================================================================
struct NvArgs {
    const uint16_t *a;   // fp16 rows: x [T][d] (gate/up, gathered by perm) or h [S][F] (down)
    const float *as;     // their per-row scales
    const int32_t *perm;
    const Tile *tiles;
    const SchedItem *sched;  // gate/up: the workgroups' items (down: null, tile ranges)
    const int32_t *ntiles;
    const uint8_t *wpk;  // packed code tiles
    const uint8_t *sc;   // packed E4M3 scale tiles
    const float *gs;     // matrix scales [E][3]: gate, up, down
    uint16_t *out;       // h [S][F] or o [S][d] (bf16, grouped order)
    float *ssq;
    int d, F, k, ntn;
};

template <bool GATE_UP>
__global__ __launch_bounds__(512) void gemm_nv_kernel(const NvArgs pa)
{
    constexpr int NW = 8;
    constexpr int MR = kNvTileRows;        // rows per tile (192)
    constexpr int ST = 2;                  // ring stages (66 KB a stage)
    constexpr int MB = MR / 32;            // row blocks of 16 per wave
    constexpr int AU = MR * 16;            // 16-byte units of an A stage
    constexpr int BU = kTN * 4;            // of a code tile
    constexpr int AL = AU / (64 * NW), BL = BU / (64 * NW);
    __shared__ uint4 As[ST][AU];
    __shared__ uint4 Bs[ST][BU];
    __shared__ uint32_t Ss[ST][kTN * 2];
    __shared__ uint2 lut[256];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int d = pa.d, F = pa.F;
    // the item from the schedule (as gemm_mx_kernel)
    ItemRows tl;
    if (!item_take(pa.sched, pa.tiles, pa.ntiles, pa.ntn, tl)) return;
    const int nt = tl.ntile;
    const int K = GATE_UP ? d : F;
    auto src_row = [&](int r) -> int64_t {
        const int rr = r < tl.nrows ? r : 0;  // rows past nrows re-read row 0 (never stored)
        return GATE_UP ? (int64_t)(pa.perm[tl.row0 + rr] / pa.k) : (int64_t)(tl.row0 + rr);
    };

    // ---- load assignment ----------------------------------------------------
    // A: load i of this wave fills units 64*(NW*i + wv) + lane: row
    // 4*(NW*i + wv) + lane/16, stored slot lane%16 = global slot ^ (row & 7).
    // Rows past nrows are not loaded (their LDS rows hold stale data and only
    // feed output rows that are never stored); every wait below is vmcnt(0),
    // so loads skipped this way cannot upset a count.
    static_assert(AL == 6 && BL == 2, "the load parts below assume 6 + 2 loads a wave");
    const uint16_t *asrc[AL];
    bool aload[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int r = 4 * (NW * i + wv) + (lane >> 4);
        const int q = (lane & 15) ^ (r & 7);
        aload[i] = r < tl.nrows;
        asrc[i] = pa.a + src_row(r) * K + q * 8;
    }
    const WView v = GATE_UP ? w1_codes(pa.wpk, tl.expert, d, F) : w2_codes(pa.wpk, tl.expert, d, F);
    const NvScales vs = GATE_UP ? w1_nv_scales(pa.sc, tl.expert, d, F)
                                : w2_nv_scales(pa.sc, tl.expert, d, F);
    const uint8_t *bsrc = v.tile(nt, 0) + (64 * wv + lane) * 16;
    const uint8_t *ssrc = vs.stile(nt, 0) + tid * 4;
    const int nk = K / kKStep;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    // The loads of a chunk go out in three parts spread over the multiply of
    // the chunk before (the code and scale tiles, then the two halves of the
    // activation rows: HBM loads first, measured 3% faster), so a wave is
    // not held at the address unit while its MFMAs could be issuing.
    auto issue_part = [&](int part, int kc, int b) {
        if (part < 2) {
#pragma unroll
            for (int i = 3 * part; i < 3 * part + 3; ++i)
                if (aload[i]) dma16(asrc[i] + kc * kKStep, lds_off(&As[b][(NW * i + wvu) * 64]));
        } else {
#pragma unroll
            for (int i = 0; i < BL; ++i)
                dma16(bsrc + (int64_t)kc * kWTileBytes + i * NW * 1024,
                      lds_off(&Bs[b][(NW * i + wvu) * 64]));
            dma4(ssrc + (int64_t)kc * kNvTileScaleBytes, lds_off(&Ss[b][64 * wvu]));
        }
    };

    // ---- compute assignment -------------------------------------------------
    // 8 waves as 2 (rows) x 4 (columns); wave row wm takes the row blocks
    // 2j + wm (interleaved, so a partly filled tile keeps both busy)
    const int wm = wv & 1, wn = wv >> 1;
    const int n16 = lane & 15, g = lane >> 4;
    const int nblk = (tl.nrows + 15) >> 4;
    int mb_act = (nblk - wm + 1) >> 1;
    mb_act = mb_act < 0 ? 0 : (mb_act > MB ? MB : mb_act);
    // packed weight rows of the wave's 4 column blocks; gate/up: blocks 0, 1
    // gate features, 2, 3 the same up features
    int rho[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
        rho[nb] = GATE_UP ? (wn >> 1) * 128 + (wn & 1) * 32 + (nb >> 1) * 64 + (nb & 1) * 16 + n16
                          : wn * 64 + nb * 16 + n16;

    floatx4_t acc[MB][4];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // Multiply the chunk in stage b with NA active row blocks (a wave's count
    // is fixed for the tile, so each count is its own unrolled loop with no
    // branch between MFMAs).  K step st+1's activation fragments are read and
    // its weights widened while step st's MFMAs run.  When kn >= 0 the parts
    // of chunk kn's loads (into the other stage) are issued along the way.
    auto compute = [&](int b, int kn, auto na) {
        constexpr int NA = decltype(na)::value;
        const uint4 *A = As[b];
        const uint4 *B = Bs[b];
        const uint16_t *S = reinterpret_cast<const uint16_t *>(Ss[b]);
        uint4 bw[4];
        E4m3Parts sp[4][2];
        f16x8_t bcur[4], bnxt[4];
        f16x8_t acur[NA > 0 ? NA : 1], anxt[NA > 0 ? NA : 1];
        auto read_a = [&](int st, f16x8_t *a) {
#pragma unroll
            for (int mb = 0; mb < NA; ++mb) {
                const int row = (2 * mb + wm) * 16 + n16;
                a[mb] = as_f16x8(A[row * 16 + ((4 * g + st) ^ (row & 7))]);
            }
        };
        auto widen = [&](int st, f16x8_t *bh) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const uint32_t c = st == 0 ? bw[nb].x : st == 1 ? bw[nb].y : st == 2 ? bw[nb].z : bw[nb].w;
                bh[nb] = fp4x8_to_f16(c, sp[nb][st >> 1]);
            }
        };
        if (NA > 0) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                bw[nb] = B[rho[nb] * 4 + (g ^ bswz(rho[nb]))];
                const uint32_t s2 = S[rho[nb] * 4 + g];
                sp[nb][0] = e4m3_lookup(lut, s2 & 0xFFu);
                sp[nb][1] = e4m3_lookup(lut, s2 >> 8);
            }
            read_a(0, acur);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (kn >= 0) issue_part(2, kn, b ^ 1);  // the code and scale tiles (from HBM) first
        __builtin_amdgcn_sched_barrier(0);
        if (NA > 0) widen(0, bcur);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            __builtin_amdgcn_sched_barrier(0);
            if (NA > 0) {
                if (st < 3) {
                    read_a(st + 1, anxt);
                    widen(st + 1, bnxt);
                }
#pragma unroll
                for (int mb = 0; mb < NA; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma16h(acur[mb], bcur[nb], acc[mb][nb]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (st < 2 && kn >= 0) issue_part(st, kn, b ^ 1);  // then the two halves of the rows
            if (NA > 0 && st < 3) {
#pragma unroll
                for (int mb = 0; mb < NA; ++mb) acur[mb] = anxt[mb];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) bcur[nb] = bnxt[nb];
            }
        }
    };

    // ---- pipeline --------------------------------------------------------------
    // The scale table is written before the first barrier of the ring.  The
    // barrier before chunk kc waits for all of this wave's loads of chunk kc;
    // the stage chunk kc+1 then refills was last read in step kc-1, whose LDS
    // reads every wave consumed before reaching that barrier.
    fill_e4m3_table(lut);
    lds_barrier();
#pragma unroll
    for (int part = 0; part < 3; ++part) issue_part(part, 0, 0);
    auto kloop = [&](auto na) {
        for (int kc = 0; kc < nk; ++kc) {
            chunk_sync<0>();
            compute(kc & 1, kc + 1 < nk ? kc + 1 : -1, na);
        }
    };
    static_assert(MB == 6, "one K loop per active row-block count");
    switch (mb_act) {
    case 6: kloop(std::integral_constant<int, 6>{}); break;
    case 5: kloop(std::integral_constant<int, 5>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
    }

    // ---- epilogue ----------------------------------------------------------------
    // lane holds C[g*4 + r][n16] of every 16x16 block
    if (GATE_UP) {
        const float gg = pa.gs[3 * tl.expert], gu = pa.gs[3 * tl.expert + 1];
        const int fbase = nt * 128 + (wn >> 1) * 64 + (wn & 1) * 32;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = (2 * mb + wm) * 16 + g * 4 + r;
                if (row < tl.nrows) {
                    const float xr = pa.as[pa.perm[tl.row0 + row] / pa.k];
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        pa.out[(int64_t)(tl.row0 + row) * F + fbase + nb * 16 + n16] = f32_to_bf16(
                            silu(acc[mb][nb][r] * (xr * gg)) * (acc[mb][nb + 2][r] * (xr * gu)));
                }
            }
        }
    } else {
        // bf16 o and the sum of o^2 over the wave's 64 columns
        const float gd = pa.gs[3 * tl.expert + 2];
        const int P = d / 64;
        const int cbase = nt * kTN + wn * 64;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = (2 * mb + wm) * 16 + g * 4 + r;
                const float hr = pa.as[tl.row0 + (row < tl.nrows ? row : 0)] * gd;
                float ov[4], ss = 0.f;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    ov[nb] = acc[mb][nb][r] * hr;
                    ss += ov[nb] * ov[nb];
                }
                ss = sum16(ss);
                if (row < tl.nrows) {
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        pa.out[(int64_t)(tl.row0 + row) * d + cbase + nb * 16 + n16] = f32_to_bf16(ov[nb]);
                    if (n16 == 0) pa.ssq[(int64_t)(tl.row0 + row) * P + cbase / 64] = ss;
                }
            }
        }
    }
}

hipError_t launch_f16_rows(const uint16_t *src, int64_t rows, int K, uint16_t *dst, float *scale,
                           hipStream_t st)
{
    if (rows <= 0) return hipSuccess;
    f16_rows_kernel<<<(unsigned)rows, 256, 0, st>>>(src, K, dst, scale);
    return hipGetLastError();
}


// bf16 rows -> FP8 E4M3 hi/lo parts + E8M0 scales per 32-block (one thread per block).
__global__ __launch_bounds__(256) void split_rows_kernel(const uint16_t *__restrict__ src,
                                                         int64_t nblk, uint8_t *__restrict__ hi,
                                                         uint8_t *__restrict__ lo,
                                                         uint8_t *__restrict__ shi,
                                                         uint8_t *__restrict__ slo)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    split_bf16_block(src + b * 32, hi + b * 32, lo + b * 32, shi + b, slo + b);
}

static hipError_t launch_split(const uint16_t *src, int64_t rows, int K, uint8_t *hi, uint8_t *lo,
                               uint8_t *shi, uint8_t *slo, hipStream_t st)
{
    const int64_t nblk = rows * (K / 32);
    split_rows_kernel<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(src, nblk, hi, lo, shi, slo);
    return hipGetLastError();
}

// bf16 rows -> three-part FP6 records (one thread per 32-block; the four
// blocks of a chunk are neighbouring threads writing one record).
__global__ __launch_bounds__(256) void split6_rows_kernel(const uint16_t *__restrict__ src,
                                                          int64_t nblk, uint8_t *__restrict__ dst)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblk) return;
    const uint4 *p = reinterpret_cast<const uint4 *>(src + b * 32);
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
    uint32_t code[3][6], sc[3];
    split_e2m3x3_block(v, code, sc);
    uint8_t *rec = dst + (b >> 2) * kA6Bytes;
    const int g = (int)(b & 3);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        uint2 *o = reinterpret_cast<uint2 *>(rec + 96 * q + 24 * g);
        o[0] = make_uint2(code[q][0], code[q][1]);
        o[1] = make_uint2(code[q][2], code[q][3]);
        o[2] = make_uint2(code[q][4], code[q][5]);
        rec[288 + 4 * q + g] = (uint8_t)sc[q];
    }
    if (g == 0) *reinterpret_cast<uint32_t *>(rec + 300) = 0u;
}

static hipError_t launch_split6(const uint16_t *src, int64_t rows, int K, uint8_t *dst, hipStream_t st)
{
    const int64_t nblk = rows * (K / 32);
    split6_rows_kernel<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(src, nblk, dst);
    return hipGetLastError();
}

hipError_t launch_split_x_fp8(const Shape &s, const Workspace &ws, const uint16_t *x, hipStream_t st)
{
    return launch_split(x, s.T, s.d, ws.xhi, ws.xlo, ws.xshi, ws.xslo, st);
}

hipError_t launch_split_x(const Shape &s, const Workspace &ws, const uint16_t *x, hipStream_t st)
{
    if (wide_gate_up(s)) return launch_split6(x, s.T, s.d, ws.xa6, st);
    return launch_split(x, s.T, s.d, ws.xhi, ws.xlo, ws.xshi, ws.xslo, st);
}

// =========================================================================
// Streaming gate/up kernel for a few tokens (decode).  The time is the read
// of the chosen experts' FP4 weights, so the kernel is built to keep that
// read going without gaps:
//  * persistent workgroups: each takes a contiguous run of work items
//    (tile, 16 features) and walks it, so there is no per-item launch,
//    start-up load chain or tail of short workgroups;
//  * the weights of the next batch of chunks are in flight while the current
//    batch is multiplied (two register buffers), also across item borders;
//    in the packed layout a wave's 16 rows of one chunk are 1 KB contiguous;
//  * the scaled MX MFMA takes the FP4 codes and E8M0 scales as stored, so no
//    vector ALU work is spent per weight;
//  * the tile's activation rows arrive as FP8 hi/lo parts with their E8M0
//    scales (split by the router pass) and are copied to LDS once per tile.
// The 4 waves take quarters of K; their partial sums meet in LDS (two
// buffers, alternating per item, one barrier per item) and wave 0 writes
// silu(gate) * up.  Requirements (checked by the plan): d % 2048 == 0,
// tiles of at most R rows.
// =========================================================================
// NV: weights in the 16-block format, the activations the bf16 rows of x
// (ghi; glo, gsh, gsl, xsc unused), converted to fp16 with a scale per row
// as the tile is staged (f16_row_block), matrix scales gs [E][3]; the chunk is multiplied by four fp16 MFMAs on
// weights widened in registers (mfma_chunk_nv) instead of the scaled MX MFMA.
template <int U, bool NV, bool ROUTE>
__global__ __launch_bounds__(256) void gemm1_stream_kernel(
    const uint8_t *__restrict__ ghi, const uint8_t *__restrict__ glo,
    const uint8_t *__restrict__ gsh, const uint8_t *__restrict__ gsl,
    int32_t *__restrict__ perm, Tile *__restrict__ tiles,
    int32_t *__restrict__ ntiles, const uint8_t *__restrict__ wpk,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ h, int d, int F, int k, int R,
    const float *__restrict__ xsc, const float *__restrict__ gs, const RouteArgs ra)
{
    static_assert(!(NV && ROUTE), "the 16-block path reads the routing kernel's tile list");
    constexpr int NB = 2;  // gate block, up block
    extern __shared__ uint4 xs4[];
    __shared__ floatx4_t red[2][3][NB][64];
    // NV: the E4M3 table and the staged rows' scales (R <= 16, checked by
    // the launcher)
    __shared__ uint2 lut[NV ? 256 : 1];
    __shared__ uint32_t wmax[4];
    __shared__ float rsc[16];
    uint8_t *xs = reinterpret_cast<uint8_t *>(xs4);
    uint8_t *xhi = xs, *xlo = xs + (size_t)R * d;
    uint8_t *xsh = xs + (size_t)2 * R * d, *xsl = xsh + (size_t)R * (d / 32);

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int groups = F / 16;
    // ROUTE: the call's routing, computed here (route_few) instead of read
    __shared__ typename std::conditional<ROUTE, FewRoute, char>::type fr;
    if constexpr (ROUTE) route_few(ra.scores, ra.T, ra.E, k, R, fr);
    // workgroup 0 stores the routing for the later kernels when it is done
    auto store_route = [&]() {
        if constexpr (ROUTE)
            if (blockIdx.x == 0)
                route_few_store(fr, ra.T, ra.E, k, ra.ids, ra.wts, ra.counts, ra.offsets, perm, ra.inv, tiles,
                                ntiles);
    };
    auto tile_at = [&](int ti) -> Tile {
        if constexpr (ROUTE) return uniform_tile(fr.tiles[ti]);
        else return tiles[ti];
    };
    auto perm_at = [&](int row) -> int {
        if constexpr (ROUTE) return __builtin_amdgcn_readfirstlane(fr.perm[row]);
        else return perm[row];
    };
    int ntl;
    if constexpr (ROUTE) ntl = fr.ntiles;
    else ntl = *ntiles;
    const int64_t nitems = (int64_t)ntl * groups;
    const int i0 = (int)(nitems * blockIdx.x / gridDim.x);
    const int i1 = (int)(nitems * (blockIdx.x + 1) / gridDim.x);
    if (i0 >= i1) {
        store_route();
        return;
    }
    const int cw = d / kKStep / 4;  // chunks per wave
    const int c_begin = wv * cw;
    const int nbat = cw / U;
    const int total = (i1 - i0) * nbat;

    // ---- weight loads (one batch = U chunks of the gate and the up block) --
    uint4 b0[U][NB], b1[U][NB];
    uint32_t s0[U][NB], s1[U][NB];
    int l_ti = -1;
    Tile l_tl{0, 0, 0, 0};
    auto load = [&](uint4 (&b)[U][NB], uint32_t (&sv)[U][NB], int st) {
        const int it = i0 + st / nbat, bt = st % nbat;
        const int ti = it / groups, grp = it - ti * groups;
        if (ti != l_ti) {
            l_tl = tile_at(ti);
            l_ti = ti;
        }
        const WView v = NV ? w1_codes(wpk, l_tl.expert, d, F) : w1_view(wpk, sc, l_tl.expert, d, F);
        const NvScales vs = w1_nv_scales(sc, l_tl.expert, d, F);
        const int c = c_begin + bt * U;
        const int f = grp * 16 + n, nt = f >> 7;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int rho = w1_rho(f, nb == 1);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                b[u][nb] = ld_stream16(v.slot(nt, c + u, rho, g));
                if constexpr (NV) sv[u][nb] = __builtin_nontemporal_load(vs.pair(nt, c + u, rho, g));
                else sv[u][nb] = ld_stream4(v.scales(nt, c + u, rho));
            }
        }
    };

    // ---- activation staging: the tile's FP8 rows and scales -> LDS --------
    int c_ti = -1;
    Tile c_tl{0, 0, 0, 0};
    auto stage = [&](int ti) {
        c_tl = tile_at(ti);
        c_ti = ti;
        const int q = d / 16, qs = d / 32 / 16;  // 16-byte units per part row / scale row
        if constexpr (NV) {
            // the bf16 rows converted here (f16_row_block) into fp16 rows of
            // 2d bytes, the space of both FP8 parts, with their scales
            for (int r = 0; r < c_tl.nrows; ++r) {
                const int64_t tok = perm_at(c_tl.row0 + r) / k;
                const float sc = f16_row_block(reinterpret_cast<const uint4 *>(ghi + tok * 2 * d),
                                               reinterpret_cast<uint4 *>(xs + (size_t)r * 2 * d), 2 * q,
                                               wmax);
                if (threadIdx.x == 0) rsc[r] = sc;
            }
            lds_barrier();
            return;
        }
        for (int r = 0; r < c_tl.nrows; ++r) {
            const int64_t tok = perm_at(c_tl.row0 + r) / k;
            const uint4 *sh = reinterpret_cast<const uint4 *>(ghi + tok * d);
            const uint4 *sl = reinterpret_cast<const uint4 *>(glo + tok * d);
            uint4 *dh = reinterpret_cast<uint4 *>(xhi + (size_t)r * d);
            uint4 *dl = reinterpret_cast<uint4 *>(xlo + (size_t)r * d);
            for (int j = threadIdx.x; j < q; j += 256) {
                dh[j] = sh[j];
                dl[j] = sl[j];
            }
            const uint4 *ssh = reinterpret_cast<const uint4 *>(gsh + tok * (d / 32));
            const uint4 *ssl = reinterpret_cast<const uint4 *>(gsl + tok * (d / 32));
            if ((int)threadIdx.x < qs) {
                reinterpret_cast<uint4 *>(xsh + (size_t)r * (d / 32))[threadIdx.x] = ssh[threadIdx.x];
                reinterpret_cast<uint4 *>(xsl + (size_t)r * (d / 32))[threadIdx.x] = ssl[threadIdx.x];
            }
        }
        lds_barrier();
    };

    // NV: the scale table, written before the first stage() barrier
    if constexpr (NV) fill_e4m3_table(lut);

    floatx4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    auto consume = [&](const uint4 (&b)[U][NB], const uint32_t (&sv)[U][NB], int st) {
        const int it = i0 + st / nbat, bt = st % nbat;
        const int ti = it / groups, grp = it - ti * groups;
        // a new tile's rows replace the old ones: every wave has passed the
        // previous item's barrier, so no wave still reads them
        if (ti != c_ti) stage(ti);
        const int m = n < c_tl.nrows ? n : 0;  // rows past nrows are computed on row 0, never stored
        const int c = c_begin + bt * U;
        if constexpr (NV) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint4 *ap = reinterpret_cast<const uint4 *>(xs + (size_t)m * 2 * d) +
                                  (c + u) * (kKStep / 8) + g * 4;
                const uint4 a[4] = {ap[0], ap[1], ap[2], ap[3]};
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[nb] = mfma_chunk_nv(a, b[u][nb], sv[u][nb], lut, acc[nb]);
            }
        } else
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint4 *hp = reinterpret_cast<const uint4 *>(xhi + (size_t)m * d + (c + u) * kKStep);
            const uint4 *lp = reinterpret_cast<const uint4 *>(xlo + (size_t)m * d + (c + u) * kKStep);
            const uint4 h0 = hp[g], h1 = hp[4 + g], l0 = lp[g], l1 = lp[4 + g];
            const int sidx = m * (d / 32) + (c + u) * 4 + g;
            const uint32_t sah = xsh[sidx], sal = xsl[sidx];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const uint32_t sb = (sv[u][nb] >> (8 * g)) & 0xFFu;
                acc[nb] = mfma_mx(h0, h1, b[u][nb], sah, sb, acc[nb]);
                acc[nb] = mfma_mx(l0, l1, b[u][nb], sal, sb, acc[nb]);
            }
        }
        if (bt == nbat - 1) {
            const int par = (it - i0) & 1;
            if (wv > 0) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) red[par][wv - 1][nb][lane] = acc[nb];
            }
            lds_barrier();
            if (wv == 0) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = ((acc[nb] + red[par][0][nb][lane]) + red[par][1][nb][lane]) + red[par][2][nb][lane];
                const int fcol = grp * 16 + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = g * 4 + r;
                    if (row < c_tl.nrows) {
                        float gv = acc[0][r], uv = acc[1][r];
                        if constexpr (NV) {
                            const float xr = rsc[row];
                            gv *= xr * gs[3 * c_tl.expert];
                            uv *= xr * gs[3 * c_tl.expert + 1];
                        }
                        h[(int64_t)(c_tl.row0 + row) * F + fcol] = f32_to_bf16(silu(gv) * uv);
                    }
                }
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
    };

    load(b0, s0, 0);
    if (total > 1) load(b1, s1, 1);
    for (int st = 0; st < total; st += 2) {
        consume(b0, s0, st);
        if (st + 2 < total) load(b0, s0, st + 2);
        if (st + 1 < total) {
            consume(b1, s1, st + 1);
            if (st + 3 < total) load(b1, s1, st + 3);
        }
    }
    store_route();
}

// =========================================================================
// Few tokens over many experts (decode at T >= 2 with E = 256, k = 8): the
// streaming gate/up kernel on whole weight tile columns.  An item is (tile,
// weight tile nt): the gate and up rows of 128 features over all of K.  The
// workgroup's 8 waves split it 4 x 2: wave w reads the gate and the up rows
// of 32 features (quarter w & 3: two 2 KB runs of the tile a chunk) over K
// half w >> 2, so the workgroup reads every 16 KB code tile and 1 KB scale
// tile of its column whole and the chip's loads stay close together in
// memory.  Measured on the address stream alone (no arithmetic), 540 MB at
// decode T=4: 83 us this way against 92 us for 16-feature items.  One chunk
// per batch, two batches in flight; with 4 row blocks a wave (116 VGPRs,
// four waves per SIMD) a chunk's MFMAs hide behind the stream better than
// with 8 on half as many waves (decode T=4 89.7 -> 86.8 us).  x's FP8 parts
// staged in LDS per tile (as gemm1_stream_kernel); the two K halves meet in
// LDS in a fixed order and the first half's waves write h.  Tiles of at most
// R rows.
// =========================================================================
template <bool ROUTE, bool NV>
__global__ __launch_bounds__(512) void gemm1_col_kernel(
    const uint8_t *__restrict__ ghi, const uint8_t *__restrict__ glo,
    const uint8_t *__restrict__ gsh, const uint8_t *__restrict__ gsl,
    int32_t *__restrict__ perm, Tile *__restrict__ tiles,
    int32_t *__restrict__ ntiles, const uint8_t *__restrict__ wpk,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ h, int d, int F, int k, int R,
    const float *__restrict__ gs, const RouteArgs ra)
{
    static_assert(!(NV && ROUTE), "the 16-block path reads the routing kernel's tile list");
    constexpr int NB = 4;  // row blocks a wave: 2 gate, then the same 2 up
    extern __shared__ uint4 xs4[];
    __shared__ floatx4_t red[2][4][NB][64];  // [item parity][row quarter][block][lane]
    // NV: the E4M3 table, the per-wave maxima of the row conversion and the
    // staged rows' scales (R <= 16, checked by the launcher)
    __shared__ uint2 lut[NV ? 256 : 1];
    __shared__ uint32_t wmax[8];
    __shared__ float rsc[NV ? 16 : 1];
    if constexpr (NV) fill_e4m3_table(lut);  // read after the first stage() barrier
    uint8_t *xs = reinterpret_cast<uint8_t *>(xs4);
    uint8_t *xhi = xs, *xlo = xs + (size_t)R * d;
    uint8_t *xsh = xs + (size_t)2 * R * d, *xsl = xsh + (size_t)R * (d / 32);

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int quarter = wv & 3, kh = wv >> 2;
    const int cols = F / 128;  // items per tile
    // ROUTE: the call's routing, computed here (route_few) instead of read
    __shared__ typename std::conditional<ROUTE, FewRoute, char>::type fr;
    if constexpr (ROUTE) route_few(ra.scores, ra.T, ra.E, k, R, fr);
    // workgroup 0 stores the routing for the later kernels when it is done
    auto store_route = [&]() {
        if constexpr (ROUTE)
            if (blockIdx.x == 0)
                route_few_store(fr, ra.T, ra.E, k, ra.ids, ra.wts, ra.counts, ra.offsets, perm, ra.inv, tiles,
                                ntiles);
    };
    auto tile_at = [&](int ti) -> Tile {
        if constexpr (ROUTE) return uniform_tile(fr.tiles[ti]);
        else return tiles[ti];
    };
    auto perm_at = [&](int row) -> int {
        if constexpr (ROUTE) return __builtin_amdgcn_readfirstlane(fr.perm[row]);
        else return perm[row];
    };
    int ntl;
    if constexpr (ROUTE) ntl = fr.ntiles;
    else ntl = *ntiles;
    const int64_t nitems = (int64_t)ntl * cols;
    const int i0 = (int)(nitems * blockIdx.x / gridDim.x);
    const int i1 = (int)(nitems * (blockIdx.x + 1) / gridDim.x);
    if (i0 >= i1) {
        store_route();
        return;
    }
    const int ch = d / kKStep / 2;  // chunks per K half
    const int total = (i1 - i0) * ch;
    // ---- weight loads: one chunk of the wave's 4 row blocks ----------------
    // row block i of quarter q: packed rows 128(q >> 1) + 32(q & 1) +
    // 64(i >> 1) + 16(i & 1) .. +15, i.e. feature 128nt + 64(q >> 1) +
    // 32(q & 1) + 16(i & 1) + n of the gate (i < 2) or up matrix
    uint4 b0[NB], b1[NB];
    uint32_t s0[NB], s1[NB];
    int l_ti = -1;
    Tile l_tl{0, 0, 0, 0};
    auto load = [&](uint4 (&b)[NB], uint32_t (&sv)[NB], int st) {
        const int it = i0 + st / ch, c = kh * ch + st % ch;
        const int ti = it / cols, nt = it - ti * cols;
        if (ti != l_ti) {
            l_tl = tile_at(ti);
            l_ti = ti;
        }
        const WView v = NV ? w1_codes(wpk, l_tl.expert, d, F) : w1_view(wpk, sc, l_tl.expert, d, F);
        const NvScales vs = w1_nv_scales(sc, l_tl.expert, d, F);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int rho = 128 * (quarter >> 1) + 32 * (quarter & 1) + 64 * (i >> 1) + 16 * (i & 1) + n;
            b[i] = ld_stream16(v.slot(nt, c, rho, g));
            if constexpr (NV) sv[i] = __builtin_nontemporal_load(vs.pair(nt, c, rho, g));
            else sv[i] = ld_stream4(v.scales(nt, c, rho));
        }
    };
    // ---- activation staging: the tile's FP8 rows and scales -> LDS --------
    int c_ti = -1;
    Tile c_tl{0, 0, 0, 0};
    auto stage = [&](int ti) {
        c_tl = tile_at(ti);
        c_ti = ti;
        const int q = d / 16, qs = d / 32 / 16;  // 16-byte units per part row / scale row
        if constexpr (NV) {
            // the bf16 rows (ghi) converted here (f16_row_block) into fp16
            // rows of 2d bytes, the space of both FP8 parts, with their scales
            for (int r = 0; r < c_tl.nrows; ++r) {
                const int64_t tok = perm_at(c_tl.row0 + r) / k;
                const float scr = f16_row_block(reinterpret_cast<const uint4 *>(ghi + tok * 2 * d),
                                                reinterpret_cast<uint4 *>(xs + (size_t)r * 2 * d), 2 * q, wmax);
                if (threadIdx.x == 0) rsc[r] = scr;
            }
            lds_barrier();
            return;
        }
        for (int r = 0; r < c_tl.nrows; ++r) {
            const int64_t tok = perm_at(c_tl.row0 + r) / k;
            const uint4 *sh = reinterpret_cast<const uint4 *>(ghi + tok * d);
            const uint4 *sl = reinterpret_cast<const uint4 *>(glo + tok * d);
            uint4 *dh = reinterpret_cast<uint4 *>(xhi + (size_t)r * d);
            uint4 *dl = reinterpret_cast<uint4 *>(xlo + (size_t)r * d);
            for (int j = threadIdx.x; j < q; j += (int)blockDim.x) {
                dh[j] = sh[j];
                dl[j] = sl[j];
            }
            const uint4 *ssh = reinterpret_cast<const uint4 *>(gsh + tok * (d / 32));
            const uint4 *ssl = reinterpret_cast<const uint4 *>(gsl + tok * (d / 32));
            if ((int)threadIdx.x < qs) {
                reinterpret_cast<uint4 *>(xsh + (size_t)r * (d / 32))[threadIdx.x] = ssh[threadIdx.x];
                reinterpret_cast<uint4 *>(xsl + (size_t)r * (d / 32))[threadIdx.x] = ssl[threadIdx.x];
            }
        }
        lds_barrier();
    };
    floatx4_t acc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const uint4 (&b)[NB], const uint32_t (&sv)[NB], int st) {
        const int it = i0 + st / ch, bt = st % ch;
        const int ti = it / cols, nt = it - ti * cols;
        // a new tile's rows replace the old ones: every wave has passed the
        // previous item's barrier, so no wave still reads them
        if (ti != c_ti) stage(ti);
        const int m = n < c_tl.nrows ? n : 0;  // rows past nrows are computed on row 0, never stored
        const int c = kh * ch + bt;
        if constexpr (NV) {
            // the lane's 32 fp16 activations of K block g; four fp16 MFMAs
            // per row block on the weights expanded through the table
            const uint4 *ap = reinterpret_cast<const uint4 *>(xs + (size_t)m * 2 * d) + c * (kKStep / 8) + g * 4;
            const uint4 a[4] = {ap[0], ap[1], ap[2], ap[3]};
#pragma unroll
            for (int i = 0; i < NB; ++i) acc[i] = mfma_chunk_nv(a, b[i], sv[i], lut, acc[i]);
        } else {
            const uint4 *hp = reinterpret_cast<const uint4 *>(xhi + (size_t)m * d + c * kKStep);
            const uint4 *lp = reinterpret_cast<const uint4 *>(xlo + (size_t)m * d + c * kKStep);
            const uint4 h0 = hp[g], h1 = hp[4 + g], l0 = lp[g], l1 = lp[4 + g];
            const int sidx = m * (d / 32) + c * 4 + g;
            const uint32_t sah = xsh[sidx], sal = xsl[sidx];
            // all hi products, then all lo products: no MFMA waits on the one
            // before it (each block still adds hi before lo)
            uint32_t sb[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                sb[i] = (sv[i] >> (8 * g)) & 0xFFu;
                acc[i] = mfma_mx(h0, h1, b[i], sah, sb[i], acc[i]);
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) acc[i] = mfma_mx(l0, l1, b[i], sal, sb[i], acc[i]);
        }
        if (bt == ch - 1) {
            // the item's two K halves meet: the second writes, the first adds
            // (one order) and stores h = silu(gate) * up
            const int par = (it - i0) & 1;
            if (kh == 1) {
#pragma unroll
                for (int i = 0; i < NB; ++i) red[par][quarter][i][lane] = acc[i];
            }
            lds_barrier();
            if (kh == 0) {
#pragma unroll
                for (int i = 0; i < NB; ++i) acc[i] += red[par][quarter][i][lane];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int fcol = nt * 128 + 64 * (quarter >> 1) + 32 * (quarter & 1) + 16 * q + n;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = g * 4 + r;
                        if (row < c_tl.nrows) {
                            float gv = acc[q][r], uv = acc[q + 2][r];
                            if constexpr (NV) {
                                const float xr = rsc[row];
                                gv *= xr * gs[3 * c_tl.expert];
                                uv *= xr * gs[3 * c_tl.expert + 1];
                            }
                            h[(int64_t)(c_tl.row0 + row) * F + fcol] = f32_to_bf16(silu(gv) * uv);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < NB; ++i) acc[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
    };

    // total is even (d % 512 = 0: an even number of chunks per K half), so
    // every load is unconditional (past the end they re-read chunk total - 1):
    // with the same loads on every path the compiler's waits before a chunk's
    // MFMAs leave the other buffer's loads in flight; a skipped load on one
    // path made every chunk wait for both buffers
    const int last = total - 1;
    load(b0, s0, 0);
    load(b1, s1, 1);
    for (int st = 0; st < total; st += 2) {
        consume(b0, s0, st);
        load(b0, s0, min(st + 2, last));
        consume(b1, s1, st + 1);
        load(b1, s1, min(st + 3, last));
    }
    store_route();
}

// Workgroups that fit on the device at once for a kernel of `threads`
// threads with `lds` bytes of dynamic LDS (0 on error).  Queried on every call: nothing
// is cached, so the library keeps no state between calls.
static int persistent_grid(const void *kfn, size_t lds, int threads = 256)
{
    int dev = 0, per_cu = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, threads, lds) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return per_cu * cus;
}

// ---- launchers ----------------------------------------------------------------

// The streaming gate/up kernels (few tokens): whole tile columns when there
// are enough of them for the device and the kernel's larger LDS fits, else
// 16-feature items.  ROUTE: the kernel routes in its prologue.
template <bool ROUTE>
static hipError_t launch_stream_gate_up(const Shape &s, const Plan &p, const Workspace &ws,
                                        const uint8_t *wpk, const uint8_t *sc, const RouteArgs &ra,
                                        hipStream_t st, hipEvent_t ev0, hipEvent_t ev1)
{
    const int R = p.tile_rows;
    const size_t lds = (size_t)R * (2 * s.d + 2 * (s.d / 32));
    const int cgrid = stream_columns(s)
                          ? persistent_grid(reinterpret_cast<const void *>(gemm1_col_kernel<ROUTE, false>), lds, 512)
                          : 0;
    if (cgrid > 0) {
        hipExtLaunchKernelGGL(gemm1_col_kernel<ROUTE, false>, dim3(cgrid), dim3(512), (uint32_t)lds, st, ev0, ev1,
                              0, (const uint8_t *)ws.xhi, (const uint8_t *)ws.xlo, (const uint8_t *)ws.xshi,
                              (const uint8_t *)ws.xslo, ws.perm, ws.tiles, ws.ntiles, wpk, sc, ws.h, s.d,
                              s.F, s.k, R, (const float *)nullptr, ra);
        return hipGetLastError();
    }
    // a refused occupancy query must not surface as this launch's error
    if (stream_columns(s)) (void)hipGetLastError();
    auto kfn = gemm1_stream_kernel<kG1StreamU, false, ROUTE>;
    const int grid = persistent_grid(reinterpret_cast<const void *>(kfn), lds);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    hipExtLaunchKernelGGL(kfn, dim3(grid), dim3(256), (uint32_t)lds, st, ev0, ev1, 0,
                          (const uint8_t *)ws.xhi, (const uint8_t *)ws.xlo, (const uint8_t *)ws.xshi,
                          (const uint8_t *)ws.xslo, ws.perm, ws.tiles, ws.ntiles, wpk, sc, ws.h, s.d, s.F,
                          s.k, R, (const float *)nullptr, (const float *)nullptr, ra);
    return hipGetLastError();
}

hipError_t launch_gemm1(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                        const uint8_t *wpk, const uint8_t *sc, hipStream_t st, hipEvent_t ev0,
                        hipEvent_t ev1)
{
    if (p.tiled) {
        // x was split in the router stage (launch_split_x): FP6 records for
        // the wide kernel, FP8 parts otherwise
        // workgroups and their items as the tile-list code scheduled them
        if (!ws.sched || p.grid1 <= 0) return hipErrorInvalidValue;
        MxArgs pa{ws.xhi, ws.xlo, ws.xshi, ws.xslo, ws.xa6, ws.perm, ws.tiles, ws.sched, ws.ntiles, wpk,
                  sc, ws.h, nullptr, s.d, s.F, s.k, p.ntn1, nullptr};
        const dim3 grid((unsigned)p.grid1);
        if (wide_gate_up(s)) {
            // h goes straight to the down kernel's FP6 records when that kernel is wide
            if (wide_down(s)) pa.h6 = ws.ha6;
            if (p.tile_rows == 64)
                hipExtLaunchKernelGGL(gemm_mxw_kernel<true, 64>, grid, dim3(512), 0, st, ev0, ev1, 0, pa);
            else
                hipExtLaunchKernelGGL(gemm_mxw_kernel<true, 128>, grid, dim3(512), 0, st, ev0, ev1, 0, pa);
        } else {
            hipExtLaunchKernelGGL(gemm_mx_kernel<true>, grid, dim3(512), 0, st, ev0, ev1, 0, pa);
        }
    } else if (p.stream) {
        const RouteArgs ra{ws.scores, s.T, s.E, ws.ids, ws.wts, ws.counts, ws.offsets, ws.inv};
        return p.fuse_route ? launch_stream_gate_up<true>(s, p, ws, wpk, sc, ra, st, ev0, ev1)
                            : launch_stream_gate_up<false>(s, p, ws, wpk, sc, ra, st, ev0, ev1);
    } else {
        const int groups = s.F / 16;
        const int64_t grid = max_tiles(s, p.tile_rows) * groups;
        // a tile holds at most min(T, 16) rows (a token picks an expert once)
        int rows_fit = kDecodeLdsBytes / (s.d * 2);
        rows_fit = rows_fit < s.T ? rows_fit : s.T;
        if (rows_fit > 16) rows_fit = 16;
        const size_t lds = (size_t)rows_fit * s.d * 2;
        hipExtLaunchKernelGGL(gemm1_decode_kernel<kUnroll, false>, dim3((unsigned)grid), dim3(256),
                              (uint32_t)lds, st, ev0, ev1, 0, x, (const int32_t *)ws.perm,
                              (const Tile *)ws.tiles, (const int32_t *)ws.ntiles, wpk, sc, ws.h,
                              s.d, s.F, s.k, groups, rows_fit, (const float *)nullptr,
                              (const float *)nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_gemm2(const Shape &s, const Plan &p, const Workspace &ws, const uint8_t *wpk,
                        const uint8_t *sc, hipStream_t st)
{
    if (p.tiled) {
        // h records were written by the wide gate/up kernel; otherwise split h here
        hipError_t e = hipSuccess;
        if (!wide_down(s)) e = launch_split(ws.h, s.S(), s.F, ws.hhi, ws.hlo, ws.hshi, ws.hslo, st);
        else if (!wide_gate_up(s)) e = launch_split6(ws.h, s.S(), s.F, ws.ha6, st);
        if (e != hipSuccess) return e;
        MxArgs pa{ws.hhi, ws.hlo, ws.hshi, ws.hslo, ws.ha6, nullptr, ws.tiles, nullptr, ws.ntiles, wpk,
                  sc, ws.o, ws.ssq, s.d, s.F, s.k, wide_down(s) ? s.d / 512 : s.d / 256, nullptr};
        const int64_t grid = 8 * ((max_tiles(s, p.tile_rows) * pa.ntn + 7) / 8);
        if (wide_down(s) && p.tile_rows == 64) gemm_mxw_kernel<false, 64><<<(unsigned)grid, 512, 0, st>>>(pa);
        else if (wide_down(s)) gemm_mxw_kernel<false, 128><<<(unsigned)grid, 512, 0, st>>>(pa);
        else gemm_mx_kernel<false><<<(unsigned)grid, 512, 0, st>>>(pa);
    } else {
        const int wgs = s.d / 64;
        const int64_t grid = max_tiles(s, p.tile_rows) * wgs;
        int rows_fit = kDecodeLdsBytes / (s.F * 2);
        rows_fit = rows_fit < s.T ? rows_fit : s.T;
        if (rows_fit > 16) rows_fit = 16;
        const size_t lds = (size_t)rows_fit * s.F * 2;
        gemm2_decode_kernel<kDownU, false, 2><<<(unsigned)grid, 512, lds, st>>>(
            ws.h, ws.perm, ws.tiles, ws.ntiles, wpk, sc, ws.o, ws.ssq, s.d, s.F, wgs, rows_fit,
            nullptr, nullptr, false);
    }
    return hipGetLastError();
}

// ---- the 16-block format --------------------------------------------------------

// x was converted to fp16 rows (ws.xhi) with scales (ws.xshi) after the router.
hipError_t launch_gemm1_nv(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                           const uint8_t *wpk, const uint8_t *sc, const float *gs, hipStream_t st,
                           hipEvent_t ev0, hipEvent_t ev1)
{
    const uint16_t *x16 = reinterpret_cast<const uint16_t *>(ws.xhi);
    const float *xs = reinterpret_cast<const float *>(ws.xshi);
    if (p.tiled) {
        if (!ws.sched || p.grid1 <= 0) return hipErrorInvalidValue;
        NvArgs pa{x16, xs, ws.perm, ws.tiles, ws.sched, ws.ntiles, wpk, sc, gs, ws.h, nullptr,
                  s.d, s.F, s.k, p.ntn1};
        hipExtLaunchKernelGGL(gemm_nv_kernel<true>, dim3((unsigned)p.grid1), dim3(512), 0, st,
                              ev0, ev1, 0, pa);
    } else if (p.stream) {
        // the persistent streaming kernel: it converts the bf16 x rows of a
        // tile into fp16 as it stages them (in the space of the FP8 parts)
        const int R = p.tile_rows;
        if (R > 16) return hipErrorInvalidConfiguration;
        const size_t lds = (size_t)R * (2 * s.d + 2 * (s.d / 32));
        const uint8_t *xb = reinterpret_cast<const uint8_t *>(x);
        // whole tile columns when there are enough of them and the LDS fits
        // (as for MXFP4 weights), else 16-feature items
        const int cgrid = stream_columns(s)
                              ? persistent_grid(reinterpret_cast<const void *>(gemm1_col_kernel<false, true>), lds, 512)
                              : 0;
        if (cgrid > 0) {
            hipExtLaunchKernelGGL(gemm1_col_kernel<false, true>, dim3(cgrid), dim3(512), (uint32_t)lds, st, ev0,
                                  ev1, 0, xb, xb, xb, xb, ws.perm, ws.tiles, ws.ntiles, wpk, sc, ws.h, s.d, s.F,
                                  s.k, R, gs, RouteArgs{});
            return hipGetLastError();
        }
        if (stream_columns(s)) (void)hipGetLastError();
        auto kfn = gemm1_stream_kernel<kG1StreamU, true, false>;
        const int grid = persistent_grid(reinterpret_cast<const void *>(kfn), lds);
        if (grid <= 0) return hipErrorInvalidConfiguration;
        hipExtLaunchKernelGGL(kfn, dim3(grid), dim3(256), (uint32_t)lds, st, ev0, ev1, 0, xb, xb, xb,
                              xb, ws.perm, ws.tiles, ws.ntiles, wpk, sc, ws.h, s.d, s.F, s.k, R, xs, gs,
                              RouteArgs{});
    } else {
        const int groups = s.F / 16;
        const int64_t grid = max_tiles(s, p.tile_rows) * groups;
        int rows_fit = kDecodeLdsBytes / (s.d * 2);
        rows_fit = rows_fit < s.T ? rows_fit : s.T;
        if (rows_fit > 16) rows_fit = 16;
        const size_t lds = (size_t)rows_fit * s.d * 2;
        hipExtLaunchKernelGGL(gemm1_decode_kernel<kUnroll, true>, dim3((unsigned)grid), dim3(256),
                              (uint32_t)lds, st, ev0, ev1, 0, x16, (const int32_t *)ws.perm,
                              (const Tile *)ws.tiles, (const int32_t *)ws.ntiles, wpk, sc, ws.h,
                              s.d, s.F, s.k, groups, rows_fit, xs, gs);
    }
    return hipGetLastError();
}

// h (bf16, from the gate/up kernel) -> fp16 rows + scales, then the down product.
hipError_t launch_gemm2_nv(const Shape &s, const Plan &p, const Workspace &ws, const uint8_t *wpk,
                           const uint8_t *sc, const float *gs, hipStream_t st)
{
    uint16_t *h16 = reinterpret_cast<uint16_t *>(ws.hhi);
    float *hs = reinterpret_cast<float *>(ws.hshi);
    // few-row tiles hold at most min(T, tile_rows) rows (a token picks an
    // expert once); when they fit in kNvFuseLds the down kernel converts h
    // itself, else h is converted first
    const int mr = s.T < p.tile_rows ? s.T : p.tile_rows;
    const bool fuse = !p.tiled && mr <= 16 && (size_t)mr * s.F * 2 <= kNvFuseLds;
    if (!fuse) {
        const hipError_t e = launch_f16_rows(ws.h, s.S(), s.F, h16, hs, st);
        if (e != hipSuccess) return e;
    }
    if (p.tiled) {
        NvArgs pa{h16, hs, nullptr, ws.tiles, nullptr, ws.ntiles, wpk, sc, gs, ws.o, ws.ssq,
                  s.d, s.F, s.k, s.d / 256};
        const int64_t grid = 8 * ((max_tiles(s, p.tile_rows) * pa.ntn + 7) / 8);
        gemm_nv_kernel<false><<<(unsigned)grid, 512, 0, st>>>(pa);
    } else {
        const int wgs = s.d / 64;
        const int64_t grid = max_tiles(s, p.tile_rows) * wgs;
        int rows_fit = kDecodeLdsBytes / (s.F * 2);
        rows_fit = rows_fit < s.T ? rows_fit : s.T;
        if (rows_fit > 16) rows_fit = 16;
        if (fuse) rows_fit = mr;
        const size_t lds = (size_t)rows_fit * s.F * 2;
        gemm2_decode_kernel<kUnroll, true><<<(unsigned)grid, 256, lds, st>>>(
            fuse ? ws.h : h16, ws.perm, ws.tiles, ws.ntiles, wpk, sc, ws.o, ws.ssq, s.d, s.F, wgs,
            rows_fit, hs, gs, fuse);
    }
    return hipGetLastError();
}

}  // namespace moe
