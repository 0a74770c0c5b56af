// expert.hip -- the grouped expert FFN on MXFP4 weights.
//
// "Muse Spark Open を段階的に分解する" (animemo.app):
//   section ⑨  each expert is a gate, an up and a down matrix; gate decides
//              what passes, up how much, down maps back to the token width
//              (here SwiGLU: h = silu(g) * u, o = h W_down^T);
//   section ⑪  the weights are 4-bit values sharing a small scale per block
//              and are expanded to BF16 for the multiply (here the gfx950
//              scaled convert expands FP4 E2M1 x E8M0 straight into bf16
//              MFMA operands in registers);
//   section ⑬  below ~58 tokens per expert the time is the weight read, above
//              it the multiply: the decode kernels are built to keep weight
//              bytes in flight, the tiled kernels to keep the MFMA pipe busy.
//
// Operand layout shared by every kernel here (mfma 16x16x32 bf16): lane l
// holds A[m = l%16][k] and B[k][n = l%16] for the 8 k of k-group l/16 and
// step s: k = 32*(l/16) + 8*s + [0..8) inside a 128-wide K chunk.  So one
// 16-byte weight load per lane is exactly one 32-element scale block, and
// four MFMA steps consume it.  The order of k inside the instruction does not
// matter because A and B use the same map.
#include "device.h"
#include "internal.h"

namespace moe {

constexpr int kKStep = 128;  // K elements per chunk
constexpr int kUnroll = 4;   // chunks in flight per wave (decode kernels)

__device__ __forceinline__ floatx4_t mfma_chunk(const uint4 *a, uint4 b, float scale, floatx4_t acc)
{
    acc = mfma16(as_bf16x8(a[0]), fp4x8_to_bf16(b.x, scale), acc);
    acc = mfma16(as_bf16x8(a[1]), fp4x8_to_bf16(b.y, scale), acc);
    acc = mfma16(as_bf16x8(a[2]), fp4x8_to_bf16(b.z, scale), acc);
    acc = mfma16(as_bf16x8(a[3]), fp4x8_to_bf16(b.w, scale), acc);
    return acc;
}

// =========================================================================
// Decode kernels: tiles of <= 16 grouped rows, weights streamed once.
//
// The tile's activation rows (usually 1-4 valid rows) are copied once into
// LDS when they fit (rows_fit rows); each lane then reads its A fragment
// from LDS instead of issuing per-chunk global loads, so the vector-memory
// path carries almost only weight bytes.  Each wave streams NB blocks of 16
// weight rows with U chunks of loads in flight.
// =========================================================================

// gate/up: a workgroup owns 16*NBP features (NBP gate blocks + the NBP up
// blocks of the same features); its 4 waves take quarters of the K chunks and
// their partial sums are added in LDS in a fixed order.
template <int NBP, int U>
__global__ __launch_bounds__(256) void gemm1_decode_kernel(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ perm,
    const Tile *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    const uint8_t *__restrict__ wpk, const uint8_t *__restrict__ sc, uint16_t *__restrict__ h,
    int d, int F, int k, int groups, int rows_fit)
{
    constexpr int NB = 2 * NBP;
    extern __shared__ uint4 arows[];  // [rows_fit][d/8]
    __shared__ floatx4_t red[3][NB][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t tile = blockIdx.x / groups;
    const int grp = (int)(blockIdx.x % groups);
    if (tile >= *ntiles) return;
    const Tile tl = tiles[tile];
    const int n = lane & 15, g = lane >> 4;
    const int fbase = grp * 16 * NBP;
    const int64_t ebytes = (int64_t)3 * d * F / 2, escales = (int64_t)3 * d * F / 32;
    const uint8_t *bp[NB];
    const uint32_t *sp[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int f = fbase + 16 * (nb % NBP) + n;
        const int64_t row = nb < NBP ? f : F + f;
        bp[nb] = wpk + tl.expert * ebytes + row * (d / 2) + g * 16;
        sp[nb] = reinterpret_cast<const uint32_t *>(sc + tl.expert * escales + row * (d / 32));
    }
    const bool valid = n < tl.nrows;
    const bool use_lds = tl.nrows <= rows_fit;
    const int rowq = d / 8;  // 16-byte units per activation row
    const int nc = d / kKStep;
    const int c_begin = wv * nc / 4, c_end = (wv + 1) * nc / 4;
    // first batch of weight loads goes out before the activations are staged
    uint4 b[U][NB];
    uint32_t sw[U][NB];
    // scale words: one 16-byte load covers 4 chunks when rows and batches align
    const bool svec = U == 4 && (d / 32) % 16 == 0 && c_begin % 4 == 0;
    auto load_b = [&](int c) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c + u < c_end) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    b[u][nb] = *reinterpret_cast<const uint4 *>(bp[nb] + (int64_t)(c + u) * (kKStep / 2));
            }
        if (svec && c + U <= c_end) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const uint4 v = *reinterpret_cast<const uint4 *>(sp[nb] + c);
                sw[0][nb] = v.x;
                sw[1 % U][nb] = v.y;
                sw[2 % U][nb] = v.z;
                sw[3 % U][nb] = v.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c + u < c_end) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) sw[u][nb] = sp[nb][c + u];
                }
        }
    };
    load_b(c_begin);
    if (use_lds) {
        for (int q = threadIdx.x; q < tl.nrows * rowq; q += 256) {
            const int r = q / rowq, c = q - r * rowq;
            const int tok = perm[tl.row0 + r] / k;
            arows[q] = *reinterpret_cast<const uint4 *>(x + (int64_t)tok * d + c * 8);
        }
        __syncthreads();
    }
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
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = mfma_chunk(a, b[u][nb], e8m0_to_f32((sw[u][nb] >> (8 * g)) & 0xFFu),
                                         acc[nb]);
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
    // lane holds C[g*4 + r][n] of every block; gate block nb pairs with up block nb + NBP
#pragma unroll
    for (int nb = 0; nb < NBP; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = g * 4 + r;
            if (row < tl.nrows)
                h[(int64_t)(tl.row0 + row) * F + fbase + 16 * nb + n] =
                    f32_to_bf16(silu(acc[nb][r]) * acc[nb + NBP][r]);
        }
}

// down: a workgroup owns 64*NB output columns, NB 16-column blocks per wave,
// each wave runs all of K.  The tile's h rows (contiguous in the grouped
// order) are copied to LDS when they fit.  Epilogue: bf16 o and the sum of o^2
// over each 16-column block.
template <int NB, int U>
__global__ __launch_bounds__(256) void gemm2_decode_kernel(
    const uint16_t *__restrict__ h, const Tile *__restrict__ tiles,
    const int32_t *__restrict__ ntiles, const uint8_t *__restrict__ wpk,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ o, float *__restrict__ ssq, int d,
    int F, int wgs_per_tile, int rows_fit)
{
    extern __shared__ uint4 arows[];  // [rows_fit][F/8]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t tile = blockIdx.x / wgs_per_tile;
    const int blk0 = ((int)(blockIdx.x % wgs_per_tile) * 4 + wv) * NB;
    if (tile >= *ntiles) return;
    const Tile tl = tiles[tile];
    const int n = lane & 15, g = lane >> 4;
    const int64_t ebytes = (int64_t)3 * d * F / 2, escales = (int64_t)3 * d * F / 32;
    const uint8_t *bp[NB];
    const uint32_t *sp[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t row = (int64_t)(blk0 + nb) * 16 + n;
        bp[nb] = wpk + tl.expert * ebytes + (int64_t)2 * F * (d / 2) + row * (F / 2) + g * 16;
        sp[nb] = reinterpret_cast<const uint32_t *>(sc + tl.expert * escales +
                                                    (int64_t)2 * F * (d / 32) + row * (F / 32));
    }
    const bool valid = n < tl.nrows;
    const bool use_lds = tl.nrows <= rows_fit;
    const int rowq = F / 8;
    const int nc = F / kKStep;
    uint4 b[U][NB];
    uint32_t sw[U][NB];
    const bool svec = U == 4 && (F / 32) % 16 == 0;
    auto load_b = [&](int c) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c + u < nc) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    b[u][nb] = *reinterpret_cast<const uint4 *>(bp[nb] + (int64_t)(c + u) * (kKStep / 2));
            }
        if (svec && c + U <= nc) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const uint4 v = *reinterpret_cast<const uint4 *>(sp[nb] + c);
                sw[0][nb] = v.x;
                sw[1 % U][nb] = v.y;
                sw[2 % U][nb] = v.z;
                sw[3 % U][nb] = v.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (c + u < nc) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) sw[u][nb] = sp[nb][c + u];
                }
        }
    };
    load_b(0);
    if (use_lds) {
        const uint4 *src = reinterpret_cast<const uint4 *>(h + (int64_t)tl.row0 * F);
        for (int q = threadIdx.x; q < tl.nrows * rowq; q += 256) arows[q] = src[q];
        __syncthreads();
    }
    const uint16_t *ap = h + (int64_t)(tl.row0 + (valid ? n : 0)) * F + g * 32;
    const uint4 *al = arows + n * rowq + g * 4;

    floatx4_t acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nc; c += U) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c + u < nc) {
                uint4 a[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (!valid) a[s] = make_uint4(0, 0, 0, 0);
                    else if (use_lds) a[s] = al[(c + u) * (kKStep / 8) + s];
                    else a[s] = *reinterpret_cast<const uint4 *>(ap + (c + u) * kKStep + s * 8);
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = mfma_chunk(a, b[u][nb], e8m0_to_f32((sw[u][nb] >> (8 * g)) & 0xFFu),
                                         acc[nb]);
            }
        if (c + U < nc) load_b(c + U);
    }
    // sum of o^2 over the workgroup's 64*NB columns: per wave over its blocks
    // (DPP within 16-lane rows), then the four waves in LDS in a fixed order
    __shared__ float wsum[4][16];
    const int P = d / (64 * NB);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float ss = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float v = acc[nb][r];
            ss += v * v;
            const int row = g * 4 + r;
            if (row < tl.nrows)
                o[(int64_t)(tl.row0 + row) * d + (blk0 + nb) * 16 + n] = f32_to_bf16(v);
        }
        ss = sum16(ss);
        if (n == 0) wsum[wv][g * 4 + r] = ss;
    }
    __syncthreads();
    if (threadIdx.x < 16 && (int)threadIdx.x < tl.nrows) {
        const int row = threadIdx.x;
        const float t = (wsum[0][row] + wsum[1][row]) + (wsum[2][row] + wsum[3][row]);
        ssq[(int64_t)(tl.row0 + row) * P + (int)(blockIdx.x % wgs_per_tile)] = t;
    }
}

// =========================================================================
// Tiled kernels: tiles of <= 128 grouped rows.  The workgroup stages A
// (128 rows x 128 K, bf16) through LDS, double-buffered, with an XOR swizzle
// of the 16-byte slots so the MFMA fragment reads are conflict-free; every
// wave reads its own weight rows straight from HBM/L2 into registers and
// covers all 128 rows x 64 columns.  Workgroup w runs on XCD w % 8; tiles are
// handed out in contiguous ranges per XCD so neighbouring tiles (same rows,
// same expert) share that XCD's L2.
// =========================================================================
#ifndef MOE_TILED_WAVES
#define MOE_TILED_WAVES 2
#endif
constexpr int kTM = 128;                // rows per tile
constexpr int kSlots = kKStep / 8;      // 16-byte slots per A row per chunk
constexpr int kMB = kTM / 16;           // 16-row MFMA blocks per tile

// Contiguous per-XCD tile ranges; returns false for surplus workgroups.
__device__ __forceinline__ bool xcd_tile(int total, int &idx)
{
    const int per = (total + 7) >> 3;
    const int local = (int)(blockIdx.x >> 3);
    if (local >= per) return false;
    idx = (int)(blockIdx.x & 7) * per + local;
    return idx < total;
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MOE_TILED_WAVES, MOE_TILED_WAVES))) void gemm_tiled_kernel(
    const uint16_t *__restrict__ act, const int32_t *__restrict__ perm,
    const Tile *__restrict__ tiles, const int32_t *__restrict__ ntiles,
    const uint8_t *__restrict__ wpk, const uint8_t *__restrict__ sc,
    uint16_t *__restrict__ out, float *__restrict__ ssq, int d, int F, int k, int ntn)
{
    __shared__ uint4 As[2][kTM * kSlots];  // 64 KB
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int idx;
    if (!xcd_tile(*ntiles * ntn, idx)) return;
    const int mt = idx / ntn, nt = idx - mt * ntn;
    const Tile tl = tiles[mt];
    const int mb_act = (tl.nrows + 15) >> 4;
    const int K = GATE_UP ? d : F;            // contraction length
    const int row_elems = GATE_UP ? d : F;    // A row length
    const int64_t ebytes = (int64_t)3 * d * F / 2, escales = (int64_t)3 * d * F / 32;

    // A loader: thread copies 16-byte slot ac of rows ar + 16*i
    const int ar = tid >> 4, ac = tid & 15;
    int64_t aoff[kMB];
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        const int r = ar + 16 * i;
        if (r < tl.nrows) {
            const int64_t src = GATE_UP ? (int64_t)(perm[tl.row0 + r] / k) : (int64_t)(tl.row0 + r);
            aoff[i] = src * row_elems + ac * 8;
        } else {
            aoff[i] = -1;
        }
    }
    // B rows of this wave: 4 blocks of 16 columns
    const int n = lane & 15, g = lane >> 4;
    const uint8_t *bp[4];
    const uint8_t *sp[4];
    const uint8_t *eb = wpk + tl.expert * ebytes;
    const uint8_t *es = sc + tl.expert * escales;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        int64_t row;
        if (GATE_UP) {
            // nb 0,1: gate features f0+16*nb+n; nb 2,3: up rows of the same features
            const int f = nt * 128 + wv * 32 + (nb & 1) * 16 + n;
            row = nb < 2 ? f : F + f;
            bp[nb] = eb + row * (d / 2) + g * 16;
            sp[nb] = es + row * (d / 32) + g;
        } else {
            row = (int64_t)nt * 256 + wv * 64 + nb * 16 + n;
            bp[nb] = eb + (int64_t)2 * F * (d / 2) + row * (F / 2) + g * 16;
            sp[nb] = es + (int64_t)2 * F * (d / 32) + row * (F / 32) + g;
        }
    }

    floatx4_t acc[kMB][4];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = K / kKStep;
    uint4 areg[kMB];
    uint4 b[4];
    uint32_t sb[4];
    auto load_a = [&](int kc) {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
            areg[i] = aoff[i] >= 0 ? *reinterpret_cast<const uint4 *>(act + aoff[i] + kc * kKStep)
                                   : make_uint4(0, 0, 0, 0);
    };
    auto store_a = [&](int stage) {
#pragma unroll
        for (int i = 0; i < kMB; ++i) As[stage][(ar + 16 * i) * kSlots + (ac ^ ar)] = areg[i];
    };
    load_a(0);
    store_a(0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        b[nb] = *reinterpret_cast<const uint4 *>(bp[nb]);
        sb[nb] = sp[nb][0];
    }
    for (int kc = 0; kc < nk; ++kc) {
        __syncthreads();
        uint4 bn[4];
        uint32_t sbn[4];
        const bool more = kc + 1 < nk;
        if (more) {
            load_a(kc + 1);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                bn[nb] = *reinterpret_cast<const uint4 *>(bp[nb] + (int64_t)(kc + 1) * (kKStep / 2));
                sbn[nb] = sp[nb][(kc + 1) * (kKStep / 32)];
            }
        }
        const uint4 *Ab = As[kc & 1];
        float scale[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) scale[nb] = e8m0_to_f32(sb[nb]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8_t bq[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const uint32_t w = s == 0 ? b[nb].x : s == 1 ? b[nb].y : s == 2 ? b[nb].z : b[nb].w;
                bq[nb] = fp4x8_to_bf16(w, scale[nb]);
            }
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) {
                if (mb < mb_act) {
                    const uint4 av = Ab[(mb * 16 + n) * kSlots + ((4 * g + s) ^ n)];
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[mb][nb] = mfma16(as_bf16x8(av), bq[nb], acc[mb][nb]);
                }
            }
        }
        if (more) {
            store_a((kc + 1) & 1);
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                b[nb] = bn[nb];
                sb[nb] = sbn[nb];
            }
        }
    }

    if (GATE_UP) {
        const int fbase = nt * 128 + wv * 32;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = mb * 16 + g * 4 + r;
                    if (row < tl.nrows)
                        out[(int64_t)(tl.row0 + row) * F + fbase + hb * 16 + n] =
                            f32_to_bf16(silu(acc[mb][hb][r]) * acc[mb][hb + 2][r]);
                }
        }
    } else {
        const int P = d / 64;
        const int pcol = nt * 4 + wv;
        const int cbase = nt * 256 + wv * 64;
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb) {
            if (mb >= mb_act) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mb * 16 + g * 4 + r;
                float ss = 0.f;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) ss += acc[mb][nb][r] * acc[mb][nb][r];
                ss = sum16(ss);
                if (row < tl.nrows) {
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        out[(int64_t)(tl.row0 + row) * d + cbase + nb * 16 + n] =
                            f32_to_bf16(acc[mb][nb][r]);
                    if (n == 0) ssq[(int64_t)(tl.row0 + row) * P + pcol] = ss;
                }
            }
        }
    }
}

// LDS budget for the decode kernels' staged activation rows.
#ifndef MOE_DEC_LDS
#define MOE_DEC_LDS (32 * 1024)
#endif
constexpr int kDecodeLdsBytes = MOE_DEC_LDS;
#ifndef MOE_G1NBP
#define MOE_G1NBP 1
#define MOE_G1U 4
#define MOE_G2NB 1  // the sum-of-squares partials assume 64 columns per workgroup
#define MOE_G2U 4
#endif
constexpr int kG1NBP = MOE_G1NBP, kG1U = MOE_G1U;  // gate/up decode: 16*NBP features per workgroup
constexpr int kG2NB = MOE_G2NB, kG2U = MOE_G2U;    // down decode: 64*NB columns per workgroup

hipError_t launch_gemm1(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                        const uint8_t *wpk, const uint8_t *sc, hipStream_t st)
{
    if (p.tiled) {
        const int ntn = s.F / 128;
        const int64_t grid = 8 * ((max_tiles(s, p.tile_rows) * ntn + 7) / 8);
        gemm_tiled_kernel<true><<<(unsigned)grid, 256, 0, st>>>(
            x, ws.perm, ws.tiles, ws.ntiles, wpk, sc, ws.h, nullptr, s.d, s.F, s.k, ntn);
    } else {
        const int groups = s.F / (16 * kG1NBP);
        const int64_t grid = max_tiles(s, p.tile_rows) * groups;
        // a tile holds at most min(T, 16) rows (a token picks an expert once)
        int rows_fit = kDecodeLdsBytes / (s.d * 2);
        rows_fit = rows_fit < s.T ? rows_fit : s.T;
        if (rows_fit > 16) rows_fit = 16;
        const size_t lds = (size_t)rows_fit * s.d * 2;
        gemm1_decode_kernel<kG1NBP, kG1U><<<(unsigned)grid, 256, lds, st>>>(
            x, ws.perm, ws.tiles, ws.ntiles, wpk, sc, ws.h, s.d, s.F, s.k, groups, rows_fit);
    }
    return hipGetLastError();
}

hipError_t launch_gemm2(const Shape &s, const Plan &p, const Workspace &ws, const uint8_t *wpk,
                        const uint8_t *sc, hipStream_t st)
{
    if (p.tiled) {
        const int ntn = s.d / 256;
        const int64_t grid = 8 * ((max_tiles(s, p.tile_rows) * ntn + 7) / 8);
        gemm_tiled_kernel<false><<<(unsigned)grid, 256, 0, st>>>(
            ws.h, nullptr, ws.tiles, ws.ntiles, wpk, sc, ws.o, ws.ssq, s.d, s.F, s.k, ntn);
    } else {
        const int wgs = s.d / (64 * kG2NB);
        const int64_t grid = max_tiles(s, p.tile_rows) * wgs;
        int rows_fit = kDecodeLdsBytes / (s.F * 2);
        rows_fit = rows_fit < s.T ? rows_fit : s.T;
        if (rows_fit > 16) rows_fit = 16;
        const size_t lds = (size_t)rows_fit * s.F * 2;
        gemm2_decode_kernel<kG2NB, kG2U><<<(unsigned)grid, 256, lds, st>>>(
            ws.h, ws.tiles, ws.ntiles, wpk, sc, ws.o, ws.ssq, s.d, s.F, wgs, rows_fit);
    }
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
