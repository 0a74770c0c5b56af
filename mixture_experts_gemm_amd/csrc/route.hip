// route.hip -- router scores, top-k with softmax weights, and the stable
// counting sort of token slots by expert.
//
// "Muse Spark Open を段階的に分解する" (animemo.app):
//   section ⑧  one matrix product of the token vector scores all experts, in
//              FP32; the 8 best are chosen, there is no shared expert;
//   section ⑨  the chosen experts' outputs are weighted by the router scores
//              (weights of a token sum to one: softmax over the chosen k);
//   section ⑫  tokens are batched per expert and each expert's tokens are
//              gathered and computed together (here: grouped order sorted by
//              (expert, token)).
//
// Grouping without order-dependent atomics: tokens are cut into chunks of
// 64; for every (chunk, expert) an LDS 64-bit mask records which tokens of
// the chunk chose the expert (atomic OR: the result does not depend on the
// order the ORs land in).  A slot's place inside its expert segment is then
// the segment base plus the popcount of the mask bits of earlier tokens.
#include "device.h"
#include "internal.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router scores, few tokens: one workgroup per expert streams that expert's
// fp32 router row; all tokens are accumulated in registers and reduced once.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t *__restrict__ x,
                                                          const float *__restrict__ wr,
                                                          float *__restrict__ scores, int T,
                                                          int d, int E, uint8_t *__restrict__ xhi,
                                                          uint8_t *__restrict__ xlo,
                                                          uint8_t *__restrict__ xsh,
                                                          uint8_t *__restrict__ xsl)
{
    // blockIdx.x < E: expert; blockIdx.y: group of NT tokens.  Every load of a
    // 8192-wide slice is issued before the first multiply-add.  When xhi is
    // set, workgroups blockIdx.x >= E split the group's x rows into FP8 hi/lo
    // parts for the expert kernels (one 32-block per thread), alongside the
    // dot products.
    constexpr int R = 8;  // float4 per thread per 8192-element slice
    __shared__ float part[4][NT];
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * NT;
    if (e >= E) {
        const int64_t nblk = (int64_t)min(NT, T - t0) * (d / 32);
        const int64_t j = (int64_t)(e - E) * 256 + threadIdx.x;
        if (xhi && j < nblk) {
            const int64_t b = (int64_t)t0 * (d / 32) + j;
            split_bf16_block(x + b * 32, xhi + b * 32, xlo + b * 32, xsh + b, xsl + b);
        }
        return;
    }
    const float *w = wr + (int64_t)e * d;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;
    for (int base = 0; base < d; base += 1024 * R) {
        float4 wq[R];
        uint2 xq[NT][R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = base + r * 1024 + threadIdx.x * 4;
            wq[r] = i < d ? *reinterpret_cast<const float4 *>(w + i) : make_float4(0, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int64_t tt = min(t0 + t, T - 1);  // clamped: rows past T are computed, not stored
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = base + r * 1024 + threadIdx.x * 4;
                xq[t][r] = i < d ? *reinterpret_cast<const uint2 *>(x + tt * d + i) : make_uint2(0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float a = acc[t];
                a = fmaf(__uint_as_float(xq[t][r].x << 16), wq[r].x, a);
                a = fmaf(__uint_as_float(xq[t][r].x & 0xFFFF0000u), wq[r].y, a);
                a = fmaf(__uint_as_float(xq[t][r].y << 16), wq[r].z, a);
                a = fmaf(__uint_as_float(xq[t][r].y & 0xFFFF0000u), wq[r].w, a);
                acc[t] = a;
            }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float v = wave_sum(acc[t]);
        if (lane == 0) part[wv][t] = v;
    }
    __syncthreads();
    if (threadIdx.x < NT && t0 + (int)threadIdx.x < T) {
        const int t = threadIdx.x;
        scores[(int64_t)(t0 + t) * E + e] = (part[0][t] + part[1][t]) + (part[2][t] + part[3][t]);
    }
}

// ---------------------------------------------------------------------------
// Router scores, many tokens: bf16 MFMA on an exact three-way bf16 split of
// the fp32 router weights.  w = hi + mid + lo exactly (truncating splits:
// each part keeps 8 significant bits of what is left), x is bf16, so every
// product is exact and the sum is accumulated in fp32 like an fp32 GEMM.
// A workgroup computes 128 tokens x 128 experts (256 x 64 when E <= 64)
// over one slice of d; its 4 waves take 64 x 64 each (4 x 4 MFMA blocks).
// Slice s writes its partial sums to part[s][T][E]; top-k adds the slices
// in order.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void split3_trunc(const float4 &a, const float4 &b, uint4 &hi, uint4 &mid,
                                             uint4 &lo)
{
    const float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t wb = __float_as_uint(w[i]);
        h[i] = wb & 0xFFFF0000u;
        const float r1 = w[i] - __uint_as_float(h[i]);
        m[i] = __float_as_uint(r1) & 0xFFFF0000u;
        l[i] = __float_as_uint(r1 - __uint_as_float(m[i]));  // <= 8 significant bits: exact in bf16
    }
    auto pk = [](uint32_t a0, uint32_t a1) { return (a0 >> 16) | (a1 & 0xFFFF0000u); };
    hi = make_uint4(pk(h[0], h[1]), pk(h[2], h[3]), pk(h[4], h[5]), pk(h[6], h[7]));
    mid = make_uint4(pk(m[0], m[1]), pk(m[2], m[3]), pk(m[4], m[5]), pk(m[6], m[7]));
    lo = make_uint4(pk(l[0], l[1]), pk(l[2], l[3]), pk(l[4], l[5]), pk(l[6], l[7]));
}

// The workgroup's operands are staged through LDS: each 32-wide K step of
// the tile's x rows (64 B a row) and router rows (128 B a row, fp32) is
// copied once by direct-to-LDS loads into a three-stage ring and read by
// every wave that needs it (16-byte slot q of an x row r at
// q ^ ((r >> 1) & 3), of a router row at q ^ (r & 7): the fragment reads of
// 16 consecutive rows then fall on distinct banks).  WE waves along the
// experts, 4/WE along the tokens.
template <int WE>
__global__ __launch_bounds__(256) void router_gemm_lds_kernel(const uint16_t *__restrict__ x,
                                                              const float *__restrict__ wr,
                                                              float *__restrict__ part, int T, int d,
                                                              int E, int kslice)
{
    constexpr int WT = 4 / WE;
    constexpr int TT = 64 * WT, TE = 64 * WE;        // tile tokens, tile experts
    constexpr int XU = TT * 4, WU = TE * 8;          // 16-byte units per stage
    constexpr int NL = (XU + WU) / 256;              // loads per thread per stage (6)
    __shared__ uint4 Xs[3][XU];
    __shared__ uint4 Ws[3][WU];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int T0 = blockIdx.x * TT, E0 = blockIdx.y * TE;
    const int k0 = blockIdx.z * kslice;
    const int nk = kslice / 32;
    // load j of this thread: unit u = 256 j + tid of the stage (x units first)
    const void *src[NL];
    uint32_t dst[NL];
    bool isx[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int u = 256 * j + tid;
        isx[j] = u < XU;
        if (u < XU) {
            const int r = u >> 2, p = u & 3, q = p ^ ((r >> 1) & 3);
            src[j] = x + (int64_t)min(T0 + r, T - 1) * d + k0 + q * 8;
        } else {
            const int v = u - XU, r = v >> 3, p = v & 7, q = p ^ (r & 7);
            src[j] = wr + (int64_t)min(E0 + r, E - 1) * d + k0 + q * 4;
        }
        dst[j] = (uint32_t)(256 * j + wv * 64);  // unit of lane 0 of this wave
    }
    auto issue = [&](int kc) {
        const int b = kc % 3;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const uint32_t base = isx[j] ? lds_off(&Xs[b][dst[j]]) : lds_off(&Ws[b][dst[j] - XU]);
            const int64_t off = isx[j] ? (int64_t)kc * 64 : (int64_t)kc * 128;
            dma16(static_cast<const uint8_t *>(src[j]) + off,
                   __builtin_amdgcn_readfirstlane(base));
        }
    };

    const int tr0 = (wv % WT) * 64, er0 = (wv / WT) * 64;  // the wave's rows inside the tile
    floatx4_t acc[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    issue(0);
    if (nk > 1) issue(1);
    for (int kc = 0; kc < nk; ++kc) {
        if (kc + 1 < nk) asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(NL) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        if (kc + 2 < nk) issue(kc + 2);
        const uint4 *X = Xs[kc % 3];
        const uint4 *W = Ws[kc % 3];
        uint4 a[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int r = tr0 + mb * 16 + m;
            a[mb] = X[r * 4 + (g ^ ((r >> 1) & 3))];
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int r = er0 + nb * 16 + m;
            const uint4 w0 = W[r * 8 + ((2 * g) ^ (r & 7))], w1 = W[r * 8 + ((2 * g + 1) ^ (r & 7))];
            uint4 hi, mid, lo;
            split3_trunc(__builtin_bit_cast(float4, w0), __builtin_bit_cast(float4, w1), hi, mid, lo);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const bf16x8_t av = as_bf16x8(a[mb]);
                acc[mb][nb] = mfma16(av, as_bf16x8(lo), acc[mb][nb]);
                acc[mb][nb] = mfma16(av, as_bf16x8(mid), acc[mb][nb]);
                acc[mb][nb] = mfma16(av, as_bf16x8(hi), acc[mb][nb]);
            }
        }
    }
    float *out = part + (int64_t)blockIdx.z * T * E;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = T0 + tr0 + mb * 16 + g * 4 + r, e = E0 + er0 + nb * 16 + m;
                if (t < T && e < E) out[(int64_t)t * E + e] = acc[mb][nb][r];
            }
}

hipError_t launch_router(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                         const float *wr, hipStream_t st)
{
    // the streaming gate/up kernel reads x as FP8 hi/lo parts, split alongside
    // the few-token router; the tiled kernels' split follows the router below
    uint8_t *xhi = p.stream ? ws.xhi : nullptr;
    if (s.T == 1) {
        const int xs = xhi ? (s.d / 32 + 255) / 256 : 0;  // split workgroups per token group
        router_gemv_kernel<1><<<s.E + xs, 256, 0, st>>>(x, wr, ws.scores, s.T, s.d, s.E, xhi, ws.xlo,
                                                        ws.xshi, ws.xslo);
    } else if (s.T <= 32) {
        const int xs = xhi ? (4 * (s.d / 32) + 255) / 256 : 0;
        router_gemv_kernel<4><<<dim3(s.E + xs, (s.T + 3) / 4), 256, 0, st>>>(
            x, wr, ws.scores, s.T, s.d, s.E, xhi, ws.xlo, ws.xshi, ws.xslo);
    } else {
        const int ks = router_splits(s);
        const int tt = router_tile_tokens(s.E), te = router_tile_experts(s.E);
        dim3 grid((s.T + tt - 1) / tt, (s.E + te - 1) / te, ks);
        if (te == 64)
            router_gemm_lds_kernel<1><<<grid, 256, 0, st>>>(x, wr, ws.scores, s.T, s.d, s.E, s.d / ks);
        else
            router_gemm_lds_kernel<2><<<grid, 256, 0, st>>>(x, wr, ws.scores, s.T, s.d, s.E, s.d / ks);
    }
    if (p.tiled) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_split_x(s, ws, x, st);
    }
    return hipGetLastError();
}

template <int SLOTS>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ scores,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ wts, int T, int E, int k,
                                                   int nsplit)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_row<SLOTS>(scores + (int64_t)t * E, E, k, ids + (int64_t)t * k, wts + (int64_t)t * k,
                    nullptr, lane, nsplit, (int64_t)T * E);
}

// ---------------------------------------------------------------------------
// Block-wide exclusive prefix sums of a[0..n) and b[0..n) together, n <= 1024,
// in LDS, by 256 threads (one pass, two barriers); returns both totals.
// Integer, so order-free.
// ---------------------------------------------------------------------------
// Inclusive prefix sums of a and b over the wave: shift-and-add steps by
// DPP row_shr inside rows of 16 lanes (lanes shifted in from outside the
// row read 0), then the totals of the earlier rows (lanes 15, 31, 47) added.
template <int N>
__device__ __forceinline__ int row_shr_add(int v)
{
    return v + __builtin_amdgcn_update_dpp(0, v, 0x110 + N, 0xF, 0xF, false);
}
__device__ __forceinline__ void wave_incl_scan2(int &a, int &b, int lane)
{
    a = row_shr_add<1>(a);
    b = row_shr_add<1>(b);
    a = row_shr_add<2>(a);
    b = row_shr_add<2>(b);
    a = row_shr_add<4>(a);
    b = row_shr_add<4>(b);
    a = row_shr_add<8>(a);
    b = row_shr_add<8>(b);
    const int a15 = __builtin_amdgcn_readlane(a, 15), a31 = __builtin_amdgcn_readlane(a, 31),
              a47 = __builtin_amdgcn_readlane(a, 47);
    const int b15 = __builtin_amdgcn_readlane(b, 15), b31 = __builtin_amdgcn_readlane(b, 31),
              b47 = __builtin_amdgcn_readlane(b, 47);
    const int row = lane >> 4;
    a += (row >= 1 ? a15 : 0) + (row >= 2 ? a31 : 0) + (row >= 3 ? a47 : 0);
    b += (row >= 1 ? b15 : 0) + (row >= 2 ? b31 : 0) + (row >= 3 ? b47 : 0);
}

__device__ int2 block_exclusive_scan2(int32_t *a, int32_t *b, int n, int32_t (*wtot)[4])
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int va[4], vb[4];
    int sa = 0, sb = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = tid * 4 + q;
        va[q] = i < n ? a[i] : 0;
        vb[q] = i < n ? b[i] : 0;
        sa += va[q];
        sb += vb[q];
    }
    int ia = sa, ib = sb;
    wave_incl_scan2(ia, ib, lane);
    if (lane == 63) {
        wtot[0][wv] = ia;
        wtot[1][wv] = ib;
    }
    __syncthreads();
    int basea = 0, baseb = 0;
    for (int w = 0; w < wv; ++w) {
        basea += wtot[0][w];
        baseb += wtot[1][w];
    }
    const int2 total = make_int2(wtot[0][0] + wtot[0][1] + wtot[0][2] + wtot[0][3],
                                 wtot[1][0] + wtot[1][1] + wtot[1][2] + wtot[1][3]);
    int ra = basea + ia - sa, rb = baseb + ib - sb;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = tid * 4 + q;
        if (i < n) {
            a[i] = ra;
            b[i] = rb;
        }
        ra += va[q];
        rb += vb[q];
    }
    __syncthreads();
    return total;
}

// The order in which the tiled gate/up kernel's workgroups take the tiles.
// Every workgroup handles one (tile, N-tile) item, described in full by
// out[workgroup] (SchedItem), so it starts with one load.  Items go
// longest first (experts by rows per tile, descending, then by id), an
// expert's items together and N-tile-major as in the tile list; the
// sequence is cut into runs of 2 * ntn items dealt to the XCDs as sched_pos
// describes.  So each XCD holds about an eighth of the work, an expert's
// items share an XCD's L2 (a run is two tiles' worth), and the last
// workgroups an XCD starts are its shortest: the tail of the launch is
// short.
struct Sched {
    SchedItem *out;  // null: not a tiled plan
    int ntn;         // workgroups per tile (weight-tile groups); runs of 2 * ntn items
};

// offsets / counts / tile list from per-expert counts cnt[] (LDS, E entries);
// cnt is replaced by the exclusive offsets.  With a schedule (sc.out set)
// also the tiled gate/up kernel's work order.
__device__ void finish_offsets(int32_t *cnt, int32_t *toff, int32_t (*wtot)[4], int E, int tile_rows,
                               int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                               Tile *__restrict__ tiles, int32_t *__restrict__ ntiles, int *c_out,
                               const Sched &sc)
{
    __shared__ int32_t skey[1024];   // expert -> rows per tile / 16 (0: no rows)
    __shared__ int32_t srank[1024];  // expert -> ranked position
    __shared__ int32_t stn[1024];    // ranked position -> tiles, then their exclusive prefix
    __shared__ int32_t sdum[1024];
    __shared__ int32_t bcnt[16][16]; // [64-expert chunk][bin] experts of the bin
    __shared__ int32_t bpre[16][16]; // the same, summed over the earlier chunks
    __shared__ int32_t btot[16];     // experts of a bin
    __shared__ int32_t bstart[16];   // ranked position of a bin's first expert
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    for (int e = tid; e < E; e += 256) {
        c_out[e / 256] = cnt[e];
        toff[e] = (cnt[e] + tile_rows - 1) / tile_rows;
    }
    __syncthreads();
    const int2 tot = block_exclusive_scan2(cnt, toff, E, wtot);
    const int total = tot.x, ntot = tot.y;
    if (tid == 0) {
        offsets[E] = total;
        *ntiles = ntot;
    }
    for (int e = tid, q = 0; e < E; e += 256, ++q) {
        const int c = c_out[q];
        counts[e] = c;
        offsets[e] = cnt[e];
        // an expert's rows are spread about evenly over its tiles, so its
        // tiles (which read the same weights) advance at about the same pace;
        // for large tiles the share is rounded up to 16 rows, the MFMA row
        // block, so only the last tile has a partial block (140 rows: 80 + 60,
        // 9 blocks, not 70 + 70, 10 blocks).  (nt-1)*per < c still holds:
        // per <= tile_rows and nt = ceil(c / tile_rows).
        const int nt = (c + tile_rows - 1) / tile_rows;
        int per = nt > 0 ? (c + nt - 1) / nt : 0;
        if (tile_rows >= 32) per = min(tile_rows, (per + 15) & ~15);
        for (int i = 0; i < nt; ++i) {
            Tile tl;
            tl.expert = e;
            tl.row0 = cnt[e] + i * per;
            tl.nrows = min(per, c - i * per);
            tl.first = toff[e];
            tl.count = nt;
            tl.pad[0] = tl.pad[1] = tl.pad[2] = 0;
            tiles[toff[e] + i] = tl;
        }
        skey[e] = nt > 0 ? (per + 15) >> 4 : 0;
    }
    if (!sc.out) return;

    // ---- rank the experts: bins of rows per tile, descending; by id inside
    // a bin (ballots over 64-expert chunks, chunk q*4 + wave of expert
    // q*256 + tid) ----
    reinterpret_cast<int32_t *>(bcnt)[tid] = 0;
    __syncthreads();
    const int NB = min(16, (tile_rows + 15) / 16 + 1);
    const int NQ = (E + 255) >> 8;
    int my_bin[4], my_within[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (q >= NQ) break;
        const int e = q * 256 + tid;
        const int b = e < E ? min(skey[e], NB - 1) : -1;
        my_bin[q] = b;
        my_within[q] = 0;
        for (int bb = 0; bb < NB; ++bb) {
            const uint64_t m = __ballot(b == bb);
            if (lane == 0) bcnt[q * 4 + wv][bb] = __popcll(m);
            if (b == bb) my_within[q] = __popcll(m & ((1ull << lane) - 1ull));
        }
    }
    __syncthreads();
    {
        // thread (bin tid/16, chunk tid%16): prefix over the chunks of its
        // bin by shuffles within 16 lanes; the bin's total in chunk 15
        const int bb = tid >> 4, c = tid & 15;
        const int own = bb < NB ? bcnt[c][bb] : 0;
        int v = own;
#pragma unroll
        for (int dd = 1; dd < 16; dd <<= 1) {
            const int u = __shfl_up(v, dd, 16);
            if (c >= dd) v += u;
        }
        bpre[c][bb] = v - own;
        if (c == 15) btot[bb] = v;
    }
    __syncthreads();
    if (tid < 64) {
        // a bin's first ranked position: the experts of all higher bins
        const int own = tid < NB ? btot[tid] : 0;
        int v = own;
#pragma unroll
        for (int dd = 1; dd < 16; dd <<= 1) {
            const int u = __shfl_down(v, dd, 16);
            if (tid + dd < 16) v += u;
        }
        if (tid < 16) bstart[tid] = v - own;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = q * 256 + tid;
        if (q >= NQ || e >= E) continue;
        const int b = my_bin[q], chunk = q * 4 + wv;
        const int r = bstart[b] + bpre[chunk][b] + my_within[q];
        srank[e] = r;
        stn[r] = (c_out[q] + tile_rows - 1) / tile_rows;
        sdum[r] = 0;
    }
    __syncthreads();
    (void)block_exclusive_scan2(stn, sdum, E, wtot);  // totals: ntot tiles

    // ---- deal the items: one thread per tile (original order).  Tile mo
    // of expert e (ranked r) holds items j = np * nte + mo of the expert's
    // N-tile-major sequence, sorted position stn[r] * ntn + j. ----
    const int ntn = sc.ntn;
    const SchedShape q = sched_shape(2 * ntn, ntot * ntn);
    for (int t = tid; t < ntot; t += 256) {
        int e = 0, hi = E;  // the last expert with toff[e] <= t (it has tiles)
        while (hi - e > 1) {
            const int mid = (e + hi) >> 1;
            if (toff[mid] <= t) e = mid;
            else hi = mid;
        }
        const int r = srank[e];
        const int nte = (e + 1 < E ? toff[e + 1] : ntot) - toff[e], mo = t - toff[e];
        const int per = skey[e] << 4;
        const int ce = (e + 1 < E ? cnt[e + 1] : total) - cnt[e];
        const int row0 = cnt[e] + mo * per, nrows = min(per, ce - mo * per);
        const int base = stn[r] * ntn;
        for (int np = 0; np < ntn; ++np)
            sc.out[sched_slot(base + np * nte + mo, q)] = sched_item(e, row0, nrows, np);
    }
}

// ---------------------------------------------------------------------------
// Few tokens (T <= 64, T*k <= 4096): top-k, weights, grouping and the tile
// list in one workgroup.
// ---------------------------------------------------------------------------
template <int SLOTS>
__global__ __launch_bounds__(256) void route_small_kernel(
    const float *__restrict__ scores, int32_t *__restrict__ ids, float *__restrict__ wts,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
    int32_t *__restrict__ inv, Tile *__restrict__ tiles, int32_t *__restrict__ ntiles, int T,
    int E, int k, int tile_rows, int nsplit, const Sched sc)
{
    __shared__ unsigned long long mask[1024];
    __shared__ int32_t sid[4096];
    __shared__ int32_t cnt[1024];
    __shared__ int32_t toff[1024];
    __shared__ int32_t wtot[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int S = T * k;
    for (int e = tid; e < E; e += 256) mask[e] = 0ull;
    for (int t = wv; t < T; t += 4)
        topk_row<SLOTS>(scores + (int64_t)t * E, E, k, ids + (int64_t)t * k, wts + (int64_t)t * k,
                        sid + t * k, lane, nsplit, (int64_t)T * E);
    __syncthreads();
    for (int s = tid; s < S; s += 256) atomicOr(&mask[sid[s]], 1ull << (s / k));
    __syncthreads();
    for (int e = tid; e < E; e += 256) cnt[e] = __popcll(mask[e]);
    __syncthreads();
    int c_own[4];
    finish_offsets(cnt, toff, wtot, E, tile_rows, counts, offsets, tiles, ntiles, c_own, sc);
    for (int s = tid; s < S; s += 256) {
        const int e = sid[s];
        const int t = s / k;
        const int pos = cnt[e] + __popcll(mask[e] & ((1ull << t) - 1ull));
        perm[pos] = s;
        inv[s] = pos;
    }
}

// ---------------------------------------------------------------------------
// Many tokens: per-chunk masks, one scan block, per-chunk scatter.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void group_mask_kernel(const int32_t *__restrict__ ids,
                                                         uint64_t *__restrict__ masks, int T,
                                                         int E, int k)
{
    __shared__ unsigned long long mask[1024];
    const int c = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += 256) mask[e] = 0ull;
    __syncthreads();
    const int t0 = c * kChunkTokens;
    const int nt = min(T - t0, kChunkTokens);
    const int64_t s0 = (int64_t)t0 * k;
    for (int q = threadIdx.x; q < nt * k; q += 256)
        atomicOr(&mask[ids[s0 + q]], 1ull << (q / k));
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) masks[(int64_t)c * E + e] = mask[e];
}

// Rows of expert e in chunks c0 .. c0+B-1 (clamped loads, value masked
// after: a conditional load would end its own basic block with a wait).
template <int B>
__device__ __forceinline__ void chunk_popcounts(const uint64_t *__restrict__ masks, int E, int e,
                                                int nchunks, int c0, int (&pc)[B])
{
    uint64_t mv[B];
#pragma unroll
    for (int i = 0; i < B; ++i) mv[i] = masks[(int64_t)min(c0 + i, nchunks - 1) * E + e];
#pragma unroll
    for (int i = 0; i < B; ++i) pc[i] = c0 + i < nchunks ? __popcll(mv[i]) : 0;
}

// One expert per thread (E <= 256) and all chunks in one batch of B: the
// per-chunk row counts stay in registers from the count pass to the base
// pass, so the masks are read once.
template <int B>
__device__ __forceinline__ void group_scan_resident(const uint64_t *__restrict__ masks,
                                                    int32_t *__restrict__ chunk_base, int32_t *cnt,
                                                    int32_t *toff, int32_t (*wtot)[4],
                                                    int32_t *__restrict__ counts,
                                                    int32_t *__restrict__ offsets, Tile *__restrict__ tiles,
                                                    int32_t *__restrict__ ntiles, int E, int nchunks,
                                                    int tile_rows, const Sched &sc)
{
    const int tid = threadIdx.x;
    int pc[B];
    if (tid < E) {
        chunk_popcounts<B>(masks, E, tid, nchunks, 0, pc);
        int run = 0;
#pragma unroll
        for (int i = 0; i < B; ++i) run += pc[i];
        cnt[tid] = run;
    }
    __syncthreads();
    int c_own[4];
    finish_offsets(cnt, toff, wtot, E, tile_rows, counts, offsets, tiles, ntiles, c_own, sc);
    if (tid < E) {
        int run = cnt[tid];
#pragma unroll
        for (int i = 0; i < B; ++i)
            if (i < nchunks) {
                chunk_base[(int64_t)i * E + tid] = run;
                run += pc[i];
            }
    }
}

__global__ __launch_bounds__(256) void group_scan_kernel(
    const uint64_t *__restrict__ masks, int32_t *__restrict__ chunk_base,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, Tile *__restrict__ tiles,
    int32_t *__restrict__ ntiles, int E, int nchunks, int tile_rows, const Sched sc)
{
    __shared__ int32_t cnt[1024];
    __shared__ int32_t toff[1024];
    __shared__ int32_t wtot[2][4];
    if (E <= 256 && nchunks <= 16) {
        group_scan_resident<16>(masks, chunk_base, cnt, toff, wtot, counts, offsets, tiles, ntiles, E,
                                nchunks, tile_rows, sc);
        return;
    }
    if (E <= 256 && nchunks <= 64) {
        group_scan_resident<64>(masks, chunk_base, cnt, toff, wtot, counts, offsets, tiles, ntiles, E,
                                nchunks, tile_rows, sc);
        return;
    }
    // two passes over the masks (counts, then bases); loads go out in batches
    // of 64 (all chunks of a 4096-token call at once), so each pass is one
    // round trip to memory per batch rather than a chain of dependent reads
    constexpr int B = 64;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) {
        int run = 0;
        for (int c0 = 0; c0 < nchunks; c0 += B) {
            int pc[B];
            chunk_popcounts<B>(masks, E, e, nchunks, c0, pc);
#pragma unroll
            for (int i = 0; i < B; ++i) run += pc[i];
        }
        cnt[e] = run;
    }
    __syncthreads();
    int c_own[4];
    finish_offsets(cnt, toff, wtot, E, tile_rows, counts, offsets, tiles, ntiles, c_own, sc);
    for (int e = tid; e < E; e += 256) {
        int run = cnt[e];
        for (int c0 = 0; c0 < nchunks; c0 += B) {
            int pc[B];
            chunk_popcounts<B>(masks, E, e, nchunks, c0, pc);
#pragma unroll
            for (int i = 0; i < B; ++i)
                if (c0 + i < nchunks) {
                    chunk_base[(int64_t)(c0 + i) * E + e] = run;
                    run += pc[i];
                }
        }
    }
}

__global__ __launch_bounds__(256) void group_scatter_kernel(
    const int32_t *__restrict__ ids, const uint64_t *__restrict__ masks,
    const int32_t *__restrict__ chunk_base, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int T, int E, int k)
{
    const int c = blockIdx.x;
    const int t0 = c * kChunkTokens;
    const int nt = min(T - t0, kChunkTokens);
    const int64_t s0 = (int64_t)t0 * k;
    for (int q = threadIdx.x; q < nt * k; q += 256) {
        const int64_t s = s0 + q;
        const int e = ids[s];
        const int tl = q / k;
        const int64_t ce = (int64_t)c * E + e;
        const int pos = chunk_base[ce] + __popcll(masks[ce] & ((1ull << tl) - 1ull));
        perm[pos] = (int32_t)s;
        inv[s] = pos;
    }
}

// The tiled gate/up kernel's schedule the tile-list code writes (none for
// the few-row plans).
static Sched schedule(const Plan &p, const Workspace &ws)
{
    Sched sc{};
    if (!p.tiled || !ws.sched) return sc;
    sc.out = ws.sched;
    sc.ntn = p.ntn1;
    return sc;
}

template <int SLOTS>
static void launch_topk_slots(const Shape &s, const Plan &p, const Workspace &ws, hipStream_t st)
{
    if (p.small_route) {
        route_small_kernel<SLOTS><<<1, 256, 0, st>>>(ws.scores, ws.ids, ws.wts, ws.counts,
                                                     ws.offsets, ws.perm, ws.inv, ws.tiles,
                                                     ws.ntiles, s.T, s.E, s.k, p.tile_rows,
                                                     router_splits(s), schedule(p, ws));
    } else {
        topk_kernel<SLOTS><<<(s.T + 3) / 4, 256, 0, st>>>(ws.scores, ws.ids, ws.wts, s.T, s.E, s.k,
                                                          router_splits(s));
    }
}

hipError_t launch_topk(const Shape &s, const Plan &p, const Workspace &ws, hipStream_t st)
{
    if (p.fuse_route) return hipSuccess;  // the gate/up kernel routes in its prologue
    if (s.E <= 64) launch_topk_slots<1>(s, p, ws, st);
    else if (s.E <= 256) launch_topk_slots<4>(s, p, ws, st);
    else launch_topk_slots<16>(s, p, ws, st);
    return hipGetLastError();
}

hipError_t launch_group(const Shape &s, const Plan &p, const Workspace &ws, hipStream_t st)
{
    if (p.small_route) return hipSuccess;  // done by route_small_kernel
    const int nchunks = (int)num_chunks(s);
    group_mask_kernel<<<nchunks, 256, 0, st>>>(ws.ids, ws.masks, s.T, s.E, s.k);
    group_scan_kernel<<<1, 256, 0, st>>>(ws.masks, ws.chunk_base, ws.counts, ws.offsets, ws.tiles,
                                         ws.ntiles, s.E, nchunks, p.tile_rows, schedule(p, ws));
    group_scatter_kernel<<<nchunks, 256, 0, st>>>(ws.ids, ws.masks, ws.chunk_base, ws.perm, ws.inv,
                                                  s.T, s.E, s.k);
    return hipGetLastError();
}

}  // namespace moe
