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
//              (expert, token), built without order-dependent atomics).
#include "device.h"
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router scores, few tokens: one workgroup per expert streams that expert's
// fp32 router row once per token; fixed-order block reduction.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t *__restrict__ x,
                                                          const float *__restrict__ wr,
                                                          float *__restrict__ scores, int T,
                                                          int d, int E)
{
    __shared__ float part[4];
    const int e = blockIdx.x;
    const float *w = wr + (int64_t)e * d;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int t = 0; t < T; ++t) {
        const uint16_t *xt = x + (int64_t)t * d;
        float acc = 0.f;
        for (int i = threadIdx.x * 4; i < d; i += 1024) {
            float4 wq = *reinterpret_cast<const float4 *>(w + i);
            uint2 xq = *reinterpret_cast<const uint2 *>(xt + i);
            acc = fmaf(__uint_as_float(xq.x << 16), wq.x, acc);
            acc = fmaf(__uint_as_float(xq.x & 0xFFFF0000u), wq.y, acc);
            acc = fmaf(__uint_as_float(xq.y << 16), wq.z, acc);
            acc = fmaf(__uint_as_float(xq.y & 0xFFFF0000u), wq.w, acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) part[wv] = acc;
        __syncthreads();
        if (threadIdx.x == 0) scores[(int64_t)t * E + e] = (part[0] + part[1]) + (part[2] + part[3]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Router scores, many tokens: bf16 MFMA on an exact three-way bf16 split of
// the fp32 router weights (w = hi + mid + lo exactly; x is bf16, so every
// product is exact and the sum is accumulated in fp32 like an fp32 GEMM).
// One wave computes a 16-token x 16-expert tile over all of d.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split3(float w, uint16_t &hi, uint16_t &mid, uint16_t &lo)
{
    hi = f32_to_bf16(w);
    float r1 = w - bf16_to_f32(hi);
    mid = f32_to_bf16(r1);
    float r2 = r1 - bf16_to_f32(mid);
    lo = f32_to_bf16(r2);
}

__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t *__restrict__ x,
                                                          const float *__restrict__ wr,
                                                          float *__restrict__ scores, int T,
                                                          int d, int E, int eblocks)
{
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int tb = gw / eblocks, eb = gw % eblocks;
    const int t0 = tb * 16, e0 = eb * 16;
    if (t0 >= T) return;
    const int r = lane & 15, g = lane >> 4;
    const bool tv = t0 + r < T, ev = e0 + r < E;
    const uint16_t *xp = x + (int64_t)(tv ? t0 + r : 0) * d + g * 8;
    const float *wp = wr + (int64_t)(ev ? e0 + r : 0) * d + g * 8;
    floatx4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < d; k0 += 32) {
        uint4 xa = tv ? *reinterpret_cast<const uint4 *>(xp + k0) : make_uint4(0, 0, 0, 0);
        float4 w0 = ev ? *reinterpret_cast<const float4 *>(wp + k0) : make_float4(0, 0, 0, 0);
        float4 w1 = ev ? *reinterpret_cast<const float4 *>(wp + k0 + 4) : make_float4(0, 0, 0, 0);
        float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        uint16_t hi[8], mi[8], lo[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) split3(wv[i], hi[i], mi[i], lo[i]);
        uint4 bh, bm, bl;
        bh.x = hi[0] | (uint32_t)hi[1] << 16; bh.y = hi[2] | (uint32_t)hi[3] << 16;
        bh.z = hi[4] | (uint32_t)hi[5] << 16; bh.w = hi[6] | (uint32_t)hi[7] << 16;
        bm.x = mi[0] | (uint32_t)mi[1] << 16; bm.y = mi[2] | (uint32_t)mi[3] << 16;
        bm.z = mi[4] | (uint32_t)mi[5] << 16; bm.w = mi[6] | (uint32_t)mi[7] << 16;
        bl.x = lo[0] | (uint32_t)lo[1] << 16; bl.y = lo[2] | (uint32_t)lo[3] << 16;
        bl.z = lo[4] | (uint32_t)lo[5] << 16; bl.w = lo[6] | (uint32_t)lo[7] << 16;
        bf16x8_t a = as_bf16x8(xa);
        acc = mfma16(a, as_bf16x8(bl), acc);
        acc = mfma16(a, as_bf16x8(bm), acc);
        acc = mfma16(a, as_bf16x8(bh), acc);
    }
    // lane holds scores for tokens t0 + g*4 + i, expert e0 + r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int t = t0 + g * 4 + i;
        if (t < T && ev) scores[(int64_t)t * E + e0 + r] = acc[i];
    }
}

hipError_t launch_router(const Shape &s, const uint16_t *x, const float *wr, float *scores,
                         hipStream_t st)
{
    if (s.T <= 32) {
        router_gemv_kernel<<<s.E, 256, 0, st>>>(x, wr, scores, s.T, s.d, s.E);
    } else {
        int eblocks = (s.E + 15) / 16;
        int64_t waves = (int64_t)((s.T + 15) / 16) * eblocks;
        router_mfma_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(x, wr, scores, s.T, s.d,
                                                                          s.E, eblocks);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k + softmax: one wave per token.  Each lane keeps E/64 scores in
// registers; k rounds of a wave-wide arg-max under the order
// (score descending, expert id ascending).
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ scores,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ wts, int T, int E, int k)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float *l = scores + (int64_t)t * E;
    float v[16];
    uint32_t avail = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        int e = lane + 64 * j;
        v[j] = e < E ? l[e] : 0.f;
        if (e < E) avail |= 1u << j;
    }
    float top0 = 0.f;
    for (int j = 0; j < k; ++j) {
        float bv = 0.f;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int q = 0; q < 16; ++q)
            if ((avail >> q) & 1u) {
                int e = lane + 64 * q;
                if (bi == 0x7FFFFFFF || better(v[q], e, bv, bi)) { bv = v[q]; bi = e; }
            }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            float ov = __shfl_xor(bv, off);
            int oi = __shfl_xor(bi, off);
            if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || better(ov, oi, bv, bi))) { bv = ov; bi = oi; }
        }
        if ((bi & 63) == lane) avail &= ~(1u << (bi >> 6));
        if (j == 0) top0 = bv;
        if (lane == 0) {
            ids[(int64_t)t * k + j] = bi;
            wts[(int64_t)t * k + j] = bv;  // the score for now; normalised below
        }
    }
    // softmax over the chosen scores, in choice order (lane 0 owns the row)
    if (lane == 0) {
        float *wt = wts + (int64_t)t * k;
        float z = 0.f;
        for (int j = 0; j < k; ++j) z += expf(wt[j] - top0);
        const float inv = 1.0f / z;
        for (int j = 0; j < k; ++j) wt[j] = expf(wt[j] - top0) * inv;
    }
}

hipError_t launch_topk(const Shape &s, const float *scores, int32_t *ids, float *wts,
                       hipStream_t st)
{
    topk_kernel<<<(s.T + 3) / 4, 256, 0, st>>>(scores, ids, wts, s.T, s.E, s.k);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouping: stable counting sort of slots t*k+j by (expert, token).
//   count:   per chunk of tokens, per-expert counts (LDS integer atomics;
//            counts do not depend on the order the atomics land in)
//   scan:    per expert, exclusive prefix over chunks; offsets = exclusive
//            prefix over experts; tile list of <= kTileRows rows per tile
//   scatter: per chunk, thread e walks the chunk's tokens in order and
//            places every slot that chose e
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void group_count_kernel(const int32_t *__restrict__ ids,
                                                          int32_t *__restrict__ chunk_base,
                                                          int T, int E, int k, int chunk)
{
    __shared__ int32_t hist[1024];
    const int c = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
    __syncthreads();
    int64_t s0 = (int64_t)c * chunk * k;
    int64_t s1 = (int64_t)min(T, (c + 1) * chunk) * k;
    for (int64_t s = s0 + threadIdx.x; s < s1; s += 256) atomicAdd(&hist[ids[s]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) chunk_base[(int64_t)c * E + e] = hist[e];
}

__global__ __launch_bounds__(1024) void group_scan_kernel(int32_t *__restrict__ chunk_base,
                                                          int32_t *__restrict__ counts,
                                                          int32_t *__restrict__ offsets,
                                                          Tile *__restrict__ tiles,
                                                          int32_t *__restrict__ ntiles, int E,
                                                          int nchunks)
{
    __shared__ int32_t cnt[1024];
    __shared__ int32_t off[1025];
    __shared__ int32_t toff[1025];
    const int e = threadIdx.x;
    int total = 0;
    if (e < E) {
        for (int c = 0; c < nchunks; ++c) {
            int h = chunk_base[(int64_t)c * E + e];
            chunk_base[(int64_t)c * E + e] = total;
            total += h;
        }
        cnt[e] = total;
    }
    __syncthreads();
    if (e == 0) {
        int acc = 0, tacc = 0;
        for (int q = 0; q < E; ++q) {
            off[q] = acc;
            toff[q] = tacc;
            acc += cnt[q];
            tacc += (cnt[q] + kTileRows - 1) / kTileRows;
        }
        off[E] = acc;
        toff[E] = tacc;
        offsets[E] = acc;
        *ntiles = tacc;
    }
    __syncthreads();
    if (e < E) {
        counts[e] = total;
        offsets[e] = off[e];
        for (int c = 0; c < nchunks; ++c) chunk_base[(int64_t)c * E + e] += off[e];
        int nt = (total + kTileRows - 1) / kTileRows;
        for (int i = 0; i < nt; ++i) {
            Tile tl;
            tl.expert = e;
            tl.row0 = off[e] + i * kTileRows;
            tl.nrows = min(kTileRows, total - i * kTileRows);
            tl.pad = 0;
            tiles[toff[e] + i] = tl;
        }
    }
}

__global__ __launch_bounds__(256) void group_scatter_kernel(const int32_t *__restrict__ ids,
                                                            const int32_t *__restrict__ chunk_base,
                                                            int32_t *__restrict__ perm,
                                                            int32_t *__restrict__ inv, int T,
                                                            int E, int k, int chunk)
{
    __shared__ int32_t cids[2048];
    const int c = blockIdx.x;
    const int t0 = c * chunk;
    const int nt = min(T, t0 + chunk) - t0;
    const int64_t s0 = (int64_t)t0 * k;
    for (int q = threadIdx.x; q < nt * k; q += 256) cids[q] = ids[s0 + q];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) {
        int pos = chunk_base[(int64_t)c * E + e];
        for (int t = 0; t < nt; ++t)
            for (int j = 0; j < k; ++j)
                if (cids[t * k + j] == e) {
                    int64_t slot = s0 + (int64_t)t * k + j;
                    perm[pos] = (int32_t)slot;
                    inv[slot] = pos;
                    ++pos;
                    break;
                }
    }
}

hipError_t launch_group(const Shape &s, const Workspace &ws, hipStream_t st)
{
    const int chunk = group_chunk_tokens(s.k);
    const int nchunks = (s.T + chunk - 1) / chunk;
    group_count_kernel<<<nchunks, 256, 0, st>>>(ws.ids, ws.chunk_base, s.T, s.E, s.k, chunk);
    group_scan_kernel<<<1, 1024, 0, st>>>(ws.chunk_base, ws.counts, ws.offsets, ws.tiles,
                                          ws.ntiles, s.E, nchunks);
    group_scatter_kernel<<<nchunks, 256, 0, st>>>(ws.ids, ws.chunk_base, ws.perm, ws.inv, s.T,
                                                  s.E, s.k, chunk);
    return hipGetLastError();
}

}  // namespace moe
