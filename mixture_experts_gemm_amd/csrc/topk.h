// Top-k + softmax for one token by one wave, and the whole routing of a
// few-token call by one workgroup (route_few), shared by the routing kernels
// and the gate/up kernels that route in their prologue.
// "Muse Spark Open を段階的に分解する" (animemo.app): section ⑧ (the 8 best
// experts by router score), section ⑨ (their weights: a softmax over the
// chosen scores) and section ⑫ (each expert's tokens gathered together;
// here sorted by (expert, token)).
#pragma once

#include <math.h>

#include "device.h"
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Top-k + softmax for one token, by one wave.  A candidate (score, expert) is
// one 64-bit key that orders as (score desc, id asc): the score's bits made
// order-preserving as an unsigned integer in the high word (-0 counted as +0,
// NaN as -inf) and ~id in the low word, so a comparison is one 64-bit max.
// Each lane keeps SLOTS keys (experts lane + 64*q) sorted best first; each of
// the k rounds takes the wave's largest head (a 32-bit max over the score
// words by DPP steps inside rows of 16 lanes, then row_bcast15/31 across
// rows, the maximum landing in lane 63; ties of the score word, rare, are
// settled by a second max over the id words) and the owning lane pops it.
// The j-th choice is parked in lane j%64, slot j/64; the softmax over the
// chosen scores is one wave sum.
// ---------------------------------------------------------------------------
constexpr int kNone = 0x7FFFFFFF;

__device__ __forceinline__ uint64_t topk_key(float v, int id)
{
    if (!(v == v)) v = -INFINITY;
    if (v == 0.f) v = 0.f;  // -0 ties with +0 (then the lower id wins)
    uint32_t b = __float_as_uint(v);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)id);
}

__device__ __forceinline__ float key_score(uint64_t key)
{
    const uint32_t b = (uint32_t)(key >> 32);
    return __uint_as_float((b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b);
}

__device__ __forceinline__ int key_id(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// max of a 32-bit value over the wave, in every lane: max steps within rows
// of 16 lanes (quad_perm, half_mirror, mirror), then row_bcast15 / 31 (the
// maximum lands in lane 63), read back from lane 63
template <int C, int ROW_MASK>
__device__ __forceinline__ uint32_t u32_max_step(uint32_t v)
{
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, C, ROW_MASK, 0xF, false);
    return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = u32_max_step<0xB1, 0xF>(v);
    v = u32_max_step<0x4E, 0xF>(v);
    v = u32_max_step<0x141, 0xF>(v);
    v = u32_max_step<0x140, 0xF>(v);
    v = u32_max_step<0x142, 0xA>(v);
    v = u32_max_step<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The wave's largest key, in every lane, as a 32-bit max over the high
// words (the order-preserving score) and, only when several lanes hold that
// score, a second one over their low words (~id: the lowest id wins): the
// same result as a 64-bit max, in about half the dependent steps.
__device__ __forceinline__ uint64_t wave_max_key_split(uint64_t key)
{
    const uint32_t hi = (uint32_t)(key >> 32), lo = (uint32_t)key;
    const uint32_t mh = wave_max_u32(hi);
    const bool tie = hi == mh;
    const uint64_t ties = __ballot(tie);
    uint32_t ml;
    if (__popcll(ties) == 1) ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, (int)__ffsll((long long)ties) - 1);
    else ml = wave_max_u32(tie ? lo : 0u);
    return ((uint64_t)mh << 32) | ml;
}


// The k rounds: each takes the wave's largest head key and the owning lane
// pops it; choice j is parked in mine[j / 64] of lane j % 64.  MS = 1 when
// k <= 64 (every choice in one register).
template <int SLOTS, int MS>
__device__ __forceinline__ void topk_rounds(uint64_t (&key)[SLOTS], uint64_t (&mine)[MS], int k, int lane)
{
    const uint64_t none = topk_key(-INFINITY, kNone);
#pragma unroll
    for (int q = 0; q < MS; ++q) mine[q] = none;
    for (int j = 0; j < k; ++j) {
        const uint64_t best = wave_max_key_split(key[0]);
        if (key[0] == best) {  // keys are distinct: exactly the owner lane
#pragma unroll
            for (int q = 0; q + 1 < SLOTS; ++q) key[q] = key[q + 1];
            key[SLOTS - 1] = none;
        }
        if (MS == 1) {
            if (j == lane) mine[0] = best;
        } else {
#pragma unroll
            for (int q = 0; q < MS; ++q)
                if ((j >> 6) == q && (j & 63) == lane) mine[q] = best;
        }
    }
}

// Softmax over the parked choices (relative to the first, the largest) and
// the stores of choice j = lane + 64q.
template <int MS>
__device__ __forceinline__ void topk_store(const uint64_t (&mine)[MS], int k, int lane,
                                           int32_t *__restrict__ ids_out, float *__restrict__ w_out,
                                           int32_t *sid_out)
{
    const uint32_t th = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mine[0] >> 32), 0);
    const float top0 = key_score((uint64_t)th << 32);
    float z = 0.f;
    float ex[MS];
#pragma unroll
    for (int q = 0; q < MS; ++q) {
        ex[q] = (lane + 64 * q < k) ? expf(key_score(mine[q]) - top0) : 0.f;
        z += ex[q];
    }
    z = wave_sum(z);
    const float inv = 1.0f / z;
#pragma unroll
    for (int q = 0; q < MS; ++q) {
        const int j = lane + 64 * q;
        if (j < k) {
            const int e = key_id(mine[q]);
            ids_out[j] = e;
            w_out[j] = ex[q] * inv;
            if (sid_out) sid_out[j] = e;
        }
    }
}

// l: the token's scores, or its first partial-score plane when the router
// split its sums over nsplit slices of d (planes `stride` floats apart,
// added in slice order).  The loads of every slot go out together (one
// round trip for a single plane; PG planes of all slots at a time
// otherwise).
template <int SLOTS>
__device__ __forceinline__ void topk_row(const float *__restrict__ l, int E, int k,
                                         int32_t *__restrict__ ids_out, float *__restrict__ w_out,
                                         int32_t *sid_out, int lane, int nsplit, int64_t stride)
{
    constexpr int PG = SLOTS <= 4 ? 8 : 2;
    float x[SLOTS];
    if (nsplit == 1) {
#pragma unroll
        for (int q = 0; q < SLOTS; ++q) x[q] = l[min(lane + 64 * q, E - 1)];
    } else {
#pragma unroll
        for (int q = 0; q < SLOTS; ++q) x[q] = 0.f;
        for (int sp = 0; sp < nsplit; sp += PG) {
            float v[SLOTS][PG];
#pragma unroll
            for (int i = 0; i < PG; ++i) {
                const float *pl = l + (int64_t)min(sp + i, nsplit - 1) * stride;
#pragma unroll
                for (int q = 0; q < SLOTS; ++q) v[q][i] = pl[min(lane + 64 * q, E - 1)];
            }
#pragma unroll
            for (int q = 0; q < SLOTS; ++q)
#pragma unroll
                for (int i = 0; i < PG; ++i)
                    if (sp + i < nsplit) x[q] = (sp + i == 0) ? v[q][i] : x[q] + v[q][i];
        }
    }
    uint64_t key[SLOTS];
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) {
        const int e = lane + 64 * q;
        key[q] = topk_key(e < E ? x[q] : -INFINITY, e < E ? e : kNone);
    }
#pragma unroll
    for (int pass = 0; pass < SLOTS; ++pass)
#pragma unroll
        for (int q = pass & 1; q + 1 < SLOTS; q += 2)
            if (key[q + 1] > key[q]) {
                const uint64_t t = key[q];
                key[q] = key[q + 1];
                key[q + 1] = t;
            }
    if (SLOTS == 1 || k <= 64) {
        uint64_t mine[1];
        topk_rounds<SLOTS, 1>(key, mine, k, lane);
        topk_store<1>(mine, k, lane, ids_out, w_out, sid_out);
    } else {
        uint64_t mine[SLOTS];
        topk_rounds<SLOTS, SLOTS>(key, mine, k, lane);
        topk_store<SLOTS>(mine, k, lane, ids_out, w_out, sid_out);
    }
}

// ---------------------------------------------------------------------------
// The routing of a call with few slots (S = T*k <= kFewSlots, E <= 256,
// T <= 64, the scores in one plane) by one workgroup (of whole waves), into
// LDS: top-k and weights per token (topk_row, one wave a token), then wave 0 with
// slot s in lane s: the stable grouping by expert (row of slot s: the slots
// of lower experts, then the earlier slots of its own expert -- a token picks
// an expert once, so that is token order) and the tile list (an expert's rows
// cut into ceil(c / tile_rows) tiles of about equal size, experts in id
// order), by broadcasts between lanes.  The same values route_small_kernel
// computes; route_few_store writes them to the workspace.
// ---------------------------------------------------------------------------
struct FewRoute {
    int32_t sid[kFewSlots];     // slot -> expert
    int32_t pos[kFewSlots];     // slot -> grouped row
    int32_t perm[kFewSlots];    // grouped row -> slot
    int32_t sorted[kFewSlots];  // grouped row -> expert
    int32_t ids[kFewSlots];     // top-k outputs [T][k]
    float wts[kFewSlots];
    Tile tiles[kFewSlots];
    int32_t ntiles;
};

__device__ __forceinline__ void route_few(const float *__restrict__ scores, int T, int E, int k,
                                          int tile_rows, FewRoute &r)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = (int)blockDim.x >> 6;
    for (int t = wv; t < T; t += nw) {
        const float *l = scores + (int64_t)t * E;
        if (E <= 64) topk_row<1>(l, E, k, r.ids + t * k, r.wts + t * k, r.sid + t * k, lane, 1, (int64_t)T * E);
        else topk_row<4>(l, E, k, r.ids + t * k, r.wts + t * k, r.sid + t * k, lane, 1, (int64_t)T * E);
    }
    __syncthreads();
    if (wv == 0) {
        const int S = T * k;
        const bool act = lane < S;
        const int e = act ? r.sid[lane] : kNone;
        int less = 0, cnt = 0, before = 0;
        for (int j = 0; j < S; ++j) {
            const int f = __builtin_amdgcn_readlane(e, j);
            less += f < e;
            cnt += f == e;
            before += f == e && j < lane;
        }
        // the lane of each expert's first slot carries its tile count; the
        // expert's tiles follow those of the lower experts
        const bool first = act && before == 0;
        const int nt = first ? (cnt + tile_rows - 1) / tile_rows : 0;
        int toff = 0, total = 0;
        for (int j = 0; j < S; ++j) {
            const int ntj = __builtin_amdgcn_readlane(nt, j);
            toff += __builtin_amdgcn_readlane(e, j) < e ? ntj : 0;
            total += ntj;
        }
        if (act) {
            const int p = less + before;
            r.pos[lane] = p;
            r.perm[p] = lane;
            r.sorted[p] = e;
        }
        if (first) {
            int per = (cnt + nt - 1) / nt;
            if (tile_rows >= 32) per = min(tile_rows, (per + 15) & ~15);
            for (int i = 0; i < nt; ++i) {
                Tile tl;
                tl.expert = e;
                tl.row0 = less + i * per;
                tl.nrows = min(per, cnt - i * per);
                tl.first = toff;
                tl.count = nt;
                tl.pad[0] = tl.pad[1] = tl.pad[2] = 0;
                r.tiles[toff + i] = tl;
            }
        }
        if (lane == 0) r.ntiles = total;
    }
    __syncthreads();
}

// route_few's results into the workspace arrays (ids, weights, counts,
// offsets, perm, inv, tiles, ntiles), for the kernels that run after the
// caller; offsets and counts by binary search over the sorted experts.
__device__ __forceinline__ void route_few_store(const FewRoute &r, int T, int E, int k,
                                                int32_t *__restrict__ ids, float *__restrict__ wts,
                                                int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                int32_t *__restrict__ perm, int32_t *__restrict__ inv,
                                                Tile *__restrict__ tiles, int32_t *__restrict__ ntiles)
{
    const int tid = threadIdx.x, S = T * k;
    if (tid < S) {
        ids[tid] = r.ids[tid];
        wts[tid] = r.wts[tid];
        perm[tid] = r.perm[tid];
        inv[tid] = r.pos[tid];
    }
    if (tid < r.ntiles) tiles[tid] = r.tiles[tid];
    if (tid == 0) *ntiles = r.ntiles;
    for (int e = tid; e <= E; e += (int)blockDim.x) {
        int lo = 0, hi = S;  // first row of an expert >= e
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (r.sorted[mid] < e) lo = mid + 1;
            else hi = mid;
        }
        offsets[e] = lo;
        if (e < E) {
            int lo2 = lo, hi2 = S;  // first row of an expert > e
            while (lo2 < hi2) {
                const int mid = (lo2 + hi2) >> 1;
                if (r.sorted[mid] <= e) lo2 = mid + 1;
                else hi2 = mid;
            }
            counts[e] = lo2 - lo;
        }
    }
}

}  // namespace moe
