// internal.h -- kernel launchers, the launch plan and the workspace layout
// shared by the library's translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One row range of one expert's grouped segment: rows [row0, row0+nrows)
// of the grouped order all belong to `expert`, whose tiles are the `count`
// consecutive entries of the tile list starting at `first`.
struct Tile {
    int32_t expert;
    int32_t row0;
    int32_t nrows;
    int32_t first;
    int32_t count;
    int32_t pad[3];
};

// One workgroup's item of a tiled product: rows [row0, row0+nrows) of the
// grouped order, all of `expert`, times the expert's N-tile `ntile`; packed
// as row0 and expert | nrows << 10 | ntile << 18 (E <= 1024, nrows <= 255,
// ntile < 2048).  The tile-list code writes one per item (the schedule).
struct SchedItem {
    int32_t row0;
    uint32_t packed;
};
__host__ __device__ inline SchedItem sched_item(int expert, int row0, int nrows, int ntile)
{
    return SchedItem{row0, (uint32_t)expert | (uint32_t)nrows << 10 | (uint32_t)ntile << 18};
}

// Where the items of the tiled gate/up product go.  The items, longest
// first, are cut into runs of `run`; each round deals 8 runs to the 8 XCDs
// in snake order (round r gives XCD x run 8r + x, or 8r + 7 - x when r is
// odd), and the items left after the last full round are split evenly over
// the 8 XCDs in the same way.  Workgroup b runs on XCD b % 8 (the
// dispatcher's order), so XCD x's workgroups take its runs in order.
// Item counts fit int32 (they are bounded by S * F / 128).
struct SchedShape {
    int run;     // items per run
    int full;    // items in the full rounds (a multiple of 8 * run)
    int rem;     // items after them
    int lr;      // items per XCD in the last round, ceil(rem / 8)
};
__host__ __device__ inline SchedShape sched_shape(int run, int nitems)
{
    SchedShape q;
    q.run = run;
    q.full = nitems / (8 * run) * 8 * run;
    q.rem = nitems - q.full;
    q.lr = (q.rem + 7) / 8;
    return q;
}
__host__ __device__ inline int sched_snake(int round, int x) { return (round & 1) ? 7 - x : x; }
// workgroup b -> sorted item, or -1 when b has none
__host__ __device__ inline int sched_pos(int b, const SchedShape &q)
{
    const int p = b >> 3, x = b & 7, full_p = q.full / 8;  // positions of the full rounds
    if (p < full_p) {
        const int round = p / q.run, o = p - round * q.run;
        return (round * 8 + sched_snake(round, x)) * q.run + o;
    }
    const int o = p - full_p;
    if (o >= q.lr) return -1;
    const int i = sched_snake(q.full / (8 * q.run), x) * q.lr + o;
    return i < q.rem ? q.full + i : -1;
}
// sorted item s (< nitems) -> its workgroup
__host__ __device__ inline int sched_slot(int s, const SchedShape &q)
{
    if (s < q.full) {
        const int rid = s / q.run, o = s - rid * q.run, round = rid >> 3;
        return 8 * (round * q.run + o) + sched_snake(round, rid & 7);
    }
    const int i = s - q.full, xr = i / q.lr, o = i - xr * q.lr;
    return 8 * (q.full / 8 + o) + sched_snake(q.full / (8 * q.run), xr);
}

// Tokens per chunk of the counting sort (one 64-bit token mask per expert).
constexpr int kChunkTokens = 64;

struct Shape {
    int T, d, E, F, k;
    float eps;
    int64_t S() const { return (int64_t)T * k; }
};

// Which kernels run.  Few rows per expert (decode): 16-row tiles, one wave
// per 16 output columns streaming weights.  Many rows per expert (prefill):
// 128-row tiles staged through LDS and shared by a workgroup.
// Very few tokens (at most kStreamMaxT, d a multiple of 2048): the gate/up
// product runs as a persistent streaming kernel whose tiles hold at most
// kStreamRows rows (an expert chosen by more tokens gets several tiles).
constexpr int kStreamMaxT = 8;
constexpr int kStreamRows = 2;

// Average rows per expert from which the tiled (MX) kernels run.  Below
// it the few-row kernels use 16-row tiles, which read an expert's weights
// once per tile: from about 16 rows per expert the 128-row tiles read them
// fewer times (measured: 753 rows over 32 experts, 586 -> 301 us).
constexpr int kTiledMinRows = 16;

// Average rows per expert below which the wide kernels take 64-row tiles on
// a three-stage ring: with so few rows a workgroup's multiply is short next
// to its loads, and a third stage keeps two chunks of weights in flight.
constexpr int kShortTileMaxRows = 48;

// Slots (T*k) up to which the streaming gate/up kernel routes a call in its
// prologue (route_few) instead of a routing kernel running before it.  Every
// workgroup routes, so the prologue's time is on the kernel's critical path:
// at decode T=1 (8 slots) the step is 2.3 us shorter, at T=4 (32 slots) the
// same as with the routing kernel.
constexpr int kFewSlots = 16;

// What a gate/up kernel that routes in its prologue reads (the router's
// scores, one plane) and stores besides perm / tiles / ntiles (workgroup 0).
struct RouteArgs {
    const float *scores;
    int T, E;
    int32_t *ids;
    float *wts;
    int32_t *counts;
    int32_t *offsets;
    int32_t *inv;
};

struct Plan {
    bool tiled;
    bool stream;    // persistent streaming gate/up kernel (decode)
    int tile_rows;  // rows per tile of the tile list
    int ssq_cols;   // columns of o per partial sum of squares
    bool small_route;  // single-workgroup routing (T <= 64 and T*k <= 4096)
    // the streaming gate/up kernel routes in its prologue (route_few, every
    // workgroup alike; workgroup 0 stores the routing for the later kernels)
    // and no routing kernel runs: streaming plans with T*k <= kFewSlots and
    // E <= 256 (MXFP4 weights)
    bool fuse_route;
    // tiled plans: the gate/up kernel's workgroups per tile and its launch
    // (the schedule the tile-list code writes, Sched)
    int ntn1;
    int grid1;
};

// Upper bound of the tile count for tiles of tile_rows rows (1: any plan).
inline int64_t max_tiles(const Shape &s, int tile_rows)
{
    int64_t S = s.S();
    int64_t u = S < s.E ? S : s.E;
    return S / tile_rows + u + 1;
}

// The wide kernel (128 x 512 or 64 x 512 tiles) runs a matrix with an even
// number of 256-row weight tiles; an odd count runs on the 128 x 256 kernel.
inline bool wide_gate_up(const Shape &s) { return (s.F / 128) % 2 == 0; }
inline bool wide_down(const Shape &s) { return (s.d / 256) % 2 == 0; }

// Workgroups of the tiled gate/up launch: runs of 2*ntn items dealt to the
// 8 XCDs in rounds, enough rounds for every item of the largest tile list.
inline int64_t sched_grid(const Shape &s, int tile_rows, int ntn)
{
    const int64_t run = 2 * (int64_t)ntn;
    const int64_t items = max_tiles(s, tile_rows) * ntn;
    return 8 * run * ((items + 8 * run - 1) / (8 * run));
}

inline void set_schedule(const Shape &s, Plan &p, int ntn_gate_up)
{
    p.ntn1 = ntn_gate_up;
    p.grid1 = (int)sched_grid(s, p.tile_rows, ntn_gate_up);
}

// The streaming gate/up path on whole tile columns (gemm1_col_kernel) when
// the expected number of (tile, 128-feature column) items fills the device:
// E (1 - (1 - k/E)^T) distinct experts, F/128 columns each (at T = 1 with
// E = 256, k = 8 there are 128 items and the 16-feature items of
// gemm1_stream_kernel run faster).
inline bool stream_columns(const Shape &s)
{
    if (s.F % 128 != 0 || s.d % 512 != 0) return false;  // an even number of chunks per K half
    double miss = 1.0;  // probability that a given expert is chosen by no token
    for (int t = 0; t < s.T; ++t) miss *= 1.0 - (double)s.k / s.E;
    return s.E * (1.0 - miss) * (s.F / 128) >= 192.0;
}

inline Plan make_plan(const Shape &s)
{
    Plan p;
    const int64_t S = s.S();
    p.tiled = S >= (int64_t)kTiledMinRows * s.E && s.d % 256 == 0 && s.F % 128 == 0;
    p.stream = !p.tiled && s.d % 2048 == 0 && s.T <= kStreamMaxT;
    p.tile_rows = p.tiled ? 128 : p.stream ? (s.T < kStreamRows ? s.T : kStreamRows) : 16;
    if (p.tiled && wide_gate_up(s) && wide_down(s) && S < (int64_t)kShortTileMaxRows * s.E)
        p.tile_rows = 64;
    if (p.tile_rows < 1) p.tile_rows = 1;
    p.ssq_cols = 64;  // both down kernels reduce o^2 over 64-column groups
    p.small_route = s.T <= kChunkTokens && S <= 4096;
    p.fuse_route = p.stream && S <= kFewSlots && s.E <= 256;
    p.ntn1 = p.grid1 = 0;
    // MXFP4 tiled gate/up kernel: pairs of 256-row weight tiles (wide) or single ones
    if (p.tiled) set_schedule(s, p, wide_gate_up(s) ? s.F / 256 : s.F / 128);
    return p;
}

// Workgroup tile of the many-token router: 128 tokens x 128 experts, or
// 256 tokens x 64 experts when there are at most 64 experts.
inline int router_tile_experts(int E) { return E <= 64 ? 64 : 128; }
inline int router_tile_tokens(int E) { return E <= 64 ? 256 : 128; }

// Slices of d the many-token router splits its sums into (partial score
// planes added by top-k): enough workgroups to fill the device (at least
// 256, at most 512 when possible), at most 32 slices, each a multiple of 32
// long.
inline int router_splits(const Shape &s)
{
    if (s.T <= 32) return 1;
    const int tt = router_tile_tokens(s.E), te = router_tile_experts(s.E);
    const int64_t tiles = (int64_t)((s.T + tt - 1) / tt) * ((s.E + te - 1) / te);
    int ks = 1;
    while (ks < 32 && tiles * ks * 2 <= 512 && (s.d / (ks * 2)) % 32 == 0) ks *= 2;
    return ks;
}

// Activation rows for the wide tiled kernels: three FP6 E2M3 parts with E8M0
// scales per 32-block (split_e2m3x3_block), stored per row and 128-wide K
// chunk as one 304-byte record: part p at bytes 96p .. 96p+95 (K values in
// order, 6 bits each, little-endian), the 12 scale bytes at 288 (part p's
// scales of blocks 0..3 at 288 + 4p), 4 zero bytes.  Records of a row follow
// each other: row r, chunk c at (r * K/128 + c) * 304.
constexpr int kA6Bytes = 304;
constexpr int kA6Units = kA6Bytes / 16;

// Rows per tile of the 16-block format's tiled kernel: 192 keeps an
// expert's prefill rows (about 128 +- 40) in one tile, so its weights are
// loaded and widened once.
constexpr int kNvTileRows = 192;

// The 16-block format's tiled kernels: kNvTileRows-row tiles, one 256-row
// weight tile per workgroup.
inline void nv_plan(const Shape &s, Plan &p)
{
    p.fuse_route = false;  // the 16-block kernels read the routing kernel's tile list
    if (!p.tiled) return;
    p.tile_rows = kNvTileRows;
    set_schedule(s, p, s.F / 128);
}

// Entries of the workspace's schedule: enough for any tiled plan (128-row
// tiles and single weight tiles give the most workgroups).
inline int64_t sched_entries(const Shape &s) { return sched_grid(s, 128, s.F / 128); }

inline int64_t num_chunks(const Shape &s) { return (s.T + kChunkTokens - 1) / kChunkTokens; }

struct Workspace {
    float *scores;        // [router_splits][T][E] partial router scores
    int32_t *ids;         // [S]
    float *wts;           // [S]
    uint64_t *masks;      // [nchunks][E] token bits of each expert in a chunk
    int32_t *chunk_base;  // [nchunks][E] first grouped position of (chunk, expert)
    int32_t *counts;      // [E]
    int32_t *offsets;     // [E+1]
    int32_t *perm;        // [S]
    int32_t *inv;         // [S]
    Tile *tiles;          // [max_tiles]
    int32_t *ntiles;      // [1]
    SchedItem *sched;     // tiled plans: the gate/up kernel's item per workgroup, else null
    uint16_t *h;          // bf16 [S][F]
    uint16_t *o;          // bf16 [S][d]
    float *ssq;           // [S][d / 64]
    // FP8 E4M3 hi/lo parts of x and h with E8M0 scales per 32-block, or
    // (same memory) their three-part FP6 records for the wide kernels
    uint8_t *xhi, *xlo;   // [T][d]
    uint8_t *xshi, *xslo; // [T][d/32]
    uint8_t *hhi, *hlo;   // [S][F]
    uint8_t *hshi, *hslo; // [S][F/32]
    uint8_t *xa6;         // [T][d/128] records of kA6Bytes
    uint8_t *ha6;         // [S][F/128] records of kA6Bytes
    size_t bytes;
};

// Lays the workspace out from `base` (NULL: only computes .bytes).
Workspace carve_workspace(const Shape &s, void *base);

// ---- launchers (all asynchronous on `st`) ---------------------------------
hipError_t launch_router(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                         const float *wr, hipStream_t st);
// bf16 x -> its split for the tiled gate/up kernel: FP6 records when that
// kernel is the wide one, else FP8 hi/lo parts + E8M0 scales.
hipError_t launch_split_x(const Shape &s, const Workspace &ws, const uint16_t *x, hipStream_t st);
hipError_t launch_topk(const Shape &s, const Plan &p, const Workspace &ws, hipStream_t st);
hipError_t launch_group(const Shape &s, const Plan &p, const Workspace &ws, hipStream_t st);
// The gate/up stage is one kernel; ev_begin / ev_end (may be null) are
// recorded by its dispatch itself, so they time exactly that kernel.
hipError_t launch_gemm1(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                        const uint8_t *wpk, const uint8_t *sc, hipStream_t st,
                        hipEvent_t ev_begin, hipEvent_t ev_end);
hipError_t launch_gemm2(const Shape &s, const Plan &p, const Workspace &ws, const uint8_t *wpk,
                        const uint8_t *sc, hipStream_t st);
hipError_t launch_combine(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                          const float *alpha, const float *beta, uint16_t *s_out,
                          hipStream_t st);
// Norms and weighted sum only: y = bf16(sum_j w_j * norm(o_j)) [T][d].
hipError_t launch_combine_sum(const Shape &s, const Plan &p, const Workspace &ws, uint16_t *y,
                              hipStream_t st);
// Norms and weighted sum only, fp32 y [T][d].
hipError_t launch_combine_sum_f32(const Shape &s, const Plan &p, const Workspace &ws, float *y,
                                  hipStream_t st);
// The block's stream norms: x_n = bf16(x * rms(x)^-1 * gamma); s_out =
// bf16(alpha * x + beta * y * rms(y)^-1 * gamma), one workgroup per row.
hipError_t launch_prenorm(const uint16_t *x, const float *gamma, uint16_t *xn, int T, int d, float eps,
                          hipStream_t st);
hipError_t launch_postnorm_gate(const uint16_t *x, const float *y, const float *gamma,
                                const float *alpha, const float *beta, uint16_t *s_out, int T, int d,
                                float eps, hipStream_t st);
// The block's combine and post-norm gate in one kernel, for rows of at most
// kBlockFusedMaxD columns and at most kBlockFusedMaxK slots per token
// (hipErrorInvalidValue otherwise; the caller then takes fp32 y and
// launch_postnorm_gate).
hipError_t launch_combine_postnorm(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                                   const float *gamma, const float *alpha, const float *beta,
                                   uint16_t *s_out, hipStream_t st);
constexpr int kBlockFusedMaxD = 16384;
constexpr int kBlockFusedMaxK = 64;
// bf16 x -> FP8 hi/lo parts + E8M0 scales in the workspace (the streaming
// gate/up kernel's input when the router does not split x itself).
hipError_t launch_split_x_fp8(const Shape &s, const Workspace &ws, const uint16_t *x, hipStream_t st);
// c[T][N] = a[T][K] w[N][K]^T, bf16 operands, fp32 accumulation on the bf16
// MFMA (the latent-width variant's shared matrices); c is stored as bf16
// (kDenseBf16), fp32 (kDenseF32) or as the gated residual
// bf16(alpha[n] * x[t][n] + beta[n] * c[t][n]) (kDenseGate, x bf16 [T][N],
// c may be x).
enum { kDenseBf16 = 0, kDenseF32 = 1, kDenseGate = 2 };
struct DenseGate {
    const uint16_t *x;
    const float *alpha, *beta;
};
hipError_t launch_dense(const uint16_t *a, const uint16_t *w, void *c, int out, int T, int N, int K,
                        hipStream_t st, const DenseGate &g = DenseGate{nullptr, nullptr, nullptr});
hipError_t launch_pack(const uint8_t *w, const uint8_t *s, int E, int d, int F, uint8_t *wp,
                       uint8_t *sp, hipStream_t st);
// The 16-block format (one E4M3 scale per 16 values, matrix scales gs [E][3]).
hipError_t launch_pack_nv(const uint8_t *w, const uint8_t *s16, int E, int d, int F, uint8_t *wp,
                          uint8_t *sp, hipStream_t st);
// bf16 rows -> fp16 rows times a per-row power of two, scale[r] = its inverse.
hipError_t launch_f16_rows(const uint16_t *src, int64_t rows, int K, uint16_t *dst, float *scale,
                           hipStream_t st);
// The streaming plan reads the bf16 x itself; the others expect x converted
// by launch_f16_rows into ws.xhi (rows) / ws.xshi (scales).
hipError_t launch_gemm1_nv(const Shape &s, const Plan &p, const Workspace &ws, const uint16_t *x,
                           const uint8_t *wpk, const uint8_t *sc, const float *gs, hipStream_t st,
                           hipEvent_t ev_begin, hipEvent_t ev_end);
hipError_t launch_gemm2_nv(const Shape &s, const Plan &p, const Workspace &ws, const uint8_t *wpk,
                           const uint8_t *sc, const float *gs, hipStream_t st);
hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int64_t rows, int K,
                          uint16_t *out, hipStream_t st);

}  // namespace moe
