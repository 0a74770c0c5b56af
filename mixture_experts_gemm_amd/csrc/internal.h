// internal.h -- kernel launchers and the workspace layout shared by the
// library's translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// One row range of one expert's grouped segment: rows [row0, row0+nrows)
// of the grouped order all belong to `expert`.
struct Tile {
    int32_t expert;
    int32_t row0;
    int32_t nrows;
    int32_t pad;
};

// Rows per tile of the tile list.
constexpr int kTileRows = 16;
// Columns of o covered by one partial sum of squares.
constexpr int kSsqCols = 16;

struct Shape {
    int T, d, E, F, k;
    float eps;
    int64_t S() const { return (int64_t)T * k; }
};

// Tokens per chunk of the counting sort: chunk*k slot ids stay in LDS.
inline int group_chunk_tokens(int k)
{
    int c = 2048 / k;
    if (c > 256) c = 256;
    if (c < 1) c = 1;
    return c;
}

inline int64_t max_tiles(const Shape &s)
{
    int64_t S = s.S();
    int64_t u = S < s.E ? S : s.E;
    return S / kTileRows + u + 1;
}

struct Workspace {
    float *scores;        // [T][E]
    int32_t *ids;         // [S]
    float *wts;           // [S]
    int32_t *chunk_base;  // [nchunks][E]
    int32_t *counts;      // [E]
    int32_t *offsets;     // [E+1]
    int32_t *perm;        // [S]
    int32_t *inv;         // [S]
    Tile *tiles;          // [max_tiles]
    int32_t *ntiles;      // [1]
    uint16_t *h;          // bf16 [S][F]
    uint16_t *o;          // bf16 [S][d]
    float *ssq;           // [S][d / kSsqCols]
    size_t bytes;
};

// Lays the workspace out from `base` (NULL: only computes .bytes).
Workspace carve_workspace(const Shape &s, void *base);

// ---- launchers (all asynchronous on `st`) ---------------------------------
hipError_t launch_router(const Shape &s, const uint16_t *x, const float *wr, float *scores,
                         hipStream_t st);
hipError_t launch_topk(const Shape &s, const float *scores, int32_t *ids, float *wts,
                       hipStream_t st);
hipError_t launch_group(const Shape &s, const Workspace &ws, hipStream_t st);
hipError_t launch_gemm1(const Shape &s, const Workspace &ws, const uint16_t *x,
                        const uint8_t *wpk, const uint8_t *sc, hipStream_t st);
hipError_t launch_gemm2(const Shape &s, const Workspace &ws, const uint8_t *wpk,
                        const uint8_t *sc, hipStream_t st);
hipError_t launch_combine(const Shape &s, const Workspace &ws, const uint16_t *x,
                          const float *alpha, const float *beta, uint16_t *s_out,
                          hipStream_t st);
hipError_t launch_dequant(const uint8_t *codes, const uint8_t *scales, int64_t rows, int K,
                          uint16_t *out, hipStream_t st);

}  // namespace moe
