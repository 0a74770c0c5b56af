// layout.h -- the packed expert-weight layout the layer kernels read.
//
// "Muse Spark Open を段階的に分解する" (animemo.app), section ⑪: the expert
// weights are 4-bit values with a small scale per block; section ⑬: for few
// tokens the layer time is the read of those bytes.  The packed layout is a
// permutation of the natural row-major MXFP4 matrices (same byte count) that
// makes every 128-element K chunk of a 256-row block one contiguous 16 KB
// tile, so the weight stream reads whole tiles and the prefill kernels copy a
// tile into LDS with linear loads.
//
// Per expert e (bytes at e*3dF/2, scales at e*3dF/32):
//   W1 (gate and up, K = d):  tiles (nt, kc), nt < F/128, kc < d/128, tile
//       at (nt*(d/128) + kc) * 16384; packed row rho < 256 of tile nt holds
//       feature f = nt*128 + (rho>>7)*64 + (rho & 63) of the up matrix if
//       bit 6 of rho is set, else of the gate matrix.
//   W2 (down, K = F): at byte d*F, tiles (nt, kc), nt < d/256, kc < F/128,
//       packed row rho = output row nt*256 + rho.
//   Inside a tile, row rho's 64 bytes are its K chunk kc (codes of elements
//   128kc .. 128kc+127, natural nibble order) as four 16-byte slots; slot s
//   holds the natural 32-element block s ^ bswz(rho) (an LDS bank swizzle).
//   Scales: same tiles of 256 rows x 4 bytes (1024 bytes, W2 at d*F/16);
//   row rho's 4 bytes are the E8M0 bytes of blocks 4kc .. 4kc+3, in order.
#pragma once

#include <stdint.h>

namespace moe {

constexpr int kKStep = 128;                        // K elements per chunk
constexpr int kWRows = 256;                        // rows per weight tile
constexpr int kWTileBytes = kWRows * kKStep / 2;   // 16384
constexpr int kWTileScaleBytes = kWRows * 4;       // 1024

// Slot swizzle: row r's 16-byte slot g is stored at g ^ bswz(r).  With it the
// 16-byte reads of 16 consecutive rows (slot g of each) by one lane group
// are free of LDS bank conflicts (measured on gfx950; ((r >> 1) ^ (r >> 3))
// halves the read rate).
__host__ __device__ __forceinline__ int bswz(int r) { return (r >> 1) & 3; }

// Packed row of W1 for feature f of the gate (up = false) or up matrix,
// inside tile f / 128.
__host__ __device__ __forceinline__ int w1_rho(int f, bool up)
{
    const int fl = f & 127;
    return (fl >> 6) * 128 + (up ? 64 : 0) + (fl & 63);
}

// One matrix of one expert in the packed layout.
struct WView {
    const uint8_t *w;  // code tiles
    const uint8_t *s;  // scale tiles
    int nk;            // K chunks per row
    __device__ __forceinline__ const uint8_t *tile(int nt, int kc) const
    {
        return w + ((int64_t)nt * nk + kc) * kWTileBytes;
    }
    __device__ __forceinline__ const uint8_t *stile(int nt, int kc) const
    {
        return s + ((int64_t)nt * nk + kc) * kWTileScaleBytes;
    }
    // 16 bytes of natural block g of packed row rho in chunk kc of tile nt
    __device__ __forceinline__ const uint8_t *slot(int nt, int kc, int rho, int g) const
    {
        return tile(nt, kc) + rho * 64 + ((g ^ bswz(rho)) << 4);
    }
    // E8M0 bytes of blocks 4kc..4kc+3 of packed row rho
    __device__ __forceinline__ const uint32_t *scales(int nt, int kc, int rho) const
    {
        return reinterpret_cast<const uint32_t *>(stile(nt, kc) + rho * 4);
    }
};

// The 16-block format (one E4M3 scale per 16 values): the code tiles are
// laid out exactly as above; the scale tiles hold 256 rows x 8 bytes per
// chunk (2048 bytes): row rho's bytes are the scales of its 16-blocks
// 8kc .. 8kc+7, in order.  Per expert the scales take 3dF/16 bytes, W2's at
// byte dF/8.
constexpr int kNvTileScaleBytes = kWRows * 8;

struct NvScales {
    const uint8_t *s;
    int nk;
    __device__ __forceinline__ const uint8_t *stile(int nt, int kc) const
    {
        return s + ((int64_t)nt * nk + kc) * kNvTileScaleBytes;
    }
    // the two scale bytes of natural 32-block g of packed row rho
    __device__ __forceinline__ const uint16_t *pair(int nt, int kc, int rho, int g) const
    {
        return reinterpret_cast<const uint16_t *>(stile(nt, kc) + rho * 8 + g * 2);
    }
};

__device__ __forceinline__ WView w1_codes(const uint8_t *wpk, int e, int d, int F)
{
    return WView{wpk + e * ((int64_t)3 * d * F / 2), nullptr, d / kKStep};
}
__device__ __forceinline__ WView w2_codes(const uint8_t *wpk, int e, int d, int F)
{
    return WView{wpk + e * ((int64_t)3 * d * F / 2) + (int64_t)d * F, nullptr, F / kKStep};
}
__device__ __forceinline__ NvScales w1_nv_scales(const uint8_t *sc, int e, int d, int F)
{
    return NvScales{sc + e * ((int64_t)3 * d * F / 16), d / kKStep};
}
__device__ __forceinline__ NvScales w2_nv_scales(const uint8_t *sc, int e, int d, int F)
{
    return NvScales{sc + e * ((int64_t)3 * d * F / 16) + (int64_t)d * F / 8, F / kKStep};
}

__device__ __forceinline__ WView w1_view(const uint8_t *wpk, const uint8_t *sc, int e, int d, int F)
{
    const int64_t eb = (int64_t)3 * d * F / 2, es = (int64_t)3 * d * F / 32;
    return WView{wpk + e * eb, sc + e * es, d / kKStep};
}

__device__ __forceinline__ WView w2_view(const uint8_t *wpk, const uint8_t *sc, int e, int d, int F)
{
    const int64_t eb = (int64_t)3 * d * F / 2, es = (int64_t)3 * d * F / 32;
    return WView{wpk + e * eb + (int64_t)d * F, sc + e * es + (int64_t)d * F / 16, F / kKStep};
}

}  // namespace moe
