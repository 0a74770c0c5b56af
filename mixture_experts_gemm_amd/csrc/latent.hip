// latent.hip -- the two shared-matrix products and the gate of the
// latent-width variant.
//
// "Muse Spark Open を段階的に分解する" (animemo.app), section ⑨: a matrix
// shared by the chosen experts narrows the token before them, a second one
// widens their weighted sum after them; section ③: the widened sum joins
// the residual through the per-dimension gate s <- alpha*s + beta*(.).
//
// Both products are C[T][N] = A[T][K] W[N][K]^T with bf16 A and W (K
// contiguous in both), fp32 accumulation on the bf16 MFMA, and C bf16 (the
// narrowed token z, rounded to nearest even) or, for the widened sum f, the
// gated residual s_out = bf16(alpha * x + beta * f) formed in the epilogue
// (f never leaves the registers).
// Few tokens: each matrix row is read once from HBM, so the product is a
// weight stream (dense_stream_kernel).  Many tokens: 256 x 256 output tiles
// staged through LDS (dense_gemm_kernel).
#include "device.h"
#include "internal.h"
#include "layout.h"

namespace moe {

// One output element: c bf16 (kDenseBf16), fp32 (kDenseF32), or, for the
// widening product, the gated residual s_out = bf16(alpha * x + beta * c)
// at the same place of [T][N] (kDenseGate; x is read before s_out is
// written by the same thread, so s_out may be x).
template <int OUT>
__device__ __forceinline__ void store_dense(void *C, int64_t idx, int col, float v, const DenseGate &g)
{
    if constexpr (OUT == kDenseF32) {
        static_cast<float *>(C)[idx] = v;
    } else if constexpr (OUT == kDenseGate) {
        const float xf = __uint_as_float((uint32_t)g.x[idx] << 16);
        static_cast<uint16_t *>(C)[idx] = f32_to_bf16(fmaf(g.beta[col], v, g.alpha[col] * xf));
    } else {
        static_cast<uint16_t *>(C)[idx] = f32_to_bf16(v);
    }
}

// ---- few tokens: the weight stream ---------------------------------------------
// One workgroup per 16 rows of W (16 output columns), all T <= 8 tokens.
// The NW waves (4, or 8 when K >= 8192) take equal parts of K in 128-wide
// chunks.  Each load instruction
// reads 8 rows x 128 contiguous bytes (whole cache lines): lane l takes row
// 8o + l%8 of the octet o and the 8 K values 64h + 8(l/8) .. +7 of the
// chunk's half h.  A fragments follow the same lane map (token l%8, same 8
// K values), so one 16x16x32 MFMA per (half, octet) pairs A lane m + 16g
// with B lane n + 16g on equal K values wherever m and n are both below 8
// (K groups 2g) or both at least 8 (K groups 2g+1): C[t][j] + C[t+8][j+8]
// is token t times row 8o + j over the whole half, and the off-diagonal
// blocks are discarded.  Two batches of kDenseU chunks are in flight while
// one is multiplied.  A is copied to LDS by direct-to-LDS loads issued
// between the first two weight batches and waited for once (16-byte unit u
// of row m at u ^ (m & 7): the 8 tokens' reads at one K offset fall on
// distinct banks); tokens >= T enter as zeros.  The waves' partial sums meet
// in LDS in a fixed order.  Needs K a multiple of 512 * NW (the A copy) and
// at least 2 * kDenseU * kKStep * NW (every wave then runs two or more whole
// batches; the launcher asks for K >= 4096).  HBM bound:
// N*K*2 bytes of W per launch.
constexpr int kDenseStreamMaxT = 8;
constexpr int kDenseU = 1;  // chunks per batch (1 measured 4% faster than 2 or 4: fewer bytes in flight)

template <int OUT, int NW>
__global__ __launch_bounds__(64 * NW) void dense_stream_kernel(const uint16_t *__restrict__ A,
                                                               const uint16_t *__restrict__ W, void *C,
                                                               int T, int N, int K, const DenseGate gate)
{
    extern __shared__ uint4 as4[];  // [T][K/8] swizzled units
    __shared__ floatx4_t red[NW - 1][2][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r8 = lane & 7, kg = lane >> 3;  // row in the octet / token; K group of 8
    const int row0 = blockIdx.x * 16;
    const int nc = K / kKStep;
    const int c0 = wv * nc / NW, c1 = (wv + 1) * nc / NW;
    // loads (half h, octet o) of chunk c: W[row0 + 8o + r8][128c + 64h + 8kg .. +7]
    const uint16_t *wp = W + (int64_t)(row0 + r8) * K + 8 * kg;
    const int64_t oct = (int64_t)8 * K;
    uint4 b0[kDenseU][4], b1[kDenseU][4];  // [chunk][2h + o]
    auto load = [&](uint4 (&b)[kDenseU][4], int c) {
#pragma unroll
        for (int u = 0; u < kDenseU; ++u)
            if (c + u < c1) {
                const uint16_t *p = wp + (int64_t)(c + u) * kKStep;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int o = 0; o < 2; ++o) b[u][2 * h + o] = ld_stream16(p + o * oct + 64 * h);
            }
    };
    load(b0, c0);
    // A: LDS unit P = 64 * (NW j + wv) + lane holds logical unit (P % ku) ^ (m & 7)
    // of row m = P / ku (ku = K/8 is a multiple of 64, so a wave's 64 units
    // lie in one row)
    const int ku = K / 8;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    for (int j = 0; j < T * ku / (64 * NW); ++j) {
        const int P0 = 64 * (NW * j + wvu);
        const int m = P0 / ku, cu = P0 - m * ku + lane;
        dma16(A + (int64_t)m * K + (cu ^ (m & 7)) * 8, lds_off(as4 + P0));
    }
    load(b1, c0 + kDenseU);
    // A and the first batch have landed once at most the second batch's
    // kDenseU * 4 loads are outstanding
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(kDenseU * 4) : "memory");
    floatx4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const bool arow = r8 < T;
    auto consume = [&](const uint4 (&b)[kDenseU][4], int c) {
#pragma unroll
        for (int u = 0; u < kDenseU; ++u)
            if (c + u < c1) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int unit = 16 * (c + u) + 8 * h + kg;
                    const uint4 a = arow ? as4[r8 * ku + (unit ^ r8)] : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int o = 0; o < 2; ++o) acc[o] = mfma16(as_bf16x8(a), as_bf16x8(b[u][2 * h + o]), acc[o]);
                }
            }
    };
    for (int c = c0; c < c1; c += 2 * kDenseU) {
        consume(b0, c);
        if (c + 2 * kDenseU < c1) load(b0, c + 2 * kDenseU);
        if (c + kDenseU < c1) {
            consume(b1, c + kDenseU);
            if (c + 3 * kDenseU < c1) load(b1, c + 3 * kDenseU);
        }
    }
    // the two diagonal blocks: lane L (L % 16 < 8, L < 32) adds lane L + 40
    // and then holds token 4(L/16) + r, row 8o + L%16
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[o][r] += __shfl_down(acc[o][r], 40);
    if (wv > 0) {
        red[wv - 1][0][lane] = acc[0];
        red[wv - 1][1][lane] = acc[1];
    }
    __syncthreads();
    if (wv != 0 || (lane & 15) >= 8 || lane >= 32) return;
#pragma unroll
    for (int o = 0; o < 2; ++o) {
        floatx4_t v = acc[o];
#pragma unroll
        for (int w = 0; w < NW - 1; ++w) v += red[w][o][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * (lane >> 4) + r;
            if (t < T) {
                const int col = row0 + 8 * o + (lane & 7);
                const int64_t idx = (int64_t)t * N + col;
                store_dense<OUT>(C, idx, col, v[r], gate);
            }
        }
    }
}

// ---- many tokens: LDS-tiled bf16 MFMA GEMM ----------------------------------------
// 256 tokens x 256 output columns per workgroup, K in steps of 32, a
// four-stage LDS ring filled by direct-to-LDS loads (each stage 256 A rows
// and 256 W rows of 64 bytes; 16-byte slot q of row r at q ^ ((r >> 1) & 3),
// so the fragment reads of 16 consecutive rows fall on distinct banks).  8
// waves as 2 (tokens) x 4 (columns), 128 x 64 each: 8 x 4 blocks of 16 x 16,
// 32 MFMAs per K step.  Token rows past T are loaded as row T-1 and never
// stored.  Tiles are spread over the XCDs in contiguous ranges, row-major,
// so the workgroups sharing an A row panel run on one XCD.  MFMA bound:
// 2*T*N*K flops.
constexpr int kGemmTile = 256;
constexpr int kGemmStages = 4;

template <int OUT>
__global__ __launch_bounds__(512) void dense_gemm_kernel(const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ W, void *C,
                                                         int T, int N, int K, int tiles_m, int tiles_n,
                                                         const DenseGate gate)
{
    constexpr int AU = kGemmTile * 4, BU = kGemmTile * 4;  // 16-byte units per stage
    constexpr int NL = (AU + BU) / 512;                    // loads per thread per stage (4)
    __shared__ uint4 As[kGemmStages][AU];
    __shared__ uint4 Bs[kGemmStages][BU];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int tile;
    if (!xcd_tile(tiles_m * tiles_n, tile)) return;
    const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
    const int M0 = tm * kGemmTile, N0 = tn * kGemmTile;
    const int nk = K / 32;
    // load j of this thread: stage unit u = 512 j + tid (A units first)
    const uint16_t *src[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int u = 512 * j + tid;
        const int v = u < AU ? u : u - AU;
        const int r = v >> 2, q = (v & 3) ^ ((r >> 1) & 3);
        src[j] = u < AU ? A + (int64_t)min(M0 + r, T - 1) * K + q * 8
                        : W + (int64_t)(N0 + r) * K + q * 8;
    }
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    auto issue = [&](int kc) {
        const int b = kc % kGemmStages;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int u0 = 512 * j + 64 * wvu;  // unit of lane 0
            const uint32_t dst = u0 < AU ? lds_off(&As[b][u0]) : lds_off(&Bs[b][u0 - AU]);
            dma16(src[j] + kc * 32, dst);
        }
    };
    const int wm = wv & 1, wn = wv >> 1;
    const int m16 = lane & 15, g = lane >> 4;
    floatx4_t acc[8][4];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < kGemmStages - 1 && s < nk; ++s) issue(s);
    for (int kc = 0; kc < nk; ++kc) {
        // stage kc complete; the stages issued after it may stay in flight
        const int ahead = min(kGemmStages - 2, nk - 1 - kc);
        if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(2 * NL) : "memory");
        else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(NL) : "memory");
        else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // the slot refilled now was last read in step kc-1, before the barrier
        if (kc + kGemmStages - 1 < nk) issue(kc + kGemmStages - 1);
        const uint4 *Ab = As[kc % kGemmStages];
        const uint4 *Bb = Bs[kc % kGemmStages];
        uint4 bw[4], a[8];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int r = wn * 64 + nb * 16 + m16;
            bw[nb] = Bb[r * 4 + (g ^ ((r >> 1) & 3))];
        }
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int r = wm * 128 + mb * 16 + m16;
            a[mb] = Ab[r * 4 + (g ^ ((r >> 1) & 3))];
        }
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma16(as_bf16x8(a[mb]), as_bf16x8(bw[nb]), acc[mb][nb]);
    }
    // lane holds C[token g*4 + r][column m16] of every 16 x 16 block
    if constexpr (OUT == kDenseGate) {
        // the gated residual: alpha and beta once per column, and each row
        // block's 16 x values loaded together before its stores
        float al[4], be[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int col = N0 + wn * 64 + nb * 16 + m16;
            al[nb] = gate.alpha[col];
            be[nb] = gate.beta[col];
        }
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            uint32_t xv[4][4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = min(M0 + wm * 128 + mb * 16 + g * 4 + r, T - 1);  // rows past T: read, not stored
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) xv[r][nb] = gate.x[(int64_t)t * N + N0 + wn * 64 + nb * 16 + m16];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = M0 + wm * 128 + mb * 16 + g * 4 + r;
                if (t >= T) continue;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int col = N0 + wn * 64 + nb * 16 + m16;
                    const float xf = __uint_as_float(xv[r][nb] << 16);
                    static_cast<uint16_t *>(C)[(int64_t)t * N + col] =
                        f32_to_bf16(fmaf(be[nb], acc[mb][nb][r], al[nb] * xf));
                }
            }
        }
        return;
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = M0 + wm * 128 + mb * 16 + g * 4 + r;
            if (t >= T) continue;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int col = N0 + wn * 64 + nb * 16 + m16;
                store_dense<OUT>(C, (int64_t)t * N + col, col, acc[mb][nb][r], gate);
            }
        }
}

template <int OUT>
static hipError_t launch_dense_out(const uint16_t *a, const uint16_t *w, void *c, int T, int N, int K,
                                   hipStream_t st, const DenseGate &g)
{
    if (T <= 0) return hipSuccess;
    // few tokens with their rows in LDS (at most 128 KB): the weight stream
    const size_t lds = (size_t)T * K * 2;
    // the A copy needs T*K/8 divisible by 64 * NW for any T: K % (512 * NW) == 0
    if (T <= kDenseStreamMaxT && lds <= 128 * 1024 && N % 16 == 0 && K % 2048 == 0 && K >= 4096) {
        if (K % 4096 == 0 && K >= 8192)  // 8 waves
            dense_stream_kernel<OUT, 8><<<N / 16, 512, lds, st>>>(a, w, c, T, N, K, g);
        else
            dense_stream_kernel<OUT, 4><<<N / 16, 256, lds, st>>>(a, w, c, T, N, K, g);
        return hipGetLastError();
    }
    if (N % kGemmTile != 0 || K % 32 != 0) return hipErrorInvalidValue;
    const int tiles_m = (T + kGemmTile - 1) / kGemmTile, tiles_n = N / kGemmTile;
    const int64_t grid = 8 * (((int64_t)tiles_m * tiles_n + 7) / 8);
    dense_gemm_kernel<OUT><<<(unsigned)grid, 512, 0, st>>>(a, w, c, T, N, K, tiles_m, tiles_n, g);
    return hipGetLastError();
}

hipError_t launch_dense(const uint16_t *a, const uint16_t *w, void *c, int out, int T, int N, int K,
                        hipStream_t st, const DenseGate &g)
{
    if (out == kDenseGate && (!g.x || !g.alpha || !g.beta)) return hipErrorInvalidValue;
    if (out == kDenseF32) return launch_dense_out<kDenseF32>(a, w, c, T, N, K, st, g);
    if (out == kDenseGate) return launch_dense_out<kDenseGate>(a, w, c, T, N, K, st, g);
    return launch_dense_out<kDenseBf16>(a, w, c, T, N, K, st, g);
}

}  // namespace moe
