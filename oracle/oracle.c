/*
 * oracle.c -- plain, slow CPU reference for the MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with
 * the GPU kernels.
 *
 * What it computes, step by step, with the passage each step follows:
 *
 *   The source pages are
 *     [MS]  "Muse Spark Open を段階的に分解する" (animemo.app), sections ①-⑭
 *     [TS]  "TensorSharp ... Muse Spark 816B" benchmark article (devotd.net),
 *           section "性能" / "Performance"
 *     [DG]  "DGX Spark MoE inference optimizations" article (devotd.net),
 *           section 2
 *
 *   O1  x is bf16; it is widened to double exactly.
 *   O2  router score of token t for expert e: one matrix product of the
 *       token vector with the router matrix, done in FP32 ([MS] section ⑧).
 *       Reading: the score is the fp32 rounding of the exact dot product
 *       (accumulated here in double in index order, every product exact).
 *   O3  each token picks the 8 (k) best-scoring experts ([MS] section ⑧);
 *       reading: order by score descending, then expert id ascending.
 *   O4  the chosen experts' outputs are weighted by the router's scores and
 *       the weights of one token sum to one ([MS] section ⑨ figure);
 *       reading: softmax over the k chosen scores, in double.
 *   O5  tokens are gathered per expert so each expert runs its batch at once
 *       ([MS] section ⑫); reading: slot id t*k+j, ordered by
 *       (expert asc, token asc); offsets = exclusive prefix of counts.
 *   O6  each expert is gate / up / down ([MS] section ⑨): gate decides what
 *       passes, up how much, down maps back.  Reading: SwiGLU,
 *       a_f = silu(g_f) * u_f with silu(z) = z / (1 + exp(-z)).
 *       Weights are block-scaled 4-bit ([MS] section ⑪, MXFP4 named in [DG]
 *       section 2): FP4 E2M1 codes (sign bit 3, exponent bits 2..1 with bias
 *       1, mantissa bit 0; exponent 0 is the subnormal 0 / 0.5) times an
 *       E8M0 scale 2^(s-127) shared by 32 consecutive K elements of a row.
 *       Byte b of a row holds element 2b in its low nibble, 2b+1 in its high.
 *   O7  every expert output is normalised before the weighted sum
 *       ([MS] section ⑨; [TS] "性能": the per-expert normalisation is why
 *       tensor parallelism moves 8x the data).  Reading: RMSNorm over d with
 *       eps inside the square root and no learned gain.
 *   O8  y_t = sum_j w_tj * n_tj (j in order), and the gated residual
 *       s = alpha * x + beta * y, alpha and beta learned per dimension
 *       ([MS] section ③).  Output kept in double.
 *
 * Expert weight layout (per expert e, all row-major):
 *   bytes  at e*(3dF/2):  gate [F][d/2] | up [F][d/2] | down [d][F/2]
 *   scales at e*(3dF/32): gate [F][d/32] | up [F][d/32] | down [d][F/32]
 *
 * The 16-element block format (NV1-NV3 below, [MS] section ⑪) uses the same
 * code bytes, scales at e*(3dF/16) (gate [F][d/16] | up [F][d/16] |
 * down [d][F/16]) and three fp32 matrix scales per expert (gate, up, down).
 *
 * Every function is deterministic for any OpenMP thread count: parallel
 * loops only run independent rows/slots and write disjoint outputs.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads the parallel loops below use from now on (n >= 1), and the
 * current count; for timing the oracle on a given number of host cores. */
void oracle_set_num_threads(int n)
{
    if (n >= 1) omp_set_num_threads(n);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

/* ---- O1 / O6: number formats ------------------------------------------ */

double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* fp64 -> bf16 bits, round to nearest, ties to even (finite inputs). */
uint16_t oracle_double_to_bf16(double v)
{
    /* bf16 keeps 8 significant bits; find the two neighbours and pick. */
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return 0x7FC0u;
    int neg = v < 0;
    double a = neg ? -v : v;
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;                /* a in [2^e, 2^(e+1)) */
    if (e < -126) e = -126;        /* bf16 subnormal range: fixed quantum */
    double q = ldexp(1.0, e - 7);  /* spacing of bf16 values near a */
    double lo = floor(a / q) * q;
    double hi = lo + q;
    double r;
    if (a - lo < hi - a) r = lo;
    else if (a - lo > hi - a) r = hi;
    else r = (fmod(lo / q, 2.0) == 0.0) ? lo : hi;
    float f = (float)r;            /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t b = (uint16_t)(u >> 16);
    if (isinf(f)) b = 0x7F80u;
    return (uint16_t)(b | (neg ? 0x8000u : 0u));
}

double oracle_e2m1(unsigned code)
{
    unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return s ? -mag : mag;
}

double oracle_e8m0(unsigned s)
{
    if (s == 255u) return NAN;
    return ldexp(1.0, (int)s - 127);
}

/*
 * NV1  [MS] section ⑪: the released 4-bit format shares one small scale per
 *      16 values, about 4.5 bits per value (4 + 8/16: an 8-bit scale).  The
 *      pages do not give the scale's encoding.  Reading: the scale byte is an
 *      FP8 E4M3 number (sign bit 7, exponent bits 6..3 with bias 7, mantissa
 *      bits 2..0; exponent 0 is subnormal, 2^-6 * m/8; exponent 15 with
 *      mantissa 7 is NaN; no infinities), as in the published NVFP4 format.
 */
double oracle_e4m3(unsigned b)
{
    unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
    if (e == 15u && m == 7u) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* value tables filled from the functions above when the library loads */
static double e2m1_tab[16], e8m0_tab[256], e4m3_tab[256];

__attribute__((constructor)) static void fill_tables(void)
{
    for (unsigned c = 0; c < 16; ++c) e2m1_tab[c] = oracle_e2m1(c);
    for (unsigned s = 0; s < 256; ++s) e8m0_tab[s] = oracle_e8m0(s);
    for (unsigned s = 0; s < 256; ++s) e4m3_tab[s] = oracle_e4m3(s);
}

/* element i of a packed row of K elements */
static double fp4_elem(const uint8_t *row, const uint8_t *srow, int64_t i)
{
    uint8_t byte = row[i / 2];
    unsigned code = (i & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
    return e2m1_tab[code] * e8m0_tab[srow[i / 32]];
}

void oracle_dequant_rows(int64_t rows, int64_t K, const uint8_t *codes,
                         const uint8_t *scales, double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < K; ++i)
            out[r * K + i] = fp4_elem(codes + r * (K / 2), scales + r * (K / 32), i);
}

/*
 * NV2  element i of a row in the 16-block format: the E2M1 code times the
 *      E4M3 scale of its 16-block times the matrix's fp32 scale g.  Reading:
 *      the published NVFP4 format also carries one fp32 scale per tensor;
 *      here one per matrix of an expert (1.0 leaves the block scales alone).
 */
static double nv_elem(const uint8_t *row, const uint8_t *srow, double g, int64_t i)
{
    uint8_t byte = row[i / 2];
    unsigned code = (i & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
    return e2m1_tab[code] * e4m3_tab[srow[i / 16]] * g;
}

void oracle_dequant_rows_nv(int64_t rows, int64_t K, const uint8_t *codes,
                            const uint8_t *scales, double g, double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < K; ++i)
            out[r * K + i] = nv_elem(codes + r * (K / 2), scales + r * (K / 16), g, i);
}

/* One expert matrix in either block format. */
typedef struct {
    const uint8_t *codes, *scales;
    int64_t K;  /* elements per row */
    int nv;     /* 0: E8M0 per 32, 1: E4M3 per 16 times g */
    double g;
} wmat_t;

/* element i of row `row` of a matrix; nv is the matrix's format, passed
 * separately so the loops below test it once per row, not per element */
static inline double wm_get(const wmat_t *m, int nv, int64_t row, int64_t i)
{
    const uint8_t *c = m->codes + row * (m->K / 2);
    return nv ? nv_elem(c, m->scales + row * (m->K / 16), m->g, i)
              : fp4_elem(c, m->scales + row * (m->K / 32), i);
}

/* ---- O2: router scores ------------------------------------------------- */

void oracle_router_scores(int T, int d, int E, const uint16_t *x, const float *wr,
                          float *scores)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += oracle_bf16_to_double(x[(int64_t)t * d + i]) * (double)wr[(int64_t)e * d + i];
            scores[(int64_t)t * E + e] = (float)acc;
        }
}

/* ---- O3 / O4: top-k and weights ---------------------------------------- */

void oracle_topk_softmax(int T, int E, int k, const float *scores, int32_t *ids, double *w)
{
    char *taken = (char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *l = scores + (int64_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;  /* ties keep the lower id */
            }
            taken[best] = 1;
            ids[(int64_t)t * k + j] = best;
        }
        double l0 = (double)l[ids[(int64_t)t * k]];
        double z = 0.0;
        for (int j = 0; j < k; ++j) z += exp((double)l[ids[(int64_t)t * k + j]] - l0);
        for (int j = 0; j < k; ++j)
            w[(int64_t)t * k + j] = exp((double)l[ids[(int64_t)t * k + j]] - l0) / z;
    }
    free(taken);
}

/* ---- O5: grouping by expert --------------------------------------------- */

void oracle_group(int T, int E, int k, const int32_t *ids, int32_t *counts,
                  int32_t *offsets, int32_t *perm, int32_t *inv)
{
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t s = 0; s < (int64_t)T * k; ++s) counts[ids[s]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int64_t pos = 0;
    for (int e = 0; e < E; ++e)
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j)
                if (ids[(int64_t)t * k + j] == e) {
                    perm[pos] = t * k + j;
                    inv[t * k + j] = (int32_t)pos;
                    ++pos;
                }
}

/* ---- O6 / O7: one expert on one token ----------------------------------- */

/*
 * x: d doubles.  w_e / s_e: the expert's packed bytes and scales.
 * o_out (d) receives the down projection, n_out (d) its RMS-normalised form;
 * either may be NULL.  Returns the mean square of o.
 */
/* O6 / O7 on matrices of either format (see oracle_expert). */
static double expert_mats(int d, int F, const wmat_t *gate, const wmat_t *up,
                          const wmat_t *down, const double *x, double eps, double *o_out,
                          double *n_out)
{
    double *a = (double *)malloc(sizeof(double) * (size_t)F);
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    const int nv = gate->nv;  /* the three matrices share one format */
    for (int f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        if (nv)
            for (int i = 0; i < d; ++i) {
                g += wm_get(gate, 1, f, i) * x[i];
                u += wm_get(up, 1, f, i) * x[i];
            }
        else
            for (int i = 0; i < d; ++i) {
                g += wm_get(gate, 0, f, i) * x[i];
                u += wm_get(up, 0, f, i) * x[i];
            }
        a[f] = g / (1.0 + exp(-g)) * u;
    }
    double ss = 0.0;
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        if (nv)
            for (int f = 0; f < F; ++f) acc += wm_get(down, 1, i, f) * a[f];
        else
            for (int f = 0; f < F; ++f) acc += wm_get(down, 0, i, f) * a[f];
        o[i] = acc;
        ss += acc * acc;
    }
    double ms = ss / (double)d;
    double r = 1.0 / sqrt(ms + eps);
    for (int i = 0; i < d; ++i) {
        if (o_out) o_out[i] = o[i];
        if (n_out) n_out[i] = o[i] * r;
    }
    free(a);
    free(o);
    return ms;
}

/* the three matrices of expert e: nv = 0 MXFP4, nv = 1 the 16-block format */
static void expert_view(int d, int F, int nv, const uint8_t *wpk, const uint8_t *sc,
                        const float *gs, int e, wmat_t m[3])
{
    const uint8_t *w_e = wpk + (int64_t)e * ((int64_t)3 * d * F / 2);
    const int64_t bs = nv ? 16 : 32;
    const uint8_t *s_e = sc + (int64_t)e * ((int64_t)3 * d * F / bs);
    m[0] = (wmat_t){w_e, s_e, d, nv, nv ? (double)gs[3 * e] : 1.0};
    m[1] = (wmat_t){w_e + (int64_t)F * (d / 2), s_e + (int64_t)F * (d / bs), d, nv,
                    nv ? (double)gs[3 * e + 1] : 1.0};
    m[2] = (wmat_t){w_e + (int64_t)2 * F * (d / 2), s_e + (int64_t)2 * F * (d / bs), F, nv,
                    nv ? (double)gs[3 * e + 2] : 1.0};
}

double oracle_expert(int d, int F, const uint8_t *w_e, const uint8_t *s_e, const double *x,
                     double eps, double *o_out, double *n_out)
{
    wmat_t m[3];
    expert_view(d, F, 0, w_e, s_e, NULL, 0, m);
    return expert_mats(d, F, &m[0], &m[1], &m[2], x, eps, o_out, n_out);
}

/* NV3  O6 / O7 for one expert of the 16-block format; gs: its 3 matrix scales. */
double oracle_expert_nv(int d, int F, const uint8_t *w_e, const uint8_t *s_e, const float *gs,
                        const double *x, double eps, double *o_out, double *n_out)
{
    wmat_t m[3];
    expert_view(d, F, 1, w_e, s_e, gs, 0, m);
    return expert_mats(d, F, &m[0], &m[1], &m[2], x, eps, o_out, n_out);
}

/* ---- whole layer on a set of tokens -------------------------------------- */

/*
 * Runs O1-O8 for the tokens listed in sel (n_sel of them; sel == NULL means
 * all T tokens in order).  s_out: [n_sel][d] doubles.  ids_out [n_sel][k]
 * and w_out [n_sel][k] receive the routing when non-NULL.
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
static int moe_forward(int T, int d, int E, int F, int k, double eps, const uint16_t *x,
                       const float *wr, int nv, const uint8_t *wpk, const uint8_t *sc,
                       const float *gs, const float *alpha, const float *beta, int n_sel,
                       const int32_t *sel, double *s_out, int32_t *ids_out, double *w_out)
{
    if (T < 0 || d <= 0 || E <= 0 || F <= 0 || k < 1 || k > E || d % 32 || F % 32) return -1;
    if (sel == NULL) n_sel = T;
    if (n_sel <= 0) return 0;

    uint16_t *xs = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n_sel * d);
    float *scores = (float *)malloc(sizeof(float) * (size_t)n_sel * E);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_sel * k);
    double *w = (double *)malloc(sizeof(double) * (size_t)n_sel * k);
    double *n = (double *)malloc(sizeof(double) * (size_t)n_sel * k * d);
    if (!xs || !scores || !ids || !w || !n) {
        free(xs); free(scores); free(ids); free(w); free(n);
        return -1;
    }
    for (int r = 0; r < n_sel; ++r) {
        int t = sel ? sel[r] : r;
        memcpy(xs + (int64_t)r * d, x + (int64_t)t * d, sizeof(uint16_t) * (size_t)d);
    }
    oracle_router_scores(n_sel, d, E, xs, wr, scores);
    oracle_topk_softmax(n_sel, E, k, scores, ids, w);

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < (int64_t)n_sel * k; ++q) {
        int64_t r = q / k;
        int e = ids[q];
        double *xd = (double *)malloc(sizeof(double) * (size_t)d);
        for (int i = 0; i < d; ++i) xd[i] = oracle_bf16_to_double(xs[r * d + i]);
        wmat_t m[3];
        expert_view(d, F, nv, wpk, sc, gs, e, m);
        expert_mats(d, F, &m[0], &m[1], &m[2], xd, eps, NULL, n + q * d);
        free(xd);
    }

    for (int64_t r = 0; r < n_sel; ++r)
        for (int i = 0; i < d; ++i) {
            double y = 0.0;
            for (int j = 0; j < k; ++j) y += w[r * k + j] * n[(r * k + j) * d + i];
            s_out[r * d + i] = (double)alpha[i] * oracle_bf16_to_double(xs[r * d + i]) +
                               (double)beta[i] * y;
        }
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)n_sel * k);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)n_sel * k);
    free(xs); free(scores); free(ids); free(w); free(n);
    return 0;
}

int oracle_moe_forward(int T, int d, int E, int F, int k, double eps,
                       const uint16_t *x, const float *wr, const uint8_t *wpk,
                       const uint8_t *sc, const float *alpha, const float *beta,
                       int n_sel, const int32_t *sel, double *s_out,
                       int32_t *ids_out, double *w_out)
{
    return moe_forward(T, d, E, F, k, eps, x, wr, 0, wpk, sc, NULL, alpha, beta, n_sel, sel,
                       s_out, ids_out, w_out);
}

/*
 * The layer (O1-O8) with expert weights in the 16-block format (NV1-NV3):
 * codes as oracle_moe_forward, sc16 E4M3 bytes at e*(3dF/16), gs fp32 [E][3]
 * (gate, up, down).  Same arguments otherwise.
 */
int oracle_moe_forward_nv(int T, int d, int E, int F, int k, double eps,
                          const uint16_t *x, const float *wr, const uint8_t *wpk,
                          const uint8_t *sc16, const float *gs, const float *alpha,
                          const float *beta, int n_sel, const int32_t *sel, double *s_out,
                          int32_t *ids_out, double *w_out)
{
    if (!gs || d % 16 || F % 16) return -1;
    return moe_forward(T, d, E, F, k, eps, x, wr, 1, wpk, sc16, gs, alpha, beta, n_sel, sel,
                       s_out, ids_out, w_out);
}

/* ---- latent-width variant ----------------------------------------------- */

/*
 * [MS] section ⑨: the chosen experts do not take the token at its full
 * width.  A matrix shared by all of them first narrows the token (8,192 to
 * 4,096 on the page); each chosen expert runs gate / up / down at that
 * width; the outputs are normalised and summed with the router weights; a
 * second shared matrix widens the sum back before it joins the residual.
 *
 *   L1  routing (O2-O4) on the full-width token x: the router reads the
 *       token vector itself ([MS] section ⑧ figure).
 *   L2  z = Wc x, Wc [d][D] bf16.  Reading: the shared matrices are bf16;
 *       the pages give a 4-bit format for the expert weights only ([MS]
 *       section ⑪).  Kept in double.
 *   L3  O6 / O7 for each chosen expert on z, at width d.
 *   L4  y = sum_j w_j n_j (width d, j in order), then f = We y with
 *       We [D][d] bf16, in double.
 *   L5  s = alpha * x + beta * f at width D (O8's gate).
 *
 * Arguments as oracle_moe_forward, plus D (token width), wc and we (bf16
 * bits, row-major).  Expert weights are laid out for width d.
 */
int oracle_latent_forward(int T, int D, int d, int E, int F, int k, double eps,
                          const uint16_t *x, const float *wr, const uint16_t *wc,
                          const uint8_t *wpk, const uint8_t *sc, const uint16_t *we,
                          const float *alpha, const float *beta, int n_sel,
                          const int32_t *sel, double *s_out, int32_t *ids_out, double *w_out)
{
    if (T < 0 || D <= 0 || d <= 0 || E <= 0 || F <= 0 || k < 1 || k > E || D % 32 || d % 32 ||
        F % 32)
        return -1;
    if (sel == NULL) n_sel = T;
    if (n_sel <= 0) return 0;
    const int64_t eb = (int64_t)3 * d * F / 2, esb = (int64_t)3 * d * F / 32;

    uint16_t *xs = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n_sel * D);
    float *scores = (float *)malloc(sizeof(float) * (size_t)n_sel * E);
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_sel * k);
    double *w = (double *)malloc(sizeof(double) * (size_t)n_sel * k);
    double *z = (double *)malloc(sizeof(double) * (size_t)n_sel * d);
    double *n = (double *)malloc(sizeof(double) * (size_t)n_sel * k * d);
    double *y = (double *)malloc(sizeof(double) * (size_t)n_sel * d);
    if (!xs || !scores || !ids || !w || !z || !n || !y) {
        free(xs); free(scores); free(ids); free(w); free(z); free(n); free(y);
        return -1;
    }
    for (int r = 0; r < n_sel; ++r) {
        int t = sel ? sel[r] : r;
        memcpy(xs + (int64_t)r * D, x + (int64_t)t * D, sizeof(uint16_t) * (size_t)D);
    }
    /* L1 */
    oracle_router_scores(n_sel, D, E, xs, wr, scores);
    oracle_topk_softmax(n_sel, E, k, scores, ids, w);

    /* L2 */
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < (int64_t)n_sel * d; ++q) {
        const int64_t r = q / d, j = q % d;
        double acc = 0.0;
        for (int i = 0; i < D; ++i)
            acc += oracle_bf16_to_double(wc[j * D + i]) * oracle_bf16_to_double(xs[r * D + i]);
        z[q] = acc;
    }

    /* L3 */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < (int64_t)n_sel * k; ++q) {
        const int64_t r = q / k;
        const int e = ids[q];
        oracle_expert(d, F, wpk + (int64_t)e * eb, sc + (int64_t)e * esb, z + r * d, eps, NULL,
                      n + q * d);
    }

    /* L4, L5 */
    for (int64_t r = 0; r < n_sel; ++r)
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int s = 0; s < k; ++s) acc += w[r * k + s] * n[(r * k + s) * d + j];
            y[r * d + j] = acc;
        }
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < (int64_t)n_sel * D; ++q) {
        const int64_t r = q / D, i = q % D;
        double f = 0.0;
        for (int j = 0; j < d; ++j) f += oracle_bf16_to_double(we[i * d + j]) * y[r * d + j];
        s_out[q] = (double)alpha[i] * oracle_bf16_to_double(xs[r * D + i]) + (double)beta[i] * f;
    }
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)n_sel * k);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)n_sel * k);
    free(xs); free(scores); free(ids); free(w); free(z); free(n); free(y);
    return 0;
}

/* ---- the block with its stream norms -------------------------------------- */

/*
 * [MS] section ③: the MoE part of a layer does not write the residual stream
 * s directly.  A copy of s is normalised and run through the part; the
 * part's output is normalised as well and mixed in by the gate,
 * s <- alpha * s + beta * norm(output).
 *
 *   B1  x_n = bf16(s * r_s * gamma_pre), r_s = 1 / sqrt(mean(s^2) + eps):
 *       RMSNorm with a learned per-dimension gain.  Reading: the normalised
 *       copy enters the block as bf16, like every activation handed between
 *       kernels; the rounding is part of the definition because the
 *       router's choice depends on it.
 *   B2  O2-O7 on x_n, and y = sum_j w_j n_j (O8 without the gate), double.
 *   B3  s_out = alpha * s + beta * (y * r_y * gamma_post),
 *       r_y = 1 / sqrt(mean(y^2) + eps).  Kept in double.
 */

/* B1 on the rows listed in sel (all T when sel == NULL): xn [n_sel][d]. */
int oracle_block_prenorm(int T, int d, double eps, const uint16_t *x, const float *gamma_pre,
                         int n_sel, const int32_t *sel, uint16_t *xn)
{
    if (T < 0 || d <= 0) return -1;
    if (sel == NULL) n_sel = T;
    for (int r = 0; r < n_sel; ++r) {
        const int t = sel ? sel[r] : r;
        double ss = 0.0;
        for (int i = 0; i < d; ++i) {
            const double v = oracle_bf16_to_double(x[(int64_t)t * d + i]);
            ss += v * v;
        }
        const double rs = 1.0 / sqrt(ss / (double)d + eps);
        for (int i = 0; i < d; ++i)
            xn[(int64_t)r * d + i] = oracle_double_to_bf16(
                oracle_bf16_to_double(x[(int64_t)t * d + i]) * rs * (double)gamma_pre[i]);
    }
    return 0;
}

/*
 * B1-B3.  Arguments as oracle_moe_forward plus the two gains (fp32 [d]).
 * xn_in: NULL, or the normalised rows [n_sel][d] to use in place of B1's
 * (the rows another implementation computed, so that B2-B3 can be checked
 * on exactly the input it saw).
 */
int oracle_block_forward(int T, int d, int E, int F, int k, double eps, const uint16_t *x,
                         const float *gamma_pre, const float *wr, const uint8_t *wpk,
                         const uint8_t *sc, const float *gamma_post, const float *alpha,
                         const float *beta, int n_sel, const int32_t *sel, const uint16_t *xn_in,
                         double *s_out, int32_t *ids_out, double *w_out)
{
    if (T < 0 || d <= 0 || E <= 0 || F <= 0 || k < 1 || k > E || d % 32 || F % 32) return -1;
    if (sel == NULL) n_sel = T;
    if (n_sel <= 0) return 0;
    uint16_t *xn = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n_sel * d);
    double *y = (double *)malloc(sizeof(double) * (size_t)n_sel * d);
    float *zero = (float *)calloc((size_t)d, sizeof(float));
    float *one = (float *)malloc(sizeof(float) * (size_t)d);
    if (!xn || !y || !zero || !one) {
        free(xn); free(y); free(zero); free(one);
        return -1;
    }
    for (int i = 0; i < d; ++i) one[i] = 1.0f;
    /* B1 */
    if (xn_in)
        memcpy(xn, xn_in, sizeof(uint16_t) * (size_t)n_sel * d);
    else
        oracle_block_prenorm(T, d, eps, x, gamma_pre, n_sel, sel, xn);
    /* B2: the layer on x_n with alpha = 0, beta = 1 returns y */
    int rc = oracle_moe_forward(n_sel, d, E, F, k, eps, xn, wr, wpk, sc, zero, one, n_sel, NULL, y,
                                ids_out, w_out);
    /* B3 */
    if (rc == 0)
        for (int r = 0; r < n_sel; ++r) {
            const int t = sel ? sel[r] : r;
            double ss = 0.0;
            for (int i = 0; i < d; ++i) ss += y[(int64_t)r * d + i] * y[(int64_t)r * d + i];
            const double ry = 1.0 / sqrt(ss / (double)d + eps);
            for (int i = 0; i < d; ++i)
                s_out[(int64_t)r * d + i] =
                    (double)alpha[i] * oracle_bf16_to_double(x[(int64_t)t * d + i]) +
                    (double)beta[i] * (y[(int64_t)r * d + i] * ry * (double)gamma_post[i]);
        }
    free(xn); free(y); free(zero); free(one);
    return rc;
}
