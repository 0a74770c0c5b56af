/* The oracle (oracle/oracle.c) under the address and undefined-behaviour
 * sanitizers: reads the tiny layer's inputs from a directory of raw files
 * written by tests/test_sanitizers.py, runs routing, grouping, the layer,
 * the block and the 16-block layer, and writes their outputs back for the
 * test to compare with the regular build's. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_moe_forward(int T, int d, int E, int F, int k, double eps, const uint16_t *x,
                       const float *wr, const uint8_t *wpk, const uint8_t *sc, const float *alpha,
                       const float *beta, int n_sel, const int32_t *sel, double *s_out,
                       int32_t *ids_out, double *w_out);
int oracle_moe_forward_nv(int T, int d, int E, int F, int k, double eps, const uint16_t *x,
                          const float *wr, const uint8_t *wpk, const uint8_t *sc16, const float *gs,
                          const float *alpha, const float *beta, int n_sel, const int32_t *sel,
                          double *s_out, int32_t *ids_out, double *w_out);
int oracle_block_forward(int T, int d, int E, int F, int k, double eps, const uint16_t *x,
                         const float *gamma_pre, const float *wr, const uint8_t *wpk,
                         const uint8_t *sc, const float *gamma_post, const float *alpha,
                         const float *beta, int n_sel, const int32_t *sel, const uint16_t *xn_in,
                         double *s_out, int32_t *ids_out, double *w_out);
void oracle_group(int T, int E, int k, const int32_t *ids, int32_t *counts, int32_t *offsets,
                  int32_t *perm, int32_t *inv);

static void *load(const char *dir, const char *name, size_t n)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) { perror(path); exit(2); }
    void *p = malloc(n);
    if (fread(p, 1, n, f) != n) { fprintf(stderr, "short read %s\n", path); exit(2); }
    fclose(f);
    return p;
}

static void save(const char *dir, const char *name, const void *p, size_t n)
{
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, n, f) != n) { perror(path); exit(2); }
    fclose(f);
}

int main(int argc, char **argv)
{
    if (argc != 7) { fprintf(stderr, "usage: dir T d E F k\n"); return 2; }
    const char *dir = argv[1];
    const int T = atoi(argv[2]), d = atoi(argv[3]), E = atoi(argv[4]), F = atoi(argv[5]), k = atoi(argv[6]);
    const size_t S = (size_t)T * k;
    uint16_t *x = load(dir, "x", sizeof(uint16_t) * T * d);
    float *wr = load(dir, "wr", sizeof(float) * E * d);
    uint8_t *w = load(dir, "w", (size_t)E * 3 * d * F / 2);
    uint8_t *sc = load(dir, "sc", (size_t)E * 3 * d * F / 32);
    uint8_t *sc16 = load(dir, "sc16", (size_t)E * 3 * d * F / 16);
    float *gs = load(dir, "gs", sizeof(float) * E * 3);
    float *a = load(dir, "alpha", sizeof(float) * d);
    float *b = load(dir, "beta", sizeof(float) * d);
    float *gpre = load(dir, "gpre", sizeof(float) * d);
    float *gpost = load(dir, "gpost", sizeof(float) * d);
    double *s = malloc(sizeof(double) * T * d);
    int32_t *ids = malloc(sizeof(int32_t) * S);
    double *wt = malloc(sizeof(double) * S);
    int32_t *counts = malloc(sizeof(int32_t) * E), *offsets = malloc(sizeof(int32_t) * (E + 1));
    int32_t *perm = malloc(sizeof(int32_t) * S), *inv = malloc(sizeof(int32_t) * S);
    int rc = oracle_moe_forward(T, d, E, F, k, 1e-6, x, wr, w, sc, a, b, 0, NULL, s, ids, wt);
    save(dir, "out_layer", s, sizeof(double) * T * d);
    save(dir, "out_ids", ids, sizeof(int32_t) * S);
    oracle_group(T, E, k, ids, counts, offsets, perm, inv);
    save(dir, "out_perm", perm, sizeof(int32_t) * S);
    rc |= oracle_block_forward(T, d, E, F, k, 1e-6, x, gpre, wr, w, sc, gpost, a, b, 0, NULL, NULL, s,
                               ids, wt);
    save(dir, "out_block", s, sizeof(double) * T * d);
    rc |= oracle_moe_forward_nv(T, d, E, F, k, 1e-6, x, wr, w, sc16, gs, a, b, 0, NULL, s, ids, wt);
    save(dir, "out_nv", s, sizeof(double) * T * d);
    free(x); free(wr); free(w); free(sc); free(sc16); free(gs); free(a); free(b); free(gpre);
    free(gpost); free(s); free(ids); free(wt); free(counts); free(offsets); free(perm); free(inv);
    printf("oracle under sanitizers: rc %d\n", rc);
    return rc ? 1 : 0;
}
