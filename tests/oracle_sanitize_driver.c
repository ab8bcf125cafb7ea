/*
 * oracle_sanitize_driver.c -- runs every entry point of the CPU oracle on
 * small seeded inputs, for a build of the oracle with AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only; tests/test_oracle_sanitize.py
 * compiles and runs it).  Exits 0 when every call returns its expected
 * status; the sanitizers abort the process on the first memory or undefined-
 * behaviour error.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_check_tree(const int32_t *parents, const int32_t *tokens, int B, int V);
int oracle_exit_law(const void *logits, int dtype, const int32_t *parents, const int32_t *tokens,
                    int R, int B, int V, double inv_temperature, double *rho, double *reach,
                    double *exit_mass, double *coverage, double *logZ, int nthreads);
int oracle_residual_cdf(const void *logits, int dtype, const int32_t *parents,
                        const int32_t *tokens, int B, int V, int node, double inv_temperature,
                        double *cdf);
int oracle_sample(const void *logits, int dtype, const int32_t *parents, const int32_t *tokens,
                  int R, int B, int V, double inv_temperature, const double *exit_mass,
                  const float *uniforms, int n_draws, int32_t *exit_node, int32_t *bonus_token,
                  unsigned char *band, int nthreads);
int oracle_predraw(const void *logits, int dtype, const int32_t *parents, const int32_t *tokens,
                   int R, int B, int V, double inv_temperature, const float *uniforms,
                   int n_draws, int32_t *node_draw, int32_t *exit_node, int32_t *bonus_token,
                   unsigned char *band, unsigned char *node_band, int nthreads);
int oracle_tree_attn(const void *q, const void *k, const void *v, int dtype, const int32_t *parents,
                     int R, int B, int Hq, int Hkv, int D, int P, double scale, double *out,
                     const int64_t *rows, int64_t n_rows, int nthreads);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* splitmix64: a seeded source of test inputs only */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static double uniform01(void) { return (double)(next_u64() >> 11) * 0x1.0p-53; }

static int fail(const char *what, int got, int want) {
    fprintf(stderr, "%s returned %d, expected %d\n", what, got, want);
    return 1;
}

/* A random tree with distinct sibling tokens: node i > 0 picks a parent
 * before it and a token not yet used by its siblings. */
static void random_tree(int B, int V, int32_t *par, int32_t *tok) {
    par[0] = -1;
    tok[0] = (int32_t)(next_u64() % (uint64_t)V);
    for (int i = 1; i < B; i++) {
        par[i] = (int32_t)(next_u64() % (uint64_t)i);
        for (;;) {
            int t = (int)(next_u64() % (uint64_t)V), clash = 0;
            for (int j = 1; j < i; j++)
                if (par[j] == par[i] && tok[j] == t) clash = 1;
            if (!clash) { tok[i] = t; break; }
        }
    }
}

int main(void) {
    enum { R = 2, B = 9, V = 300, N = 64, HQ = 4, HKV = 2, D = 64, P = 37 };
    int bad = 0;
    float *logits = malloc(sizeof(float) * R * B * V);
    int32_t par[R * B], tok[R * B];
    for (int r = 0; r < R; r++) random_tree(B, V, par + r * B, tok + r * B);
    for (int i = 0; i < R * B * V; i++) logits[i] = (float)(4.0 * uniform01() - 2.0);
    logits[5] = -INFINITY;   /* -inf is allowed: probability zero */

    double rho[R * B], reach[R * B], w[R * B], cov[R], logZ[R * B];
    int st = oracle_exit_law(logits, 0, par, tok, R, B, V, 1.0, rho, reach, w, cov, logZ, 2);
    if (st != 0) bad |= fail("oracle_exit_law", st, 0);

    double *cdf = malloc(sizeof(double) * V);
    st = oracle_residual_cdf(logits, 0, par, tok, B, V, 0, 1.0, cdf);
    if (st != 0) bad |= fail("oracle_residual_cdf", st, 0);

    float u2[R * N * 2];
    for (int i = 0; i < R * N * 2; i++) u2[i] = (float)((double)(next_u64() >> 40) * 0x1.0p-24);
    int32_t en[R * N], bt[R * N];
    unsigned char band2[R * N * 2];
    st = oracle_sample(logits, 0, par, tok, R, B, V, 1.0, w, u2, N, en, bt, band2, 2);
    if (st != 0) bad |= fail("oracle_sample", st, 0);

    float *ub = malloc(sizeof(float) * R * N * B);
    for (int i = 0; i < R * N * B; i++) ub[i] = (float)((double)(next_u64() >> 40) * 0x1.0p-24);
    int32_t *nd = malloc(sizeof(int32_t) * R * N * B);
    unsigned char *nb = malloc((size_t)R * N * B), band1[R * N];
    st = oracle_predraw(logits, 0, par, tok, R, B, V, 1.0, ub, N, nd, en, bt, band1, nb, 2);
    if (st != 0) bad |= fail("oracle_predraw", st, 0);

    const int nkv = P + B;
    float *q = malloc(sizeof(float) * R * B * HQ * D);
    float *kk = malloc(sizeof(float) * R * HKV * nkv * D);
    float *vv = malloc(sizeof(float) * R * HKV * nkv * D);
    for (int i = 0; i < R * B * HQ * D; i++) q[i] = (float)(uniform01() - 0.5);
    for (int i = 0; i < R * HKV * nkv * D; i++) {
        kk[i] = (float)(uniform01() - 0.5);
        vv[i] = (float)(uniform01() - 0.5);
    }
    double *out = malloc(sizeof(double) * R * B * HQ * D);
    st = oracle_tree_attn(q, kk, vv, 0, par, R, B, HQ, HKV, D, P, 0.125, out, NULL, 0, 2);
    if (st != 0) bad |= fail("oracle_tree_attn (all rows)", st, 0);
    int64_t rows[3] = {0, 7, R * B * HQ - 1};
    st = oracle_tree_attn(q, kk, vv, 0, par, R, B, HQ, HKV, D, P, 0.125, out, rows, 3, 2);
    if (st != 0) bad |= fail("oracle_tree_attn (rows)", st, 0);

    /* error paths: an invalid tree, a NaN row, bad arguments */
    int32_t par_bad[R * B], tok_dup[R * B];
    for (int i = 0; i < R * B; i++) { par_bad[i] = par[i]; tok_dup[i] = tok[i]; }
    par_bad[B + 3] = 5;
    st = oracle_exit_law(logits, 0, par_bad, tok, R, B, V, 1.0, rho, reach, w, cov, logZ, 1);
    if (st != 1) bad |= fail("oracle_exit_law (invalid tree)", st, 1);
    if (oracle_check_tree(par, tok, B, V) != 0) bad |= fail("oracle_check_tree", 1, 0);
    tok_dup[2] = tok_dup[1];
    par_bad[2] = par[1];
    if (oracle_check_tree(par_bad, tok_dup, B, V) == 0) bad |= fail("oracle_check_tree (duplicate)", 0, 1);
    logits[B * V + 17] = NAN;
    st = oracle_exit_law(logits, 0, par, tok, R, B, V, 1.0, rho, reach, w, cov, logZ, 1);
    if (st != 5) bad |= fail("oracle_exit_law (NaN logit)", st, 5);
    st = oracle_tree_attn(q, kk, vv, 0, par, R, B, 3, HKV, D, P, 0.125, out, NULL, 0, 1);
    if (st != 3) bad |= fail("oracle_tree_attn (Hq % Hkv)", st, 3);

    free(out); free(vv); free(kk); free(q); free(nb); free(nd); free(ub); free(cdf); free(logits);
    if (!bad) printf("oracle sanitize driver ok\n");
    return bad;
}
