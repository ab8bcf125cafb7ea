/*
 * tev_oracle.c -- plain, slow, fp64 CPU oracle for draft-tree verification.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load this file
 * or the library built from it: only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark call it.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * Every function below evaluates the definitions of the method directly, in
 * double precision, with plain loops.  Inputs are widened exactly to double
 * (bf16 -> f32 -> f64 by bit placement, f32 -> f64 by conversion).
 *
 * Source ("Where Draft Trees Lose Target Mass: Exit-Guided Speculative
 * Decoding", arXiv 2610.11750):
 *   Sec. 3, Eq. 1-2   per-node target law p_v and reach P(v)
 *   Sec. 3.1, Eq. 4   child-token set A(v), local exit rho(v), exit mass w(v)
 *   Lemma 1, Eq. 5    sum_v w(v) = 1
 *   Sec. 3.2, Eq. 6   coverage C = sum_{u != r} P(u) = sum_v w(v) depth(v)
 *   Eq. 7             residual law p_v^res
 *   App. B, Alg. 1    TEV: one exit-node draw from w, one bonus draw from
 *                     p_V (leaf) or p_V^res (internal node)
 * Tree attention ("CAST: Cost-Aware Speculative Trees from One-Pass Block
 * Drafters", arXiv 2610.00321, App. B Lemma 1 and App. C "Packed
 * verification"): every packed node sees all cached prefix entries plus
 * its own root path, itself included.
 *
 * Readings where the pages leave a step open (each is listed in the
 * design notes of the repository):
 *   - node 0 is the root (parents[0] == -1) and parents[i] < i;
 *   - a categorical draw from a uniform u is the inverse CDF in index order
 *     with a strict "<" against u * total;
 *   - the softmax temperature multiplies the logits by inv_temperature;
 *   - tree attention uses the GQA map h -> h / (Hq / Hkv) and the caller's
 *     scale; the root's K/V row is cache row P, node i's is row P + i.
 *
 * Status codes returned: 0 ok, 1 invalid tree, 2 self-check failure,
 * 3 bad argument, 4 out of memory, 5 non-finite or all -inf row.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };

/* Exact widening of one input element to double. */
static double widen(const void *data, int dtype, size_t idx) {
    if (dtype == OR_F64) return ((const double *)data)[idx];
    if (dtype == OR_F32) return (double)((const float *)data)[idx];
    /* bf16: the 16 stored bits are the top half of an IEEE binary32 value */
    uint32_t bits = ((uint32_t)((const uint16_t *)data)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Number of threads an OpenMP region would use (1 without OpenMP). */
int oracle_max_threads(int nthreads) {
#ifdef _OPENMP
    set_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Tree validity: root first with no parent, every other parent earlier in
 * the order, tokens in range, sibling tokens distinct (2610.11750 Sec. 3
 * "Fixed-tree setup": sibling tokens are distinct).  Returns 0 if valid. */
int oracle_check_tree(const int32_t *parents, const int32_t *tokens, int B, int V) {
    if (B < 1) return 1;
    if (parents[0] != -1) return 1;
    for (int i = 1; i < B; i++) {
        if (parents[i] < 0 || parents[i] >= i) return 1;
        if (tokens[i] < 0 || tokens[i] >= V) return 1;
    }
    for (int i = 1; i < B; i++)
        for (int j = 1; j < i; j++)
            if (parents[j] == parents[i] && tokens[j] == tokens[i]) return 1;
    return 0;
}

/* depth(0) = 0, depth(i) = depth(parents[i]) + 1  (Sec. 3: depth = |pi(v)|). */
static void tree_depths(const int32_t *parents, int B, int *depth) {
    depth[0] = 0;
    for (int i = 1; i < B; i++) depth[i] = depth[parents[i]] + 1;
}

/* Row softmax pieces of Eq. 1: x_a = s * l_a, m = max_a x_a,
 * Z = sum_a exp(x_a - m), so that p(a) = exp(x_a - m) / Z.
 * Sums over the vocabulary are accumulated in long double (x87 extended
 * precision) so that the identities checked below hold to 1e-12 even for
 * V ~ 1.5e5 terms.
 * Returns 0, or 5 if the row holds NaN or +inf or is entirely -inf. */
static int row_softmax_parts(const void *logits, int dtype, size_t row_off, int V, double s,
                             double *m_out, double *Z_out) {
    double m = -INFINITY;
    for (int a = 0; a < V; a++) {
        double x = s * widen(logits, dtype, row_off + (size_t)a);
        if (isnan(x) || x == INFINITY) return 5;
        if (x > m) m = x;
    }
    if (m == -INFINITY) return 5;
    long double Z = 0.0L;
    for (int a = 0; a < V; a++) Z += (long double)exp(s * widen(logits, dtype, row_off + (size_t)a) - m);
    *m_out = m;
    *Z_out = (double)Z;
    return 0;
}

/*
 * Exit law of 2610.11750 Sec. 3 for R independent requests.
 *   logits   [R][B][V]  (dtype OR_F32 / OR_BF16 / OR_F64)
 *   parents, tokens [R][B]
 * Outputs (double, [R][B] unless noted):
 *   rho        local exit rho(v) = sum_{a not in A(v)} p_v(a)   (Eq. 4),
 *              summed directly over non-child tokens; exactly 1 at a leaf
 *   reach      P(0) = 1, P(i) = P(pa(i)) p_{pa(i)}(x_i)          (Eq. 2)
 *   exit_mass  w(v) = P(v) rho(v)                                (Eq. 4)
 *   coverage   [R]  C = sum_{i >= 1} P(i)                        (Eq. 6)
 *   logZ       [R][B] or NULL: m_v + log Z_v, the row log-normaliser
 * Self-checks (return 2 on failure): |rho - (1 - sum_children p)| <= 1e-12,
 * |sum_v w - 1| <= 1e-12 (Lemma 1), |C - sum_v w depth| <= 1e-12 max(1, C)
 * (Eq. 6).  A request whose tree is invalid returns 1; a non-finite row 5.
 */
int oracle_exit_law(const void *logits, int dtype, const int32_t *parents, const int32_t *tokens,
                    int R, int B, int V, double inv_temperature,
                    double *rho, double *reach, double *exit_mass, double *coverage,
                    double *logZ, int nthreads) {
    if (R < 1 || B < 1 || V < 1 || !(inv_temperature > 0.0)) return 3;
    set_threads(nthreads);
    int status = 0;
    for (int r = 0; r < R; r++)
        if (oracle_check_tree(parents + (size_t)r * B, tokens + (size_t)r * B, B, V)) return 1;

    double *m = (double *)malloc(sizeof(double) * (size_t)R * B);
    double *Z = (double *)malloc(sizeof(double) * (size_t)R * B);
    if (!m || !Z) { free(m); free(Z); return 4; }

    /* Per-node softmax normaliser and local exit, one row at a time. */
#pragma omp parallel for schedule(dynamic, 1)
    for (long long rv = 0; rv < (long long)R * B; rv++) {
        int r = (int)(rv / B), v = (int)(rv % B);
        const int32_t *par = parents + (size_t)r * B;
        const int32_t *tok = tokens + (size_t)r * B;
        size_t row = (size_t)rv * V;
        int st = row_softmax_parts(logits, dtype, row, V, inv_temperature, &m[rv], &Z[rv]);
        if (st) {
#pragma omp critical
            status = st;
            continue;
        }
        /* A(v): tokens of v's children. */
        unsigned char *in_A = (unsigned char *)calloc((size_t)V, 1);
        if (!in_A) {
#pragma omp critical
            status = 4;
            continue;
        }
        int n_children = 0;
        long double child_sum = 0.0L;
        for (int u = 1; u < B; u++)
            if (par[u] == v) {
                in_A[tok[u]] = 1;
                n_children++;
                child_sum += exp(inv_temperature * widen(logits, dtype, row + (size_t)tok[u]) - m[rv]) / Z[rv];
            }
        double res = 0.0;
        if (n_children == 0) {
            res = 1.0; /* a leaf exits with certainty (Sec. 3.1) */
        } else {
            long double acc = 0.0L;
            for (int a = 0; a < V; a++)
                if (!in_A[a]) acc += (long double)exp(inv_temperature * widen(logits, dtype, row + (size_t)a) - m[rv]);
            res = (double)(acc / (long double)Z[rv]);
            if (fabs(res - (double)(1.0L - child_sum)) > 1e-12) {
#pragma omp critical
                status = 2;
            }
        }
        rho[rv] = res;
        if (logZ) logZ[rv] = m[rv] + log(Z[rv]);
        free(in_A);
    }
    if (status) { free(m); free(Z); return status; }

    /* Reach, exit mass and coverage, request by request, nodes in index
     * order (parents precede children, so P(pa(i)) is already known). */
    for (int r = 0; r < R; r++) {
        const int32_t *par = parents + (size_t)r * B;
        const int32_t *tok = tokens + (size_t)r * B;
        double *P = reach + (size_t)r * B;
        P[0] = 1.0;
        for (int i = 1; i < B; i++) {
            size_t prow = (size_t)r * B + par[i];
            double p_child = exp(inv_temperature * widen(logits, dtype, prow * V + (size_t)tok[i]) - m[prow]) / Z[prow];
            P[i] = P[par[i]] * p_child;
        }
        long double C = 0.0L, wsum = 0.0L, wdepth = 0.0L;
        int *depth = (int *)malloc(sizeof(int) * (size_t)B);
        if (!depth) { status = 4; break; }
        tree_depths(par, B, depth);
        for (int v = 0; v < B; v++) {
            double w = P[v] * rho[(size_t)r * B + v];
            exit_mass[(size_t)r * B + v] = w;
            wsum += w;
            wdepth += w * depth[v];
            if (v >= 1) C += P[v];
        }
        free(depth);
        coverage[r] = (double)C;
        if (fabsl(wsum - 1.0L) > 1e-12L) status = 2;
        if (fabsl(C - wdepth) > 1e-12L * (C > 1.0L ? C : 1.0L)) status = 2;
    }
    free(m);
    free(Z);
    return status;
}

/*
 * Normalised residual CDF of one node's row, token-id order (Eq. 7 and
 * Alg. 1's bonus draw): r_a = p_v(a) 1[a not in A(v)], a leaf keeps p_v.
 * cdf[a] = (sum_{a' <= a} r_a') / T with T = sum_a r_a.  Returns 0, or 5
 * if the row is non-finite or the residual total is zero.
 */
int oracle_residual_cdf(const void *logits, int dtype, const int32_t *parents, const int32_t *tokens,
                        int B, int V, int node, double inv_temperature, double *cdf) {
    double m, Z;
    int st = row_softmax_parts(logits, dtype, (size_t)node * V, V, inv_temperature, &m, &Z);
    if (st) return st;
    unsigned char *in_A = (unsigned char *)calloc((size_t)V, 1);
    if (!in_A) return 4;
    for (int u = 1; u < B; u++)
        if (parents[u] == node) in_A[tokens[u]] = 1;
    long double run = 0.0L;
    for (int a = 0; a < V; a++) {
        double ra = in_A[a] ? 0.0 : exp(inv_temperature * widen(logits, dtype, (size_t)node * V + a) - m) / Z;
        run += (long double)ra;
        cdf[a] = (double)run;
    }
    free(in_A);
    if (!(run > 0.0L)) return 5;
    for (int a = 0; a < V; a++) cdf[a] = (double)((long double)cdf[a] / run);
    return 0;
}

/* Inverse CDF with strict "<": the smallest j with u * total < cum[j].
 * If rounding leaves none, the last j whose own mass is positive.
 * band = 1 when u lies within 1e-6 of either boundary of bin j on the
 * normalised CDF (lower boundary of bin 0 is 0). */
static int inverse_cdf(const double *cum, int n, double u, unsigned char *band) {
    double total = cum[n - 1];
    double t = u * total;
    int lo = 0, hi = n; /* smallest j in [lo, hi) with t < cum[j]; hi == n: none */
    while (lo < hi) {
        int mid = lo + (hi - lo) / 2;
        if (t < cum[mid]) hi = mid; else lo = mid + 1;
    }
    int j = lo;
    if (j >= n) {
        j = n - 1;
        while (j > 0 && !(cum[j] > cum[j - 1])) j--;
    }
    double lower = (j == 0) ? 0.0 : cum[j - 1] / total;
    double upper = cum[j] / total;
    *band = (fabs(u - lower) < 1e-6 || fabs(u - upper) < 1e-6) ? 1 : 0;
    return j;
}

/*
 * TEV's two draws (2610.11750 App. B, Alg. 1, lines "Draw V" and "Draw Y"),
 * for n_draws uniform pairs per request.
 *   exit_mass [R][B]        the oracle's own w(v)
 *   uniforms  [R][n][2]     (u1 for the exit node, u2 for the bonus token)
 * Outputs [R][n]: exit_node, bonus_token; band [R][n][2] flags (exit, bonus).
 * Exit node: inverse CDF of the running sums of w in node-index order.
 * Bonus token: inverse CDF of node V's residual row in token-id order
 * (children of V removed; a leaf keeps its full row).
 */
int oracle_sample(const void *logits, int dtype, const int32_t *parents, const int32_t *tokens,
                  int R, int B, int V, double inv_temperature, const double *exit_mass,
                  const float *uniforms, int n_draws, int32_t *exit_node, int32_t *bonus_token,
                  unsigned char *band, int nthreads) {
    if (R < 1 || B < 1 || V < 1 || n_draws < 1 || !(inv_temperature > 0.0)) return 3;
    set_threads(nthreads);
    for (int r = 0; r < R; r++)
        if (oracle_check_tree(parents + (size_t)r * B, tokens + (size_t)r * B, B, V)) return 1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < R; r++) {
        const int32_t *par = parents + (size_t)r * B;
        const int32_t *tok = tokens + (size_t)r * B;
        const void *rows = (dtype == OR_F64) ? (const void *)((const double *)logits + (size_t)r * B * V)
                         : (dtype == OR_F32) ? (const void *)((const float *)logits + (size_t)r * B * V)
                                             : (const void *)((const uint16_t *)logits + (size_t)r * B * V);
        double *W = (double *)malloc(sizeof(double) * (size_t)B);
        double **res_cum = (double **)calloc((size_t)B, sizeof(double *)); /* built on first use */
        if (!W || !res_cum) {
            free(W);
            free(res_cum);
#pragma omp critical
            status = 4;
            continue;
        }
        double run = 0.0;
        for (int j = 0; j < B; j++) { run += exit_mass[(size_t)r * B + j]; W[j] = run; }
        for (int n = 0; n < n_draws; n++) {
            size_t k = (size_t)r * n_draws + n;
            double u1 = (double)uniforms[2 * k], u2 = (double)uniforms[2 * k + 1];
            int Vn = inverse_cdf(W, B, u1, &band[2 * k]);
            if (!res_cum[Vn]) {
                res_cum[Vn] = (double *)malloc(sizeof(double) * (size_t)V);
                if (!res_cum[Vn]) {
#pragma omp critical
                    status = 4;
                    break;
                }
                int st = oracle_residual_cdf(rows, dtype, par, tok, B, V, Vn, inv_temperature, res_cum[Vn]);
                if (st) {
#pragma omp critical
                    status = st;
                    break;
                }
            }
            exit_node[k] = Vn;
            bonus_token[k] = inverse_cdf(res_cum[Vn], V, u2, &band[2 * k + 1]);
        }
        for (int j = 0; j < B; j++) free(res_cum[j]);
        free(res_cum);
        free(W);
    }
    return status;
}

/*
 * Predraw-and-follow verification (2610.11750 App. A.4.1), the baseline the
 * pages measure TEV against.  Before any test, every node v draws its own
 * token R_v from its full target row p_v (Eq. 1), children included.  The
 * walk starts at the root; at node v it moves to the child whose incoming
 * token equals R_v (sibling tokens are distinct, so at most one does) and
 * otherwise stops there: the exit node is v and the bonus token is R_v.
 *   uniforms  [R][n][B]  u for node v's draw of draw n
 * Outputs: node_draw [R][n][B] (R_v, the inverse CDF of p_v in token order at
 * u), exit_node and bonus_token [R][n]; band [R][n] = 1 when the draw of any
 * node on the walked path lies within 1e-6 of a boundary of its bin (the
 * draws of nodes off the path cannot change the outcome); node_band
 * [R][n][B] (or NULL) = 1 when node v's own draw lies within 1e-6 of a
 * boundary of its bin.
 * Rows are processed one request at a time: B cumulative rows of V doubles.
 */
int oracle_predraw(const void *logits, int dtype, const int32_t *parents, const int32_t *tokens,
                   int R, int B, int V, double inv_temperature, const float *uniforms,
                   int n_draws, int32_t *node_draw, int32_t *exit_node, int32_t *bonus_token,
                   unsigned char *band, unsigned char *node_band, int nthreads) {
    if (R < 1 || B < 1 || V < 1 || n_draws < 1 || !(inv_temperature > 0.0)) return 3;
    set_threads(nthreads);
    for (int r = 0; r < R; r++)
        if (oracle_check_tree(parents + (size_t)r * B, tokens + (size_t)r * B, B, V)) return 1;
    double *cum = (double *)malloc(sizeof(double) * (size_t)B * (size_t)V);
    unsigned char *nb = (unsigned char *)malloc((size_t)n_draws * (size_t)B);
    if (!cum || !nb) { free(cum); free(nb); return 4; }
    int status = 0;
    for (int r = 0; r < R && status == 0; r++) {
        const int32_t *par = parents + (size_t)r * B;
        const int32_t *tok = tokens + (size_t)r * B;
        size_t row0 = (size_t)r * B * V;
        /* running sums of exp(s x_a - m_v) in token order, one row per node */
#pragma omp parallel for schedule(dynamic, 1)
        for (int v = 0; v < B; v++) {
            double m, Z;
            int st = row_softmax_parts(logits, dtype, row0 + (size_t)v * V, V, inv_temperature, &m, &Z);
            if (st) {
#pragma omp critical
                status = st;
                continue;
            }
            double run = 0.0;
            for (int a = 0; a < V; a++) {
                run += exp(inv_temperature * widen(logits, dtype, row0 + (size_t)v * V + a) - m);
                cum[(size_t)v * V + a] = run;
            }
        }
        if (status) break;
#pragma omp parallel for schedule(dynamic, 16)
        for (int n = 0; n < n_draws; n++) {
            size_t k = (size_t)r * n_draws + n;
            for (int v = 0; v < B; v++) {
                node_draw[k * B + v] = inverse_cdf(cum + (size_t)v * V, V,
                                                   (double)uniforms[k * B + v], &nb[(size_t)n * B + v]);
                if (node_band) node_band[k * B + v] = nb[(size_t)n * B + v];
            }
            int v = 0;
            unsigned char on_band = 0;
            for (;;) {
                int d = node_draw[k * B + v];
                on_band |= nb[(size_t)n * B + v];
                int next = -1;
                for (int u = v + 1; u < B; u++)
                    if (par[u] == v && tok[u] == d) { next = u; break; }
                if (next < 0) break;
                v = next;
            }
            exit_node[k] = v;
            bonus_token[k] = node_draw[k * B + v];
            band[k] = on_band;
        }
    }
    free(cum);
    free(nb);
    return status;
}

/*
 * One layer of ancestor-masked tree attention (2610.00321 App. B Lemma 1;
 * App. C "Packed verification"; App. F varlen verifier).
 *   q   [R][B][Hq][D];  k, v [R][Hkv][P + B][D]  (cache row P + i is node i)
 * Query (r, i, h) attends to key set J(i) = {0..P-1} U {P + j : j on the
 * root path of i, i included} of kv head g = h / (Hq / Hkv):
 *   s_j = scale * <q[r,i,h,:], k[r,g,j,:]>,
 *   out[r,i,h,:] = sum_j softmax(s)_j v[r,g,j,:].
 * rows: NULL to compute every (r, i, h), else n_rows flat query indices
 * ((r * B + i) * Hq + h); out then holds n_rows * D values in that order.
 */
int oracle_tree_attn(const void *q, const void *k, const void *v, int dtype, const int32_t *parents,
                     int R, int B, int Hq, int Hkv, int D, int P, double scale, double *out,
                     const int64_t *rows, int64_t n_rows, int nthreads) {
    if (R < 1 || B < 1 || Hq < 1 || Hkv < 1 || D < 1 || P < 0 || Hq % Hkv) return 3;
    set_threads(nthreads);
    for (int r = 0; r < R; r++) {
        const int32_t *par = parents + (size_t)r * B;
        if (par[0] != -1) return 1;
        for (int i = 1; i < B; i++)
            if (par[i] < 0 || par[i] >= i) return 1;
    }
    int G = Hq / Hkv;
    int status = 0;
    int64_t total = rows ? n_rows : (int64_t)R * B * Hq;
    size_t kv_rows = (size_t)P + B;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t n = 0; n < total; n++) {
        int64_t flat = rows ? rows[n] : n;
        int h = (int)(flat % Hq);
        int i = (int)((flat / Hq) % B);
        int r = (int)(flat / ((int64_t)Hq * B));
        int g = h / G;
        const int32_t *par = parents + (size_t)r * B;
        /* key set J(i): prefix rows, then the root path of i */
        int n_keys = P;
        int *keys = (int *)malloc(sizeof(int) * ((size_t)P + B));
        double *s = (double *)malloc(sizeof(double) * ((size_t)P + B));
        if (!keys || !s) {
            free(keys);
            free(s);
#pragma omp critical
            status = 4;
            continue;
        }
        for (int j = 0; j < P; j++) keys[j] = j;
        for (int a = i; a >= 0; a = par[a]) keys[n_keys++] = P + a;
        size_t qoff = (((size_t)r * B + i) * Hq + h) * D;
        size_t kvbase = ((size_t)r * Hkv + g) * kv_rows * D;
        double smax = -INFINITY;
        for (int t = 0; t < n_keys; t++) {
            double dot = 0.0;
            for (int d = 0; d < D; d++)
                dot += widen(q, dtype, qoff + d) * widen(k, dtype, kvbase + (size_t)keys[t] * D + d);
            s[t] = scale * dot;
            if (s[t] > smax) smax = s[t];
        }
        double Z = 0.0;
        for (int t = 0; t < n_keys; t++) { s[t] = exp(s[t] - smax); Z += s[t]; }
        double *o = out + (size_t)n * D;
        for (int d = 0; d < D; d++) o[d] = 0.0;
        for (int t = 0; t < n_keys; t++) {
            double pt = s[t] / Z;
            for (int d = 0; d < D; d++) o[d] += pt * widen(v, dtype, kvbase + (size_t)keys[t] * D + d);
        }
        free(s);
        free(keys);
    }
    return status;
}
