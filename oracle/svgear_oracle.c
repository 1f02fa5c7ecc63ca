/*
 * svgear_oracle.c -- plain, slow, fp64 CPU definition of one SVG-EAR routed
 * attention call (cluster -> probe -> route -> hybrid attention), per head.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the HIP library and includes nothing from it.
 *
 * Sources (the SVG-EAR pages):
 *   [R]  "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video Generation
 *        via Error-aware Routing", Chinese review (paper.rainbus.top), the
 *        inference-pipeline paragraph, steps (1)-(5), and the weaknesses
 *        paragraph (greedy selection as an approximate 0-1 knapsack).
 *   [DE] gist.science (German), technical summary, section 2A (clustering and
 *        centroid compensation) and 2B (error-aware routing).
 *   [IT] gist.science (Italian), technical summary, section 2A/2B.
 *
 * Every routine works on one head.  All floating point is IEEE fp64 with no
 * reassociation: compile without -ffast-math.  Inputs are the exact input
 * values (bf16 or fp32) promoted to fp64.  Row-major layouts throughout:
 * X[i*d + t], centroids cent[m*d + t], block arrays [c*Ck + g].
 *
 * Readings of points the pages leave open:
 *   k-means: squared Euclidean distance, fixed iteration count, initial
 *   centroids are given token rows, argmin ties go to the lowest cluster
 *   index, an empty cluster keeps its previous centroid, the returned labels
 *   come from the last assignment and the centroids from the last update.
 *   V-bar of a key cluster is the mean of V over that key cluster's tokens.
 *   The probe uses the query-cluster centroid in both exponentials.  The
 *   block sum runs over all (i, j) pairs of the block.  The budget is
 *   floor(rho*Nq*Nk) pairs per head; greedy takes the longest prefix of the
 *   ratio order (descending, ties to the lower block index) whose cost fits.
 *   A skipped key cluster stands in for each of its m_g keys, so its
 *   compensation logit carries + ln(m_g), inside one joint softmax.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define SVGO_OK 0
#define SVGO_EARG (-1)
#define SVGO_ENOMEM (-2)

static double dot(const double* a, const double* b, int d)
{
    double s = 0.0;
    for (int t = 0; t < d; ++t) s += a[t] * b[t];
    return s;
}

/* Squared Euclidean distance, summed in coordinate order t = 0 .. d-1. */
static double sqdist(const double* x, const double* c, int d)
{
    double s = 0.0;
    for (int t = 0; t < d; ++t) {
        double u = x[t] - c[t];
        s += u * u;
    }
    return s;
}

/* k-means assignment ([R] step 1, [DE] 2A): label of every row of X is the
 * nearest centroid; a strictly smaller distance is needed to move past a lower
 * index, so ties resolve to the lowest cluster index. */
int svgo_assign(int N, int d, int C, const double* X, const double* cent, int32_t* labels)
{
    if (N < 0 || d <= 0 || C <= 0 || !X || !cent || !labels) return SVGO_EARG;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < N; ++i) {
        const double* x = X + (size_t)i * d;
        int best = 0;
        double bd = sqdist(x, cent, d);
        for (int m = 1; m < C; ++m) {
            double dm = sqdist(x, cent + (size_t)m * d, d);
            if (dm < bd) {
                bd = dm;
                best = m;
            }
        }
        labels[i] = best;
    }
    return SVGO_OK;
}

/* k-means update: each centroid becomes the mean of its rows (sum in row
 * order, then one division by the count); an empty cluster keeps its
 * previous centroid.  counts[m] receives the member count. */
int svgo_update(int N, int d, int C, const double* X, const int32_t* labels, double* cent,
                int32_t* counts)
{
    if (N < 0 || d <= 0 || C <= 0 || !X || !labels || !cent || !counts) return SVGO_EARG;
    double* sums = (double*)calloc((size_t)C * d, sizeof(double));
    if (!sums) return SVGO_ENOMEM;
    for (int m = 0; m < C; ++m) counts[m] = 0;
    for (int i = 0; i < N; ++i) {
        int m = labels[i];
        if (m < 0 || m >= C) {
            free(sums);
            return SVGO_EARG;
        }
        counts[m] += 1;
        for (int t = 0; t < d; ++t) sums[(size_t)m * d + t] += X[(size_t)i * d + t];
    }
    for (int m = 0; m < C; ++m) {
        if (counts[m] == 0) continue;
        for (int t = 0; t < d; ++t)
            cent[(size_t)m * d + t] = sums[(size_t)m * d + t] / (double)counts[m];
    }
    free(sums);
    return SVGO_OK;
}

/* Lloyd's k-means with given initial token indices and a fixed number of
 * iterations, each one assignment followed by one update ([R] step 1). */
int svgo_kmeans(int N, int d, int C, const double* X, const int32_t* init, int iters,
                int32_t* labels, double* cent, int32_t* counts)
{
    if (N <= 0 || d <= 0 || C <= 0 || C > N || iters < 1 || !X || !init || !labels || !cent ||
        !counts)
        return SVGO_EARG;
    for (int m = 0; m < C; ++m) {
        if (init[m] < 0 || init[m] >= N) return SVGO_EARG;
        memcpy(cent + (size_t)m * d, X + (size_t)init[m] * d, sizeof(double) * d);
    }
    for (int it = 0; it < iters; ++it) {
        int rc = svgo_assign(N, d, C, X, cent, labels);
        if (rc) return rc;
        rc = svgo_update(N, d, C, X, labels, cent, counts);
        if (rc) return rc;
    }
    return SVGO_OK;
}

/* Reorder so that same-cluster tokens are contiguous ([R] step 1): a stable
 * counting sort by label.  perm[r] is the token at sorted position r,
 * inv_perm[token] its position, offsets[m] .. offsets[m+1] cluster m's range. */
int svgo_permutation(int N, int C, const int32_t* labels, int32_t* counts, int32_t* offsets,
                     int32_t* perm, int32_t* inv_perm)
{
    if (N < 0 || C <= 0 || !labels || !counts || !offsets || !perm || !inv_perm) return SVGO_EARG;
    for (int m = 0; m < C; ++m) counts[m] = 0;
    for (int i = 0; i < N; ++i) {
        if (labels[i] < 0 || labels[i] >= C) return SVGO_EARG;
        counts[labels[i]] += 1;
    }
    offsets[0] = 0;
    for (int m = 0; m < C; ++m) offsets[m + 1] = offsets[m] + counts[m];
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    if (!cursor) return SVGO_ENOMEM;
    for (int m = 0; m < C; ++m) cursor[m] = offsets[m];
    for (int i = 0; i < N; ++i) {
        int r = cursor[labels[i]]++;
        perm[r] = i;
        inv_perm[i] = r;
    }
    free(cursor);
    return SVGO_OK;
}

/* Mean of the rows of Y over each label group (used for V-bar: V grouped by
 * the key clustering: [DE] 2A replaces the keys and values of a skipped block
 * by their cluster centroids).
 * An empty group gets the zero vector. */
int svgo_group_means(int N, int d, int C, const double* Y, const int32_t* labels, double* means)
{
    if (N < 0 || d <= 0 || C <= 0 || !Y || !labels || !means) return SVGO_EARG;
    int64_t* cnt = (int64_t*)calloc((size_t)C, sizeof(int64_t));
    if (!cnt) return SVGO_ENOMEM;
    memset(means, 0, sizeof(double) * (size_t)C * d);
    for (int i = 0; i < N; ++i) {
        int m = labels[i];
        if (m < 0 || m >= C) {
            free(cnt);
            return SVGO_EARG;
        }
        cnt[m] += 1;
        for (int t = 0; t < d; ++t) means[(size_t)m * d + t] += Y[(size_t)i * d + t];
    }
    for (int m = 0; m < C; ++m)
        if (cnt[m] > 0)
            for (int t = 0; t < d; ++t) means[(size_t)m * d + t] /= (double)cnt[m];
    free(cnt);
    return SVGO_OK;
}

/* Value-aware centroid probe ([R] step 2) and error-to-cost ratio ([R] step 3).
 *
 * For query cluster c (centroid qbar_c, n_c members) and key j in key cluster
 * g = labels_k[j]:
 *     e[c,j] = || exp(qbar_c . kbar_g / sqrt(d)) vbar_g - exp(qbar_c . k_j / sqrt(d)) v_j ||^2
 * evaluated directly (no expansion).  Every query of cluster c shares this
 * estimate ([R] step 2), so the block error is the sum over its n_c x m_g pairs,
 * E[c,g] = n_c * sum_{j in g} e[c,j], and the ratio ([R] step 3) is
 *     r[c,g] = E[c,g] / (n_c * m_g),   or 0 when n_c * m_g == 0.
 * eps2 (optional, [Cq*Nk], token order of the keys) receives e[c,j]. */
int svgo_probe(int Cq, int Nk, int Ck, int d, const double* qbar, const int32_t* counts_q,
               const double* K, const double* V, const int32_t* labels_k, const double* kbar,
               const double* vbar, const int32_t* counts_k, double* eps2, double* ratio)
{
    if (Cq <= 0 || Nk < 0 || Ck <= 0 || d <= 0 || !qbar || !counts_q || !K || !V || !labels_k ||
        !kbar || !vbar || !counts_k || !ratio)
        return SVGO_EARG;
    const double tau = 1.0 / sqrt((double)d);
    for (int j = 0; j < Nk; ++j)
        if (labels_k[j] < 0 || labels_k[j] >= Ck) return SVGO_EARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int c = 0; c < Cq; ++c) {
        const double* qc = qbar + (size_t)c * d;
        double* row = ratio + (size_t)c * Ck;
        for (int g = 0; g < Ck; ++g) row[g] = 0.0;
        for (int j = 0; j < Nk; ++j) {
            int g = labels_k[j];
            double a = exp(tau * dot(qc, kbar + (size_t)g * d, d));
            double b = exp(tau * dot(qc, K + (size_t)j * d, d));
            double e = 0.0;
            for (int t = 0; t < d; ++t) {
                double u = a * vbar[(size_t)g * d + t] - b * V[(size_t)j * d + t];
                e += u * u;
            }
            if (eps2) eps2[(size_t)c * Nk + j] = e;
            row[g] += e;
        }
        for (int g = 0; g < Ck; ++g) {
            double cost = (double)counts_q[c] * (double)counts_k[g];
            row[g] = cost > 0.0 ? ((double)counts_q[c] * row[g]) / cost : 0.0;
        }
    }
    return SVGO_OK;
}

/* The same probe in the log domain: ln r[c, g] (and ln e[c, j]).  The printed
 * estimate multiplies raw exponentials e^{tau qbar.kbar} and e^{tau qbar.k_j},
 * which overflow IEEE fp64 once tau qbar.k exceeds about 354 (heavy-tailed
 * keys reach that).  Factoring the larger exponential out of the norm is exact
 * algebra:
 *     e = e^{2M} sum_t (e^{alpha-M} vbar_t - e^{beta-M} v_t)^2,
 *     alpha = tau qbar.kbar_g, beta = tau qbar.k_j, M = max(alpha, beta),
 * so ln e = 2M + ln(sum ...), still evaluated directly (not expanded).  The
 * block value is ln r = ln(sum_{j in g} e_j) - ln m_g, the sum taken as a
 * log-sum-exp over the keys of g; -inf when n_c m_g = 0 or every e_j is 0.
 * With logit_only the estimate is the logit-difference variant that the
 * pages name but do not print ([R] step 2 calls the printed formula the
 * value-aware version; [DE] 2B speaks of a logit difference), read as
 * e = (exp(tau qbar.kbar_g) - exp(tau qbar.k_j))^2. */
int svgo_probe_log(int Cq, int Nk, int Ck, int d, const double* qbar, const int32_t* counts_q,
                   const double* K, const double* V, const int32_t* labels_k, const double* kbar,
                   const double* vbar, const int32_t* counts_k, double* log_eps2,
                   double* log_ratio, int logit_only)
{
    if (Cq <= 0 || Nk < 0 || Ck <= 0 || d <= 0 || !qbar || !counts_q || !K || !V || !labels_k ||
        !kbar || !vbar || !counts_k || !log_ratio)
        return SVGO_EARG;
    const double tau = 1.0 / sqrt((double)d);
    for (int j = 0; j < Nk; ++j)
        if (labels_k[j] < 0 || labels_k[j] >= Ck) return SVGO_EARG;
    int err = SVGO_OK;
#pragma omp parallel
    {
        double* le = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double* mx = (double*)malloc(sizeof(double) * (size_t)Ck);
        double* sm = (double*)malloc(sizeof(double) * (size_t)Ck);
        if (!le || !mx || !sm) {
#pragma omp atomic write
            err = SVGO_ENOMEM;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int c = 0; c < Cq; ++c) {
                const double* qc = qbar + (size_t)c * d;
                for (int j = 0; j < Nk; ++j) {
                    const int g = labels_k[j];
                    const double alpha = tau * dot(qc, kbar + (size_t)g * d, d);
                    const double beta = tau * dot(qc, K + (size_t)j * d, d);
                    const double M = alpha > beta ? alpha : beta;
                    const double a = exp(alpha - M), b = exp(beta - M);
                    double e = 0.0;
                    if (logit_only) {
                        /* the logit-difference estimate: the values drop out */
                        e = (a - b) * (a - b);
                    } else {
                        for (int t = 0; t < d; ++t) {
                            double u = a * vbar[(size_t)g * d + t] - b * V[(size_t)j * d + t];
                            e += u * u;
                        }
                    }
                    le[j] = e > 0.0 ? 2.0 * M + log(e) : -INFINITY;
                    if (log_eps2) log_eps2[(size_t)c * Nk + j] = le[j];
                }
                for (int g = 0; g < Ck; ++g) {
                    mx[g] = -INFINITY;
                    sm[g] = 0.0;
                }
                for (int j = 0; j < Nk; ++j)
                    if (le[j] > mx[labels_k[j]]) mx[labels_k[j]] = le[j];
                for (int j = 0; j < Nk; ++j) {
                    const int g = labels_k[j];
                    if (le[j] > -INFINITY) sm[g] += exp(le[j] - mx[g]);
                }
                double* row = log_ratio + (size_t)c * Ck;
                for (int g = 0; g < Ck; ++g) {
                    const int ok = counts_q[c] > 0 && counts_k[g] > 0 && sm[g] > 0.0;
                    row[g] = ok ? mx[g] + log(sm[g]) - log((double)counts_k[g]) : -INFINITY;
                }
            }
        }
        free(le);
        free(mx);
        free(sm);
    }
    return err;
}

/* Attention-score comparator: the selection rule the pages argue against
 * ([R] novelty paragraph: score-based selection is misaligned with the output
 * error once a compensation branch exists; [DE] 1 and 2B; [IT] 1).  The pages
 * give no formula for the score; read here as the centroid estimate of the
 * attention mass that query cluster c puts on key cluster g,
 *     P[c, g] = m_g e^{tau qbar_c.kbar_g} / sum_{g'} m_g' e^{tau qbar_c.kbar_g'}
 * (each key of g stands in as its centroid), with the value-to-cost rule of
 * the error-aware router: block value n_c P[c, g], cost n_c m_g, so
 *     ln r[c, g] = tau qbar_c.kbar_g - ln sum_{g'} m_g' e^{tau qbar_c.kbar_g'},
 * the sum over non-empty clusters, taken as a log-sum-exp; -inf where
 * n_c m_g = 0. */
int svgo_score_log(int Cq, int Ck, int d, const double* qbar, const int32_t* counts_q,
                   const double* kbar, const int32_t* counts_k, double* log_ratio)
{
    if (Cq <= 0 || Ck <= 0 || d <= 0 || !qbar || !counts_q || !kbar || !counts_k || !log_ratio)
        return SVGO_EARG;
    const double tau = 1.0 / sqrt((double)d);
    double* sb = (double*)malloc(sizeof(double) * (size_t)Ck);
    if (!sb) return SVGO_ENOMEM;
    for (int c = 0; c < Cq; ++c) {
        double mx = -INFINITY;
        for (int g = 0; g < Ck; ++g) {
            double s = 0.0;
            for (int t = 0; t < d; ++t) s += qbar[(size_t)c * d + t] * kbar[(size_t)g * d + t];
            sb[g] = tau * s;
            if (counts_k[g] > 0 && sb[g] + log((double)counts_k[g]) > mx) mx = sb[g] + log((double)counts_k[g]);
        }
        double sum = 0.0;
        for (int g = 0; g < Ck; ++g)
            if (counts_k[g] > 0) sum += exp(sb[g] + log((double)counts_k[g]) - mx);
        const double lse = mx + log(sum);
        for (int g = 0; g < Ck; ++g)
            log_ratio[(size_t)c * Ck + g] = (counts_q[c] > 0 && counts_k[g] > 0) ? sb[g] - lse : -INFINITY;
    }
    free(sb);
    return SVGO_OK;
}

/* Density budget in (query, key) pairs: floor(rho * Nq * Nk), evaluated as
 * (rho * Nq) * Nk in fp64 ([R] step 3, "density budget rho"). */
int64_t svgo_budget(double rho, int Nq, int Nk)
{
    return (int64_t)floor((rho * (double)Nq) * (double)Nk);
}

typedef struct {
    double r;
    int32_t idx;
} svgo_key;

static int by_ratio_desc_index_asc(const void* pa, const void* pb)
{
    const svgo_key* a = (const svgo_key*)pa;
    const svgo_key* b = (const svgo_key*)pb;
    if (a->r > b->r) return -1;
    if (a->r < b->r) return 1;
    return (a->idx > b->idx) - (a->idx < b->idx);
}

/* Greedy error-aware routing ([R] step 3; [R] weaknesses: greedy is an
 * approximate 0-1 knapsack).  Blocks are visited in descending ratio order
 * (equal ratios: lower block index c*Ck+g first); a block of cost
 * n_c * m_g is selected while the running cost stays within the budget, and
 * the walk stops at the first block that does not fit.  mask[c*Ck+g] = 1 for
 * exact blocks.  Returns the selected cost, or a negative error code. */
int64_t svgo_route(int Cq, int Ck, const double* ratio, const int32_t* counts_q,
                   const int32_t* counts_k, int64_t budget, uint8_t* mask)
{
    if (Cq <= 0 || Ck <= 0 || !ratio || !counts_q || !counts_k || !mask || budget < 0)
        return SVGO_EARG;
    size_t nb = (size_t)Cq * Ck;
    svgo_key* keys = (svgo_key*)malloc(sizeof(svgo_key) * nb);
    if (!keys) return SVGO_ENOMEM;
    for (size_t b = 0; b < nb; ++b) {
        keys[b].r = ratio[b];
        keys[b].idx = (int32_t)b;
    }
    qsort(keys, nb, sizeof(svgo_key), by_ratio_desc_index_asc);
    memset(mask, 0, nb);
    int64_t used = 0;
    for (size_t k = 0; k < nb; ++k) {
        int32_t b = keys[k].idx;
        int64_t w = (int64_t)counts_q[b / Ck] * (int64_t)counts_k[b % Ck];
        if (used + w > budget) break;
        used += w;
        mask[b] = 1;
    }
    free(keys);
    return used;
}

/* Exact 0-1 knapsack over the blocks, the optimum that the greedy rule
 * approximates ([R] weaknesses paragraph: greedy selection is an approximate
 * 0-1 knapsack; dynamic programming is named as the exact alternative).
 * Block b = c*Ck+g has integer weight w_b = counts_q[c] * counts_k[g] and value
 * val_b = w_b * e^{log_ratio_b - shift}, shift = the largest finite log_ratio
 * (a common factor, so the optimum is that of the unscaled values; blocks with
 * log_ratio = -inf have value 0).  Classic DP over capacities 0..budget:
 * best[w] = max(best[w], best[w - w_b] + val_b) item by item, with one bit per
 * (item, capacity) recording a take, then a backward walk from capacity
 * budget.  Of several optimal sets the walk returns one; the value is unique.
 * Returns the selected weight and writes mask and *value (in the shifted
 * scale), or a negative error code; SVGO_ENOMEM also when the bit table
 * (blocks x (budget + 1) bits) exceeds 2^33 bits. */
int64_t svgo_route_optimal(int Cq, int Ck, const double* log_ratio, const int32_t* counts_q,
                           const int32_t* counts_k, int64_t budget, uint8_t* mask, double* value)
{
    if (Cq <= 0 || Ck <= 0 || !log_ratio || !counts_q || !counts_k || !mask || budget < 0)
        return SVGO_EARG;
    const size_t nb = (size_t)Cq * Ck, cap = (size_t)budget + 1;
    if ((double)nb * (double)cap > 8589934592.0) return SVGO_ENOMEM;
    double shift = -INFINITY;
    for (size_t b = 0; b < nb; ++b)
        if (isfinite(log_ratio[b]) && log_ratio[b] > shift) shift = log_ratio[b];
    const size_t row_bytes = (cap + 7) / 8;
    uint8_t* take = (uint8_t*)calloc(nb, row_bytes);
    double* best = (double*)calloc(cap, sizeof(double));
    if (!take || !best) {
        free(take);
        free(best);
        return SVGO_ENOMEM;
    }
    for (size_t b = 0; b < nb; ++b) {
        const int64_t wb = (int64_t)counts_q[b / Ck] * (int64_t)counts_k[b % Ck];
        const double vb = isfinite(log_ratio[b]) ? (double)wb * exp(log_ratio[b] - shift) : 0.0;
        if (wb > budget) continue;
        uint8_t* tb = take + b * row_bytes;
        for (int64_t w = budget; w >= wb; --w) {
            const double cand = best[w - wb] + vb;
            if (cand > best[w]) {
                best[w] = cand;
                tb[w >> 3] |= (uint8_t)(1u << (w & 7));
            }
        }
    }
    memset(mask, 0, nb);
    int64_t w = budget, used = 0;
    for (size_t b = nb; b-- > 0;) {
        if (take[b * row_bytes + (w >> 3)] & (1u << (w & 7))) {
            const int64_t wb = (int64_t)counts_q[b / Ck] * (int64_t)counts_k[b % Ck];
            mask[b] = 1;
            used += wb;
            w -= wb;
        }
    }
    *value = best[budget];
    free(take);
    free(best);
    return used;
}

/* Hybrid attention output ([R] step 4; [DE] 2A).  For query i of cluster
 * c = labels_q[i], one softmax runs over
 *   exact terms        tau*q_i.k_j                for keys j with mask[c, labels_k[j]] = 1,
 *                      value v_j;
 *   compensation terms tau*q_i.kbar_g + ln(m_g)   for key clusters g with
 *                      mask[c,g] = 0 and m_g > 0, value vbar_g,
 * i.e. each skipped key is replaced by its cluster centroid and the m_g equal
 * terms are merged.  rows (optional) lists the query token indices to
 * evaluate; O[r*d + t] receives row r of the output (token order). */
int svgo_hybrid(int Nq, int Nk, int d, int Cq, int Ck, const double* Q, const double* K,
                const double* V, const int32_t* labels_q, const int32_t* labels_k,
                const double* kbar, const double* vbar, const int32_t* counts_k,
                const uint8_t* mask, int nrows, const int32_t* rows, double* O)
{
    if (Nq < 0 || Nk < 0 || d <= 0 || Cq <= 0 || Ck <= 0 || !Q || !K || !V || !labels_q ||
        !labels_k || !kbar || !vbar || !counts_k || !mask || !O || nrows < 0)
        return SVGO_EARG;
    const double tau = 1.0 / sqrt((double)d);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(| : bad)
    for (int r = 0; r < nrows; ++r) {
        int i = rows ? rows[r] : r;
        double* o = O + (size_t)r * d;
        if (i < 0 || i >= Nq || labels_q[i] < 0 || labels_q[i] >= Cq) {
            bad = 1;
            continue;
        }
        const double* q = Q + (size_t)i * d;
        const uint8_t* mrow = mask + (size_t)labels_q[i] * Ck;
        double* logit = (double*)malloc(sizeof(double) * ((size_t)Nk + Ck));
        if (!logit) {
            bad = 1;
            continue;
        }
        double mx = -INFINITY;
        for (int j = 0; j < Nk; ++j) {
            logit[j] = -INFINITY;
            if (mrow[labels_k[j]]) logit[j] = tau * dot(q, K + (size_t)j * d, d);
            if (logit[j] > mx) mx = logit[j];
        }
        for (int g = 0; g < Ck; ++g) {
            logit[Nk + g] = -INFINITY;
            if (!mrow[g] && counts_k[g] > 0)
                logit[Nk + g] = tau * dot(q, kbar + (size_t)g * d, d) + log((double)counts_k[g]);
            if (logit[Nk + g] > mx) mx = logit[Nk + g];
        }
        for (int t = 0; t < d; ++t) o[t] = 0.0;
        double den = 0.0;
        if (mx > -INFINITY) {
            for (int j = 0; j < Nk; ++j) {
                if (logit[j] == -INFINITY) continue;
                double w = exp(logit[j] - mx);
                den += w;
                for (int t = 0; t < d; ++t) o[t] += w * V[(size_t)j * d + t];
            }
            for (int g = 0; g < Ck; ++g) {
                if (logit[Nk + g] == -INFINITY) continue;
                double w = exp(logit[Nk + g] - mx);
                den += w;
                for (int t = 0; t < d; ++t) o[t] += w * vbar[(size_t)g * d + t];
            }
            for (int t = 0; t < d; ++t) o[t] /= den;
        }
        free(logit);
    }
    return bad ? SVGO_EARG : SVGO_OK;
}

/* Number of OpenMP threads the routines above will use. */
int svgo_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
