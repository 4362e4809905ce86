/*
 * fp64 CPU oracle for one exact Lloyd k-means iteration.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes is the plain definition of a Lloyd iteration, which the
 * Flash-KMeans article (lumevalley.com, article 3696) says its two kernels
 * reach exactly, with no approximation:
 *   - section "Why being fast took so long" (为什么"快"这件事被拖了这么久):
 *     an iteration assigns each of N points to one of K clusters using the
 *     N x K distances, then reduce-sums the points of each cluster and
 *     divides by the cluster size;
 *   - section "Two kernels rewrite the GPU pipeline" (两个 Kernel，重写了 GPU
 *     流水线): the maths of k-means is left as it is and nothing is
 *     approximated; only the data flow on the GPU changes.
 * The metric is squared Euclidean distance; cosine is handled by
 * L2-normalising every vector first, a zero norm being replaced by 1 before
 * the divide (LEANN FlashLib backend guide, mhpn.cn, paragraph
 * "距离度量" (distance metric)).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - ties in the minimum distance go to the lowest centroid index;
 *   - a cluster that receives no point keeps the centroid it was given;
 *   - distances are taken by direct difference, sum_j (x_j - c_j)^2, in
 *     fp64, accumulated in increasing j; inputs are fp32 and are promoted to
 *     fp64 exactly;
 *   - cluster sums are accumulated in fp64 in increasing point index.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -fPIC -shared.
 * Points are independent in the assignment, so the OpenMP split over points
 * does not change any result.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FKO_METRIC_L2 0
#define FKO_METRIC_COSINE 1
#define FKO_METRIC_INNER_PRODUCT 2
#define FKO_METRIC_SPHERICAL 3

/* Spherical k-means assigns as cosine does (rows normalised) and returns
 * centroids normalised to unit length. */
static int normalises(int metric)
{
    return metric == FKO_METRIC_COSINE || metric == FKO_METRIC_SPHERICAL;
}

static int known_metric(int metric)
{
    return metric == FKO_METRIC_L2 || metric == FKO_METRIC_COSINE || metric == FKO_METRIC_INNER_PRODUCT ||
           metric == FKO_METRIC_SPHERICAL;
}

/* Promote one fp32 row to fp64; for cosine divide it by its L2 norm, the
 * norm being taken as 1 when it is 0 (FlashLib guide, "距离度量"). */
static void promote_row(const float *src, int64_t d, int metric, double *dst)
{
    for (int64_t j = 0; j < d; ++j)
        dst[j] = (double)src[j];
    if (normalises(metric)) {
        double s = 0.0;
        for (int64_t j = 0; j < d; ++j)
            s = s + dst[j] * dst[j];
        double n = sqrt(s);
        if (n == 0.0)
            n = 1.0;
        for (int64_t j = 0; j < d; ++j)
            dst[j] = dst[j] / n;
    }
}

/* Squared Euclidean distance by direct difference, in increasing j. */
static double sqdist(const double *x, const double *c, int64_t d)
{
    double acc = 0.0;
    for (int64_t j = 0; j < d; ++j) {
        double t = x[j] - c[j];
        acc = acc + t * t;
    }
    return acc;
}

/* Negated inner product -x.c, the dot product summed in increasing j: the
 * largest inner product is the smallest of these, so the same lowest-index
 * argmin gives the inner-product assignment. */
static double negdot(const double *x, const double *c, int64_t d)
{
    double acc = 0.0;
    for (int64_t j = 0; j < d; ++j)
        acc = acc + x[j] * c[j];
    return -acc;
}

static double score(const double *x, const double *c, int64_t d, int metric)
{
    return metric == FKO_METRIC_INNER_PRODUCT ? negdot(x, c, d) : sqdist(x, c, d);
}

/* Rows of C promoted (and, for cosine, normalised) once.  Returns NULL on
 * allocation failure. */
static double *promote_matrix(const float *M, int64_t rows, int64_t d, int metric)
{
    double *out = (double *)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)(d > 0 ? d : 1) * sizeof(double));
    if (!out)
        return NULL;
    for (int64_t r = 0; r < rows; ++r)
        promote_row(M + r * d, d, metric, out + r * d);
    return out;
}

/*
 * Assignment step.  For every point i:
 *   D_ik = ||x_i - c_k||^2 for all k (inner product: D_ik = -x_i.c_k),
 *   a_i  = smallest k attaining min_k D_ik,
 *   D1_i = D_{i,a_i},
 *   D2_i = min over k != a_i of D_ik (+inf when K == 1).
 * Any of a, D1, D2 may be NULL.  Returns 0, or -1 on bad arguments or
 * allocation failure.
 */
int fko_assign(const float *X, int64_t N, int64_t d, const float *C, int64_t K,
               int metric, int32_t *a, double *D1, double *D2)
{
    if (N < 0 || d <= 0 || K <= 0 || (N > 0 && !X) || !C)
        return -1;
    if (!known_metric(metric))
        return -1;
    double *Cd = promote_matrix(C, K, d, metric);
    if (!Cd)
        return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *xi = (double *)malloc((size_t)d * sizeof(double));
        if (!xi) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t i = 0; i < N; ++i) {
            if (!xi)
                continue;
            promote_row(X + i * d, d, metric, xi);
            int64_t best_k = 0;
            double best = score(xi, Cd, d, metric);
            double second = INFINITY;
            for (int64_t k = 1; k < K; ++k) {
                double D = score(xi, Cd + k * d, d, metric);
                if (D < best) {
                    second = best;
                    best = D;
                    best_k = k;
                } else if (D < second) {
                    second = D;
                }
            }
            if (a)
                a[i] = (int32_t)best_k;
            if (D1)
                D1[i] = best;
            if (D2)
                D2[i] = second;
        }
        free(xi);
    }
    free(Cd);
    return failed ? -1 : 0;
}

/*
 * Update step.  n_k = #{i : a_i = k}; s_k = sum of x_i over those i, in
 * increasing i, in fp64 (rows normalised for cosine and spherical; taken as
 * they are for L2 and inner product); C_out[k] = s_k / n_k, or C_in[k] (as
 * passed, not normalised) when n_k == 0.  Spherical k-means (the explicit
 * spherical-centroid option beside cosine, named in the Flash-KMeans article's
 * section "Not a silver bullet" as where the metrics go next) then divides
 * each C_out[k] by its L2 norm (summed in increasing j; a zero norm taken as
 * 1, the guard of the FlashLib guide's "距离度量").  Returns 0, or -1 on bad
 * arguments (including a label outside [0, K)) or allocation failure.
 */
int fko_update(const float *X, int64_t N, int64_t d, const int32_t *a, int64_t K,
               int metric, const float *C_in, double *C_out, int64_t *counts)
{
    if (N < 0 || d <= 0 || K <= 0 || (N > 0 && (!X || !a)) || !C_in || !C_out || !counts)
        return -1;
    if (!known_metric(metric))
        return -1;
    for (int64_t i = 0; i < N; ++i)
        if (a[i] < 0 || (int64_t)a[i] >= K)
            return -1;
    double *xi = (double *)malloc((size_t)d * sizeof(double));
    if (!xi)
        return -1;
    memset(C_out, 0, (size_t)K * (size_t)d * sizeof(double));
    memset(counts, 0, (size_t)K * sizeof(int64_t));
    for (int64_t i = 0; i < N; ++i) {
        int64_t k = a[i];
        promote_row(X + i * d, d, metric, xi);
        counts[k] += 1;
        double *s = C_out + k * d;
        for (int64_t j = 0; j < d; ++j)
            s[j] = s[j] + xi[j];
    }
    for (int64_t k = 0; k < K; ++k) {
        double *s = C_out + k * d;
        if (counts[k] > 0) {
            double n = (double)counts[k];
            for (int64_t j = 0; j < d; ++j)
                s[j] = s[j] / n;
        } else {
            for (int64_t j = 0; j < d; ++j)
                s[j] = (double)C_in[k * d + j];
        }
        /* spherical: the mean direction, a zero vector staying zero (the
         * norm taken as 1), and an empty cluster's centroid normalised too */
        if (metric == FKO_METRIC_SPHERICAL) {
            double q = 0.0;
            for (int64_t j = 0; j < d; ++j)
                q = q + s[j] * s[j];
            double n = sqrt(q);
            if (n == 0.0)
                n = 1.0;
            for (int64_t j = 0; j < d; ++j)
                s[j] = s[j] / n;
        }
    }
    free(xi);
    return 0;
}

/*
 * One full iteration from C_in: assignment, then update, then the objective
 * J = sum_i D1_i under C_in (summed in increasing i).  a, D1, D2 are
 * optional outputs; C_out and counts are required.
 */
int fko_lloyd_iter(const float *X, int64_t N, int64_t d, const float *C_in, int64_t K,
                   int metric, int32_t *a, double *D1, double *D2, double *C_out,
                   int64_t *counts, double *J)
{
    if (N < 0)
        return -1;
    int32_t *a_use = a;
    double *d1_use = D1;
    int32_t *a_own = NULL;
    double *d1_own = NULL;
    if (!a_use) {
        a_own = (int32_t *)malloc((size_t)(N > 0 ? N : 1) * sizeof(int32_t));
        a_use = a_own;
    }
    if (!d1_use) {
        d1_own = (double *)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        d1_use = d1_own;
    }
    int rc = -1;
    if (a_use && d1_use) {
        rc = fko_assign(X, N, d, C_in, K, metric, a_use, d1_use, D2);
        if (rc == 0)
            rc = fko_update(X, N, d, a_use, K, metric, C_in, C_out, counts);
        if (rc == 0 && J) {
            double s = 0.0;
            for (int64_t i = 0; i < N; ++i)
                s = s + d1_use[i];
            *J = s;
        }
    }
    free(a_own);
    free(d1_own);
    return rc;
}

/* Number of OpenMP threads the assignment step will use. */
int fko_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/* The rows of X as the cosine metric sees them, rounded once to fp32: each
 * row promoted to fp64 and divided by its L2 norm, a zero norm taken as 1
 * (FlashLib guide, "距离度量"; the IVF lists of the same guide, paragraph
 * "工作原理", hold these normalised rows).  Returns 0, or -1 on bad sizes. */
int fko_normalize_rows(const float *X, int64_t N, int64_t d, float *out)
{
    if (N < 0 || d < 1 || (N > 0 && (X == NULL || out == NULL)))
        return -1;
    double *row = (double *)malloc((size_t)d * sizeof(double));
    if (row == NULL)
        return -1;
    for (int64_t i = 0; i < N; ++i) {
        promote_row(X + i * d, d, FKO_METRIC_COSINE, row);
        for (int64_t j = 0; j < d; ++j)
            out[i * d + j] = (float)row[j];
    }
    free(row);
    return 0;
}

/*
 * Exact k nearest neighbours by brute force (the exact GPU k-NN backend of
 * the LEANN FlashLib guide, paragraph "何时使用" (when to use)).  For every
 * query q: D_j = the distance of q to database row j by the metric above (for
 * cosine both rows normalised; inner product: -q.x_j) for every j, and
 * idx[q, 0..k) = the k rows that come first when all rows are ordered by
 * (D_j, j), with dist[q, r] = D of idx[q, r].  The scan over j in increasing
 * order keeps the k first rows seen so far in that order: a new row goes
 * after every kept row of distance <= its own, so ties keep the lower index
 * first.  Requires 1 <= k <= Ndb.  Returns 0, or -1 on bad arguments or
 * allocation failure.
 */
int fko_knn(const float *Q, int64_t M, int64_t d, const float *DB, int64_t Ndb, int64_t k,
            int metric, int32_t *idx, double *dist)
{
    if (M < 0 || d <= 0 || Ndb <= 0 || k < 1 || k > Ndb || (M > 0 && (!Q || !idx || !dist)) || !DB)
        return -1;
    if (metric != FKO_METRIC_L2 && metric != FKO_METRIC_COSINE && metric != FKO_METRIC_INNER_PRODUCT)
        return -1;
    double *Dd = promote_matrix(DB, Ndb, d, metric);
    if (!Dd)
        return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *qi = (double *)malloc((size_t)d * sizeof(double));
        double *bd = (double *)malloc((size_t)k * sizeof(double));
        int64_t *bi = (int64_t *)malloc((size_t)k * sizeof(int64_t));
        if (!qi || !bd || !bi) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t q = 0; q < M; ++q) {
            if (!qi || !bd || !bi)
                continue;
            promote_row(Q + q * d, d, metric, qi);
            int64_t kept = 0;
            for (int64_t j = 0; j < Ndb; ++j) {
                double D = score(qi, Dd + j * d, d, metric);
                if (kept == k && !(D < bd[k - 1]))
                    continue;
                /* position: after every kept entry with distance <= D */
                int64_t pos = kept < k ? kept : k - 1;
                while (pos > 0 && bd[pos - 1] > D) {
                    bd[pos] = bd[pos - 1];
                    bi[pos] = bi[pos - 1];
                    --pos;
                }
                bd[pos] = D;
                bi[pos] = j;
                if (kept < k)
                    ++kept;
            }
            for (int64_t r = 0; r < k; ++r) {
                idx[q * k + r] = (int32_t)bi[r];
                dist[q * k + r] = bd[r];
            }
        }
        free(qi);
        free(bd);
        free(bi);
    }
    free(Dd);
    return failed ? -1 : 0;
}
