/*
 * oracle.c -- CPU reference for the exact epsilon-distance self-join.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that tests, the package's smoke check and the
 * benchmark's CPU-baseline leg can compare the GPU library against a plain,
 * slow, obviously correct computation.  It shares no code, header, table or
 * constant with the GPU library.
 *
 * What it computes ("RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
 * Similarity Searches", Sec. II-A "Problem Statement"): two points are
 * neighbours iff their Euclidean distance is at most epsilon; the self-join
 * pairs every point of the dataset with every point of the same dataset, and
 * the result is the set of (query id, point id) key-value pairs (Sec. II-A1).
 * Self pairs are part of the result: the selectivity z = (|R| - |D|) / |D| of
 * Sec. V-B counts neighbours per query excluding the point itself, which only
 * makes sense when |R| includes the |D| self pairs.
 *
 * Readings fixed here (the pages leave them open):
 *   - the test compares squared distances: D64(a,b) <= E64 with E64 = fl(eps*eps);
 *   - D64 is the canonical binary64 value: s = 0; for k = 0..d-1 in the
 *     input's own dimension order: t = (double)a[k] - (double)b[k]; s = s + t*t;
 *     every operation a single round-to-nearest-even binary64 operation, no
 *     fused multiply-add (this file is built with -ffp-contract=off) and no
 *     reassociation;
 *   - both (i,j) and (j,i) are reported, and (i,i) for every i.
 *
 * Every routine scans all candidate points in index order, so neighbour
 * lists come out sorted by point id.  orc_semijoin_rows does the same for
 * a query set distinct from the dataset (the semi-join of Sec. II-A).
 * orc_knn gives the exact k nearest neighbours (Sec. VI), ranked by the same
 * canonical D64, ties by the smaller point id.  orc_digest_rows and
 * orc_digest_all summarise neighbour lists too long to keep (a count and a
 * fingerprint per row, plus the pairs near the threshold) for the full-size
 * comparisons.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORC_VERSION 4

int orc_version(void) { return ORC_VERSION; }

int orc_threads(void) { return omp_get_max_threads(); }

/* Canonical squared distance (see header). */
double orc_d64(const float *a, const float *b, int64_t d)
{
    double s = 0.0;
    for (int64_t k = 0; k < d; ++k) {
        double t = (double)a[k] - (double)b[k];
        double tt = t * t;
        s = s + tt;
    }
    return s;
}

double orc_e64(double eps) { return eps * eps; }

static int check_inputs(const float *X, int64_t n, int64_t d, int64_t ld, double eps)
{
    if (!X || n < 1 || d < 1 || ld < d) return -1;
    if (isnan(eps) || eps < 0.0) return -1;
    int bad = 0;
#pragma omp parallel for reduction(| : bad) schedule(static)
    for (int64_t i = 0; i < n; ++i)
        for (int64_t k = 0; k < d; ++k)
            if (!isfinite(X[i * ld + k])) bad |= 1;
    return bad ? -2 : 0;
}

/*
 * Neighbour lists of selected rows (all rows when rows == NULL).
 * Phase 1 (cols == NULL): counts[r] = |{ j : D64(x_row(r), x_j) <= E64 }|.
 * Phase 2 (cols != NULL): colptr[r] .. colptr[r+1] receives those j ascending.
 * Returns 0, -1 on bad arguments, -2 if X holds a non-finite value.
 */
int orc_join_rows(const float *X, int64_t n, int64_t d, int64_t ld, double eps,
                  const int64_t *rows, int64_t nrows, uint64_t *counts,
                  uint32_t *cols, const uint64_t *colptr)
{
    int rc = check_inputs(X, n, d, ld, eps);
    if (rc) return rc;
    if (!rows) nrows = n;
    if (nrows < 0 || (!cols && !counts) || (cols && !colptr)) return -1;
    const double e64 = orc_e64(eps);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        const float *xi = X + i * ld;
        uint64_t c = 0, at = cols ? colptr[r] : 0;
        for (int64_t j = 0; j < n; ++j) {
            if (orc_d64(xi, X + j * ld, d) <= e64) {
                if (cols) cols[at + c] = (uint32_t)j;
                ++c;
            }
        }
        if (counts) counts[r] = c;
    }
    return 0;
}

/*
 * Semi-join (Sec. II-A: the query set Q distinct from the dataset D; the pair
 * (q_j, p_i) is in the result iff dist(p_i, q_j) <= eps): neighbour lists of
 * selected query rows of Q (all when rows == NULL) over all n points of X.
 * Same two phases, return codes and canonical D64 (query first, point
 * second) as orc_join_rows; with Q == X it is the self-join.
 */
int orc_semijoin_rows(const float *Q, int64_t nq, int64_t ldq, const float *X, int64_t n,
                      int64_t ld, int64_t d, double eps, const int64_t *rows, int64_t nrows,
                      uint64_t *counts, uint32_t *cols, const uint64_t *colptr)
{
    int rc = check_inputs(X, n, d, ld, eps);
    if (rc) return rc;
    rc = check_inputs(Q, nq, d, ldq, eps);
    if (rc) return rc;
    if (!rows) nrows = nq;
    if (nrows < 0 || (!cols && !counts) || (cols && !colptr)) return -1;
    const double e64 = orc_e64(eps);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= nq) continue;
        const float *qi = Q + i * ldq;
        uint64_t c = 0, at = cols ? colptr[r] : 0;
        for (int64_t j = 0; j < n; ++j) {
            if (orc_d64(qi, X + j * ld, d) <= e64) {
                if (cols) cols[at + c] = (uint32_t)j;
                ++c;
            }
        }
        if (counts) counts[r] = c;
    }
    return 0;
}

/*
 * Number of ordered pairs (row(r), j) whose D64 lies within rel*E64 of E64:
 * the pairs that a classifier working at lower precision cannot decide
 * without an exact re-check.
 */
int64_t orc_band_count(const float *X, int64_t n, int64_t d, int64_t ld, double eps,
                       double rel, const int64_t *rows, int64_t nrows)
{
    if (check_inputs(X, n, d, ld, eps)) return -1;
    if (!rows) nrows = n;
    const double e64 = orc_e64(eps), w = rel * e64;
    int64_t total = 0;
#pragma omp parallel for schedule(dynamic, 4) reduction(+ : total)
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t i = rows ? rows[r] : r;
        for (int64_t j = 0; j < n; ++j)
            if (fabs(orc_d64(X + i * ld, X + j * ld, d) - e64) <= w) ++total;
    }
    return total;
}

/* ---- neighbour-list fingerprints -------------------------------------------
 * For joins too large to hold as pair lists, each row's neighbour set N(i) is
 * summarised by its size and a fingerprint h_i = sum over j in N(i) of
 * mix64(j), modulo 2^64.  mix64 is the output function of the splitmix64
 * generator (state advanced by the golden-ratio constant 0x9e3779b97f4a7c15,
 * then two xor-shift-multiply rounds), a bijection on 64-bit words, so a
 * missing, extra or wrong neighbour changes h_i except with probability
 * about 2^-64.  The fingerprint belongs to the checking, not to the join.
 */
uint64_t orc_mix64(uint64_t j)
{
    uint64_t z = j + 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

/*
 * Per selected row r (all rows when rows == NULL), i = rows[r]:
 *   counts[r]  = |N(i)|, N(i) = { j : D64(x_i, x_j) <= E64 };
 *   digests[r] = sum of mix64(j) over N(i), mod 2^64;
 *   band[r]    = |{ j : |D64(x_i, x_j) - E64| <= rel * E64 }|  (band may be NULL).
 * One pass over all n points per row.  Returns 0, -1, -2 as orc_join_rows.
 */
int orc_digest_rows(const float *X, int64_t n, int64_t d, int64_t ld, double eps, double rel,
                    const int64_t *rows, int64_t nrows, uint32_t *counts, uint64_t *digests,
                    uint32_t *band)
{
    int rc = check_inputs(X, n, d, ld, eps);
    if (rc) return rc;
    if (!rows) nrows = n;
    if (nrows < 0 || !counts || !digests || !(rel >= 0.0)) return -1;
    const double e64 = orc_e64(eps), w = rel * e64;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        uint32_t c = 0, nb = 0;
        uint64_t h = 0;
        if (i >= 0 && i < n) {
            for (int64_t j = 0; j < n; ++j) {
                const double s = orc_d64(X + i * ld, X + j * ld, d);
                if (s <= e64) {
                    ++c;
                    h += orc_mix64((uint64_t)j);
                }
                if (fabs(s - e64) <= w) ++nb;
            }
        }
        counts[r] = c;
        digests[r] = h;
        if (band) band[r] = nb;
    }
    return 0;
}

/*
 * The same three arrays for every row of the self-join (length n), with each
 * unordered pair evaluated once: D64(x_i, x_j) and D64(x_j, x_i) are the
 * same binary64 value (each difference is the negation of the other, exactly,
 * so the squares and their running sums agree), so the pair (i, j), j > i,
 * counts for row i and, mirrored, for row j.  Each thread accumulates into
 * arrays of its own, summed at the end.  Returns 0, -1, -2 (bad input),
 * -3 (out of host memory).
 */
int orc_digest_all(const float *X, int64_t n, int64_t d, int64_t ld, double eps, double rel,
                   uint32_t *counts, uint64_t *digests, uint32_t *band)
{
    int rc = check_inputs(X, n, d, ld, eps);
    if (rc) return rc;
    if (!counts || !digests || !band || !(rel >= 0.0)) return -1;
    const double e64 = orc_e64(eps), w = rel * e64;
    memset(counts, 0, sizeof(uint32_t) * (size_t)n);
    memset(digests, 0, sizeof(uint64_t) * (size_t)n);
    memset(band, 0, sizeof(uint32_t) * (size_t)n);
    int oom = 0;
#pragma omp parallel reduction(| : oom)
    {
        uint32_t *lc = (uint32_t *)calloc((size_t)n, sizeof(uint32_t));
        uint32_t *lb = (uint32_t *)calloc((size_t)n, sizeof(uint32_t));
        uint64_t *lh = (uint64_t *)calloc((size_t)n, sizeof(uint64_t));
        const int ok = lc && lb && lh;
        if (!ok) oom = 1;
#pragma omp for schedule(dynamic, 16)
        for (int64_t i = 0; i < n; ++i) {
            if (!ok) continue;
            const uint64_t mi = orc_mix64((uint64_t)i);
            for (int64_t j = i; j < n; ++j) {
                const double s = orc_d64(X + i * ld, X + j * ld, d);
                const int in = s <= e64, bd = fabs(s - e64) <= w;
                if (!in && !bd) continue;
                lc[i] += (uint32_t)in;
                lb[i] += (uint32_t)bd;
                if (in) lh[i] += orc_mix64((uint64_t)j);
                if (j != i) {
                    lc[j] += (uint32_t)in;
                    lb[j] += (uint32_t)bd;
                    if (in) lh[j] += mi;
                }
            }
        }
#pragma omp critical
        if (ok) {
            for (int64_t i = 0; i < n; ++i) {
                counts[i] += lc[i];
                band[i] += lb[i];
                digests[i] += lh[i];
            }
        }
        free(lc);
        free(lb);
        free(lh);
    }
    return oom ? -3 : 0;
}

/* ---- epsilon calibration ------------------------------------------------
 * The workloads fix epsilon as the value giving a mean of k neighbours per
 * query (self excluded, as in the selectivity of Sec. V-B) over the first nq
 * rows.  With K = nq*k, the routine returns a = the K-th and b = the
 * (K+1)-th smallest D64 over all pairs (q, j), q < nq, j != q.  Any E64 with
 * a <= E64 < b then gives exactly K non-self neighbours over those rows.
 * Each query keeps its m smallest values in a max-heap; the answer is
 * certified only if every query whose heap was full has an m-th value above
 * b (otherwise an unseen value could belong to the K+1 smallest): the
 * return value is then 0, else 1 (call again with a larger m).
 */
static void heap_push(double *h, int64_t *size, int64_t cap, double v)
{
    if (*size < cap) {
        int64_t i = (*size)++;
        h[i] = v;
        while (i > 0) {
            int64_t p = (i - 1) / 2;
            if (h[p] >= h[i]) break;
            double t = h[p]; h[p] = h[i]; h[i] = t;
            i = p;
        }
    } else if (v < h[0]) {
        h[0] = v;
        int64_t i = 0;
        for (;;) {
            int64_t l = 2 * i + 1, r = l + 1, m = i;
            if (l < cap && h[l] > h[m]) m = l;
            if (r < cap && h[r] > h[m]) m = r;
            if (m == i) break;
            double t = h[m]; h[m] = h[i]; h[i] = t;
            i = m;
        }
    }
}

static int cmp_double(const void *a, const void *b)
{
    double x = *(const double *)a, y = *(const double *)b;
    return (x > y) - (x < y);
}

int orc_calibrate(const float *X, int64_t n, int64_t d, int64_t ld, int64_t nq, int64_t k,
                  int64_t m, double *out_a, double *out_b)
{
    if (check_inputs(X, n, d, ld, 0.0)) return -1;
    if (nq < 1 || nq > n || k < 1 || m < 1 || !out_a || !out_b) return -1;
    if (m > n - 1) m = n - 1;
    int64_t K = nq * k;
    if (K + 1 > nq * (n - 1)) return -1;
    if (m < k + 1) m = k + 1;
    double *pool = (double *)malloc(sizeof(double) * (size_t)(nq * m));
    int64_t *sizes = (int64_t *)malloc(sizeof(int64_t) * (size_t)nq);
    if (!pool || !sizes) { free(pool); free(sizes); return -1; }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < nq; ++q) {
        double *h = pool + q * m;
        int64_t sz = 0;
        for (int64_t j = 0; j < n; ++j) {
            if (j == q) continue;
            heap_push(h, &sz, m, orc_d64(X + q * ld, X + j * ld, d));
        }
        sizes[q] = sz;
    }
    /* the m-th value of each full heap is its root; record before sorting */
    double *roots = (double *)malloc(sizeof(double) * (size_t)nq);
    double *flat = (double *)malloc(sizeof(double) * (size_t)(nq * m));
    int64_t nflat = 0;
    for (int64_t q = 0; q < nq; ++q) {
        roots[q] = (sizes[q] == m && m < n - 1) ? pool[q * m] : INFINITY;
        memcpy(flat + nflat, pool + q * m, sizeof(double) * (size_t)sizes[q]);
        nflat += sizes[q];
    }
    qsort(flat, (size_t)nflat, sizeof(double), cmp_double);
    double a = flat[K - 1], b = flat[K];
    int ok = 1;
    for (int64_t q = 0; q < nq; ++q)
        if (roots[q] <= b) ok = 0;
    *out_a = a;
    *out_b = b;
    free(pool); free(sizes); free(roots); free(flat);
    return ok ? 0 : 1;
}

/* ---- exact k nearest neighbours -------------------------------------------
 * Sec. VI recasts the k-nearest-neighbours search as distance similarity
 * searches whose radius grows until a query has k neighbours, which gives
 * the exact kNN.  The oracle computes that result from its definition: for
 * each selected query row, every one of the n points is ranked by the key
 * (D64(query, point), point id) ascending, and the first k keys are the
 * answer.  With Q == X the query itself is its own first neighbour (D64 = 0)
 * unless an identical point has a smaller id, just as the self-join counts
 * self pairs.
 *   ids  : [nrows][k] point ids, ascending key
 *   d64s : [nrows][k] their D64 (may be NULL)
 * Returns 0, -1 on bad arguments (also k < 1 or k > n), -2 if an input
 * holds a non-finite value, -3 if memory runs out.
 */
typedef struct {
    double d;
    uint32_t j;
} orc_ranked;

static int orc_ranked_cmp(const void *pa, const void *pb)
{
    const orc_ranked *a = (const orc_ranked *)pa, *b = (const orc_ranked *)pb;
    if (a->d < b->d) return -1;
    if (a->d > b->d) return 1;
    return (a->j > b->j) - (a->j < b->j);
}

int orc_knn(const float *Q, int64_t nq, int64_t ldq, const float *X, int64_t n, int64_t ld,
            int64_t d, int64_t k, const int64_t *rows, int64_t nrows, uint32_t *ids, double *d64s)
{
    int rc = check_inputs(X, n, d, ld, 0.0);
    if (rc) return rc;
    rc = check_inputs(Q, nq, d, ldq, 0.0);
    if (rc) return rc;
    if (!rows) nrows = nq;
    if (nrows < 0 || !ids || k < 1 || k > n || n > (int64_t)UINT32_MAX) return -1;
    int oom = 0;
#pragma omp parallel reduction(| : oom)
    {
        orc_ranked *all = (orc_ranked *)malloc(sizeof(orc_ranked) * (size_t)n);
        if (!all) oom = 1;
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!all) continue;
            const int64_t i = rows ? rows[r] : r;
            if (i < 0 || i >= nq) continue;
            const float *qi = Q + i * ldq;
            for (int64_t j = 0; j < n; ++j) {
                all[j].d = orc_d64(qi, X + j * ld, d);
                all[j].j = (uint32_t)j;
            }
            qsort(all, (size_t)n, sizeof(orc_ranked), orc_ranked_cmp);
            for (int64_t t = 0; t < k; ++t) {
                ids[r * k + t] = all[t].j;
                if (d64s) d64s[r * k + t] = all[t].d;
            }
        }
        free(all);
    }
    return oom ? -3 : 0;
}
