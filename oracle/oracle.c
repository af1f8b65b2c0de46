/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU oracle for dense nearest-neighbour (NN) search and
 * reciprocal matching between two per-pixel maps: descriptor maps (nearest =
 * largest inner product) or pointmaps (nearest = smallest Euclidean distance
 * between 3D points).  Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg load it; the
 * matching library never does, and the two share no code.
 *
 * Arithmetic: every similarity is an IEEE binary64 sum of binary64 products of
 * the fp32 inputs (bf16 inputs arrive exactly widened to fp32), accumulated
 * over the descriptor components in ascending order.  fp32 x fp32 products
 * are exact in binary64 and a 24-term sum of unit-vector products errs by
 * about 1e-15, so for these inputs the oracle is exact for all practical
 * purposes.  Pointmap distances are binary64 sums of the squared binary64
 * differences of the fp32 coordinates (each difference of two fp32 values of
 * similar magnitude is exact in binary64).  No blocking, no reordering, no vectorisation tricks; threads only
 * split independent queries.
 *
 * Sources (the pages are cited by title and section, never by line):
 *  [P1] "MASt3R dissection" (kensou.mintlify.app), section 1 architecture
 *       diagram: the match set is the set of pixel pairs (i, j) with
 *       NN(D1[i], D2) = j and NN(D2[j], D1) = i;
 *       section 3 "Napkin Formula": NN is the argmax of the inner product of
 *       L2-normalised descriptors, and the reciprocal test gives built-in
 *       outlier filtering.
 *  [P3] "DUSt3R and MASt3R explained" (3dgaussiansplattingcourse.com), the
 *       paragraph on MASt3R's third change (fast reciprocal matching): start
 *       from a sparse grid of seed pixels, repeatedly map each one to its best
 *       match in the other image and map that match back, collecting the
 *       pairs that map onto each other.
 *  [P3b] "DUSt3R and MASt3R explained", the paragraph on recovering the cameras:
 *       each image's pointmap holds one 3D point per pixel, both in the first
 *       camera's frame, and two pixels correspond when their predicted 3D
 *       points are nearest neighbours in that shared space.
 * Readings where the pages are silent (tie-break, seed origin, what one
 * iteration is, which pair is collected, which distance for pointmaps) are
 * stated at each function.
 *
 * Parity status: every function here is pinned by tests under tests/
 * (closed forms, brute force on tiny inputs, invariants); none is unpinned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_NOMEM (-2)
#define ORC_ERR_CAP (-3)

/* ------------------------------------------------------------------------
 * Similarity of two descriptors: sum over c = 0..d-1 of a[c] * b[c], in that
 * order, in binary64.  [P1] section 3: similarity is the inner product.
 * ------------------------------------------------------------------------ */
static double orc_similarity(const float* a, const float* b, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c)
        s += (double)a[c] * (double)b[c];
    return s;
}

/* ------------------------------------------------------------------------
 * Score of a (query, database) row pair under a metric; larger is nearer.
 *  ORC_INNER     : the similarity above (descriptor maps).
 *  ORC_NEG_SQ_L2 : minus the squared Euclidean distance, the differences and
 *                  their squares summed over ascending components in binary64
 *                  (pointmaps; [P3b]: nearest neighbours in the shared 3D space.
 *                  The pages name no norm; the plain reading is Euclidean, and
 *                  its square has the same nearest neighbour).
 * ------------------------------------------------------------------------ */
#define ORC_INNER 0
#define ORC_NEG_SQ_L2 1

static double orc_score(const float* a, const float* b, int d, int metric)
{
    if (metric == ORC_NEG_SQ_L2) {
        double acc = 0.0;
        for (int k = 0; k < d; ++k) {
            const double diff = (double)a[k] - (double)b[k];
            acc += diff * diff;
        }
        return -acc;
    }
    return orc_similarity(a, b, d);
}

/* ------------------------------------------------------------------------
 * NN of one query among n database rows: the first (lowest) index attaining
 * the maximum similarity, found by a scan with a strict ">" update.  Also
 * returns the best score (top1) and the best score over all other indices
 * (top2; an exact duplicate of the best gives top2 == top1).
 * [P1] section 3: j = argmax_k <D1[i], D2[k]>.  The pages do not say how ties
 * are broken; the reading here is the lowest index.
 * ------------------------------------------------------------------------ */
static void orc_nn_one(const float* q, const float* db, int64_t n, int d, int metric,
                       int32_t* idx, double* top1, double* top2)
{
    double best = -INFINITY, second = -INFINITY;
    int64_t arg = -1;
    for (int64_t k = 0; k < n; ++k) {
        double s = orc_score(q, db + k * (int64_t)d, d, metric);
        if (s > best) {
            second = best;
            best = s;
            arg = k;
        } else if (s > second) {
            second = s;
        }
    }
    *idx = (int32_t)arg;
    *top1 = best;
    *top2 = second;
}

/* ---- a parallel loop over independent queries ------------------------- */
typedef struct {
    const float* qmap;       /* query map rows */
    const int32_t* qidx;     /* rows of qmap to query, or NULL for 0..nq-1 */
    int64_t nq;
    const float* db;
    int64_t ndb;
    int d;
    int metric;
    int32_t* out_idx;
    double* out_top1;
    double* out_top2;
    int64_t begin, end;
} orc_nn_job;

static void* orc_nn_worker(void* p)
{
    orc_nn_job* j = (orc_nn_job*)p;
    for (int64_t t = j->begin; t < j->end; ++t) {
        int64_t row = j->qidx ? (int64_t)j->qidx[t] : t;
        double t1, t2;
        int32_t id;
        orc_nn_one(j->qmap + row * (int64_t)j->d, j->db, j->ndb, j->d, j->metric, &id, &t1, &t2);
        j->out_idx[t] = id;
        if (j->out_top1) j->out_top1[t] = t1;
        if (j->out_top2) j->out_top2[t] = t2;
    }
    return NULL;
}

static int orc_nn_parallel(const float* qmap, const int32_t* qidx, int64_t nq, const float* db,
                           int64_t ndb, int d, int metric, int nthreads, int32_t* out_idx,
                           double* out_top1, double* out_top2)
{
    if (nq <= 0) return ORC_OK;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > nq) nthreads = (int)nq;
    orc_nn_job jobs[256];
    pthread_t th[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (orc_nn_job){qmap, qidx, nq, db, ndb, d, metric, out_idx, out_top1, out_top2,
                               nq * i / nthreads, nq * (i + 1) / nthreads};
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i)
        started[i] = pthread_create(&th[i], NULL, orc_nn_worker, &jobs[i]) == 0;
    orc_nn_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (started[i]) pthread_join(th[i], NULL);
        else orc_nn_worker(&jobs[i]); /* could not start a thread: do the share here */
    }
    return ORC_OK;
}

/* ========================================================================
 * Exported entry points
 * ===================================================================== */

/* NN of every query row q[0..nq) among db[0..ndb) (rows of d floats) under a
 * metric (ORC_INNER or ORC_NEG_SQ_L2), as defined by orc_nn_one.
 * out_top1/out_top2 (the two best scores) may be NULL. */
int orc_nn_metric(const float* q, int64_t nq, const float* db, int64_t ndb, int32_t d, int32_t metric,
                  int32_t nthreads, int32_t* out_idx, double* out_top1, double* out_top2)
{
    if (!q || !db || !out_idx || nq < 0 || ndb < 0 || d < 1 || metric < 0 || metric > 1)
        return ORC_ERR_ARG;
    return orc_nn_parallel(q, NULL, nq, db, ndb, d, metric, nthreads, out_idx, out_top1, out_top2);
}

/* Same, for the query rows qmap[qidx[t]], t < nq. */
int orc_nn_rows_metric(const float* qmap, const int32_t* qidx, int64_t nq, const float* db, int64_t ndb,
                       int32_t d, int32_t metric, int32_t nthreads, int32_t* out_idx, double* out_top1,
                       double* out_top2)
{
    if (!qmap || !qidx || !db || !out_idx || nq < 0 || ndb < 0 || d < 1 || metric < 0 || metric > 1)
        return ORC_ERR_ARG;
    return orc_nn_parallel(qmap, qidx, nq, db, ndb, d, metric, nthreads, out_idx, out_top1, out_top2);
}

/* Score of the given row pairs: out[t] = score(A[ia[t]], B[ib[t]]). */
int orc_similarity_pairs_metric(const float* A, const float* B, int32_t d, int32_t metric,
                                const int32_t* ia, const int32_t* ib, int64_t n, double* out)
{
    if (!A || !B || !ia || !ib || !out || d < 1 || n < 0 || metric < 0 || metric > 1) return ORC_ERR_ARG;
    for (int64_t t = 0; t < n; ++t)
        out[t] = orc_score(A + (int64_t)ia[t] * d, B + (int64_t)ib[t] * d, d, metric);
    return ORC_OK;
}

/* The inner-product forms of the three calls above. */
int orc_nn(const float* q, int64_t nq, const float* db, int64_t ndb, int32_t d, int32_t nthreads,
           int32_t* out_idx, double* out_top1, double* out_top2)
{
    return orc_nn_metric(q, nq, db, ndb, d, ORC_INNER, nthreads, out_idx, out_top1, out_top2);
}

int orc_nn_rows(const float* qmap, const int32_t* qidx, int64_t nq, const float* db, int64_t ndb,
                int32_t d, int32_t nthreads, int32_t* out_idx, double* out_top1, double* out_top2)
{
    return orc_nn_rows_metric(qmap, qidx, nq, db, ndb, d, ORC_INNER, nthreads, out_idx, out_top1, out_top2);
}

int orc_similarity_pairs(const float* A, const float* B, int32_t d, const int32_t* ia,
                         const int32_t* ib, int64_t n, double* out)
{
    return orc_similarity_pairs_metric(A, B, d, ORC_INNER, ia, ib, n, out);
}

/* ------------------------------------------------------------------------
 * Mutual (reciprocal) NN set from the two NN maps.
 * [P1] section 1 diagram and section 3: (i, j) is a match iff
 * NN(D1[i], D2) = j and NN(D2[j], D1) = i.
 * Output pairs (i, nn12[i]) in ascending i; returns the count (or < 0).
 * ------------------------------------------------------------------------ */
int64_t orc_mutual(const int32_t* nn12, int64_t n1, const int32_t* nn21, int64_t n2,
                   int32_t* pairs, int64_t cap)
{
    if (!nn12 || !nn21 || !pairs || n1 < 0 || n2 < 0) return ORC_ERR_ARG;
    int64_t m = 0;
    for (int64_t i = 0; i < n1; ++i) {
        int32_t j = nn12[i];
        if (j < 0 || j >= n2) continue;
        if (nn21[j] != i) continue;
        if (m >= cap) return ORC_ERR_CAP;
        pairs[2 * m] = (int32_t)i;
        pairs[2 * m + 1] = j;
        ++m;
    }
    return m;
}

/* Margin of an NN decision from its two best scores: absolute for the inner
 * product, relative to the second distance for pointmaps (no second candidate:
 * infinite; a zero second distance, i.e. a tie at distance 0: zero). */
static double orc_margin(double top1, double top2, int metric)
{
    if (metric != ORC_NEG_SQ_L2) return top1 - top2;
    if (top2 == -INFINITY) return INFINITY;
    if (top2 == 0.0) return 0.0;
    return (top1 - top2) / -top2;
}

/* ------------------------------------------------------------------------
 * Fast reciprocal matching.  [P3], the fast-matching paragraph; [P1] section 3.
 *
 * Readings (the pages give the idea, not the exact steps):
 *  - seeds: the regular grid {(y, x): y = offset + stride*a < H1,
 *    x = offset + stride*b < W1} of image 1, pixel id y*W1 + x;
 *    seed_limit >= 0 keeps only the first seed_limit seeds in row-major order
 *    (used to time a bounded sample), -1 keeps all;
 *  - one iteration maps the current pixel u_t forward, v_t = NN12(u_t), and
 *    back, u_{t+1} = NN21(v_t);
 *  - if u_{t+1} == u_t the chain has converged and (u_t, v_t) is collected
 *    (a reciprocal pair); otherwise it restarts from u_{t+1};
 *  - iterations t = 0 .. T-1; a chain that has not converged after T
 *    iterations contributes nothing;
 *  - the output is the set of collected pairs, ascending in u.
 * Every NN here is orc_nn_one under the given metric (lowest index on ties);
 * results are memoised per pixel, which changes no result.
 *
 * Extra records for the tests:
 *  - active[t]   : number of distinct pixels carried by live chains at the
 *                  start of iteration t (NULL to skip);
 *  - pair_clean  : per output pair, 1 if some chain that collected it made
 *                  only NN decisions whose margin exceeds eps: top1 - top2 for
 *                  the inner product; for pointmaps the relative margin
 *                  (d2 - d1) / d2 of the two smallest squared distances;
 *  - nn_queries  : number of NN searches performed (after memoisation);
 *  - fresh[t]    : number of those pixels live at iteration t that were live
 *                  in no earlier iteration (NULL to skip).  A policy that
 *                  never restarts a chain on a pixel that has ever been live
 *                  (the set of pairs is the same, see the characterisation
 *                  above) carries exactly these pixels at iteration t;
 *  - seed_u[c]   : the image-1 pixel at which seed c's chain converged, -1 if
 *                  it had not converged after T iterations (NULL to skip);
 *  - seed_clean[c]: 1 if every NN decision made along seed c's chain (up to
 *                  its convergence, or through iteration T-1) had a margin
 *                  above eps (NULL to skip).
 * A chain whose decisions all clear the margin is followed identically by any
 * search whose chosen NN equals the exact one wherever the margin exceeds
 * eps; only the other chains can end elsewhere.
 * ------------------------------------------------------------------------ */
int orc_fast_ex(const float* A, int32_t H1, int32_t W1, const float* B, int64_t n2, int32_t d,
                int32_t metric, int32_t stride, int32_t offset, int32_t T, int32_t seed_limit,
                int32_t nthreads, double eps, int32_t* pairs, int64_t cap, int64_t* n_pairs,
                uint8_t* pair_clean, int64_t* active, int64_t* nn_queries, int64_t* fresh,
                int32_t* seed_u, uint8_t* seed_clean)
{
    if (!A || !B || !pairs || !n_pairs || H1 < 0 || W1 < 0 || n2 < 0 || d < 1 || stride < 1 ||
        offset < 0 || T < 0 || metric < 0 || metric > 1)
        return ORC_ERR_ARG;
    const int64_t n1 = (int64_t)H1 * W1;
    *n_pairs = 0;
    if (nn_queries) *nn_queries = 0;
    if (active)
        for (int t = 0; t < T; ++t) active[t] = 0;
    if (fresh)
        for (int t = 0; t < T; ++t) fresh[t] = 0;

    /* seeds */
    int64_t ns = 0;
    for (int64_t y = offset; y < H1; y += stride)
        for (int64_t x = offset; x < W1; x += stride) ++ns;
    if (seed_limit >= 0 && ns > seed_limit) ns = seed_limit;
    for (int64_t c = 0; c < ns; ++c) {
        if (seed_u) seed_u[c] = -1;
        if (seed_clean) seed_clean[c] = 1;
    }
    if (ns == 0 || n1 == 0 || n2 == 0 || T == 0) return ORC_OK;

    int rc = ORC_ERR_NOMEM;
    int32_t* cur = malloc(sizeof(int32_t) * ns);       /* chain position u_t */
    uint8_t* alive = malloc(ns);
    uint8_t* clean = malloc(ns);
    int32_t* nn12 = malloc(sizeof(int32_t) * n1);      /* memo: -1 = not yet known */
    double* mg12 = malloc(sizeof(double) * n1);
    int32_t* nn21 = malloc(sizeof(int32_t) * n2);
    double* mg21 = malloc(sizeof(double) * n2);
    int32_t* match = malloc(sizeof(int32_t) * n1);     /* collected v per u, -1 = none */
    uint8_t* mclean = malloc(n1);
    uint8_t* seen1 = malloc(n1);
    uint8_t* seen2 = malloc(n2);
    uint8_t* ever1 = malloc(n1);                         /* live in some earlier iteration */
    int32_t* todo = malloc(sizeof(int32_t) * ns);
    int32_t* res = malloc(sizeof(int32_t) * ns);
    double* t1 = malloc(sizeof(double) * ns);
    double* t2 = malloc(sizeof(double) * ns);
    if (!cur || !alive || !clean || !nn12 || !mg12 || !nn21 || !mg21 || !match || !mclean ||
        !seen1 || !seen2 || !ever1 || !todo || !res || !t1 || !t2)
        goto done;

    for (int64_t i = 0; i < n1; ++i) { nn12[i] = -1; match[i] = -1; mclean[i] = 0; seen1[i] = 0; ever1[i] = 0; }
    for (int64_t i = 0; i < n2; ++i) { nn21[i] = -1; seen2[i] = 0; }
    {
        int64_t c = 0;
        for (int64_t y = offset; y < H1 && c < ns; y += stride)
            for (int64_t x = offset; x < W1 && c < ns; x += stride) {
                cur[c] = (int32_t)(y * W1 + x);
                alive[c] = 1;
                clean[c] = 1;
                ++c;
            }
    }

    for (int32_t t = 0; t < T; ++t) {
        /* forward: NN12 of every distinct live pixel not yet known */
        int64_t nt = 0, distinct = 0, first_visits = 0;
        for (int64_t c = 0; c < ns; ++c) {
            if (!alive[c]) continue;
            int32_t u = cur[c];
            if (!seen1[u]) {
                seen1[u] = 1;
                ++distinct;
                if (!ever1[u]) ++first_visits;
                if (nn12[u] < 0) todo[nt++] = u;
            }
        }
        for (int64_t c = 0; c < ns; ++c)
            if (alive[c]) { seen1[cur[c]] = 0; ever1[cur[c]] = 1; }
        if (active) active[t] = distinct;
        if (fresh) fresh[t] = first_visits;
        if (distinct == 0) break;
        orc_nn_parallel(A, todo, nt, B, n2, d, metric, nthreads, res, t1, t2);
        for (int64_t k = 0; k < nt; ++k) { nn12[todo[k]] = res[k]; mg12[todo[k]] = orc_margin(t1[k], t2[k], metric); }
        if (nn_queries) *nn_queries += nt;

        /* backward: NN21 of every distinct landing pixel not yet known */
        nt = 0;
        for (int64_t c = 0; c < ns; ++c) {
            if (!alive[c]) continue;
            int32_t v = nn12[cur[c]];
            if (!seen2[v]) { seen2[v] = 1; if (nn21[v] < 0) todo[nt++] = v; }
        }
        for (int64_t c = 0; c < ns; ++c) if (alive[c]) seen2[nn12[cur[c]]] = 0;
        orc_nn_parallel(B, todo, nt, A, n1, d, metric, nthreads, res, t1, t2);
        for (int64_t k = 0; k < nt; ++k) { nn21[todo[k]] = res[k]; mg21[todo[k]] = orc_margin(t1[k], t2[k], metric); }
        if (nn_queries) *nn_queries += nt;

        /* reciprocity check: converged chains are collected, the rest restart */
        for (int64_t c = 0; c < ns; ++c) {
            if (!alive[c]) continue;
            int32_t u = cur[c];
            int32_t v = nn12[u];
            int32_t u2 = nn21[v];
            if (!(mg12[u] > eps) || !(mg21[v] > eps)) clean[c] = 0;
            if (u2 == u) {
                match[u] = v;
                if (clean[c]) mclean[u] = 1;
                if (seed_u) seed_u[c] = u;
                alive[c] = 0;
            } else {
                cur[c] = u2;
            }
        }
    }

    {
        int64_t m = 0;
        for (int64_t u = 0; u < n1; ++u) {
            if (match[u] < 0) continue;
            if (m >= cap) { rc = ORC_ERR_CAP; goto done; }
            pairs[2 * m] = (int32_t)u;
            pairs[2 * m + 1] = match[u];
            if (pair_clean) pair_clean[m] = mclean[u];
            ++m;
        }
        *n_pairs = m;
    }
    if (seed_clean)
        for (int64_t c = 0; c < ns; ++c) seed_clean[c] = clean[c];
    rc = ORC_OK;
done:
    free(cur); free(alive); free(clean); free(nn12); free(mg12); free(nn21); free(mg21);
    free(match); free(mclean); free(seen1); free(seen2); free(ever1); free(todo); free(res); free(t1);
    free(t2);
    return rc;
}

/* orc_fast_ex without the per-seed and first-visit records. */
int orc_fast_metric(const float* A, int32_t H1, int32_t W1, const float* B, int64_t n2, int32_t d,
                    int32_t metric, int32_t stride, int32_t offset, int32_t T, int32_t seed_limit,
                    int32_t nthreads, double eps, int32_t* pairs, int64_t cap, int64_t* n_pairs,
                    uint8_t* pair_clean, int64_t* active, int64_t* nn_queries)
{
    return orc_fast_ex(A, H1, W1, B, n2, d, metric, stride, offset, T, seed_limit, nthreads, eps, pairs, cap,
                       n_pairs, pair_clean, active, nn_queries, NULL, NULL, NULL);
}

/* The inner-product form of orc_fast_metric. */
int orc_fast(const float* A, int32_t H1, int32_t W1, const float* B, int64_t n2, int32_t d,
             int32_t stride, int32_t offset, int32_t T, int32_t seed_limit, int32_t nthreads,
             double eps, int32_t* pairs, int64_t cap, int64_t* n_pairs, uint8_t* pair_clean,
             int64_t* active, int64_t* nn_queries)
{
    return orc_fast_metric(A, H1, W1, B, n2, d, ORC_INNER, stride, offset, T, seed_limit, nthreads, eps,
                           pairs, cap, n_pairs, pair_clean, active, nn_queries);
}

/* ------------------------------------------------------------------------
 * Matching loss (InfoNCE).  [P1] section 3 ("Napkin Formula"): over the
 * ground-truth matches M_gt,
 *     L = - sum_{(i,j) in M_gt} log( exp(<D1[i], D2[j]> / tau)
 *                                    / sum_k exp(<D1[i], D2[k]> / tau) ),
 * the softmax running over every pixel k of image 2.  Term (i, j) is
 * LSE_i - <D1[i], D2[j]> / tau with LSE_i = log sum_k exp(<D1[i], D2[k]> / tau),
 * evaluated here in binary64 as m + log sum_k exp(s_k / tau - m), m the largest
 * s_k / tau (exact algebra; it only keeps the exponentials finite).
 * gt: int32 [n_gt][2] pairs (i, j); out_terms[t] = term of pair t; *out_total =
 * their sum.  Pairs with an index out of range are rejected.
 * ------------------------------------------------------------------------ */
typedef struct {
    const float* A; const float* B; int64_t n2; int d; double tau;
    const int32_t* gt; double* terms; int64_t begin, end;
} orc_nce_job;

static void* orc_nce_worker(void* p)
{
    orc_nce_job* j = (orc_nce_job*)p;
    for (int64_t t = j->begin; t < j->end; ++t) {
        const float* q = j->A + (int64_t)j->gt[2 * t] * j->d;
        double m = -INFINITY;
        for (int64_t k = 0; k < j->n2; ++k) {
            const double z = orc_similarity(q, j->B + k * (int64_t)j->d, j->d) / j->tau;
            if (z > m) m = z;
        }
        double sum = 0.0;
        for (int64_t k = 0; k < j->n2; ++k)
            sum += exp(orc_similarity(q, j->B + k * (int64_t)j->d, j->d) / j->tau - m);
        const double pos = orc_similarity(q, j->B + (int64_t)j->gt[2 * t + 1] * j->d, j->d) / j->tau;
        j->terms[t] = m + log(sum) - pos;
    }
    return NULL;
}

int orc_infonce(const float* A, int64_t n1, const float* B, int64_t n2, int32_t d, const int32_t* gt,
                int64_t n_gt, double tau, int32_t nthreads, double* out_terms, double* out_total)
{
    if (!A || !B || !gt || !out_terms || !out_total || n1 < 0 || n2 < 1 || d < 1 || n_gt < 0 || !(tau > 0))
        return ORC_ERR_ARG;
    for (int64_t t = 0; t < n_gt; ++t)
        if (gt[2 * t] < 0 || gt[2 * t] >= n1 || gt[2 * t + 1] < 0 || gt[2 * t + 1] >= n2) return ORC_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (n_gt > 0 && nthreads > n_gt) nthreads = (int)n_gt;
    orc_nce_job jobs[256];
    pthread_t th[256];
    int started[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = (orc_nce_job){A, B, n2, d, tau, gt, out_terms, n_gt * i / nthreads, n_gt * (i + 1) / nthreads};
        started[i] = 0;
    }
    for (int i = 1; i < nthreads; ++i) started[i] = pthread_create(&th[i], NULL, orc_nce_worker, &jobs[i]) == 0;
    if (nthreads > 0) orc_nce_worker(&jobs[0]);
    for (int i = 1; i < nthreads; ++i) {
        if (started[i]) pthread_join(th[i], NULL);
        else orc_nce_worker(&jobs[i]);
    }
    double total = 0.0;
    for (int64_t t = 0; t < n_gt; ++t) total += out_terms[t];
    *out_total = total;
    return ORC_OK;
}

/* ------------------------------------------------------------------------
 * Gradient of the matching loss L = sum_t term_t (orc_infonce) with respect to
 * both descriptor maps.  The derivative of a log-sum-exp is the softmax, so with
 *     p[t][k] = exp(<D1[i_t], D2[k]> / tau - LSE_t)
 * (term t's softmax over the rows k of image 2),
 *     dL/dD1[i] = (1/tau) sum_{t: i_t = i} ( sum_k p[t][k] D2[k] - D2[j_t] ),
 *     dL/dD2[k] = (1/tau) sum_t p[t][k] D1[i_t] - (1/tau) sum_{t: j_t = k} D1[i_t].
 * Steps, in binary64: (1) LSE_t for every t, as orc_infonce does (threads over
 * t); (2) for every t the vector sum_k p[t][k] D2[k] - D2[j_t] (threads over t);
 * (3) dA[i] = sum of those vectors over t with i_t = i, ascending t, times 1/tau;
 * (4) for every listed row k of image 2 (threads over the list): dB = the sum over
 * t ascending of p[t][k] D1[i_t], minus D1[i_t] for each t with j_t = k, times
 * 1/tau, and colmass = sum_t p[t][k] (the scale of that row's gradient).
 * dA: [n1][d], fully written; dB, colmass: one row per entry of b_rows.
 * ------------------------------------------------------------------------ */
typedef struct {
    const float* A; const float* B; int64_t n2; int d; double tau; const int32_t* gt; int64_t n_gt;
    double* lse; double* g; const int32_t* rows; double* dB; double* colmass; int64_t begin, end;
} orc_grad_job;

static void* orc_grad_rows_worker(void* p)
{
    orc_grad_job* j = (orc_grad_job*)p;
    const int d = j->d;
    for (int64_t t = j->begin; t < j->end; ++t) {
        const float* q = j->A + (int64_t)j->gt[2 * t] * d;
        double m = -INFINITY;
        for (int64_t k = 0; k < j->n2; ++k) {
            const double z = orc_similarity(q, j->B + k * (int64_t)d, d) / j->tau;
            if (z > m) m = z;
        }
        double sum = 0.0;
        for (int64_t k = 0; k < j->n2; ++k) sum += exp(orc_similarity(q, j->B + k * (int64_t)d, d) / j->tau - m);
        const double lse = m + log(sum);
        j->lse[t] = lse;
        double* g = j->g + t * (int64_t)d;
        for (int e = 0; e < d; ++e) g[e] = 0.0;
        for (int64_t k = 0; k < j->n2; ++k) {
            const double pk = exp(orc_similarity(q, j->B + k * (int64_t)d, d) / j->tau - lse);
            for (int e = 0; e < d; ++e) g[e] += pk * (double)j->B[k * (int64_t)d + e];
        }
        const float* bj = j->B + (int64_t)j->gt[2 * t + 1] * d;
        for (int e = 0; e < d; ++e) g[e] -= (double)bj[e];
    }
    return NULL;
}

static void* orc_grad_cols_worker(void* p)
{
    orc_grad_job* j = (orc_grad_job*)p;
    const int d = j->d;
    for (int64_t r = j->begin; r < j->end; ++r) {
        const int64_t k = j->rows[r];
        const float* bk = j->B + k * d;
        double* out = j->dB + r * (int64_t)d;
        double mass = 0.0;
        for (int e = 0; e < d; ++e) out[e] = 0.0;
        for (int64_t t = 0; t < j->n_gt; ++t) {
            const float* a = j->A + (int64_t)j->gt[2 * t] * d;
            const double pk = exp(orc_similarity(a, bk, d) / j->tau - j->lse[t]);
            mass += pk;
            for (int e = 0; e < d; ++e) out[e] += pk * (double)a[e];
            if (j->gt[2 * t + 1] == k)
                for (int e = 0; e < d; ++e) out[e] -= (double)a[e];
        }
        for (int e = 0; e < d; ++e) out[e] /= j->tau;
        j->colmass[r] = mass;
    }
    return NULL;
}

static void orc_run_jobs(orc_grad_job* jobs, int n, void* (*fn)(void*))
{
    pthread_t th[256];
    int started[256];
    for (int i = 1; i < n; ++i) started[i] = pthread_create(&th[i], NULL, fn, &jobs[i]) == 0;
    if (n > 0) fn(&jobs[0]);
    for (int i = 1; i < n; ++i) {
        if (started[i]) pthread_join(th[i], NULL);
        else fn(&jobs[i]);
    }
}

int orc_infonce_grad(const float* A, int64_t n1, const float* B, int64_t n2, int32_t d, const int32_t* gt,
                     int64_t n_gt, double tau, const int32_t* b_rows, int64_t n_rows, int32_t nthreads,
                     double* dA, double* dB, double* colmass)
{
    if (!A || !B || !gt || !dA || n1 < 0 || n2 < 1 || d < 1 || n_gt < 0 || !(tau > 0) || n_rows < 0 ||
        (n_rows > 0 && (!b_rows || !dB || !colmass)))
        return ORC_ERR_ARG;
    for (int64_t t = 0; t < n_gt; ++t)
        if (gt[2 * t] < 0 || gt[2 * t] >= n1 || gt[2 * t + 1] < 0 || gt[2 * t + 1] >= n2) return ORC_ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r)
        if (b_rows[r] < 0 || b_rows[r] >= n2) return ORC_ERR_ARG;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    double* lse = (double*)malloc(sizeof(double) * (size_t)(n_gt > 0 ? n_gt : 1));
    double* g = (double*)malloc(sizeof(double) * (size_t)(n_gt > 0 ? n_gt : 1) * (size_t)d);
    if (!lse || !g) { free(lse); free(g); return ORC_ERR_NOMEM; }
    orc_grad_job jobs[256];
    int nt = n_gt > 0 && nthreads > n_gt ? (int)n_gt : nthreads;
    for (int i = 0; i < nt; ++i)
        jobs[i] = (orc_grad_job){A, B, n2, d, tau, gt, n_gt, lse, g, b_rows, dB, colmass,
                                 n_gt * i / nt, n_gt * (i + 1) / nt};
    orc_run_jobs(jobs, nt, orc_grad_rows_worker);
    for (int64_t x = 0; x < n1 * (int64_t)d; ++x) dA[x] = 0.0;
    for (int64_t t = 0; t < n_gt; ++t) {
        double* row = dA + (int64_t)gt[2 * t] * d;
        for (int e = 0; e < d; ++e) row[e] += g[t * (int64_t)d + e] / tau;
    }
    nt = n_rows > 0 && nthreads > n_rows ? (int)n_rows : nthreads;
    for (int i = 0; i < nt; ++i)
        jobs[i] = (orc_grad_job){A, B, n2, d, tau, gt, n_gt, lse, g, b_rows, dB, colmass,
                                 n_rows * i / nt, n_rows * (i + 1) / nt};
    if (n_rows > 0) orc_run_jobs(jobs, nt, orc_grad_cols_worker);
    free(lse);
    free(g);
    return ORC_OK;
}
