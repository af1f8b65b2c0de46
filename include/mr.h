/*
 * mr.h -- dense nearest-neighbour search and reciprocal matching between two
 * per-pixel descriptor maps (or two pointmaps, see the mr_point_* calls), on AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (the pages are cited by title and section):
 *  - Similarity of two descriptors is their inner product; the maps hold one
 *    L2-normalised descriptor per pixel (d = 24 in MASt3R).
 *    ["MASt3R dissection", section 3 "Napkin Formula"; "DUSt3R and MASt3R
 *    explained", paragraph on MASt3R's dense local-feature head.]
 *  - The NN of a query is the database row of maximal similarity, compared
 *    after clearing the 4 lowest bits of the fp32 score (a relative step of at
 *    most 2^-19, far inside the 1e-5 parity tolerance); ties go to the lowest
 *    row index (the pages are silent on ties).  Both search directions use
 *    this one rule, so reciprocity is judged consistently.
 *  - A reciprocal (mutual) match is a pair (i, j) with NN(D1[i], D2) = j and
 *    NN(D2[j], D1) = i.  ["MASt3R dissection", section 1 diagram, section 3.]
 *  - The fast reciprocal scheme seeds a regular grid of image 1, maps every
 *    live pixel to its NN in image 2 and back, keeps the pairs that map onto
 *    each other and restarts the others from where they landed, for a fixed
 *    number of iterations.  ["DUSt3R and MASt3R explained", the paragraph on
 *    MASt3R's fast reciprocal matching.]
 *
 * Arithmetic: bf16 maps use exact bf16 products with fp32 accumulation on the
 * matrix cores.  fp32 maps with d a multiple of 8 (d <= 32) are split exactly
 * into three bf16 parts x = h + m + l and the six products hh, hm, mh, mm, hl,
 * lh are accumulated in fp32 (the dropped terms are below 2^-23 |x||y|, i.e.
 * fp32-accurate); other fp32 maps use fp32 products on the matrix cores.
 * Every kernel computes s(i, j) with the same instruction and the same
 * component order, so a score is bitwise the same whichever map plays the
 * query.  -0.0 is treated as +0.0.  Inputs must be finite (NaN/Inf are out of
 * contract).
 *
 * Conventions shared by every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates no device memory: scratch space comes in through `ws`
 *    (`ws_bytes` long, 256-byte aligned, size from mr_workspace_bytes).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls are asynchronous on that stream; outputs are valid once the stream
 *    has completed the call.  Calls that share a workspace must not overlap.
 *  - The entry points keep no state between calls (the measurement aid at the
 *    end of this file is the one opt-in exception, confined to the thread that
 *    opens it) and are thread-safe given distinct workspaces.
 *  - Arguments are validated on the host before anything is launched; a
 *    nonzero return means nothing was enqueued.  MR_ERR_DEVICE reports a
 *    launch failure after some work may have been enqueued.
 *  - A map is a contiguous row-major array [batch][h][w][d]; pixel id
 *    p = y*w + x.  Supported: 1 <= d <= 64, dtype MR_F32 or MR_BF16 (bf16
 *    needs d to be a multiple of 8), h*w <= 2^28.  Both maps of a call must
 *    agree on batch, d and dtype; their h and w may differ.
 */
#ifndef MR_H
#define MR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MR_F32 = 0, MR_BF16 = 1 } mr_dtype;

typedef enum {
    MR_OK = 0,
    MR_ERR_NULL = 1,      /* a required pointer is NULL */
    MR_ERR_SHAPE = 2,     /* sizes out of range or inconsistent between the maps */
    MR_ERR_DTYPE = 3,     /* unknown dtype, dtypes differ, or bf16 with d % 8 != 0 */
    MR_ERR_PARAM = 4,     /* stride < 1, offset < 0, max_iters < 0, bad op, n_q < 0 */
    MR_ERR_WORKSPACE = 5, /* ws NULL/misaligned while needed, or ws_bytes too small */
    MR_ERR_CAPACITY = 6,  /* cap below the static bound on the number of pairs */
    MR_ERR_DEVICE = 7,    /* a HIP call failed */
    MR_ERR_SCRATCH = 8    /* mr_fast_reciprocal_static: more scratch than its static buffer */
} mr_status;

typedef struct {
    const void* data; /* device pointer to [batch][h][w][d] */
    int32_t batch, h, w, d;
    int32_t dtype;    /* mr_dtype */
} mr_map;

enum {
    MR_OP_NN_ARGMAX = 0, MR_OP_MUTUAL_NN = 1, MR_OP_FAST_RECIPROCAL = 2,
    MR_OP_POINT_NN = 3, MR_OP_POINT_MUTUAL_NN = 4, MR_OP_POINT_FAST_RECIPROCAL = 5,
    MR_OP_FAST_RECIPROCAL_GRAPH = 6,  /* a = b = the image collection, n_q = number of edges */
    MR_OP_INFONCE = 7,                /* n_q = ground-truth pairs per image pair */
    MR_OP_INFONCE_BACKWARD = 8        /* n_q = ground-truth pairs per image pair */
};

/* Workspace bytes that entry point `op` needs for these maps and parameters
 * (n_q: queries per pair for MR_OP_NN_ARGMAX; stride/offset for
 * MR_OP_FAST_RECIPROCAL; other arguments are ignored).  Returns 0 for invalid
 * arguments (the entry point itself then reports the error). */
size_t mr_workspace_bytes(int op, const mr_map* a, const mr_map* b, int64_t n_q, int32_t stride,
                          int32_t offset);

/* Static text for a status code. */
const char* mr_status_str(int status);

/* Number of seeds on the grid {(offset + stride*a, offset + stride*b)} of an
 * h x w image, i.e. the capacity mr_fast_reciprocal needs per pair; -1 for
 * invalid arguments. */
int64_t mr_seed_count(int32_t h, int32_t w, int32_t stride, int32_t offset);

/* ---------------------------------------------------------------------------
 * mr_nn_argmax: nearest neighbour of query rows of map q among all rows of
 * map db of the same pair ("MASt3R dissection", section 3: j = argmax_k of
 * the inner product).
 *   q_idx    : NULL to query every row of q (then n_q must be q->h*q->w), or
 *              [batch][n_q] row ids local to each pair's q map.
 *   out_idx  : [batch][n_q] NN row id in db (lowest index on ties); -1 when
 *              db has no rows.
 *   out_score: NULL or [batch][n_q] fp32 similarity of that NN (with its 4
 *              lowest bits cleared, as compared).
 * --------------------------------------------------------------------------- */
int mr_nn_argmax(const mr_map* q, const mr_map* db, const int32_t* q_idx, int64_t n_q,
                 int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * mr_mutual_nn: brute-force reciprocal NN ("MASt3R dissection", section 1
 * diagram and section 3; "DUSt3R and MASt3R explained": the quadratic
 * all-pairs baseline).
 *   nn_ab  : [batch][Na] NN in b of every pixel of a.
 *   nn_ba  : [batch][Nb] NN in a of every pixel of b.
 *   pairs  : [batch][cap][2] (i, j) with nn_ab[i] = j and nn_ba[j] = i,
 *            ascending in i; cap >= min(Na, Nb).
 *   n_pairs: [batch] int64 counts.
 * --------------------------------------------------------------------------- */
int mr_mutual_nn(const mr_map* a, const mr_map* b, int32_t* nn_ab, int32_t* nn_ba, int32_t* pairs,
                 int64_t cap, int64_t* n_pairs, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * mr_fast_reciprocal: the fast reciprocal matching scheme ("DUSt3R and
 * MASt3R explained", paragraph on the fast reciprocal matching; "MASt3R
 * dissection", section 3: early termination plus bidirectional NN).
 *   Seeds: pixels (y, x) of image a with y = offset + stride*i < h and
 *   x = offset + stride*j < w.  One iteration maps every live pixel u to
 *   v = NN(a[u], b) and back to u' = NN(b[v], a).  If u' == u, (u, v) is kept
 *   and u stops; otherwise u' becomes live unless it is already matched or was
 *   live in this or an earlier iteration (its future is then already being
 *   followed).  max_iters iterations at most; max_iters = 0 gives no pairs.
 *   The kept set equals {(p, NN(a[p], b)) : p = f(p), p = f^t(seed),
 *   t < max_iters} with f(u) = u'.
 *   pairs      : [batch][cap][2] ascending in u; cap >= mr_seed_count(...).
 *   n_pairs    : [batch] int64 counts.
 *   iter_active: NULL or [batch][max_iters] int32: live pixels at the start
 *                of each iteration.
 * --------------------------------------------------------------------------- */
int mr_fast_reciprocal(const mr_map* a, const mr_map* b, int32_t stride, int32_t offset,
                       int32_t max_iters, int32_t* pairs, int64_t cap, int64_t* n_pairs,
                       int32_t* iter_active, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * mr_fast_reciprocal_static: mr_fast_reciprocal without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments (minus ws and
 * ws_bytes), results, validation and error codes as mr_fast_reciprocal.
 *   Scratch: a static device array of 16 MiB per GPU, held by the library until the
 *   process ends; the calling thread's current device must be the one `stream` and
 *   the maps belong to.  Problems needing more (mr_workspace_bytes with
 *   MR_OP_FAST_RECIPROCAL above 16 MiB: e.g. more than nine 512x384 pairs per call
 *   at stride 8; one 1024x768 pair needs 6.5 MiB) return MR_ERR_SCRATCH before
 *   anything is launched.  The call allocates
 *   nothing: no hipMalloc, hipFree or allocating library routine.
 *   Every call on a GPU shares that GPU's buffer, and each call re-initialises the
 *   part it uses on its stream: calls that overlap in time on one GPU (other threads,
 *   other streams) race and must be serialised by the caller.
 * --------------------------------------------------------------------------- */
int mr_fast_reciprocal_static(const mr_map* a, const mr_map* b, int32_t stride, int32_t offset,
                              int32_t max_iters, int32_t* pairs, int64_t cap, int64_t* n_pairs,
                              int32_t* iter_active, void* stream);

/* ---------------------------------------------------------------------------
 * mr_fast_reciprocal_graph: the fast scheme on many pairs of one collection of
 * images (a reconstruction runs the pair model on every useful pair of a
 * collection, organised as a graph: "DUSt3R and MASt3R explained", the
 * paragraph on reconstructing a collection).  Each map is stored once.
 *   images : the collection, batch = number of images (one map per image).
 *   edges  : HOST int32 [n_edges][2]: edge e matches image edges[e][0] (seeded,
 *            "image a") against image edges[e][1] ("image b"); ids must lie in
 *            [0, images->batch) (else MR_ERR_PARAM); 1 <= n_edges <= 65535.
 *            Copied into the workspace on `stream` before the call returns.
 *   pairs, n_pairs, iter_active: per edge, as mr_fast_reciprocal's per pair.
 *   ws     : mr_workspace_bytes(MR_OP_FAST_RECIPROCAL_GRAPH, images, images,
 *            n_edges, stride, offset) bytes.
 * Results equal mr_fast_reciprocal on each edge's two maps.
 * --------------------------------------------------------------------------- */
int mr_fast_reciprocal_graph(const mr_map* images, const int32_t* edges, int32_t n_edges, int32_t stride,
                             int32_t offset, int32_t max_iters, int32_t* pairs, int64_t cap, int64_t* n_pairs,
                             int32_t* iter_active, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Pointmaps.  A pointmap holds, for every pixel, the 3D point that pixel
 * observes; both maps of a pair are expressed in the first camera's frame, and
 * two pixels correspond when their points are nearest neighbours in that shared
 * space ("DUSt3R and MASt3R explained", the paragraph on recovering the
 * cameras).  Nearest = smallest squared Euclidean distance, computed in fp32 as
 * t0*t0 + t1*t1 + ... with t_c = x_c - y_c, in ascending c, each step rounded
 * once (a fused multiply-add after the first product); equal fp32 distances go
 * to the lowest row.  Against binary64 the distance errs by at most about
 * 2^-21 of itself.
 * The three calls mirror the descriptor calls above -- same arguments, workspace
 * (from mr_workspace_bytes with the MR_OP_POINT_* codes), outputs, ordering and
 * error behaviour -- with nearest-point search in place of the largest inner
 * product.  Maps: dtype MR_F32 (else MR_ERR_DTYPE), 1 <= d <= 4 (else
 * MR_ERR_SHAPE); d = 3 for pointmaps.  Finite coordinates of any scale.
 *   mr_point_nn       : out_dist2 NULL or [batch][n_q] fp32 squared distance
 *                       of the chosen row (+INF when db has no rows).
 *   mr_point_mutual_nn: reciprocal nearest points, as mr_mutual_nn.
 *   mr_point_fast_reciprocal: the fast scheme of mr_fast_reciprocal with
 *                       nearest points.
 * --------------------------------------------------------------------------- */
int mr_point_nn(const mr_map* q, const mr_map* db, const int32_t* q_idx, int64_t n_q, int32_t* out_idx,
                float* out_dist2, void* ws, size_t ws_bytes, void* stream);
int mr_point_mutual_nn(const mr_map* a, const mr_map* b, int32_t* nn_ab, int32_t* nn_ba, int32_t* pairs,
                       int64_t cap, int64_t* n_pairs, void* ws, size_t ws_bytes, void* stream);
int mr_point_fast_reciprocal(const mr_map* a, const mr_map* b, int32_t stride, int32_t offset,
                             int32_t max_iters, int32_t* pairs, int64_t cap, int64_t* n_pairs,
                             int32_t* iter_active, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * mr_infonce_forward: the matching loss of a descriptor pair over its
 * ground-truth correspondences ("MASt3R dissection", section 3 "Napkin
 * Formula": the InfoNCE objective with temperature tau, negatives taken from
 * every pixel of the second image).  For ground-truth pair t = (i, j):
 *     term[t] = log sum_k exp(<a_i, b_k> / tau) - <a_i, b_j> / tau,
 * k over all rows of b; loss = sum_t term[t] (a sum, not a mean).
 * Scores use the similarity kernel's arithmetic (see the top of this file);
 * the log-sum-exp is accumulated online in fp32 with the largest score as its
 * shift, so no exponential overflows for any finite input; the positive score
 * is an fp32 dot product in component order.
 *   a, b     : maps of equal batch, d and dtype; b has at least one row, and
 *              a too when n_gt > 0 (else MR_ERR_SHAPE).  bf16 maps: any supported d; fp32 maps: d in
 *              {8, 16, 24, 32} (else MR_ERR_SHAPE).
 *   gt       : DEVICE int32 [batch][n_gt][2] rows (i in a, j in b) of each
 *              pair; an out-of-range pair is not an error: its term is NaN
 *              (and so is that pair's loss).  0 <= n_gt <= 2^28.
 *   tau      : > 0 and finite (else MR_ERR_PARAM).
 *   out_terms: [batch][n_gt] fp32 (may be NULL only when n_gt = 0).
 *   out_loss : [batch] binary64: per image pair, the terms added in binary64
 *              in a fixed order (deterministic); 0 when n_gt = 0.
 *   ws       : mr_workspace_bytes(MR_OP_INFONCE, a, b, n_gt, 0, 0) bytes
 *              (unused when n_gt = 0).
 * --------------------------------------------------------------------------- */
int mr_infonce_forward(const mr_map* a, const mr_map* b, const int32_t* gt, int64_t n_gt, float tau,
                       float* out_terms, double* out_loss, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * mr_infonce_backward: the matching loss of mr_infonce_forward (same terms and
 * loss outputs) and its gradient with respect to both maps ("MASt3R
 * dissection", section 3 "Napkin Formula": the loss the descriptor head is
 * trained with).  The derivative of each term's log-sum-exp is its softmax
 * p[t][k] over the rows of b, so for image pair b of the batch
 *     grad_a[i] = (1/tau) sum_{t: i_t = i} ( sum_k p[t][k] b[k] - b[j_t] ),
 *     grad_b[k] = (1/tau) sum_t p[t][k] a[i_t] - (1/tau) sum_{t: j_t = k} a[i_t],
 * the gradient of that pair's loss (a sum over its terms); rows of a that no
 * ground-truth pair names get 0.
 *   a, b   : as mr_infonce_forward, with d <= 32 (else MR_ERR_SHAPE): bf16
 *            maps, or fp32 maps with d in {8, 16, 24, 32}.
 *   grad_a : [batch][h_a][w_a][d] fp32 (may be NULL only when a has no rows);
 *   grad_b : [batch][h_b][w_b][d] fp32.
 *   ws     : mr_workspace_bytes(MR_OP_INFONCE_BACKWARD, a, b, n_gt, 0, 0) bytes
 *            (unused when n_gt = 0).
 * The softmax-weighted sums are formed on the matrix cores with each softmax
 * value split into two bf16 parts (relative error below 2^-17), fp32 map rows
 * split exactly into three, and fp32 accumulation; rows that several ground-truth pairs share are accumulated with
 * binary64 atomic adds of fp32 values before the final scaling and rounding, so
 * the result can differ between runs only where such a sum rounds in binary64.
 * A ground-truth pair with an index out of range makes that image pair's loss
 * NaN; its gradient is then unspecified (finite or not), never out of bounds.
 * --------------------------------------------------------------------------- */
int mr_infonce_backward(const mr_map* a, const mr_map* b, const int32_t* gt, int64_t n_gt, float tau,
                        float* out_terms, double* out_loss, float* grad_a, float* grad_b, void* ws,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement aid.  The one piece of state the library keeps between calls, and
 * only on request: a profiling window belongs to the calling thread (one open
 * window per thread).  Entry points called on that thread while its window is
 * open record events into it; calls on any other thread, and calls outside a
 * window, never read or write it, so the entry points stay thread-safe given
 * distinct workspaces.
 * mr_profile_begin(n): from now on, record a pair of hipEvents on the call's
 * stream around every launch of the similarity/argmax kernel (both metrics),
 * of the matching loss's log-sum-exp kernel (mr_infonce_forward) and of the two
 * gradient passes (mr_infonce_backward), for up to n launches.
 * mr_profile_end: wait for those events, return the summed kernel time in
 * milliseconds and the number of launches timed, release the events.
 * mr_profile_end_each: the same, and also each launch's time in milliseconds,
 * in launch order, into each_ms[0 .. min(cap, launches)) (cap >= 0; each_ms may
 * be NULL only when cap = 0).
 * mr_profile_end_queries: the same, and also into each_queries[0 .. min(cap,
 * launches)) the number of queries each search launch ran, summed over the batch
 * (-1 for the loss kernels' launches, which are not counted).  The fast scheme
 * searches the backward NN of a pixel of image 2 once per call, so its backward
 * launches run fewer queries than there are live pixels; these counts give the
 * work each launch did.  Either array may be NULL (not both when cap > 0).
 * All three return MR_ERR_PARAM without an open window.  A window holds
 * max_launches * 8 bytes of device memory (the counts) and its events from
 * mr_profile_begin until it ends; a count is taken by a one-workgroup kernel on the
 * call's stream just before the launch's start event, so it is not timed.
 * --------------------------------------------------------------------------- */
int mr_profile_begin(int32_t max_launches);
int mr_profile_end(double* total_ms, int64_t* launches);
int mr_profile_end_each(double* total_ms, int64_t* launches, float* each_ms, int32_t cap);
int mr_profile_end_queries(double* total_ms, int64_t* launches, float* each_ms, int64_t* each_queries,
                           int32_t cap);

/* ---------------------------------------------------------------------------
 * Launch log (no function): with the environment variable MR_LOG set to anything
 * but "" or "0" when the library first checks it (once per process), every entry
 * point writes to stderr one line on entry (its maps: batch x h x w x d, dtype,
 * address; and its sizes and parameters), one line per kernel launch (kernel,
 * the launching function's template arguments, grid, block, LDS bytes, stream)
 * and one line with the status it returns.  Lines start with "[mr]".  Lines of
 * calls made from several threads may interleave.  Unset, nothing is printed.
 * --------------------------------------------------------------------------- */

#ifdef __cplusplus
}
#endif

#endif /* MR_H */
