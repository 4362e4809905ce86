/*
 * fk.h -- C ABI of an exact Lloyd k-means iteration for AMD MI355X (gfx950).
 *
 * One Lloyd iteration takes points X[N,d] and centroids C[K,d], assigns every
 * point to its nearest centroid under squared L2 distance, then recomputes
 * each centroid as the mean of its points.  The Flash-KMeans article
 * (lumevalley.com, article 3696) describes two kernels for this and insists
 * that the result is the exact standard Lloyd iteration, not an
 * approximation:
 *   - FlashAssign (section "FlashAssign: cutting the distance matrix into a
 *     pipeline"): the N x K distance matrix is never written out; blocks of
 *     points are scored against all centroids on the spot and reduced to an
 *     argmin at once, so the IO falls from O(NK) to O(Nd + Kd);
 *   - Sort-Inverse Update (section "Sort-Inverse Update: another answer to
 *     atomics"): the assignments are sorted by cluster id into an inverse
 *     index, and the per-cluster sums are reduced by reading that index
 *     contiguously, with no global atomic operations (the sort's per-tile
 *     digit counts are LDS atomic adds, where the order does not matter).
 * The article lists squared L2 and cosine as the supported metrics and inner
 * product as the next one (section "Not a silver bullet").  Cosine is L2 on
 * L2-normalised vectors, a zero norm being taken as 1 before the divide
 * (LEANN FlashLib backend guide, mhpn.cn, paragraph "distance metric").
 * Inner product assigns each point to the centroid of largest x.c (lowest
 * index on ties, the dot product taken in fp64 in increasing j where it is
 * settled) and updates with plain means; its min_dist is -max_k x.c.
 * Spherical is the explicit spherical-centroid option beside cosine: points
 * are assigned as for cosine, and every returned centroid (an empty
 * cluster's kept one too) is divided by its L2 norm (fp64, a zero norm taken
 * as 1), so chained iterations are spherical k-means.  The
 * out-of-core entry point follows the article's out-of-core mode, which keeps
 * the data in host memory and computes on the GPU (section "Real-time MoE
 * routing").
 *
 * Conventions for every entry point
 *   - Layout: row-major, fp32 X[N,d] and C[K,d]; int32 labels and counts.
 *   - Ownership: the caller owns every buffer.  Device pointers are HIP device
 *     memory on the current device.  The library allocates no device memory;
 *     the caller passes a workspace of at least fk_workspace_size() bytes,
 *     256-byte aligned, that nothing else uses while the call's work runs.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Work is enqueued asynchronously on it; the caller
 *     synchronises.  fk_lloyd_iter_stream also uses one library-owned copy
 *     stream, joined to `stream` by events.
 *   - Validation: every argument is checked before anything is enqueued; on
 *     an error nothing is written and nothing is enqueued.
 *   - Errors: a status code is returned; fk_status_str() names it and
 *     fk_last_error() gives a message for the calling thread's last failure.
 *     HIP launch or runtime errors map to FK_ERR_HIP.  No C++ exception
 *     crosses the ABI.
 *   - Limits: 0 <= N <= 2^31-1; 1 <= d <= FK_MAX_D; 1 <= K <= FK_MAX_K.
 *     K > N is accepted (some clusters are then empty).
 *   - Exactness: assignments equal the lowest-index argmin of the fp64
 *     direct-difference distance sum_j (x_j - c_j)^2 taken in increasing j:
 *     the MFMA scores (fp32, or split bf16) carry a proven error bound, and
 *     for every point
 *     whose top-2 score gap is within twice that bound, every centroid that
 *     can still win is compared in fp64 by that definition.
 *     Cluster sums are accumulated in fp64.  An empty cluster keeps the
 *     centroid it was given.  Results are bitwise reproducible run to run.
 */
#ifndef FK_H
#define FK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FK_MAX_K 65536
#define FK_MAX_D 4096
#define FK_MAX_KNN_K 24          /* largest k of fk_knn          */
#define FK_MAX_KNN_DB 1073741824 /* most database rows of fk_knn */

typedef enum {
    FK_OK = 0,
    FK_ERR_INVALID_ARG = 1,  /* null pointer, bad size, aliasing, bad layout */
    FK_ERR_UNSUPPORTED = 2,  /* a metric or size the library does not do    */
    FK_ERR_WORKSPACE = 3,    /* workspace missing, short or misaligned       */
    FK_ERR_NO_DEVICE = 4,    /* no HIP device is visible                     */
    FK_ERR_HIP = 5           /* a HIP runtime or launch error                */
} fk_status;

typedef enum {
    FK_METRIC_L2 = 0,            /* squared Euclidean distance                 */
    FK_METRIC_COSINE = 1,        /* L2 on rows normalised to unit length       */
    FK_METRIC_INNER_PRODUCT = 2, /* largest x.c (no normalisation)             */
    FK_METRIC_SPHERICAL = 3      /* cosine assignment, unit-length centroids   */
} fk_metric;

/*
 * How FlashAssign scores x.c before near ties are settled in fp64.  Both give
 * the same (exact) assignment; they differ in speed and in how many points
 * fall inside the error window and go to the fp64 paths.
 *   FK_SCORE_FP32: fp32 MFMA (v_mfma_f32_32x32x2_f32) on the fp32 inputs.
 *   FK_SCORE_SPLIT_BF16: each fp32 value v is split into bf16 parts
 *     hi = bf16(v), lo = bf16(v - hi); x.c is taken as hi.hi + hi.lo + lo.hi
 *     on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.  The
 *     large products are accumulated as in fp32 scoring (the small cross
 *     terms first), so the error bound is the fp32 one plus a per-point bound
 *     on the dropped parts (lo.lo and the bf16 rounding remainders, from the
 *     actual remainder norms): about 1.6 times the fp32 window at d = 128.
 *     About 3 times faster than FK_SCORE_FP32 on MI355X at d = 128.
 */
typedef enum {
    FK_SCORE_FP32 = 0,
    FK_SCORE_SPLIT_BF16 = 1
} fk_score;

/*
 * Bytes of workspace needed by a call with these sizes.  chunk_rows = 0 sizes
 * the in-core calls (fk_assign, fk_sort_inverse, fk_update, fk_lloyd_iter)
 * for N rows; chunk_rows > 0 sizes fk_lloyd_iter_stream with that chunk
 * length (two device chunk buffers of chunk_rows x d floats are included).
 * Returns 0 when the sizes are outside the limits above.
 */
size_t fk_workspace_size(int64_t N, int32_t d, int32_t K, int32_t metric, int64_t chunk_rows);

/*
 * FlashAssign: assign[i] = the nearest centroid of point i (lowest index on
 * ties), and, when min_dist is not NULL, min_dist[i] = its distance by the
 * definition -- sum_j (x_j - c_j)^2 in fp64 by direct differences in
 * increasing j (cosine: of the fp64-normalised rows; inner product: -x.c),
 * rounded once to fp32, so sum_i min_dist[i] is the objective of the
 * iteration's centroids (an extra pass over X that reads each point's row
 * and its centroid's).  score is an
 * fk_score.  X, C, assign and min_dist are device pointers.  The N x K
 * distance matrix is never stored: each workgroup keeps a block of points in
 * registers, streams centroid tiles through LDS into MFMA (fp32, or
 * split-bf16) and keeps a running top-3 per point in registers (FlashAssign
 * section of the Flash-KMeans article).  Near ties are settled in fp64 (see
 * Exactness above).
 */
fk_status fk_assign(const float *X, int64_t N, int32_t d, const float *C, int32_t K, int32_t metric,
                    int32_t score, int32_t *assign, float *min_dist, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * The inverse index of the Sort-Inverse Update: perm[0..N) lists the point
 * ids ordered by cluster id (stable: increasing point id within a cluster),
 * and offsets[0..K] gives the start of each cluster's run in perm, with
 * offsets[K] = N, so cluster k has offsets[k+1] - offsets[k] points.  Built
 * with an LSD radix sort (Sort-Inverse Update section of the Flash-KMeans
 * article) whose ranking is ballot-based and stable; its per-tile digit
 * counts are LDS atomic adds, and no global memory is updated atomically.  Every assign[i] must lie in [0, K); other values
 * give undefined results.  All pointers are device pointers.
 */
fk_status fk_sort_inverse(const int32_t *assign, int64_t N, int32_t K, int32_t *perm, int32_t *offsets,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sort-Inverse Update: counts[k] = #{i : assign[i] = k} and
 * C_out[k] = mean of the points of cluster k (of the normalised points for
 * cosine), accumulated in fp64; a cluster with no point keeps C_prev[k] as
 * passed.  The per-cluster reduction walks the inverse index over
 * equal-length row segments with a deterministic carry fix-up, so it uses no
 * atomics (the sort under it counts digits with LDS atomic adds).  C_out must not overlap C_prev.  All pointers are device
 * pointers; assign[i] must lie in [0, K).
 */
fk_status fk_update(const float *X, int64_t N, int32_t d, const int32_t *assign, int32_t K, int32_t metric,
                    const float *C_prev, float *C_out, int32_t *counts, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * One full Lloyd iteration: fk_assign (with `score`) then fk_update, from C_in
 * to C_out.
 * assign and counts receive the assignment under C_in and the cluster sizes;
 * min_dist may be NULL.  C_out must not overlap C_in.  Device pointers.
 */
fk_status fk_lloyd_iter(const float *X, int64_t N, int32_t d, const float *C_in, int32_t K, int32_t metric,
                        int32_t score, int32_t *assign, float *min_dist, float *C_out, int32_t *counts,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * fk_lloyd_iter for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as fk_lloyd_iter, without the
 * workspace: the call uses a scratch array of FK_NOALLOC_SCRATCH_BYTES that
 * the library holds on every device it runs on until the process ends, and
 * calls no allocating routine (phase timing is skipped).  Sizes whose
 * fk_workspace_size(N, d, K, metric, 0) exceeds FK_NOALLOC_SCRATCH_BYTES are
 * rejected with FK_ERR_WORKSPACE.  Every call on a device shares that
 * device's scratch: calls that overlap on one device (other streams, other
 * host threads) race and must be ordered by the caller.
 */
#define FK_NOALLOC_SCRATCH_BYTES (128u << 20)
fk_status fk_lloyd_iter_noalloc(const float *X, int64_t N, int32_t d, const float *C_in, int32_t K, int32_t metric,
                                int32_t score, int32_t *assign, float *min_dist, float *C_out, int32_t *counts,
                                void *stream);

/*
 * Out-of-core Lloyd iteration: X_host is PINNED host memory (hipHostMalloc
 * or a pinned torch tensor) holding N x d floats; it is copied to the device
 * in chunks of at most chunk_rows rows, double-buffered on a copy stream that
 * overlaps the compute of the previous chunk (the first chunks ramp up, from
 * chunk_rows / 16 doubling to chunk_rows when chunk_rows / 16 exceeds 2^20
 * rows, so that the one copy not hidden behind compute is short).  Each chunk is assigned and
 * reduced into fp64 cluster sums; the means are taken once at the end.  The
 * result equals fk_lloyd_iter on the same data.  C_in, C_out and counts are
 * device pointers; assign_host, when not NULL, is pinned host memory of N
 * int32 that receives the assignment.  The call returns once every chunk is
 * enqueued; the caller synchronises `stream`.  X_host must not be modified
 * until then.  Calls on one device share the library's copy stream: calls
 * from several host threads are enqueued one at a time (each with its own
 * workspace).  Returns FK_ERR_INVALID_ARG when X_host or assign_host is not
 * pinned.
 */
fk_status fk_lloyd_iter_stream(const float *X_host, int64_t N, int32_t d, const float *C_in, int32_t K,
                               int32_t metric, int32_t score, int64_t chunk_rows, int32_t *assign_host,
                               float *C_out, int32_t *counts, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Lloyd k-means: up to n_iter >= 1 iterations of fk_lloyd_iter (the plain
 * iteration of the Flash-KMeans article, repeated; the LEANN FlashLib guide,
 * paragraph "parameters", trains its IVF quantizer with niter = 20 such
 * iterations and a seed).
 *   Start: from C_init[K, d] (device) when it is not NULL (K > N is then
 *   accepted: some clusters stay empty).  With C_init NULL the guide's
 *   clamp K' = min(K, N) applies (paragraph "nlist and nprobe"), N >= 1, and
 *   the initial centroids are K' rows of X drawn with `seed`: the first K'
 *   positions of a Fisher-Yates shuffle of 0..N-1 (step i swaps position i
 *   with position i + r, r uniform in [0, N - i)), r taken from SplitMix64
 *   (Steele, Lea and Flood 2014; state += 0x9E3779B97F4A7C15, output mixed
 *   with shifts 30/27/31 and multipliers 0xBF58476D1CE4E5B9,
 *   0x94D049BB133111EB) by rejecting draws at or above the largest multiple
 *   of N - i below 2^64 and reducing the rest modulo N - i.
 *   Stop: tol < 0 runs exactly n_iter iterations and the call only enqueues
 *   work.  tol >= 0 also stops after the first iteration whose largest
 *   squared centroid move, sum_j (c_new - c_old)^2 in fp64 over the fp32
 *   centroids, is at most tol (tol = 0: a fixed point, after which further
 *   iterations would change nothing); the call then waits for `stream` after
 *   every iteration.
 * C_out[0..K') receives the centroids after the last iteration, assign the
 * last iteration's assignment (under the centroids before it) and
 * counts[0..K') its cluster sizes.  info (host memory, may be NULL) receives
 * K', the iterations run and the last measured move (-1 when tol < 0).
 * Workspace: fk_fit_workspace_size() bytes.  C_out must not overlap C_init.
 * Device pointers except info; errors as fk_lloyd_iter, plus
 * FK_ERR_INVALID_ARG for n_iter < 1 or a draw from N = 0 rows.
 */
typedef struct {
    int32_t k_used;      /* clusters fitted: K, or min(K, N) when rows were drawn */
    int32_t iterations;  /* iterations run                                      */
    double last_shift;   /* largest squared centroid move of the last one (-1
                            when tol < 0: not measured)                         */
} fk_fit_info;
size_t fk_fit_workspace_size(int64_t N, int32_t d, int32_t K, int32_t metric);
fk_status fk_fit(const float *X, int64_t N, int32_t d, int32_t K, int32_t metric, int32_t score, const float *C_init,
                 uint64_t seed, int32_t n_iter, double tol, float *C_out, int32_t *assign, int32_t *counts,
                 fk_fit_info *info, void *workspace, size_t workspace_bytes, void *stream);

/*
 * IVF-Flat index build (LEANN FlashLib guide, paragraphs "how it works",
 * "parameters", "nlist and nprobe"): nl = min(nlist, N) cells (the guide's
 * clamp); a coarse quantizer of nl centroids trained by n_iter Lloyd
 * iterations from the rows init_idx_host[0..nl) of X, or, when
 * init_idx_host is NULL, from nl rows drawn with `seed` as fk_fit draws
 * them; then every row assigned to its nearest final centroid and the rows
 * grouped by cell:
 *   centroids[nl, d]         the quantizer (fp32),
 *   list_offsets[nl + 1]     CSR offsets: cell k holds list positions
 *                            [list_offsets[k], list_offsets[k+1]),
 *   list_ids[N]              the row of X at each list position (increasing
 *                            within a cell),
 *   list_data[N, d]          those rows, cell-contiguous.
 * Buffers sized for nlist rows are large enough.  metric COSINE
 * L2-normalises the rows first (zero norm taken as 1), trains plain L2
 * k-means on them and stores the normalised rows; L2 uses X as is; inner
 * product and spherical give FK_ERR_UNSUPPORTED.  Requires N >= 1.
 * init_idx_host (nl int32 row indices, each checked to lie in [0, N)) and
 * nlist_used (receives nl; may be NULL) are HOST memory; every other pointer
 * is device memory.  Workspace: fk_ivf_workspace_size() bytes.  list_data
 * must not overlap X.  The assignments are exact in the sense of fk_assign.
 */
size_t fk_ivf_workspace_size(int64_t N, int32_t d, int32_t nlist, int32_t metric);
fk_status fk_ivf_build(const float *X, int64_t N, int32_t d, int32_t nlist, int32_t metric, int32_t score,
                       int32_t n_iter, const int32_t *init_idx_host, uint64_t seed, float *centroids,
                       int32_t *list_offsets, int32_t *list_ids, float *list_data, int32_t *nlist_used,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Exact k nearest neighbours by brute force (flash-knn, the exact GPU k-NN
 * backend of the LEANN FlashLib guide, paragraph "when to use FlashLib"):
 * for each query q of Q[M,d], idx[q, 0..k) are the k database rows of DB[Ndb,d]
 * with the smallest fp64 distances, in increasing (distance, row index)
 * order, and dist[q, j] is that distance rounded to fp32:
 *   L2      sum_j (q_j - x_j)^2 (direct differences, increasing j),
 *   COSINE  the same on both rows L2-normalised (zero norm taken as 1),
 *   INNER_PRODUCT  -sum_j q_j x_j (largest inner product first).
 * The FlashAssign sweep runs with the queries as points and the database
 * rows as centroids, and keeps for every query its L best MFMA scores
 * (L = 16 for k <= 12, else 32) instead of the top 3.  The exact top k lies
 * among those L whenever the k-th score beats the L-th by more than twice the
 * score error bound (as for fk_assign); the L candidates are then ranked in
 * fp64.  The other queries are ranked against every database row in fp64.
 * The backend clamps k to the database size: with k > Ndb, idx[q, Ndb..k)
 * = -1 and dist[q, Ndb..k) = +inf.  Limits: 0 <= M <= 2^31-1,
 * 1 <= Ndb <= FK_MAX_KNN_DB, k >= 1 and min(k, Ndb) <= FK_MAX_KNN_K; metric
 * L2, COSINE or INNER_PRODUCT (SPHERICAL, a centroid option, gives
 * FK_ERR_UNSUPPORTED); FK_SCORE_SPLIT_BF16 also needs the database's bf16
 * copy (about 4 Ndb d bytes: Ndb rounded up to 256, d up to 16, 32, 64, 128
 * or a multiple of 64) under 4 GiB, else FK_ERR_UNSUPPORTED.  Q, DB,
 * idx[M,k] (int32) and dist[M,k] (fp32) are device pointers; workspace:
 * fk_knn_workspace_size() bytes.
 */
size_t fk_knn_workspace_size(int64_t M, int32_t d, int64_t Ndb, int32_t k, int32_t metric);
fk_status fk_knn(const float *Q, int64_t M, int32_t d, const float *DB, int64_t Ndb, int32_t k, int32_t metric,
                 int32_t score, int32_t *idx, float *dist, void *workspace, size_t workspace_bytes, void *stream);

/* Static name of a status code. */
const char *fk_status_str(int32_t status);

/* Message describing the calling thread's last failed call ("" if none). */
const char *fk_last_error(void);

/*
 * Phase timing.  While enabled, every phase the library enqueues is bracketed
 * by HIP events on the stream it runs on; fk_profile_read() waits for them,
 * adds their durations into `out` and resets the pending list.  The
 * accumulated totals are reset by fk_profile_enable(1).  Timing adds two event
 * records per phase and is off by default.
 */
enum {
    FK_PH_PREP = 0,      /* centroid norms (and cosine normalisation)       */
    FK_PH_ASSIGN = 1,    /* the FlashAssign kernel                          */
    FK_PH_RECHECK = 2,   /* fp64 rescoring of near-tie points (and the
                            exact min_dist pass when it is asked for)       */
    FK_PH_SORT = 3,      /* radix sort (the inverse index)                  */
    FK_PH_REDUCE = 4,    /* segmented reduction (with the cluster offsets;
                            rows in one batch: also the divide by count of
                            the clusters inside a segment; rows in several
                            batches: also the carry fix-up)                 */
    FK_PH_FINALIZE = 5,  /* rows in one batch: carry fix-up, counts, empty
                            centroids kept; in several batches: the divide  */
    FK_PH_H2D = 6,       /* host-to-device chunk copies (out-of-core)       */
    FK_NPHASE = 7
};

typedef struct {
    int64_t calls[FK_NPHASE];
    double ms[FK_NPHASE];
    int64_t rechecked;      /* near-tie points rescored in fp64 against all K      */
    int64_t paired;         /* near-tie points settled by an fp64 two-way compare  */
    int64_t windowed;       /* near-tie points settled by an fp64 compare of the
                               centroids collected within their error window     */
    int64_t assigned;       /* points assigned, summed over the calls read         */
} fk_profile;

fk_status fk_profile_enable(int32_t on);
fk_status fk_profile_read(fk_profile *out);

#ifdef __cplusplus
}
#endif

#endif /* FK_H */
