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
 *     contiguously, with no atomic operations.
 * The article lists squared L2 and cosine as the supported metrics and inner
 * product as the next one (section "Not a silver bullet").  Cosine is L2 on
 * L2-normalised vectors, a zero norm being taken as 1 before the divide
 * (LEANN FlashLib backend guide, mhpn.cn, paragraph "distance metric").
 * Inner product assigns each point to the centroid of largest x.c (lowest
 * index on ties, the dot product taken in fp64 in increasing j where it is
 * settled) and updates with plain means; its min_dist is -max_k x.c.  The
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
    FK_METRIC_INNER_PRODUCT = 2  /* largest x.c (no normalisation)             */
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
 * ties), and, when min_dist is not NULL, min_dist[i] = its squared distance
 * (fp32; the fp64 value rounded for rescored points).  score is an
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
 * with an atomic-free LSD radix sort (Sort-Inverse Update section of the
 * Flash-KMeans article).  Every assign[i] must lie in [0, K); other values
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
 * atomics.  C_out must not overlap C_prev.  All pointers are device
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
 * in chunks of chunk_rows rows, double-buffered on a copy stream that
 * overlaps the compute of the previous chunk.  Each chunk is assigned and
 * reduced into fp64 cluster sums; the means are taken once at the end.  The
 * result equals fk_lloyd_iter on the same data.  C_in, C_out and counts are
 * device pointers; assign_host, when not NULL, is pinned host memory of N
 * int32 that receives the assignment.  The call returns once every chunk is
 * enqueued; the caller synchronises `stream`.  X_host must not be modified
 * until then.  Returns FK_ERR_INVALID_ARG when X_host or assign_host is not
 * pinned.
 */
fk_status fk_lloyd_iter_stream(const float *X_host, int64_t N, int32_t d, const float *C_in, int32_t K,
                               int32_t metric, int32_t score, int64_t chunk_rows, int32_t *assign_host,
                               float *C_out, int32_t *counts, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * Lloyd k-means: n_iter >= 1 iterations of fk_lloyd_iter starting from
 * C_init (the plain iteration of the Flash-KMeans article, repeated; the
 * LEANN FlashLib guide, paragraph "parameters", trains its IVF quantizer with
 * niter = 20 such iterations).  C_out receives the centroids after the last
 * iteration, assign the last iteration's assignment (under the centroids
 * before it) and counts its cluster sizes.  Workspace:
 * fk_fit_workspace_size() bytes (it also holds the intermediate centroids).
 * C_out must not overlap C_init.  Device pointers; errors as fk_lloyd_iter,
 * plus FK_ERR_INVALID_ARG for n_iter < 1.
 */
size_t fk_fit_workspace_size(int64_t N, int32_t d, int32_t K, int32_t metric);
fk_status fk_fit(const float *X, int64_t N, int32_t d, const float *C_init, int32_t K, int32_t metric, int32_t score,
                 int32_t n_iter, float *C_out, int32_t *assign, int32_t *counts, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * IVF-Flat index build (LEANN FlashLib guide, paragraphs "how it works",
 * "parameters"): a coarse quantizer of nlist centroids trained by n_iter
 * Lloyd iterations from the rows init_idx_host[0..nlist) of X, then every row
 * assigned to its nearest final centroid and the rows grouped by cell:
 *   centroids[nlist, d]      the quantizer (fp32),
 *   list_offsets[nlist + 1]  CSR offsets: cell k holds list positions
 *                            [list_offsets[k], list_offsets[k+1]),
 *   list_ids[N]              the row of X at each list position (increasing
 *                            within a cell),
 *   list_data[N, d]          those rows, cell-contiguous.
 * metric COSINE L2-normalises the rows first (zero norm taken as 1), trains
 * plain L2 k-means on them and stores the normalised rows; L2 uses X as is.
 * Requires 1 <= nlist <= N (the guide clamps nlist to N; the Python binding
 * does that).  init_idx_host is HOST memory (nlist int32 row indices, each
 * checked to lie in [0, N)); every other pointer is device memory.  Workspace:
 * fk_ivf_workspace_size() bytes.  list_data must not overlap X.  The
 * assignments are exact in the sense of fk_assign.
 */
size_t fk_ivf_workspace_size(int64_t N, int32_t d, int32_t nlist, int32_t metric);
fk_status fk_ivf_build(const float *X, int64_t N, int32_t d, int32_t nlist, int32_t metric, int32_t score,
                       int32_t n_iter, const int32_t *init_idx_host, float *centroids, int32_t *list_offsets,
                       int32_t *list_ids, float *list_data, void *workspace, size_t workspace_bytes, void *stream);

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
 * Limits: 0 <= M <= 2^31-1, 1 <= Ndb <= FK_MAX_KNN_DB,
 * 1 <= k <= min(FK_MAX_KNN_K, Ndb); FK_SCORE_SPLIT_BF16 also needs the
 * database's bf16 copy (about 4 Ndb d bytes: Ndb rounded up to 128, d up to
 * 16, 32, 64, 128 or a multiple of 64) under 4 GiB, else FK_ERR_UNSUPPORTED.
 * Q, DB, idx[M,k] (int32) and dist[M,k] (fp32) are device pointers; workspace:
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
    FK_PH_RECHECK = 2,   /* fp64 rescoring of near-tie points               */
    FK_PH_SORT = 3,      /* radix sort (the inverse index)                  */
    FK_PH_REDUCE = 4,    /* segmented reduction + carry fix-up (with the
                            cluster offsets; rows in one batch: also the
                            divide by count)                                */
    FK_PH_FINALIZE = 5,  /* counts, empty centroids kept (and the divide
                            when rows came in several batches)              */
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
