// Host side of libfk: argument validation, workspace carving, phase
// sequencing on the caller's stream, the out-of-core chunk pipeline, and
// phase timing.  Declared in include/fk.h.
#include <cmath>
#include <mutex>
#include <stdarg.h>
#include <unordered_map>
#include <stdio.h>
#include <string.h>
#include <vector>

#include "fk.h"
#include "fk_internal.h"

using namespace fk;

namespace {

thread_local char g_err[512] = "";

fk_status fail(fk_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

fk_status hip_fail(hipError_t e, const char *what) {
    (void)hipGetLastError();
    return fail(FK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define FK_TRY(expr, what)                                  \
    do {                                                    \
        hipError_t e_ = (expr);                             \
        if (e_ != hipSuccess) return hip_fail(e_, (what));  \
    } while (0)

// Cosine and spherical normalise the rows they compare; spherical also
// returns unit-length centroids.
bool normalises(int metric) { return metric == FK_METRIC_COSINE || metric == FK_METRIC_SPHERICAL; }

// ---- workspace layout -----------------------------------------------------
struct Layout {
    size_t total = 0;
    size_t ncn, cmax_part, scal, counter, flags, thr, pairs, cand, ccount, ovf;
    size_t c64, c32, cnrm64, xnorm64;  // cosine only (else ~0)
    size_t keys_sorted, perm, tmp_keys, tmp_vals, sort_scratch, offsets;
    size_t sums, cnt, pfirst, plast, csplit;
    size_t xchunk[2], achunk[2];      // out-of-core only
    size_t ctmp, cinit, init_idx, labels, xcopy;  // fit / IVF build only
    size_t shift_part, shift;                     // fit only (the stopping test)
    size_t knn_cand, knn_score, knn_win, knn_list, knn_tau;  // k nearest neighbours only
};

constexpr size_t kNone = ~(size_t)0;

// extras: kFitExtras adds a second centroid buffer (the fit's ping-pong),
// the drawn initial rows and the stopping test's partial maxima; kIvfExtras
// adds the initial centroids, the list labels and, for cosine, a normalised
// copy of X.
constexpr int kFitExtras = 1, kIvfExtras = 2;

Layout make_layout(int64_t rows, int d, int K, int metric, bool ooc, int extras = 0) {
    Layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    const int64_t r = rows > 0 ? rows : 1;
    const int64_t Kpad = cdiv(K, kCentroidPad) * kCentroidPad;
    const int64_t nseg = seg_count_bound(r);
    const bool cos = normalises(metric);
    L.ncn = take((size_t)Kpad * 4);
    L.cmax_part = take((size_t)cdiv(Kpad, 4) * 3 * 4);
    L.scal = take(64);
    L.counter = take(64);
    L.flags = take((size_t)r * 4);
    L.thr = take((size_t)r * 4);
    L.pairs = take((size_t)r * 12);
    L.cand = take((size_t)near_tie_cap(r) * kCandPerSlot * 4);
    L.ccount = take((size_t)near_tie_cap(r) * 2 * 4);
    L.ovf = take((size_t)r * 4);
    L.c64 = cos ? take((size_t)K * d * 8) : kNone;
    L.c32 = cos ? take((size_t)K * d * 4) : kNone;
    L.cnrm64 = cos ? take((size_t)K * 8) : kNone;
    L.xnorm64 = cos ? take((size_t)r * 8) : kNone;
    L.keys_sorted = take((size_t)r * 4);
    L.perm = take((size_t)r * 4);
    L.tmp_keys = take((size_t)r * 4);
    L.tmp_vals = take((size_t)r * 4);
    L.sort_scratch = take(sort_scratch_bytes(r));
    L.offsets = take((size_t)(K + 1) * 4);
    L.csplit = take((size_t)Kpad * 2 * split_width(d) * 2);
    L.sums = take((size_t)K * d * 8);
    L.cnt = take((size_t)K * 4);
    L.pfirst = take((size_t)nseg * d * 8);
    L.plast = take((size_t)nseg * d * 8);
    for (int i = 0; i < 2; ++i) {
        L.xchunk[i] = ooc ? take((size_t)r * d * 4) : kNone;
        L.achunk[i] = ooc ? take((size_t)r * 4) : kNone;
    }
    const bool fit = (extras & (kFitExtras | kIvfExtras)) != 0, ivf = (extras & kIvfExtras) != 0;
    L.ctmp = fit ? take((size_t)K * d * 4) : kNone;
    L.cinit = fit ? take((size_t)K * d * 4) : kNone;
    L.init_idx = fit ? take((size_t)K * 4) : kNone;
    L.shift_part = (extras & kFitExtras) ? take((size_t)cdiv(K, 4) * 8) : kNone;
    L.shift = (extras & kFitExtras) ? take(64) : kNone;
    L.labels = ivf ? take((size_t)r * 4) : kNone;
    L.xcopy = (ivf && cos) ? take((size_t)r * d * 4) : kNone;
    L.knn_cand = L.knn_score = L.knn_win = L.knn_list = L.knn_tau = kNone;
    L.total = off;
    return L;
}

// k nearest neighbours of M queries among Ndb database rows: the database
// takes the centroids' buffers (norms, split copy, cosine copies), the queries
// the points' (norms), plus L candidates and a list slot per query.
Layout make_knn_layout(int64_t M, int d, int64_t Ndb, int k, int metric) {
    Layout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(bytes > 0 ? bytes : 1, 256);
        return o;
    };
    const int64_t m = M > 0 ? M : 1;
    const int64_t Kpad = cdiv(Ndb, kCentroidPad) * kCentroidPad;
    const bool cos = normalises(metric);
    L.ncn = take((size_t)Kpad * 4);
    L.cmax_part = take((size_t)cdiv(Kpad, 4) * 3 * 4);
    L.scal = take(64);
    L.counter = take(64);
    L.c64 = cos ? take((size_t)Ndb * d * 8) : kNone;
    L.c32 = cos ? take((size_t)Ndb * d * 4) : kNone;
    L.cnrm64 = cos ? take((size_t)Ndb * 8) : kNone;
    L.xnorm64 = cos ? take((size_t)m * 8) : kNone;
    L.csplit = take((size_t)Kpad * 2 * split_width(d) * 2);
    const size_t ncand = (size_t)m * knn_slices(m, Ndb).slices * knn_list_len(k);
    L.knn_cand = take(ncand * 4);
    L.knn_score = take(ncand * 4);
    L.knn_win = take((size_t)m * 4);
    L.knn_list = take((size_t)m * 4);
    L.knn_tau = take((size_t)m * 4);
    L.flags = L.thr = L.pairs = L.cand = L.ccount = L.ovf = kNone;
    L.keys_sorted = L.perm = L.tmp_keys = L.tmp_vals = L.sort_scratch = L.offsets = kNone;
    L.sums = L.cnt = L.pfirst = L.plast = kNone;
    L.xchunk[0] = L.xchunk[1] = L.achunk[0] = L.achunk[1] = kNone;
    L.ctmp = L.cinit = L.init_idx = L.labels = L.xcopy = L.shift_part = L.shift = kNone;
    L.total = off;
    return L;
}

template <typename T>
T *at(void *ws, size_t off) {
    return off == kNone ? nullptr : reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

// ---- validation -----------------------------------------------------------
fk_status check_sizes(int64_t N, int64_t d, int64_t K) {
    if (N < 0 || N > INT32_MAX) return fail(FK_ERR_INVALID_ARG, "N=%lld outside [0, 2^31-1]", (long long)N);
    if (d < 1 || d > FK_MAX_D) return fail(FK_ERR_INVALID_ARG, "d=%lld outside [1, %d]", (long long)d, FK_MAX_D);
    if (K < 1 || K > FK_MAX_K) return fail(FK_ERR_INVALID_ARG, "K=%lld outside [1, %d]", (long long)K, FK_MAX_K);
    return FK_OK;
}

fk_status check_score(int32_t score) {
    if (score != FK_SCORE_FP32 && score != FK_SCORE_SPLIT_BF16)
        return fail(FK_ERR_INVALID_ARG, "unknown score mode %d", (int)score);
    return FK_OK;
}

bool known_metric(int32_t metric) {
    return metric == FK_METRIC_L2 || metric == FK_METRIC_COSINE || metric == FK_METRIC_INNER_PRODUCT ||
           metric == FK_METRIC_SPHERICAL;
}

fk_status check_metric(int32_t metric) {
    if (!known_metric(metric)) return fail(FK_ERR_INVALID_ARG, "unknown metric %d", (int)metric);
    return FK_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void *a, size_t an, const void *b, size_t bn) {
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + bn && pb < pa + an;
}

fk_status check_workspace(void *ws, size_t ws_bytes, size_t need) {
    if (ws == nullptr) return fail(FK_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (!aligned(ws, 256)) return fail(FK_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need) return fail(FK_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    return FK_OK;
}

fk_status check_device() {
    int n = 0;
    const hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return fail(FK_ERR_NO_DEVICE, "no HIP device is visible");
    }
    return FK_OK;
}

// ---- phase timing -----------------------------------------------------------
struct Pending {
    int phase;
    hipEvent_t a, b;
};

struct Prof {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> pool;
    std::vector<Pending> pending;
    std::vector<int32_t *> count_slots;  // pinned host slots receiving near-tie counts
    size_t slots_used = 0;
    fk_profile acc{};
};
Prof g_prof;

// Set for the duration of an fk_lloyd_iter_noalloc call on this thread: phase
// timing is skipped there, since it creates events and pinned count slots.
thread_local bool t_no_alloc = false;

hipEvent_t prof_event() {
    if (!g_prof.pool.empty()) {
        hipEvent_t e = g_prof.pool.back();
        g_prof.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

struct PhaseScope {
    int phase;
    hipStream_t s;
    hipEvent_t a = nullptr, b = nullptr;
    PhaseScope(int ph, hipStream_t st) : phase(ph), s(st) {
        if (t_no_alloc) return;
        std::lock_guard<std::mutex> g(g_prof.mu);
        if (!g_prof.on) return;
        a = prof_event();
        b = prof_event();
        if (a && b) (void)hipEventRecord(a, s);
    }
    ~PhaseScope() {
        if (!a || !b) return;
        std::lock_guard<std::mutex> g(g_prof.mu);
        (void)hipEventRecord(b, s);
        g_prof.pending.push_back({phase, a, b});
    }
};

void prof_count_rechecks(const int32_t *dev_counters, int64_t n_assigned, hipStream_t s) {
    if (t_no_alloc) return;
    std::lock_guard<std::mutex> g(g_prof.mu);
    if (!g_prof.on) return;
    if (g_prof.slots_used == g_prof.count_slots.size()) {
        int32_t *h = nullptr;
        if (hipHostMalloc((void **)&h, 3 * sizeof(int32_t)) != hipSuccess) return;
        g_prof.count_slots.push_back(h);
    }
    int32_t *slot = g_prof.count_slots[g_prof.slots_used++];
    slot[0] = slot[1] = slot[2] = 0;
    (void)hipMemcpyAsync(slot, dev_counters, 3 * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    g_prof.acc.assigned += n_assigned;
}

// ---- the steps --------------------------------------------------------------
struct Ctx {
    const Layout &L;
    void *ws;
    hipStream_t s;
    int d, K, metric;
    int score;
    SplitC split() const {
        if (score != FK_SCORE_SPLIT_BF16) return SplitC{nullptr, 0};
        return SplitC{at<__bf16>(ws, L.csplit), split_width(d)};
    }
};

// Centroid norms (and, for cosine, the normalised centroids).  Returns the
// centroid array the MFMA kernel reads.
fk_status step_prep(const Ctx &c, const float *C, const float **C_use) {
    PhaseScope ph(FK_PH_PREP, c.s);
    const float *Cu = C;
    if (normalises(c.metric)) {
        FK_TRY(launch_row_norm64(C, c.K, c.d, at<double>(c.ws, c.L.cnrm64), c.s), "centroid norms");
        FK_TRY(launch_normalize_rows(C, c.K, c.d, at<double>(c.ws, c.L.cnrm64), at<double>(c.ws, c.L.c64),
                                     at<float>(c.ws, c.L.c32), c.s),
               "centroid normalisation");
        Cu = at<float>(c.ws, c.L.c32);
    }
    int nparts = 0;
    FK_TRY(launch_centroid_prep(Cu, c.K, c.d, at<float>(c.ws, c.L.ncn), at<float>(c.ws, c.L.cmax_part), &nparts,
                                c.split(), c.metric == FK_METRIC_INNER_PRODUCT, c.s),
           "centroid prep");
    FK_TRY(launch_prep_finish(at<float>(c.ws, c.L.cmax_part), nparts, at<float>(c.ws, c.L.scal),
                              at<int32_t>(c.ws, c.L.counter), c.s),
           "centroid prep finish");
    *C_use = Cu;
    return FK_OK;
}

fk_status step_xnorm(const Ctx &c, const float *X, int64_t rows) {
    if (!normalises(c.metric)) return FK_OK;
    PhaseScope ph(FK_PH_PREP, c.s);
    FK_TRY(launch_row_norm64(X, rows, c.d, at<double>(c.ws, c.L.xnorm64), c.s), "point norms");
    return FK_OK;
}

// FlashAssign + fp64 recheck of the listed near-tie points.  Needs step_prep
// (and step_xnorm for cosine) first; resets nothing itself except that
// step_prep zeroed the near-tie counter.
fk_status step_assign(const Ctx &c, const float *X, int64_t rows, const float *C, const float *C_use,
                      int32_t *a_out, float *d1_out) {
    const double *xn = normalises(c.metric) ? at<double>(c.ws, c.L.xnorm64) : nullptr;
    NearTies nt;
    nt.full_list = at<int32_t>(c.ws, c.L.flags);
    nt.full_thr = at<float>(c.ws, c.L.thr);
    nt.pair_list = at<int32_t>(c.ws, c.L.pairs);
    nt.counters = at<int32_t>(c.ws, c.L.counter);
    nt.cand = at<int32_t>(c.ws, c.L.cand);
    nt.ccount = at<int32_t>(c.ws, c.L.ccount);
    nt.ovf_list = at<int32_t>(c.ws, c.L.ovf);
    // the assignment kernels write no distances: min_dist is taken at the
    // end, exactly, from the final labels
    {
        PhaseScope ph(FK_PH_ASSIGN, c.s);
        FK_TRY(launch_flash_assign(X, rows, c.d, C_use, at<float>(c.ws, c.L.ncn), c.K, at<float>(c.ws, c.L.scal), xn,
                                   a_out, nt, c.split(), c.metric == FK_METRIC_INNER_PRODUCT, c.s),
               "flash assign");
    }
    {
        PhaseScope ph(FK_PH_RECHECK, c.s);
        const double *c64 = normalises(c.metric) ? at<double>(c.ws, c.L.c64) : nullptr;
        FK_TRY(launch_recheck(X, rows, c.d, C_use, C, c64, at<float>(c.ws, c.L.ncn), c.K, at<float>(c.ws, c.L.scal),
                              xn, nt, c.split(), c.metric == FK_METRIC_INNER_PRODUCT, a_out, c.s),
               "near-tie recheck");
        if (d1_out != nullptr)
            FK_TRY(launch_exact_d1(X, rows, c.d, C, c64, xn, a_out, d1_out, c.metric == FK_METRIC_INNER_PRODUCT, c.s),
                   "exact distances");
    }
    prof_count_rechecks(at<int32_t>(c.ws, c.L.counter), rows, c.s);
    return FK_OK;
}

// Inverse index of `a` into the workspace (keys_sorted, perm, offsets), or
// into caller arrays when given.  with_offsets = false leaves the offsets to
// the segmented reduction, which meets every key change anyway.
fk_status step_sort(const Ctx &c, const int32_t *a, int64_t rows, int32_t *perm_out, int32_t *offsets_out,
                    bool with_offsets = true) {
    PhaseScope ph(FK_PH_SORT, c.s);
    int32_t *perm = perm_out ? perm_out : at<int32_t>(c.ws, c.L.perm);
    int32_t *offs = offsets_out ? offsets_out : at<int32_t>(c.ws, c.L.offsets);
    FK_TRY(launch_sort_by_key(a, rows, c.K, at<int32_t>(c.ws, c.L.keys_sorted), perm,
                              at<int32_t>(c.ws, c.L.tmp_keys), at<int32_t>(c.ws, c.L.tmp_vals),
                              at<void>(c.ws, c.L.sort_scratch), c.s),
           "radix sort");
    if (with_offsets)
        FK_TRY(launch_offsets(at<int32_t>(c.ws, c.L.keys_sorted), rows, c.K, offs, c.s), "cluster offsets");
    return FK_OK;
}

// Accumulators for rows fed in several batches start at zero.  A single batch
// writes the centroids and counts directly, so only an empty one (finalized
// from zero counts) needs them.
fk_status step_zero_accumulators(const Ctx &c, bool batches, int64_t rows) {
    PhaseScope ph(FK_PH_REDUCE, c.s);
    if (batches) FK_TRY(launch_fill_zero(at<void>(c.ws, c.L.sums), (size_t)c.K * c.d * 8, c.s), "zero sums");
    if (batches || rows <= 0) FK_TRY(launch_fill_zero(at<void>(c.ws, c.L.cnt), (size_t)c.K * 4, c.s), "zero counts");
    return FK_OK;
}

// Sort-Inverse reduction of `rows` rows.  batches: added into the fp64 sums
// and counts, which step_finalize divides once every batch is in.  Otherwise
// the rows are all of them (rows > 0) and the new centroids and counts go
// straight to C_out and counts (C_prev for an empty cluster).
fk_status step_accumulate(const Ctx &c, const float *X, int64_t rows, const int32_t *a, bool batches,
                          const float *C_prev = nullptr, float *C_out = nullptr, int32_t *counts = nullptr) {
    if (rows <= 0) return FK_OK;
    fk_status st = step_sort(c, a, rows, nullptr, nullptr, false);
    if (st != FK_OK) return st;
    int32_t *offs = at<int32_t>(c.ws, c.L.offsets);
    {
        PhaseScope ph(FK_PH_REDUCE, c.s);
        const double *xn = normalises(c.metric) ? at<double>(c.ws, c.L.xnorm64) : nullptr;
        FK_TRY(launch_seg_reduce(X, rows, c.d, c.K, at<int32_t>(c.ws, c.L.keys_sorted), at<int32_t>(c.ws, c.L.perm),
                                 xn, at<double>(c.ws, c.L.sums), at<double>(c.ws, c.L.pfirst),
                                 at<double>(c.ws, c.L.plast), batches, offs, C_out, c.s),
               "segmented reduction");
        if (batches) {
            FK_TRY(launch_seg_fixup(at<int32_t>(c.ws, c.L.keys_sorted), offs, rows, c.d, c.K,
                                    at<double>(c.ws, c.L.pfirst), at<double>(c.ws, c.L.plast),
                                    at<double>(c.ws, c.L.sums), true, nullptr, c.s),
                   "segment fix-up");
            FK_TRY(launch_count_accumulate(offs, c.K, at<int32_t>(c.ws, c.L.cnt), true, c.s), "count accumulate");
        }
    }
    if (!batches) {
        PhaseScope ph(FK_PH_FINALIZE, c.s);
        FK_TRY(launch_seg_finish(at<int32_t>(c.ws, c.L.keys_sorted), offs, rows, c.d, c.K, at<double>(c.ws, c.L.pfirst),
                                 at<double>(c.ws, c.L.plast), C_prev, C_out, counts, c.s),
               "segment fix-up and counts");
        if (c.metric == FK_METRIC_SPHERICAL) FK_TRY(launch_unit_rows(C_out, c.K, c.d, c.s), "unit centroids");
    }
    return FK_OK;
}

// Centroids from the accumulated sums and counts (C_prev for an empty cluster)
fk_status step_finalize(const Ctx &c, const float *C_prev, float *C_out, int32_t *counts) {
    PhaseScope ph(FK_PH_FINALIZE, c.s);
    FK_TRY(launch_finalize(at<double>(c.ws, c.L.sums), at<int32_t>(c.ws, c.L.cnt), C_prev, c.K, c.d, C_out, counts,
                           c.s),
           "finalize");
    if (c.metric == FK_METRIC_SPHERICAL) FK_TRY(launch_unit_rows(C_out, c.K, c.d, c.s), "unit centroids");
    return FK_OK;
}

fk_status check_common(const float *X, int64_t N, int32_t d, const void *C, int32_t K, int32_t metric) {
    fk_status st = check_sizes(N, d, K);
    if (st != FK_OK) return st;
    if ((st = check_metric(metric)) != FK_OK) return st;
    if (N > 0 && X == nullptr) return fail(FK_ERR_INVALID_ARG, "X is NULL");
    if (C == nullptr) return fail(FK_ERR_INVALID_ARG, "centroid array is NULL");
    if (X != nullptr && !aligned(X, 16)) return fail(FK_ERR_INVALID_ARG, "X must be 16-byte aligned");
    if (!aligned(C, 16)) return fail(FK_ERR_INVALID_ARG, "centroids must be 16-byte aligned");
    return FK_OK;
}

// One Lloyd iteration on validated arguments (the body of fk_lloyd_iter).
fk_status lloyd_step(const Ctx &c, const float *X, int64_t N, const float *C_in, int32_t *assign, float *min_dist,
                     float *C_out, int32_t *counts) {
    fk_status st;
    if ((st = step_zero_accumulators(c, false, N)) != FK_OK) return st;
    if (N > 0) {
        const float *Cu = nullptr;
        if ((st = step_prep(c, C_in, &Cu)) != FK_OK) return st;
        if ((st = step_xnorm(c, X, N)) != FK_OK) return st;
        if ((st = step_assign(c, X, N, C_in, Cu, assign, min_dist)) != FK_OK) return st;
        return step_accumulate(c, X, N, assign, false, C_in, C_out, counts);
    }
    return step_finalize(c, C_in, C_out, counts);
}

// n_iter Lloyd iterations from C_init; the centroid buffers alternate between
// C_out and the workspace so that the last iteration writes C_out.
fk_status fit_steps(const Ctx &c, const float *X, int64_t N, const float *C_init, int n_iter, float *C_out,
                    int32_t *assign, int32_t *counts) {
    float *ctmp = at<float>(c.ws, c.L.ctmp);
    const float *cur = C_init;
    for (int i = 0; i < n_iter; ++i) {
        float *next = ((n_iter - 1 - i) % 2 == 0) ? C_out : ctmp;
        const fk_status st = lloyd_step(c, X, N, cur, assign, nullptr, next, counts);
        if (st != FK_OK) return st;
        cur = next;
    }
    return FK_OK;
}

}  // namespace

namespace {
// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): the state advances by 0x9E3779B97F4A7C15 and
// every output is the new state through the variant-13 mix.
struct SplitMix64 {
    uint64_t st;
    uint64_t next() {
        st += 0x9E3779B97F4A7C15ull;
        uint64_t z = st;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    // uniform in [0, m): draws at or above the largest multiple of m below
    // 2^64 are rejected, the rest reduced modulo m
    uint64_t below(uint64_t m) {
        const uint64_t rem = (UINT64_MAX % m + 1) % m;  // 2^64 mod m
        for (;;) {
            const uint64_t r = next();
            if (rem == 0 || r < (uint64_t)0 - rem) return r % m;
        }
    }
};

// K distinct rows of [0, N): the first K positions of a Fisher-Yates shuffle
// of 0..N-1 (step i swaps position i with i + below(N - i)), the shuffled
// array kept as a map of the positions moved.
std::vector<int32_t> sample_rows(int64_t N, int32_t K, uint64_t seed) {
    SplitMix64 g{seed};
    std::unordered_map<int64_t, int64_t> moved;
    moved.reserve((size_t)K * 2);
    std::vector<int32_t> out((size_t)K);
    for (int64_t i = 0; i < K; ++i) {
        const int64_t j = i + (int64_t)g.below((uint64_t)(N - i));
        const auto fi = moved.find(i);
        const int64_t vi = fi == moved.end() ? i : fi->second;
        const auto fj = moved.find(j);
        const int64_t vj = fj == moved.end() ? j : fj->second;
        moved[j] = vi;
        moved[i] = vj;
        out[(size_t)i] = (int32_t)vj;
    }
    return out;
}
}  // namespace

extern "C" {

size_t fk_workspace_size(int64_t N, int32_t d, int32_t K, int32_t metric, int64_t chunk_rows) {
    if (N < 0 || N > INT32_MAX || d < 1 || d > FK_MAX_D || K < 1 || K > FK_MAX_K) return 0;
    if (!known_metric(metric)) return 0;
    if (chunk_rows < 0 || chunk_rows > INT32_MAX) return 0;
    const bool ooc = chunk_rows > 0;
    return make_layout(ooc ? chunk_rows : N, d, K, metric, ooc).total;
}

const char *fk_status_str(int32_t s) {
    switch (s) {
    case FK_OK: return "FK_OK";
    case FK_ERR_INVALID_ARG: return "FK_ERR_INVALID_ARG";
    case FK_ERR_UNSUPPORTED: return "FK_ERR_UNSUPPORTED";
    case FK_ERR_WORKSPACE: return "FK_ERR_WORKSPACE";
    case FK_ERR_NO_DEVICE: return "FK_ERR_NO_DEVICE";
    case FK_ERR_HIP: return "FK_ERR_HIP";
    default: return "FK_ERR_UNKNOWN";
    }
}

const char *fk_last_error(void) { return g_err; }

fk_status fk_assign(const float *X, int64_t N, int32_t d, const float *C, int32_t K, int32_t metric, int32_t score,
                    int32_t *assign, float *min_dist, void *workspace, size_t workspace_bytes, void *stream) {
    g_err[0] = 0;
    fk_status st = check_common(X, N, d, C, K, metric);
    if (st != FK_OK) return st;
    if ((st = check_score(score)) != FK_OK) return st;
    if (N > 0 && assign == nullptr) return fail(FK_ERR_INVALID_ARG, "assign is NULL");
    const Layout L = make_layout(N, d, K, metric, false);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != FK_OK) return st;
    if ((st = check_device()) != FK_OK) return st;
    if (N == 0) return FK_OK;
    const Ctx c{L, workspace, (hipStream_t)stream, d, K, metric, score};
    const float *Cu = nullptr;
    if ((st = step_prep(c, C, &Cu)) != FK_OK) return st;
    if ((st = step_xnorm(c, X, N)) != FK_OK) return st;
    return step_assign(c, X, N, C, Cu, assign, min_dist);
}

fk_status fk_sort_inverse(const int32_t *assign, int64_t N, int32_t K, int32_t *perm, int32_t *offsets,
                          void *workspace, size_t workspace_bytes, void *stream) {
    g_err[0] = 0;
    fk_status st = check_sizes(N, 1, K);
    if (st != FK_OK) return st;
    if (N > 0 && (assign == nullptr || perm == nullptr))
        return fail(FK_ERR_INVALID_ARG, "assign and perm must not be NULL");
    if (offsets == nullptr) return fail(FK_ERR_INVALID_ARG, "offsets is NULL");
    const Layout L = make_layout(N, 1, K, FK_METRIC_L2, false);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != FK_OK) return st;
    if ((st = check_device()) != FK_OK) return st;
    const Ctx c{L, workspace, (hipStream_t)stream, 1, K, FK_METRIC_L2, FK_SCORE_FP32};
    if (N == 0) {
        FK_TRY(launch_offsets(nullptr, 0, K, offsets, c.s), "cluster offsets");
        return FK_OK;
    }
    return step_sort(c, assign, N, perm, offsets);
}

fk_status fk_update(const float *X, int64_t N, int32_t d, const int32_t *assign, int32_t K, int32_t metric,
                    const float *C_prev, float *C_out, int32_t *counts, void *workspace, size_t workspace_bytes,
                    void *stream) {
    g_err[0] = 0;
    fk_status st = check_common(X, N, d, C_prev, K, metric);
    if (st != FK_OK) return st;
    if (N > 0 && assign == nullptr) return fail(FK_ERR_INVALID_ARG, "assign is NULL");
    if (C_out == nullptr || counts == nullptr) return fail(FK_ERR_INVALID_ARG, "C_out and counts must not be NULL");
    const size_t cb = (size_t)K * d * 4;
    if (overlap(C_out, cb, C_prev, cb)) return fail(FK_ERR_INVALID_ARG, "C_out overlaps C_prev");
    const Layout L = make_layout(N, d, K, metric, false);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != FK_OK) return st;
    if ((st = check_device()) != FK_OK) return st;
    const Ctx c{L, workspace, (hipStream_t)stream, d, K, metric, FK_SCORE_FP32};
    if ((st = step_zero_accumulators(c, false, N)) != FK_OK) return st;
    if ((st = step_xnorm(c, X, N)) != FK_OK) return st;
    if (N > 0) return step_accumulate(c, X, N, assign, false, C_prev, C_out, counts);
    return step_finalize(c, C_prev, C_out, counts);
}

namespace {
// Arguments of fk_lloyd_iter and fk_lloyd_iter_noalloc, workspace aside.
fk_status check_lloyd_args(const float *X, int64_t N, int32_t d, const float *C_in, int32_t K, int32_t metric,
                           int32_t score, const int32_t *assign, const float *C_out, const int32_t *counts) {
    fk_status st = check_common(X, N, d, C_in, K, metric);
    if (st != FK_OK) return st;
    if ((st = check_score(score)) != FK_OK) return st;
    if (N > 0 && assign == nullptr) return fail(FK_ERR_INVALID_ARG, "assign is NULL");
    if (C_out == nullptr || counts == nullptr) return fail(FK_ERR_INVALID_ARG, "C_out and counts must not be NULL");
    const size_t cb = (size_t)K * d * 4;
    if (overlap(C_out, cb, C_in, cb)) return fail(FK_ERR_INVALID_ARG, "C_out overlaps C_in");
    return FK_OK;
}

struct NoAllocScope {
    NoAllocScope() { t_no_alloc = true; }
    ~NoAllocScope() { t_no_alloc = false; }
};
}  // namespace

fk_status fk_lloyd_iter(const float *X, int64_t N, int32_t d, const float *C_in, int32_t K, int32_t metric,
                        int32_t score, int32_t *assign, float *min_dist, float *C_out, int32_t *counts,
                        void *workspace, size_t workspace_bytes, void *stream) {
    g_err[0] = 0;
    fk_status st = check_lloyd_args(X, N, d, C_in, K, metric, score, assign, C_out, counts);
    if (st != FK_OK) return st;
    const Layout L = make_layout(N, d, K, metric, false);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != FK_OK) return st;
    if ((st = check_device()) != FK_OK) return st;
    const Ctx c{L, workspace, (hipStream_t)stream, d, K, metric, score};
    return lloyd_step(c, X, N, C_in, assign, min_dist, C_out, counts);
}

fk_status fk_lloyd_iter_noalloc(const float *X, int64_t N, int32_t d, const float *C_in, int32_t K, int32_t metric,
                                int32_t score, int32_t *assign, float *min_dist, float *C_out, int32_t *counts,
                                void *stream) {
    g_err[0] = 0;
    fk_status st = check_lloyd_args(X, N, d, C_in, K, metric, score, assign, C_out, counts);
    if (st != FK_OK) return st;
    const Layout L = make_layout(N, d, K, metric, false);
    if (L.total > (size_t)FK_NOALLOC_SCRATCH_BYTES)
        return fail(FK_ERR_WORKSPACE,
                    "N=%lld, d=%d, K=%d needs %zu bytes of scratch; fk_lloyd_iter_noalloc holds %zu (use "
                    "fk_lloyd_iter with a workspace)",
                    (long long)N, (int)d, (int)K, L.total, (size_t)FK_NOALLOC_SCRATCH_BYTES);
    if ((st = check_device()) != FK_OK) return st;
    void *ws = nullptr;
    int dev = 0;
    FK_TRY(hipGetDevice(&dev), "hipGetDevice");
    FK_TRY(noalloc_scratch(dev, &ws), "hipGetSymbolAddress of the static scratch");
    if (ws == nullptr || !aligned(ws, 256)) return fail(FK_ERR_HIP, "the static scratch has no usable device address");
    NoAllocScope no_alloc;
    const Ctx c{L, ws, (hipStream_t)stream, d, K, metric, score};
    return lloyd_step(c, X, N, C_in, assign, min_dist, C_out, counts);
}

// Library-owned copy stream and events for the out-of-core pipeline (one set
// per device, created on first use, default priority).  Calls on one device
// share them, so a call holds the device's mutex while it enqueues: calls
// from several host threads are then enqueued one after the other (a stream
// wait takes the event's record at the time it is enqueued, so each call's
// waits see its own records).
namespace {
constexpr int kMaxOocDevices = 64;
struct OocRes {
    bool ready = false;
    hipStream_t copy = nullptr;
    hipEvent_t copied[2] = {nullptr, nullptr};
    hipEvent_t freed[2] = {nullptr, nullptr};
    hipEvent_t entry = nullptr;
    std::mutex mu;
};
std::mutex g_ooc_mu;
OocRes g_ooc[kMaxOocDevices];

fk_status ooc_resources(OocRes **out) {
    int dev = 0;
    FK_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxOocDevices)
        return fail(FK_ERR_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxOocDevices);
    std::lock_guard<std::mutex> g(g_ooc_mu);
    OocRes &r = g_ooc[dev];
    if (!r.ready) {
        FK_TRY(hipStreamCreateWithFlags(&r.copy, hipStreamNonBlocking), "copy stream");
        for (int i = 0; i < 2; ++i) {
            FK_TRY(hipEventCreateWithFlags(&r.copied[i], hipEventDisableTiming), "event");
            FK_TRY(hipEventCreateWithFlags(&r.freed[i], hipEventDisableTiming), "event");
        }
        FK_TRY(hipEventCreateWithFlags(&r.entry, hipEventDisableTiming), "event");
        r.ready = true;
    }
    *out = &r;
    return FK_OK;
}

bool is_pinned_host(const void *p) {
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof attr);
    const hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeHost;
}
}  // namespace

fk_status fk_lloyd_iter_stream(const float *X_host, int64_t N, int32_t d, const float *C_in, int32_t K,
                               int32_t metric, int32_t score, int64_t chunk_rows, int32_t *assign_host,
                               float *C_out, int32_t *counts, void *workspace, size_t workspace_bytes,
                               void *stream) {
    g_err[0] = 0;
    fk_status st = check_common(X_host, N, d, C_in, K, metric);
    if (st != FK_OK) return st;
    if ((st = check_score(score)) != FK_OK) return st;
    if (chunk_rows < 1 || chunk_rows > INT32_MAX)
        return fail(FK_ERR_INVALID_ARG, "chunk_rows=%lld must be in [1, 2^31-1]", (long long)chunk_rows);
    if (C_out == nullptr || counts == nullptr) return fail(FK_ERR_INVALID_ARG, "C_out and counts must not be NULL");
    const size_t cb = (size_t)K * d * 4;
    if (overlap(C_out, cb, C_in, cb)) return fail(FK_ERR_INVALID_ARG, "C_out overlaps C_in");
    const Layout L = make_layout(chunk_rows, d, K, metric, true);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != FK_OK) return st;
    if ((st = check_device()) != FK_OK) return st;
    if (N > 0 && !is_pinned_host(X_host)) return fail(FK_ERR_INVALID_ARG, "X_host is not pinned host memory");
    if (N > 0 && assign_host != nullptr && !is_pinned_host(assign_host))
        return fail(FK_ERR_INVALID_ARG, "assign_host is not pinned host memory");
    OocRes *R = nullptr;
    if ((st = ooc_resources(&R)) != FK_OK) return st;
    std::lock_guard<std::mutex> serial(R->mu);

    const Ctx c{L, workspace, (hipStream_t)stream, d, K, metric, score};
    if ((st = step_zero_accumulators(c, true, N)) != FK_OK) return st;
    const float *Cu = nullptr;
    if (N > 0 && (st = step_prep(c, C_in, &Cu)) != FK_OK) return st;
    // the copy stream may not touch the chunk buffers before the work already
    // queued on the caller's stream is done with the workspace
    FK_TRY(hipEventRecord(R->entry, c.s), "event record");
    FK_TRY(hipStreamWaitEvent(R->copy, R->entry, 0), "stream wait");

    // Chunk lengths: a ramp that doubles from chunk_rows / 16 (when that is
    // over 2^20 rows) up to chunk_rows.  Only the first copy is not hidden
    // behind compute, and assigning a chunk takes about twice as long as
    // copying one twice its length, so each copy still lands before it is
    // needed while the first one is short.
    int64_t len = chunk_rows / 16 > ((int64_t)1 << 20) ? chunk_rows / 16 : chunk_rows;
    int64_t r0 = 0;
    for (int64_t ci = 0; r0 < N; ++ci, r0 += len, len = (2 * len < chunk_rows ? 2 * len : chunk_rows)) {
        const int b = (int)(ci & 1);
        const int64_t rows = (N - r0) < len ? (N - r0) : len;
        float *Xd = at<float>(workspace, L.xchunk[b]);
        int32_t *ad = at<int32_t>(workspace, L.achunk[b]);
        if (ci >= 2) FK_TRY(hipStreamWaitEvent(R->copy, R->freed[b], 0), "stream wait");
        {
            PhaseScope ph(FK_PH_H2D, R->copy);
            FK_TRY(hipMemcpyAsync(Xd, X_host + (size_t)r0 * d, (size_t)rows * d * 4, hipMemcpyHostToDevice, R->copy),
                   "chunk copy");
        }
        FK_TRY(hipEventRecord(R->copied[b], R->copy), "event record");
        FK_TRY(hipStreamWaitEvent(c.s, R->copied[b], 0), "stream wait");
        if ((st = step_xnorm(c, Xd, rows)) != FK_OK) return st;
        // the near-tie list is per chunk: reset its counter
        FK_TRY(launch_fill_zero(at<void>(workspace, L.counter), 16, c.s), "reset counters");
        if ((st = step_assign(c, Xd, rows, C_in, Cu, ad, nullptr)) != FK_OK) return st;
        if ((st = step_accumulate(c, Xd, rows, ad, true)) != FK_OK) return st;
        FK_TRY(hipEventRecord(R->freed[b], c.s), "event record");
        if (assign_host != nullptr)
            FK_TRY(hipMemcpyAsync(assign_host + r0, ad, (size_t)rows * 4, hipMemcpyDeviceToHost, c.s),
                   "assignment copy");
    }
    return step_finalize(c, C_in, C_out, counts);
}

size_t fk_fit_workspace_size(int64_t N, int32_t d, int32_t K, int32_t metric) {
    if (N < 0 || N > INT32_MAX || d < 1 || d > FK_MAX_D || K < 1 || K > FK_MAX_K) return 0;
    if (!known_metric(metric)) return 0;
    return make_layout(N, d, K, metric, false, kFitExtras).total;
}

fk_status fk_fit(const float *X, int64_t N, int32_t d, int32_t K, int32_t metric, int32_t score, const float *C_init,
                 uint64_t seed, int32_t n_iter, double tol, float *C_out, int32_t *assign, int32_t *counts,
                 fk_fit_info *info, void *workspace, size_t workspace_bytes, void *stream) {
    g_err[0] = 0;
    fk_status st = check_sizes(N, d, K);
    if (st != FK_OK) return st;
    if ((st = check_metric(metric)) != FK_OK) return st;
    if ((st = check_score(score)) != FK_OK) return st;
    if (n_iter < 1) return fail(FK_ERR_INVALID_ARG, "n_iter=%d must be at least 1", (int)n_iter);
    if (C_init == nullptr && N < 1) return fail(FK_ERR_INVALID_ARG, "initial rows cannot be drawn from N=0 rows");
    if (std::isnan(tol)) return fail(FK_ERR_INVALID_ARG, "tol is NaN");
    if (N > 0 && (X == nullptr || assign == nullptr)) return fail(FK_ERR_INVALID_ARG, "X and assign are required");
    if (C_out == nullptr || counts == nullptr) return fail(FK_ERR_INVALID_ARG, "C_out and counts must not be NULL");
    if ((X != nullptr && !aligned(X, 16)) || (C_init != nullptr && !aligned(C_init, 16)) || !aligned(C_out, 16))
        return fail(FK_ERR_INVALID_ARG, "X, C_init and C_out must be 16-byte aligned");
    // the guide's clamp: no more clusters than rows when the rows are drawn
    const int32_t Ku = C_init != nullptr ? K : (int32_t)(N < K ? N : K);
    const size_t cb = (size_t)Ku * d * 4;
    if (C_init != nullptr && overlap(C_out, cb, C_init, cb)) return fail(FK_ERR_INVALID_ARG, "C_out overlaps C_init");
    const Layout L = make_layout(N, d, K, metric, false, kFitExtras);  // regions sized for K >= Ku
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != FK_OK) return st;
    if ((st = check_device()) != FK_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    const Ctx c{L, workspace, s, d, Ku, metric, score};
    const float *cur = C_init;
    if (cur == nullptr) {
        const std::vector<int32_t> idx = sample_rows(N, Ku, seed);
        int32_t *idx_dev = at<int32_t>(workspace, L.init_idx);
        FK_TRY(hipMemcpyAsync(idx_dev, idx.data(), (size_t)Ku * 4, hipMemcpyHostToDevice, s), "initial row indices");
        FK_TRY(hipStreamSynchronize(s), "stream sync");  // idx leaves scope
        FK_TRY(launch_gather_rows(X, idx_dev, Ku, d, at<float>(workspace, L.cinit), s), "initial centroids");
        cur = at<float>(workspace, L.cinit);
    }
    float *ctmp = at<float>(workspace, L.ctmp);
    int32_t done = 0;
    double last = -1.0;
    for (int32_t i = 0; i < n_iter; ++i) {
        // the buffers alternate so that a full run ends in C_out
        float *next = ((n_iter - 1 - i) % 2 == 0) ? C_out : ctmp;
        if ((st = lloyd_step(c, X, N, cur, assign, nullptr, next, counts)) != FK_OK) return st;
        done = i + 1;
        if (tol >= 0.0) {
            FK_TRY(launch_max_shift(cur, next, Ku, d, at<double>(workspace, L.shift_part),
                                    at<double>(workspace, L.shift), s),
                   "centroid shift");
            double h = 0.0;
            FK_TRY(hipMemcpyAsync(&h, at<double>(workspace, L.shift), sizeof h, hipMemcpyDeviceToHost, s),
                   "centroid shift copy");
            FK_TRY(hipStreamSynchronize(s), "stream sync");
            last = h;
            cur = next;
            if (h <= tol) break;
        } else {
            cur = next;
        }
    }
    if (cur != C_out) FK_TRY(hipMemcpyAsync(C_out, cur, cb, hipMemcpyDeviceToDevice, s), "centroid copy");
    if (info != nullptr) {
        info->k_used = Ku;
        info->iterations = done;
        info->last_shift = last;
    }
    return FK_OK;
}

size_t fk_ivf_workspace_size(int64_t N, int32_t d, int32_t nlist, int32_t metric) {
    if (N < 1 || N > INT32_MAX || d < 1 || d > FK_MAX_D || nlist < 1 || nlist > FK_MAX_K) return 0;
    if (metric != FK_METRIC_L2 && metric != FK_METRIC_COSINE) return 0;
    const int32_t nl = (int32_t)(N < nlist ? N : nlist);
    return make_layout(N, d, nl, metric, false, kIvfExtras).total;
}

fk_status fk_ivf_build(const float *X, int64_t N, int32_t d, int32_t nlist, int32_t metric, int32_t score,
                       int32_t n_iter, const int32_t *init_idx_host, uint64_t seed, float *centroids,
                       int32_t *list_offsets, int32_t *list_ids, float *list_data, int32_t *nlist_used,
                       void *workspace, size_t workspace_bytes, void *stream) {
    g_err[0] = 0;
    fk_status st = check_sizes(N, d, nlist);
    if (st != FK_OK) return st;
    if ((st = check_metric(metric)) != FK_OK) return st;
    if (metric == FK_METRIC_INNER_PRODUCT || metric == FK_METRIC_SPHERICAL)
        return fail(FK_ERR_UNSUPPORTED, "the IVF build takes L2 or cosine (inner product: normalise, i.e. cosine)");
    if ((st = check_score(score)) != FK_OK) return st;
    if (N < 1) return fail(FK_ERR_INVALID_ARG, "the IVF build needs N >= 1 rows");
    if (n_iter < 1) return fail(FK_ERR_INVALID_ARG, "n_iter=%d must be at least 1", (int)n_iter);
    if (X == nullptr || centroids == nullptr || list_offsets == nullptr || list_ids == nullptr || list_data == nullptr)
        return fail(FK_ERR_INVALID_ARG, "X, centroids, list_offsets, list_ids and list_data are required");
    if (!aligned(X, 16) || !aligned(centroids, 16) || !aligned(list_data, 16))
        return fail(FK_ERR_INVALID_ARG, "X, centroids and list_data must be 16-byte aligned");
    // the guide clamps the cell count to the row count
    const int32_t nl = (int32_t)(N < nlist ? N : nlist);
    if (init_idx_host != nullptr)
        for (int32_t k = 0; k < nl; ++k)
            if (init_idx_host[k] < 0 || init_idx_host[k] >= N)
                return fail(FK_ERR_INVALID_ARG, "init_idx[%d]=%d outside [0, N)", (int)k, (int)init_idx_host[k]);
    const size_t xb = (size_t)N * d * 4;
    if (overlap(list_data, xb, X, xb)) return fail(FK_ERR_INVALID_ARG, "list_data overlaps X");
    const Layout L = make_layout(N, d, nl, metric, false, kIvfExtras);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != FK_OK) return st;
    if ((st = check_device()) != FK_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    // cosine: the lists hold the normalised rows and the quantizer is L2
    // k-means on them (normalising X and C on entry of every iteration would
    // train a different, spherical, quantizer)
    const Ctx c{L, workspace, s, d, nl, FK_METRIC_L2, score};
    const float *Xu = X;
    if (metric == FK_METRIC_COSINE) {
        PhaseScope ph(FK_PH_PREP, s);
        FK_TRY(launch_row_norm64(X, N, d, at<double>(workspace, L.xnorm64), s), "row norms");
        FK_TRY(launch_normalize_rows(X, N, d, at<double>(workspace, L.xnorm64), nullptr, at<float>(workspace, L.xcopy),
                                     s),
               "row normalisation");
        Xu = at<float>(workspace, L.xcopy);
    }
    int32_t *idx_dev = at<int32_t>(workspace, L.init_idx);
    {
        std::vector<int32_t> drawn;
        const int32_t *idx_host = init_idx_host;
        if (idx_host == nullptr) {
            drawn = sample_rows(N, nl, seed);
            idx_host = drawn.data();
        }
        FK_TRY(hipMemcpyAsync(idx_dev, idx_host, (size_t)nl * 4, hipMemcpyHostToDevice, s), "init indices");
        FK_TRY(hipStreamSynchronize(s), "stream sync");  // the host indices may leave scope
    }
    FK_TRY(launch_gather_rows(Xu, idx_dev, nl, d, at<float>(workspace, L.cinit), s), "initial centroids");
    int32_t *labels = at<int32_t>(workspace, L.labels);
    int32_t *cnt = at<int32_t>(workspace, L.cnt);
    if ((st = fit_steps(c, Xu, N, at<float>(workspace, L.cinit), n_iter, centroids, labels, cnt)) != FK_OK) return st;
    // the lists: every row under the final centroids, grouped by cell
    const float *Cu = nullptr;
    if ((st = step_prep(c, centroids, &Cu)) != FK_OK) return st;
    if ((st = step_assign(c, Xu, N, centroids, Cu, labels, nullptr)) != FK_OK) return st;
    if ((st = step_sort(c, labels, N, list_ids, list_offsets)) != FK_OK) return st;
    {
        PhaseScope ph(FK_PH_REDUCE, s);
        FK_TRY(launch_gather_rows(Xu, list_ids, N, d, list_data, s), "list rows");
    }
    if (nlist_used != nullptr) *nlist_used = nl;
    return FK_OK;
}

size_t fk_knn_workspace_size(int64_t M, int32_t d, int64_t Ndb, int32_t k, int32_t metric) {
    if (M < 0 || M > INT32_MAX || d < 1 || d > FK_MAX_D || Ndb < 1 || Ndb > FK_MAX_KNN_DB || k < 1) return 0;
    const int32_t kk = (int32_t)(Ndb < k ? Ndb : k);
    if (kk > FK_MAX_KNN_K) return 0;
    if (metric != FK_METRIC_L2 && metric != FK_METRIC_COSINE && metric != FK_METRIC_INNER_PRODUCT) return 0;
    return make_knn_layout(M, d, Ndb, kk, metric).total;
}

fk_status fk_knn(const float *Q, int64_t M, int32_t d, const float *DB, int64_t Ndb, int32_t k, int32_t metric,
                 int32_t score, int32_t *idx, float *dist, void *workspace, size_t workspace_bytes, void *stream) {
    g_err[0] = 0;
    if (M < 0 || M > INT32_MAX) return fail(FK_ERR_INVALID_ARG, "M=%lld outside [0, 2^31-1]", (long long)M);
    if (d < 1 || d > FK_MAX_D) return fail(FK_ERR_INVALID_ARG, "d=%d outside [1, %d]", (int)d, FK_MAX_D);
    if (Ndb < 1 || Ndb > FK_MAX_KNN_DB)
        return fail(FK_ERR_INVALID_ARG, "Ndb=%lld outside [1, %d]", (long long)Ndb, FK_MAX_KNN_DB);
    // the backend clamps k to the database size; the columns past it are padding
    const int32_t kk = (int32_t)(Ndb < k ? Ndb : k);
    if (k < 1 || kk > FK_MAX_KNN_K)
        return fail(FK_ERR_INVALID_ARG, "k=%d: need k >= 1 and min(k, Ndb=%lld) <= %d", (int)k, (long long)Ndb,
                    FK_MAX_KNN_K);
    fk_status st = check_metric(metric);
    if (st != FK_OK) return st;
    if (metric == FK_METRIC_SPHERICAL)
        return fail(FK_ERR_UNSUPPORTED, "spherical is a centroid option; k-NN takes L2, cosine or inner product");
    if ((st = check_score(score)) != FK_OK) return st;
    if (DB == nullptr) return fail(FK_ERR_INVALID_ARG, "DB is NULL");
    if (M > 0 && (Q == nullptr || idx == nullptr || dist == nullptr))
        return fail(FK_ERR_INVALID_ARG, "Q, idx and dist are required");
    if (!aligned(DB, 16) || (Q != nullptr && !aligned(Q, 16)))
        return fail(FK_ERR_INVALID_ARG, "Q and DB must be 16-byte aligned");
    if (score == FK_SCORE_SPLIT_BF16 &&
        cdiv(Ndb, kCentroidPad) * kCentroidPad * 4 * (int64_t)split_width(d) > (int64_t)UINT32_MAX)
        return fail(FK_ERR_UNSUPPORTED, "split scoring: the database's bf16 copy (Ndb=%lld, d=%d) exceeds 4 GiB",
                    (long long)Ndb, (int)d);
    const Layout L = make_knn_layout(M, d, Ndb, kk, metric);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != FK_OK) return st;
    if ((st = check_device()) != FK_OK) return st;
    if (M == 0) return FK_OK;
    const hipStream_t s = (hipStream_t)stream;
    const Ctx c{L, workspace, s, d, (int)Ndb, metric, score};
    const float *DBu = nullptr;
    if ((st = step_prep(c, DB, &DBu)) != FK_OK) return st;
    if ((st = step_xnorm(c, Q, M)) != FK_OK) return st;
    const bool cos = metric == FK_METRIC_COSINE, ip = metric == FK_METRIC_INNER_PRODUCT;
    const double *qn = cos ? at<double>(workspace, L.xnorm64) : nullptr;
    int32_t *cand = at<int32_t>(workspace, L.knn_cand), *list = at<int32_t>(workspace, L.knn_list);
    float *cscore = at<float>(workspace, L.knn_score), *win = at<float>(workspace, L.knn_win);
    int32_t *counters = at<int32_t>(workspace, L.counter);
    {
        PhaseScope ph(FK_PH_ASSIGN, s);
        FK_TRY(launch_knn_sweep(Q, M, d, DBu, at<float>(workspace, L.ncn), (int)Ndb, at<float>(workspace, L.scal), qn,
                                c.split(), ip, kk, cand, cscore, win, at<float>(workspace, L.knn_tau), s),
               "knn sweep");
    }
    {
        PhaseScope ph(FK_PH_RECHECK, s);
        FK_TRY(launch_knn_finish(Q, M, d, DB, cos ? at<double>(workspace, L.c64) : nullptr, qn, ip, cand, cscore, win,
                                 kk, k, (int)Ndb, list, counters, idx, dist, s),
               "knn finish");
    }
    return FK_OK;
}

fk_status fk_profile_enable(int32_t on) {
    g_err[0] = 0;
    std::lock_guard<std::mutex> g(g_prof.mu);
    g_prof.on = on != 0;
    if (g_prof.on) {
        g_prof.acc = fk_profile{};
        for (auto &p : g_prof.pending) {
            g_prof.pool.push_back(p.a);
            g_prof.pool.push_back(p.b);
        }
        g_prof.pending.clear();
        g_prof.slots_used = 0;
    }
    return FK_OK;
}

fk_status fk_profile_read(fk_profile *out) {
    g_err[0] = 0;
    if (out == nullptr) return fail(FK_ERR_INVALID_ARG, "out is NULL");
    std::lock_guard<std::mutex> g(g_prof.mu);
    for (auto &p : g_prof.pending) {
        FK_TRY(hipEventSynchronize(p.b), "event sync");
        float ms = 0.f;
        FK_TRY(hipEventElapsedTime(&ms, p.a, p.b), "event time");
        g_prof.acc.ms[p.phase] += ms;
        g_prof.acc.calls[p.phase] += 1;
        g_prof.pool.push_back(p.a);
        g_prof.pool.push_back(p.b);
    }
    g_prof.pending.clear();
    if (g_prof.slots_used > 0) FK_TRY(hipDeviceSynchronize(), "device sync");
    for (size_t i = 0; i < g_prof.slots_used; ++i) {
        g_prof.acc.windowed += g_prof.count_slots[i][0];
        g_prof.acc.paired += g_prof.count_slots[i][1];
        g_prof.acc.rechecked += g_prof.count_slots[i][2];
    }
    g_prof.slots_used = 0;
    *out = g_prof.acc;
    g_prof.acc = fk_profile{};
    return FK_OK;
}

}  // extern "C"
