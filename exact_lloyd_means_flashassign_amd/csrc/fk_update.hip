// Sort-Inverse Update for gfx950: per-cluster sums over the inverse index,
// without atomics.
//
// The Flash-KMeans article (lumevalley.com, article 3696, section
// "Sort-Inverse Update: another answer to atomics") reduces each cluster by
// reading the sorted inverse index contiguously, one thread block per few
// clusters.  Under a skewed (Zipf) size distribution one cluster can hold a
// fifth of all points, so a block per cluster would leave one block reading
// millions of rows.  Here the sorted rows are cut into equal segments of
// seg_rows(N, d) rows, one wave each:
//   * a cluster that lies inside one segment is summed and written by that
//     wave alone;
//   * a cluster that crosses segment boundaries leaves one partial row per
//     segment it touches (pfirst: the segment's first cluster when it started
//     earlier; plast: the segment's last cluster when it continues later), and
//     k_seg_finish (rows in one batch) or k_seg_fixup (several batches) adds
//     those partials in a fixed order.
// Every output element has exactly one writer and a fixed summation order, so
// the result is bitwise reproducible.  Sums are fp64.  The gathered rows
// X[perm[r]] are read as whole coalesced rows.  When all rows come in one
// batch, the divide by the count is done where a cluster's sum is complete
// (the wave of an inner cluster, k_seg_fixup for a crossing one), so the fp64
// sums never go through memory; the cluster offsets are written by the
// reduction as it meets each key change.
#include <mutex>

#include "fk.h"
#include "fk_internal.h"

namespace fk {

typedef float f2v __attribute__((ext_vector_type(2)));
typedef float f4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_fill_zero(uint32_t *__restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// NV loads of E consecutive floats per lane cover 64*E*NV columns starting at
// blockIdx.y * 64*E*NV.  U rows are loaded before they are accumulated so that
// U row reads per lane are in flight at once.  RP = 2 (rows of 128 floats or
// fewer, E = 4, NV = 1): each half-wave loads one row, so one 16-byte load per
// lane brings two rows (half the load instructions of 8-byte loads); the
// lower half sums the pair's first rows and the upper half the second ones,
// and a cluster's total is the lower half's sum plus the upper half's.
// COS: rows are scaled by 1/xnorm64 (cosine).  ACC: cluster sums are added to what sums holds (rows
// fed in several batches; the finalize step divides).  Otherwise the rows
// come in one batch and a cluster inside the segment is written to C_out as
// its sum divided by its row count (clusters that no row reaches are left to
// k_seg_finish).  The column block blockIdx.y == 0 also writes offsets[k] =
// the first sorted row whose key is >= k (offsets[K] = N): the entries between
// two consecutive keys are written by the wave that sees the change.
template <int NV, int E, int U, bool COS, bool ACC, int RP>
__global__ __launch_bounds__(256) void k_seg_reduce(const float *__restrict__ X, int64_t N, int d, int K, int srows,
                                                    const int32_t *__restrict__ ks, const int32_t *__restrict__ perm,
                                                    const double *__restrict__ xnorm64, double *__restrict__ sums,
                                                    double *__restrict__ pfirst, double *__restrict__ plast,
                                                    int32_t *__restrict__ offsets, float *__restrict__ C_out) {
    // the wave index is uniform across the wave: taking it as a scalar makes
    // the segment bounds, the keys and every branch on them scalar
    static_assert(RP == 1 || (RP == 2 && NV == 1 && E == 4), "paired rows take one 16-byte load per lane");
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // RP = 2: the half-wave (which row of a pair) and the lane within it
    const int half = RP == 2 ? lane >> 5 : 0;
    const int cl = RP == 2 ? lane & 31 : lane;
    const int64_t seg = (int64_t)blockIdx.x * kSegWaves + w;
    const int64_t r0 = seg * srows;
    if (r0 >= N) return;
    const int64_t r1 = (r0 + srows < N) ? r0 + srows : N;
    const int cbase = blockIdx.y * (64 / RP * E * NV);

    const int first_k = ks[r0];
    const int prev_k = r0 > 0 ? ks[r0 - 1] : -1;
    const bool started_before = r0 > 0 && prev_k == first_k;
    const int last_k = ks[r1 - 1];
    const bool cont_after = r1 < N && ks[r1] == last_k;
    int32_t *const offs = blockIdx.y == 0 ? offsets : nullptr;
    // offsets[from+1 .. to] = row, spread over the lanes (the clamps only keep
    // a key outside [0, K) from writing outside offsets[0..K])
    auto mark = [&](int from, int to, int64_t row) {
        const int lo = max(from + 1, 0), hi = min(to, K);
        for (int k = lo + lane; k <= hi; k += 64) offs[k] = (int32_t)row;
    };
    if (offs != nullptr) mark(prev_k, first_k, r0);

    int col[NV];
    bool cok[NV], wok[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        col[v] = cbase + (v * (64 / RP) + cl) * E;
        cok[v] = col[v] < d;  // d is a multiple of E, so the whole E-group is in or out
        wok[v] = cok[v] && half == 0;  // paired rows: the lower half writes the totals
    }

    double acc[NV][E];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[v][e] = 0.0;
    int cur = first_k;
    int64_t cstart = r0;  // first row of cluster cur in this segment

    // the sum of cluster k, whose rows in this segment end before row rend
    auto flush = [&](int k, int64_t rend) {
        if constexpr (RP == 2) {
            // both halves get the same total (a0 + a1 == a1 + a0)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[0][e] += __shfl_xor(acc[0][e], 32);
        }
        // keys are documented to lie in [0, K); a bad key is dropped rather
        // than written outside the sums
        if ((unsigned)k >= (unsigned)K) {
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[v][e] = 0.0;
            return;
        }
        const bool part_first = k == first_k && started_before;
        const bool part_last = k == last_k && cont_after;
        if (!ACC && !part_first && !part_last) {
            // the whole cluster is in this segment: its centroid
            const double n = (double)(rend - cstart);
            float *o = C_out + (int64_t)k * d;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                if (!wok[v]) {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[v][e] = 0.0;
                    continue;
                }
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    o[col[v] + e] = (float)(acc[v][e] / n);
                    acc[v][e] = 0.0;
                }
            }
            return;
        }
        double *dst = part_first  ? pfirst + seg * (int64_t)d
                      : part_last ? plast + seg * (int64_t)d
                                  : sums + (int64_t)k * d;
        const bool add = !part_first && !part_last;  // ACC here
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (!wok[v]) {
#pragma unroll
                for (int e = 0; e < E; ++e) acc[v][e] = 0.0;
                continue;
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double val = add ? dst[col[v] + e] + acc[v][e] : acc[v][e];
                dst[col[v] + e] = val;
                acc[v][e] = 0.0;
            }
        }
    };

    // Rows go in windows of 64 (one key and one row index per lane) and
    // batches of U rows.  The loads of the next batch are issued before the
    // current one is added, and every load is unconditional (row indices past
    // the segment repeat its last row, columns past d repeat the last valid
    // group), so that the wait for a batch never waits on later loads or on
    // the stores of a flush.
    constexpr int RB = U * RP;   // rows per batch
    static_assert(64 % (2 * RB) == 0, "batches must pair up inside a window");
    constexpr int NBW = 64 / RB;  // batches per window
    auto load_window = [&](int64_t r, int &kk, int &pp) {
        const int64_t q = (r + lane < r1) ? r + lane : r1 - 1;
        kk = ks[q];
        pp = perm[q];
    };
    int ccol[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) ccol[v] = cok[v] ? col[v] : d - E;
    auto load_batch = [&](float (&vb)[U][NV][E], double (&sb)[U], int pp, int off) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int p = __builtin_amdgcn_readlane(pp, off + RP * u);
            if constexpr (RP == 2) {
                const int p2 = __builtin_amdgcn_readlane(pp, off + 2 * u + 1);
                p = half ? p2 : p;
            }
            const float *row = X + (size_t)p * d;
            if (COS) sb[u] = 1.0 / xnorm64[p];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                // each row is read once: non-temporal loads keep the stream
                // from evicting the sorted keys and the sums
                if constexpr (E == 4) {
                    const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(row + ccol[v]));
                    vb[u][v][0] = t.x;
                    vb[u][v][1] = t.y;
                    vb[u][v][2] = t.z;
                    vb[u][v][3] = t.w;
                } else if constexpr (E == 2) {
                    const f2v t = __builtin_nontemporal_load(reinterpret_cast<const f2v *>(row + ccol[v]));
                    vb[u][v][0] = t.x;
                    vb[u][v][1] = t.y;
                } else {
                    vb[u][v][0] = __builtin_nontemporal_load(row + ccol[v]);
                }
            }
        }
    };
    auto add_row = [&](const float (&vb)[U][NV][E], const double (&sb)[U], int u) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double x = (double)vb[u][v][e];
                acc[v][e] += COS ? x * sb[u] : x;
            }
    };
    auto consume = [&](const float (&vb)[U][NV][E], const double (&sb)[U], int kk, int64_t r, int off) {
        if constexpr (RP == 2) {
            // pair u: rows ra (lower half) and ra + 1 (upper half)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t ra = r + off + 2 * u;
                if (ra >= r1) break;
                const int ka = __builtin_amdgcn_readlane(kk, off + 2 * u);
                const int kb = __builtin_amdgcn_readlane(kk, off + 2 * u + 1);
                const bool bv = ra + 1 < r1;
                if (ka != cur) {
                    if (offs != nullptr) mark(cur, ka, ra);
                    flush(cur, ra);
                    cur = ka;
                    cstart = ra;
                }
                if (bv && kb == ka) {
                    add_row(vb, sb, u);
                } else {
                    if (half == 0) add_row(vb, sb, u);
                    if (bv) {
                        if (offs != nullptr) mark(cur, kb, ra + 1);
                        flush(cur, ra + 1);
                        cur = kb;
                        cstart = ra + 1;
                        if (half == 1) add_row(vb, sb, u);
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (r + off + u >= r1) break;
            const int key = __builtin_amdgcn_readlane(kk, off + u);
            if (key != cur) {
                const int64_t rr = r + off + u;
                if (offs != nullptr) mark(cur, key, rr);
                flush(cur, rr);
                cur = key;
                cstart = rr;
            }
            // columns past d add into accumulators that are never written
            add_row(vb, sb, u);
        }
    };

    int kkc, ppc, kkn, ppn;
    load_window(r0, kkc, ppc);
    load_window(r0 + 64, kkn, ppn);
    float va[U][NV][E], vb[U][NV][E];
    double sa[U], sb[U];
    load_batch(va, sa, ppc, 0);
    for (int64_t r = r0; r < r1; r += 64) {
#pragma unroll
        for (int j = 0; j < NBW; j += 2) {
            // even batches sit in va, odd ones in vb
            load_batch(vb, sb, ppc, (j + 1) * RB);
            consume(va, sa, kkc, r, j * RB);
            if (j + 2 < NBW)
                load_batch(va, sa, ppc, (j + 2) * RB);
            else
                load_batch(va, sa, ppn, 0);
            consume(vb, sb, kkc, r, (j + 1) * RB);
        }
        kkc = kkn;
        ppc = ppn;
        load_window(r + 128, kkn, ppn);
    }
    flush(cur, r1);
    if (offs != nullptr && r1 == N) mark(cur, K, N);
}

// One workgroup per segment boundary b (between segments b and b+1).  If a
// cluster k crosses it and b is the first boundary k crosses, the workgroup
// adds k's partials: plast of k's first segment, then pfirst of every later
// segment k touches, into sums[k] (acc), or (rows in one batch) divides the
// total by the cluster's row count into C_out[k].  Wave w takes the
// segments sa+1+w, sa+1+w+8, ... in order (eight loads in flight: the
// largest cluster of a skewed mixture crosses thousands of boundaries); the
// 8 wave sums are added in wave order.  Most workgroups find no cluster to
// finish and exit at once, so they stay small.
constexpr int kFixWaves = 8;

// Whether cluster k crosses boundary b (between segments b and b+1) and b is
// the first boundary it crosses; then *sa, *sb are its first and last
// segments and *n its row count.
__device__ __forceinline__ bool first_crossing(int64_t b, const int32_t *__restrict__ ks,
                                               const int32_t *__restrict__ offsets, int64_t N, int K, int srows,
                                               int *k_out, int64_t *sa, int64_t *sb, int64_t *n) {
    const int64_t rb = (b + 1) * srows;
    if (rb >= N) return false;
    const int k = ks[rb];
    if (ks[rb - 1] != k || (unsigned)k >= (unsigned)K) return false;
    const int64_t o0 = offsets[k], o1 = offsets[k + 1];
    if (o0 / srows != b) return false;
    *k_out = k;
    *sa = b;
    *sb = (o1 - 1) / srows;
    *n = o1 - o0;
    return true;
}

// The whole workgroup adds cluster k's partials: plast of its first segment
// sa, then pfirst of every later segment up to sb; wave w takes the segments
// sa+1+w, sa+1+w+8, ... in order (eight loads in flight: the largest cluster
// of a skewed mixture crosses thousands of boundaries) and the eight wave
// sums are added in wave order.  The total goes into sums[k] (acc) or,
// divided by the row count n, into C_out[k].
__device__ __forceinline__ void sum_partials(int k, int64_t sa, int64_t sb, int64_t n, int d,
                                             const double *__restrict__ pfirst, const double *__restrict__ plast,
                                             double *__restrict__ sums, bool acc, float *__restrict__ C_out) {
    __shared__ double red[kFixWaves][64];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int c0 = 0; c0 < d; c0 += 64) {
        const int c = c0 + lane;
        double s = 0.0;
        if (c < d) {
            if (w == 0) s = plast[sa * d + c];
            int64_t sg = sa + 1 + w;
            for (; sg + 7 * kFixWaves <= sb; sg += 8 * kFixWaves) {
                double a[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) a[i] = pfirst[(sg + i * kFixWaves) * d + c];
#pragma unroll
                for (int i = 0; i < 8; ++i) s += a[i];
            }
            for (; sg <= sb; sg += kFixWaves) s += pfirst[sg * d + c];
        }
        red[w][lane] = s;
        __syncthreads();
        if (w == 0 && c < d) {
            double t = red[0][lane];
#pragma unroll
            for (int ww = 1; ww < kFixWaves; ++ww) t += red[ww][lane];
            if (acc) {
                double *dst = sums + (int64_t)k * d + c;
                *dst += t;
            } else {
                C_out[(int64_t)k * d + c] = (float)(t / (double)n);
            }
        }
        __syncthreads();
    }
}

// A cluster that crosses at most kShortCross boundaries is finished by the
// one wave that finds it: each lane takes columns lane, lane + 64, ... and
// issues the loads of all its partials of a column at once, then adds them
// in segment order: plast of the first segment, then pfirst of each later
// one.  That is the order sum_partials gives with at most eight later
// segments (wave w's sum is then just segment sa+1+w, added in wave order),
// so both give the same bits.  Without it a workgroup would run through
// d / 64 dependent load rounds, two barriers each, per cluster (1M x 768,
// K = 4096: about 1,900 such clusters, 62 us).
constexpr int kShortCross = kFixWaves;
__device__ __forceinline__ void wave_sum_partials(int k, int64_t sa, int64_t sb, int64_t n, int d,
                                                  const double *__restrict__ pfirst,
                                                  const double *__restrict__ plast, float *__restrict__ C_out) {
    const int lane = threadIdx.x & 63;
    const int np = (int)(sb - sa);  // later segments, 1 .. kShortCross
    for (int c = lane; c < d; c += 64) {
        double v[kShortCross + 1];
        v[0] = plast[sa * d + c];
#pragma unroll
        for (int i = 1; i <= kShortCross; ++i)
            if (i <= np) v[i] = pfirst[(sa + i) * d + c];
        double t = v[0];
#pragma unroll
        for (int i = 1; i <= kShortCross; ++i)
            if (i <= np) t += v[i];
        C_out[(int64_t)k * d + c] = (float)(t / (double)n);
    }
}

// Rows in several batches: one workgroup per segment boundary b; if b is the
// first boundary a cluster crosses, the workgroup adds its partials into the
// fp64 sums.  Most workgroups find nothing to do and exit at once.
__global__ __launch_bounds__(kFixWaves * 64) void k_seg_fixup(const int32_t *__restrict__ ks,
                                                             const int32_t *__restrict__ offsets, int64_t N, int d,
                                                             int K, int srows,
                                                             const double *__restrict__ pfirst,
                                                             const double *__restrict__ plast,
                                                             double *__restrict__ sums, bool acc,
                                                             float *__restrict__ C_out) {
    int k;
    int64_t sa, sb, n;
    if (first_crossing(blockIdx.x, ks, offsets, N, K, srows, &k, &sa, &sb, &n))
        sum_partials(k, sa, sb, n, d, pfirst, plast, sums, acc, C_out);
}

// Rows in one batch: workgroup g takes clusters 8g .. 8g+7 (then 8(g + G) ..,
// G workgroups), one per wave (counts_out[k] from the offsets; an empty
// cluster's previous centroid copied by the whole wave, coalesced); then the
// segment boundaries 8g .. 8g+7 (then 8(g + G) ..): each wave checks one of
// them; a cluster found crossing its first boundary there is summed and
// divided into C_out by that wave when it crosses at most kShortCross
// boundaries, else by the whole workgroup.  Checking eight boundaries at
// once keeps their dependent loads in parallel.
__global__ __launch_bounds__(kFixWaves * 64) void k_seg_finish(const int32_t *__restrict__ ks,
                                                              const int32_t *__restrict__ offsets, int64_t N, int d,
                                                              int K, int srows, int64_t nbound,
                                                              const double *__restrict__ pfirst,
                                                              const double *__restrict__ plast,
                                                              const float *__restrict__ C_prev,
                                                              float *__restrict__ C_out,
                                                              int32_t *__restrict__ counts_out) {
    __shared__ int jk[kFixWaves];
    __shared__ int64_t jsa[kFixWaves], jsb[kFixWaves], jn[kFixWaves];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int64_t k = (int64_t)blockIdx.x * kFixWaves + w; k < K; k += (int64_t)gridDim.x * kFixWaves) {
        const int c = offsets[k + 1] - offsets[k];
        if (lane == 0) counts_out[k] = c;
        if (c == 0)
            for (int j = lane; j < d; j += 64) C_out[k * d + j] = C_prev[k * d + j];
    }
    for (int64_t b0 = (int64_t)blockIdx.x * kFixWaves; b0 < nbound; b0 += (int64_t)gridDim.x * kFixWaves) {
        int k = -1;
        int64_t sa = 0, sb = 0, n = 0;
        if (b0 + w < nbound && first_crossing(b0 + w, ks, offsets, N, K, srows, &k, &sa, &sb, &n)) {
            if (sb - sa <= kShortCross) {
                wave_sum_partials(k, sa, sb, n, d, pfirst, plast, C_out);
                k = -1;
            }
        } else {
            k = -1;
        }
        if (lane == 0) {
            jk[w] = k;
            jsa[w] = sa;
            jsb[w] = sb;
            jn[w] = n;
        }
        __syncthreads();
        for (int j = 0; j < kFixWaves; ++j)
            if (jk[j] >= 0) sum_partials(jk[j], jsa[j], jsb[j], jn[j], d, pfirst, plast, nullptr, false, C_out);
        __syncthreads();
    }
}

// cnt[k] (+)= size of cluster k in this batch of rows.
__global__ __launch_bounds__(256) void k_count_acc(const int32_t *__restrict__ offsets, int K,
                                                   int32_t *__restrict__ cnt, bool acc) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k < K) cnt[k] = (acc ? cnt[k] : 0) + offsets[k + 1] - offsets[k];
}

// Rows in several batches: C_out = sums / n_k, or C_prev for an empty
// cluster; counts_out = n_k = cnt[k].
__global__ __launch_bounds__(256) void k_finalize(const double *__restrict__ sums, const int32_t *__restrict__ cnt,
                                                  const float *__restrict__ C_prev, int64_t total, int d,
                                                  float *__restrict__ C_out, int32_t *__restrict__ counts_out) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= total) return;
    const int64_t k = q / d;
    const int c = cnt[k];
    C_out[q] = c > 0 ? (float)(sums[q] / (double)c) : C_prev[q];
    if (q == k * d) counts_out[k] = c;
}

// ---------------------------------------------------------------------------
// The scratch of the allocation-free Lloyd iteration (fk_lloyd_iter_noalloc):
// every device holds its own copy of this array, from the library's load on
// that device until the process ends, at its own address.  It sits in this
// file beside kernels that every iteration launches.  Host code never uses
// its name as an address: the device address comes from
// hipGetSymbolAddress, once per device, and is kept.
static_assert(FK_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[FK_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(int device, void **ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (g_scratch_ptr[device] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

// Spherical centroids: every row of C divided by its L2 norm, the norm taken
// in fp64 (a zero norm is taken as 1, so a zero row stays zero).  One wave
// per row.
__global__ __launch_bounds__(256) void k_unit_rows(float *__restrict__ C, int K, int d) {
    const int k = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (k >= K) return;
    float *row = C + (size_t)k * d;
    double q = 0.0;
    for (int j = lane; j < d; j += 64) {
        const double v = (double)row[j];
        q += v * v;
    }
    for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off);
    double n = sqrt(q);
    if (n == 0.0) n = 1.0;
    for (int j = lane; j < d; j += 64) row[j] = (float)((double)row[j] / n);
}

hipError_t launch_unit_rows(float *C, int K, int d, hipStream_t s) {
    if (K <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_unit_rows, dim3((unsigned)cdiv(K, 4)), dim3(256), 0, s, C, K, d);
    return hipGetLastError();
}

// The fit's stopping measure: part[block] = the largest sum_j (b - a)^2 (fp64)
// over the block's four rows (one wave per row), then one workgroup takes the
// maximum over the blocks (max is exact, so the order does not matter).
__global__ __launch_bounds__(256) void k_row_shift(const float *__restrict__ a, const float *__restrict__ b, int K,
                                                   int d, double *__restrict__ part) {
    __shared__ double wm[4];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int k = blockIdx.x * 4 + w;
    double q = 0.0;
    if (k < K) {
        for (int j = lane; j < d; j += 64) {
            const double t = (double)b[(size_t)k * d + j] - (double)a[(size_t)k * d + j];
            q += t * t;
        }
        for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off);
    }
    if (lane == 0) wm[w] = q;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmax(fmax(wm[0], wm[1]), fmax(wm[2], wm[3]));
}

__global__ __launch_bounds__(256) void k_max_of(const double *__restrict__ part, int n, double *__restrict__ out) {
    __shared__ double sm[256];
    double m = 0.0;
    for (int i = threadIdx.x; i < n; i += 256) m = fmax(m, part[i]);
    sm[threadIdx.x] = m;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) sm[threadIdx.x] = fmax(sm[threadIdx.x], sm[threadIdx.x + o]);
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = sm[0];
}

hipError_t launch_max_shift(const float *a, const float *b, int K, int d, double *part, double *shift, hipStream_t s) {
    const int nb = (int)cdiv(K, 4);
    hipLaunchKernelGGL(k_row_shift, dim3((unsigned)nb), dim3(256), 0, s, a, b, K, d, part);
    hipLaunchKernelGGL(k_max_of, dim3(1), dim3(256), 0, s, part, nb, shift);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
    const int64_t n = (int64_t)(bytes / 4);
    if (n <= 0) return hipSuccess;
    int64_t nb = cdiv(n, 256);
    if (nb > 4096) nb = 4096;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)nb), dim3(256), 0, s, (uint32_t *)p, n);
    return hipGetLastError();
}

template <int NV, int E, int RP = 1>
static hipError_t seg_launch(const float *X, int64_t N, int d, int K, const int32_t *ks, const int32_t *perm,
                             const double *xnorm64, double *sums, double *pfirst, double *plast, bool acc,
                             int32_t *offsets, float *C_out, hipStream_t s) {
    // rows in flight per wave: two batches of U (of row pairs with RP = 2:
    // 2 x 2 pairs keeps the paired kernel at 58 registers, eight waves per
    // SIMD, and measured as fast as 2 x 4 pairs at 2^20 and 2^24 rows)
    constexpr int U = RP == 2 ? 2 : (NV * E <= 8 ? 8 : 4);
    const int srows = seg_rows(N, d);
    const int64_t nseg = cdiv(N, srows);
    const dim3 grid((unsigned)cdiv(nseg, kSegWaves), (unsigned)cdiv(d, 64 / RP * E * NV));
    const dim3 block(kSegWaves * 64);
    if (xnorm64 != nullptr) {
        if (acc)
            hipLaunchKernelGGL((k_seg_reduce<NV, E, U, true, true, RP>), grid, block, 0, s, X, N, d, K, srows, ks,
                               perm, xnorm64, sums, pfirst, plast, offsets, C_out);
        else
            hipLaunchKernelGGL((k_seg_reduce<NV, E, U, true, false, RP>), grid, block, 0, s, X, N, d, K, srows, ks,
                               perm, xnorm64, sums, pfirst, plast, offsets, C_out);
    } else {
        if (acc)
            hipLaunchKernelGGL((k_seg_reduce<NV, E, U, false, true, RP>), grid, block, 0, s, X, N, d, K, srows, ks,
                               perm, xnorm64, sums, pfirst, plast, offsets, C_out);
        else
            hipLaunchKernelGGL((k_seg_reduce<NV, E, U, false, false, RP>), grid, block, 0, s, X, N, d, K, srows, ks,
                               perm, xnorm64, sums, pfirst, plast, offsets, C_out);
    }
    return hipGetLastError();
}

template <int E>
static hipError_t seg_launch_e(const float *X, int64_t N, int d, int K, const int32_t *ks, const int32_t *perm,
                               const double *xnorm64, double *sums, double *pfirst, double *plast, bool acc,
                               int32_t *offsets, float *C_out, hipStream_t s) {
    const int need = (int)cdiv(d, 64 * E);
#define FK_SEG(nv) seg_launch<nv, E>(X, N, d, K, ks, perm, xnorm64, sums, pfirst, plast, acc, offsets, C_out, s)
    if (need <= 1) return FK_SEG(1);
    if (need <= 2) return FK_SEG(2);
    if (need <= 3) return FK_SEG(3);
    return FK_SEG(4);
#undef FK_SEG
}

// Row loads of E floats per lane: float4 when a row spans at least 256
// floats, or (two rows per load, one per half-wave) between 65 and 128
// floats; float2 from 128 otherwise, scalar below (or when d is not a
// multiple); column blocks of up to 4 loads per lane, more blocks on
// blockIdx.y.
hipError_t launch_seg_reduce(const float *X, int64_t N, int d, int K, const int32_t *ks, const int32_t *perm,
                             const double *xnorm64, double *sums, double *pfirst, double *plast, bool acc,
                             int32_t *offsets, float *C_out, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    if (d % 4 == 0 && d > 64 && d <= 128)
        return seg_launch<1, 4, 2>(X, N, d, K, ks, perm, xnorm64, sums, pfirst, plast, acc, offsets, C_out, s);
    if (d % 4 == 0 && d >= 256)
        return seg_launch_e<4>(X, N, d, K, ks, perm, xnorm64, sums, pfirst, plast, acc, offsets, C_out, s);
    if (d % 2 == 0 && d >= 128)
        return seg_launch_e<2>(X, N, d, K, ks, perm, xnorm64, sums, pfirst, plast, acc, offsets, C_out, s);
    return seg_launch_e<1>(X, N, d, K, ks, perm, xnorm64, sums, pfirst, plast, acc, offsets, C_out, s);
}

hipError_t launch_seg_fixup(const int32_t *ks, const int32_t *offsets, int64_t N, int d, int K, const double *pfirst,
                            const double *plast, double *sums, bool acc, float *C_out, hipStream_t s) {
    const int srows = seg_rows(N, d);
    const int64_t nseg = cdiv(N, srows);
    if (nseg <= 1) return hipSuccess;
    hipLaunchKernelGGL(k_seg_fixup, dim3((unsigned)(nseg - 1)), dim3(kFixWaves * 64), 0, s, ks, offsets, N, d, K,
                       srows, pfirst, plast, sums, acc, C_out);
    return hipGetLastError();
}

hipError_t launch_count_accumulate(const int32_t *offsets, int K, int32_t *cnt, bool acc, hipStream_t s) {
    hipLaunchKernelGGL(k_count_acc, dim3((unsigned)cdiv(K, 256)), dim3(256), 0, s, offsets, K, cnt, acc);
    return hipGetLastError();
}

hipError_t launch_seg_finish(const int32_t *ks, const int32_t *offsets, int64_t N, int d, int K,
                             const double *pfirst, const double *plast, const float *C_prev, float *C_out,
                             int32_t *counts_out, hipStream_t s) {
    const int srows = seg_rows(N > 0 ? N : 1, d);
    const int64_t nbound = N > 0 ? cdiv(N, srows) - 1 : 0;
    int64_t g = cdiv(K, kFixWaves);
    if (g < cdiv(nbound, kFixWaves)) g = cdiv(nbound, kFixWaves);
    if (g > 2048) g = 2048;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(k_seg_finish, dim3((unsigned)g), dim3(kFixWaves * 64), 0, s, ks, offsets, N, d, K, srows,
                       nbound, pfirst, plast, C_prev, C_out, counts_out);
    return hipGetLastError();
}

hipError_t launch_finalize(const double *sums, const int32_t *cnt, const float *C_prev, int K, int d, float *C_out,
                           int32_t *counts_out, hipStream_t s) {
    const int64_t total = (int64_t)K * d;
    hipLaunchKernelGGL(k_finalize, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s, sums, cnt, C_prev, total, d,
                       C_out, counts_out);
    return hipGetLastError();
}

}  // namespace fk
