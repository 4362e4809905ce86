// Internal declarations shared by the HIP translation units of libfk.
// Kernels are written for gfx950 (CDNA4): wave64, fp32 MFMA, 160 KB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fk {

constexpr int kWave = 64;

// ---- FlashAssign geometry -------------------------------------------------
// A workgroup is WAVES waves.  Each wave owns PB blocks of 32 points and keeps
// their coordinates for one d-chunk of DP dims in VGPRs; all waves share
// centroid tiles of CB*32 rows x DP dims staged through LDS.
// Centroid counts are padded to a multiple of this (largest tile height).
constexpr int kCentroidPad = 256;

// ---- radix sort geometry --------------------------------------------------
constexpr int kSortWaves = 8;
constexpr int kSortThreads = kSortWaves * kWave;
// (a tile is kSortWaves waves of 4 to 16 rows of 64 keys, chosen from N)

// ---- segmented reduction geometry -----------------------------------------
constexpr int kSegWaves = 4;
// Sorted rows per wave segment, 64..2048: the longest segments (up to 2048
// rows) that still give at least 2048 waves up to d = 128 (fewer for longer
// rows, at least 1024), since every cluster that crosses a segment boundary
// leaves partial sums that the fix-up reads back.  At 16M rows that is 8192
// segments of 2048 rows; at 2^20 rows x 128, 512-row segments took the
// update 139 -> 130 us against the 128-row ones of a target of 8192 waves.
inline int seg_rows(int64_t N, int d) {
    int64_t target = ((int64_t)1 << 18) / (d > 128 ? d : 128);
    if (target < 1024) target = 1024;
    int r = 2048;
    while (r > 64 && N / r < target) r >>= 1;
    return r;
}
// An upper bound of cdiv(n, seg_rows(n, d)) over all n <= rows and all d (the
// count is not monotone in n, and longer rows only lengthen the segments):
// either the rows were shortened, and then n / (2r) < 8192, or they were not
// (2048-row segments), or they stopped at 64.
inline int64_t seg_count_bound(int64_t rows) {
    const int64_t a = (rows + 63) / 64;
    int64_t b = (rows + 2047) / 2048;
    if (b < 16385) b = 16385;
    return a < b ? a : b;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Which FlashAssign variant handles dimension d, and its geometry.
struct AssignShape {
    int DP;       // dims per chunk held in registers
    int PB;       // 32-point blocks per wave
    int CB;       // 32-centroid blocks per tile
    int nch;      // number of d-chunks
};
// The point-block geometry of the kernel variant used for d.
AssignShape assign_shape(int d);
// Split-bf16 scoring operands: Kpad rows (Kpad = K rounded up to
// kCentroidPad, rows past K are zero), each holding the bf16 high parts of
// dims [0, w) and then the bf16 low parts, w = split_width(d) (d rounded up to
// the FlashAssign chunk width).  cs == nullptr selects fp32 scoring.
struct SplitC {
    __bf16 *cs;
    int w;
};
int split_width(int d);

// ---- launchers (each returns the launch status) ---------------------------
hipError_t launch_row_norm64(const float *M, int64_t rows, int d, double *nrm, hipStream_t s);
// out64 may be null (only the fp32 normalised rows are written then)
hipError_t launch_normalize_rows(const float *M, int64_t rows, int d, const double *nrm, double *out64,
                                 float *out32, hipStream_t s);
// out[r, :] = M[idx[r], :] for r < rows
hipError_t launch_gather_rows(const float *M, const int32_t *idx, int64_t rows, int d, float *out, hipStream_t s);
// -||c||^2/2 (padded with -inf to kCentroidPad) and per-block maxima of the
// centroid norms; with split scoring also writes the split operands.
// ip: inner product (the scores are x.c: no -||c||^2/2 term)
hipError_t launch_centroid_prep(const float *C, int K, int d, float *ncn, float *cmax_part, int *nparts,
                                const SplitC &sc, bool ip, hipStream_t s);
hipError_t launch_prep_finish(const float *cmax_part, int nparts, float *scal, int32_t *counter,
                              hipStream_t s);
// Near-tie bookkeeping of FlashAssign (all in the workspace):
//   counters[0] = length of full_list (near ties whose third score is also in
//   the window), counters[1] = length of pair_list (near ties between two known
//   centroids, 3 ints per entry: point, k1, k2), counters[2] = length of
//   ovf_list (points rescored against all K).
struct NearTies {
    int32_t *full_list;
    float *full_thr;
    int32_t *pair_list;
    int32_t *counters;
    int32_t *cand;    // near_tie_cap(N) slots x 2 halves x 8 candidates
    int32_t *ccount;  // near_tie_cap(N) slots x 2 halves
    int32_t *ovf_list;
};
constexpr int kCandPerSlot = 16;
int64_t near_tie_cap(int64_t N);
hipError_t launch_flash_assign(const float *X, int64_t N, int d, const float *C, const float *ncn, int K,
                               const float *scal, const double *xnorm64, int32_t *a_out,
                               const NearTies &nt, const SplitC &sc, bool ip, hipStream_t s);
// Settles every listed near tie exactly (fp64 direct-difference distances).
// C_mfma is the centroid array the MFMA pass used (normalised for cosine); C32
// (L2) or C64 (cosine, normalised in fp64) is the one the distances use.
hipError_t launch_recheck(const float *X, int64_t N, int d, const float *C_mfma, const float *C32,
                          const double *C64, const float *ncn, int K, const float *scal, const double *xnorm64,
                          const NearTies &nt, const SplitC &sc, bool ip, int32_t *a_out, hipStream_t s);

// d1[p] = fp32 rounding of the fp64 direct-difference distance of point p to
// centroid a[p] (C32 for L2 and inner product, C64 normalised for cosine).
hipError_t launch_exact_d1(const float *X, int64_t N, int d, const float *C32, const double *C64,
                           const double *xnorm64, const int32_t *a, float *d1, bool ip, hipStream_t s);

// Radix sort of (key = assign[i], value = i), stable, no global atomics.  Writes the
// sorted keys and the permutation.  tmp* are N-sized scratch arrays.
size_t sort_scratch_bytes(int64_t N);
hipError_t launch_sort_by_key(const int32_t *keys, int64_t N, int K, int32_t *keys_sorted, int32_t *perm,
                              int32_t *tmp_keys, int32_t *tmp_vals, void *scratch, hipStream_t s);
hipError_t launch_offsets(const int32_t *keys_sorted, int64_t N, int K, int32_t *offsets, hipStream_t s);

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
// Device address of the static scratch of the allocation-free Lloyd
// iteration (FK_NOALLOC_SCRATCH_BYTES) on device `device`, which must be the
// current device: looked up once per device, then kept.
hipError_t noalloc_scratch(int device, void **ptr);
// The segmented reduction also writes the cluster offsets (first sorted row of
// each key, offsets[K] = N).  acc: rows fed in several batches, cluster sums
// added to sums (divided by launch_finalize at the end); otherwise the rows
// came in one batch and the reduction and its fix-up write the new centroids
// of the non-empty clusters to C_out, launch_seg_finish the rest.
hipError_t launch_seg_reduce(const float *X, int64_t N, int d, int K, const int32_t *keys_sorted, const int32_t *perm,
                             const double *xnorm64, double *sums, double *pfirst, double *plast, bool acc,
                             int32_t *offsets, float *C_out, hipStream_t s);
hipError_t launch_seg_fixup(const int32_t *keys_sorted, const int32_t *offsets, int64_t N, int d, int K,
                            const double *pfirst, const double *plast, double *sums, bool acc, float *C_out,
                            hipStream_t s);
hipError_t launch_count_accumulate(const int32_t *offsets, int K, int32_t *cnt, bool acc, hipStream_t s);
// Rows in one batch, after launch_seg_reduce: the crossing clusters' partials
// added and divided into C_out, counts from the offsets, and the previous
// centroid kept for an empty cluster (one launch)
hipError_t launch_seg_finish(const int32_t *keys_sorted, const int32_t *offsets, int64_t N, int d, int K,
                             const double *pfirst, const double *plast, const float *C_prev, float *C_out,
                             int32_t *counts_out, hipStream_t s);
// every row of C[K, d] divided by its L2 norm (fp64, a zero norm taken as 1):
// the spherical centroids
hipError_t launch_unit_rows(float *C, int K, int d, hipStream_t s);
// *shift = max_k sum_j (b[k,j] - a[k,j])^2 in fp64 (part: cdiv(K, 4) doubles)
hipError_t launch_max_shift(const float *a, const float *b, int K, int d, double *part, double *shift, hipStream_t s);
// counts from cnt, C_out = sums / count (C_prev for an empty cluster)
hipError_t launch_finalize(const double *sums, const int32_t *cnt, const float *C_prev, int K, int d, float *C_out,
                           int32_t *counts_out, hipStream_t s);

// k nearest neighbours (k <= kMaxKnn): the sweep cuts the database into
// slices (a second grid dimension) and writes, per query and slice, the L
// best MFMA scores and their rows (L = knn_list_len(k), a power of two above
// k) and the query's score error window; the finish step merges the slices,
// ranks the L best in fp64 when they must hold the exact top k, and lists the
// other queries (counters[0] = list length, zeroed by launch_prep_finish),
// which are then ranked against every row.
constexpr int kMaxKnn = 24;
constexpr int kKnnShort = 12;   // k <= 12: 16 candidates per query and slice, else 32
constexpr int kKnnMaxSlices = 64;
constexpr int kKnnSampleRows = 4096;  // rows per slice of the threshold sweep (a multiple of kCentroidPad)
constexpr int kKnnSampleSlices = 16;  // slices of the threshold sweep (at most)
int knn_list_len(int k);
struct KnnSlices {
    int slices, rows;  // rows per slice: a multiple of kCentroidPad
};
KnnSlices knn_slices(int64_t M, int64_t Ndb);
hipError_t launch_knn_sweep(const float *Q, int64_t M, int d, const float *DB, const float *ncn, int Ndb,
                            const float *scal, const double *qnorm64, const SplitC &sc, bool ip, int k,
                            int32_t *cand, float *score, float *win, float *tau, hipStream_t s);
// idx and dist rows are ld >= k entries long; entries k..ld-1 get -1 and +inf
hipError_t launch_knn_finish(const float *Q, int64_t M, int d, const float *DB32, const double *DB64,
                             const double *qnorm64, bool ip, const int32_t *cand, const float *score,
                             const float *win, int k, int ld, int Ndb, int32_t *list, int32_t *counters, int32_t *idx,
                             float *dist, hipStream_t s);

}  // namespace fk
