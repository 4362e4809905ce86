// FlashAssign for gfx950: the assignment step of an exact Lloyd iteration.
//
// The Flash-KMeans article (lumevalley.com, article 3696, section
// "FlashAssign: cutting the distance matrix into a pipeline") computes the
// distances of a block of points to every centroid on the spot and reduces
// them to an argmin at once, so the N x K distance matrix is never written and
// the IO is O(Nd + Kd).  This file does that on CDNA4:
//   * the score s_ik = ||c_k||^2 - 2 x_i.c_k is a dense contraction, so it runs
//     on the matrix cores: v_mfma_f32_32x32x2_f32 on the fp32 operands, or
//     (split scoring) v_mfma_f32_32x32x16_bf16 on bf16 high and low parts of
//     both operands, three products per fp32 product; the accumulator holds
//     x.c - ||c||^2/2 = (||x||^2 - D_ik) / 2, so the nearest centroid is the
//     largest accumulator;
//   * each wave keeps its points in VGPRs (for d > 128 they are streamed in
//     64-dim chunks, fetched a stage or two ahead); centroid tiles are staged
//     through LDS (double-buffered) and shared by the waves of a workgroup;
//   * the MFMA output puts one point per lane and 16 centroids per lane, so
//     the running top-3 is kept per lane with no cross-lane traffic; lanes l
//     and l^32 are merged once, after the last tile;
//   * exactness: the accumulator has a proven error bound e_i.  A point whose
//     top-2 gap is within 2 e_i is a near tie.  If its third score is more
//     than 2 e_i below the best, only the top two can win and k_recheck_pair
//     compares those two in fp64 by direct difference (the distance
//     definition); otherwise a second sweep (collect mode) gathers every
//     centroid within the window and k_recheck_cand compares those in fp64,
//     and a point with more than it can hold goes to k_recheck, which
//     rescores it against all K.
#include <type_traits>

#include "fk_internal.h"

namespace fk {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// candidates kept per point half-lane when the full near-tie list is collected
constexpr int kMaxCand = 8;

struct FlashArgs {
    const float *X;
    int64_t N;
    int d, nch;
    const float *C;
    const float *ncn;  // -||c||^2/2, padded with -inf
    int K, ntiles;
    const float *scal;
    const double *xnorm64;  // cosine: fp64 row norms of X, else null
    int32_t *a_out;
    int32_t *full_list;  // near ties with a third score within the window
    float *full_thr;     // their score threshold
    int32_t *pair_list;  // near ties settled by the top two: (point, k1, k2)
    int32_t *counters;   // [0] full, [1] pair, [2] overflow list lengths
    int32_t *cand;       // collect mode: candidates per (slot, half)
    int32_t *ccount;     // collect mode: candidate counts per (slot, half)
    int64_t cap_slots;   // collect mode: slots with candidate storage
    const __bf16 *Cs;    // split scoring: per centroid row, w bf16 high parts then
    int sw;              // w bf16 low parts (C - high, rounded); Kpad rows
    unsigned cs_bytes;   // size of the split copy
    int ip;              // inner product: scores are x.c (no -||c||^2/2 term)
    // top-L mode: the centroid rows are cut into knn_slices slices of
    // knn_rows rows (a multiple of the tile height); workgroup (x, y) sweeps
    // point block x against slice y and writes, per point and slice, its L
    // best scores and their indices, best first (lower index first on equal
    // scores), at ((point * knn_slices + y) * L); slice 0 also writes each
    // point's score error window
    int knn_slices, knn_rows, knn_tps;
    int32_t *knn_cand;
    float *knn_score;
    float *knn_win;
    // knn_tau: per point, a score at or below its L-th best over all rows
    // (the lists start from it instead of -inf), or null
    const float *knn_tau;
};

__device__ __forceinline__ uint64_t lanemask_lt() {
    const unsigned lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// ---------------------------------------------------------------------------
// Row norms in fp64, summed in increasing j with no fused multiply-add:
// nrm[r] = sqrt(sum_j M[r,j]^2), replaced by 1 when it is 0 (the zero-norm
// guard of the cosine metric, LEANN FlashLib guide, paragraph "distance
// metric").  One thread per row.
__global__ __launch_bounds__(256) void k_row_norm64(const float *__restrict__ M, int64_t rows, int d,
                                                    double *__restrict__ nrm) {
#pragma clang fp contract(off)
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const float *row = M + (size_t)r * d;
    double s = 0.0;
    for (int j = 0; j < d; ++j) {
        const double v = (double)row[j];
        s = s + v * v;
    }
    double n = sqrt(s);
    if (n == 0.0) n = 1.0;
    nrm[r] = n;
}

// out64[r,j] = M[r,j] / nrm[r] in fp64 (the normalised row), out32 its fp32
// rounding.
__global__ __launch_bounds__(256) void k_normalize_rows(const float *__restrict__ M, int64_t total, int d,
                                                        const double *__restrict__ nrm, double *__restrict__ out64,
                                                        float *__restrict__ out32) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= total) return;
    const int64_t r = q / d;
    const double v = (double)M[q] / nrm[r];
    if (out64 != nullptr) out64[q] = v;
    out32[q] = (float)v;
}

// out[r, :] = M[idx[r], :] (rows of d floats; indices checked by the caller).
__global__ __launch_bounds__(256) void k_gather_rows(const float *__restrict__ M, const int32_t *__restrict__ idx,
                                                     int64_t total, int d, float *__restrict__ out) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= total) return;
    const int64_t r = q / d;
    out[q] = M[(int64_t)idx[r] * d + (q - r * d)];
}

// Four floats per thread when d is a multiple of 4 (rows 16-byte aligned).
__global__ __launch_bounds__(256) void k_gather_rows4(const float4 *__restrict__ M, const int32_t *__restrict__ idx,
                                                      int64_t total4, int d4, float4 *__restrict__ out) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= total4) return;
    const int64_t r = q / d4;
    out[q] = M[(int64_t)idx[r] * d4 + (q - r * d4)];
}

hipError_t launch_gather_rows(const float *M, const int32_t *idx, int64_t rows, int d, float *out, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (d % 4 == 0) {
        const int64_t total4 = rows * (int64_t)(d / 4);
        hipLaunchKernelGGL(k_gather_rows4, dim3((unsigned)cdiv(total4, 256)), dim3(256), 0, s,
                           reinterpret_cast<const float4 *>(M), idx, total4, d / 4, reinterpret_cast<float4 *>(out));
    } else {
        const int64_t total = rows * (int64_t)d;
        hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s, M, idx, total, d, out);
    }
    return hipGetLastError();
}

// ncn[k] = -||c_k||^2 / 2 in fp32 for k < K, -inf for K <= k < Kpad (padded
// centroids then never win), and the largest ||c_k||^2 of the block.  One wave
// per centroid row.
__global__ __launch_bounds__(256) void k_centroid_prep(const float *__restrict__ C, int K, int Kpad, int d,
                                                       float *__restrict__ ncn, float *__restrict__ cmax_part,
                                                       __bf16 *__restrict__ cs, int w,
                                                       int ip) {
    __shared__ float wmax[3][4];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int k = blockIdx.x * 4 + wv;
    float cn = 0.f, dn = 0.f, rn = 0.f;
    if (k < K) {
        const float *row = C + (size_t)k * d;
        float s = 0.f;
        for (int j = lane; j < d; j += 64) {
            const float v = row[j];
            s = fmaf(v, v, s);
        }
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        cn = s;
    }
    if (cs != nullptr && k < Kpad) {
        // split scoring operands: hi = bf16(c) (round to nearest even), lo =
        // bf16(c - hi); the row holds hi of dims [0, w) then lo of dims
        // [0, w), zero past d and for k >= K.  dn and rn are the squared
        // norms of the remainders c - hi (exact in fp32) and c - hi - lo.
        __bf16 *out = cs + (size_t)k * 2 * w;
        auto split1 = [&](float v, __bf16 &hi, __bf16 &lo) {
            hi = (__bf16)v;
            const float dl = v - (float)hi;
            lo = (__bf16)dl;
            const float r = dl - (float)lo;
            dn = fmaf(dl, dl, dn);
            rn = fmaf(r, r, rn);
        };
        if ((d & 1) == 0) {
            // pairs of dims: one 8-byte load and two 4-byte stores per lane
            // (w is even, and so is every pair start below d)
            for (int j = 2 * lane; j < w; j += 128) {
                float2 v = make_float2(0.f, 0.f);
                if (k < K && j < d) v = *reinterpret_cast<const float2 *>(C + (size_t)k * d + j);
                __bf16 h2[2], l2[2];
                split1(v.x, h2[0], l2[0]);
                split1(v.y, h2[1], l2[1]);
                *reinterpret_cast<uint32_t *>(out + j) = __builtin_bit_cast(uint32_t, h2);
                *reinterpret_cast<uint32_t *>(out + w + j) = __builtin_bit_cast(uint32_t, l2);
            }
        } else {
            for (int j = lane; j < w; j += 64) {
                const float v = (k < K && j < d) ? C[(size_t)k * d + j] : 0.f;
                split1(v, out[j], out[w + j]);
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            dn += __shfl_xor(dn, off);
            rn += __shfl_xor(rn, off);
        }
    }
    if (lane == 0) {
        if (k < K)
            ncn[k] = ip ? 0.f : -0.5f * cn;
        else if (k < Kpad)
            ncn[k] = -INFINITY;
        wmax[0][wv] = cn;
        wmax[1][wv] = dn;
        wmax[2][wv] = rn;
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        const float *m = wmax[threadIdx.x];
        cmax_part[(size_t)blockIdx.x * 3 + threadIdx.x] = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
    }
}

// scal[0] = max_k ||c_k||^2, scal[1] = max_k ||c_k - hi_k||^2, scal[2] =
// max_k ||c_k - hi_k - lo_k||^2 (fp32; the last two are zero without split
// scoring); resets the three near-tie list counters.  One workgroup of 1024
// threads, eight partial rows in flight per thread (a k-NN database of a
// million rows leaves a quarter of a million partials).
__global__ __launch_bounds__(1024) void k_prep_finish(const float *__restrict__ cmax_part, int nparts,
                                                      float *__restrict__ scal, int32_t *__restrict__ counter) {
    constexpr int NT = 1024, U = 8;
    __shared__ float sm[3][NT];
    float m[3] = {0.f, 0.f, 0.f};
    int i = threadIdx.x;
    for (; i + (U - 1) * NT < nparts; i += U * NT) {
        float a[U][3];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < 3; ++c) a[u][c] = cmax_part[(size_t)(i + u * NT) * 3 + c];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < 3; ++c) m[c] = fmaxf(m[c], a[u][c]);
    }
    for (; i < nparts; i += NT)
        for (int c = 0; c < 3; ++c) m[c] = fmaxf(m[c], cmax_part[(size_t)i * 3 + c]);
    for (int c = 0; c < 3; ++c) sm[c][threadIdx.x] = m[c];
    __syncthreads();
    for (int o = NT / 2; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o)
            for (int c = 0; c < 3; ++c) sm[c][threadIdx.x] = fmaxf(sm[c][threadIdx.x], sm[c][threadIdx.x + o]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        scal[0] = sm[0][0];
        scal[1] = sm[1][0];
        scal[2] = sm[2][0];
        counter[0] = 0;
        counter[1] = 0;
        counter[2] = 0;
    }
}

// ---------------------------------------------------------------------------
// The FlashAssign kernel.
//
// DP: dims per chunk in VGPRs (multiple of 8); PB: 32-point blocks per wave;
// CB: 32-centroid blocks per tile.  nch d-chunks of DP dims cover d (padding
// is zero, which changes neither dots nor norms).  With nch == 1 a wave loads
// its points once; otherwise it reloads its chunk for every stage.
//
// MFMA operands (v_mfma_f32_32x32x2_f32, checked on gfx950): lane l gives
// A[l%32][l/32] and B[l/32][l%32]; D[i][j] sits in lane j + 32*((i/4)%2),
// register (i%4) + 4*(i/8).  A = centroid rows, B = points, so a lane holds
// one point and 16 centroids.  The two k-slots of each MFMA step take dims
// h*DP/2 + s (h = l/32), so a lane reads 4 consecutive floats of its row per
// ds_read_b128 and its points' coordinates are contiguous in memory.
//
// Error bound (why unflagged points are exact).  Let a_ik be the exact real
// value x_i.c_k - ||c_k||^2/2 from the fp32 inputs.  The fp32 ||c||^2 has
// relative error <= gamma_d, and the accumulator is a sum of d+1 terms
// (-||c||^2/2 and the d products) in which every term passes through at most
// d+2 roundings, so |acc - a| <= gamma_{d+3} (||c||^2 + ||x|| ||c||) with
// gamma_n = n u / (1 - n u), u = 2^-24.  With g = (d+4) u >= gamma_{d+3},
// M >= max ||c||^2 and the norms rounded up,
//     e_i = 1.0625 g (M + ||x_i|| sqrt(M))
// bounds the error of every accumulator of point i.  If best - second > 2 e_i
// the fp32 winner is the strict exact winner, with a margin (at least
// 0.125 e_i) far above the fp64 rounding of a direct-difference distance.
// Otherwise, if best - third > 2 e_i, every centroid but the top two is
// excluded with the same margin and the point goes on the pair list; else on
// the full list.  For cosine, the fp32 normalised rows differ from the fp64
// normalised ones by at most 3.1u relative, which moves a by at most
// 3.1u (||x|| ||c|| + ||c||^2); 8u is added to g for it.
// Tile slices of the collect sweep for a full list of nslots points.  The
// list's ng slot groups times s slices are the units that the persistent
// grid (grid workgroups) strides over.  A list that fills less than one
// round takes as many slices as the grid has room for.  A longer one would
// leave its last round mostly idle with one slice (1.3 rounds take two), so
// it is cut into the fewest slices whose estimated time -- rounds times the
// tiles a unit sweeps, plus one for its prologue -- is within 3 % of the
// least.  At most 64 slices and at most the tile count, and the candidate
// storage (cap_slots slots) must hold nslots * s lists; the count is
// rounded so that every slice has tiles.  The fp64 checks read it back from
// counters[3].
constexpr int kStagedMinList = 65536;  // listed points for the staged checks
__device__ __forceinline__ int collect_slices(int64_t nslots, int64_t cap_slots, int ntiles, int bm, int grid) {
    if (nslots <= 0) return 1;
    const int64_t ng = (nslots + bm - 1) / bm;
    const int64_t smax = min((int64_t)min(ntiles, 64), cap_slots / (ng * bm));
    if (smax < 1) return 1;
    int64_t s;
    if (ng <= grid) {
        s = min((int64_t)grid / ng, smax);
    } else {
        auto cost = [&](int64_t sl) { return ((ng * sl + grid - 1) / grid) * ((ntiles + sl - 1) / sl + 1); };
        int64_t cmin = cost(1);
        for (int64_t sl = 2; sl <= smax; ++sl) cmin = min(cmin, cost(sl));
        s = 1;
        while (s < smax && cost(s) * 100 > cmin * 103) ++s;
    }
    const int64_t tps = (ntiles + s - 1) / s;
    return (int)((ntiles + tps - 1) / tps);
}

template <int DP, int PB, int CB, int WAVES, int MINB, bool RES, bool VEC, bool COLLECT, bool SPLIT, int TL = 0>
__global__ __launch_bounds__(WAVES * 64, MINB) void k_flash_assign(const FlashArgs A) {
    // TL > 0: k-nearest-neighbour mode; every lane keeps its TL best scores
    // (and their indices) sorted, the two half-lanes of a point are merged at
    // the end and the point's TL best candidates are written out.
    static_assert(TL == 0 || (!COLLECT && (TL & (TL - 1)) == 0), "top-L mode: a power of two, no collect pass");
    constexpr int NT = WAVES * 64;
    constexpr int HALF = DP / 2;
    constexpr int ROWS = CB * 32;
    constexpr int LDR = DP + 4;  // padded fp32 LDS row: 8 consecutive lanes hit distinct 16-B bank groups
    constexpr int LDB = DP + 8;  // padded bf16 LDS row (split scoring), same property
    constexpr int Q4 = DP / 4;
    constexpr int NQ4 = ROWS * Q4;
    constexpr int PFN = SPLIT ? 1 : (NQ4 + NT - 1) / NT;
    constexpr int Q8 = DP / 8;
    constexpr int NQ8 = ROWS * Q8;
    constexpr int PFS = SPLIT ? (NQ8 + NT - 1) / NT : 1;
    constexpr int NS = DP / 16;           // split scoring: 16-dim MFMA steps per chunk
    constexpr int BM = WAVES * PB * 32;  // points per workgroup pass
    static_assert(HALF % 4 == 0, "DP must be a multiple of 8");
    static_assert(!SPLIT || DP % 16 == 0, "split scoring needs DP a multiple of 16");
    // Split scoring with resident points runs each tile in phases on one
    // accumulator: the two cross terms from zero, then -||c||^2/2 (its fp32
    // value, one add per score), then the hi.hi products.  Chunked points keep
    // the cross terms in a second accumulator instead (the phases would span
    // chunks).
    constexpr bool PHASED = SPLIT && RES;
    // Split scoring on streamed chunks (no candidate lists) sums all three
    // products in the one accumulator: every partial sum then holds up to
    // 3d + 1 terms, so the error bound takes (3d + 4) u in place of (d + 4) u
    // (the window is three times wider), and the 64 registers of a second
    // accumulator go, which leaves room for two waves per SIMD.
    constexpr bool ONEACC = SPLIT && !RES && TL == 0;
    // Streamed chunks fetch the next stage's points a stage ahead, except
    // beside 32-long candidate lists (no registers left for them there: the
    // points are loaded at the start of their own stage).
    constexpr bool PRE = !RES && TL <= 16;
    // top-L lists that may start from a threshold (the 16-long lists beside
    // streamed d-chunks never do: that sweep runs without the threshold pass)
    constexpr bool TAU = TL > 0 && (RES || TL > 16);
    // The phased kernel at DP = 128 moves each centroid stage into LDS with
    // buffer loads that write LDS themselves (no staging registers, which
    // the resident points need).  One such load of a wave fills 64
    // consecutive 16-byte LDS chunks (lane i the i-th); the padded rows
    // (DP + 8 bf16 = 17 chunks) are filled chunk by chunk, a row's pad chunk
    // with a copy of its first chunk (never read).
    constexpr bool DMA = PHASED && DP == 128;

    __shared__ __attribute__((aligned(16))) float sC[2][SPLIT ? 4 : ROWS * LDR];
    __shared__ __attribute__((aligned(16))) __bf16 sCh[2][SPLIT ? ROWS * LDB : 8];
    __shared__ __attribute__((aligned(16))) __bf16 sCl[2][SPLIT ? ROWS * LDB : 8];
    __shared__ __attribute__((aligned(16))) float sN[2][ROWS];

    const float *__restrict__ X = A.X;
    const float *__restrict__ C = A.C;
    const int d = A.d, K = A.K;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: a scalar
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int jl = lane & 31;

    // buffer resource of the split centroid copy (raw, byte-addressed,
    // loads past its end read zero)
    const __amdgpu_buffer_rsrc_t cs_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)A.Cs, (short)0, SPLIT ? (int)A.cs_bytes : 0, 0x00020000);

    // Assign mode: workgroup g takes points [g*BM, (g+1)*BM).  Collect mode:
    // the workgroups stride over (slot group, tile slice) units of the full
    // near-tie list: a short list is swept by several workgroups at once,
    // each over a slice of the centroid tiles with its own candidate lists
    // (collect_slices), instead of one workgroup walking all K.
    const int64_t nslots = COLLECT ? (int64_t)min((int64_t)A.counters[0], A.cap_slots) : A.N;
    const int64_t ngroups = COLLECT ? (nslots + BM - 1) / BM : 1;
    const int nsl = COLLECT ? collect_slices(nslots, A.cap_slots, A.ntiles, BM, gridDim.x) : 1;
    const int tps = COLLECT ? (A.ntiles + nsl - 1) / nsl : 0;
    if (COLLECT && blockIdx.x == 0 && tid == 0) A.counters[3] = nsl;  // for the fp64 check
    for (int64_t unit = COLLECT ? (int64_t)blockIdx.x : 0; unit < ngroups * nsl; unit += COLLECT ? gridDim.x : 1) {
        const int64_t grp = COLLECT ? unit / nsl : 0;
        const int slice = COLLECT ? (int)(unit % nsl) : 0;
        const int64_t sbase = ((COLLECT ? grp : (int64_t)blockIdx.x) * WAVES + wv) * (PB * 32);

        // global -> registers for one centroid stage (tile t, d-chunk ch)
        float4 pf[PFN];
        float4 pfh[PFS], pfl[PFS];
        float pn = 0.f;
        auto load_stage = [&](int t, int ch) {
            if constexpr (SPLIT) {
                // the split copy has Kpad zero-padded rows of sw >= DP * nch
                // dims, so a whole stage is in bounds.  Buffer loads: the
                // lane's byte offset in the tile stays in one VGPR per load
                // slot, the tile (and the low half) offsets are scalars.
                const unsigned tile_b = (unsigned)t * ROWS * (4u * A.sw) + ch * DP * 2u;
#pragma unroll
                for (int i = 0; i < PFS; ++i) {
                    const int q = tid + i * NT;
                    float4 vh = make_float4(0.f, 0.f, 0.f, 0.f), vl = vh;
                    if (NQ8 % NT == 0 || q < NQ8) {
                        const unsigned o = (unsigned)((q / Q8) * (4 * A.sw) + (q % Q8) * 16);
                        vh = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(cs_rsrc, o, tile_b, 0));
                        vl = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(cs_rsrc, o,
                                                                                              tile_b + 2u * A.sw, 0));
                    }
                    pfh[i] = vh;
                    pfl[i] = vl;
                }
            } else {
#pragma unroll
                for (int i = 0; i < PFN; ++i) {
                    const int q = tid + i * NT;
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (q < NQ4) {
                        const int row = q / Q4;
                        const int col = ch * DP + (q % Q4) * 4;
                        const int k = t * ROWS + row;
                        if (k < K) {
                            const float *src = C + (size_t)k * d + col;
                            if (VEC) {
                                if (col < d) v = *reinterpret_cast<const float4 *>(src);
                            } else {
                                if (col < d) v.x = src[0];
                                if (col + 1 < d) v.y = src[1];
                                if (col + 2 < d) v.z = src[2];
                                if (col + 3 < d) v.w = src[3];
                            }
                        }
                    }
                    pf[i] = v;
                }
            }
            if (ch == 0 && tid < ROWS) pn = A.ncn[t * ROWS + tid];
        };
        // global -> LDS buffer directly (DMA): stage t of the split copy and
        // of -||c||^2/2
        auto dma_to = [&](const __bf16 *cs, const float *ncn, __bf16 *dh, __bf16 *dl, float *dn, int t) {
            const __amdgpu_buffer_rsrc_t cs_rsrc =
                __builtin_amdgcn_make_buffer_rsrc((void *)cs, (short)0, (int)A.cs_bytes, 0x00020000);
            const __amdgpu_buffer_rsrc_t ncn_rsrc =
                __builtin_amdgcn_make_buffer_rsrc((void *)ncn, (short)0, A.ntiles * ROWS * 4, 0x00020000);
            constexpr int RCH = LDB / 8;    // 16-byte chunks per padded row
            constexpr int NINS = ROWS * RCH / 64;
            static_assert(!DMA || (ROWS * RCH) % 64 == 0, "whole wave loads per buffer");
            static_assert(!DMA || ROWS % 64 == 0, "whole wave loads of the norms");
            typedef __attribute__((address_space(3))) void *lds_ptr;
            const unsigned tile_b = (unsigned)t * ROWS * (4u * A.sw);
#pragma unroll
            for (int i = 0; i < (NINS + WAVES - 1) / WAVES; ++i) {
                const int j = wv + i * WAVES;  // wave-uniform
                if (j < NINS) {
                    const int q = j * 64 + lane;
                    const int row = q / RCH, c = q % RCH;
                    const unsigned o = (unsigned)row * (4u * A.sw) + (c < DP / 8 ? c : 0) * 16u;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(cs_rsrc, (lds_ptr)(dh + j * 512), 16, o, tile_b, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(cs_rsrc, (lds_ptr)(dl + j * 512), 16, o,
                                                             tile_b + 2u * A.sw, 0, 0);
                }
            }
            if (wv == WAVES - 1) {
#pragma unroll
                for (int j = 0; j < ROWS / 64; ++j)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ncn_rsrc, (lds_ptr)(dn + j * 64), 4, 4u * lane,
                                                             (unsigned)(t * ROWS + j * 64) * 4u, 0, 0);
            }
        };
        // registers -> LDS buffer
        auto store_stage = [&](int buf, int ch) {
            if constexpr (SPLIT) {
#pragma unroll
                for (int i = 0; i < PFS; ++i) {
                    const int q = tid + i * NT;
                    if (q < NQ8) {
                        const int o = (q / Q8) * LDB + (q % Q8) * 8;
                        *reinterpret_cast<float4 *>(&sCh[buf][o]) = pfh[i];
                        *reinterpret_cast<float4 *>(&sCl[buf][o]) = pfl[i];
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < PFN; ++i) {
                    const int q = tid + i * NT;
                    if (q < NQ4) *reinterpret_cast<float4 *>(&sC[buf][(q / Q4) * LDR + (q % Q4) * 4]) = pf[i];
                }
            }
            if (ch == 0 && tid < ROWS) sN[buf][tid] = pn;
        };

        float xr[PB][SPLIT ? 1 : HALF];
        v8bf xh[PB][SPLIT ? NS : 1], xl[PB][SPLIT ? NS : 1];
        // assign mode: running top-3 scores per point (b1 >= b2 >= b3) and the
        // indices of the first two.  collect mode: the listed point's
        // threshold and this half-lane's candidate count.
        float xn[PB], xsc[PB], b1[PB], b2[PB], b3[PB];
        // split scoring: squared norms of this half-lane's low parts and of
        // the remainders x - hi - lo (for the bound on the dropped terms)
        float xl2[PB], xr2[PB];
        int i1[PB], i2[PB];
        // top-L mode: sorted best-first scores and indices (lower index first
        // on equal scores)
        float bl[PB][TL > 0 ? TL : 1];
        int il[PB][TL > 0 ? TL : 1];
#pragma unroll
        for (int b = 0; b < PB; ++b)
#pragma unroll
            for (int j = 0; j < (TL > 0 ? TL : 1); ++j) {
                bl[b][j] = -INFINITY;
                il[b][j] = 0x7fffffff;
            }
        int64_t pt[PB];
        bool pv[PB];
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            const int64_t slot = sbase + b * 32 + jl;
            if (COLLECT) {
                pv[b] = slot < nslots;
                pt[b] = pv[b] ? A.full_list[slot] : 0;
                b1[b] = pv[b] ? A.full_thr[slot] : INFINITY;
            } else {
                pv[b] = slot < A.N;
                pt[b] = slot;
                b1[b] = -INFINITY;
            }
            xn[b] = 0.f;
            xl2[b] = 0.f;
            xr2[b] = 0.f;
            xsc[b] = (A.xnorm64 != nullptr && pv[b]) ? (float)(1.0 / A.xnorm64[pt[b]]) : 1.f;
            b2[b] = -INFINITY;
            b3[b] = -INFINITY;
            i1[b] = 0;
            i2[b] = 0;
        }
        if constexpr (TAU) {
            // a lower bound of the point's L-th best score: a row scoring at
            // or below it cannot be among the L best, so the lists start
            // full of it (index 0x7fffffff: no row)
            if (A.knn_tau != nullptr) {
#pragma unroll
                for (int b = 0; b < PB; ++b) {
                    const float t0 = pv[b] ? A.knn_tau[pt[b]] : -INFINITY;
#pragma unroll
                    for (int j = 0; j < TL; ++j) bl[b][j] = t0;
                }
            }
        }
        // This wave's points in registers.  Slot q (of HALF per point block
        // and lane) holds, for fp32 scoring, dim ch*DP + h*HALF + q; for split
        // scoring, dim ch*DP + 16(q/8) + 8h + q%8 of MFMA step q/8, as a bf16
        // high part (the round-to-nearest value) and a bf16 low part (the
        // rounded remainder).
        // fetch_x4: the fp32 values of slots q..q+3 (zero outside the data)
        auto fetch_x4 = [&](int ch, int b, int q, float *v) {
            const int col0 = SPLIT ? ch * DP + 16 * (q / 8) + 8 * h + (q % 8) : ch * DP + h * HALF + q;
            const float *src = X + (size_t)pt[b] * d + col0;
            if (VEC) {
                float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
                if (pv[b] && col0 < d) u = *reinterpret_cast<const float4 *>(src);
                v[0] = u.x;
                v[1] = u.y;
                v[2] = u.z;
                v[3] = u.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (pv[b] && col0 + e < d) ? src[e] : 0.f;
            }
        };
        // put_x: slot q's value into the MFMA operand registers (scaled for
        // cosine; streamed chunks multiply by xsc, which is 1 otherwise, to
        // save the select on every stage) and,
        // with add_norm (a compile-time flag: std::true_type or
        // std::false_type), into the point's squared norms
        auto put_x = [&](int b, int q, float v, auto add_norm_c, float &nacc, float &lacc, float &racc) {
            constexpr bool add_norm = decltype(add_norm_c)::value;
            const float xv = (RES && A.xnorm64 == nullptr) ? v : v * xsc[b];
            if constexpr (SPLIT) {
                const __bf16 hi = (__bf16)xv;
                const float dl = xv - (float)hi;  // exact
                const __bf16 lo = (__bf16)dl;
                xh[b][q / 8][q % 8] = hi;
                xl[b][q / 8][q % 8] = lo;
                if constexpr (add_norm) {
                    const float lf = (float)lo, r = dl - lf;  // exact
                    nacc = fmaf(xv, xv, nacc);
                    lacc = fmaf(lf, lf, lacc);
                    racc = fmaf(r, r, racc);
                }
            } else {
                xr[b][q] = xv;
                if constexpr (add_norm) nacc = fmaf(xv, xv, nacc);
            }
        };
        // resident split points: the same values with unconditional loads
        // (the row index and column clamped into X, out-of-range values
        // zeroed by a select), so that no load sits in a branch of its own
        auto fetch_x4_nb = [&](int b, int q, float *v) {
            const int col0 = 16 * (q / 8) + 8 * h + (q % 8);
            const float *row = X + (size_t)(pv[b] ? pt[b] : 0) * d;
            if constexpr (VEC) {
                const bool ok = pv[b] && col0 < d;
                const float4 u = *reinterpret_cast<const float4 *>(row + (col0 < d ? col0 : d - 4));
                v[0] = ok ? u.x : 0.f;
                v[1] = ok ? u.y : 0.f;
                v[2] = ok ? u.z : 0.f;
                v[3] = ok ? u.w : 0.f;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float t = row[col0 + e < d ? col0 + e : d - 1];
                    v[e] = (pv[b] && col0 + e < d) ? t : 0.f;
                }
            }
        };
        auto load_x = [&](int ch, auto add_norm) {
            if constexpr (SPLIT && RES && !COLLECT && TL == 0) {
                // (the assignment sweep; the window and top-L passes keep the
                // form below, which spills less there)
                // Groups of 8 slots go through a ring of LDEP register
                // groups: group g + LDEP - 1 is loaded while group g is split,
                // and the scheduling barriers keep the compiler from hoisting
                // every load of the rows ahead of the splits (it would hold
                // all the fp32 values and the bf16 halves live at once, and
                // spill).
                constexpr int NG = HALF / 8, TOT = PB * NG, LDEP = 4;
                float rq[LDEP][8];
#pragma unroll
                for (int g = 0; g < LDEP - 1; ++g)
                    if (g < TOT) {
                        fetch_x4_nb(g / NG, (g % NG) * 8, rq[g]);
                        fetch_x4_nb(g / NG, (g % NG) * 8 + 4, rq[g] + 4);
                    }
#pragma unroll
                for (int g = 0; g < TOT; ++g) {
                    const int gn = g + LDEP - 1;
                    if (gn < TOT) {
                        fetch_x4_nb(gn / NG, (gn % NG) * 8, rq[gn % LDEP]);
                        fetch_x4_nb(gn / NG, (gn % NG) * 8 + 4, rq[gn % LDEP] + 4);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    const int b = g / NG, q = (g % NG) * 8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) put_x(b, q + e, rq[g % LDEP][e], add_norm, xn[b], xl2[b], xr2[b]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                return;
            }
#pragma unroll
            for (int b = 0; b < PB; ++b) {
                float nacc = xn[b], lacc = xl2[b], racc = xr2[b];
#pragma unroll
                for (int q = 0; q < HALF; q += 8) {
                    float v[8];
                    fetch_x4(ch, b, q, v);
                    fetch_x4(ch, b, q + 4, v + 4);
#pragma unroll
                    for (int e = 0; e < 8; ++e) put_x(b, q + e, v[e], add_norm, nacc, lacc, racc);
                    // split scoring: keep the scheduler from hoisting every
                    // load of the row ahead of the splits (it would hold all
                    // the fp32 values and the bf16 halves live at once)
                    if constexpr (SPLIT) __builtin_amdgcn_sched_barrier(0);
                }
                xn[b] = nacc;
                xl2[b] = lacc;
                xr2[b] = racc;
            }
        };
        // streamed chunks: the next stage's point values, fetched a whole
        // stage ahead and put into the operand registers at its end
        float xraw[PB][PRE ? HALF : 4];
        auto fetch_next = [&](int ch) {
#pragma unroll
            for (int b = 0; b < PB; ++b)
#pragma unroll
                for (int q = 0; q < HALF; q += 4) fetch_x4(ch, b, q, &xraw[b][q]);
        };
        auto put_next = [&](auto add_norm) {
#pragma unroll
            for (int b = 0; b < PB; ++b) {
                float nacc = xn[b], lacc = xl2[b], racc = xr2[b];
#pragma unroll
                for (int q = 0; q < HALF; ++q) put_x(b, q, xraw[b][q], add_norm, nacc, lacc, racc);
                xn[b] = nacc;
                xl2[b] = lacc;
                xr2[b] = racc;
            }
        };

        // Per-point bound of the accumulator error (see the derivation above
        // the kernel): on return xn[b] holds ||x||^2 (both half-lanes) and
        // xl2[b] holds 2 e_i, the near-tie window.
        const float u = 5.9604645e-8f;
        // roundings per accumulator path: at most d + 3 for -||c||^2/2 and
        // the fp32 (or hi.hi) products; the split cross terms come first,
        // their absolute values sum to at most 2 (1 + 2^-8) 2^-9 ||x|| ||c||
        // < 0.004 ||x|| ||c||, and passing through at most 3d + 1 roundings
        // they add less than 0.004 (3d + 1) u ||x|| ||c||, which the 1.0625
        // factor covers
        const float g = (float)(ONEACC ? 3 * d + 4 : d + 4) * u + (A.xnorm64 != nullptr ? 8.f * u : 0.f);
        auto point_bounds = [&]() {
            const float M = A.scal[0] * (1.f + g);
            const float sqM = sqrtf(M) * (1.f + 2.f * u);
#pragma unroll
            for (int b = 0; b < PB; ++b) {
                const float xnt = xn[b] + __shfl_xor(xn[b], 32);
                const float xnorm = sqrtf(xnt * (1.f + g)) * (1.f + 2.f * u);
                // split scoring computes hx.hc + hx.lc + lx.hc; with the
                // remainders dx = x - hx, rx = x - hx - lx (and likewise for c)
                // the dropped part of x.c is exactly lx.dc + rx.c + hx.rc, at
                // most ||lx|| max||dc|| + ||rx|| max||c|| + ||hx|| max||rc|| by
                // Cauchy-Schwarz (||hx|| <= (1 + 2^-8) ||x||).  The norms are
                // fp32 sums of squares: relative error far below the 1% added,
                // and a square under 2^-126 that is flushed to zero loses at
                // most sqrt(d) * 1.1e-19 of a norm, which is added back.
                float drop = 0.f;
                if constexpr (SPLIT) {
                    const float uf = 1.1e-19f * sqrtf((float)d);
                    const float l2 = xl2[b] + __shfl_xor(xl2[b], 32);
                    const float r2 = xr2[b] + __shfl_xor(xr2[b], 32);
                    drop = 1.01f * ((sqrtf(l2) + uf) * (sqrtf(A.scal[1]) + uf) + (sqrtf(r2) + uf) * sqM +
                                    1.004f * xnorm * (sqrtf(A.scal[2]) + uf));
                }
                // the last term covers flushed denormal operands
                // inner product: no -||c||^2/2 term, so no M term
                xl2[b] = 2.f * (1.0625f * (g * ((A.ip ? 0.f : M) + xnorm * sqM) + drop) +
                                7.6e-37f * (float)d * (sqM + xnorm) + 1e-30f);
                xn[b] = xnt;
            }
        };

        // acc: -||c||^2/2 + the fp32 (or hi.hi) products; split scoring keeps
        // the two small cross terms in a second accumulator (acl) that is
        // added once per tile, so that they pass through few roundings
        // phased split scoring computes its centroid blocks one after another
        // (each with its epilogue), so one accumulator per point block serves
        v16f acc[PB][PHASED ? 1 : CB];
        v16f acl[PB][SPLIT && !PHASED && !ONEACC ? CB : 1];

        // Fold one 32-centroid block of scores (a) of point block b, centroid
        // indices kb + 8(r/4) + r%4, into this lane's state.
        auto epilogue = [&](const v16f &a, int b, int kb) {
            if constexpr (TL > 0) {
                // take the group's values in decreasing order (the lowest
                // index first among equals) while any lane of the wave still
                // has one above its L-th best, and insert each by bubbling
                float v[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) v[r] = a[r];
                auto vmax = [&]() {
                    float m = v[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) m = fmaxf(m, v[r]);
                    return m;
                };
                float m = vmax();
                while (__ballot(m > bl[b][TL - 1]) != 0ull) {
                    if (m > bl[b][TL - 1]) {
                        int rs = 15;
#pragma unroll
                        for (int r = 15; r >= 0; --r) rs = (v[r] == m) ? r : rs;
                        const int sk = kb + 8 * (rs >> 2) + (rs & 3);
                        // m goes to the first place j with m > bl[j] (a
                        // suffix of the sorted list): a place past it takes
                        // the entry before it, the places before it keep
                        // theirs -- for the scores, the median of the entry
                        // before, the entry and m (v_med3_f32)
                        float pv = 0.f;
                        int pk = 0;
                        bool pc = false;
#pragma unroll
                        for (int j = 0; j < TL; ++j) {
                            const float ov = bl[b][j];
                            const int ok = il[b][j];
                            const bool c = m > ov;
                            bl[b][j] = j == 0 ? (c ? m : ov) : __builtin_amdgcn_fmed3f(pv, ov, m);
                            il[b][j] = pc ? pk : (c ? sk : ok);
                            pv = ov;
                            pk = ok;
                            pc = c;
                        }
#pragma unroll
                        for (int r = 0; r < 16; ++r) v[r] = (r == rs) ? -INFINITY : v[r];
                        m = vmax();
                    }
                }
                return;
            }
            // A value changes this lane's state only if it beats the third
            // best (top-3) or reaches the threshold (collect).  Late in the
            // sweep most 16-value groups change no lane; a lane (and then a
            // value) that changes nothing sits out with its execution bit
            // off: the work is skipped when no lane of the wave needs it, and
            // idle lanes draw less power when some do (the matrix cores run
            // near the chip's power limit here).
            bool any = false;
#pragma unroll
            for (int r = 0; r < 16; ++r) any |= COLLECT ? (a[r] >= b1[b]) : (a[r] > b3[b]);
            if (!any) return;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float v = a[r];
                const int k = kb + 8 * (r >> 2) + (r & 3);
                if (COLLECT) {
                    // every centroid within the window may win
                    if (v >= b1[b]) {
                        if (i1[b] < kMaxCand)
                            A.cand[(((sbase + b * 32 + jl) * nsl + slice) * 2 + h) * kMaxCand + i1[b]] = k;
                        ++i1[b];
                    }
                } else if (v > b3[b]) {
                    // insert v into the sorted top-3 with medians of three
                    // (v_med3_f32); a strict '>' keeps the lower index first on
                    // equal scores (k increases per lane); a value at or below
                    // the third best would leave the state as it is
                    const bool c1 = v > b1[b];
                    const bool c2 = v > b2[b];
                    const int t2 = c2 ? k : i2[b];
                    i2[b] = c1 ? i1[b] : t2;
                    i1[b] = c1 ? k : i1[b];
                    b3[b] = __builtin_amdgcn_fmed3f(b2[b], b3[b], v);
                    b2[b] = __builtin_amdgcn_fmed3f(b1[b], b2[b], v);
                    b1[b] = c1 ? v : b1[b];
                }
            }
        };
        const int cnch = RES ? 1 : A.nch;
        // the tiles this workgroup sweeps: all, or its slice (top-L mode,
        // collect mode)
        const int tb = TL > 0 ? (int)blockIdx.y * A.knn_tps : COLLECT ? slice * tps : 0;
        const int te = TL > 0 ? min(A.ntiles, tb + A.knn_tps) : COLLECT ? min(A.ntiles, tb + tps) : A.ntiles;
        const int nst = (te - tb) * cnch;
        if (RES || PRE) load_x(0, std::true_type{});
        if (RES) {
            if (!COLLECT) point_bounds();
            if constexpr (PHASED) {
                // the split points are packed into their MFMA operand
                // registers here (left to itself the compiler would pack them
                // after the first stage's loads and spill the halves)
#pragma unroll
                for (int b = 0; b < PB; ++b)
#pragma unroll
                    for (int st = 0; st < NS; ++st) asm volatile("" : "+v"(xh[b][st]), "+v"(xl[b][st]));
            }
        }
        if constexpr (DMA) {
            dma_to(A.Cs, A.ncn, sCh[0], sCl[0], sN[0], tb);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else {
            load_stage(tb, 0);
            store_stage(0, 0);
        }
        __syncthreads();

        int t = tb, ch = 0;
        for (int st = 0; st < nst; ++st) {
            const int buf = st & 1;
            int nt = t, nc = ch + 1;
            if (nc == cnch) {
                nc = 0;
                nt = t + 1;
            }
            const bool more = st + 1 < nst;
            // streamed chunks: the next stage's points are fetched with the
            // next centroid stage, a whole stage before they are used (beside
            // 32-long lists: this stage's points, loaded now)
            if constexpr (PRE) {
                if (more) fetch_next(nc);
            } else if constexpr (!RES) {
                if (t == tb)
                    load_x(ch, std::true_type{});
                else
                    load_x(ch, std::false_type{});
            }
            if constexpr (!DMA) {
                if (more) load_stage(nt, nc);
            }

            if constexpr (!PHASED) {
              if (ch == 0) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 nv = *reinterpret_cast<const float4 *>(&sN[buf][cb * 32 + 8 * q + 4 * h]);
#pragma unroll
                        for (int b = 0; b < PB; ++b) {
                            acc[b][cb][4 * q + 0] = nv.x;
                            acc[b][cb][4 * q + 1] = nv.y;
                            acc[b][cb][4 * q + 2] = nv.z;
                            acc[b][cb][4 * q + 3] = nv.w;
                            if constexpr (SPLIT && !ONEACC)
                                for (int e = 0; e < 4; ++e) acl[b][cb][4 * q + e] = 0.f;
                        }
                    }
                }
              }
            }

            if constexpr (PHASED) {
            // The phased stage reads its LDS buffer (rh, rl, rn) and, with
            // DMA, first sends the next stage into the other one (wh, wl,
            // wn).  Both come in as restrict pointers, one inlined copy per
            // buffer: the compiler then knows that this stage's LDS reads do
            // not touch what the in-flight loads write, and does not make
            // them wait for those loads.
            auto phased = [&](const __bf16 *__restrict__ rh, const __bf16 *__restrict__ rl,
                              const float *__restrict__ rn, __bf16 *__restrict__ wh, __bf16 *__restrict__ wl,
                              float *__restrict__ wn, const __bf16 *__restrict__ cs,
                              const float *__restrict__ ncn) {
                // into the other buffer, which no wave reads in this stage
                if (DMA && more) dma_to(cs, ncn, wh, wl, wn, nt);
                const __bf16 *sh = rh + jl * LDB + 8 * h;
                const __bf16 *sl = rl + jl * LDB + 8 * h;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    // phase 1: lo.hi + hi.lo, from zero; each step's LDS
                    // operands are read one step ahead.  The wave issuing
                    // products takes priority over the other wave of its SIMD
                    // (which may be in its epilogue) until its block is done.
                    // The high parts read here are kept for phase 3 (ahs).
                    __builtin_amdgcn_s_setprio(1);
                    v8bf ahs[NS];
                    v8bf ah = *reinterpret_cast<const v8bf *>(sh + cb * 32 * LDB);
                    v8bf al = *reinterpret_cast<const v8bf *>(sl + cb * 32 * LDB);
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        ahs[st] = ah;
                        v8bf ahn = ah, aln = al;
                        if (st + 1 < NS) {
                            ahn = *reinterpret_cast<const v8bf *>(sh + cb * 32 * LDB + 16 * (st + 1));
                            aln = *reinterpret_cast<const v8bf *>(sl + cb * 32 * LDB + 16 * (st + 1));
                        }
#pragma unroll
                        for (int b = 0; b < PB; ++b) {
                            const v16f c0 = {};
                            acc[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xh[b][st], st == 0 ? c0 : acc[b][0],
                                                                                0, 0, 0);
                            acc[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xl[b][st], acc[b][0], 0, 0, 0);
                        }
                        ah = ahn;
                        al = aln;
                    }
                    // phase 2: + -||c||^2/2 (fp32) of this lane's 16 centroid rows
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 nv = *reinterpret_cast<const float4 *>(rn + cb * 32 + 8 * q + 4 * h);
#pragma unroll
                        for (int b = 0; b < PB; ++b) {
                            acc[b][0][4 * q + 0] += nv.x;
                            acc[b][0][4 * q + 1] += nv.y;
                            acc[b][0][4 * q + 2] += nv.z;
                            acc[b][0][4 * q + 3] += nv.w;
                        }
                    }
                    // phase 3: hi.hi, on the high parts phase 1 read (held in
                    // registers: reading them from LDS again measured 1 %
                    // slower at 16M x 128, K = 32768)
#pragma unroll
                    for (int st = 0; st < NS; ++st)
#pragma unroll
                        for (int b = 0; b < PB; ++b)
                            acc[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahs[st], xh[b][st], acc[b][0], 0, 0, 0);
                    __builtin_amdgcn_s_setprio(0);
#pragma unroll
                    for (int b = 0; b < PB; ++b) epilogue(acc[b][0], b, t * ROWS + cb * 32 + 4 * h);
                    // the next stage goes to the other LDS buffer (which no
                    // wave reads during this tile) once the first block is
                    // done, so the prefetch registers are free for the rest
                    if (!DMA && CB > 1 && cb == 0 && more) store_stage(buf ^ 1, nc);
                }
            };
                if (buf == 0)
                    phased(sCh[0], sCl[0], sN[0], sCh[1], sCl[1], sN[1], A.Cs, A.ncn);
                else
                    phased(sCh[1], sCl[1], sN[1], sCh[0], sCl[0], sN[0], A.Cs, A.ncn);
            } else if constexpr (ONEACC) {
                // x.c ~ hi.lo + lo.hi + hi.hi, one 32-centroid block after
                // another (only one block's operands live at a time)
                const __bf16 *sh = &sCh[buf][jl * LDB + 8 * h];
                const __bf16 *sl = &sCl[buf][jl * LDB + 8 * h];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
                    for (int st = 0; st < NS; ++st) {
                        const v8bf ah = *reinterpret_cast<const v8bf *>(sh + cb * 32 * LDB + 16 * st);
                        const v8bf al = *reinterpret_cast<const v8bf *>(sl + cb * 32 * LDB + 16 * st);
#pragma unroll
                        for (int b = 0; b < PB; ++b) {
                            acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xh[b][st], acc[b][cb], 0, 0, 0);
                            acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xl[b][st], acc[b][cb], 0, 0, 0);
                            acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xh[b][st], acc[b][cb], 0, 0, 0);
                        }
                    }
                }
            } else if constexpr (SPLIT) {
                // x.c ~ hi.hi + (hi.lo + lo.hi)
                const __bf16 *sh = &sCh[buf][jl * LDB + 8 * h];
                const __bf16 *sl = &sCl[buf][jl * LDB + 8 * h];
#pragma unroll
                for (int st = 0; st < NS; ++st) {
                    v8bf ah[CB], al[CB];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        ah[cb] = *reinterpret_cast<const v8bf *>(sh + cb * 32 * LDB + 16 * st);
                        al[cb] = *reinterpret_cast<const v8bf *>(sl + cb * 32 * LDB + 16 * st);
                    }
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
                        for (int b = 0; b < PB; ++b) {
                            acl[b][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[cb], xh[b][st], acl[b][cb], 0, 0, 0);
                            acl[b][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[cb], xl[b][st], acl[b][cb], 0, 0, 0);
                            acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[cb], xh[b][st], acc[b][cb], 0, 0, 0);
                        }
                    }
                }
            } else {
                const float *sc = &sC[buf][jl * LDR + h * HALF];
                __builtin_amdgcn_s_setprio(1);  // as above: products first
#pragma unroll
                for (int s = 0; s < HALF; s += 4) {
                    float4 av[CB];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) av[cb] = *reinterpret_cast<const float4 *>(sc + cb * 32 * LDR + s);
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
                        for (int b = 0; b < PB; ++b) {
                            acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[cb].x, xr[b][s + 0], acc[b][cb], 0, 0, 0);
                            acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[cb].y, xr[b][s + 1], acc[b][cb], 0, 0, 0);
                            acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[cb].z, xr[b][s + 2], acc[b][cb], 0, 0, 0);
                            acc[b][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[cb].w, xr[b][s + 3], acc[b][cb], 0, 0, 0);
                        }
                    }
                }
                __builtin_amdgcn_s_setprio(0);
            }

            if constexpr (!PHASED) {
                if (ch == cnch - 1) {
#pragma unroll
                    for (int b = 0; b < PB; ++b) {
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb) {
                            if constexpr (SPLIT && !ONEACC) acc[b][cb] += acl[b][cb];
                            epilogue(acc[b][cb], b, t * ROWS + cb * 32 + 4 * h);
                        }
                    }
                }
            }
            if (!DMA && !(PHASED && CB > 1) && more) store_stage(buf ^ 1, nc);
            if constexpr (PRE) {
                if (more) {
                    // after this stage's products: the wait for the fetched
                    // values must not move ahead of them
                    __builtin_amdgcn_sched_barrier(0);
                    if (nt == tb)
                        put_next(std::true_type{});
                    else
                        put_next(std::false_type{});
                }
            }
            // (the next stage's LDS loads have landed once vmcnt is zero)
            if constexpr (DMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            t = nt;
            ch = nc;
        }

        if (COLLECT) {
#pragma unroll
            for (int b = 0; b < PB; ++b)
                if (pv[b]) A.ccount[((sbase + b * 32 + jl) * nsl + slice) * 2 + h] = i1[b];
            continue;
        }

        if (!RES) point_bounds();
        if constexpr (TL > 0) {
#pragma unroll
            for (int b = 0; b < PB; ++b) {
                // bitonic merge with the other half-lane's list (reversed):
                // the larger of each pair forms the top L, then TL/2, ...
                // sorting steps; "larger" = higher score, lower index on ties
                float mv[TL];
                int mi[TL];
#pragma unroll
                for (int j = 0; j < TL; ++j) {
                    const float ov = __shfl_xor(bl[b][TL - 1 - j], 32);
                    const int oi = __shfl_xor(il[b][TL - 1 - j], 32);
                    const bool own = (bl[b][j] > ov) || (bl[b][j] == ov && il[b][j] < oi);
                    mv[j] = own ? bl[b][j] : ov;
                    mi[j] = own ? il[b][j] : oi;
                }
#pragma unroll
                for (int w = TL / 2; w > 0; w >>= 1) {
#pragma unroll
                    for (int j = 0; j < TL; ++j) {
                        if ((j & w) == 0) {
                            const int q = j + w;
                            const bool keep = (mv[j] > mv[q]) || (mv[j] == mv[q] && mi[j] < mi[q]);
                            const float hv = keep ? mv[j] : mv[q], lv = keep ? mv[q] : mv[j];
                            const int hi_ = keep ? mi[j] : mi[q], li = keep ? mi[q] : mi[j];
                            mv[j] = hv;
                            mi[j] = hi_;
                            mv[q] = lv;
                            mi[q] = li;
                        }
                    }
                }
                const int64_t p = sbase + b * 32 + jl;
                if (h == 0 && p < A.N) {
                    const size_t o = ((size_t)p * A.knn_slices + blockIdx.y) * TL;
#pragma unroll
                    for (int j = 0; j < TL; j += 4) {
                        *reinterpret_cast<int4 *>(A.knn_cand + o + j) = make_int4(mi[j], mi[j + 1], mi[j + 2], mi[j + 3]);
                        *reinterpret_cast<float4 *>(A.knn_score + o + j) =
                            make_float4(mv[j], mv[j + 1], mv[j + 2], mv[j + 3]);
                    }
                    if (blockIdx.y == 0) A.knn_win[p] = xl2[b];
                }
            }
            continue;
        }
        // merge the two half-waves (same point, the other 16 centroids of each
        // 32-block): larger score first, lower index first on equal scores
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            const float o1 = __shfl_xor(b1[b], 32);
            const float o2 = __shfl_xor(b2[b], 32);
            const float o3 = __shfl_xor(b3[b], 32);
            const int oi1 = __shfl_xor(i1[b], 32);
            const int oi2 = __shfl_xor(i2[b], 32);
            // W = the list whose head wins, L = the other
            const bool take = (o1 > b1[b]) || (o1 == b1[b] && oi1 < i1[b]);
            const float w1 = take ? o1 : b1[b], w2 = take ? o2 : b2[b], w3 = take ? o3 : b3[b];
            const int wi1 = take ? oi1 : i1[b], wi2 = take ? oi2 : i2[b];
            const float l1 = take ? b1[b] : o1, l2 = take ? b2[b] : o2;
            const int li1 = take ? i1[b] : oi1;
            const bool wsec = (w2 > l1) || (w2 == l1 && wi2 < li1);
            const float s2 = wsec ? w2 : l1;
            const int si2 = wsec ? wi2 : li1;
            const float s3 = wsec ? fmaxf(w3, l1) : fmaxf(w2, l2);

            const float e2 = xl2[b];
            const int64_t p = sbase + b * 32 + jl;
            const bool valid = (h == 0) && p < A.N;
            // near tie: the exact winner is not certain
            const bool flagged = !((w1 - s2) > e2);
            // only the top two can win: every other score is more than 2e below
            const bool pair = flagged && ((w1 - s3) > e2);
            const bool full = flagged && !pair;
            if (valid) A.a_out[p] = wi1;
            const uint64_t lt = lanemask_lt();
            const uint64_t mp = __ballot(valid && pair);
            if (mp != 0ull) {
                const int leader = __ffsll((unsigned long long)mp) - 1;
                int base = 0;
                if (lane == leader) base = atomicAdd(&A.counters[1], __popcll(mp));
                base = __shfl(base, leader);
                if (valid && pair) {
                    int32_t *e = A.pair_list + 3 * (int64_t)(base + __popcll(mp & lt));
                    e[0] = (int32_t)p;
                    e[1] = wi1;
                    e[2] = si2;
                }
            }
            const uint64_t mf = __ballot(valid && full);
            if (mf != 0ull) {
                const int leader = __ffsll((unsigned long long)mf) - 1;
                int base = 0;
                if (lane == leader) base = atomicAdd(&A.counters[0], __popcll(mf));
                base = __shfl(base, leader);
                if (valid && full) {
                    const int slot = base + __popcll(mf & lt);
                    A.full_list[slot] = (int32_t)p;
                    // any centroid that can still win scores at least this
                    A.full_thr[slot] = w1 - e2;
                }
            }
        }
    }
}

// Four consecutive elements of a centroid row as fp64.
__device__ __forceinline__ void load4_64(const float *c, double (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4 *>(c);
    o[0] = (double)v.x;
    o[1] = (double)v.y;
    o[2] = (double)v.z;
    o[3] = (double)v.w;
}
__device__ __forceinline__ void load4_64(const double *c, double (&o)[4]) {
    const double2 a = *reinterpret_cast<const double2 *>(c);
    const double2 b = *reinterpret_cast<const double2 *>(c + 2);
    o[0] = a.x;
    o[1] = a.y;
    o[2] = b.x;
    o[3] = b.y;
}

// The fp64 direct-difference distances of one point to NC centroids:
// D[m] = sum_j (x_j - c_mj)^2 in increasing j, with no fused multiply-add
// (inner product: D[m] = -sum_j x_j c_mj, the same order, whose negation is
// exact so that the smallest D is the largest dot product);
// for cosine x_j is first divided by the row norm nx (as the definition
// does).  Rows are read four elements at a time when d is a multiple of 4
// (X, C and the fp64 normalised centroids are then 16-byte aligned).
template <typename CT, int NC>
__device__ __forceinline__ void sqdist64(const float *__restrict__ x, const CT *const (&c)[NC], int d, double nx,
                                         bool cosine, bool ip, double (&D)[NC]) {
#pragma clang fp contract(off)
#pragma unroll
    for (int m = 0; m < NC; ++m) D[m] = 0.0;
    int j = 0;
    if ((d & 3) == 0) {
        for (; j < d; j += 4) {
            const float4 xv4 = *reinterpret_cast<const float4 *>(x + j);
            double xv[4] = {(double)xv4.x, (double)xv4.y, (double)xv4.z, (double)xv4.w};
            if (cosine) {
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[e] = xv[e] / nx;
            }
#pragma unroll
            for (int m = 0; m < NC; ++m) {
                double cv[4];
                load4_64(c[m] + j, cv);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (ip) {
                        D[m] = D[m] - xv[e] * cv[e];
                    } else {
                        const double t = xv[e] - cv[e];
                        D[m] = D[m] + t * t;
                    }
                }
            }
        }
    }
    for (; j < d; ++j) {
        double xv = (double)x[j];
        if (cosine) xv = xv / nx;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            if (ip) {
                D[m] = D[m] - xv * (double)c[m][j];
            } else {
                const double t = xv - (double)c[m][j];
                D[m] = D[m] + t * t;
            }
        }
    }
}

// The near-tie checks below stage rows through LDS when there are many
// listed points with short rows; with few listed points, or d > 128, a wave
// would run through its d / J dependent stages (and, in the window check,
// once per candidate) with too few waves in flight to hide them, and one
// lane per point reading its own rows is faster (measured: 1M x 128, K =
// 1024 with 3,000 listed pairs and 1M x 768 with 360).  These are those
// per-lane versions.
template <typename CT>
__device__ __forceinline__ void recheck_cand_rows(const float *__restrict__ X, int d, const CT *__restrict__ C,
                                                  const double *__restrict__ xnorm64,
                                                  const int32_t *__restrict__ full_list,
                                                  const int32_t *__restrict__ cand,
                                                  const int32_t *__restrict__ ccount, int64_t cap_slots,
                                                  int32_t *__restrict__ ovf_list, int32_t *__restrict__ counters,
                                                  int32_t *__restrict__ a_out, int ip) {
#pragma clang fp contract(off)
    const int cnt = counters[0];
    const int nl = 2 * max(counters[3], 1);  // candidate lists per slot
    for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < cnt; q += gridDim.x * blockDim.x) {
        const int64_t p = full_list[q];
        bool ovf = q >= cap_slots;
        for (int l = 0; l < nl && !ovf; ++l) ovf = ccount[(int64_t)q * nl + l] > kMaxCand;
        if (ovf) {
            ovf_list[atomicAdd(&counters[2], 1)] = (int32_t)p;
            continue;
        }
        const double nx = xnorm64 != nullptr ? xnorm64[p] : 1.0;
        double best = INFINITY;
        int bk = 0x7fffffff;
        for (int l = 0; l < nl; ++l) {
            for (int m = 0; m < ccount[(int64_t)q * nl + l]; ++m) {
                const int k = cand[((int64_t)q * nl + l) * kMaxCand + m];
                const CT *const row[1] = {C + (size_t)k * d};
                double D[1];
                sqdist64<CT, 1>(X + (size_t)p * d, row, d, nx, xnorm64 != nullptr, ip != 0, D);
                if (D[0] < best || (D[0] == best && k < bk)) {
                    best = D[0];
                    bk = k;
                }
            }
        }
        a_out[p] = bk;
    }
}

// The same fp64 distances by a group of 32 lanes (one point, NC centroid
// rows): lane g of the group loads dims [gS, gS + S) of every row at once (S
// = ceil(d / 32) rounded up to 4, at most kGroupSpan), and the running sums
// then pass from lane to lane, each lane adding its own dims in increasing j
// -- the same terms in the same order as sqdist64, so the same bits -- while
// the loads of all lanes were in flight together.  `base` is the group's
// first lane in the wave; every lane of the group returns the sums.
constexpr int kGroupSpan = 24;                  // dims per lane: d <= 768
constexpr int kGroupMaxD = 32 * kGroupSpan;
template <typename CT, int NC>
__device__ __forceinline__ void group_sqdist64(const float *__restrict__ x, const CT *const (&c)[NC], int d,
                                               double nx, bool cosine, bool ip, int gl, int base, double (&D)[NC]) {
#pragma clang fp contract(off)
    const int S = ((d + 31) / 32 + 3) & ~3;
    const int j0 = gl * S;
    const int ns = max(0, min(S, d - j0));
    float xr[kGroupSpan];
    CT cr[NC][kGroupSpan];
#pragma unroll
    for (int s = 0; s < kGroupSpan; ++s) {
        xr[s] = 0.f;
#pragma unroll
        for (int m = 0; m < NC; ++m) cr[m][s] = (CT)0;
    }
    if ((d & 3) == 0) {
#pragma unroll
        for (int s = 0; s < kGroupSpan; s += 4) {
            if (s < ns) {
                const float4 v = *reinterpret_cast<const float4 *>(x + j0 + s);
                xr[s] = v.x;
                xr[s + 1] = v.y;
                xr[s + 2] = v.z;
                xr[s + 3] = v.w;
#pragma unroll
                for (int m = 0; m < NC; ++m) {
                    double cv[4];
                    load4_64(c[m] + j0 + s, cv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) cr[m][s + e] = (CT)cv[e];
                }
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < kGroupSpan; ++s) {
            if (s < ns) {
                xr[s] = x[j0 + s];
#pragma unroll
                for (int m = 0; m < NC; ++m) cr[m][s] = c[m][j0 + s];
            }
        }
    }
#pragma unroll
    for (int m = 0; m < NC; ++m) D[m] = 0.0;
    for (int g = 0; g < 32; ++g) {
        if (gl == g) {
#pragma unroll
            for (int s = 0; s < kGroupSpan; ++s) {
                if (s < ns) {
                    double xv = (double)xr[s];
                    if (cosine) xv = xv / nx;
#pragma unroll
                    for (int m = 0; m < NC; ++m) {
                        if (ip) {
                            D[m] = D[m] - xv * (double)cr[m][s];
                        } else {
                            const double t = xv - (double)cr[m][s];
                            D[m] = D[m] + t * t;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < NC; ++m) D[m] = __shfl(D[m], base + g);
    }
}

// Pair check, one 32-lane group per listed point (d <= kGroupMaxD).
template <typename CT>
__device__ __forceinline__ void recheck_pair_group(const float *__restrict__ X, int d, const CT *__restrict__ C,
                                                   const double *__restrict__ xnorm64,
                                                   const int32_t *__restrict__ pair_list,
                                                   const int32_t *__restrict__ counters,
                                                   int32_t *__restrict__ a_out, int ip) {
    const int cnt = counters[1];
    const int lane = threadIdx.x & 63, gl = lane & 31, base = lane & 32;
    const int64_t ng = (int64_t)gridDim.x * (blockDim.x / 32);
    for (int64_t q = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 32; q < cnt; q += ng) {
        const int64_t p = pair_list[3 * q];
        const int k1 = pair_list[3 * q + 1];
        const int k2 = pair_list[3 * q + 2];
        const CT *const rows[2] = {C + (size_t)k1 * d, C + (size_t)k2 * d};
        double D[2];
        group_sqdist64<CT, 2>(X + (size_t)p * d, rows, d, xnorm64 != nullptr ? xnorm64[p] : 1.0,
                              xnorm64 != nullptr, ip != 0, gl, base, D);
        if (gl == 0) {
            const bool second = (D[1] < D[0]) || (D[1] == D[0] && k2 < k1);
            a_out[p] = second ? k2 : k1;
        }
    }
}

// Window check, one workgroup per listed point (d <= kGroupMaxD): its
// 32-lane groups take the candidates round-robin, and the lowest (distance,
// index) of the groups is taken in LDS.
template <typename CT>
__device__ __forceinline__ void recheck_cand_group(const float *__restrict__ X, int d, const CT *__restrict__ C,
                                                   const double *__restrict__ xnorm64,
                                                   const int32_t *__restrict__ full_list,
                                                   const int32_t *__restrict__ cand,
                                                   const int32_t *__restrict__ ccount, int64_t cap_slots,
                                                   int32_t *__restrict__ ovf_list, int32_t *__restrict__ counters,
                                                   int32_t *__restrict__ a_out, int ip) {
    __shared__ double sD[16];
    __shared__ int sK[16];
    const int cnt = counters[0];
    const int nl = 2 * max(counters[3], 1);  // candidate lists per slot
    const int lane = threadIdx.x & 63, gl = lane & 31, base = lane & 32;
    const int grp = threadIdx.x / 32, ngrp = blockDim.x / 32;  // at most 16
    for (int64_t q = blockIdx.x; q < cnt; q += gridDim.x) {
        const int64_t p = full_list[q];
        bool ovf = q >= cap_slots;
        int ntot = 0;
        for (int l = 0; l < nl && !ovf; ++l) {
            const int c = ccount[q * nl + l];
            ovf = c > kMaxCand;
            ntot += c;
        }
        if (ovf) {
            if (threadIdx.x == 0) ovf_list[atomicAdd(&counters[2], 1)] = (int32_t)p;
            continue;
        }
        const double nx = xnorm64 != nullptr ? xnorm64[p] : 1.0;
        double best = INFINITY;
        int bk = 0x7fffffff;
        for (int m = grp; m < ntot; m += ngrp) {
            int l = 0, r = m;  // the m-th candidate: list l, rank r
            for (int c = ccount[q * nl]; r >= c; c = ccount[q * nl + l]) {
                r -= c;
                ++l;
            }
            const int k = cand[(q * nl + l) * kMaxCand + r];
            const CT *const row[1] = {C + (size_t)k * d};
            double D[1];
            group_sqdist64<CT, 1>(X + (size_t)p * d, row, d, nx, xnorm64 != nullptr, ip != 0, gl, base, D);
            if (D[0] < best || (D[0] == best && k < bk)) {
                best = D[0];
                bk = k;
            }
        }
        if (gl == 0) {
            sD[grp] = best;
            sK[grp] = bk;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int g = 1; g < ngrp; ++g) {
                if (sD[g] < best || (sD[g] == best && sK[g] < bk)) {
                    best = sD[g];
                    bk = sK[g];
                }
            }
            a_out[p] = bk;
        }
        __syncthreads();
    }
}

template <typename CT>
__device__ __forceinline__ void recheck_pair_rows(const float *__restrict__ X, int d, const CT *__restrict__ C,
                                                  const double *__restrict__ xnorm64,
                                                  const int32_t *__restrict__ pair_list,
                                                  const int32_t *__restrict__ counters,
                                                  int32_t *__restrict__ a_out, int ip) {
    const int cnt = counters[1];
    for (int q = blockIdx.x * blockDim.x + threadIdx.x; q < cnt; q += gridDim.x * blockDim.x) {
        const int64_t p = pair_list[3 * (int64_t)q];
        const int k1 = pair_list[3 * (int64_t)q + 1];
        const int k2 = pair_list[3 * (int64_t)q + 2];
        const CT *const rows[2] = {C + (size_t)k1 * d, C + (size_t)k2 * d};
        double D[2];
        sqdist64<CT, 2>(X + (size_t)p * d, rows, d, xnorm64 != nullptr ? xnorm64[p] : 1.0, xnorm64 != nullptr,
                        ip != 0, D);
        const bool second = (D[1] < D[0]) || (D[1] == D[0] && k2 < k1);
        a_out[p] = second ? k2 : k1;
    }
}

// fp64 check of a near-tie point from the full list whose candidates were
// collected: the lowest-index minimum of the direct-difference fp64 distance
// over its candidates (both half-lane lists).  A point whose lists overflowed,
// or that lies beyond the collected slots, goes to the overflow list for a
// rescoring against all K.  A wave takes 64 listed points (one per lane) at a
// time; for each candidate rank m it stages the points' rows and their m-th
// candidate rows through LDS as k_recheck_pair does, and each lane sums its
// own rows in increasing j.
// four consecutive floats into a padded LDS row (the rows are J + 1 floats
// long, so no 16-byte LDS store fits them)
__device__ __forceinline__ void stage4(float *dst, const float4 v) {
    dst[0] = v.x;
    dst[1] = v.y;
    dst[2] = v.z;
    dst[3] = v.w;
}

template <typename CT>
__global__ __launch_bounds__(256) void k_recheck_cand(const float *__restrict__ X, int d, const CT *__restrict__ C,
                                                      const double *__restrict__ xnorm64,
                                                      const int32_t *__restrict__ full_list,
                                                      const int32_t *__restrict__ cand,
                                                      const int32_t *__restrict__ ccount, int64_t cap_slots,
                                                      int32_t *__restrict__ ovf_list, int32_t *__restrict__ counters,
                                                      int32_t *__restrict__ a_out, int ip) {
#pragma clang fp contract(off)
    constexpr int J = sizeof(CT) == 4 ? 16 : 8;  // dims per stage
    constexpr int JP = J + 1;                    // padded LDS row
    __shared__ float sx[4][64 * JP];
    __shared__ CT sc[4][64 * JP];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cnt = counters[0];
    const bool vec4 = sizeof(CT) == 4 && d % J == 0;
    if (d > 128 || cnt < kStagedMinList) {
        if (d <= kGroupMaxD)
            recheck_cand_group<CT>(X, d, C, xnorm64, full_list, cand, ccount, cap_slots, ovf_list, counters, a_out,
                                   ip);
        else
            recheck_cand_rows<CT>(X, d, C, xnorm64, full_list, cand, ccount, cap_slots, ovf_list, counters, a_out,
                                  ip);
        return;
    }
    const int nl = 2 * max(counters[3], 1);  // candidate lists per slot (two per tile slice)
    for (int64_t q0 = ((int64_t)blockIdx.x * 4 + w) * 64; q0 < cnt; q0 += (int64_t)gridDim.x * 4 * 64) {
        const int64_t q = q0 + lane;
        bool ok = q < cnt;
        const int64_t p = ok ? full_list[q] : 0;
        bool ovf = ok && q >= cap_slots;
        int nc = 0;
        if (ok && !ovf)
            for (int l = 0; l < nl; ++l) {
                const int c = ccount[q * nl + l];
                ovf = ovf || c > kMaxCand;
                nc += c;
            }
        if (ovf) {
            ovf_list[atomicAdd(&counters[2], 1)] = (int32_t)p;
            ok = false;
        }
        if (!ok) nc = 0;
        int ncw = nc;  // the wave's largest candidate count
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ncw = max(ncw, __shfl_xor(ncw, off));
        const double nx = (xnorm64 != nullptr) ? xnorm64[p] : 1.0;
        double best = INFINITY;
        int bk = 0x7fffffff;
        for (int m = 0; m < ncw; ++m) {
            const bool has = m < nc;
            int k = 0;
            if (has) {
                int l = 0, r = m;  // the m-th candidate: list l, rank r
                for (int c = ccount[q * nl]; r >= c; c = ccount[q * nl + l]) {
                    r -= c;
                    ++l;
                }
                k = cand[(q * nl + l) * kMaxCand + r];
            }
            double D = 0.0;
            for (int j0 = 0; j0 < d; j0 += J) {
                const int nj = min(J, d - j0);
                if (vec4) {
                    // fp32 rows and d a multiple of J: 16-byte loads, four
                    // dims of a row per lane (X and C are 16-byte aligned)
#pragma unroll
                    for (int i = 0; i < J / 4; ++i) {
                        const int e = lane + 64 * i, r = e / (J / 4), c = (e % (J / 4)) * 4;
                        const int64_t pr = __shfl(p, r);
                        const int kr = __shfl(k, r);
                        const float4 xv = *reinterpret_cast<const float4 *>(X + (size_t)pr * d + j0 + c);
                        const float4 cv = *reinterpret_cast<const float4 *>(
                            reinterpret_cast<const float *>(C) + (size_t)kr * d + j0 + c);
                        stage4(&sx[w][r * JP + c], xv);
                        stage4(reinterpret_cast<float *>(&sc[w][r * JP + c]), cv);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < J; ++i) {
                        const int e = lane + 64 * i, r = e / J, c = e % J;
                        const int64_t pr = __shfl(p, r);
                        const int kr = __shfl(k, r);
                        if (c < nj) {
                            sx[w][r * JP + c] = X[(size_t)pr * d + j0 + c];
                            sc[w][r * JP + c] = C[(size_t)kr * d + j0 + c];
                        }
                    }
                }
                __builtin_amdgcn_wave_barrier();
                for (int c = 0; c < nj; ++c) {
                    double xv = (double)sx[w][lane * JP + c];
                    if (xnorm64 != nullptr) xv = xv / nx;
                    const double cv = (double)sc[w][lane * JP + c];
                    if (ip) {
                        D = D - xv * cv;
                    } else {
                        const double t = xv - cv;
                        D = D + t * t;
                    }
                }
                __builtin_amdgcn_wave_barrier();
            }
            if (has && (D < best || (D == best && k < bk))) {
                best = D;
                bk = k;
            }
        }
        if (ok) {
            a_out[p] = bk;
        }
    }
}

// fp64 check of a near-tie point whose winner is one of two known centroids:
// the smaller direct-difference distance wins, the lower index on a tie.
// A wave takes 64 listed points (one per lane) at a time and stages their
// rows and both centroid rows through LDS, J dims at a time, with coalesced
// loads (consecutive lanes read consecutive dims of a row; a lane reading
// its own row from memory would touch 64 rows per load instruction); each
// lane then runs the definition's sums over its own rows, in increasing j.
template <typename CT>
__global__ __launch_bounds__(256) void k_recheck_pair(const float *__restrict__ X, int d, const CT *__restrict__ C,
                                                      const double *__restrict__ xnorm64,
                                                      const int32_t *__restrict__ pair_list,
                                                      const int32_t *__restrict__ counters,
                                                      int32_t *__restrict__ a_out, int ip) {
#pragma clang fp contract(off)
    constexpr int J = sizeof(CT) == 4 ? 16 : 8;  // dims per stage
    constexpr int JP = J + 1;                    // padded LDS row
    __shared__ float sx[4][64 * JP];
    __shared__ CT sc[4][2][64 * JP];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cnt = counters[1];
    const bool vec4 = sizeof(CT) == 4 && d % J == 0;
    if (d > 128 || cnt < kStagedMinList) {
        if (d <= kGroupMaxD)
            recheck_pair_group<CT>(X, d, C, xnorm64, pair_list, counters, a_out, ip);
        else
            recheck_pair_rows<CT>(X, d, C, xnorm64, pair_list, counters, a_out, ip);
        return;
    }
    for (int64_t q0 = ((int64_t)blockIdx.x * 4 + w) * 64; q0 < cnt; q0 += (int64_t)gridDim.x * 4 * 64) {
        const int64_t q = q0 + lane;
        const bool ok = q < cnt;
        const int64_t p = ok ? pair_list[3 * q] : 0;
        const int k1 = ok ? pair_list[3 * q + 1] : 0;
        const int k2 = ok ? pair_list[3 * q + 2] : 0;
        const double nx = (xnorm64 != nullptr) ? xnorm64[p] : 1.0;
        double D1 = 0.0, D2 = 0.0;
        for (int j0 = 0; j0 < d; j0 += J) {
            const int nj = min(J, d - j0);
            // element e of the stage: row e / J, dim e % J (rows of lanes
            // that hold no pair are those of row 0: read, never used)
            if (vec4) {
                // fp32 rows and d a multiple of J: 16-byte loads, four dims
                // of a row per lane (X and C are 16-byte aligned)
#pragma unroll
                for (int i = 0; i < J / 4; ++i) {
                    const int e = lane + 64 * i, r = e / (J / 4), c = (e % (J / 4)) * 4;
                    const int64_t pr = __shfl(p, r);
                    const int kr1 = __shfl(k1, r), kr2 = __shfl(k2, r);
                    const float *Cf = reinterpret_cast<const float *>(C);
                    const float4 xv = *reinterpret_cast<const float4 *>(X + (size_t)pr * d + j0 + c);
                    const float4 c1 = *reinterpret_cast<const float4 *>(Cf + (size_t)kr1 * d + j0 + c);
                    const float4 c2 = *reinterpret_cast<const float4 *>(Cf + (size_t)kr2 * d + j0 + c);
                    stage4(&sx[w][r * JP + c], xv);
                    stage4(reinterpret_cast<float *>(&sc[w][0][r * JP + c]), c1);
                    stage4(reinterpret_cast<float *>(&sc[w][1][r * JP + c]), c2);
                }
            } else {
#pragma unroll
                for (int i = 0; i < J; ++i) {
                    const int e = lane + 64 * i, r = e / J, c = e % J;
                    const int64_t pr = __shfl(p, r);
                    const int kr1 = __shfl(k1, r), kr2 = __shfl(k2, r);
                    if (c < nj) {
                        sx[w][r * JP + c] = X[(size_t)pr * d + j0 + c];
                        sc[w][0][r * JP + c] = C[(size_t)kr1 * d + j0 + c];
                        sc[w][1][r * JP + c] = C[(size_t)kr2 * d + j0 + c];
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            for (int c = 0; c < nj; ++c) {
                double xv = (double)sx[w][lane * JP + c];
                if (xnorm64 != nullptr) xv = xv / nx;
                const double c1 = (double)sc[w][0][lane * JP + c];
                const double c2 = (double)sc[w][1][lane * JP + c];
                if (ip) {
                    D1 = D1 - xv * c1;
                    D2 = D2 - xv * c2;
                } else {
                    const double t1 = xv - c1, t2 = xv - c2;
                    D1 = D1 + t1 * t1;
                    D2 = D2 + t2 * t2;
                }
            }
            // every lane has read this stage before the next one overwrites it
            __builtin_amdgcn_wave_barrier();
        }
        if (ok) {
            const bool second = (D2 < D1) || (D2 == D1 && k2 < k1);
            a_out[p] = second ? k2 : k1;
        }
    }
}

// ---------------------------------------------------------------------------
// fp64 rescoring of listed near-tie points: D_ik = sum_j (x_ij - c_kj)^2 in
// fp64 in increasing j, no fused multiply-add, for every k; the lowest index
// attaining the minimum wins.  That is the distance definition itself, so the
// result is the exact assignment.  For cosine the rows are normalised in fp64
// exactly as the definition says (C64 holds the normalised centroids).
// A workgroup takes RP listed points at a time; thread t scores centroids
// t, t+256, ...
template <typename CT, int RP>
__global__ __launch_bounds__(256) void k_recheck(const float *__restrict__ X, int d, const CT *__restrict__ C,
                                                 int K, const double *__restrict__ xnorm64,
                                                 const int32_t *__restrict__ flag_list,
                                                 const int32_t *__restrict__ counters, int P,
                                                 int32_t *__restrict__ a_out, int ip) {
#pragma clang fp contract(off)
    extern __shared__ double sx[];  // P * d
    __shared__ double rb[4][RP];
    __shared__ int ri[4][RP];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int cnt = counters[0];
    for (int base = blockIdx.x * P; base < cnt; base += gridDim.x * P) {
        const int np = min(P, cnt - base);
        for (int q = tid; q < np * d; q += 256) {
            const int pi = q / d, jj = q - pi * d;
            const int64_t p = flag_list[base + pi];
            double v = (double)X[(size_t)p * d + jj];
            if (xnorm64 != nullptr) v = v / xnorm64[p];
            sx[pi * d + jj] = v;
        }
        __syncthreads();
        double best[RP];
        int bidx[RP];
#pragma unroll
        for (int pi = 0; pi < RP; ++pi) {
            best[pi] = INFINITY;
            bidx[pi] = 0x7fffffff;
        }
        for (int k = tid; k < K; k += 256) {
            double acc[RP];
#pragma unroll
            for (int pi = 0; pi < RP; ++pi) acc[pi] = 0.0;
            const CT *crow = C + (size_t)k * d;
            auto step = [&](int jj, double c) {
#pragma clang fp contract(off)
#pragma unroll
                for (int pi = 0; pi < RP; ++pi) {
                    if (pi < np) {
                        if (ip) {
                            acc[pi] = acc[pi] - sx[pi * d + jj] * c;
                        } else {
                            const double tt = sx[pi * d + jj] - c;
                            acc[pi] = acc[pi] + tt * tt;
                        }
                    }
                }
            };
            int jj = 0;
            if ((d & 3) == 0) {
                // the row in 16-byte (fp32) or 32-byte (fp64) loads: each
                // lane reads its own row, so wide loads cut the number of
                // scattered load instructions by four
                for (; jj < d; jj += 4) {
                    double c4[4];
                    load4_64(crow + jj, c4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) step(jj + e, c4[e]);
                }
            }
            for (; jj < d; ++jj) step(jj, (double)crow[jj]);
#pragma unroll
            for (int pi = 0; pi < RP; ++pi) {
                if (acc[pi] < best[pi]) {
                    best[pi] = acc[pi];
                    bidx[pi] = k;
                }
            }
        }
#pragma unroll
        for (int pi = 0; pi < RP; ++pi) {
            double b = best[pi];
            int i = bidx[pi];
            for (int off = 32; off > 0; off >>= 1) {
                const double ob = __shfl_xor(b, off);
                const int oi = __shfl_xor(i, off);
                if (ob < b || (ob == b && oi < i)) {
                    b = ob;
                    i = oi;
                }
            }
            if (lane == 0) {
                rb[w][pi] = b;
                ri[w][pi] = i;
            }
        }
        __syncthreads();
        if (tid < np) {
            double b = rb[0][tid];
            int i = ri[0][tid];
            for (int ww = 1; ww < 4; ++ww) {
                const double ob = rb[ww][tid];
                const int oi = ri[ww][tid];
                if (ob < b || (ob == b && oi < i)) {
                    b = ob;
                    i = oi;
                }
            }
            const int64_t p = flag_list[base + tid];
            a_out[p] = i;
        }
        __syncthreads();
    }
}

int split_width(int d) {
    const AssignShape sh = assign_shape(d);
    return sh.DP * sh.nch;
}

// ---------------------------------------------------------------------------
AssignShape assign_shape(int d) {
    if (d <= 16) return {16, 1, 1, 1};
    if (d <= 32) return {32, 1, 1, 1};
    if (d <= 64) return {64, 1, 1, 1};
    if (d <= 128) return {128, 2, 1, 1};
    return {64, 1, 2, (int)cdiv(d, 64)};
}

hipError_t launch_row_norm64(const float *M, int64_t rows, int d, double *nrm, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_row_norm64, dim3((unsigned)cdiv(rows, 256)), dim3(256), 0, s, M, rows, d, nrm);
    return hipGetLastError();
}

hipError_t launch_normalize_rows(const float *M, int64_t rows, int d, const double *nrm, double *out64,
                                 float *out32, hipStream_t s) {
    const int64_t total = rows * (int64_t)d;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_normalize_rows, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s, M, total, d, nrm,
                       out64, out32);
    return hipGetLastError();
}

hipError_t launch_centroid_prep(const float *C, int K, int d, float *ncn, float *cmax_part, int *nparts,
                                const SplitC &sc, bool ip, hipStream_t s) {
    const int Kpad = (int)(cdiv(K, kCentroidPad) * kCentroidPad);
    const int nb = (int)cdiv(Kpad, 4);
    *nparts = nb;
    hipLaunchKernelGGL(k_centroid_prep, dim3(nb), dim3(256), 0, s, C, K, Kpad, d, ncn, cmax_part, sc.cs, sc.w,
                       ip ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_prep_finish(const float *cmax_part, int nparts, float *scal, int32_t *counter, hipStream_t s) {
    hipLaunchKernelGGL(k_prep_finish, dim3(1), dim3(1024), 0, s, cmax_part, nparts, scal, counter);
    return hipGetLastError();
}

template <int DP, int PB, int CB, int WAVES, int MINB, bool RES, bool COLLECT, bool SPLIT, int TL = 0>
static hipError_t launch_fa(const FlashArgs &A0, hipStream_t s) {
    // the tile count and chunk count follow this instantiation's geometry:
    // the -||c||^2/2 array is padded to kCentroidPad, a multiple of every
    // tile height, so the tiles never read past it
    static_assert(kCentroidPad % (CB * 32) == 0, "tile height must divide the centroid padding");
    FlashArgs A = A0;
    A.ntiles = (int)cdiv(A.K, CB * 32);
    A.nch = RES ? 1 : (int)cdiv(A.d, DP);
    if (RES && A.d > DP) return hipErrorInvalidValue;
    constexpr int BM = WAVES * PB * 32;
    int64_t nb = COLLECT ? cdiv(A.cap_slots, BM) : cdiv(A.N, BM);
    if (COLLECT && nb > 512) nb = 512;  // persistent: the workgroups stride over the listed slots
    unsigned gy = 1;
    if (TL > 0) {
        if (A.knn_rows % (CB * 32) != 0) return hipErrorInvalidValue;
        A.knn_tps = A.knn_rows / (CB * 32);
        gy = (unsigned)A.knn_slices;
    }
    if (A.d % 4 == 0)
        hipLaunchKernelGGL((k_flash_assign<DP, PB, CB, WAVES, MINB, RES, true, COLLECT, SPLIT, TL>),
                           dim3((unsigned)nb, gy), dim3(WAVES * 64), 0, s, A);
    else
        hipLaunchKernelGGL((k_flash_assign<DP, PB, CB, WAVES, MINB, RES, false, COLLECT, SPLIT, TL>),
                           dim3((unsigned)nb, gy), dim3(WAVES * 64), 0, s, A);
    return hipGetLastError();
}

template <bool COLLECT, bool SPLIT>
static hipError_t launch_fa_shape(const FlashArgs &A, hipStream_t s) {
    const AssignShape sh = assign_shape(A.d);
    if (sh.nch > 1) {
        // streamed points are re-read for every centroid tile, and that
        // traffic (not the products) bounds the kernel: 128-row tiles were
        // 20 % faster than 64-row ones for fp32 scoring at d = 768,
        // K = 4096, and 256-row tiles 20 % faster again than 128-row ones
        // for split scoring (one accumulator, 216 registers, two waves per
        // SIMD).  More waves per CU are slower there (38 ms against 27 ms
        // at four per SIMD): the points in flight then outgrow the caches.
        if constexpr (SPLIT)
            return launch_fa<32, 1, 8, 8, 2, false, COLLECT, SPLIT>(A, s);
        else
            return launch_fa<64, 1, 4, 4, 2, false, COLLECT, SPLIT>(A, s);
    }
    switch (sh.DP) {
    case 16: return launch_fa<16, 1, 1, 8, 4, true, COLLECT, SPLIT>(A, s);
    case 32: return launch_fa<32, 1, 1, 8, 4, true, COLLECT, SPLIT>(A, s);
    case 64: return launch_fa<64, 1, 1, 8, 4, true, COLLECT, SPLIT>(A, s);
    default:
        // split scoring: 4 waves of 2 point blocks (two waves per SIMD), so
        // two workgroups share a CU and one's prologue and epilogue overlap
        // the other's products: 3 % faster than 8-wave workgroups at
        // 16M x 128, K = 32768 and 5 % at 1M x 128, K = 1024, measured side
        // by side (252 registers, no scratch); one point block per wave:
        // 10-14 % slower
        if constexpr (SPLIT)
            return launch_fa<128, 2, 2, 4, 2, true, COLLECT, SPLIT>(A, s);
        else
            return launch_fa<128, 2, 1, 4, 2, true, COLLECT, SPLIT>(A, s);
    }
}

template <bool COLLECT>
static hipError_t launch_fa_score(const FlashArgs &A, bool split, hipStream_t s) {
    return split ? launch_fa_shape<COLLECT, true>(A, s) : launch_fa_shape<COLLECT, false>(A, s);
}

static FlashArgs flash_args(const float *X, int64_t N, int d, const float *C, const float *ncn, int K,
                            const float *scal, const double *xnorm64, int32_t *a_out,
                            const NearTies &nt, const SplitC &sc, bool ip) {
    const AssignShape sh = assign_shape(d);
    FlashArgs A;
    A.X = X;
    A.N = N;
    A.d = d;
    A.nch = sh.nch;
    A.C = C;
    A.ncn = ncn;
    A.K = K;
    A.ntiles = (int)cdiv(K, sh.CB * 32);
    A.scal = scal;
    A.xnorm64 = xnorm64;
    A.a_out = a_out;
    A.full_list = nt.full_list;
    A.full_thr = nt.full_thr;
    A.pair_list = nt.pair_list;
    A.counters = nt.counters;
    A.cand = nt.cand;
    A.ccount = nt.ccount;
    A.cap_slots = near_tie_cap(N);
    A.Cs = sc.cs;
    A.sw = sc.w;
    A.ip = ip ? 1 : 0;
    A.cs_bytes = (unsigned)(cdiv(K, kCentroidPad) * kCentroidPad * 4 * (int64_t)sc.w);
    A.knn_tau = nullptr;
    return A;
}

int64_t near_tie_cap(int64_t N) {
    int64_t cap = N / 8;
    if (cap < 65536) cap = 65536;
    if (cap > N) cap = N;
    return cap < 1 ? 1 : cap;
}

hipError_t launch_flash_assign(const float *X, int64_t N, int d, const float *C, const float *ncn, int K,
                               const float *scal, const double *xnorm64, int32_t *a_out,
                               const NearTies &nt, const SplitC &sc, bool ip, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    return launch_fa_score<false>(flash_args(X, N, d, C, ncn, K, scal, xnorm64, a_out, nt, sc, ip),
                                  sc.cs != nullptr, s);
}

// The objective terms: d1[p] = the fp64 distance of point p to its assigned
// centroid a[p] by the definition (direct differences in increasing j, no
// fused multiply-add; cosine on the fp64-normalised rows; inner product
// -x.c), rounded once to fp32 -- the oracle's D1 rounded, bit for bit.  One
// 32-lane group per point with coalesced row loads (d <= kGroupMaxD), else
// one lane per point.
// Inner product: the sums subtract each product from +0, which gives the
// negated dot product -(x.c) in value, rounding included (rounding to nearest
// is symmetric in sign); only a zero differs, +0 where -(x.c) is -0.
__device__ __forceinline__ float exact_d1_value(double D, int ip) {
    return (float)((ip && D == 0.0) ? -0.0 : D);
}
template <typename CT>
__global__ __launch_bounds__(256) void k_exact_d1(const float *__restrict__ X, int64_t N, int d,
                                                  const CT *__restrict__ C, const double *__restrict__ xnorm64,
                                                  const int32_t *__restrict__ a, float *__restrict__ d1, int ip) {
    if (d <= kGroupMaxD) {
        const int lane = threadIdx.x & 63, gl = lane & 31, base = lane & 32;
        const int64_t ng = (int64_t)gridDim.x * (blockDim.x / 32);
        for (int64_t p = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 32; p < N; p += ng) {
            const CT *const row[1] = {C + (size_t)a[p] * d};
            double D[1];
            group_sqdist64<CT, 1>(X + (size_t)p * d, row, d, xnorm64 != nullptr ? xnorm64[p] : 1.0,
                                  xnorm64 != nullptr, ip != 0, gl, base, D);
            if (gl == 0) d1[p] = exact_d1_value(D[0], ip);
        }
    } else {
        for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < N; p += (int64_t)gridDim.x * blockDim.x) {
            const CT *const row[1] = {C + (size_t)a[p] * d};
            double D[1];
            sqdist64<CT, 1>(X + (size_t)p * d, row, d, xnorm64 != nullptr ? xnorm64[p] : 1.0, xnorm64 != nullptr,
                            ip != 0, D);
            d1[p] = exact_d1_value(D[0], ip);
        }
    }
}

hipError_t launch_exact_d1(const float *X, int64_t N, int d, const float *C32, const double *C64,
                           const double *xnorm64, const int32_t *a, float *d1, bool ip, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    const int64_t per_block = d <= kGroupMaxD ? 8 : 256;  // points per workgroup pass
    int64_t nb = cdiv(N, per_block);
    if (nb > 8192) nb = 8192;
    if (C64 != nullptr)
        hipLaunchKernelGGL(k_exact_d1<double>, dim3((unsigned)nb), dim3(256), 0, s, X, N, d, C64, xnorm64, a, d1,
                           ip ? 1 : 0);
    else
        hipLaunchKernelGGL(k_exact_d1<float>, dim3((unsigned)nb), dim3(256), 0, s, X, N, d, C32, xnorm64, a, d1,
                           ip ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_recheck(const float *X, int64_t N, int d, const float *C_mfma, const float *C32,
                          const double *C64, const float *ncn, int K, const float *scal, const double *xnorm64,
                          const NearTies &nt, const SplitC &sc, bool ip, int32_t *a_out, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    hipError_t e;
    // 1. near ties between two known centroids
    {
        int64_t nb = cdiv(N, 256);
        if (nb > 4096) nb = 4096;
#define FK_PAIR(KERNEL, CT, CP)                                                                                    \
    hipLaunchKernelGGL(KERNEL<CT>, dim3((unsigned)nb), dim3(256), 0, s, X, d, CP, xnorm64, nt.pair_list, nt.counters, \
                       a_out, ip ? 1 : 0)
        if (C64 != nullptr)
            FK_PAIR(k_recheck_pair, double, C64);
        else
            FK_PAIR(k_recheck_pair, float, C32);
#undef FK_PAIR
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 2. the full list: collect every centroid within each point's window
    if ((e = launch_fa_score<true>(flash_args(X, N, d, C_mfma, ncn, K, scal, xnorm64, a_out, nt, sc, ip),
                                   sc.cs != nullptr, s)) != hipSuccess)
        return e;
    // 3. fp64 over the collected candidates; overflows go to the last list
    {
        const int64_t cap = near_tie_cap(N);
        int64_t nb = cdiv(N, 256);
        if (nb > 4096) nb = 4096;
#define FK_CAND(KERNEL, CT, CP)                                                                                   \
    hipLaunchKernelGGL(KERNEL<CT>, dim3((unsigned)nb), dim3(256), 0, s, X, d, CP, xnorm64, nt.full_list, nt.cand,  \
                       nt.ccount, cap, nt.ovf_list, nt.counters, a_out, ip ? 1 : 0)
        if (C64 != nullptr)
            FK_CAND(k_recheck_cand, double, C64);
        else
            FK_CAND(k_recheck_cand, float, C32);
#undef FK_CAND
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 4. overflow: rescore against all K
    constexpr int RP = 8;
    int P = (int)(49152 / (8 * (int64_t)d));
    if (P > RP) P = RP;
    if (P < 1) P = 1;
    const size_t lds = (size_t)P * d * sizeof(double);
    int64_t nb = cdiv(N, P);
    if (nb > 2048) nb = 2048;
    if (C64 != nullptr)
        hipLaunchKernelGGL((k_recheck<double, RP>), dim3((unsigned)nb), dim3(256), lds, s, X, d, C64, K, xnorm64,
                           nt.ovf_list, nt.counters + 2, P, a_out, ip ? 1 : 0);
    else
        hipLaunchKernelGGL((k_recheck<float, RP>), dim3((unsigned)nb), dim3(256), lds, s, X, d, C32, K, xnorm64,
                           nt.ovf_list, nt.counters + 2, P, a_out, ip ? 1 : 0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// k nearest neighbours: the FlashAssign sweep with a per-lane top-L list
// (queries are the points, database rows the centroids), then fp64.

// Resident point blocks: two 32-row blocks per LDS stage, two waves per SIMD
// (256 VGPRs each), of which the candidate lists take 2L per lane.  With
// L = 32 and d > 64 the resident point block no longer fits beside them, and
// for d > 128 it never does: the points are streamed in 64-dim chunks, four
// 32-row blocks per stage (which halves the re-reads of the query chunks),
// one wave per SIMD with the accumulators in AGPRs.
template <bool SPLIT, int TL>
static hipError_t launch_knn_shape(const FlashArgs &A, hipStream_t s) {
    const AssignShape sh = assign_shape(A.d);
    if (sh.nch > 1 || (TL > 16 && A.d > 64)) return launch_fa<64, 1, 4, 4, 1, false, false, SPLIT, TL>(A, s);
    if constexpr (TL <= 16) {
        if (sh.DP == 128) return launch_fa<128, 1, 2, 8, 2, true, false, SPLIT, TL>(A, s);
    }
    switch (sh.DP) {
    case 16: return launch_fa<16, 1, 2, 8, 2, true, false, SPLIT, TL>(A, s);
    case 32: return launch_fa<32, 1, 2, 8, 2, true, false, SPLIT, TL>(A, s);
    default: return launch_fa<64, 1, 2, 8, 2, true, false, SPLIT, TL>(A, s);
    }
}

int knn_list_len(int k) { return k <= kKnnShort ? 16 : 32; }

// Database slices: enough (point blocks x slices) workgroups to fill the chip
// (one workgroup per CU at a time) many times over when there are few
// queries -- about 4096 blocks of 256 queries, which at 10,000 queries is 64
// slices and exactly ten rounds of 256 CUs (the streamed-chunk kernels take
// 128 queries per workgroup, so twice as many) -- each slice at least 4096
// rows and a multiple of kCentroidPad rows (so of every tile height), at most
// kKnnMaxSlices of them.
KnnSlices knn_slices(int64_t M, int64_t Ndb) {
    constexpr int64_t kTargetGroups = 4096, kMinRows = 4096;
    const int64_t qb = cdiv(M > 0 ? M : 1, 256);
    int64_t S = cdiv(kTargetGroups, qb);
    if (S > kKnnMaxSlices) S = kKnnMaxSlices;
    const int64_t smax = cdiv(Ndb, kMinRows);
    if (S > smax) S = smax;
    if (S < 1) S = 1;
    const int64_t R = cdiv(cdiv(Ndb, S), kCentroidPad) * kCentroidPad;
    return KnnSlices{(int)cdiv(Ndb, R), (int)R};
}

// tau[q] = the TL-th best score of query q over the S1 lists of the sample
// sweep (each list sorted best first, TL long, -inf where a slice had fewer
// rows): TL steps of taking the best remaining list head.  Any value at or
// below the query's TL-th best over all rows would do; this one is the
// largest the sample gives.  One thread per query.
template <int TL>
__global__ __launch_bounds__(256) void k_knn_tau(const float *__restrict__ score, int64_t M, int S1,
                                                 float *__restrict__ tau) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= M) return;
    const float *base = score + (size_t)q * S1 * TL;
    int pos[kKnnSampleSlices];
    for (int i = 0; i < S1; ++i) pos[i] = 0;
    float v = -INFINITY;
    for (int r = 0; r < TL; ++r) {
        int bi = 0;
        float bv = -INFINITY;
        for (int i = 0; i < S1; ++i) {
            const float h = pos[i] < TL ? base[i * TL + pos[i]] : -INFINITY;
            if (h > bv) {
                bv = h;
                bi = i;
            }
        }
        v = bv;
        ++pos[bi];
    }
    tau[q] = v;
}

hipError_t launch_knn_sweep(const float *Q, int64_t M, int d, const float *DB, const float *ncn, int Ndb,
                            const float *scal, const double *qnorm64, const SplitC &sc, bool ip, int k,
                            int32_t *cand, float *score, float *win, float *tau, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    NearTies nt{};
    FlashArgs A = flash_args(Q, M, d, DB, ncn, Ndb, scal, qnorm64, nullptr, nt, sc, ip);
    const KnnSlices ks = knn_slices(M, Ndb);
    A.knn_slices = ks.slices;
    A.knn_rows = ks.rows;
    A.knn_cand = cand;
    A.knn_score = score;
    A.knn_win = win;
    const bool split = sc.cs != nullptr;
    auto sweep = [&](const FlashArgs &a) {
        if (knn_list_len(k) == 16)
            return split ? launch_knn_shape<true, 16>(a, s) : launch_knn_shape<false, 16>(a, s);
        return split ? launch_knn_shape<true, 32>(a, s) : launch_knn_shape<false, 32>(a, s);
    };
    // Every slice starts its lists from scratch, and while they fill, most
    // values are inserted (a pass of list updates each).  With several
    // slices, a first sweep over a sample of the first rows gives each query
    // its L-th best score there, which is at or below its L-th best over all
    // rows; the slices' lists start full of it, so only values above it are
    // ever inserted.  The sample is S1 slices of kKnnSampleRows rows (up to
    // 65,536 rows, at most a sixteenth of the database), each writing its
    // own lists, which k_knn_tau merges into the L-th best of the sample:
    // the larger the sample, the closer that comes to the final L-th best and
    // the fewer values pass it.  Only for d <= 128: with streamed d-chunks
    // the products outweigh the list updates and the extra sweep does not
    // pay (measured at d = 768).
    if (tau != nullptr && d <= 128 && ks.slices >= 4 && Ndb >= 4 * kKnnSampleRows) {
        int s1 = (int)(Ndb / (16 * (int64_t)kKnnSampleRows));
        s1 = s1 < 1 ? 1 : s1 > kKnnSampleSlices ? kKnnSampleSlices : s1;
        if (s1 > ks.slices) s1 = ks.slices;
        FlashArgs P = A;
        P.knn_slices = s1;
        P.knn_rows = kKnnSampleRows;
        hipError_t e = sweep(P);
        if (e != hipSuccess) return e;
        const int TL = knn_list_len(k);
        const int64_t nb = cdiv(M, 256);
        if (TL == 16)
            hipLaunchKernelGGL((k_knn_tau<16>), dim3((unsigned)nb), dim3(256), 0, s, score, M, s1, tau);
        else
            hipLaunchKernelGGL((k_knn_tau<32>), dim3((unsigned)nb), dim3(256), 0, s, score, M, s1, tau);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        A.knn_tau = tau;
    }
    return sweep(A);
}

// One thread per query: merge the slices' candidate lists into the L best
// MFMA scores (lower index first on equal scores).  Every row outside them
// scores at most the L-th: when the k-th beats it by more than the window
// the exact top k lies among the L, which are then ranked by their fp64
// distances (the definition: direct differences, or the negated dot product,
// in increasing j) by (distance, index).  Otherwise the query is listed for
// k_knn_full.
template <typename CT, int TL>
__global__ __launch_bounds__(256) void k_knn_finish(const float *__restrict__ Q, int64_t M, int d,
                                                    const CT *__restrict__ DB, const double *__restrict__ qnorm64,
                                                    int ip, const int32_t *__restrict__ cand,
                                                    const float *__restrict__ score, const float *__restrict__ win,
                                                    int S, int k, int ld, int Ndb, int32_t *__restrict__ list,
                                                    int32_t *__restrict__ counter, int32_t *__restrict__ idx,
                                                    float *__restrict__ dist) {
#pragma clang fp contract(off)
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= M) return;
    // columns past the database size (k clamped to Ndb): no row
    for (int r = k; r < ld; ++r) {
        idx[q * ld + r] = -1;
        dist[q * ld + r] = INFINITY;
    }
    float V[TL];
    int I[TL];
#pragma unroll
    for (int j = 0; j < TL; ++j) {
        V[j] = -INFINITY;
        I[j] = 0x7fffffff;
    }
    const size_t base = (size_t)q * S * TL;
    for (int e = 0; e < S * TL; ++e) {
        float v = score[base + e];
        int c = cand[base + e];
        if (!(v > V[TL - 1] || (v == V[TL - 1] && c < I[TL - 1]))) continue;
#pragma unroll
        for (int j = 0; j < TL; ++j) {
            const bool sw = v > V[j] || (v == V[j] && c < I[j]);
            const float tv = V[j];
            const int tc = I[j];
            V[j] = sw ? v : tv;
            I[j] = sw ? c : tc;
            v = sw ? tv : v;
            c = sw ? tc : c;
        }
    }
    float sk = V[0];
#pragma unroll
    for (int j = 0; j < TL; ++j) sk = (j == k - 1) ? V[j] : sk;
    if (!((sk - V[TL - 1]) > win[q])) {
        // wave-aggregated append to the list of queries ranked against all rows
        const uint64_t mk = __ballot(true);
        const int leader = __ffsll((unsigned long long)mk) - 1;
        int pos = 0;
        if ((int)__lane_id() == leader) pos = atomicAdd(counter, __popcll(mk));
        pos = __shfl(pos, leader);
        list[pos + __popcll(mk & lanemask_lt())] = (int32_t)q;
        return;
    }
    double D[TL];
    const double nx = qnorm64 != nullptr ? qnorm64[q] : 1.0;
#pragma unroll
    for (int j = 0; j < TL; ++j) {
        // fewer than L real rows: the sweep's padding rows (index >= Ndb)
        if (I[j] < 0 || I[j] >= Ndb) {
            I[j] = 0x7fffffff;
            D[j] = INFINITY;
            continue;
        }
        const CT *const row[1] = {DB + (size_t)I[j] * d};
        double Dj[1];
        sqdist64<CT, 1>(Q + (size_t)q * d, row, d, nx, qnorm64 != nullptr, ip != 0, Dj);
        D[j] = Dj[0];
    }
    // k passes of a minimum by (distance, index), static indexing only
    for (int r = 0; r < k; ++r) {
        double b = INFINITY;
        int bi = 0x7fffffff, bj = 0;
#pragma unroll
        for (int j = 0; j < TL; ++j) {
            const bool t = D[j] < b || (D[j] == b && I[j] < bi);
            b = t ? D[j] : b;
            bi = t ? I[j] : bi;
            bj = t ? j : bj;
        }
        idx[q * ld + r] = bi;
        dist[q * ld + r] = exact_d1_value(b, ip);
#pragma unroll
        for (int j = 0; j < TL; ++j) D[j] = (j == bj) ? (double)INFINITY : D[j];
#pragma unroll
        for (int j = 0; j < TL; ++j) I[j] = (j == bj) ? 0x7fffffff : I[j];
    }
}

// The exact k best database rows of each listed query against all Ndb rows
// in fp64 (the definition itself).  One workgroup per query: each thread keeps
// the k best of its rows (t, t + 256, ...), then k rounds of a workgroup-wide
// minimum of (distance, index) take them out in order.
template <typename CT>
__global__ __launch_bounds__(256) void k_knn_full(const float *__restrict__ Q, int d, const CT *__restrict__ DB,
                                                  int Ndb, const double *__restrict__ qnorm64, int ip,
                                                  const int32_t *__restrict__ list,
                                                  const int32_t *__restrict__ counters, int k, int ld,
                                                  int32_t *__restrict__ idx, float *__restrict__ dist) {
#pragma clang fp contract(off)
    __shared__ double wd[4];
    __shared__ int wi[4], wt[4];
    __shared__ int win_t;
    const int tid = threadIdx.x, w = tid >> 6;
    const int cnt = counters[0];
    for (int li = blockIdx.x; li < cnt; li += gridDim.x) {
        const int64_t q = list[li];
        const double nx = qnorm64 != nullptr ? qnorm64[q] : 1.0;
        double D[kMaxKnn];
        int I[kMaxKnn];
#pragma unroll
        for (int j = 0; j < kMaxKnn; ++j) {
            D[j] = INFINITY;
            I[j] = 0x7fffffff;
        }
        for (int c = tid; c < Ndb; c += 256) {
            const CT *const row[1] = {DB + (size_t)c * d};
            double Dc[1];
            sqdist64<CT, 1>(Q + (size_t)q * d, row, d, nx, qnorm64 != nullptr, ip != 0, Dc);
            // rows come in increasing index: a strict '<' keeps the lower
            // index first among equal distances
            double dv = Dc[0];
            int iv = c;
#pragma unroll
            for (int j = 0; j < kMaxKnn; ++j) {
                const bool sw = j < k && dv < D[j];
                const double td = D[j];
                const int ti = I[j];
                D[j] = sw ? dv : td;
                I[j] = sw ? iv : ti;
                dv = sw ? td : dv;
                iv = sw ? ti : iv;
            }
        }
        for (int r = 0; r < k; ++r) {
            double b = D[0];
            int bi = I[0];
            int bt = tid;
            for (int off = 32; off > 0; off >>= 1) {
                const double ob = __shfl_xor(b, off);
                const int oi = __shfl_xor(bi, off);
                const int ot = __shfl_xor(bt, off);
                if (ob < b || (ob == b && oi < bi)) {
                    b = ob;
                    bi = oi;
                    bt = ot;
                }
            }
            if ((tid & 63) == 0) {
                wd[w] = b;
                wi[w] = bi;
                wt[w] = bt;
            }
            __syncthreads();
            if (tid == 0) {
                double bb = wd[0];
                int bbi = wi[0], btt = wt[0];
                for (int ww = 1; ww < 4; ++ww)
                    if (wd[ww] < bb || (wd[ww] == bb && wi[ww] < bbi)) {
                        bb = wd[ww];
                        bbi = wi[ww];
                        btt = wt[ww];
                    }
                idx[q * ld + r] = bbi;
                dist[q * ld + r] = exact_d1_value(bb, ip);
                win_t = btt;
            }
            __syncthreads();
            if (tid == win_t) {
                // take this thread's best out
#pragma unroll
                for (int j = 0; j < kMaxKnn - 1; ++j) {
                    D[j] = D[j + 1];
                    I[j] = I[j + 1];
                }
                D[kMaxKnn - 1] = INFINITY;
                I[kMaxKnn - 1] = 0x7fffffff;
            }
            __syncthreads();
        }
    }
}

hipError_t launch_knn_finish(const float *Q, int64_t M, int d, const float *DB32, const double *DB64,
                             const double *qnorm64, bool ip, const int32_t *cand, const float *score,
                             const float *win, int k, int ld, int Ndb, int32_t *list, int32_t *counters, int32_t *idx,
                             float *dist, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (ld < k) return hipErrorInvalidValue;
    const unsigned nb = (unsigned)cdiv(M, 256);
    const int ipi = ip ? 1 : 0;
    const int S = knn_slices(M, Ndb).slices;
#define FK_KNN_FINISH(CT, TLV, DBP)                                                                              \
    hipLaunchKernelGGL((k_knn_finish<CT, TLV>), dim3(nb), dim3(256), 0, s, Q, M, d, DBP, qnorm64, ipi, cand, score, \
                       win, S, k, ld, Ndb, list, counters, idx, dist)
    if (knn_list_len(k) == 16) {
        if (DB64 != nullptr)
            FK_KNN_FINISH(double, 16, DB64);
        else
            FK_KNN_FINISH(float, 16, DB32);
    } else {
        if (DB64 != nullptr)
            FK_KNN_FINISH(double, 32, DB64);
        else
            FK_KNN_FINISH(float, 32, DB32);
    }
#undef FK_KNN_FINISH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nf = M < 4096 ? M : 4096;
    if (DB64 != nullptr)
        hipLaunchKernelGGL(k_knn_full<double>, dim3((unsigned)nf), dim3(256), 0, s, Q, d, DB64, Ndb, qnorm64, ipi,
                           list, counters, k, ld, idx, dist);
    else
        hipLaunchKernelGGL(k_knn_full<float>, dim3((unsigned)nf), dim3(256), 0, s, Q, d, DB32, Ndb, qnorm64, ipi,
                           list, counters, k, ld, idx, dist);
    return hipGetLastError();
}

}  // namespace fk
