// The inverse index of the Sort-Inverse Update: a stable LSD radix sort of
// (key = cluster id, value = point id) with no global atomic operation.
//
// The Flash-KMeans article (lumevalley.com, article 3696, section
// "Sort-Inverse Update: another answer to atomics") sorts the assignment by
// cluster id to obtain an inverse index, so that clusters can be reduced by
// contiguous reads without any atomic operation.  Keys are below K <= 65536:
// keys of up to 11 bits (K <= 2048) take one pass, wider keys two (8 bits,
// then the rest).
//
// Each pass is hist -> scan -> scatter over tiles of 8192 keys.  Inside a tile
// the scatter ranks 64 keys at a time with ballots: for a digit of B bits, B
// ballots give every lane the mask of lanes holding the same digit; its rank
// is the number of such lanes below it, and the lowest such lane (the leader)
// alone updates that digit's running count in LDS, so the order of equal
// digits is kept without any atomic operation.  Only the per-tile digit
// counts, where order does not matter, are LDS atomic adds; nothing touches
// global memory atomically.
#include "fk_internal.h"

namespace fk {

__device__ __forceinline__ uint64_t lanemask_lt_s() {
    const unsigned lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Mask of the lanes (among `active`) whose digit equals this lane's.
template <int BITS>
__device__ __forceinline__ uint64_t match_digit(unsigned dig, uint64_t active) {
    uint64_t m = active;
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
        const bool bit = (dig >> b) & 1u;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Per-wave digit counts of the tile into wcnt_w[digit] (this wave's LDS
// sub-histogram).  Counting has no order, so lanes add with LDS atomic adds:
// taking the counts from the ballot groups instead (the leader of each group
// adding its size, no atomic) was measured 0.1 ms slower per iteration at
// 16M keys (B ballots per row of 64 keys against one LDS add per key).
template <int BITS, int ROWS>
__device__ __forceinline__ void tile_counts(const unsigned (&dig)[ROWS], const int64_t row0, int64_t N,
                                            int *wcnt_w) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
        if (row0 + r * 64 + lane < N) atomicAdd(&wcnt_w[dig[r]], 1);
}

// hist[tile * NB + digit] = number of keys of the tile with that digit (one
// contiguous row per tile), summed over the waves' LDS sub-histograms.
template <int BITS, int ROWS>
__global__ __launch_bounds__(kSortThreads) void k_radix_hist(const int32_t *__restrict__ keys, int64_t N, int shift,
                                                             int32_t *__restrict__ hist, int ntiles) {
    constexpr int NB = 1 << BITS;
    __shared__ int wcnt[kSortWaves][NB];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    for (int i = tid; i < kSortWaves * NB; i += kSortThreads) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    constexpr int TILE = kSortWaves * ROWS * 64;
    const int64_t row0 = (int64_t)blockIdx.x * TILE + (int64_t)w * (ROWS * 64);
    unsigned dig[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int64_t i = row0 + r * 64 + lane;
        dig[r] = i < N ? (((unsigned)keys[i] >> shift) & (NB - 1)) : 0u;
    }
    tile_counts<BITS, ROWS>(dig, row0, N, wcnt[w]);
    __syncthreads();
    for (int v = tid; v < NB; v += kSortThreads) {
        int s = 0;
#pragma unroll
        for (int ww = 0; ww < kSortWaves; ++ww) s += wcnt[ww][v];
        hist[(int64_t)blockIdx.x * NB + v] = s;
    }
}

// Stable scatter of one pass.  vals_in == nullptr means value = index.
// The tile is first ordered by digit in LDS (stable), then written out so
// that consecutive threads write consecutive positions of a digit's run: the
// global writes are coalesced instead of one scattered 4-byte write per key.
template <int BITS, int ROWS>
__global__ __launch_bounds__(kSortThreads) void k_radix_scatter(const int32_t *__restrict__ keys_in,
                                                                const int32_t *__restrict__ vals_in, int64_t N,
                                                                int shift, const int32_t *__restrict__ hist_scan,
                                                                const int32_t *__restrict__ dtot, int ntiles,
                                                                int32_t *__restrict__ keys_out,
                                                                int32_t *__restrict__ vals_out) {
    constexpr int NB = 1 << BITS;
    __shared__ int wcnt[kSortWaves][NB];
    __shared__ int dstart[NB];   // first tile-local position of each digit
    __shared__ int gbase[NB];    // global position of each digit's first key of this tile
    constexpr int TILE = kSortWaves * ROWS * 64;
    __shared__ int skey[TILE];
    __shared__ int sval[TILE];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    for (int i = tid; i < kSortWaves * NB; i += kSortThreads) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const int64_t tile0 = (int64_t)blockIdx.x * TILE;
    const int64_t row0 = tile0 + (int64_t)w * (ROWS * 64);
    const int tcount = (int)((N - tile0) < TILE ? (N - tile0) : TILE);
    int32_t key[ROWS], val[ROWS];
    unsigned dig[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int64_t i = row0 + r * 64 + lane;
        const bool valid = i < N;
        key[r] = valid ? keys_in[i] : 0;
        val[r] = valid ? (vals_in != nullptr ? vals_in[i] : (int32_t)i) : 0;
        dig[r] = ((unsigned)key[r] >> shift) & (NB - 1);
    }
    tile_counts<BITS, ROWS>(dig, row0, N, wcnt[w]);
    __syncthreads();
    // exclusive scans of the tile's digit counts and of the whole pass's
    // digit totals (DPT consecutive digits per thread, then across the
    // threads), then each (wave, digit) run start
    {
        constexpr int DPT = NB > kSortThreads ? NB / kSortThreads : 1;
        __shared__ int tot[kSortWaves], all[kSortWaves];
        const int v0 = tid * DPT;
        int t[DPT], g[DPT], ts = 0, gs = 0;
#pragma unroll
        for (int i = 0; i < DPT; ++i) {
            t[i] = 0;
            g[i] = 0;
            if (v0 + i < NB) {
#pragma unroll
                for (int ww = 0; ww < kSortWaves; ++ww) t[i] += wcnt[ww][v0 + i];
                g[i] = dtot[v0 + i];
            }
            ts += t[i];
            gs += g[i];
        }
        // inclusive scans of the thread sums within each wave (shuffles),
        // then of the eight wave totals
        int it = ts, ig = gs;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int a = __shfl_up(it, o), b = __shfl_up(ig, o);
            if (lane >= o) {
                it += a;
                ig += b;
            }
        }
        if (lane == 63) {
            tot[w] = it;
            all[w] = ig;
        }
        __syncthreads();
        int bt = 0, bg = 0;
#pragma unroll
        for (int ww = 0; ww < kSortWaves; ++ww) {
            bt += ww < w ? tot[ww] : 0;
            bg += ww < w ? all[ww] : 0;
        }
        int s = bt + it - ts, ga = bg + ig - gs;  // exclusive, at digit v0
#pragma unroll
        for (int i = 0; i < DPT; ++i) {
            const int v = v0 + i;
            if (v < NB) {
                dstart[v] = s;
                // keys of lower digits, plus keys of this digit in earlier tiles
                gbase[v] = ga + hist_scan[(int64_t)v * ntiles + blockIdx.x];
                int run = s;
#pragma unroll
                for (int ww = 0; ww < kSortWaves; ++ww) {
                    const int c = wcnt[ww][v];
                    wcnt[ww][v] = run;
                    run += c;
                }
            }
            s += t[i];
            ga += g[i];
        }
    }
    __syncthreads();
    int *run = wcnt[w];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const bool valid = row0 + r * 64 + lane < N;
        const uint64_t act = __ballot(valid);
        if (act == 0ull) break;
        const uint64_t m = match_digit<BITS>(dig[r], act);
        const uint64_t below = m & lanemask_lt_s();
        int pos = 0;
        if (valid) pos = run[dig[r]] + __popcll(below);
        // every lane has read its run start before a leader moves it on
        __builtin_amdgcn_wave_barrier();
        if (valid && below == 0ull) run[dig[r]] += __popcll(m);
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            skey[pos] = key[r];
            sval[pos] = val[r];
        }
    }
    __syncthreads();
    for (int i = tid; i < tcount; i += kSortThreads) {
        const int k = skey[i];
        const unsigned dg = ((unsigned)k >> shift) & (NB - 1);
        const int pos = gbase[dg] + (i - dstart[dg]);
        if (keys_out != nullptr) keys_out[pos] = k;
        vals_out[pos] = sval[i];
    }
}

// ---- global digit offsets.  One wave per digit v scans that digit's column
// of tile counts (stride NB in the tile-major histogram; the waves of
// neighbouring digits read the same lines): hscan[v][t] = digit-v keys in the
// tiles before t (digit-major, so the writes are contiguous), dtot[v] = all
// digit-v keys.  The scatter adds the keys of lower digits (a scan of dtot).
// Each lane takes kColPer consecutive tiles of a 64 * kColPer chunk, and the
// lane sums are scanned across the wave with shuffles (no barrier).
constexpr int kColPer = 8;

__global__ __launch_bounds__(256) void k_col_scan(const int32_t *__restrict__ hist, int ntiles, int NB,
                                                  int32_t *__restrict__ hscan, int32_t *__restrict__ dtot) {
    const int lane = threadIdx.x & 63;
    const int v = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (v >= NB) return;
    int32_t *out = hscan + (int64_t)v * ntiles;
    int carry = 0;
    for (int c0 = 0; c0 < ntiles; c0 += 64 * kColPer) {
        const int t0 = c0 + lane * kColPer;
        int x[kColPer];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < kColPer; ++i) {
            x[i] = t0 + i < ntiles ? hist[(int64_t)(t0 + i) * NB + v] : 0;
            sum += x[i];
        }
        int inc = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        int run = carry + inc - sum;
#pragma unroll
        for (int i = 0; i < kColPer; ++i) {
            if (t0 + i < ntiles) out[t0 + i] = run;
            run += x[i];
        }
        carry += __shfl(inc, 63);
    }
    if (lane == 0) dtot[v] = carry;
}

// offsets[k] = first position of key k in the sorted keys (= position of the
// first key >= k); offsets[K] = N.  Each offsets[k] is written by exactly one
// thread: the one at the boundary where the key first reaches k.  A thread
// covers four consecutive positions (one 16-byte load).
__global__ __launch_bounds__(256) void k_offsets(const int32_t *__restrict__ ks, int64_t N, int K,
                                                 int32_t *__restrict__ offsets) {
    const int64_t r0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (r0 > N) return;
    int cur[4];
    if (r0 + 4 <= N) {
        const int4 v = *reinterpret_cast<const int4 *>(ks + r0);
        cur[0] = v.x;
        cur[1] = v.y;
        cur[2] = v.z;
        cur[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = r0 + i < N ? ks[r0 + i] : K;
    }
    int prev = r0 == 0 ? -1 : ks[r0 - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + i;
        if (r > N) break;
        // keys are documented to lie in [0, K); the clamps only keep a bad key
        // from writing outside offsets[0..K]
        const int lo = max(prev + 1, 0);
        const int hi = min(cur[i], K);
        for (int k = lo; k <= hi; ++k) offsets[k] = (int32_t)r;
        prev = cur[i];
    }
}

// ---------------------------------------------------------------------------
static int key_bits(int K) {
    int b = 0;
    while ((1 << b) < K) ++b;
    return b < 1 ? 1 : b;
}

// 64-key rows per wave: tiles of 8 waves x 16 rows (8192 keys) when that
// still leaves at least 512 tiles (two per CU), else shorter tiles, so that a
// small sort still spreads over the chip: 4096 keys while that leaves 256
// tiles (at 2^20 keys: 4 us faster than 512 tiles of 2048), then 2048.
static int sort_rows(int64_t N) {
    if (N >= (int64_t)512 * kSortWaves * 16 * kWave) return 16;
    if (N >= (int64_t)256 * kSortWaves * 8 * kWave) return 8;
    return 4;
}
constexpr int kMinSortTile = kSortWaves * 4 * kWave;

static int64_t ntiles_of(int64_t N) { return cdiv(N, (int64_t)kSortWaves * sort_rows(N) * kWave); }

// keys of up to this many bits are sorted in one pass
constexpr int kOnePassBits = 11;
constexpr int kMaxDigits = 1 << kOnePassBits;

// The histograms of any sort of up to N keys: at most cdiv(N, kMinSortTile)
// tiles (the shortest tiles), each with up to kMaxDigits digits.
size_t sort_scratch_bytes(int64_t N) {
    const int64_t nt = cdiv(N > 0 ? N : 1, kMinSortTile);
    const int64_t hn = (int64_t)kMaxDigits * nt;
    return align_up((size_t)hn * 4, 256) * 2 + align_up((size_t)kMaxDigits * 4, 256);
}

template <int BITS, int ROWS>
static hipError_t radix_pass_rows(const int32_t *kin, const int32_t *vin, int64_t N, int shift, int32_t *kout,
                                  int32_t *vout, int32_t *hist, int32_t *hscan, int32_t *dtot, hipStream_t s) {
    constexpr int NB = 1 << BITS;
    const int nt = (int)ntiles_of(N);
    hipLaunchKernelGGL((k_radix_hist<BITS, ROWS>), dim3(nt), dim3(kSortThreads), 0, s, kin, N, shift, hist, nt);
    hipLaunchKernelGGL(k_col_scan, dim3((NB + 3) / 4), dim3(256), 0, s, hist, nt, NB, hscan, dtot);
    hipLaunchKernelGGL((k_radix_scatter<BITS, ROWS>), dim3(nt), dim3(kSortThreads), 0, s, kin, vin, N, shift, hscan,
                       dtot, nt, kout, vout);
    return hipGetLastError();
}

template <int BITS>
static hipError_t radix_pass(const int32_t *kin, const int32_t *vin, int64_t N, int shift, int32_t *kout,
                             int32_t *vout, int32_t *hist, int32_t *hscan, int32_t *dtot, hipStream_t s) {
    switch (sort_rows(N)) {
    case 16: return radix_pass_rows<BITS, 16>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 8: return radix_pass_rows<BITS, 8>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    default: return radix_pass_rows<BITS, 4>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    }
}

static hipError_t radix_pass_bits(int bits, const int32_t *kin, const int32_t *vin, int64_t N, int shift,
                                  int32_t *kout, int32_t *vout, int32_t *hist, int32_t *hscan, int32_t *dtot,
                                  hipStream_t s) {
    switch (bits) {
    case 11: return radix_pass<11>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 10: return radix_pass<10>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 9: return radix_pass<9>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 1: return radix_pass<1>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 2: return radix_pass<2>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 3: return radix_pass<3>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 4: return radix_pass<4>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 5: return radix_pass<5>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 6: return radix_pass<6>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    case 7: return radix_pass<7>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    default: return radix_pass<8>(kin, vin, N, shift, kout, vout, hist, hscan, dtot, s);
    }
}

hipError_t launch_sort_by_key(const int32_t *keys, int64_t N, int K, int32_t *keys_sorted, int32_t *perm,
                              int32_t *tmp_keys, int32_t *tmp_vals, void *scratch, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    const int64_t nt = cdiv(N, kMinSortTile);
    const int64_t hn = (int64_t)kMaxDigits * nt;
    char *p = (char *)scratch;
    int32_t *hist = (int32_t *)p;
    p += align_up((size_t)hn * 4, 256);
    int32_t *hscan = (int32_t *)p;
    p += align_up((size_t)hn * 4, 256);
    int32_t *dtot = (int32_t *)p;
    const int bits = key_bits(K);
    if (bits <= kOnePassBits)
        return radix_pass_bits(bits, keys, nullptr, N, 0, keys_sorted, perm, hist, hscan, dtot, s);
    hipError_t e = radix_pass_bits(8, keys, nullptr, N, 0, tmp_keys, tmp_vals, hist, hscan, dtot, s);
    if (e != hipSuccess) return e;
    return radix_pass_bits(bits - 8, tmp_keys, tmp_vals, N, 8, keys_sorted, perm, hist, hscan, dtot, s);
}

hipError_t launch_offsets(const int32_t *keys_sorted, int64_t N, int K, int32_t *offsets, hipStream_t s) {
    hipLaunchKernelGGL(k_offsets, dim3((unsigned)cdiv(N / 4 + 1, 256)), dim3(256), 0, s, keys_sorted, N, K, offsets);
    return hipGetLastError();
}

}  // namespace fk
