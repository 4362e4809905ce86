// On-box microbenchmarks behind the roofline peaks the benchmark reports
// beside the published ones: HBM streaming, the row gather of the segmented
// reduction, and back-to-back matrix products (bf16 and fp32) with the clock
// they ran at.  Measurement only: nothing on the library's path calls these.
// Each entry point enqueues on `stream` and returns the launch status; the
// caller times the work (events) and synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// dst[i] = src[i] for n float4s (n a multiple of 4 * 256 * gridDim.x):
// each thread moves four float4s per round, all four loads in flight.
__global__ __launch_bounds__(256) void k_stream_copy(const f4 *__restrict__ src, f4 *__restrict__ dst,
                                                     int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
        f4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
}

// Reads n float4s (n a multiple of 4 * 256 * gridDim.x), four in flight per
// thread, and writes one float per workgroup (so the reads stay).
__global__ __launch_bounds__(256) void k_stream_read(const f4 *__restrict__ src, int64_t n,
                                                     float *__restrict__ out) {
    __shared__ float part[4];
    const int64_t stride = (int64_t)gridDim.x * 256;
    float s = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
        f4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) s += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

// The segmented reduction's access pattern: rows X[perm[r]] of d floats (d a
// multiple of 4 dividing 256, or a multiple of 256), one wave per run of
// `rows_per_wave` consecutive r; a wave reads 64 / (d / 4) rows at a time
// (each row with consecutive lanes, 16 bytes each), eight such steps in
// flight, and sums in fp64 per lane; each wave writes its lanes' sums once.
__global__ __launch_bounds__(256) void k_gather_rows_sum(const float *__restrict__ X, const int32_t *__restrict__ perm,
                                                         int64_t N, int d, int rows_per_wave, double *__restrict__ out) {
    constexpr int U = 8;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t r0 = wave * rows_per_wave;
    if (r0 >= N) return;
    const int64_t r1 = r0 + rows_per_wave < N ? r0 + rows_per_wave : N;
    const int q4 = d / 4;
    const int per = q4 >= 64 ? 1 : 64 / q4;           // rows per step
    const int sub = q4 >= 64 ? 0 : lane / q4;         // this lane's row in the step
    const int j0 = q4 >= 64 ? lane : lane % q4;       // its first float4 of the row
    const int jstep = q4 >= 64 ? 64 : q4;
    double acc = 0.0;
    for (int64_t r = r0; r < r1; r += (int64_t)per * U) {
        f4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int64_t rr = r + (int64_t)u * per + sub;
            if (rr >= r1) rr = r1 - 1;
            const f4 *row = reinterpret_cast<const f4 *>(X + (int64_t)perm[rr] * d);
            v[u] = __builtin_nontemporal_load(row + j0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc += (double)((v[u].x + v[u].y) + (v[u].z + v[u].w));
        for (int j = j0 + jstep; j < q4; j += jstep) {  // rows longer than 256 floats
            for (int u = 0; u < U; ++u) {
                int64_t rr = r + (int64_t)u * per + sub;
                if (rr >= r1) rr = r1 - 1;
                const f4 t = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(X + (int64_t)perm[rr] * d) + j);
                acc += (double)((t.x + t.y) + (t.z + t.w));
            }
        }
    }
    out[wave * 64 + lane] = acc;
}

// Back-to-back matrix products on register operands: four independent
// accumulators per wave, `iters` rounds of four products each.  Lane 0 of
// every wave records the shader clock and the 100 MHz real-time counter
// around its loop; out receives per wave (cycles, ticks) and the sum of the
// accumulators (so the products are not removed).
__global__ __launch_bounds__(256) void k_mfma_bf16(int iters, uint64_t *__restrict__ clocks, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    v8bf a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(lane - i));
    }
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (lane == 0) {
        clocks[2 * wave] = t1 - t0;
        clocks[2 * wave + 1] = r1 - r0;
    }
    sink[wave * 64 + lane] = s;
}

__global__ __launch_bounds__(256) void k_mfma_f32(int iters, uint64_t *__restrict__ clocks, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const float a = 0.001f * (float)lane, b = 0.002f * (float)(lane - 3);
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c3, 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += (c0[i] + c1[i]) + (c2[i] + c3[i]);
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (lane == 0) {
        clocks[2 * wave] = t1 - t0;
        clocks[2 * wave + 1] = r1 - r0;
    }
    sink[wave * 64 + lane] = s;
}

}  // namespace

extern "C" {

// n_float4 must be a multiple of 4 * 256 * blocks
int fkm_stream_copy(const void *src, void *dst, int64_t n_float4, int blocks, void *stream) {
    if (blocks < 1 || n_float4 % ((int64_t)4 * 256 * blocks) != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_stream_copy, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const f4 *)src,
                       (f4 *)dst, n_float4);
    return (int)hipGetLastError();
}

int fkm_stream_read(const void *src, int64_t n_float4, float *out, int blocks, void *stream) {
    if (blocks < 1 || n_float4 % ((int64_t)4 * 256 * blocks) != 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_stream_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const f4 *)src, n_float4,
                       out);
    return (int)hipGetLastError();
}

// out: 64 doubles per wave, cdiv(N, rows_per_wave) waves
int fkm_gather_rows(const float *X, const int32_t *perm, int64_t N, int d, int rows_per_wave, double *out,
                    void *stream) {
    if (d % 4 != 0 || rows_per_wave < 1 || (d < 256 && 256 % d != 0) || (d > 256 && d % 256 != 0))
        return (int)hipErrorInvalidValue;
    const int64_t waves = (N + rows_per_wave - 1) / rows_per_wave;
    hipLaunchKernelGGL(k_gather_rows_sum, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, (hipStream_t)stream, X,
                       perm, N, d, rows_per_wave, out);
    return (int)hipGetLastError();
}

// clocks: 2 per wave (4 waves per block), sink: 64 floats per wave
int fkm_mfma(int bf16, int blocks, int iters, uint64_t *clocks, float *sink, void *stream) {
    if (bf16)
        hipLaunchKernelGGL(k_mfma_bf16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, clocks, sink);
    else
        hipLaunchKernelGGL(k_mfma_f32, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, clocks, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
