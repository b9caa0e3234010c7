// Ceiling microbenchmarks: what plain streaming kernels and a plain FP32
// matrix-core loop attain on this GPU, measured with HIP events.  They give
// the solver's kernels a measured ceiling next to the data-sheet peaks
// (HBM 8 TB/s, FP32 matrix 157.3 TFLOP/s).
//
// Patterns (bytes moved per repetition in brackets, n = bytes per array):
//   PNC_READ       sum of one array                          [n]
//   PNC_WRITE      fill of one array                         [n]
//   PNC_COPY       y = x                                     [2n]
//   PNC_2R1W       s = x + 0.5 s, flat float4 grid stride    [3n]
//   PNC_2R1W_ROWS  s = x + 0.5 s in the access order of the channel-wise
//                  apply kernel: [8, T, 256] float arrays, one workgroup per
//                  (batch row, 1024-step chunk), one channel per thread, rows
//                  walked in order with 8-step register prefetch      [3n]
//   PNC_READ_ROWS  sum of x in the access order of the channel-wise sweeps
//                  that read only x: [8, T, 256], one workgroup per (batch
//                  row, 512-step chunk), one channel per thread, rows in
//                  order, 16 rows in flight while the previous 16 are summed [n]
// The MFMA loop runs independent chains of v_mfma_f32_32x32x2f32 on register
// operands (4096 flops each) on every SIMD.
//
// The sequential reference is the plain time loop of the channel-wise cell
// s_t = tanh(a s_{t-1} + x_t): one thread per (batch row, channel) walks
// t = 1..T in order, the loads 16 steps ahead of use.  It is the GPU baseline
// that a parallel-in-time solve of the same recurrence has to beat.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <functional>
#include <string>
#include <vector>

#include "../../include/pn_ceiling.h"

namespace {

thread_local std::string g_err;

int fail(const char* what, hipError_t e) {
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return -1;
}

#define PNC_HIP(call)                          \
    do {                                       \
        hipError_t e_ = (call);                \
        if (e_ != hipSuccess) return fail(#call, e_); \
    } while (0)

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_read(const float4* __restrict__ x, size_t n4, float* __restrict__ out) {
    float acc = 0.0f;
    for (size_t i = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; i < n4;
         i += static_cast<size_t>(gridDim.x) * kThreads) {
        const float4 v = x[i];
        acc += (v.x + v.y) + (v.z + v.w);
    }
    out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void k_write(float4* __restrict__ y, size_t n4) {
    const float4 v = make_float4(1.0f, 2.0f, 3.0f, 4.0f);
    for (size_t i = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; i < n4;
         i += static_cast<size_t>(gridDim.x) * kThreads)
        y[i] = v;
}

__global__ __launch_bounds__(kThreads) void k_copy(const float4* __restrict__ x, float4* __restrict__ y, size_t n4) {
    for (size_t i = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; i < n4;
         i += static_cast<size_t>(gridDim.x) * kThreads)
        y[i] = x[i];
}

__global__ __launch_bounds__(kThreads) void k_2r1w(const float4* __restrict__ x, float4* __restrict__ s, size_t n4) {
    for (size_t i = blockIdx.x * static_cast<size_t>(kThreads) + threadIdx.x; i < n4;
         i += static_cast<size_t>(gridDim.x) * kThreads) {
        const float4 a = x[i], b = s[i];
        s[i] = make_float4(a.x + 0.5f * b.x, a.y + 0.5f * b.y, a.z + 0.5f * b.z, a.w + 0.5f * b.w);
    }
}

// [B][T][D] with D = 256: block (chunk c, batch row b), thread = channel
constexpr int kRowsD = 256, kRowsB = 8, kRowsL = 1024, kPre = 8;

__global__ __launch_bounds__(kThreads) void k_2r1w_rows(const float* __restrict__ x, float* __restrict__ s, int T) {
    const int c = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int t0 = c * kRowsL;
    const int n = min(kRowsL, T - t0);
    const size_t base = (static_cast<size_t>(b) * T + t0) * kRowsD + d;
    const float* xp = x + base;
    float* sp = s + base;
    int t = 0;
    for (; t + kPre <= n; t += kPre) {
        float xv[kPre], sv[kPre];
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            xv[u] = xp[static_cast<size_t>(t + u) * kRowsD];
            sv[u] = sp[static_cast<size_t>(t + u) * kRowsD];
        }
#pragma unroll
        for (int u = 0; u < kPre; ++u) sp[static_cast<size_t>(t + u) * kRowsD] = xv[u] + 0.5f * sv[u];
    }
    for (; t < n; ++t) sp[static_cast<size_t>(t) * kRowsD] = xp[static_cast<size_t>(t) * kRowsD] + 0.5f * sp[static_cast<size_t>(t) * kRowsD];
}

constexpr int kReadL = 512, kReadPre = 16;

__global__ __launch_bounds__(kThreads) void k_read_rows(const float* __restrict__ x, float* __restrict__ out, int T) {
    const int c = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int t0 = c * kReadL;
    const int n = min(kReadL, T - t0);
    const float* xp = x + (static_cast<size_t>(b) * T + t0) * kRowsD + d;
    float acc = 0.0f;
    float xa[kReadPre], xb[kReadPre];
#pragma unroll
    for (int u = 0; u < kReadPre; ++u) xa[u] = u < n ? xp[static_cast<size_t>(u) * kRowsD] : 0.0f;
    for (int t = 0; t < n; t += 2 * kReadPre) {
#pragma unroll
        for (int u = 0; u < kReadPre; ++u) {
            const int r = t + kReadPre + u;
            xb[u] = r < n ? xp[static_cast<size_t>(r) * kRowsD] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kReadPre; ++u) acc += xa[u];
#pragma unroll
        for (int u = 0; u < kReadPre; ++u) {
            const int r = t + 2 * kReadPre + u;
            xa[u] = r < n ? xp[static_cast<size_t>(r) * kRowsD] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kReadPre; ++u) acc += xb[u];
    }
    out[(static_cast<size_t>(b) * gridDim.x + c) * kThreads + d] = acc;
}

// tanh(u) = 1 - 2 / (e^{2u} + 1), e^{2u} as exp2 of 2u log2(e)
__device__ __forceinline__ float seq_tanh(float u) {
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(u * 2.88539008177792681472f) + 1.0f);
}

constexpr int kSeqPre = 16;

__global__ __launch_bounds__(64) void k_seq_tanh(const float* __restrict__ x, const float* __restrict__ a,
                                                 const float* __restrict__ s0, float* __restrict__ out, int T, int D) {
    const int d = blockIdx.x * 64 + threadIdx.x, b = blockIdx.y;
    if (d >= D) return;
    const float ad = a[d];
    float st = s0[static_cast<size_t>(b) * D + d];
    const float* xp = x + static_cast<size_t>(b) * T * D + d;
    float* op = out + static_cast<size_t>(b) * T * D + d;
    float xa[kSeqPre], xb[kSeqPre];
#pragma unroll
    for (int u = 0; u < kSeqPre; ++u) xa[u] = u < T ? xp[static_cast<size_t>(u) * D] : 0.0f;
    for (int t = 0; t < T; t += kSeqPre) {
#pragma unroll
        for (int u = 0; u < kSeqPre; ++u) {
            const int r = t + kSeqPre + u;
            xb[u] = r < T ? xp[static_cast<size_t>(r) * D] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kSeqPre; ++u) {
            if (t + u < T) {
                st = seq_tanh(ad * st + xa[u]);
                op[static_cast<size_t>(t + u) * D] = st;
            }
        }
#pragma unroll
        for (int u = 0; u < kSeqPre; ++u) xa[u] = xb[u];
    }
}

typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kMfmaChains = 4;

__global__ __launch_bounds__(kThreads) void k_mfma(int iters, float* __restrict__ out) {
    v16f acc[kMfmaChains];
#pragma unroll
    for (int q = 0; q < kMfmaChains; ++q) acc[q] = v16f{};
    const float a = 1.0f + 1e-7f * threadIdx.x, b = 1.0f - 1e-7f * threadIdx.x;
    for (int k = 0; k < iters; ++k) {
#pragma unroll
        for (int q = 0; q < kMfmaChains; ++q) acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[q], 0, 0, 0);
    }
    float r = 0.0f;
#pragma unroll
    for (int q = 0; q < kMfmaChains; ++q) {
#pragma unroll
        for (int e = 0; e < 16; ++e) r += acc[q][e];
    }
    out[blockIdx.x * kThreads + threadIdx.x] = r;
}

int timed(hipStream_t st, int reps, const std::function<void()>& launch, std::vector<float>* ms) {
    hipEvent_t e0, e1;
    PNC_HIP(hipEventCreate(&e0));
    PNC_HIP(hipEventCreate(&e1));
    launch();          // warm-up
    PNC_HIP(hipGetLastError());
    PNC_HIP(hipStreamSynchronize(st));
    for (int r = 0; r < reps; ++r) {
        PNC_HIP(hipEventRecord(e0, st));
        launch();
        PNC_HIP(hipEventRecord(e1, st));
        PNC_HIP(hipEventSynchronize(e1));
        float t = 0.0f;
        PNC_HIP(hipEventElapsedTime(&t, e0, e1));
        ms->push_back(t);
    }
    PNC_HIP(hipGetLastError());
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return 0;
}

void best_median(std::vector<float> ms, double work, double* best, double* median) {
    std::sort(ms.begin(), ms.end());
    *best = work / (ms.front() * 1e-3);
    *median = work / (ms[ms.size() / 2] * 1e-3);
}

}  // namespace

extern "C" {

int pnc_hbm(int pattern, size_t bytes, int reps, double* best_gbs, double* median_gbs) {
    g_err.clear();
    if (!best_gbs || !median_gbs || reps < 1 || pattern < PNC_READ || pattern > PNC_READ_ROWS) {
        g_err = "bad argument";
        return -1;
    }
    int dev = 0, cus = 0;
    PNC_HIP(hipGetDevice(&dev));
    PNC_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    size_t n4 = bytes / 16;
    int T = 0;
    if (pattern == PNC_2R1W_ROWS || pattern == PNC_READ_ROWS) {
        T = static_cast<int>(bytes / (sizeof(float) * kRowsB * kRowsD));
        T = std::max(kRowsL, T / kRowsL * kRowsL);
        n4 = static_cast<size_t>(kRowsB) * T * kRowsD / 4;
    }
    const size_t nbytes = n4 * 16;
    hipStream_t st;
    PNC_HIP(hipStreamCreate(&st));
    float *x = nullptr, *y = nullptr, *out = nullptr;
    const int grid = cus * 8;
    // one partial sum per thread of either reading kernel
    const size_t nout = std::max<size_t>(static_cast<size_t>(grid), static_cast<size_t>(T / kReadL) * kRowsB) * kThreads;
    PNC_HIP(hipMalloc(&x, nbytes));
    PNC_HIP(hipMalloc(&y, nbytes));
    PNC_HIP(hipMalloc(&out, sizeof(float) * nout));
    PNC_HIP(hipMemsetAsync(x, 0, nbytes, st));
    PNC_HIP(hipMemsetAsync(y, 0, nbytes, st));
    std::vector<float> ms;
    double moved = 0.0;
    int rc = 0;
    switch (pattern) {
        case PNC_READ:
            moved = nbytes;
            rc = timed(st, reps, [&] { k_read<<<grid, kThreads, 0, st>>>(reinterpret_cast<const float4*>(x), n4, out); }, &ms);
            break;
        case PNC_WRITE:
            moved = nbytes;
            rc = timed(st, reps, [&] { k_write<<<grid, kThreads, 0, st>>>(reinterpret_cast<float4*>(y), n4); }, &ms);
            break;
        case PNC_COPY:
            moved = 2.0 * nbytes;
            rc = timed(st, reps, [&] { k_copy<<<grid, kThreads, 0, st>>>(reinterpret_cast<const float4*>(x), reinterpret_cast<float4*>(y), n4); }, &ms);
            break;
        case PNC_2R1W:
            moved = 3.0 * nbytes;
            rc = timed(st, reps, [&] { k_2r1w<<<grid, kThreads, 0, st>>>(reinterpret_cast<const float4*>(x), reinterpret_cast<float4*>(y), n4); }, &ms);
            break;
        case PNC_READ_ROWS:
            moved = nbytes;
            rc = timed(st, reps, [&] { k_read_rows<<<dim3(T / kReadL, kRowsB), kThreads, 0, st>>>(x, out, T); }, &ms);
            break;
        default:
            moved = 3.0 * nbytes;
            rc = timed(st, reps, [&] { k_2r1w_rows<<<dim3(T / kRowsL, kRowsB), kThreads, 0, st>>>(x, y, T); }, &ms);
            break;
    }
    (void)hipStreamSynchronize(st);
    (void)hipFree(x);
    (void)hipFree(y);
    (void)hipFree(out);
    (void)hipStreamDestroy(st);
    if (rc != 0) return rc;
    best_median(ms, moved / 1e9, best_gbs, median_gbs);
    return 0;
}

int pnc_mfma_f32(int reps, double* best_tflops, double* median_tflops) {
    g_err.clear();
    if (!best_tflops || !median_tflops || reps < 1) {
        g_err = "bad argument";
        return -1;
    }
    int dev = 0, cus = 0;
    PNC_HIP(hipGetDevice(&dev));
    PNC_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    hipStream_t st;
    PNC_HIP(hipStreamCreate(&st));
    const int grid = cus * 2;            // 8 wavefronts per CU, two per SIMD
    const int iters = 4096;
    float* out = nullptr;
    PNC_HIP(hipMalloc(&out, sizeof(float) * grid * kThreads));
    std::vector<float> ms;
    const int rc = timed(st, reps, [&] { k_mfma<<<grid, kThreads, 0, st>>>(iters, out); }, &ms);
    (void)hipStreamSynchronize(st);
    (void)hipFree(out);
    (void)hipStreamDestroy(st);
    if (rc != 0) return rc;
    const double flops = static_cast<double>(grid) * (kThreads / 64) * iters * kMfmaChains * 4096.0;
    best_median(ms, flops / 1e12, best_tflops, median_tflops);
    return 0;
}

int pnc_sequential_tanh(const float* x, const float* a, const float* s0, float* out, int B, int T, int D, int reps,
                        double* best_ms, double* median_ms) {
    g_err.clear();
    if (!x || !a || !s0 || !out || !best_ms || !median_ms || B < 1 || T < 1 || D < 1 || reps < 1 ||
        B > 65535) {
        g_err = "bad argument";
        return -1;
    }
    hipStream_t st;
    PNC_HIP(hipStreamCreate(&st));
    std::vector<float> ms;
    const dim3 grid((D + 63) / 64, B);
    const int rc = timed(st, reps, [&] { k_seq_tanh<<<grid, 64, 0, st>>>(x, a, s0, out, T, D); }, &ms);
    (void)hipStreamSynchronize(st);
    (void)hipStreamDestroy(st);
    if (rc != 0) return rc;
    std::sort(ms.begin(), ms.end());
    *best_ms = ms.front();
    *median_ms = ms[ms.size() / 2];
    return 0;
}

const char* pnc_last_error(void) { return g_err.c_str(); }

}  // extern "C"
