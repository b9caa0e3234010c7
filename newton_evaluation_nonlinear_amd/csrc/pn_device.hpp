// Device helpers: transcendental functions, residual bit-max reductions and
// the convergence check shared by the carry kernels.
#pragma once

#include "pn_internal.hpp"

namespace pn {

enum { kJacobi = 0, kPicard = 1, kQuasiNewton = 2, kNewton = 3 };
enum { kStOk = 0, kStNotConverged = 1, kStNonFinite = 2 };

// tanh u = 1 - 2 / (e^{2u} + 1).  e^{2u} is the hardware base-2 exponential
// of 2u*log2(e); the reciprocal is the hardware one.  Saturates correctly
// (e -> inf gives 1, e -> 0 gives -1) and propagates NaN.  Absolute error is
// a few 1e-8 plus the final rounding (tested against float64 tanh).
__device__ __forceinline__ float tanh_f(float u) {
    const float e = __builtin_amdgcn_exp2f(u * 2.88539008177792681472f);
    return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// logistic sigmoid 1 / (1 + e^{-u}), same building blocks.
__device__ __forceinline__ float sigmoid_f(float u) {
    const float e = __builtin_amdgcn_exp2f(u * -1.44269504088896340736f);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// |v| as an unsigned bit pattern.  For non-negative floats the unsigned order
// is the numeric order, and every NaN/Inf pattern is >= 0x7f800000, so an
// integer max is an exact, order-independent, NaN-preserving max of |v|.
__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7fffffffu; }

// ---------------------------------------------------------------- staging
// Global -> LDS copies by all NT threads of a workgroup.  Each thread issues
// KB loads before the matching LDS stores, so KB loads per thread are in
// flight instead of one (a plain copy loop waits for every load).

// dst[e] = src[e], e < n.  Uses 16-byte accesses when both sides allow it.
// tid: the caller's index among the NT copying threads (default threadIdx.x).
template <int NT, int KB = 8>
__device__ __forceinline__ void copy_to_lds(float* dst, const float* __restrict__ src, int n, int tid = -1) {
    const int t = tid < 0 ? static_cast<int>(threadIdx.x) : tid;
    const bool v4 = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    int done = 0;
    if (v4) {
        const int n4 = n >> 2;
        const float4* s4 = reinterpret_cast<const float4*>(src);
        float4* d4 = reinterpret_cast<float4*>(dst);
        for (int base = 0; base < n4; base += NT * KB) {
            float4 v[KB];
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const int e = base + u * NT + t;
                v[u] = e < n4 ? s4[e] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int u = 0; u < KB; ++u) {
                const int e = base + u * NT + t;
                if (e < n4) d4[e] = v[u];
            }
        }
        done = n4 << 2;
    }
    for (int base = done; base < n; base += NT * KB) {
        float v[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int e = base + u * NT + t;
            v[u] = e < n ? src[e] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int e = base + u * NT + t;
            if (e < n) dst[e] = v[u];
        }
    }
}

// rows x cols block of a row-major global array (row stride src_stride) into
// LDS rows of dst_stride >= cols floats; columns [cols, dst_stride) are zeroed.
template <int NT, int KB = 8>
__device__ __forceinline__ void copy_rows_to_lds(float* dst, int dst_stride, const float* __restrict__ src,
                                                 int64_t src_stride, int rows, int cols, int tid = -1) {
    const int t = tid < 0 ? static_cast<int>(threadIdx.x) : tid;
    const int n = rows * dst_stride;
    for (int base = 0; base < n; base += NT * KB) {
        float v[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int e = base + u * NT + t;
            const int r = e / dst_stride, q = e - r * dst_stride;
            v[u] = (e < n && q < cols) ? src[r * src_stride + q] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int e = base + u * NT + t;
            if (e < n) dst[e] = v[u];
        }
    }
}

// Diagonal coefficient of the affine map for the diagonal modes.
template <int MODE>
__device__ __forceinline__ float mode_coef(float jac_diag) {
    if constexpr (MODE == kJacobi) return 0.0f;
    else if constexpr (MODE == kPicard) return 1.0f;
    else return jac_diag;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64));
        v = v > o ? v : o;
    }
    return v;
}

// Max over the workgroup (blockDim.x a multiple of 64, <= 1024); every thread
// must call it.  Returns the result in all threads.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v) {
    __shared__ uint32_t red[16];
    v = wave_max_u32(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) red[wid] = v;
    __syncthreads();
    const int nw = blockDim.x >> 6;
    uint32_t r = 0;
    for (int k = 0; k < nw; ++k) r = r > red[k] ? r : red[k];
    __syncthreads();
    return r;
}

// Convergence decision for iteration i, taken by one workgroup: reduce the
// per-block maxima of the previous pass, apply the stop rule (non-finite,
// then r <= tol, then i == max_iter) and publish it to the device control
// word and to the pinned host record.
// The stop rule on the reduced residual bits m: -1 (continue) or a status.
__device__ __forceinline__ int check_status(uint32_t m, const CheckArgs& c) {
    if (m >= kNonFiniteBits) return kStNonFinite;
    if (__uint_as_float(m) <= c.tol) return kStOk;
    if (c.iter >= c.max_iter) return kStNotConverged;
    return -1;
}

// Publish a decision to the device control word and the pinned host record
// (payload, then epoch, then iter).  One thread.  The record's words are
// written with system-scope stores, which go past the compute die's caches
// to the host memory; waiting for each group of stores to complete before
// the next is issued orders them for the host.  No cache-wide fence: the
// workgroups still running beside this one keep their cached data.
__device__ __forceinline__ void publish_check(const CheckArgs& c, uint32_t m, int st, uint32_t first) {
    const int stop = st >= 0 ? 1 : 0;
    c.ctrl->stop = stop;
    c.ctrl->status = st;
    c.ctrl->iter = c.iter;
    c.ctrl->r_bits = m;
    __hip_atomic_store(&c.host->r_bits, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&c.host->first, first, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&c.host->status, st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(&c.host->stop, stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __hip_atomic_store(&c.host->epoch, c.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __hip_atomic_store(&c.host->iter, c.iter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// With c.advancing the check only reduces (residual max and the first step
// over tol) and publishes; the host takes the decision and the device loop
// keeps running.
__device__ __forceinline__ void run_check(const CheckArgs& c) {
    uint32_t m = 0, nf = 0;   // nf: bitwise NOT of the first failing step (max of ~f = min of f)
    for (int k = threadIdx.x; k < c.nparts; k += blockDim.x) {
        const uint32_t v = c.rpart[k];
        m = m > v ? m : v;
        if (c.fpart) {
            const uint32_t f = ~c.fpart[k];
            nf = nf > f ? nf : f;
        }
    }
    m = block_max_u32(m);
    if (c.fpart) nf = block_max_u32(nf);
    if (threadIdx.x == 0) publish_check(c, m, c.advancing ? -1 : check_status(m, c), ~nf);
}

}  // namespace pn
