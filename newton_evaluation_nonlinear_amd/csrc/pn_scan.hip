// The affine scan on its own: out_t = A_t out_{t-1} + b_t for given (A, b),
// with A_t diagonal or dense D x D.  This is the linear-recurrence step that
// the parallel methods of [PN §2.1] reduce every iteration to.  Diagonal A
// runs in one pass with a decoupled look-back; dense A uses the three-phase
// form of the solver: per-chunk composed maps, the carry scan of
// pn_cell.hip, then a per-chunk replay.

#include "pn_device.hpp"

namespace pn {

// ---- diagonal, one pass: decoupled look-back [PN §2.1]
// A workgroup takes the next chunk in ticket order (chunk-major, so every
// chunk's predecessors hold smaller tickets and are already running: the
// waits below always end), loads its L steps of (a, b) per channel into
// registers and composes them into the chunk map, which it publishes at once
// (flag 1).  It then walks back over its predecessors: a predecessor that has
// published its end state (flag 2) ends the walk, one that has only published
// its map is composed in and the walk continues.  With the state entering the
// chunk known, it publishes its own end state (flag 2) and replays its steps
// from registers.  A and b are read once and out written once: 12 bytes per
// element, against 20 for the three-phase form (maps, carry scan, replay).
// Values and flags travel through relaxed device-scope atomics (coherent
// across the XCDs' L2 caches); a flag is stored only after the workgroup's
// value stores have completed.  Every wait is bounded and sets err on a
// timeout.
__device__ __forceinline__ float ld_coh(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(kLbChannels) void scan_diag_lookback(LookbackArgs g) {
    __shared__ uint32_t sh_t, sh_flag;
    const int tid = threadIdx.x;
    if (tid == 0) sh_t = __hip_atomic_fetch_add(g.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t t = sh_t;
    const int per_c = g.B * g.nblk;
    const int c = static_cast<int>(t / per_c);
    const int r = static_cast<int>(t % per_c);
    const int b = r / g.nblk, blk = r % g.nblk;
    const int d = blk * kLbChannels + tid;
    const bool live = d < g.D;
    const int t0 = c * g.L;
    const int n = min(g.L, g.T - t0);
    const size_t base = (static_cast<size_t>(b) * g.T + t0) * g.D + d;
    float a[kLbChunk], bb[kLbChunk];
#pragma unroll
    for (int u = 0; u < kLbChunk; ++u) {
        const bool in = live && u < n;
        a[u] = in ? g.A[base + static_cast<size_t>(u) * g.D] : 1.0f;
        bb[u] = in ? g.b[base + static_cast<size_t>(u) * g.D] : 0.0f;
    }
    float ca = 1.0f, cb = 0.0f;                      // the chunk's map y -> ca y + cb
#pragma unroll
    for (int u = 0; u < kLbChunk; ++u) {
        cb = a[u] * cb + bb[u];
        ca = a[u] * ca;
    }
    const size_t ci = (static_cast<size_t>(b) * g.NC + c) * g.D + d;
    const size_t fi = (static_cast<size_t>(b) * g.NC + c) * g.nblk + blk;
    float carry = live ? g.s0[static_cast<size_t>(b) * g.D + d] : 0.0f;
    if (c > 0) {
        if (live) {
            st_coh(g.aggA + ci, ca);
            st_coh(g.aggB + ci, cb);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) __hip_atomic_store(g.flag + fi, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // walk back: M accumulates the maps of the chunks after k
        float ma = 1.0f, mb = 0.0f;
        for (int k = c - 1; k >= 0; --k) {
            const size_t fk = (static_cast<size_t>(b) * g.NC + k) * g.nblk + blk;
            if (tid == 0) {
                uint32_t f = 0, spins = 0;
                while ((f = __hip_atomic_load(g.flag + fk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0u) {
                    __builtin_amdgcn_s_sleep(1);
                    if (++spins > (1u << 22)) {
                        __hip_atomic_store(g.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        f = 2u;
                        break;
                    }
                }
                sh_flag = f;
            }
            __syncthreads();
            const uint32_t f = sh_flag;
            __syncthreads();
            const size_t ck = (static_cast<size_t>(b) * g.NC + k) * g.D + d;
            if (f == 2u) {
                if (live) carry = ma * ld_coh(g.yv + ck) + mb;
                break;
            }
            if (live) {
                const float ak = ld_coh(g.aggA + ck), bk = ld_coh(g.aggB + ck);
                mb = ma * bk + mb;
                ma = ma * ak;
            }
        }
    }
    // the end state of this chunk for the chunks after it
    if (live) st_coh(g.yv + ci, ca * carry + cb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(g.flag + fi, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // replay from registers
    if (live) {
        float y = carry;
#pragma unroll
        for (int u = 0; u < kLbChunk; ++u) {
            if (u < n) {
                y = a[u] * y + bb[u];
                g.out[base + static_cast<size_t>(u) * g.D] = y;
            }
        }
    }
}

hipError_t launch_scan_lookback(const LookbackArgs& a, hipStream_t st) {
    const int64_t nwg = static_cast<int64_t>(a.NC) * a.B * a.nblk;
    scan_diag_lookback<<<static_cast<unsigned>(nwg), kLbChannels, 0, st>>>(a);
    return hipGetLastError();
}

// ---- diagonal: thread = (b, chunk, channel), serial over the chunk
__global__ __launch_bounds__(kThreads) void scan_diag_aggregate(ScanArgs g) {
    const int e = blockIdx.x * kThreads + threadIdx.x;
    const int d = e % g.D;
    const int c = (e / g.D) % g.NC;
    const int b = e / (g.D * g.NC);
    if (b >= g.B) return;
    const int t0 = c * g.L, t1 = min(t0 + g.L, g.T);
    const size_t base = static_cast<size_t>(b) * g.T * g.D + d;
    float A = 1.0f, Bc = 0.0f;
    for (int t = t0; t < t1; ++t) {
        const float at = g.A[base + static_cast<size_t>(t) * g.D];
        const float bt = g.b[base + static_cast<size_t>(t) * g.D];
        Bc = at * Bc + bt;
        A = at * A;
    }
    const size_t ai = (static_cast<size_t>(b) * g.NC + c) * g.D + d;
    g.aggA[ai] = A;
    g.aggB[ai] = Bc;
}

__global__ __launch_bounds__(kThreads) void scan_diag_apply(ScanArgs g) {
    const int e = blockIdx.x * kThreads + threadIdx.x;
    const int d = e % g.D;
    const int c = (e / g.D) % g.NC;
    const int b = e / (g.D * g.NC);
    if (b >= g.B) return;
    const int t0 = c * g.L, t1 = min(t0 + g.L, g.T);
    const size_t base = static_cast<size_t>(b) * g.T * g.D + d;
    float y = g.carry[(static_cast<size_t>(b) * g.NC + c) * g.D + d];
    for (int t = t0; t < t1; ++t) {
        const size_t o = base + static_cast<size_t>(t) * g.D;
        y = g.A[o] * y + g.b[o];
        g.out[o] = y;
    }
}

// ---- dense: one workgroup per (b, chunk).  The chunk map is the product
// A_{t1-1} ... A_{t0} (and the folded offset), one D x D product per step on
// the matrix cores: M <- A_t M with 16x16x4 FP32 steps, M double-buffered in
// LDS, A_t staged into LDS one step ahead.  Wavefront w owns the output tiles
// (ti, tj) with ti * (DP/16) + tj = w, w + 4, ...; lane l supplies
// A_t[16 ti + l % 16][4 kk + l / 16] and M[4 kk + l / 16][16 tj + l % 16] and
// accumulates rows 16 ti + 4 (l / 16) + r, column 16 tj + l % 16.
typedef float v4f_s __attribute__((ext_vector_type(4)));

template <int DP>
__global__ __launch_bounds__(kThreads) void scan_dense_aggregate(ScanArgs g) {
    constexpr int RS = DP + 1;                   // LDS row stride: rows fall on distinct banks
    constexpr int NT = (DP / 16) * (DP / 16);    // 16 x 16 output tiles
    constexpr int TPW = (NT + 3) / 4;            // tiles per wavefront
    constexpr int PER = (DP * DP + kThreads - 1) / kThreads;   // A_t values each thread stages
    __shared__ float M[2][DP * RS];
    __shared__ float As[2][DP * RS];
    __shared__ float Bv[2][DP];
    const int c = blockIdx.x, b = blockIdx.y, D = g.D;
    const int t0 = c * g.L, t1 = min(t0 + g.L, g.T);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    auto load_step = [&](int t, float (&r)[PER]) {
        const float* At = g.A + (static_cast<size_t>(b) * g.T + t) * D * D;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * kThreads;
            const int i = e / DP, k = e % DP;
            r[u] = (e < DP * DP && i < D && k < D) ? At[i * D + k] : 0.0f;
        }
    };
    auto store_step = [&](float* dst, const float (&r)[PER]) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * kThreads;
            if (e < DP * DP) dst[(e / DP) * RS + (e % DP)] = r[u];
        }
    };
    for (int e = tid; e < DP * RS; e += kThreads) {
        const int i = e / RS, k = e % RS;
        M[0][e] = (i == k) ? 1.0f : 0.0f;
    }
    if (tid < DP) Bv[0][tid] = 0.0f;
    float ra[PER];
    if (t0 < t1) {
        load_step(t0, ra);
        store_step(As[0], ra);
    }
    __syncthreads();
    int cur = 0;
    for (int t = t0; t < t1; ++t) {
        // the next step's A into registers while this step computes
        if (t + 1 < t1) load_step(t + 1, ra);
        const float* A = As[cur];
        const float* Mc = M[cur];
        float* Mn = M[cur ^ 1];
#pragma unroll
        for (int q = 0; q < TPW; ++q) {
            const int tile = wave + 4 * q;
            if (tile < NT) {
                const int ti = tile / (DP / 16), tj = tile % (DP / 16);
                v4f_s acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < DP / 4; ++kk) {
                    const int k = 4 * kk + lq;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(16 * ti + l16) * RS + k],
                                                               Mc[k * RS + 16 * tj + l16], acc, 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) Mn[(16 * ti + 4 * lq + r) * RS + 16 * tj + l16] = acc[r];
            }
        }
        if (tid < DP) {
            float acc = tid < D ? g.b[(static_cast<size_t>(b) * g.T + t) * D + tid] : 0.0f;
#pragma unroll 8
            for (int k = 0; k < DP; ++k) acc += A[tid * RS + k] * Bv[cur][k];
            Bv[cur ^ 1][tid] = acc;
        }
        if (t + 1 < t1) store_step(As[cur ^ 1], ra);
        __syncthreads();
        cur ^= 1;
    }
    const size_t ci = static_cast<size_t>(b) * g.NC + c;
    for (int e = tid; e < D * D; e += kThreads) g.aggA[ci * D * D + e] = M[cur][(e / D) * RS + (e % D)];
    if (tid < D) g.aggB[ci * D + tid] = Bv[cur][tid];
}

// replay of a chunk from its carry: one wavefront, lane i owns row i; the
// next step's row of A is loaded while this step's dot product runs
template <int DP>
__global__ __launch_bounds__(64) void scan_dense_apply(ScanArgs g) {
    __shared__ float y[2][DP];
    const int c = blockIdx.x, b = blockIdx.y, D = g.D;
    const int t0 = c * g.L, t1 = min(t0 + g.L, g.T);
    const int i = threadIdx.x;
    const bool live = i < D;
    if (i < DP) y[0][i] = live ? g.carry[(static_cast<size_t>(b) * g.NC + c) * D + i] : 0.0f;
    float row[DP], nxt[DP];
    auto load_row = [&](int t, float (&r)[DP]) {
        const float* At = g.A + ((static_cast<size_t>(b) * g.T + t) * D + (live ? i : 0)) * D;
#pragma unroll
        for (int k = 0; k < DP; ++k) r[k] = (live && k < D) ? At[k] : 0.0f;
    };
    if (t0 < t1) load_row(t0, row);
    __syncthreads();
    int cur = 0;
    for (int t = t0; t < t1; ++t) {
        if (t + 1 < t1) load_row(t + 1, nxt);
        const size_t o = (static_cast<size_t>(b) * g.T + t) * D + i;
        float acc = live ? g.b[o] : 0.0f;
#pragma unroll
        for (int k = 0; k < DP; ++k) acc += row[k] * y[cur][k];
        if (i < DP) y[cur ^ 1][i] = acc;
        if (live) g.out[o] = acc;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < DP; ++k) row[k] = nxt[k];
        cur ^= 1;
    }
}

hipError_t launch_scan_aggregate(bool dense, int DP, const ScanArgs& a, hipStream_t st) {
    if (!dense) {
        const int64_t n = static_cast<int64_t>(a.B) * a.NC * a.D;
        scan_diag_aggregate<<<static_cast<int>((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(a);
    } else {
        const dim3 grid(a.NC, a.B);
        switch (DP) {
            case 4: case 8: case 16: scan_dense_aggregate<16><<<grid, kThreads, 0, st>>>(a); break;
            case 32: scan_dense_aggregate<32><<<grid, kThreads, 0, st>>>(a); break;
            case 64: scan_dense_aggregate<64><<<grid, kThreads, 0, st>>>(a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

hipError_t launch_scan_apply(bool dense, int DP, const ScanArgs& a, hipStream_t st) {
    if (!dense) {
        const int64_t n = static_cast<int64_t>(a.B) * a.NC * a.D;
        scan_diag_apply<<<static_cast<int>((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(a);
    } else {
        const dim3 grid(a.NC, a.B);
        switch (DP) {
            case 4: scan_dense_apply<4><<<grid, 64, 0, st>>>(a); break;
            case 8: scan_dense_apply<8><<<grid, 64, 0, st>>>(a); break;
            case 16: scan_dense_apply<16><<<grid, 64, 0, st>>>(a); break;
            case 32: scan_dense_apply<32><<<grid, 64, 0, st>>>(a); break;
            case 64: scan_dense_apply<64><<<grid, 64, 0, st>>>(a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace pn
