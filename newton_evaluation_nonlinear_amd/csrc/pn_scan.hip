// The affine scan on its own: out_t = A_t out_{t-1} + b_t for given (A, b),
// with A_t diagonal or dense D x D.  This is the linear-recurrence step that
// the parallel methods of [PN §2.1] reduce every iteration to; it uses the
// same chunk decomposition as the solver: per-chunk composed maps, the carry
// scan of pn_diag.hip / pn_cell.hip, then a per-chunk replay.

#include "pn_device.hpp"

namespace pn {

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

// ---- dense: one workgroup per (b, chunk); thread i owns row i
template <int DP>
__global__ __launch_bounds__(kThreads) void scan_dense_aggregate(ScanArgs g) {
    __shared__ float M[2][DP * DP];
    __shared__ float Bv[2][DP];
    const int c = blockIdx.x, b = blockIdx.y, D = g.D;
    const int t0 = c * g.L, t1 = min(t0 + g.L, g.T);
    const int tid = threadIdx.x;
    for (int e = tid; e < DP * DP; e += kThreads) {
        M[0][e] = ((e / DP) == (e % DP) && (e / DP) < D) ? 1.0f : 0.0f;
        M[1][e] = 0.0f;
    }
    if (tid < DP) { Bv[0][tid] = 0.0f; Bv[1][tid] = 0.0f; }
    __syncthreads();
    constexpr int NCG = kThreads / DP;
    const int i = tid % DP, cg = tid / DP;
    int cur = 0;
    for (int t = t0; t < t1; ++t) {
        const float* At = g.A + ((static_cast<size_t>(b) * g.T + t) * D + i) * D;   // row i
        if (i < D) {
            for (int col = cg; col < D; col += NCG) {
                float acc = 0.0f;
                for (int k = 0; k < D; ++k) acc += At[k] * M[cur][k * DP + col];
                M[cur ^ 1][i * DP + col] = acc;
            }
            if (cg == 0) {
                float acc = g.b[(static_cast<size_t>(b) * g.T + t) * D + i];
                for (int k = 0; k < D; ++k) acc += At[k] * Bv[cur][k];
                Bv[cur ^ 1][i] = acc;
            }
        }
        __syncthreads();
        cur ^= 1;
    }
    const size_t ci = static_cast<size_t>(b) * g.NC + c;
    for (int e = tid; e < D * D; e += kThreads) g.aggA[ci * D * D + e] = M[cur][(e / D) * DP + (e % D)];
    if (tid < D) g.aggB[ci * D + tid] = Bv[cur][tid];
}

template <int DP>
__global__ __launch_bounds__(64) void scan_dense_apply(ScanArgs g) {
    __shared__ float y[DP];
    const int c = blockIdx.x, b = blockIdx.y, D = g.D;
    const int t0 = c * g.L, t1 = min(t0 + g.L, g.T);
    const int i = threadIdx.x;
    if (i < D) y[i] = g.carry[(static_cast<size_t>(b) * g.NC + c) * D + i];
    __syncthreads();
    for (int t = t0; t < t1; ++t) {
        const size_t row = (static_cast<size_t>(b) * g.T + t) * D;
        float acc = 0.0f;
        if (i < D) {
            const float* At = g.A + (row + i) * D;
            acc = g.b[row + i];
            for (int k = 0; k < D; ++k) acc += At[k] * y[k];
        }
        __syncthreads();
        if (i < D) {
            y[i] = acc;
            g.out[row + i] = acc;
        }
        __syncthreads();
    }
}

hipError_t launch_scan_aggregate(bool dense, int DP, const ScanArgs& a, hipStream_t st) {
    if (!dense) {
        const int64_t n = static_cast<int64_t>(a.B) * a.NC * a.D;
        scan_diag_aggregate<<<static_cast<int>((n + kThreads - 1) / kThreads), kThreads, 0, st>>>(a);
    } else {
        const dim3 grid(a.NC, a.B);
        switch (DP) {
            case 4: scan_dense_aggregate<4><<<grid, kThreads, 0, st>>>(a); break;
            case 8: scan_dense_aggregate<8><<<grid, kThreads, 0, st>>>(a); break;
            case 16: scan_dense_aggregate<16><<<grid, kThreads, 0, st>>>(a); break;
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
