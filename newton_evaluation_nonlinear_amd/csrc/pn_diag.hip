// Channel-wise cell f(p, x) = tanh(a * p + x): fused iteration kernel, the
// diagonal carry scan with the convergence check, and the fill kernel.
//
// One iteration of [PN §1.2] with a diagonal A~_t is, per channel, the
// recurrence s^_t = v_t + a~_t (s^_{t-1} - p_t) (see include/pn.h).  The time
// axis is cut into chunks of L steps; a chunk's affine maps y -> a~ y + b~
// compose into one map (prod a~, folded b~) [PN §2.1], so the work per
// iteration is:
//   carry  : scan of the chunk maps -> s^ entering every chunk (tiny)
//   apply  : per chunk, replay s^ from the carry, damp, store s^(i+1), and
//            in the same sweep evaluate the maps of iteration i+1 at the new
//            iterate: residual |s_t - f_t(s_{t-1})| and the chunk's next map.
// The apply sweep therefore moves exactly x, s^(i) in and s^(i+1) out, and
// the following carry only touches the chunk maps.
//
// Layout: lanes run along channels (row-contiguous in [B, T, D]); each thread
// walks the L steps of its chunk serially, so loads are fully coalesced rows
// and the recurrence stays in registers.

#include "pn_device.hpp"

namespace pn {

// Steps per prefetch group: the loads of group g+1 are issued before group g
// is computed, so every thread keeps 2*U loads in flight.
constexpr int kU = 8;
constexpr int kUP = 16;   // the prologue only reads x, so it prefetches twice as far

template <int MODE, int PHASE>
__global__ __launch_bounds__(kThreads) void diag_tanh_pass(DiagArgs g) {
    if constexpr (PHASE != kPrologue) {
        if (g.ctrl->stop) return;    // uniform over the grid: converged earlier
    }
    const int cpb = g.cpb;
    const int dl = threadIdx.x % cpb;
    const int cl = threadIdx.x / cpb;
    const int c = blockIdx.x * (kThreads / cpb) + cl;
    const int d = blockIdx.y * cpb + dl;
    const int b = blockIdx.z;
    uint32_t rb = 0;
    if (c < g.NC && d < g.D) {
        const int D = g.D;
        const int t0 = c * g.L;
        const int n = min(g.L, g.Tw - t0);          // steps in this chunk
        const float a = g.a[d];
        const float s0v = g.s0[b * g.s0s + d];
        const float* xp = g.x + b * g.xs + static_cast<int64_t>(t0) * D + d;
        const size_t ai = (static_cast<size_t>(b) * g.NC + c) * D + d;
        float A = 1.0f, Bc = 0.0f;
        if constexpr (PHASE == kPrologue) {
            // Iteration 0: s^(0)_t = s0 for every t, so p_t = s0 throughout.
            float xb[kUP];
#pragma unroll
            for (int u = 0; u < kUP; ++u) xb[u] = u < n ? xp[u * D] : 0.0f;
            for (int j = 0; j < n; j += kUP) {
                const float* xq = xp + static_cast<int64_t>(j) * D;   // row j of the chunk
                float xn[kUP];
#pragma unroll
                for (int u = 0; u < kUP; ++u) xn[u] = (j + kUP + u < n) ? xq[(kUP + u) * D] : 0.0f;
#pragma unroll
                for (int u = 0; u < kUP; ++u) {
                    if (j + u < n) {
                        const float v = tanh_f(a * s0v + xb[u]);
                        rb = max(rb, abs_bits(s0v - v));
                        const float at = mode_coef<MODE>(a * (1.0f - v * v));
                        const float bt = v - at * s0v;
                        A = at * A;
                        Bc = at * Bc + bt;
                    }
                }
#pragma unroll
                for (int u = 0; u < kUP; ++u) xb[u] = xn[u];
            }
        } else {
            const size_t HS = static_cast<size_t>(g.B) * g.NC * D;
            float* sp = g.s + b * g.ss + static_cast<int64_t>(t0) * D + d;
            // p_old: s^(i) at t0-1 (halo of the previous chunk);  shat: s^ at t0-1.
            float p_old = (PHASE == kFirst || c == 0) ? s0v : g.halo[(g.iter & 1) * HS + ai - D];
            float shat = g.carry[ai];
            const bool has_next = (c + 1 < g.NC);
            const float shat_end = has_next ? g.carry[ai + D] : 0.0f;
            const bool und = g.undamped != 0;
            const float lam = g.lam;
            // s^(i+1) at t0-1, exactly as the previous chunk stores it.
            float snp = und ? shat : p_old + lam * (shat - p_old);
            float xb[kU], sb[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                xb[u] = u < n ? xp[u * D] : 0.0f;
                if constexpr (PHASE == kFirst) sb[u] = s0v;
                else sb[u] = u < n ? sp[u * D] : 0.0f;
            }
            for (int j = 0; j < n; j += kU) {
                const float* xq = xp + static_cast<int64_t>(j) * D;   // row j of the chunk
                float* sq = sp + static_cast<int64_t>(j) * D;
                float xn[kU], sn_[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const bool in = j + kU + u < n;
                    xn[u] = in ? xq[(kU + u) * D] : 0.0f;
                    if constexpr (PHASE == kFirst) sn_[u] = s0v;
                    else sn_[u] = in ? sq[(kU + u) * D] : 0.0f;
                }
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    if (j + u < n) {
                        const float xt = xb[u];
                        const float so = sb[u];
                        // iteration i: map at p_t = s^(i)_{t-1}
                        const float v = tanh_f(a * p_old + xt);
                        const float at = mode_coef<MODE>(a * (1.0f - v * v));
                        shat = v + at * (shat - p_old);
                        // the chunk's last value is the one the scan hands to the next chunk
                        if (j + u == n - 1 && has_next) shat = shat_end;
                        const float sn = und ? shat : so + lam * (shat - so);
                        sq[u * D] = sn;
                        // iteration i+1: residual and affine map at p_t = s^(i+1)_{t-1}
                        const float v2 = tanh_f(a * snp + xt);
                        rb = max(rb, abs_bits(sn - v2));
                        const float a2 = mode_coef<MODE>(a * (1.0f - v2 * v2));
                        const float b2 = v2 - a2 * snp;
                        A = a2 * A;
                        Bc = a2 * Bc + b2;
                        p_old = so;
                        snp = sn;
                    }
                }
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    xb[u] = xn[u];
                    sb[u] = sn_[u];
                }
            }
            g.halo[((g.iter + 1) & 1) * HS + ai] = snp;
        }
        g.aggA[ai] = A;
        g.aggB[ai] = Bc;
    }
    rb = block_max_u32(rb);
    if (threadIdx.x == 0) {
        const int bid = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        g.rpart[bid] = rb;
    }
}

static dim3 diag_grid(const DiagArgs& a) {
    const int cpg = kThreads / a.cpb;
    return dim3((a.NC + cpg - 1) / cpg, (a.D + a.cpb - 1) / a.cpb, a.B);
}

int diag_tanh_nblocks(const DiagArgs& a) {
    const dim3 g = diag_grid(a);
    return static_cast<int>(g.x * g.y * g.z);
}

template <int MODE>
static hipError_t launch_mode(int phase, const DiagArgs& a, hipStream_t st) {
    const dim3 grid = diag_grid(a);
    if (phase == kPrologue) diag_tanh_pass<MODE, kPrologue><<<grid, kThreads, 0, st>>>(a);
    else if (phase == kFirst) diag_tanh_pass<MODE, kFirst><<<grid, kThreads, 0, st>>>(a);
    else diag_tanh_pass<MODE, kSteady><<<grid, kThreads, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_diag_tanh_pass(int phase, const DiagArgs& a, hipStream_t st) {
    switch (a.mode) {
        case kJacobi: return launch_mode<kJacobi>(phase, a, st);
        case kPicard: return launch_mode<kPicard>(phase, a, st);
        default: return launch_mode<kQuasiNewton>(phase, a, st);   // Newton == QN here
    }
}

// ---------------------------------------------------------------- carry scan
// carry[b][0] = s0[b]; carry[b][c+1] = aggA[b][c] * carry[b][c] + aggB[b][c].
// Thread = (b, d, segment); each of kSeg threads of a channel composes a
// contiguous run of chunks, the runs are combined in LDS, and every thread
// replays its run from the combined carry.  Runs of up to kPer chunks are held
// in registers, so each thread issues all of its loads at once.
constexpr int kSeg = 16;          // segments per channel
constexpr int kChan = 64;         // channels per workgroup (one wave wide)
constexpr int kPer = 16;          // chunks per segment held in registers

__global__ __launch_bounds__(kSeg * kChan) void diag_carry_kernel(CarryArgs g) {
    if (g.do_check && blockIdx.x == 0 && blockIdx.y == 0) run_check(g.chk);
    __shared__ float segA[kSeg][kChan];
    __shared__ float segB[kSeg][kChan];
    const int dl = threadIdx.x % kChan;
    const int sg = threadIdx.x / kChan;
    const int d = blockIdx.x * kChan + dl;
    const int b = blockIdx.y;
    const int NC = g.NC;
    const int D = g.D;
    const int per = (NC + kSeg - 1) / kSeg;
    const int c0 = min(NC, sg * per);
    const int c1 = min(NC, c0 + per);
    const bool act = d < D;
    const size_t base = static_cast<size_t>(b) * NC * D + d;
    float A = 1.0f, Bc = 0.0f;
    float ra[kPer], rbv[kPer];
    if (act) {
        if (c1 - c0 <= kPer) {
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const bool in = c0 + k < c1;
                ra[k] = in ? g.aggA[base + static_cast<size_t>(c0 + k) * D] : 1.0f;
                rbv[k] = in ? g.aggB[base + static_cast<size_t>(c0 + k) * D] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                Bc = ra[k] * Bc + rbv[k];
                A = ra[k] * A;
            }
        } else {
            for (int c = c0; c < c1; ++c) {
                const float ac = g.aggA[base + static_cast<size_t>(c) * D];
                const float bc = g.aggB[base + static_cast<size_t>(c) * D];
                Bc = ac * Bc + bc;
                A = ac * A;
            }
        }
    }
    segA[sg][dl] = A;
    segB[sg][dl] = Bc;
    __syncthreads();
    if (act) {
        float y = g.s0[b * g.s0s + d];
        for (int k = 0; k < sg; ++k) y = segA[k][dl] * y + segB[k][dl];
        if (c1 - c0 <= kPer) {
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                if (c0 + k < c1) {
                    g.carry[base + static_cast<size_t>(c0 + k) * D] = y;
                    y = ra[k] * y + rbv[k];
                }
            }
        } else {
            for (int c = c0; c < c1; ++c) {
                g.carry[base + static_cast<size_t>(c) * D] = y;
                y = g.aggA[base + static_cast<size_t>(c) * D] * y + g.aggB[base + static_cast<size_t>(c) * D];
            }
        }
    }
}

hipError_t launch_diag_carry(const CarryArgs& a, hipStream_t st) {
    const dim3 grid((a.D + kChan - 1) / kChan, a.B);
    diag_carry_kernel<<<grid, kSeg * kChan, 0, st>>>(a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- fill
// out[b][t][:] = s0[b][:] for a window (result when no update was applied).
__global__ __launch_bounds__(kThreads) void fill_kernel(float* out, int64_t ss, const float* s0,
                                                         int64_t s0s, int Tw, int D) {
    const int b = blockIdx.y;
    const int64_t n = static_cast<int64_t>(Tw) * D;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        out[b * ss + e] = s0[b * s0s + (e % D)];
    }
}

hipError_t launch_fill(float* out, int64_t ss, const float* s0, int64_t s0s, int B, int Tw, int D,
                       hipStream_t st) {
    if (B == 0 || Tw == 0 || D == 0) return hipSuccess;
    const int64_t n = static_cast<int64_t>(Tw) * D;
    const int gx = static_cast<int>(std::min<int64_t>((n + kThreads - 1) / kThreads, 4096));
    fill_kernel<<<dim3(gx, B), kThreads, 0, st>>>(out, ss, s0, s0s, Tw, D);
    return hipGetLastError();
}

}  // namespace pn
