// Newton (dense Jacobian) iteration for the matrix cells with D padded to 16
// or 32, on the FP32 matrix cores.
//
// One wavefront owns one chunk of L steps and walks it in sub-chunks of 16
// steps staged through LDS.  Per sub-chunk it
//   1. computes the input projection U x_t + b once, on the matrix cores;
//   2. evaluates the cell at the old iterate (v_t and the Jacobian row
//      scalings) and replays s^_t = v_t + A_t (s^_{t-1} - p_t) from the carry,
//      damps, and stores s^(i+1) [the update of PN §1.2];
//   3. evaluates the cell at the new iterate (residual and the maps of
//      iteration i+1) and extends the chunk map
//          M <- A_t M,   bg <- A_t (bg - p_t) + v_t
//      [the affine-map composition of PN §2.1] with A_t = diag(z) +
//      sum_g diag(c_g) W_g (tanh RNN: A_t = diag(1 - v^2) W; Euler step:
//      A_t = diag(1 - h) + diag(h (1 - g^2)) W).
// The banded mode [PN §2.2.2] replaces A_t by its band |i - k| <= band, which
// is the same sum over the band-restricted W_g (row scaling keeps the band):
// the lane's weights for the Jacobian products are masked once at start, the
// cell itself keeps the full weights.  The chunk map of banded factors fills
// in, so it stays a dense DP x DP product.
// W_g M is a DP x DP x DP product done as MFMA k-steps: the accumulator of
// one step holds M in the instruction's output layout, whose rows per lane
// group are exactly the k indices that lane group supplies as the B operand
// of the next step, so the chain never leaves registers.  The A operand
// (W_g restricted to that k subset) is loaded once into registers and also
// serves the matrix-vector products of the replay and the offset chain.
// The cell evaluations of a sub-chunk are one tile product each: with the
// step index as the A-operand row, G^T = Q W_g^T takes the same register
// slice of W_g as its B operand (see eval_tile).
//
// Lane roles (64 lanes): i = lane % DP is a state row, h = lane / DP picks the
// k subset K_h = {krow(h, s), s < KS}.  Row-vector dot products are partial
// sums over K_h combined across the NH = 64 / DP lane groups.

#include "pn_device.hpp"
#include "pn_launch.hpp"

namespace pn {

// Maps pass of the advancing window: stage Sc rows of the iterate (window
// rows tq0 ..) into dst (row stride DP).  Rows from ff on are new steps that
// start from fillrow (the state before them, which this pass does not write)
// and are stored to s (sgj: the same rows in s).
template <int NT>
__device__ __forceinline__ void stage_maps_rows(float* dst, int DP, float* sgj, int D, int Sc, int tq0, int ff,
                                                const float* fillrow, int tid) {
    const int nld = max(0, min(Sc, ff - tq0));
    copy_rows_to_lds<NT>(dst, DP, sgj, D, nld, D, tid);
    for (int e = tid; e < (Sc - nld) * DP; e += NT) {
        const int j = nld + e / DP, q = e % DP;
        const float v = q < D ? fillrow[q] : 0.0f;
        dst[j * DP + q] = v;
        if (q < D) sgj[j * D + q] = v;
    }
}

constexpr int kCellTanhRnnD = 1;
constexpr int kCellGruD = 2;
constexpr int kCellEulerD = 3;
constexpr int kSub = 16;          // steps per LDS sub-chunk

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

template <int DP> struct MfmaTile;
template <> struct MfmaTile<32> {
    static constexpr int NH = 2, KS = 16;
    static constexpr int NSL = 8;     // accumulator slots r with krow(h, r) < kSub
    typedef v16f acc_t;
    // k index (= output row) of slot s for lane group h
    __device__ static int krow(int h, int s) { return 8 * (s >> 2) + 4 * h + (s & 3); }
    __device__ static acc_t step(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};
template <> struct MfmaTile<16> {
    static constexpr int NH = 4, KS = 4;
    static constexpr int NSL = 4;
    typedef v4f acc_t;
    __device__ static int krow(int h, int s) { return 4 * h + s; }
    __device__ static acc_t step(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// The lane's k subset of a DP-vector in LDS, as KS/4 aligned 16-byte reads:
// for DP = 32 the subset is {8g + 4h + t}, for DP = 16 it is {4h + t}.
template <int DP>
__device__ __forceinline__ float4 kgroup(const float* v, int h, int g) {
    if constexpr (DP == 32) return *reinterpret_cast<const float4*>(v + 8 * g + 4 * h);
    else return *reinterpret_cast<const float4*>(v + 4 * h);
}

// sum of v over the NH lane groups that share a row (lanes i, i+DP, ...)
template <int DP>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (DP == 32) {
        v += __shfl_xor(v, 32, 64);
    } else {
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
    }
    return v;
}

template <int CELL> struct DTraits;
template <> struct DTraits<kCellTanhRnnD> { static constexpr int NG = 1, NCO = 1; };
template <> struct DTraits<kCellGruD> { static constexpr int NG = 3, NCO = 4; };
template <> struct DTraits<kCellEulerD> { static constexpr int NG = 1, NCO = 2; };

// Rows exchanged between the lanes of one wavefront: its LDS accesses execute
// in program order, so a compiler barrier orders them (the data role of the
// split kernel cannot take the workgroup barrier, which the chain wavefront
// meets once per sub-chunk).
__device__ __forceinline__ void wave_sync() { __builtin_amdgcn_wave_barrier(); }

// LDS layout (floats) for one chunk; split: the replay's coefficients and
// two sets of the next iteration's (one set serves all three otherwise).
template <int CELL, int DP>
struct DLds {
    static constexpr int NG = DTraits<CELL>::NG, NCO = DTraits<CELL>::NCO;
    static __host__ __device__ size_t floats(int m, bool split) {
        return 2ull * (kSub + 1) * DP        // P, N rows
             + static_cast<size_t>(kSub) * m  // x rows
             + static_cast<size_t>(kSub) * DP        // v
             + (split ? 3ull : 1ull) * NCO * kSub * DP  // Jacobian coefficients
             + static_cast<size_t>(NG) * m * DP      // U^T (all gates)
             + 2 * DP;                               // vector exchange
    }
};

// (A_t d)[i] for the difference vector d in LDS (only the lane's k subset is
// read; d_i is passed for the diagonal GRU term).
template <int CELL, int DP>
__device__ __forceinline__ float jac_apply_row(const float (&wr)[DTraits<CELL>::NG][MfmaTile<DP>::KS],
                                               const float* d, int h,
                                               const float (&co)[DTraits<CELL>::NCO], float di) {
    using Tl = MfmaTile<DP>;
    constexpr int NG = DTraits<CELL>::NG;
    float acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = 0.0f;
#pragma unroll
    for (int q = 0; q < Tl::KS / 4; ++q) {
        const float4 d4 = kgroup<DP>(d, h, q);
        const float dk[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g] += wr[g][4 * q + t] * dk[t];
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = group_sum<DP>(acc[g]);
    if constexpr (CELL == kCellTanhRnnD) {
        return co[0] * acc[0];
    } else if constexpr (CELL == kCellEulerD) {
        return co[0] * di + co[1] * acc[0];
    } else {
        // gates are stored (r, z, n); coefficients (z, cz, cn, cr)
        return co[0] * di + co[1] * acc[1] + co[2] * acc[2] + co[3] * acc[0];
    }
}

// Input projection of the sub-chunk's steps as a tile product: XA[g] holds,
// in slot r of lane (i, h), (U_g x_j)[i] + bias_g[i] for step j = krow(h, r).
// The A operand is x row j = lane % DP (zero past the sub-chunk), the B
// operand U_g[i][q] read from the transposed copy in LDS; the k index q runs
// over m in groups of 4 NH, zero-padded.
template <int CELL, int DP>
__device__ __forceinline__ void proj_tile(const float* X, const float* UT, int m, int Sc, int h, int i,
                                          const float (&bias)[3],
                                          typename MfmaTile<DP>::acc_t (&XA)[DTraits<CELL>::NG]) {
    using Tl = MfmaTile<DP>;
    constexpr int NG = DTraits<CELL>::NG;
    const int jl = i;                        // A-operand row: step index
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int r = 0; r < Tl::KS; ++r) XA[g][r] = bias[g];
    const int SKM = ((m + 4 * Tl::NH - 1) / (4 * Tl::NH)) * 4;
    for (int s = 0; s < SKM; ++s) {
        const int q = 4 * Tl::NH * (s >> 2) + 4 * h + (s & 3);
        const bool qin = q < m;
        const float a = (jl < Sc && qin) ? X[jl * m + q] : 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float bu = qin ? UT[(g * m + q) * DP + i] : 0.0f;
            XA[g] = Tl::step(a, bu, XA[g]);
        }
    }
}

// Pre-activations of the sub-chunk at the rows Q (Q[j] = state before step j):
// G[g] = XA[g] + (Q W_g^T) in the slot layout of proj_tile (the GRU's
// candidate gate keeps its hidden part W_n q separate: G[2] starts at 0).
template <int CELL, int DP>
__device__ __forceinline__ void eval_tile(const float* Q, int Sc, int h, int i,
                                          const float (&wr)[DTraits<CELL>::NG][MfmaTile<DP>::KS],
                                          const typename MfmaTile<DP>::acc_t (&XA)[DTraits<CELL>::NG],
                                          typename MfmaTile<DP>::acc_t (&G)[DTraits<CELL>::NG]) {
    using Tl = MfmaTile<DP>;
    constexpr int NG = DTraits<CELL>::NG;
    const int jl = i;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        if (CELL == kCellGruD && g == 2) {
#pragma unroll
            for (int r = 0; r < Tl::KS; ++r) G[g][r] = 0.0f;
        } else {
            G[g] = XA[g];
        }
    }
#pragma unroll
    for (int q = 0; q < Tl::KS / 4; ++q) {
        const float4 a4 = jl < Sc ? kgroup<DP>(Q + jl * DP, h, q) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float ak[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g) G[g] = Tl::step(ak[t], wr[g][4 * q + t], G[g]);
    }
}

// v and the Jacobian coefficients of one state at one step, from its
// pre-activations gv (with the input projection, except the GRU candidate's
// hidden part), the candidate's input part xn (GRU), the state p_i before
// the step and the per-row constants aux (GRU hidden biases, Euler step size).
template <int CELL>
__device__ __forceinline__ float cell_point(const float (&gv)[3], float xn, float pi, const float (&aux)[3],
                                            float (&co)[DTraits<CELL>::NCO]) {
    if constexpr (CELL == kCellTanhRnnD) {
        const float v = tanh_f(gv[0]);
        co[0] = 1.0f - v * v;
        return v;
    } else if constexpr (CELL == kCellEulerD) {
        const float g = tanh_f(gv[0]);
        const float hs = aux[0];
        co[0] = 1.0f - hs;
        co[1] = hs * (1.0f - g * g);
        return pi + hs * (g - pi);
    } else {
        const float r = sigmoid_f(gv[0] + aux[0]);
        const float z = sigmoid_f(gv[1] + aux[1]);
        const float gg = gv[2] + aux[2];
        const float n = tanh_f(xn + r * gg);
        const float dn = (1.0f - z) * (1.0f - n * n);
        co[0] = z;
        co[1] = (pi - n) * z * (1.0f - z);
        co[2] = dn * r;
        co[3] = dn * gg * r * (1.0f - r);
        return (1.0f - z) * n + z * pi;
    }
}

// SPLIT: two wavefronts per chunk.  Wavefront 0 runs only the chunk-map
// chain (the matrix-core steps and row scalings); wavefront 1 runs
// everything else (staging, the cell tiles, replay, residual and the offset
// chain) one sub-chunk ahead, publishing the coefficients of sub-chunk k in
// one of two LDS buffers before the workgroup barrier k.  The dependent
// latency chains of the two roles then overlap within one chunk, which pays
// when there are too few chunks to fill the SIMDs with other chunks; with
// many chunks one wavefront per chunk runs both roles (more chunks resident).
// At D padded to 16 the one-wavefront form is held to 128 registers (no
// spills), so four wavefronts share each SIMD and hide one another's
// latencies: the planner then gives 4096 chunks where it can.
template <int CELL, int DP, int PHASE, bool BANDED, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 128 : 64)
__attribute__((amdgpu_waves_per_eu((DP == 16 && !SPLIT) ? 4 : 1))) void dense_pass(CellArgs g) {
    if constexpr (PHASE != kPrologue && PHASE != kMaps) {   // apply launches enqueued ahead
        if (g.ctrl->stop) return;
        if (g.fc & kFcCheck) {
            // The check of iteration i, taken alike by every workgroup from
            // the residual slots the sweep before filled; a stop writes
            // nothing.  Workgroup (0, 0) clears the slot set of the sweep
            // after next and publishes the check to the control word and
            // the host.
            const int ln = threadIdx.x & 63;
            const uint32_t rv = ln < kRSlots ? g.ctrl->rmax[g.iter % 3][ln][0] : 0u;
            const uint32_t r_i = wave_max_u32(rv);
            CheckArgs chk{};
            chk.iter = g.iter;
            chk.max_iter = g.max_iter;
            chk.tol = g.tol;
            chk.ctrl = g.ctrl;
            chk.host = g.host + g.iter % kHostRing;
            chk.epoch = g.epoch;
            const int st = check_status(r_i, chk);
            if (blockIdx.x == 0 && blockIdx.y == 0) {
                if (threadIdx.x < kRSlots)
                    __hip_atomic_store(&g.ctrl->rmax[(g.iter + 2) % 3][threadIdx.x][0], 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                if (threadIdx.x == 0) publish_check(chk, r_i, st, 0xffffffffu);
            }
            if (st >= 0) return;
        }
    }
    using Tl = MfmaTile<DP>;
    using acc_t = typename Tl::acc_t;
    constexpr int NG = DTraits<CELL>::NG;
    constexpr int NCO = DTraits<CELL>::NCO;
    constexpr int KS = Tl::KS;
    constexpr int COS = NCO * kSub * DP;      // floats of one coefficient set
    extern __shared__ float lds[];
    const int D = g.D, m = g.m;
    const int lane = threadIdx.x & 63;
    const int i = lane % DP, h = lane / DP;
    const bool live = i < D;
    const int c = blockIdx.x, b = blockIdx.y;
    const int t0 = c * g.L;
    const int Lc = min(g.L, g.Tw - t0);
    const int nsub = (Lc + kSub - 1) / kSub;
    const size_t ci = static_cast<size_t>(b) * g.NC + c;
    const size_t HS = static_cast<size_t>(g.B) * g.NC * D;
    const float* s0 = g.s0 + b * g.s0s;

    float* P = lds;                          // [kSub+1][DP]
    float* N = P + (kSub + 1) * DP;          // [kSub+1][DP]
    float* X = N + (kSub + 1) * DP;          // [kSub][m]
    float* V = X + kSub * m;                 // [kSub][DP]
    float* COr = V + kSub * DP;              // [NCO][kSub][DP] iteration i (replay)
    // iteration i+1, per sub-chunk parity (one wavefront: the same buffer,
    // consumed before the next sub-chunk overwrites it)
    float* CO2 = SPLIT ? COr + COS : COr;
    float* UT = COr + (SPLIT ? 3 : 1) * COS; // [NG][m][DP]
    float* YV = UT + NG * m * DP;            // [2][DP]
    auto co_set = [&](int k) { return CO2 + (SPLIT ? (k & 1) * COS : 0); };

    const float* w = g.w;
    // prepared layout: tanh RNN WT | UT | bias | wdiag (Euler: | h);
    // GRU WhT | WiT | bih | bhh | whdiag
    const float* wUT = w + NG * DP * DP;
    const float* wbi = wUT + NG * m * DP;
    const float* wbh = wbi + NG * DP;         // GRU only
    // weights of the Jacobian products: W_g itself, or its band
    float wj[NG][KS];
#pragma unroll
    for (int gt = 0; gt < NG; ++gt)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int k = Tl::krow(h, s);
            const float wv = w[(gt * DP + k) * DP + i];
            wj[gt][s] = (!BANDED || abs(k - i) <= g.band) ? wv : 0.0f;
        }

    // chunk map: M in accumulator layout (column lane%DP, rows krow(h, r))
    acc_t M;
#pragma unroll
    for (int r = 0; r < KS; ++r) M[r] = (Tl::krow(h, r) == i && live) ? 1.0f : 0.0f;
    // one chain step: C_g = W_g M, then M <- A_j M from the row scalings
    auto products = [&](acc_t (&C)[NG]) {
#pragma unroll
        for (int gt = 0; gt < NG; ++gt) {
#pragma unroll
            for (int r = 0; r < KS; ++r) C[gt][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < KS; ++s) C[gt] = Tl::step(wj[gt][s], M[s], C[gt]);
        }
    };
    auto scale = [&](const acc_t (&C)[NG], const float* COk, int j) {
        float rs[NCO][KS];
#pragma unroll
        for (int q = 0; q < NCO; ++q)
#pragma unroll
            for (int u = 0; u < KS / 4; ++u) {
                const float4 c4 = kgroup<DP>(COk + (q * kSub + j) * DP, h, u);
                rs[q][4 * u] = c4.x;
                rs[q][4 * u + 1] = c4.y;
                rs[q][4 * u + 2] = c4.z;
                rs[q][4 * u + 3] = c4.w;
            }
#pragma unroll
        for (int r = 0; r < KS; ++r) {
            if constexpr (CELL == kCellTanhRnnD) {
                M[r] = rs[0][r] * C[0][r];
            } else if constexpr (CELL == kCellEulerD) {
                M[r] = rs[0][r] * M[r] + rs[1][r] * C[0][r];
            } else {
                M[r] = rs[0][r] * M[r] + rs[1][r] * C[1][r] + rs[2][r] * C[2][r] + rs[3][r] * C[0][r];
            }
        }
    };
    auto write_map = [&]() {
        // chunk map out: M[row][col] row-major, col = i
        float* aA = g.aggA + ci * D * D;
#pragma unroll
        for (int r = 0; r < KS; ++r) {
            const int row = Tl::krow(h, r);
            if (row < D && live) aA[row * D + i] = M[r];
        }
    };

    if constexpr (SPLIT) {
        if (threadIdx.x < 64) {
            // ---- chain wavefront: sub-chunk k once its coefficients are out (barrier k)
            for (int k = 0; k < nsub; ++k) {
                __syncthreads();
                const int Sc = min(kSub, Lc - k * kSub);
                const float* COk = co_set(k);
                for (int j = 0; j < Sc; ++j) {
                    acc_t C[NG];
                    products(C);
                    scale(C, COk, j);
                }
            }
            write_map();
            return;
        }
    }

    // ---- data role: staging, cell tiles, replay, residual, offset chain
    float wr[NG][KS];
#pragma unroll
    for (int gt = 0; gt < NG; ++gt)
#pragma unroll
        for (int s = 0; s < KS; ++s) wr[gt][s] = w[(gt * DP + Tl::krow(h, s)) * DP + i];
    copy_to_lds<64>(UT, wUT, NG * m * DP, lane);
    const float bias_i[3] = {wbi[i], NG > 1 ? wbi[DP + i] : 0.0f, NG > 2 ? wbi[2 * DP + i] : 0.0f};
    float bhh_l[3] = {0.0f, 0.0f, 0.0f};
    if constexpr (CELL == kCellGruD) {
        bhh_l[0] = wbh[i];
        bhh_l[1] = wbh[DP + i];
        bhh_l[2] = wbh[2 * DP + i];
    } else if constexpr (CELL == kCellEulerD) {
        bhh_l[0] = wbi[2 * DP + i];          // step size h_i
    }

    float bg = 0.0f;                         // chunk offset, row i
    uint32_t rb = 0;
    const bool track = g.fpart != nullptr;   // first step over tol (advancing window)
    uint32_t fb = 0xffffffffu;
    const bool has_next = c + 1 < g.NC;
    const float* cr = g.carry + ci * D;
    float shat = 0.0f;                       // s^ at the row before the current one (lane row i)
    float* sg = g.s + b * g.ss + static_cast<int64_t>(t0) * D;
    // maps pass of the advancing window: new steps from window row ff on
    const int ff = g.Tw - g.fill_rows;
    const float* fillrow = ff == 0 ? s0 : g.s + b * g.ss + static_cast<int64_t>(ff - 1) * D;
    const float* xg = g.x + b * g.xs + static_cast<int64_t>(t0) * m;

    // row t0-1 of the old and the new iterate
    {
        float po = 0.0f, pn = 0.0f;
        if (live) {
            if constexpr (PHASE == kPrologue) {
                po = pn = s0[i];
            } else if constexpr (PHASE == kMaps) {
                // rows from ff on are new steps (fill_rows): they start from fillrow
                po = pn = c == 0 ? s0[i] : (t0 - 1 >= ff ? fillrow[i] : sg[i - D]);
            } else {
                po = (PHASE == kFirst || c == 0) ? s0[i] : g.halo[(g.iter & 1) * HS + (ci - 1) * D + i];
                shat = cr[i];
                pn = g.undamped ? shat : po + g.lam * (shat - po);
            }
        }
        if (h == 0) {
            P[i] = po;
            N[i] = pn;
        }
    }

    // Staging registers: the x rows of a sub-chunk (m <= 16) and, in the
    // steady sweeps, its rows of the old iterate, loaded while the chain of
    // the sub-chunk before it runs, so that their memory latency is hidden.
    constexpr int kXP = kSub * 16 / 64, kPP = kSub * DP / 64;
    const bool xpre = m <= 16;
    float xpf[kXP], ppf[kPP];
    auto prefetch = [&](int k) {
        const int j0 = k * kSub;
        const int Sc = min(kSub, Lc - j0);
        if (xpre) {
#pragma unroll
            for (int u = 0; u < kXP; ++u) {
                const int e = u * 64 + lane;
                xpf[u] = e < Sc * m ? xg[static_cast<int64_t>(j0) * m + e] : 0.0f;
            }
        }
        if constexpr (PHASE == kSteady) {
#pragma unroll
            for (int u = 0; u < kPP; ++u) {
                const int e = u * 64 + lane;
                const int r = e / DP, q = e % DP;
                ppf[u] = (r < Sc && q < D) ? sg[static_cast<int64_t>(j0 + r) * D + q] : 0.0f;
            }
        }
    };

    // Sub-chunk k: stage its rows, evaluate the cell at the old iterate and
    // replay (apply launches), store, then evaluate at the new iterate:
    // residual, V and the coefficients of iteration i+1 (co_set(k)).
    auto process = [&](int k) {
        const int j0 = k * kSub;
        const int Sc = min(kSub, Lc - j0);
        if (xpre) {
#pragma unroll
            for (int u = 0; u < kXP; ++u) {
                const int e = u * 64 + lane;
                if (e < Sc * m) X[e] = xpf[u];
            }
        } else {
            copy_to_lds<64>(X, xg + static_cast<int64_t>(j0) * m, Sc * m, lane);
        }
        if constexpr (PHASE == kPrologue || PHASE == kFirst) {
            for (int e = lane; e < Sc * DP; e += 64) {
                const int q = e % DP;
                P[DP + e] = q < D ? s0[q] : 0.0f;
            }
        } else if constexpr (PHASE == kMaps) {
            stage_maps_rows<64>(P + DP, DP, sg + static_cast<int64_t>(j0) * D, D, Sc, t0 + j0, ff, fillrow, lane);
        } else {
#pragma unroll
            for (int u = 0; u < kPP; ++u) {
                const int e = u * 64 + lane;
                if (e / DP < Sc) P[DP + e] = ppf[u];
            }
        }
        wave_sync();
        // input projection U x + b_ih for every row and gate (registers)
        acc_t XA[NG];
        proj_tile<CELL, DP>(X, UT, m, Sc, h, i, bias_i, XA);
        acc_t G[NG];
        if constexpr (PHASE != kPrologue && PHASE != kMaps) {
            eval_tile<CELL, DP>(P, Sc, h, i, wr, XA, G);
#pragma unroll
            for (int r = 0; r < Tl::NSL; ++r) {
                const int j = Tl::krow(h, r);
                if (j < Sc) {
                    const float gv[3] = {G[0][r], NG > 1 ? G[NG > 1 ? 1 : 0][r] : 0.0f,
                                         NG > 2 ? G[NG > 2 ? 2 : 0][r] : 0.0f};
                    float co[NCO];
                    const float v = cell_point<CELL>(gv, XA[NG - 1][r], P[j * DP + i], bhh_l, co);
                    V[j * DP + i] = live ? v : 0.0f;
#pragma unroll
                    for (int q = 0; q < NCO; ++q) COr[(q * kSub + j) * DP + i] = live ? co[q] : 0.0f;
                }
            }
            wave_sync();
            for (int j = 0; j < Sc; ++j) {
                const float di = live ? shat - P[j * DP + i] : 0.0f;
                if (h == 0) YV[i] = di;
                wave_sync();
                float co[NCO];
#pragma unroll
                for (int q = 0; q < NCO; ++q) co[q] = COr[(q * kSub + j) * DP + i];
                const float ad = jac_apply_row<CELL, DP>(wj, YV, h, co, di);
                shat = V[j * DP + i] + ad;
                if (j0 + j == Lc - 1 && has_next && live) shat = cr[D + i];
                const float so = P[(j + 1) * DP + i];
                const float sn = g.undamped ? shat : so + g.lam * (shat - so);
                if (h == 0) N[(j + 1) * DP + i] = live ? sn : 0.0f;
                wave_sync();
            }
            for (int e = lane; e < Sc * D; e += 64) {
                const int j = e / D, q = e % D;
                sg[static_cast<int64_t>(j0 + j) * D + q] = N[(j + 1) * DP + q];
            }
        } else {
            for (int e = lane; e < Sc * DP; e += 64) N[DP + e] = P[DP + e];
        }
        wave_sync();
        float* COk = co_set(k);
        eval_tile<CELL, DP>(N, Sc, h, i, wr, XA, G);
#pragma unroll
        for (int r = 0; r < Tl::NSL; ++r) {
            const int j = Tl::krow(h, r);
            if (j < Sc) {
                const float gv[3] = {G[0][r], NG > 1 ? G[NG > 1 ? 1 : 0][r] : 0.0f,
                                     NG > 2 ? G[NG > 2 ? 2 : 0][r] : 0.0f};
                float co[NCO];
                const float v = cell_point<CELL>(gv, XA[NG - 1][r], N[j * DP + i], bhh_l, co);
                if (live) {
                    const float d = N[(j + 1) * DP + i] - v;
                    rb = max(rb, abs_bits(d));
                    if (track && !(fabsf(d) <= g.tol)) fb = min(fb, static_cast<uint32_t>(j0 + j));
                }
                V[j * DP + i] = live ? v : 0.0f;
#pragma unroll
                for (int q = 0; q < NCO; ++q) COk[(q * kSub + j) * DP + i] = live ? co[q] : 0.0f;
            }
        }
        wave_sync();
    };

    prefetch(0);
    process(0);
    for (int k = 0; k < nsub; ++k) {
        if constexpr (SPLIT) __syncthreads();   // coefficients of sub-chunk k are out
        const int Sc = min(kSub, Lc - k * kSub);
        const float* COk = co_set(k);
        if (k + 1 < nsub) prefetch(k + 1);
        for (int j = 0; j < Sc; ++j) {
            acc_t C[NG];
            if constexpr (!SPLIT) products(C);
            // offset of the chunk map: bg <- A_j (bg - p_j) + v_j  (p_j = N[j])
            const float dbi = live ? bg - N[j * DP + i] : 0.0f;
            if (h == 0) YV[DP + i] = dbi;
            wave_sync();
            float co[NCO];
#pragma unroll
            for (int q = 0; q < NCO; ++q) co[q] = COk[(q * kSub + j) * DP + i];
            bg = V[j * DP + i] + jac_apply_row<CELL, DP>(wj, YV + DP, h, co, dbi);
            if constexpr (!SPLIT) scale(C, COk, j);
            wave_sync();
        }
        // carry the last rows into the next sub-chunk
        const float plast = P[Sc * DP + i];
        const float nlast = N[Sc * DP + i];
        wave_sync();
        if (h == 0) {
            P[i] = plast;
            N[i] = nlast;
        }
        wave_sync();
        if (k + 1 < nsub) process(k + 1);
    }

    if constexpr (!SPLIT) write_map();
    if constexpr (PHASE == kMaps) {
        // the current iterate's last row, for the apply launch that follows
        if (h == 0 && live) g.halo[(g.iter & 1) * HS + ci * D + i] = N[i];
    } else if constexpr (PHASE != kPrologue) {
        if (h == 0 && live) g.halo[((g.iter + 1) & 1) * HS + ci * D + i] = N[i];
    }
    if (h == 0 && live) g.aggB[ci * D + i] = bg;
    rb = wave_max_u32(rb);
    if (lane == 0) {
        if (g.fc & kFcCheck) {
            // r_{i+1} (r_0 in the prologue) for the check the next sweep takes
            const int set = PHASE == kPrologue ? 0 : (g.iter + 1) % 3;
            __hip_atomic_fetch_max(&g.ctrl->rmax[set][ci % kRSlots][0], rb, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
            g.rpart[ci] = rb;
        }
    }
    if (track) {
        fb = ~wave_max_u32(~fb);
        if (lane == 0) g.fpart[ci] = fb == 0xffffffffu ? fb : t0 + fb;
    }
}

// ---------------------------------------------------------------- D padded to 64
// The same iteration for 33 <= D <= 64 and the single-gate cells (tanh RNN,
// Euler step).  One wavefront per chunk; the D x D map is four 32 x 32
// accumulator tiles M[K][J] (rows 32K + krow(h, q), columns 32J + r for lane
// l = 32h + r), and W g M is 2 x 2 output tiles of 2 x 16 steps of the
// 32x32x2 FP32 MFMA, 128 steps per time step.  The lane's A operands,
// wr[I][K][s] = W[32I + r][32K + krow(h, s)], also give its two rows r and
// 32 + r of every matrix-vector product (partial sums over its k subset plus
// the partner lane l ^ 32).  The same registers are the B operand of the
// sub-chunk's cell evaluation, two 32 x 32 tiles G_I = Q W_I^T + X U_I^T
// with the step index as the A-operand row (tile I, slot q: step krow(h, q)
// of state 32I + r).  Each lane writes its own row l of the LDS rows in the
// replay and its tile entries in the evaluation.
template <int CELL> struct D64Lds {
    static constexpr int NCO = DTraits<CELL>::NCO;
    static __host__ __device__ size_t floats(int m) {
        return 2ull * (kSub + 1) * 64 + static_cast<size_t>(kSub) * m + 1ull * kSub * 64 +
               static_cast<size_t>(NCO) * kSub * 64 + static_cast<size_t>(m) * 64 + 2 * 64;
    }
};

//
// The banded mode with half-bandwidth k <= RB (RB > 0) extends the chunk map
// on the vector ALUs instead and uses the band [PN §2.2.2]: lane i holds row i
// of M (64 registers, one per column), and row i of band_k(W) M is
// sum_{|d| <= k} W[i][i+d] M[i+d][:], whose rows i +- d come from the lanes
// d below and above through whole-wavefront DPP shifts by one lane (zero
// beyond the ends).  Per time step that is (2k+1) multiply-adds and 2k lane
// shifts per column, against 128 matrix-core steps of the dense product.

// v of lane i - 1 into lane i (0 into lane 0); v of lane i + 1 into lane i
// (0 into lane 63): wavefront shifts by one lane.  Every lane must be active.
__device__ __forceinline__ float lane_from_below(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x138, 0xf, 0xf, true));
}
__device__ __forceinline__ float lane_from_above(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x130, 0xf, 0xf, true));
}

template <int CELL, int PHASE, bool BANDED, int RB = 0>
__global__ __launch_bounds__(64) void dense64_pass(CellArgs g) {
    static_assert(RB == 0 || BANDED, "the row chain is the banded mode's");
    static_assert(DTraits<CELL>::NG == 1, "single-gate cells only");
    if constexpr (PHASE != kPrologue && PHASE != kMaps) {
        if (g.ctrl->stop) return;
    }
    typedef MfmaTile<32> Tl;
    constexpr int NCO = DTraits<CELL>::NCO;
    constexpr int DP = 64;
    extern __shared__ float lds[];
    const int D = g.D, m = g.m;
    const int lane = threadIdx.x;
    const int r = lane & 31, h = lane >> 5;
    const int orow = lane;                    // the row this lane writes
    const bool olive = orow < D;
    const bool live0 = r < D, live1 = 32 + r < D;
    const int c = blockIdx.x, b = blockIdx.y;
    const int t0 = c * g.L;
    const int Lc = min(g.L, g.Tw - t0);
    const size_t ci = static_cast<size_t>(b) * g.NC + c;
    const size_t HS = static_cast<size_t>(g.B) * g.NC * D;
    const float* s0 = g.s0 + b * g.s0s;

    float* P = lds;                           // [kSub+1][64]
    float* N = P + (kSub + 1) * DP;           // [kSub+1][64]
    float* X = N + (kSub + 1) * DP;           // [kSub][m]
    float* V = X + kSub * m;                  // [kSub][64]
    float* CO = V + kSub * DP;                // [NCO][kSub][64]
    float* UT = CO + NCO * kSub * DP;         // [m][64]
    float* YV = UT + m * DP;                  // [2][64]
    (void)(V + kSub * DP);

    const float* w = g.w;                     // WT[64][64] | UT[m][64] | bias | wdiag (| h)
    const float* wUT = w + DP * DP;
    const float* wbi = wUT + m * DP;
    float wr[2][2][16], wj[2][2][16];
#pragma unroll
    for (int I = 0; I < 2; ++I)
#pragma unroll
        for (int K = 0; K < 2; ++K)
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int k = 32 * K + Tl::krow(h, s), row = 32 * I + r;
                wr[I][K][s] = w[k * DP + row];
                wj[I][K][s] = (!BANDED || abs(k - row) <= g.band) ? wr[I][K][s] : 0.0f;
            }
    // row chain: wl[RB + d] = W[lane][lane + d] inside the band and the live block
    float wl[2 * RB + 1];
#pragma unroll
    for (int d = -RB; d <= RB; ++d) {
        const int k = lane + d;
        wl[RB + d] = (abs(d) <= g.band && lane < D && k >= 0 && k < D) ? w[k * DP + lane] : 0.0f;
    }
    copy_to_lds<64>(UT, wUT, m * DP);
    const float bias2[2] = {wbi[r], wbi[32 + r]};
    float hs[2] = {0.0f, 0.0f};               // Euler step sizes of rows r, 32 + r
    if constexpr (CELL == kCellEulerD) {
        hs[0] = wbi[2 * DP + r];
        hs[1] = wbi[2 * DP + 32 + r];
    }

    // W y for rows r and 32 + r (y: 64 floats in LDS)
    auto matvec = [&](const float (&W)[2][2][16], const float* y, float (&o)[2]) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int K = 0; K < 2; ++K)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 y4 = *reinterpret_cast<const float4*>(y + 32 * K + 8 * q + 4 * h);
                const float yk[4] = {y4.x, y4.y, y4.z, y4.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    a0 += W[0][K][4 * q + t] * yk[t];
                    a1 += W[1][K][4 * q + t] * yk[t];
                }
            }
        a0 += __shfl_xor(a0, 32, 64);
        a1 += __shfl_xor(a1, 32, 64);
        o[0] = a0;
        o[1] = a1;
    };
    // Pre-activations of the sub-chunk's steps at the rows Q (Q[j] = state
    // before step j): G[I] slot q = (W q_j + U x_j + b)[32I + r], j = krow(h, q).
    auto eval_tiles = [&](const float* Q, int Sc, v16f (&G)[2]) {
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
            for (int q = 0; q < 16; ++q) G[I][q] = bias2[I];
        const int SKM = ((m + 7) / 8) * 4;
        for (int s2 = 0; s2 < SKM; ++s2) {
            const int q = 8 * (s2 >> 2) + 4 * h + (s2 & 3);
            const bool qin = q < m;
            const float a = (r < Sc && qin) ? X[r * m + q] : 0.0f;
#pragma unroll
            for (int I = 0; I < 2; ++I) G[I] = Tl::step(a, qin ? UT[q * DP + 32 * I + r] : 0.0f, G[I]);
        }
#pragma unroll
        for (int K = 0; K < 2; ++K)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const float4 a4 = r < Sc ? *reinterpret_cast<const float4*>(Q + r * DP + 32 * K + 8 * qq + 4 * h)
                                         : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                const float ak[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int I = 0; I < 2; ++I) G[I] = Tl::step(ak[t], wr[I][K][4 * qq + t], G[I]);
            }
    };
    // v and coefficients of state 32I + r at step j from its pre-activation
    auto point = [&](float pre, float pi, int I, float (&co)[NCO]) {
        if constexpr (CELL == kCellTanhRnnD) {
            const float v = tanh_f(pre);
            co[0] = 1.0f - v * v;
            return v;
        } else {
            const float gv = tanh_f(pre);
            co[0] = 1.0f - hs[I];
            co[NCO - 1] = hs[I] * (1.0f - gv * gv);
            return pi + hs[I] * (gv - pi);
        }
    };
    // A~ d for rows r, 32 + r, d in LDS; dd: the lane's two entries of d
    auto jac_apply = [&](const float* d, const float (&dd)[2], const float (&co)[2][NCO], float (&o)[2]) {
        float a[2];
        matvec(wj, d, a);
#pragma unroll
        for (int I = 0; I < 2; ++I) {
            if constexpr (CELL == kCellTanhRnnD) o[I] = co[I][0] * a[I];
            else o[I] = co[I][0] * dd[I] + co[I][NCO - 1] * a[I];
        }
    };
    auto own = [&](const float (&x)[2]) { return h ? x[1] : x[0]; };
    // Row-chain form of jac_apply (RB > 0): the band product of the lane's
    // own row from its neighbours' entries through lane shifts, the partner
    // row (l ^ 32) by one exchange; no LDS vector and no barrier.
    auto jac_apply_row = [&](const float (&dd)[2], const float (&co)[2][NCO], float (&o)[2]) {
        const float dl = own(dd);
        float y = wl[RB] * dl, up = dl, dn = dl;
#pragma unroll
        for (int e = 1; e <= RB; ++e) {
            up = lane_from_below(up);
            dn = lane_from_above(dn);
            y = fmaf(wl[RB - e], up, y);
            y = fmaf(wl[RB + e], dn, y);
        }
        const float yo = __shfl_xor(y, 32, 64);
        const float a[2] = {h ? yo : y, h ? y : yo};
#pragma unroll
        for (int I = 0; I < 2; ++I) {
            if constexpr (CELL == kCellTanhRnnD) o[I] = co[I][0] * a[I];
            else o[I] = co[I][0] * dd[I] + co[I][NCO - 1] * a[I];
        }
    };

    // chunk map: identity on the live rows (row chain: row lane of M)
    v16f M[2][2];
    float Mr[RB > 0 ? DP : 1];
    if constexpr (RB > 0) {
#pragma unroll
        for (int col = 0; col < DP; ++col) Mr[col] = (col == lane && col < D) ? 1.0f : 0.0f;
    } else {
#pragma unroll
        for (int K = 0; K < 2; ++K)
#pragma unroll
            for (int J = 0; J < 2; ++J)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int row = 32 * K + Tl::krow(h, q), col = 32 * J + r;
                    M[K][J][q] = (row == col && col < D) ? 1.0f : 0.0f;
                }
    }
    float bg[2] = {0.0f, 0.0f};
    uint32_t rb = 0;
    const bool track = g.fpart != nullptr;
    uint32_t fb = 0xffffffffu;
    const bool has_next = c + 1 < g.NC;
    const float* cr = g.carry + ci * D;
    float shat[2] = {0.0f, 0.0f};
    float* sg = g.s + b * g.ss + static_cast<int64_t>(t0) * D;
    // maps pass of the advancing window: new steps from window row ff on
    const int ff = g.Tw - g.fill_rows;
    const float* fillrow = ff == 0 ? s0 : g.s + b * g.ss + static_cast<int64_t>(ff - 1) * D;
    const float* xg = g.x + b * g.xs + static_cast<int64_t>(t0) * m;

    // row t0-1 of the old and the new iterate (lane: its own row; shat: rows r, 32 + r)
    {
        float po = 0.0f, pn = 0.0f;
        if (olive) {
            if constexpr (PHASE == kPrologue) {
                po = pn = s0[orow];
            } else if constexpr (PHASE == kMaps) {
                po = pn = c == 0 ? s0[orow] : (t0 - 1 >= ff ? fillrow[orow] : sg[orow - D]);
            } else {
                po = (PHASE == kFirst || c == 0) ? s0[orow] : g.halo[(g.iter & 1) * HS + (ci - 1) * D + orow];
                pn = g.undamped ? cr[orow] : po + g.lam * (cr[orow] - po);
            }
        }
        if constexpr (PHASE == kFirst || PHASE == kSteady) {
            shat[0] = live0 ? cr[r] : 0.0f;
            shat[1] = live1 ? cr[32 + r] : 0.0f;
        }
        P[orow] = po;
        N[orow] = pn;
    }

    for (int j0 = 0; j0 < Lc; j0 += kSub) {
        const int Sc = min(kSub, Lc - j0);
        copy_to_lds<64>(X, xg + static_cast<int64_t>(j0) * m, Sc * m);
        if constexpr (PHASE == kPrologue || PHASE == kFirst) {
            for (int e = lane; e < Sc * DP; e += 64) {
                const int q = e % DP;
                P[DP + e] = q < D ? s0[q] : 0.0f;
            }
        } else if constexpr (PHASE == kMaps) {
            stage_maps_rows<64>(P + DP, DP, sg + static_cast<int64_t>(j0) * D, D, Sc, t0 + j0, ff, fillrow,
                                threadIdx.x);
        } else {
            copy_rows_to_lds<64>(P + DP, DP, sg + static_cast<int64_t>(j0) * D, D, Sc, D);
        }
        __syncthreads();
        v16f G[2];

        if constexpr (PHASE != kPrologue && PHASE != kMaps) {
            // maps of iteration i at the old iterate
            eval_tiles(P, Sc, G);
#pragma unroll
            for (int I = 0; I < 2; ++I)
#pragma unroll
                for (int q = 0; q < Tl::NSL; ++q) {
                    const int j = Tl::krow(h, q), row = 32 * I + r;
                    if (j < Sc) {
                        float co[NCO];
                        const float v = point(G[I][q], P[j * DP + row], I, co);
                        const bool lv = row < D;
                        V[j * DP + row] = lv ? v : 0.0f;
#pragma unroll
                        for (int u = 0; u < NCO; ++u) CO[(u * kSub + j) * DP + row] = lv ? co[u] : 0.0f;
                    }
                }
            __syncthreads();
            // replay from the carry, damping
            for (int j = 0; j < Sc; ++j) {
                float dd[2];
                dd[0] = live0 ? shat[0] - P[j * DP + r] : 0.0f;
                dd[1] = live1 ? shat[1] - P[j * DP + 32 + r] : 0.0f;
                if constexpr (RB == 0) {
                    YV[orow] = own(dd);
                    __syncthreads();
                }
                float co[2][NCO];
#pragma unroll
                for (int I = 0; I < 2; ++I)
#pragma unroll
                    for (int q = 0; q < NCO; ++q) co[I][q] = CO[(q * kSub + j) * DP + 32 * I + r];
                float ad[2];
                if constexpr (RB > 0) jac_apply_row(dd, co, ad);
                else jac_apply(YV, dd, co, ad);
                float sn[2];
#pragma unroll
                for (int I = 0; I < 2; ++I) {
                    const int row = 32 * I + r;
                    shat[I] = V[j * DP + row] + ad[I];
                    if (j0 + j == Lc - 1 && has_next && row < D) shat[I] = cr[D + row];
                    const float so = P[(j + 1) * DP + row];
                    sn[I] = g.undamped ? shat[I] : so + g.lam * (shat[I] - so);
                }
                N[(j + 1) * DP + orow] = olive ? own(sn) : 0.0f;
                if constexpr (RB == 0) __syncthreads();      // YV is rewritten next step
            }
            if constexpr (RB > 0) __syncthreads();
            for (int e = lane; e < Sc * D; e += 64) {
                const int j = e / D, q = e % D;
                sg[static_cast<int64_t>(j0 + j) * D + q] = N[(j + 1) * DP + q];
            }
        } else {
            for (int e = lane; e < Sc * DP; e += 64) N[DP + e] = P[DP + e];
        }
        __syncthreads();

        // maps of iteration i+1 at the new iterate; residual
        eval_tiles(N, Sc, G);
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
            for (int q = 0; q < Tl::NSL; ++q) {
                const int j = Tl::krow(h, q), row = 32 * I + r;
                if (j < Sc) {
                    float co[NCO];
                    const float v = point(G[I][q], N[j * DP + row], I, co);
                    const bool lv = row < D;
                    if (lv) {
                        const float d = N[(j + 1) * DP + row] - v;
                        rb = max(rb, abs_bits(d));
                        if (track && !(fabsf(d) <= g.tol)) fb = min(fb, static_cast<uint32_t>(j0 + j));
                    }
                    V[j * DP + row] = lv ? v : 0.0f;
#pragma unroll
                    for (int u = 0; u < NCO; ++u) CO[(u * kSub + j) * DP + row] = lv ? co[u] : 0.0f;
                }
            }
        __syncthreads();

        // extend the chunk map over the sub-chunk
        for (int j = 0; j < Sc; ++j) {
            v16f C[2][2];
            if constexpr (RB == 0) {
#pragma unroll
                for (int I = 0; I < 2; ++I)
#pragma unroll
                    for (int J = 0; J < 2; ++J) {
#pragma unroll
                        for (int q = 0; q < 16; ++q) C[I][J][q] = 0.0f;
#pragma unroll
                        for (int K = 0; K < 2; ++K)
#pragma unroll
                            for (int s = 0; s < 16; ++s) C[I][J] = Tl::step(wj[I][K][s], M[K][J][s], C[I][J]);
                    }
            }
            // offset: bg <- A_j (bg - p_j) + v_j  (p_j = N[j])
            float dbi[2];
            dbi[0] = live0 ? bg[0] - N[j * DP + r] : 0.0f;
            dbi[1] = live1 ? bg[1] - N[j * DP + 32 + r] : 0.0f;
            if constexpr (RB == 0) {
                YV[DP + orow] = own(dbi);
                __syncthreads();
            }
            {
                float co[2][NCO];
#pragma unroll
                for (int I = 0; I < 2; ++I)
#pragma unroll
                    for (int q = 0; q < NCO; ++q) co[I][q] = CO[(q * kSub + j) * DP + 32 * I + r];
                float ad[2];
                if constexpr (RB > 0) jac_apply_row(dbi, co, ad);
                else jac_apply(YV + DP, dbi, co, ad);
#pragma unroll
                for (int I = 0; I < 2; ++I) bg[I] = V[j * DP + 32 * I + r] + ad[I];
            }
            if constexpr (RB > 0) {
                // row lane of M <- row lane of A_j M, A_j = diag(c0) band(W)
                // (tanh RNN) or diag(c0) + diag(c1) band(W) (Euler step)
                const float c0 = CO[j * DP + lane];
                const float c1 = CO[((NCO - 1) * kSub + j) * DP + lane];
#pragma unroll
                for (int col = 0; col < DP; ++col) {
                    float t = wl[RB] * Mr[col];
                    float up = Mr[col], dn = Mr[col];
#pragma unroll
                    for (int d = 1; d <= RB; ++d) {
                        up = lane_from_below(up);     // M[lane - d][col]
                        dn = lane_from_above(dn);     // M[lane + d][col]
                        t = fmaf(wl[RB - d], up, t);
                        t = fmaf(wl[RB + d], dn, t);
                    }
                    if constexpr (CELL == kCellTanhRnnD) Mr[col] = c0 * t;
                    else Mr[col] = fmaf(c0, Mr[col], c1 * t);
                }
            }
            // row scalings of the accumulator rows 32 I + krow(h, q)
#pragma unroll
            for (int I = 0; I < 2 && RB == 0; ++I) {
                float rs[NCO][16];
#pragma unroll
                for (int q = 0; q < NCO; ++q)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float4 c4 = *reinterpret_cast<const float4*>(CO + (q * kSub + j) * DP + 32 * I + 8 * u + 4 * h);
                        rs[q][4 * u] = c4.x;
                        rs[q][4 * u + 1] = c4.y;
                        rs[q][4 * u + 2] = c4.z;
                        rs[q][4 * u + 3] = c4.w;
                    }
#pragma unroll
                for (int J = 0; J < 2; ++J)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        if constexpr (CELL == kCellTanhRnnD) M[I][J][q] = rs[0][q] * C[I][J][q];
                        else M[I][J][q] = rs[0][q] * M[I][J][q] + rs[NCO - 1][q] * C[I][J][q];
                    }
            }
            if constexpr (RB == 0) __syncthreads();      // YV is rewritten next step
        }
        // carry the last rows into the next sub-chunk
        const float plast = P[Sc * DP + orow];
        const float nlast = N[Sc * DP + orow];
        __syncthreads();
        P[orow] = plast;
        N[orow] = nlast;
        __syncthreads();
    }

    if constexpr (PHASE == kMaps) {
        if (olive) g.halo[(g.iter & 1) * HS + ci * D + orow] = N[orow];
    } else if constexpr (PHASE != kPrologue) {
        if (olive) g.halo[((g.iter + 1) & 1) * HS + ci * D + orow] = N[orow];
    }
    float* aA = g.aggA + ci * D * D;
    if constexpr (RB > 0) {
#pragma unroll
        for (int col = 0; col < DP; ++col)
            if (lane < D && col < D) aA[lane * D + col] = Mr[col];
    } else {
#pragma unroll
        for (int K = 0; K < 2; ++K)
#pragma unroll
            for (int J = 0; J < 2; ++J)
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int row = 32 * K + Tl::krow(h, q), col = 32 * J + r;
                    if (row < D && col < D) aA[row * D + col] = M[K][J][q];
                }
    }
    if (olive) g.aggB[ci * D + orow] = own(bg);
    rb = wave_max_u32(rb);
    if (lane == 0) g.rpart[ci] = rb;
    if (track) {
        fb = ~wave_max_u32(~fb);
        if (lane == 0) g.fpart[ci] = fb == 0xffffffffu ? fb : t0 + fb;
    }
}

template <int CELL, bool BANDED, int RB>
static hipError_t launch_dense64_b(int phase, const CellArgs& a, hipStream_t st) {
    const size_t lds = D64Lds<CELL>::floats(a.m) * sizeof(float);
    const dim3 grid(a.NC, a.B);
    if (phase == kPrologue) dense64_pass<CELL, kPrologue, BANDED, RB><<<grid, 64, lds, st>>>(a);
    else if (phase == kFirst) dense64_pass<CELL, kFirst, BANDED, RB><<<grid, 64, lds, st>>>(a);
    else if (phase == kMaps) dense64_pass<CELL, kMaps, BANDED, RB><<<grid, 64, lds, st>>>(a);
    else return launch_maybe_timed(dense64_pass<CELL, kSteady, BANDED, RB>, grid, dim3(64), lds, st, a);
    return hipGetLastError();
}

// band < D - 1 selects the masked Jacobian weights; a band of at most
// kRowBand diagonals each side extends the chunk map on the vector ALUs.
constexpr int kRowBand = 2;

template <int CELL>
static hipError_t launch_dense64(int phase, const CellArgs& a, hipStream_t st) {
    if (a.band >= a.D - 1) return launch_dense64_b<CELL, false, 0>(phase, a, st);
    return a.band <= kRowBand ? launch_dense64_b<CELL, true, kRowBand>(phase, a, st)
                              : launch_dense64_b<CELL, true, 0>(phase, a, st);
}

template <int CELL, int DP, bool BANDED, bool SPLIT>
static hipError_t launch_dense_phase_s(int phase, const CellArgs& a, hipStream_t st) {
    const size_t lds = DLds<CELL, DP>::floats(a.m, SPLIT) * sizeof(float);
    const dim3 grid(a.NC, a.B);
    const int nt = SPLIT ? 128 : 64;
    if (phase == kPrologue) dense_pass<CELL, DP, kPrologue, BANDED, SPLIT><<<grid, nt, lds, st>>>(a);
    else if (phase == kFirst) dense_pass<CELL, DP, kFirst, BANDED, SPLIT><<<grid, nt, lds, st>>>(a);
    else if (phase == kMaps) dense_pass<CELL, DP, kMaps, BANDED, SPLIT><<<grid, nt, lds, st>>>(a);
    else return launch_maybe_timed(dense_pass<CELL, DP, kSteady, BANDED, SPLIT>, grid, dim3(nt), lds, st, a);
    return hipGetLastError();
}

// Two wavefronts per chunk when the chunks alone (one wavefront each) would
// leave SIMDs without a second chunk: at most one chunk per SIMD (the chip
// has 1024).

template <int CELL, int DP, bool BANDED>
static hipError_t launch_dense_phase_b(int phase, const CellArgs& a, hipStream_t st) {
    return static_cast<int64_t>(a.NC) * a.B <= kSplitMax
               ? launch_dense_phase_s<CELL, DP, BANDED, true>(phase, a, st)
               : launch_dense_phase_s<CELL, DP, BANDED, false>(phase, a, st);
}

// band < D - 1 selects the masked Jacobian weights; Newton passes band = D.
template <int CELL, int DP>
static hipError_t launch_dense_phase(int phase, const CellArgs& a, hipStream_t st) {
    return a.band < a.D - 1 ? launch_dense_phase_b<CELL, DP, true>(phase, a, st)
                            : launch_dense_phase_b<CELL, DP, false>(phase, a, st);
}

bool dense_mfma_supported(int kind, int DP, int m) {
    if (DP == 64) return kind != kCellGruD && dense_mfma_lds_bytes(kind, 64, m) <= 64 * 1024;
    if (DP != 16 && DP != 32) return false;
    return dense_mfma_lds_bytes(kind, 32, m) <= 64 * 1024;
}

size_t dense_mfma_lds_bytes(int kind, int DP, int m) {
    if (DP == 64) {
        return (kind == kCellEulerD ? D64Lds<kCellEulerD>::floats(m) : D64Lds<kCellTanhRnnD>::floats(m)) * sizeof(float);
    }
    // the larger (split) layout, so either launch form fits
    if (kind == kCellTanhRnnD) return (DP == 16 ? DLds<kCellTanhRnnD, 16>::floats(m, true) : DLds<kCellTanhRnnD, 32>::floats(m, true)) * sizeof(float);
    if (kind == kCellEulerD) return (DP == 16 ? DLds<kCellEulerD, 16>::floats(m, true) : DLds<kCellEulerD, 32>::floats(m, true)) * sizeof(float);
    return (DP == 16 ? DLds<kCellGruD, 16>::floats(m, true) : DLds<kCellGruD, 32>::floats(m, true)) * sizeof(float);
}

hipError_t launch_dense_mfma_pass(int kind, int DP, int phase, const CellArgs& a, hipStream_t st) {
    if (DP == 64) {
        if (kind == kCellTanhRnnD) return launch_dense64<kCellTanhRnnD>(phase, a, st);
        if (kind == kCellEulerD) return launch_dense64<kCellEulerD>(phase, a, st);
        return hipErrorInvalidValue;
    }
    if (kind == kCellTanhRnnD) {
        return DP == 16 ? launch_dense_phase<kCellTanhRnnD, 16>(phase, a, st)
                        : launch_dense_phase<kCellTanhRnnD, 32>(phase, a, st);
    }
    if (kind == kCellEulerD) {
        return DP == 16 ? launch_dense_phase<kCellEulerD, 16>(phase, a, st)
                        : launch_dense_phase<kCellEulerD, 32>(phase, a, st);
    }
    return DP == 16 ? launch_dense_phase<kCellGruD, 16>(phase, a, st)
                    : launch_dense_phase<kCellGruD, 32>(phase, a, st);
}

}  // namespace pn
