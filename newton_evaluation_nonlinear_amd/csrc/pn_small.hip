// One-workgroup solver for small problems: every window, iteration and
// convergence check of a solve in a single launch.
//
// When the whole window (B rows x W steps, at most 1024 or 512 (b, t) pairs)
// fits one workgroup, the multi-launch driver spends its time on launches and
// host round trips, not on arithmetic.  Here 256 threads hold the iterate of
// the window in LDS and run the iteration of [PN §1.2] to its stop:
//   1. each thread evaluates the cell at p_t = s_{t-1} for its S consecutive
//      (b, t) pairs (S <= 4), giving v_t = f_t(p_t), the residual |s_t - v_t|
//      and the affine map of the step, (A~_t, b_t = v_t - A~_t p_t); the
//      first step of a row has p = s_0 fixed, so its map is the constant
//      (0, v_1), which also cuts the scan at row boundaries;
//   2. the workgroup max of the residual decides the stop (non-finite, then
//      r <= tol, then the update cap), the same rule as the multi-launch
//      driver;
//   3. the thread composes its S maps serially, the workgroup scans the 256
//      thread aggregates [PN §2.1]: an in-register inclusive scan per
//      wavefront built from DPP row shifts (1, 2, 4, 8) and row broadcasts
//      (lanes 15 and 31), a whole-wavefront shift by one lane for the
//      exclusive prefix, and an LDS scan over the four wavefront totals;
//   4. the thread replays its steps from that prefix, damps, and writes the
//      new iterate back to LDS.
// The affine combine is, for an earlier map e and a later map l,
// (A_l A_e, A_l b_e + b_l).  D is padded to DM (4 or 8) with zero weights, so
// padded coordinates stay exactly zero.  Matrix cells only (tanh RNN, GRU,
// Euler step); every mode, damping and consecutive windows.

#include "pn_device.hpp"
#include "pn_launch.hpp"

namespace pn {

namespace {

constexpr int kSmallThreads = 256;
constexpr int kCellRnn = 1, kCellGruS = 2, kCellEulerS = 3;

template <int DM>
constexpr int small_max_pairs() { return DM <= 4 ? 1024 : 512; }

template <int DM, bool DENSE>
struct Map {
    static constexpr int NA = DENSE ? DM * DM : DM;
    float a[NA];    // dense: A[i][k] = a[i * DM + k]; diagonal: A[i][i] = a[i]
    float b[DM];
};

template <int DM, bool DENSE>
__device__ __forceinline__ void set_identity(Map<DM, DENSE>& m) {
#pragma unroll
    for (int q = 0; q < Map<DM, DENSE>::NA; ++q) {
        if constexpr (DENSE) m.a[q] = (q / DM == q % DM) ? 1.0f : 0.0f;
        else m.a[q] = 1.0f;
    }
#pragma unroll
    for (int i = 0; i < DM; ++i) m.b[i] = 0.0f;
}

// later o earlier = (A_l A_e, A_l b_e + b_l)
template <int DM, bool DENSE>
__device__ __forceinline__ Map<DM, DENSE> compose(const Map<DM, DENSE>& l, const Map<DM, DENSE>& e) {
    Map<DM, DENSE> r;
    if constexpr (DENSE) {
#pragma unroll
        for (int i = 0; i < DM; ++i) {
#pragma unroll
            for (int k = 0; k < DM; ++k) {
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < DM; ++j) acc = fmaf(l.a[i * DM + j], e.a[j * DM + k], acc);
                r.a[i * DM + k] = acc;
            }
            float acc = l.b[i];
#pragma unroll
            for (int j = 0; j < DM; ++j) acc = fmaf(l.a[i * DM + j], e.b[j], acc);
            r.b[i] = acc;
        }
    } else {
#pragma unroll
        for (int i = 0; i < DM; ++i) {
            r.a[i] = l.a[i] * e.a[i];
            r.b[i] = fmaf(l.a[i], e.b[i], l.b[i]);
        }
    }
    return r;
}

// Every word of v moved by one DPP pattern; lanes without a source (or
// outside ROW_MASK) receive `old`.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL,
                                                      ROW_MASK, 0xf, false));
}

template <int CTRL, int ROW_MASK, int DM, bool DENSE>
__device__ __forceinline__ Map<DM, DENSE> dpp_map(const Map<DM, DENSE>& v, const Map<DM, DENSE>& old) {
    Map<DM, DENSE> r;
#pragma unroll
    for (int q = 0; q < Map<DM, DENSE>::NA; ++q) r.a[q] = dpp_mov<CTRL, ROW_MASK>(old.a[q], v.a[q]);
#pragma unroll
    for (int i = 0; i < DM; ++i) r.b[i] = dpp_mov<CTRL, ROW_MASK>(old.b[i], v.b[i]);
    return r;
}

// DPP controls (GFX9): row_shr:n = 0x110 + n, wave_shr:1 = 0x138,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kWaveShr1 = 0x138, kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive scan of one map per lane over the 64 lanes of a wavefront.
template <int DM, bool DENSE>
__device__ __forceinline__ Map<DM, DENSE> wave_inclusive_scan(Map<DM, DENSE> v, const Map<DM, DENSE>& id) {
    v = compose(v, dpp_map<kRowShr1, 0xf>(v, id));
    v = compose(v, dpp_map<kRowShr2, 0xf>(v, id));
    v = compose(v, dpp_map<kRowShr4, 0xf>(v, id));
    v = compose(v, dpp_map<kRowShr8, 0xf>(v, id));
    // rows 1 and 3 take the prefix ending at lanes 15 and 47, then rows 2
    // and 3 the prefix ending at lane 31
    v = compose(v, dpp_map<kRowBcast15, 0xa>(v, id));
    v = compose(v, dpp_map<kRowBcast31, 0xc>(v, id));
    return v;
}

template <int KIND>
struct SmallCellTraits { static constexpr int NG = 1; };
template <>
struct SmallCellTraits<kCellGruS> { static constexpr int NG = 3; };

// Cell value v = f(p) and the step's map (A~, v - A~ p) for `mode`; `head`:
// the first step of a row, whose map is the constant (0, v).
// Wl: recurrent weights [NG][DM][DM] (row i, column k); c: the input
// projection of the step [NG][DM] (biases folded in, b_hn excluded);
// ex: GRU b_hn[DM] / Euler h[DM].
template <int KIND, int DM, bool DENSE>
__device__ __forceinline__ void eval_step(const float* Wl, const float* ex, const float* c, const float (&p)[DM],
                                          int mode, int band, bool head, float (&v)[DM],
                                          Map<DM, DENSE>& el) {
    constexpr int NG = SmallCellTraits<KIND>::NG;
    float h[NG][DM];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int i = 0; i < DM; ++i) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < DM; ++k) acc = fmaf(Wl[(g * DM + i) * DM + k], p[k], acc);
            h[g][i] = acc;
        }
    }
    float co[3][DM];      // row scalings of the weight blocks in A_t, and the diagonal term
    float dg[DM];
#pragma unroll
    for (int i = 0; i < DM; ++i) {
        if constexpr (KIND == kCellRnn) {
            v[i] = tanh_f(c[i] + h[0][i]);
            co[0][i] = 1.0f - v[i] * v[i];
            dg[i] = 0.0f;
        } else if constexpr (KIND == kCellEulerS) {
            const float gv = tanh_f(c[i] + h[0][i]);
            v[i] = fmaf(ex[i], gv - p[i], p[i]);
            co[0][i] = ex[i] * (1.0f - gv * gv);
            dg[i] = 1.0f - ex[i];
        } else {
            const float r = sigmoid_f(c[i] + h[0][i]);
            const float z = sigmoid_f(c[DM + i] + h[1][i]);
            const float gg = h[2][i] + ex[i];
            const float n = tanh_f(fmaf(r, gg, c[2 * DM + i]));
            v[i] = fmaf(z, p[i] - n, n);
            const float cn = (1.0f - z) * (1.0f - n * n) * r;
            co[0][i] = cn * gg * (1.0f - r);      // W_hr
            co[1][i] = (p[i] - n) * z * (1.0f - z);  // W_hz
            co[2][i] = cn;                        // W_hn
            dg[i] = z;
        }
    }
    if (head) {
#pragma unroll
        for (int q = 0; q < Map<DM, DENSE>::NA; ++q) el.a[q] = 0.0f;
#pragma unroll
        for (int i = 0; i < DM; ++i) el.b[i] = v[i];
        return;
    }
    if constexpr (DENSE) {
        // Newton (band >= D) or the band |i - k| <= band of A_t
#pragma unroll
        for (int i = 0; i < DM; ++i) {
#pragma unroll
            for (int k = 0; k < DM; ++k) {
                float a = (i == k) ? dg[i] : 0.0f;
#pragma unroll
                for (int g = 0; g < NG; ++g) a = fmaf(co[g][i], Wl[(g * DM + i) * DM + k], a);
                el.a[i * DM + k] = (i - k <= band && k - i <= band) ? a : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < DM; ++i) {
            float acc = v[i];
#pragma unroll
            for (int k = 0; k < DM; ++k) acc = fmaf(-el.a[i * DM + k], p[k], acc);
            el.b[i] = acc;
        }
    } else {
#pragma unroll
        for (int i = 0; i < DM; ++i) {
            float a = dg[i];
#pragma unroll
            for (int g = 0; g < NG; ++g) a = fmaf(co[g][i], Wl[(g * DM + i) * DM + i], a);
            a = mode == kJacobi ? 0.0f : mode == kPicard ? 1.0f : a;
            el.a[i] = a;
            el.b[i] = fmaf(-a, p[i], v[i]);
        }
    }
}

template <int KIND, int DM, bool DENSE>
__global__ __launch_bounds__(kSmallThreads) void small_solve_kernel(SmallArgs a) {
    constexpr int NG = SmallCellTraits<KIND>::NG;
    constexpr int NMAX = small_max_pairs<DM>();
    constexpr int SMAX = NMAX / kSmallThreads;
    using M = Map<DM, DENSE>;
    // the iterate of the window, (b, t) flattened, in two buffers: an update
    // reads one and writes the other
    __shared__ float Sb[2][NMAX * DM];
    __shared__ float s0w[NMAX * DM];         // initial state of each row of the window
    __shared__ float carr[NMAX * NG * DM];   // input projections of the window's steps
    __shared__ float Wl[NG * DM * DM];
    __shared__ float ex[DM];
    __shared__ M tot[kSmallThreads / 64];    // wavefront totals of the scan
    __shared__ uint32_t red[kSmallThreads / 64];   // wavefront maxima of the residual
    // single-gate cells at DM = 4 keep their 16 recurrent weights in registers
    constexpr bool kWReg = NG * DM * DM <= 16;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int D = a.D, m = a.m, B = a.B;
    // weights, zero-padded to DM: tanh RNN / Euler W[D*D] | U[D*m] | b[D] (| h[D]);
    // GRU W_ih[3D*m] | W_hh[3D*D] | b_ih[3D] | b_hh[3D]
    const float* P = a.params;
    const float* Wrec = KIND == kCellGruS ? P + 3 * D * m : P;
    for (int q = tid; q < NG * DM * DM; q += kSmallThreads) {
        const int g = q / (DM * DM), i = (q / DM) % DM, k = q % DM;
        Wl[q] = (i < D && k < D) ? Wrec[(g * D + i) * D + k] : 0.0f;
    }
    for (int i = tid; i < DM; i += kSmallThreads) {
        float e = 0.0f;
        if (i < D) {
            if constexpr (KIND == kCellGruS) e = P[3 * D * m + 3 * D * D + 3 * D + 2 * D + i];  // b_hn
            else if constexpr (KIND == kCellEulerS) e = P[D * D + D * m + D + i];            // h
        }
        ex[i] = e;
    }
    M id;
    set_identity(id);
    __syncthreads();
    float Wr[kWReg ? NG * DM * DM : 1];
    if constexpr (kWReg) {
#pragma unroll
        for (int q = 0; q < NG * DM * DM; ++q) Wr[q] = Wl[q];
    }
    auto eval = [&](const float* c, const float (&p)[DM], bool head, float (&v)[DM], M& el) {
        if constexpr (kWReg) eval_step<KIND, DM, DENSE>(Wr, ex, c, p, a.mode, a.band, head, v, el);
        else eval_step<KIND, DM, DENSE>(Wl, ex, c, p, a.mode, a.band, head, v, el);
    };
    int hist_len = 0, Wprev = 0, cur = 0;
    if (tid == 0) {
        for (int w = 0; w < a.nwin; ++w) a.win_iters[w] = -1;
    }
    for (int w = 0; w < a.nwin; ++w) {
        const int64_t w0 = static_cast<int64_t>(w) * a.W;
        const int Tw = static_cast<int>(a.T - w0 < a.W ? a.T - w0 : a.W);
        const int n = B * Tw;
        const int S = (n + kSmallThreads - 1) / kSmallThreads;
        // initial state of each row: s_0, or the last state of the window before
        float s0v[SMAX][DM];
#pragma unroll
        for (int u = 0; u < SMAX; ++u) {
            const int bb = tid + u * kSmallThreads;
#pragma unroll
            for (int i = 0; i < DM; ++i) {
                float e = 0.0f;
                if (bb < B && i < D) {
                    e = w == 0 ? a.s0[static_cast<int64_t>(bb) * D + i]
                               : Sb[cur][(bb * Wprev + Wprev - 1) * DM + i];
                }
                s0v[u][i] = e;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < SMAX; ++u) {
            const int bb = tid + u * kSmallThreads;
            if (bb < B) {
#pragma unroll
                for (int i = 0; i < DM; ++i) s0w[bb * DM + i] = s0v[u][i];
            }
        }
        __syncthreads();
        // initial iterate s_t = s_0 of its row, and the input projections
        for (int e = tid; e < n; e += kSmallThreads) {
            const int bb = e / Tw, t = e - bb * Tw;
#pragma unroll
            for (int i = 0; i < DM; ++i) Sb[0][e * DM + i] = s0w[bb * DM + i];
            const float* xe = a.x + (static_cast<int64_t>(bb) * a.T + w0 + t) * m;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
#pragma unroll
                for (int i = 0; i < DM; ++i) {
                    float acc = 0.0f;
                    if (i < D) {
                        if constexpr (KIND == kCellGruS) {
                            const float* Wi = P + (g * D + i) * m;
                            for (int q = 0; q < m; ++q) acc = fmaf(Wi[q], xe[q], acc);
                            const float* bih = P + 3 * D * m + 3 * D * D;
                            acc += bih[g * D + i];
                            if (g < 2) acc += bih[3 * D + g * D + i];   // b_hr, b_hz
                        } else {
                            const float* U = P + D * D + i * m;
                            for (int q = 0; q < m; ++q) acc = fmaf(U[q], xe[q], acc);
                            acc += P[D * D + D * m + i];
                        }
                    }
                    carr[(e * NG + g) * DM + i] = acc;
                }
            }
        }
        __syncthreads();

        cur = 0;
        int K = 0, status = kStOk;
        for (int it = 0;; ++it) {
            const float* Sc = Sb[cur];
            // 1. evaluate the cell at p_t for this thread's steps
            uint32_t rl = 0;
            M agg;
            set_identity(agg);
#pragma unroll
            for (int s = 0; s < SMAX; ++s) {
                const int e = tid * S + s;
                if (s >= S || e >= n) break;
                const int bb = e / Tw, t = e - bb * Tw;
                float p[DM], v[DM];
#pragma unroll
                for (int i = 0; i < DM; ++i) p[i] = t == 0 ? s0w[bb * DM + i] : Sc[(e - 1) * DM + i];
                M el;
                eval(carr + e * NG * DM, p, t == 0, v, el);
#pragma unroll
                for (int i = 0; i < DM; ++i) {
                    const uint32_t q = abs_bits(Sc[e * DM + i] - v[i]);
                    rl = rl > q ? rl : q;
                }
                agg = compose(el, agg);
            }
            // 2. the wavefront scans of the thread aggregates and the
            // wavefront maxima of the residual, published with one barrier;
            // the scan is taken before the stop decision and unused if it stops
            const M incl = wave_inclusive_scan(agg, id);
            const uint32_t wmax = wave_max_u32(rl);
            if (lane == 63) tot[wave] = incl;
            if (lane == 0) red[wave] = wmax;
            M excl = dpp_map<kWaveShr1, 0xf>(incl, id);
            __syncthreads();
            uint32_t rb = red[0];
#pragma unroll
            for (int k = 1; k < kSmallThreads / 64; ++k) rb = rb > red[k] ? rb : red[k];
            // 3. the check of iteration it
            if (tid == 0 && hist_len < a.hist_cap) a.hist[hist_len] = __uint_as_float(rb);
            ++hist_len;
            int st = -1;
            if (rb >= kNonFiniteBits) st = kStNonFinite;
            else if (__uint_as_float(rb) <= a.tol) st = kStOk;
            else if (it >= a.max_iter) st = kStNotConverged;
            if (st >= 0) {
                K = it;
                status = st;
                break;
            }
            M pre = id;
            for (int k = 0; k < wave; ++k) pre = compose(tot[k], pre);
            excl = compose(excl, pre);
            // 4. replay from the prefix, damp, store into the other buffer
            float* Sn = Sb[cur ^ 1];
            float carry[DM];
#pragma unroll
            for (int i = 0; i < DM; ++i) carry[i] = excl.b[i];
#pragma unroll
            for (int s = 0; s < SMAX; ++s) {
                const int e = tid * S + s;
                if (s >= S || e >= n) break;
                const int bb = e / Tw, t = e - bb * Tw;
                float p[DM], v[DM];
#pragma unroll
                for (int i = 0; i < DM; ++i) p[i] = t == 0 ? s0w[bb * DM + i] : Sc[(e - 1) * DM + i];
                M el;
                eval(carr + e * NG * DM, p, t == 0, v, el);
#pragma unroll
                for (int i = 0; i < DM; ++i) {
                    float acc = el.b[i];
                    if constexpr (DENSE) {
#pragma unroll
                        for (int k = 0; k < DM; ++k) acc = fmaf(el.a[i * DM + k], carry[k], acc);
                    } else {
                        acc = fmaf(el.a[i], carry[i], acc);
                    }
                    v[i] = acc;
                }
#pragma unroll
                for (int i = 0; i < DM; ++i) {
                    carry[i] = v[i];
                    const float sc = Sc[e * DM + i];
                    Sn[e * DM + i] = a.undamped ? v[i] : fmaf(a.lam, v[i] - sc, sc);
                }
            }
            // the new iterate, the totals and the maxima are read again only
            // after this barrier
            __syncthreads();
            cur ^= 1;
        }
        // the window's result (the last iterate) to out
        for (int e = tid; e < n; e += kSmallThreads) {
            const int bb = e / Tw, t = e - bb * Tw;
            float* o = a.out + (static_cast<int64_t>(bb) * a.T + w0 + t) * D;
            for (int i = 0; i < D; ++i) o[i] = Sb[cur][e * DM + i];
        }
        if (tid == 0) {
            a.win_iters[w] = K;
            a.win_status[w] = status;
        }
        Wprev = Tw;
        if (status == kStNonFinite) break;
    }
    if (tid == 0) *a.hist_len = hist_len;
}

template <int KIND, int DM>
hipError_t launch_kind(bool dense, const SmallArgs& a, hipStream_t st) {
    if (dense) return launch_maybe_timed(small_solve_kernel<KIND, DM, true>, dim3(1), dim3(kSmallThreads), 0, st, a);
    return launch_maybe_timed(small_solve_kernel<KIND, DM, false>, dim3(1), dim3(kSmallThreads), 0, st, a);
}

template <int DM>
hipError_t launch_dm(int kind, bool dense, const SmallArgs& a, hipStream_t st) {
    if (kind == kCellRnn) return launch_kind<kCellRnn, DM>(dense, a, st);
    if (kind == kCellGruS) return launch_kind<kCellGruS, DM>(dense, a, st);
    return launch_kind<kCellEulerS, DM>(dense, a, st);
}

}  // namespace

int small_max_pairs_for(int D) { return D <= 4 ? small_max_pairs<4>() : D <= 8 ? small_max_pairs<8>() : 0; }

hipError_t launch_small_solve(int kind, bool dense, const SmallArgs& a, hipStream_t st) {
    if (a.D <= 4) return launch_dm<4>(kind, dense, a, st);
    return launch_dm<8>(kind, dense, a, st);
}

}  // namespace pn
