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
// With float storage the first four updates move less: s^(0) = s0 is known
// everywhere, and s^(l) follows bit for bit from x, s0 and the carries of
// iterations 0 .. l-1 (replaying iteration l from its carry gives s^(l+1)).
// So updates 1 .. 3 (kFirstNS, kSecondNS, kThirdNS) read only x and store
// nothing, update l + 1 recomputing s^(1) .. s^(l) on the way (one more tanh
// per element and level), and update 4 (kFourthR) recomputes s^(1) .. s^(3)
// and stores s^(4): 4, 4, 4 and 8 bytes per element instead of 12.  If the
// loop stops right after update l <= 3, the form of update l that stores
// (kFirst, kSecondR, kThirdR) runs once more to write s^(l).
//
// Layout: lanes run along channels (row-contiguous in [B, T, D]); each thread
// walks the L steps of its chunk serially, so loads are fully coalesced rows
// and the recurrence stays in registers.
//
// Storage type S: float, or _Float16 for reduced-precision storage of x and
// of the iterate [PN §2.3, §4.2] (compute stays float32).  With _Float16 every
// stored state is rounded to nearest-even, and the value a thread carries on
// to the next step is the rounded one, so the state the next step sees is
// exactly the stored state.

#include <type_traits>

#include "pn_device.hpp"
#include "pn_launch.hpp"

namespace pn {

// Steps per prefetch group: the loads of group g+1 are issued before group g
// is computed, so every thread keeps 2*U loads in flight.
constexpr int kU = 8;
constexpr int kUP = 16;   // passes that only read x prefetch twice as far

// Storage element of one thread: NCH adjacent channels moved as one access
// (a float; or two binary16 values in one 4-byte access, so a wave moves as
// many bytes per load instruction as with float storage).
template <typename S, int NCH> struct Pack;
template <> struct Pack<float, 1> { typedef float V; };
template <> struct Pack<_Float16, 1> { typedef _Float16 V; };
template <> struct Pack<_Float16, 2> { typedef _Float16 V __attribute__((ext_vector_type(2))); };

template <typename S, int NCH>
__device__ __forceinline__ void unpack(const typename Pack<S, NCH>::V& v, float (&f)[NCH]) {
    if constexpr (NCH == 1) {
        f[0] = static_cast<float>(v);
    } else {
        f[0] = static_cast<float>(v.x);
        f[1] = static_cast<float>(v.y);
    }
}

// Round the NCH values to the storage type; f receives the rounded values.
template <typename S, int NCH>
__device__ __forceinline__ typename Pack<S, NCH>::V pack(float (&f)[NCH]) {
    typename Pack<S, NCH>::V v;
    if constexpr (NCH == 1) {
        v = static_cast<S>(f[0]);
        f[0] = static_cast<float>(v);
    } else {
        v.x = static_cast<S>(f[0]);
        v.y = static_cast<S>(f[1]);
        f[0] = static_cast<float>(v.x);
        f[1] = static_cast<float>(v.y);
    }
    return v;
}

// float32 value after a round trip through the storage type
template <typename S>
__device__ __forceinline__ float stored(float v) {
    return static_cast<float>(static_cast<S>(v));
}

// Rows of a [.., T, D] array inside one chunk, as seen by one wavefront:
// buffer loads and stores whose base (row 0 at the wave's first channel) is
// uniform over the wave, with the row offset a scalar operand and the lane's
// byte offset the vector one, so addressing costs no vector instruction.
// Offsets stay below 2^31 (the planner bounds chunk rows x row bytes); the
// callers' row tests keep every access inside the chunk.
// The resource is a raw buffer (stride 0) whose range (2^31 - 1 bytes) never
// clips an access here; its last word is the gfx9 format word for 32-bit data.
template <typename V> struct Rows {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lo;     // lane offset in bytes
    int32_t rs;      // row stride in bytes
    __device__ __forceinline__ Rows(const void* base, uint32_t lane_off, int32_t row_bytes)
        : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), 0x7fffffff,
                                                 0x00020000)),
          lo(lane_off), rs(row_bytes) {}
    __device__ __forceinline__ V ld(int r) const {
        if constexpr (sizeof(V) == 4)
            return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(rsrc, lo, r * rs, 0));
        else
            return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b16(rsrc, lo, r * rs, 0));
    }
    __device__ __forceinline__ void st(int r, const V& v) const {
        if constexpr (sizeof(V) == 4)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsrc, lo, r * rs, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), rsrc, lo, r * rs, 0);
    }
};

// The damped update s + lam (shat - s) as stored (shat itself when
// undamped): one expression for every pass, so that a recomputed iterate
// equals the stored one bit for bit.
template <typename S, bool UND>
__device__ __forceinline__ float damp(float s, float shat, float lam) {
    return stored<S>(UND ? shat : s + lam * (shat - s));
}

// TRACK: also reduce the first step whose residual exceeds tol (the
// advancing window); compiled out otherwise.
template <int MODE, int PHASE, typename S, int NCH, bool UND, bool TRACK = false>
__global__ __launch_bounds__(kThreads) void diag_tanh_pass(DiagArgs g) {
    if constexpr (PHASE != kPrologue && PHASE != kMaps) {
        if (g.ctrl->stop && !g.force) return;    // uniform over the grid: converged earlier
    }
    // which passes start from s0, read the stored iterate, recompute
    // s^(1) .. s^(NR), store nothing
    constexpr bool kFromS0 = PHASE == kFirst || PHASE == kFirstNS;
    constexpr bool kReadS = PHASE == kSteady;
    constexpr int NR = recompute_depth(PHASE);
    constexpr bool kRecompute = NR > 0;
    constexpr bool kNoStore = PHASE == kFirstNS || PHASE == kSecondNS || PHASE == kThirdNS;
    typedef typename Pack<S, NCH>::V V;
    const int cpb = g.cpb;                           // channel groups per block row
    const int dl = threadIdx.x % cpb;
    const int cl = threadIdx.x / cpb;
    // cpb is a multiple of 64, so a wavefront lies in one chunk: c, and with
    // it every row-count test below, is uniform over the wave (scalar)
    const int c = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / cpb) + cl);
    const int d = (blockIdx.y * cpb + dl) * NCH;     // first channel of the group
    // the wave's first channel (every lane is active here) and this lane's
    // byte offset from it: lanes hold consecutive channel groups of one row
    const int dw = __builtin_amdgcn_readfirstlane(d);
    const uint32_t lo = static_cast<uint32_t>(d - dw) * static_cast<uint32_t>(sizeof(S));
    const int b = blockIdx.z;
    uint32_t rb = 0;
    uint32_t fb = 0xffffffffu;                       // first step over tol (TRACK)
    if (c < g.NC && d < g.D) {
        const int D = g.D;
        const int DV = D / NCH;                      // row stride in groups
        const int t0 = c * g.L;
        const int n = min(g.L, g.Tw - t0);          // steps in this chunk
        float a[NCH], s0v[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            a[k] = g.a[d + k];
            s0v[k] = g.s0[b * g.s0s + d + k];
        }
        const V* xp = reinterpret_cast<const V*>(reinterpret_cast<const S*>(g.x) + b * g.xs +
                                                 static_cast<int64_t>(t0) * D + d);
        // rows of x in this chunk: a wave-uniform base plus the lane's offset
        const Rows<V> xr(reinterpret_cast<const S*>(g.x) + b * g.xs + static_cast<int64_t>(t0) * D + dw, lo,
                         D * static_cast<int32_t>(sizeof(S)));
        const size_t ai = (static_cast<size_t>(b) * g.NC + c) * D + d;
        float A[NCH], Bc[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            A[k] = 1.0f;
            Bc[k] = 0.0f;
        }
        if constexpr (PHASE == kPrologue) {
            // Iteration 0: s^(0)_t = s0 for every t, so p_t = s0 throughout.
            // group(j): issue the loads of rows j+kUP.. into xn, then take
            // rows j.. from xb.  FULL: both groups lie inside the chunk, so
            // no row test is compiled in.
            auto group = [&](auto full, int j, const V (&xb)[kUP], V (&xn)[kUP]) {
                constexpr bool F = decltype(full)::value;
#pragma unroll
                for (int u = 0; u < kUP; ++u) xn[u] = (F || j + kUP + u < n) ? xr.ld(j + kUP + u) : V{};
#pragma unroll
                for (int u = 0; u < kUP; ++u) {
                    if (F || j + u < n) {
                        float xt[NCH];
                        unpack<S, NCH>(xb[u], xt);
#pragma unroll
                        for (int k = 0; k < NCH; ++k) {
                            const float v = tanh_f(a[k] * s0v[k] + xt[k]);
                            rb = max(rb, abs_bits(s0v[k] - v));
                            const float at = mode_coef<MODE>(a[k] * (1.0f - v * v));
                            const float bt = v - at * s0v[k];
                            A[k] = at * A[k];
                            Bc[k] = at * Bc[k] + bt;
                        }
                    }
                }
            };
            V x0[kUP], x1[kUP];
#pragma unroll
            for (int u = 0; u < kUP; ++u) x0[u] = u < n ? xr.ld(u) : V{};
            int j = 0;
            // two groups per trip, their buffers alternating (no register copies)
            for (; j + 3 * kUP <= n; j += 2 * kUP) {
                group(std::true_type{}, j, x0, x1);
                group(std::true_type{}, j + kUP, x1, x0);
            }
            for (; j < n; j += kUP) {
                group(std::false_type{}, j, x0, x1);
#pragma unroll
                for (int u = 0; u < kUP; ++u) x0[u] = x1[u];
            }
        } else if constexpr (PHASE == kMaps) {
            // The iterate stored in s (the advancing window, after it slides):
            // its residual, first step over tol, chunk maps and last row.
            const V* sp = reinterpret_cast<const V*>(reinterpret_cast<const S*>(g.s) + b * g.ss +
                                                     static_cast<int64_t>(t0) * D + d);
            float prev[NCH];                         // s_{t-1}
            if (c == 0) {
#pragma unroll
                for (int k = 0; k < NCH; ++k) prev[k] = s0v[k];
            } else {
                unpack<S, NCH>(sp[-DV], prev);
            }
            V xb[kU], sb[kU];
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                xb[u] = u < n ? xp[u * DV] : V{};
                sb[u] = u < n ? sp[u * DV] : V{};
            }
            for (int j = 0; j < n; j += kU) {
                const V* xq = xp + static_cast<int64_t>(j) * DV;
                const V* sq = sp + static_cast<int64_t>(j) * DV;
                V xn[kU], sn_[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const bool in = j + kU + u < n;
                    xn[u] = in ? xq[(kU + u) * DV] : V{};
                    sn_[u] = in ? sq[(kU + u) * DV] : V{};
                }
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    if (j + u < n) {
                        float xt[NCH], st[NCH];
                        unpack<S, NCH>(xb[u], xt);
                        unpack<S, NCH>(sb[u], st);
#pragma unroll
                        for (int k = 0; k < NCH; ++k) {
                            const float v = tanh_f(a[k] * prev[k] + xt[k]);
                            const float dr = st[k] - v;
                            rb = max(rb, abs_bits(dr));
                            if (TRACK && !(fabsf(dr) <= g.tol)) fb = min(fb, static_cast<uint32_t>(t0 + j + u));
                            const float at = mode_coef<MODE>(a[k] * (1.0f - v * v));
                            const float bt = v - at * prev[k];
                            A[k] = at * A[k];
                            Bc[k] = at * Bc[k] + bt;
                            prev[k] = st[k];
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    xb[u] = xn[u];
                    sb[u] = sn_[u];
                }
            }
            // the iterate's last row, for the apply launch that follows
#pragma unroll
            for (int k = 0; k < NCH; ++k) g.halo[(g.iter & 1) * static_cast<size_t>(g.hs) + ai + k] = prev[k];
        } else {
            // halo parity stride, and the index of this chunk in the chunking
            // the carries and the halo were written in (rf fine chunks per
            // chunk of this launch)
            const size_t HS = static_cast<size_t>(g.hs);
            const size_t ri = (static_cast<size_t>(b) * g.NCr + static_cast<size_t>(c) * g.rf) * D + d;
            const bool has_next = (c + 1 < g.NC);
            const float lam = g.lam;
            // p_old: s^(i) at t0-1 (halo of the previous chunk);  shat: s^ at t0-1;
            // snp: s^(i+1) at t0-1, exactly as the previous chunk stores it.
            float p_old[NCH], shat[NCH], shat_end[NCH], snp[NCH];
            // recomputing passes, level l < NR replays iteration l: sh[l] is
            // its s^ entering this chunk (and sh_end[l] the next one), pr[l]
            // holds s^(l)_{t-1} (level 0 has p = s0 throughout)
            constexpr int NRA = NR > 0 ? NR : 1;
            float sh[NRA][NCH], sh_end[NRA][NCH], pr[NRA][NCH];
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                shat[k] = g.carry[ri + k];
                shat_end[k] = has_next ? g.carry[ri + static_cast<size_t>(g.rf) * D + k] : 0.0f;
                float q = s0v[k];       // s^(l)_{t0-1}, from the carries as the previous chunk produced it
#pragma unroll
                for (int l = 0; l < NRA; ++l) {
                    sh[l][k] = sh_end[l][k] = 0.0f;
                    pr[l][k] = q;
                    if (l < NR) {
                        sh[l][k] = g.carryr[l][ri + k];
                        sh_end[l][k] = has_next ? g.carryr[l][ri + static_cast<size_t>(g.rf) * D + k] : 0.0f;
                        q = c == 0 ? s0v[k] : damp<S, UND>(q, sh[l][k], lam);
                    }
                }
                if constexpr (kRecompute) p_old[k] = q;
                else p_old[k] = (kFromS0 || c == 0) ? s0v[k] : g.halo[(g.iter & 1) * HS + ri - D + k];
                snp[k] = damp<S, UND>(p_old[k], shat[k], lam);
            }
            // float passes that read only x prefetch as deep as the prologue
            // (binary16 sweeps are bound by their vector instructions)
            constexpr int U = (kReadS || !std::is_same<S, float>::value) ? kU : kUP;
            // rows of the iterate in this chunk (read in kSteady, written
            // except by the passes that store nothing), addressed like xr
            const Rows<V> sr(reinterpret_cast<const S*>(g.s) + b * g.ss + static_cast<int64_t>(t0) * D + dw, lo,
                             xr.rs);
            // group(j): issue the loads of rows j+U.. into xn/sn_, then take
            // rows j.. from xb/sb.  FULL: both groups lie inside the chunk
            // and hold neither its last step nor rows past it, so no row
            // test is compiled in.
            auto group = [&](auto full, int j, const V (&xb)[U], const V (&sb)[U], V (&xn)[U], V (&sn_)[U]) {
                constexpr bool F = decltype(full)::value;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool in = F || j + U + u < n;
                    xn[u] = in ? xr.ld(j + U + u) : V{};
                    if constexpr (kReadS) sn_[u] = in ? sr.ld(j + U + u) : V{};
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (F || j + u < n) {
                        // the chunk's last step takes the value the scan hands to the next chunk
                        const bool last = !F && j + u == n - 1 && has_next;
                        float xt[NCH], so[NCH], sn[NCH];
                        unpack<S, NCH>(xb[u], xt);
                        if constexpr (kFromS0) {
#pragma unroll
                            for (int k = 0; k < NCH; ++k) so[k] = s0v[k];
                        } else if constexpr (kRecompute) {
                            // s^(1)_t .. s^(NR)_t again: iteration l's replay at
                            // p = s^(l)_{t-1} (s0 for l = 0) gives s^(l+1)_t
#pragma unroll
                            for (int k = 0; k < NCH; ++k) {
                                float cur = s0v[k];          // s^(l)_t
#pragma unroll
                                for (int l = 0; l < NR; ++l) {
                                    const float p = l == 0 ? s0v[k] : pr[l][k];
                                    const float vl = tanh_f(a[k] * p + xt[k]);
                                    const float al = mode_coef<MODE>(a[k] * (1.0f - vl * vl));
                                    sh[l][k] = vl + al * (sh[l][k] - p);
                                    if (last) sh[l][k] = sh_end[l][k];
                                    const float nxt = damp<S, UND>(cur, sh[l][k], lam);
                                    pr[l][k] = cur;
                                    cur = nxt;
                                }
                                so[k] = cur;
                            }
                        } else {
                            unpack<S, NCH>(sb[u], so);
                        }
#pragma unroll
                        for (int k = 0; k < NCH; ++k) {
                            // iteration i: map at p_t = s^(i)_{t-1}
                            const float v = tanh_f(a[k] * p_old[k] + xt[k]);
                            const float at = mode_coef<MODE>(a[k] * (1.0f - v * v));
                            shat[k] = v + at * (shat[k] - p_old[k]);
                            if (last) shat[k] = shat_end[k];
                            sn[k] = damp<S, UND>(so[k], shat[k], lam);
                        }
                        if constexpr (kNoStore) {
#pragma unroll
                            for (int k = 0; k < NCH; ++k) sn[k] = stored<S>(sn[k]);
                        } else {
                            sr.st(j + u, pack<S, NCH>(sn));   // sn now holds the stored values
                        }
#pragma unroll
                        for (int k = 0; k < NCH; ++k) {
                            // iteration i+1: residual and affine map at p_t = s^(i+1)_{t-1}
                            const float v2 = tanh_f(a[k] * snp[k] + xt[k]);
                            rb = max(rb, abs_bits(sn[k] - v2));
                            if (TRACK && !(fabsf(sn[k] - v2) <= g.tol))
                                fb = min(fb, static_cast<uint32_t>(t0 + j + u));
                            const float a2 = mode_coef<MODE>(a[k] * (1.0f - v2 * v2));
                            const float b2 = v2 - a2 * snp[k];
                            A[k] = a2 * A[k];
                            Bc[k] = a2 * Bc[k] + b2;
                            p_old[k] = so[k];
                            snp[k] = sn[k];
                        }
                    }
                }
            };
            V x0[U], s0b[U], x1[U], s1b[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                x0[u] = u < n ? xr.ld(u) : V{};
                s0b[u] = s1b[u] = V{};
                if constexpr (kReadS) s0b[u] = u < n ? sr.ld(u) : V{};
            }
            int j = 0;
            // two groups per trip, their buffers alternating (no register
            // copies); the rows they take end U rows before the chunk does
            for (; j + 3 * U <= n; j += 2 * U) {
                group(std::true_type{}, j, x0, s0b, x1, s1b);
                group(std::true_type{}, j + U, x1, s1b, x0, s0b);
            }
            for (; j < n; j += U) {
                group(std::false_type{}, j, x0, s0b, x1, s1b);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    x0[u] = x1[u];
                    s0b[u] = s1b[u];
                }
            }
#pragma unroll
            for (int k = 0; k < NCH; ++k) g.halo[((g.iter + 1) & 1) * HS + ai + k] = snp[k];
        }
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            g.aggA[ai + k] = A[k];
            g.aggB[ai + k] = Bc[k];
        }
    }
    rb = block_max_u32(rb);
    const int bid = (blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    if (threadIdx.x == 0) g.rpart[bid] = rb;
    if constexpr (TRACK) {
        fb = ~block_max_u32(~fb);
        if (threadIdx.x == 0) g.fpart[bid] = fb;
    }
}

// Channel groups of a row: pairs for binary16 storage with even D.
static int diag_groups(const DiagArgs& a) { return a.half == 2 ? a.D / 2 : a.D; }

static dim3 diag_grid(const DiagArgs& a) {
    const int cpg = kThreads / a.cpb;
    return dim3((a.NC + cpg - 1) / cpg, (diag_groups(a) + a.cpb - 1) / a.cpb, a.B);
}

int diag_tanh_nblocks(const DiagArgs& a) {
    const dim3 g = diag_grid(a);
    return static_cast<int>(g.x * g.y * g.z);
}

template <int MODE, typename S, int NCH, bool UND>
static hipError_t launch_und(int phase, const DiagArgs& a, hipStream_t st) {
    const dim3 grid = diag_grid(a);
    if (phase == kPrologue) diag_tanh_pass<MODE, kPrologue, S, NCH, UND><<<grid, kThreads, 0, st>>>(a);
    else if (phase == kFirst) diag_tanh_pass<MODE, kFirst, S, NCH, UND><<<grid, kThreads, 0, st>>>(a);
    else if (phase == kSteady && !a.fpart)
        return launch_maybe_timed(diag_tanh_pass<MODE, kSteady, S, NCH, UND>, grid, dim3(kThreads), 0, st, a);
    else if constexpr (std::is_same<S, float>::value) {
        // the advancing window and the recomputing pair run with float storage only
        if (phase == kSteady)
            return launch_maybe_timed(diag_tanh_pass<MODE, kSteady, S, NCH, UND, true>, grid, dim3(kThreads), 0, st, a);
        else if (phase == kMaps) diag_tanh_pass<MODE, kMaps, S, NCH, UND, true><<<grid, kThreads, 0, st>>>(a);
        else if (phase == kFirstNS) diag_tanh_pass<MODE, kFirstNS, S, NCH, UND><<<grid, kThreads, 0, st>>>(a);
        else if (phase == kSecondR) diag_tanh_pass<MODE, kSecondR, S, NCH, UND><<<grid, kThreads, 0, st>>>(a);
        else if (phase == kSecondNS) diag_tanh_pass<MODE, kSecondNS, S, NCH, UND><<<grid, kThreads, 0, st>>>(a);
        else if (phase == kThirdR) diag_tanh_pass<MODE, kThirdR, S, NCH, UND><<<grid, kThreads, 0, st>>>(a);
        else if (phase == kThirdNS) diag_tanh_pass<MODE, kThirdNS, S, NCH, UND><<<grid, kThreads, 0, st>>>(a);
        else if (phase == kFourthR) diag_tanh_pass<MODE, kFourthR, S, NCH, UND><<<grid, kThreads, 0, st>>>(a);
        else return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// undamped (lam = 1) stores s^ itself: its own instantiation drops the damping
template <int MODE, typename S, int NCH>
static hipError_t launch_mode(int phase, const DiagArgs& a, hipStream_t st) {
    return a.undamped ? launch_und<MODE, S, NCH, true>(phase, a, st)
                      : launch_und<MODE, S, NCH, false>(phase, a, st);
}

template <typename S, int NCH>
static hipError_t launch_store(int phase, const DiagArgs& a, hipStream_t st) {
    switch (a.mode) {
        case kJacobi: return launch_mode<kJacobi, S, NCH>(phase, a, st);
        case kPicard: return launch_mode<kPicard, S, NCH>(phase, a, st);
        default: return launch_mode<kQuasiNewton, S, NCH>(phase, a, st);   // Newton == QN here
    }
}

// a.half: 0 float storage, 1 binary16 one channel per thread, 2 binary16 pairs
hipError_t launch_diag_tanh_pass(int phase, const DiagArgs& a, hipStream_t st) {
    if (a.half == 2) return launch_store<_Float16, 2>(phase, a, st);
    if (a.half == 1) return launch_store<_Float16, 1>(phase, a, st);
    return launch_store<float, 1>(phase, a, st);
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
    // With the check, one more column of workgroups: its first one takes the
    // check beside the carries instead of before a share of them.
    if (g.do_check && blockIdx.x == gridDim.x - 1) {
        if (blockIdx.y == 0) run_check(g.chk);
        return;
    }
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
    const dim3 grid((a.D + kChan - 1) / kChan + (a.do_check ? 1 : 0), a.B);
    diag_carry_kernel<<<grid, kSeg * kChan, 0, st>>>(a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- fill
// out[b][t][:] = s0[b][:] for a window (result when no update was applied).
template <typename S>
__global__ __launch_bounds__(kThreads) void fill_kernel(S* out, int64_t ss, const float* s0,
                                                         int64_t s0s, int Tw, int D) {
    const int b = blockIdx.y;
    const int64_t n = static_cast<int64_t>(Tw) * D;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        out[b * ss + e] = static_cast<S>(s0[b * s0s + (e % D)]);
    }
}

hipError_t launch_fill(float* out, int64_t ss, const float* s0, int64_t s0s, int B, int Tw, int D,
                       hipStream_t st) {
    if (B == 0 || Tw == 0 || D == 0) return hipSuccess;
    const int64_t n = static_cast<int64_t>(Tw) * D;
    const int gx = static_cast<int>(std::min<int64_t>((n + kThreads - 1) / kThreads, 4096));
    fill_kernel<float><<<dim3(gx, B), kThreads, 0, st>>>(out, ss, s0, s0s, Tw, D);
    return hipGetLastError();
}

hipError_t launch_fill_half(void* out, int64_t ss, const float* s0, int64_t s0s, int B, int Tw, int D,
                            hipStream_t st) {
    if (B == 0 || Tw == 0 || D == 0) return hipSuccess;
    const int64_t n = static_cast<int64_t>(Tw) * D;
    const int gx = static_cast<int>(std::min<int64_t>((n + kThreads - 1) / kThreads, 4096));
    fill_kernel<_Float16><<<dim3(gx, B), kThreads, 0, st>>>(static_cast<_Float16*>(out), ss, s0, s0s, Tw, D);
    return hipGetLastError();
}

}  // namespace pn
