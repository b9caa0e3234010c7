// C interface and host-side iteration driver of libpn.
//
// One call = one stream.  For every window the driver launches
//   prologue                      maps of iteration 0 (at s^(0) = s0) + r_0
//   repeat i = 0, 1, ...:
//     carry(i)   scan of the chunk maps; block 0 first reduces the residual
//                of the previous pass and takes the stop decision for i,
//                publishing it on the device and in pinned host memory
//     apply(i)   fused update s^(i) -> s^(i+1) (exits at once if stopped)
// The host reads the decision of carry(i) while apply(i) runs, so the GPU is
// never idle waiting for the host; after the stop, one apply launch exits
// immediately.  Matrix cells in the diagonal modes with few chunks per
// window skip the carry launch: each apply sweep takes its own check and
// composes its carries (CellArgs::fc), and the host keeps two sweeps queued.
// Stop rule and counting follow include/pn.h.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/pn.h"
#include "pn_internal.hpp"

namespace {

using namespace pn;

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

#define PN_HIP(call)                                                                    \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess)                                                           \
            return fail(PN_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));        \
    } while (0)

constexpr size_t kAlign = 256;
constexpr int32_t kSmallMaxIter = 1 << 14;   // updates per window the one-workgroup solver takes on
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// ---------------------------------------------------------------- planning
struct Plan {
    int kind, mode, D, m, B;
    int band;              // half-bandwidth of A~_t in the dense modes (Newton: D)
    int64_t T, W;          // horizon, window length
    int L, NC;             // chunk length, chunks of a full window
    int Lc, NCc;           // the steady updates' chunks (recompute: twice L), else L, NC
    int DP, cpb;           // padded D (matrix cells), channels per block (diag cell)
    bool dense, matrix_cell, mfma;
    bool advancing;        // one window sliding past its converged prefix
    bool half;             // x and out in IEEE binary16 (channel-wise cell)
    int hmode;             // DiagArgs::half of the channel-wise kernel
    bool persist_ok;       // shape allows the one-launch persistent solver
    bool small;            // the window fits one workgroup: every window, iteration and
                           // check in one launch (pn_small.hip)
    bool resident_ok;      // shape has the one-launch resident form (cell_resident), used
                           // when all B x NC chunks fit on the device at once
    bool adv_resident_ok;  // advancing window with a one-launch resident form
                           // (cell_resident_adv), used when its chunks fit at once
    bool recompute;        // channel-wise cell, float storage: the first kRecomputeDepth
                           // updates store nothing, the next recomputes s^(1) .. s^(i)
                           // (kFirstNS, kSecondNS, kThirdNS, kFourthR)
    int fc;                // matrix cell, diagonal mode, few chunks (CellArgs::fc): the apply
                           // sweeps compose their own carries (kFcCarry) and, with
                           // consecutive windows, take their own check (kFcCheck)
    int nblocks, nwin, hist_cap;
    size_t off_ctrl, off_rpart, off_fpart, off_aggA, off_aggB, off_carry, off_carryr, off_halo, off_w,
        total;
    size_t off_sync, off_winfo, off_hist, off_acc, off_info_end;
    size_t off_lag;        // resident solver: residual words, ready words, window-state words
};

void layout(Plan& p, const Plan* other);

// The channel-wise cell with float storage: updates 1 .. kRecomputeDepth read
// only x and store nothing, and update kRecomputeDepth + 1 recomputes the
// iterates s^(1) .. s^(kRecomputeDepth) from the carries of their iterations
// before its own replay; kNoStorePass[l] and kStorePass[l] are the passes of
// update l + 1 that recompute l iterates.
constexpr int kRecomputeDepth = 3;
constexpr int kNoStorePass[3] = {kFirstNS, kSecondNS, kThirdNS};
constexpr int kStorePass[4] = {kFirst, kSecondR, kThirdR, kFourthR};

int make_plan(Plan& p, const pn_cell* cell, int64_t B, int64_t T, int64_t D, int32_t mode,
              const pn_opts* o, bool half = false) {
    p.kind = cell->kind;
    p.half = half;
    p.hmode = 0;
    p.D = static_cast<int>(D);
    p.m = cell->input_dim;
    p.matrix_cell = p.kind != PN_CELL_DIAG_TANH;
    // band_0(A) = diag(A) and band_{D-1}(A) = A; a diagonal Jacobian is its
    // own band
    const int k = o ? o->bandwidth : 1;
    if (mode == PN_BANDED) {
        if (!p.matrix_cell || k == 0) mode = PN_QUASI_NEWTON;
        else if (k >= p.D - 1) mode = PN_NEWTON;
    }
    p.mode = mode;
    p.band = mode == PN_BANDED ? k : p.D;
    p.B = static_cast<int>(B);
    p.T = T;
    const int64_t window = o ? o->window : 0;
    p.W = (window <= 0 || window > T) ? T : window;
    p.advancing = o && o->window_mode == PN_WINDOW_ADVANCING;
    const int chunk = o ? o->chunk : 0;
    p.dense = p.matrix_cell && (mode == PN_NEWTON || mode == PN_BANDED);
    p.mfma = false;
    p.fc = 0;
    if (!p.matrix_cell) {
        // binary16 storage moves two adjacent channels per thread when D is even
        p.hmode = !half ? 0 : (p.D % 2 == 0 ? 2 : 1);
        const int groups = p.hmode == 2 ? p.D / 2 : p.D;
        // channel groups per workgroup row: 64, 128 or 256, a divisor of the
        // workgroup size, so every thread belongs to exactly one (chunk, group)
        p.cpb = groups <= 64 ? 64 : groups <= 128 ? 128 : 256;
        const bool recompute = !p.half && !p.advancing;
        if (chunk > 0) {
            p.L = p.Lc = chunk;
        } else {
            // Longest chunk that still leaves about 2^18 threads (B x channel
            // groups x chunks): the per-iteration carry scan shrinks with the
            // chunk count, while the sweeps that read only x (and the
            // binary16 sweeps, bound by their vector instructions) want the
            // occupancy.  With float storage the steady updates (two row
            // streams in, one out per thread) run on chunks twice as long:
            // fewer, longer streams measured faster.
            int64_t L = 16;
            while (L < 1024 && static_cast<int64_t>(B) * groups * ((p.W + 2 * L - 1) / (2 * L)) >= (1 << 18)) L *= 2;
            p.L = static_cast<int>(L);
            p.Lc = static_cast<int>(recompute ? std::min<int64_t>(2 * L, 1024) : L);
        }
        // the sweeps address a chunk's rows with 32-bit buffer offsets (row
        // index x row bytes): keep a chunk's rows within 2^30 bytes
        const int64_t maxL = std::max<int64_t>(1, (int64_t{1} << 30) / (static_cast<int64_t>(D) * (half ? 2 : 4)));
        p.L = static_cast<int>(std::min<int64_t>(std::min<int64_t>(p.L, p.W), maxL));
        p.Lc = static_cast<int>(std::min<int64_t>(std::min<int64_t>(std::max(p.Lc, p.L), p.W), maxL));
        if (p.Lc % p.L != 0) p.Lc = p.L;    // steady chunks are whole multiples of the first ones
        p.NC = static_cast<int>((p.W + p.L - 1) / p.L);
        DiagArgs a{};
        a.B = p.B; a.D = p.D; a.NC = p.NC; a.cpb = p.cpb; a.half = p.hmode;
        p.nblocks = diag_tanh_nblocks(a);
        p.DP = 0;
    } else if (p.dense && (next_pow2(p.D) == 16 || next_pow2(p.D) == 32 || next_pow2(p.D) == 64) &&
               dense_mfma_supported(p.kind, next_pow2(p.D), p.m)) {
        // Newton on the matrix cores: one wavefront per chunk (two when the
        // chunks are few); chunks long enough to keep the serial carry
        // short, with ~2048 chunks in flight (about two wavefronts per
        // SIMD), and shorter ones (down to 16 steps) while fewer than 1024
        // chunks would leave SIMDs idle: each launch then takes about the
        // time of one chunk's serial steps.
        p.mfma = true;
        p.DP = next_pow2(p.D);
        int64_t L = 64;
        if (chunk > 0) {
            L = chunk;
        } else {
            while (L < 512 && static_cast<int64_t>(B) * ((p.W + 2 * L - 1) / (2 * L)) >= 2048) L *= 2;
            while (L > 16 && static_cast<int64_t>(B) * ((p.W + L - 1) / L) < 1024) L /= 2;
            // the one-wavefront sweep at D padded to 16 holds four wavefronts
            // per SIMD: halve the chunks once more while that still fits
            // the 4096 wavefronts of one residency round
            if (p.DP == 16 && L > 16 && static_cast<int64_t>(B) * ((p.W + L - 1) / L) > kSplitMax &&
                static_cast<int64_t>(B) * ((p.W + L / 2 - 1) / (L / 2)) <= 4096)
                L /= 2;
        }
        p.L = p.Lc = static_cast<int>(std::min<int64_t>(L, p.W));
        p.NC = static_cast<int>((p.W + p.L - 1) / p.L);
        p.nblocks = p.NC * p.B;
        // the apply sweeps take their own check, so the carry launches need
        // not, and the sweeps are enqueued ahead of the host's reads
        if (!p.advancing && p.DP <= 32) p.fc = kFcCheck;
    } else {
        p.DP = std::max(4, next_pow2(p.D));
        const int Lmax = 64;
        int L = Lmax;
        if (chunk > 0) {
            L = std::min(chunk, Lmax);
        } else {
            // prefer a chunk whose arrays and staged weights fit the LDS budget
            while (L > 4 && !cell_pass_stages_weights(p.kind, p.DP, p.dense, L, p.m)) L /= 2;
            if (!cell_pass_stages_weights(p.kind, p.DP, p.dense, L, p.m)) {
                L = Lmax;   // weights stay in global memory
                while (L > 4 && cell_pass_lds_bytes(p.kind, p.DP, p.dense, L, p.m) > 64 * 1024) L /= 2;
            }
            while (L > 16 && static_cast<int64_t>(B) * ((p.W + L - 1) / L) < 1024) L /= 2;
        }
        p.L = p.Lc = static_cast<int>(std::min<int64_t>(L, p.W));
        p.NC = static_cast<int>((p.W + p.L - 1) / p.L);
        p.nblocks = p.NC * p.B;
        // with few chunks per row, composing a chunk's carry in its own sweep
        // costs less than a carry launch; past kFcMaxBlocks workgroups their
        // residual atomics would contend on the 16 slots, while a carry
        // launch costs little next to such a sweep
        if (!p.dense && p.NC <= kFcMaxChunks && static_cast<int64_t>(p.B) * p.NC <= kFcMaxBlocks)
            p.fc = p.advancing ? kFcCarry : (kFcCarry | kFcCheck);
        if (cell_pass_lds_bytes(p.kind, p.DP, p.dense, p.L, p.m) > 160 * 1024)
            return fail(PN_EUNSUPPORTED, "chunk of %d steps needs too much LDS for D=%d, m=%d", p.L, p.D, p.m);
    }
    p.nwin = static_cast<int>((T + p.W - 1) / p.W);
    p.recompute = !p.matrix_cell && !p.half && !p.advancing;
    if (!p.recompute) p.Lc = p.L;
    p.NCc = static_cast<int>((p.W + p.Lc - 1) / p.Lc);
    p.persist_ok = p.matrix_cell && !p.dense && !p.advancing &&
                   cell_persist_eligible(p.kind, p.DP, p.L, p.m);
    // A window of at most a few hundred (b, t) pairs of a narrow matrix cell
    // is latency, not work: one workgroup runs the whole solve.  An explicit
    // chunk or PN_FLAG_MULTI_LAUNCH keeps the multi-launch driver.
    p.small = p.matrix_cell && !half && !p.advancing && chunk == 0 &&
              !(o && (o->flags & PN_FLAG_MULTI_LAUNCH)) && p.D <= 8 &&
              static_cast<int64_t>(p.B) * p.W <= small_max_pairs_for(p.D);
    p.resident_ok = p.matrix_cell && !p.dense && !half && !p.advancing && (p.fc & kFcCheck) &&
                    p.DP % 16 == 0 && !p.small;
    p.adv_resident_ok = p.matrix_cell && p.advancing && !p.dense && !half && p.DP % 16 == 0 && p.DP <= 64;
    p.hist_cap = static_cast<int>(std::min<int64_t>(static_cast<int64_t>(p.nwin) * (p.W + 1), 1 << 16));
    layout(p, nullptr);
    return PN_OK;
}

// Workspace offsets of a plan; with `other`, every shared region is sized for
// both plans (a solve that switches modes runs both on one workspace).
void layout(Plan& p, const Plan* other) {
    size_t nparts = p.nblocks;
    size_t bnd = static_cast<size_t>(p.B) * p.NC * p.D;
    size_t nA = bnd * (p.dense ? p.D : 1);
    if (other) {
        const size_t ob = static_cast<size_t>(other->B) * other->NC * other->D;
        nparts = std::max<size_t>(nparts, other->nblocks);
        nA = std::max(nA, ob * (other->dense ? other->D : 1));
        bnd = std::max(bnd, ob);
    }
    size_t off = 0;
    p.off_ctrl = off; off = align_up(off + sizeof(Ctrl));
    p.off_rpart = off; off = align_up(off + sizeof(uint32_t) * nparts);
    p.off_fpart = off; off = align_up(off + sizeof(uint32_t) * nparts);
    // chunk maps: two sets (iterations of either parity) for fc sweeps
    // chunk maps: three sets for the resident solver (by publication), two
    // (by iteration parity) for sweeps that compose their own carries
    const size_t nsets = p.resident_ok ? 3
                         : ((p.fc & kFcCarry) || p.adv_resident_ok || (other && (other->fc & kFcCarry))) ? 2 : 1;
    p.off_aggA = off; off = align_up(off + sizeof(float) * nA * nsets);
    p.off_aggB = off; off = align_up(off + sizeof(float) * bnd * nsets);
    p.off_carry = off; off = align_up(off + sizeof(float) * bnd);
    p.off_carryr = off;     // the carries of iterations 0 .. kRecomputeDepth - 1
    if (p.recompute || (other && other->recompute)) off = align_up(off + sizeof(float) * bnd * kRecomputeDepth);
    p.off_halo = off; off = align_up(off + sizeof(float) * (p.resident_ok ? 3 : 2) * bnd);
    p.off_w = off;
    if (p.matrix_cell) off = align_up(off + sizeof(float) * prepared_total_floats(p.kind, p.DP, p.m));
    p.off_lag = off;
    if (p.resident_ok) {
        const size_t chunks = static_cast<size_t>(p.B) * p.NC;
        off = align_up(off + sizeof(unsigned long long) * 4 * chunks + sizeof(unsigned) * (chunks + p.B));
    }
    p.off_sync = p.off_winfo = p.off_hist = p.off_acc = off;
    if (p.persist_ok || p.small || p.resident_ok || p.adv_resident_ok) {
        p.off_sync = off; off = align_up(off + 256);
        p.off_winfo = off; off = align_up(off + sizeof(int32_t) * 2 * p.nwin);
        p.off_hist = off; off = align_up(off + sizeof(float) * p.hist_cap);
        p.off_acc = off;
        if (p.adv_resident_ok) off = align_up(off + sizeof(int32_t) * p.hist_cap);
    }
    p.off_info_end = off;
    p.total = off;
}

// The plan of the first mode and, when the options ask for residual-driven
// switching, the plan of the second, laid out on one workspace.
int make_plans(Plan& p, Plan& p2, bool* has2, const pn_cell* cell, int64_t B, int64_t T, int64_t D,
               int32_t mode, const pn_opts* o) {
    int rc = make_plan(p, cell, B, T, D, mode, o);
    if (rc != PN_OK) return rc;
    *has2 = o && o->switch_mode >= 0;
    if (!*has2) return PN_OK;
    rc = make_plan(p2, cell, B, T, D, o->switch_mode, o);
    if (rc != PN_OK) return rc;
    p.persist_ok = p2.persist_ok = false;
    p.small = p2.small = false;
    p.resident_ok = p2.resident_ok = false;
    p.adv_resident_ok = p2.adv_resident_ok = false;
    p.recompute = p2.recompute = false;
    p.fc = p2.fc = 0;
    p.Lc = p.L; p2.Lc = p2.L;
    p.NCc = p.NC; p2.NCc = p2.NC;
    layout(p, &p2);
    layout(p2, &p);
    return PN_OK;
}

// Number of floats in the flat parameter vector of a cell (layouts in pn.h).
int64_t param_floats(int kind, int64_t D, int64_t m) {
    switch (kind) {
        case PN_CELL_DIAG_TANH: return D;
        case PN_CELL_TANH_RNN: return D * D + D * m + D;
        case PN_CELL_GRU: return 3 * D * m + 3 * D * D + 6 * D;
        default: return D * D + D * m + 2 * D;   // PN_CELL_EULER_TANH
    }
}

// [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + static_cast<uint64_t>(nb) && pb < pa + static_cast<uint64_t>(na);
}

// es: bytes per element of x and out (4 float, 2 binary16); 0 skips the
// aliasing check (sizing calls pass placeholder pointers).
int validate(const pn_cell* cell, const float* params, const float* x, const float* s0, int64_t B,
             int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter, const float* out,
             const int32_t* iters_out, const pn_opts* o, int es = 4) {
    if (!cell) return fail(PN_EINVAL, "cell is NULL");
    if (!iters_out) return fail(PN_EINVAL, "iters_out is NULL");
    if (B < 0 || T < 0 || D < 0) return fail(PN_EINVAL, "negative size (B=%lld T=%lld D=%lld)",
                                             (long long)B, (long long)T, (long long)D);
    if (cell->kind < PN_CELL_DIAG_TANH || cell->kind > PN_CELL_EULER_TANH)
        return fail(PN_EINVAL, "unknown cell kind %d", cell->kind);
    if (mode < PN_JACOBI || mode > PN_BANDED) return fail(PN_EINVAL, "unknown mode %d", mode);
    if (mode == PN_BANDED && o && o->bandwidth < 0) return fail(PN_EINVAL, "bandwidth must be >= 0");
    if (cell->input_dim < 1) return fail(PN_EINVAL, "input_dim must be >= 1");
    if (cell->kind == PN_CELL_DIAG_TANH && cell->input_dim != D && D > 0)
        return fail(PN_EINVAL, "diag-tanh cell needs input_dim == D");
    if (!(tol >= 0.0f) || std::isinf(tol)) return fail(PN_EINVAL, "tol must be finite and >= 0");
    if (max_iter < 0) return fail(PN_EINVAL, "max_iter must be >= 0");
    if (o) {
        if (!(o->damping > 0.0f && o->damping <= 1.0f)) return fail(PN_EINVAL, "damping must lie in (0, 1]");
        if (o->window < 0) return fail(PN_EINVAL, "window must be >= 0");
        if (o->chunk < 0 || o->chunk > (1 << 20)) return fail(PN_EINVAL, "chunk out of range");
        if (o->resid_hist_len < 0 || o->window_iters_len < 0) return fail(PN_EINVAL, "negative history length");
        if (o->resid_hist_len > 0 && !o->resid_hist) return fail(PN_EINVAL, "resid_hist is NULL");
        if (o->window_iters_len > 0 && !o->window_iters) return fail(PN_EINVAL, "window_iters is NULL");
        if (o->accepted_len < 0 || (o->accepted_len > 0 && !o->accepted))
            return fail(PN_EINVAL, "accepted is NULL or its length negative");
        if (o->workspace && (reinterpret_cast<uintptr_t>(o->workspace) % kAlign) != 0)
            return fail(PN_EWORKSPACE, "workspace must be 256-byte aligned");
        if (o->window_mode != PN_WINDOW_CONSECUTIVE && o->window_mode != PN_WINDOW_ADVANCING)
            return fail(PN_EINVAL, "unknown window_mode %d", o->window_mode);
        if (o->switch_mode < -1 || o->switch_mode > PN_BANDED)
            return fail(PN_EINVAL, "unknown switch_mode %d", o->switch_mode);
        if (o->switch_mode >= 0) {
            if (!(o->switch_ratio >= 0.0f)) return fail(PN_EINVAL, "switch_ratio must be >= 0");
            if (o->switch_mode == PN_BANDED && o->bandwidth < 0)
                return fail(PN_EINVAL, "bandwidth must be >= 0");
            if (!(o->switch_damping == 0.0f || (o->switch_damping > 0.0f && o->switch_damping <= 1.0f)))
                return fail(PN_EINVAL, "switch_damping must be 0 or lie in (0, 1]");
            if (o->window_mode == PN_WINDOW_ADVANCING)
                return fail(PN_EUNSUPPORTED, "mode switching and the advancing window do not combine");
        }
        if (o->window_switch_len < 0 || (o->window_switch_len > 0 && !o->window_switch))
            return fail(PN_EINVAL, "window_switch is NULL or its length negative");
        if (o->profile_stride < 0) return fail(PN_EINVAL, "profile_stride must be >= 0");
    }
    if (B == 0 || T == 0 || D == 0) return PN_OK;
    if (!params || !x || !s0 || !out) return fail(PN_EINVAL, "a device pointer is NULL");
    if (cell->kind != PN_CELL_DIAG_TANH && D > 64)
        return fail(PN_EUNSUPPORTED, "matrix cells support D <= 64 (got %lld)", (long long)D);
    if (B > 65535) return fail(PN_EUNSUPPORTED, "B must be <= 65535");
    if (T >= (int64_t(1) << 31) || D >= (int64_t(1) << 24) || cell->input_dim >= (1 << 24))
        return fail(PN_EUNSUPPORTED, "size too large");
    if (es > 0) {
        // out is written while the inputs are still read: it must not share
        // a byte with any of them
        const int64_t nout = B * T * D * es;
        if (overlaps(out, nout, x, B * T * cell->input_dim * es))
            return fail(PN_EINVAL, "out overlaps x");
        if (overlaps(out, nout, s0, B * D * 4)) return fail(PN_EINVAL, "out overlaps s0");
        if (overlaps(out, nout, params, param_floats(cell->kind, D, cell->input_dim) * 4))
            return fail(PN_EINVAL, "out overlaps params");
    }
    return PN_OK;
}

// ---------------------------------------------------------------- per-thread resources
struct ThreadRes {
    int device = -1;
    HostRec* host = nullptr;     // pinned (or, with dev_ring, a plain host shadow)
    HostRec* host_dev = nullptr; // device-usable alias (or, with dev_ring, device memory)
    bool dev_ring = false;       // records live in device memory: copy each back to read it
    int32_t epoch = 0;           // per-thread call counter
    std::vector<hipEvent_t> timing;   // pool of timing events
    // pinned (mapped) buffer the one-workgroup solver writes its per-window
    // counts and residual history to; grown on demand
    char* small_host = nullptr;
    char* small_dev = nullptr;
    size_t small_cap = 0;
};
thread_local ThreadRes g_res;

// A pinned buffer of at least `bytes` for the one-workgroup solver's results
// (the previous call has completed: every call ends with a stream sync).
int small_info_buffer(ThreadRes* r, size_t bytes, char** host, char** dev) {
    if (r->small_cap < bytes) {
        if (r->small_host) PN_HIP(hipHostFree(r->small_host));
        r->small_host = r->small_dev = nullptr;
        r->small_cap = 0;
        const size_t cap = std::max<size_t>(bytes, 4096);
        void* p = nullptr;
        PN_HIP(hipHostMalloc(&p, cap, hipHostMallocMapped | hipHostMallocCoherent));
        r->small_host = static_cast<char*>(p);
        r->small_cap = cap;
    }
    void* dp = nullptr;
    PN_HIP(hipHostGetDevicePointer(&dp, r->small_host, 0));
    r->small_dev = static_cast<char*>(dp);
    *host = r->small_host;
    *dev = r->small_dev;
    return PN_OK;
}

// pn_eval_noalloc: the record ring at the start of the static scratch, and
// the epochs of its calls (unique across threads, so a stale record of an
// earlier call never matches)
constexpr size_t kStaticRingBytes = 256;
static_assert(sizeof(HostRec) * kHostRing <= kStaticRingBytes, "record ring");
std::atomic<int32_t> g_static_epoch{1};

int get_res(ThreadRes** out) {
    int dev = 0;
    PN_HIP(hipGetDevice(&dev));
    ThreadRes& r = g_res;
    if (r.device != dev) {
        if (!r.host) {
            void* p = nullptr;
            PN_HIP(hipHostMalloc(&p, sizeof(HostRec) * kHostRing, hipHostMallocMapped | hipHostMallocCoherent));
            r.host = static_cast<HostRec*>(p);
        }
        void* dp = nullptr;
        PN_HIP(hipHostGetDevicePointer(&dp, r.host, 0));
        r.host_dev = static_cast<HostRec*>(dp);
        for (auto e : r.timing) (void)hipEventDestroy(e);
        r.timing.clear();
        r.device = dev;
    }
    *out = &r;
    return PN_OK;
}

thread_local LaunchTiming g_launch_timing;

int timing_event(ThreadRes* r, size_t idx, hipEvent_t* ev) {
    while (r->timing.size() <= idx) {
        hipEvent_t e;
        PN_HIP(hipEventCreate(&e));
        r->timing.push_back(e);
    }
    *ev = r->timing[idx];
    return PN_OK;
}

// Wait until the check of iteration `iter` (call `epoch`) has published its
// record in pinned host memory.  Polls the record; every few thousand polls
// asks the runtime whether the stream failed or drained without writing it.
int wait_record(const ThreadRes* res, volatile HostRec* hr, hipStream_t st, int32_t epoch, int32_t iter) {
    if (res->dev_ring) {
        // records in device memory: the stream holds the check that writes
        // this one; drain it and copy the record into the host shadow
        HostRec* shadow = const_cast<HostRec*>(hr);
        const HostRec* src = res->host_dev + (shadow - res->host);
        PN_HIP(hipMemcpyAsync(shadow, src, sizeof(HostRec), hipMemcpyDeviceToHost, st));
        PN_HIP(hipStreamSynchronize(st));
        if (hr->iter == iter && hr->epoch == epoch) return PN_OK;
        return fail(PN_EHIP, "stream drained without publishing iteration %d", iter);
    }
    using clk = std::chrono::steady_clock;
    const auto t0 = clk::now();
    for (uint64_t n = 1;; ++n) {
        if (hr->iter == iter && hr->epoch == epoch) {
            std::atomic_thread_fence(std::memory_order_acquire);
            return PN_OK;
        }
        if ((n & 4095) == 0) {
            const hipError_t q = hipStreamQuery(st);
            if (q != hipSuccess && q != hipErrorNotReady)
                return fail(PN_EHIP, "stream failed while solving: %s", hipGetErrorString(q));
            if (q == hipSuccess && !(hr->iter == iter && hr->epoch == epoch))
                return fail(PN_EHIP, "stream drained without publishing iteration %d", iter);
            if (clk::now() - t0 > std::chrono::seconds(600))
                return fail(PN_EHIP, "timed out waiting for iteration %d", iter);
        }
    }
}

// ---------------------------------------------------------------- the solve
struct Timing {
    bool on = false;
    int stride = 1;          // time every stride-th steady apply launch
    int64_t seen = 0;
    std::vector<std::pair<size_t, size_t>> apply;   // event index pairs
    std::vector<double> apply_bytes, apply_flops;
    size_t next = 0;
    bool take() { return on && (seen++ % stride) == 0; }
};

struct SolveCtx {
    const Plan* p;
    hipStream_t st;
    char* ws;
    ThreadRes* res;
    const float* params;
    float tol, lam;
    int32_t max_iter;
    Timing* tm;
    std::vector<float>* hist;
    float ratio;             // switch_ratio (residual-driven switching)
    float lam2;              // switch_damping: damping after a switch (0: keep lam)
};

double apply_bytes(const Plan& p, int Tw, bool first) {
    // algorithmic bytes of one apply launch: read x, read s^(i) (not for
    // i = 0, where s^(0) = s0 is implicit), write s^(i+1)
    const double rows = static_cast<double>(p.B) * Tw;
    return rows * (p.half ? 2.0 : 4.0) * (p.m + (first ? 1 : 2) * p.D);
}

double apply_flops(const Plan& p, int Tw) {
    // algorithmic flops of one apply launch per (b, t): two cell evaluations
    // (recurrent products 2*NG*D^2 each) and one input projection (2*NG*D*m);
    // Newton adds one D x D chunk-map compose (2 D^3) and two matrix-vector
    // chains through the Jacobian (2*NG*D^2 each); the banded mode does the
    // same with nz (mean entries per row of the band) in place of one D
    if (!p.matrix_cell) return 0.0;
    const double D = p.D, m = p.m, NG = p.kind == PN_CELL_GRU ? 3.0 : 1.0;
    double per = 2.0 * (2.0 * NG * D * D) + 2.0 * NG * D * m;
    if (p.dense) {
        double nz = 0.0;
        for (int i = 0; i < p.D; ++i) nz += std::min(p.D - 1, i + p.band) - std::max(0, i - p.band) + 1;
        nz /= D;
        per += 2.0 * D * D * nz + 2.0 * (2.0 * NG * D * nz);
    }
    return static_cast<double>(p.B) * Tw * per;
}

// Timing of the next steady apply launch: two events that the launch
// records with its own dispatch (launch_maybe_timed).  After the launch,
// check_timed_launch confirms the launch took the request.
int request_timing(SolveCtx& c, size_t* i0, size_t* i1) {
    hipEvent_t e0, e1;
    int rc = timing_event(c.res, c.tm->next, &e0);
    if (rc != PN_OK) return rc;
    rc = timing_event(c.res, c.tm->next + 1, &e1);
    if (rc != PN_OK) return rc;
    *i0 = c.tm->next;
    *i1 = c.tm->next + 1;
    c.tm->next += 2;
    g_launch_timing = LaunchTiming{e0, e1};
    return PN_OK;
}

int check_timed_launch() {
    if (g_launch_timing.start) {
        g_launch_timing = LaunchTiming{};
        return fail(PN_EHIP, "a timed launch did not record its events");
    }
    return PN_OK;
}

int record(SolveCtx& c, size_t* idx) {
    hipEvent_t e;
    int rc = timing_event(c.res, c.tm->next, &e);
    if (rc != PN_OK) return rc;
    PN_HIP(hipEventRecord(e, c.st));
    *idx = c.tm->next++;
    return PN_OK;
}

// Solve one window.  Writes *K (updates) and *status.  With p2 (residual-
// driven switching [PN §5.3]), the window starts on plan p and, at the first
// check i >= 1 with r_i > ratio * r_{i-1}, moves to p2 from update i+1 on
// (apply(i) is already enqueued): the chunk maps of p2's mode are rebuilt at
// s^(i+1) by a maps pass (unless p2 has the same mode, whose maps apply(i)
// built), the damping becomes lam2 when that is set, and the loop continues
// on p2.  *sw receives that check, or -1.
int solve_window(SolveCtx& c, const float* x, int64_t xs, float* s, int64_t ss, const float* s0,
                 int64_t s0s, int Tw, int* K, int* status, const Plan* p2, int* sw) {
    const Plan* pp = c.p;
    Ctrl* ctrl = reinterpret_cast<Ctrl*>(c.ws + pp->off_ctrl);
    uint32_t* rpart = reinterpret_cast<uint32_t*>(c.ws + pp->off_rpart);
    float* aggA = reinterpret_cast<float*>(c.ws + pp->off_aggA);
    float* aggB = reinterpret_cast<float*>(c.ws + pp->off_aggB);
    float* carry = reinterpret_cast<float*>(c.ws + pp->off_carry);
    // carries of iterations 0 .. kRecomputeDepth - 1 (recomputing passes)
    float* carryr[kRecomputeDepth];
    for (int l = 0; l < kRecomputeDepth; ++l)
        carryr[l] = reinterpret_cast<float*>(c.ws + pp->off_carryr) +
                    static_cast<size_t>(l) * pp->B * pp->NC * pp->D;
    float* halo = reinterpret_cast<float*>(c.ws + pp->off_halo);
    const float* w = reinterpret_cast<const float*>(c.ws + pp->off_w);
    uint32_t* fpart = reinterpret_cast<uint32_t*>(c.ws + pp->off_fpart);
    float lam = c.lam;       // step damping of the updates still to be enqueued
    // the first kRecomputeDepth + 1 updates of the channel-wise cell move
    // less: the carries of iterations 0 .. kRecomputeDepth - 1 go to buffers
    // of their own
    const bool recompute = pp->recompute && !p2;
    constexpr int RD = kRecomputeDepth;

    DiagArgs da{};
    CellArgs ca{};
    CarryArgs cy{};
    cy.aggA = aggA; cy.aggB = aggB; cy.carry = carry; cy.s0 = s0; cy.s0s = s0s;
    cy.B = pp->B; cy.D = pp->D; cy.do_check = 1;
    cy.chk.rpart = rpart; cy.chk.max_iter = c.max_iter; cy.chk.tol = c.tol;
    cy.chk.ctrl = ctrl; cy.chk.host = c.res->host_dev;
    // kernel arguments of the plan in use
    auto configure = [&](const Plan& p) {
        const int NC = (Tw + p.L - 1) / p.L;
        int nblocks;
        if (!p.matrix_cell) {
            da = DiagArgs{};
            da.a = c.params; da.x = x; da.xs = xs; da.s = s; da.ss = ss; da.s0 = s0; da.s0s = s0s;
            da.B = p.B; da.Tw = Tw; da.D = p.D; da.L = p.L; da.NC = NC; da.cpb = p.cpb;
            da.aggA = aggA; da.aggB = aggB; da.carry = carry; da.halo = halo;
            for (int l = 0; l < RD; ++l) da.carryr[l] = carryr[l];
            da.rpart = rpart;
            da.ctrl = ctrl; da.mode = p.mode; da.lam = lam; da.undamped = lam == 1.0f;
            da.half = p.hmode;
            da.rf = 1; da.NCr = NC;
            da.hs = static_cast<int64_t>(p.B) * p.NC * p.D;
            nblocks = diag_tanh_nblocks(da);
        } else {
            ca = CellArgs{};
            ca.w = w; ca.x = x; ca.xs = xs; ca.s = s; ca.ss = ss; ca.s0 = s0; ca.s0s = s0s;
            ca.B = p.B; ca.Tw = Tw; ca.D = p.D; ca.m = p.m; ca.L = p.L; ca.NC = NC;
            ca.aggA = aggA; ca.aggB = aggB; ca.carry = carry; ca.halo = halo; ca.rpart = rpart;
            ca.ctrl = ctrl; ca.mode = p.mode; ca.lam = lam; ca.undamped = lam == 1.0f;
            ca.band = p.band;
            ca.fc = p.fc;
            if (p.fc) {
                ca.max_iter = c.max_iter; ca.tol = c.tol; ca.host = c.res->host_dev;
                ca.mstride = static_cast<int64_t>(p.B) * p.NC * p.D;
            }
            nblocks = cell_pass_nblocks(ca);
        }
        cy.NC = NC;
        cy.chk.nparts = nblocks;
    };
    auto launch_pass = [&](int phase, int iter) -> hipError_t {
        if (!pp->matrix_cell) {
            da.iter = iter;
            return launch_diag_tanh_pass(phase, da, c.st);
        }
        ca.iter = iter;
        if (pp->mfma) return launch_dense_mfma_pass(pp->kind, pp->DP, phase, ca, c.st);
        return launch_cell_pass(pp->kind, pp->DP, pp->dense, phase, ca, c.st);
    };

    configure(*pp);
    // sweeps that take their own check leave the carry launches only the
    // carries; a carry launch queued after the stop does nothing
    if (pp->fc & kFcCheck) {
        cy.do_check = 0;
        cy.stop_on = ctrl;
    }
    *sw = -1;
    // fc sweeps reduce r_0 into ctrl->rmax[0] and expect rmax[1] clear
    if (pp->fc & kFcCheck) PN_HIP(hipMemsetAsync(ctrl, 0, sizeof(Ctrl), c.st));
    PN_HIP(launch_pass(kPrologue, 0));
    volatile HostRec* ring = c.res->host;      // check i goes to ring[i % kHostRing]
    const int32_t epoch = ++c.res->epoch;
    cy.chk.epoch = epoch;
    ca.epoch = epoch;
    for (int k = 0; k < kHostRing; ++k) ring[k].iter = -1;
    float r_prev = 0.0f;
    // Chunking of the channel-wise launches with the recomputing passes: the
    // prologue and updates 1 to RD + 1 run on chunks of L, the later updates
    // on chunks of Lc (a multiple of L); the first of them reads the carries
    // and the halo of the fine chunking at chunk c * Lc / L.
    const int NCf = (Tw + pp->L - 1) / pp->L;
    const int NCc = (Tw + pp->Lc - 1) / pp->Lc;
    auto grain = [&](bool coarse, int rf) {
        da.L = coarse ? pp->Lc : pp->L;
        da.NC = coarse ? NCc : NCf;
        da.rf = rf;
        da.NCr = rf > 1 ? NCf : da.NC;
    };
    // Apply launch k (update k).  Sweeps that take their own check (fc) are
    // kept `ahead` launches in front of the check the host is reading: a
    // sweep after the stop finds the control word set and exits at once.
    // (one when the check is published at the start of the sweep, as in the
    // sweeps that keep their carry launches: the host reads it while the
    // sweep runs)
    const int ahead = (pp->fc & kFcCheck) ? ((pp->fc & kFcCarry) ? 2 : 1) : 0;
    std::vector<int> tslot;      // launch k -> its timing entry, or -1
    auto enqueue_apply = [&](int k) -> int {
        // recomputing: updates 1 .. RD store nothing, update RD + 1
        // recomputes s^(1) .. s^(RD) and stores s^(RD + 1)
        const int phase = !recompute ? (k == 0 ? kFirst : kSteady)
                          : k < RD   ? kNoStorePass[k]
                          : k == RD  ? kStorePass[RD]
                                     : kSteady;
        if (recompute) grain(k >= RD + 1, k == RD + 1 ? pp->Lc / pp->L : 1);
        // timing covers the steady-state apply launches, including the
        // final ones that exit at once
        if ((pp->fc & kFcCheck) && !(pp->fc & kFcCarry))
            // the carries of iteration k's maps (a launch after the stop exits at once)
            PN_HIP(pp->dense ? launch_dense_carry(cy, c.st) : launch_diag_carry(cy, c.st));
        const bool timed = phase == kSteady && c.tm->take();
        size_t e0 = 0, e1 = 0;
        if (timed) { int rc = request_timing(c, &e0, &e1); if (rc) return rc; }
        PN_HIP(launch_pass(phase, k));
        tslot.push_back(-1);
        if (timed) {
            int rc = check_timed_launch();
            if (rc) return rc;
            c.tm->apply.push_back({e0, e1});
            c.tm->apply_bytes.push_back(0.0);   // filled in once the check says it ran
            c.tm->apply_flops.push_back(0.0);
            tslot.back() = static_cast<int>(c.tm->apply.size()) - 1;
        }
        return PN_OK;
    };
    for (int k = 0; k < ahead; ++k) {
        int rc = enqueue_apply(k);
        if (rc != PN_OK) return rc;
    }
    for (int i = 0;; ++i) {
        volatile HostRec* hr = ring + i % kHostRing;
        cy.chk.iter = i;
        cy.chk.host = c.res->host_dev + i % kHostRing;
        cy.carry = (recompute && i < RD) ? carryr[i] : carry;
        da.carry = cy.carry;
        if (recompute) {
            // the carry scans the maps of the launch before: apply(i-1), or the prologue
            grain(i >= RD + 2, 1);
            cy.NC = da.NC;
            cy.chk.nparts = diag_tanh_nblocks(da);
        }
        if (!(pp->fc & kFcCheck)) {
            // the check of iteration i and the carries of its maps, then update i
            PN_HIP(pp->dense ? launch_dense_carry(cy, c.st) : launch_diag_carry(cy, c.st));
            int rc = enqueue_apply(i);
            if (rc != PN_OK) return rc;
        }
        {
            int rc = wait_record(c.res, hr, c.st, epoch, i);
            if (rc != PN_OK) return rc;
        }
        const int stop = hr->stop;
        const int st = hr->status;
        const uint32_t rb = hr->r_bits;
        const int it = hr->iter;
        if (it != i) return fail(PN_EHIP, "control record out of sequence (%d vs %d)", it, i);
        float r;
        std::memcpy(&r, &rb, sizeof(r));
        if (c.hist) c.hist->push_back(r);
        if (!stop && tslot[i] >= 0) {
            // update i ran
            c.tm->apply_bytes[tslot[i]] = apply_bytes(*pp, Tw, false);
            c.tm->apply_flops[tslot[i]] = apply_flops(*pp, Tw);
        }
        if (stop) {
            *K = i;
            *status = st;
            if (recompute && i >= 1 && i <= RD) {
                // the result is s^(i), which update i did not store: update i
                // again, the form that stores (its iteration is i - 1)
                grain(false, 1);
                da.carry = carryr[i - 1];
                da.force = 1;
                PN_HIP(launch_pass(kStorePass[i - 1], i - 1));
                da.force = 0;
            }
            break;
        }
        if (p2 && *sw < 0 && i >= 1 && r > c.ratio * r_prev) {
            // stagnation: update i runs on the first mode; from i+1 on, p2
            *sw = i;
            const bool new_maps = p2->mode != pp->mode;
            pp = p2;
            if (c.lam2 > 0.0f) lam = c.lam2;
            configure(*pp);
            if (new_maps) {
                // the channel-wise maps pass also reduces the first step over
                // tol, which nothing reads here
                da.fpart = fpart;
                da.tol = c.tol;
                PN_HIP(launch_pass(kMaps, i + 1));
                da.fpart = nullptr;
            }
        }
        r_prev = r;
        if (pp->fc & kFcCheck) {
            int rc = enqueue_apply(i + ahead);
            if (rc != PN_OK) return rc;
        }
    }
    if (*K == 0) {
        if (c.p->half) PN_HIP(launch_fill_half(s, ss, s0, s0s, c.p->B, Tw, c.p->D, c.st));
        else PN_HIP(launch_fill(s, ss, s0, s0s, c.p->B, Tw, c.p->D, c.st));
    }
    return PN_OK;
}

// The advancing window [PN §1.3.1] (matrix cells).  Steps [0, a) are
// accepted; the window is [a, e), e = min(T, a + W).  Each round: the device
// reduces the residual of the current iterate on the window and the first
// step over tol (a check launch), the host reads that record, accepts the
// prefix and slides the window (new steps start from its last state), then
// enqueues the chunk maps of the moved window, the carry scan and one apply
// sweep, whose fused residual feeds the next check.  The host waits once per
// round: the next window depends on the check.
int solve_advancing(SolveCtx& c, const float* x, const float* s0, float* out, int64_t T, int* K,
                    int* status, std::vector<int32_t>* accepted) {
    const Plan& p = *c.p;
    const int64_t D = p.D, m = p.m, W = p.W;
    Ctrl* ctrl = reinterpret_cast<Ctrl*>(c.ws + p.off_ctrl);
    uint32_t* rpart = reinterpret_cast<uint32_t*>(c.ws + p.off_rpart);
    uint32_t* fpart = reinterpret_cast<uint32_t*>(c.ws + p.off_fpart);
    float* aggA = reinterpret_cast<float*>(c.ws + p.off_aggA);
    float* aggB = reinterpret_cast<float*>(c.ws + p.off_aggB);
    float* carry = reinterpret_cast<float*>(c.ws + p.off_carry);
    float* halo = reinterpret_cast<float*>(c.ws + p.off_halo);

    CellArgs ca{};
    ca.w = reinterpret_cast<const float*>(c.ws + p.off_w);
    ca.xs = T * m; ca.ss = T * D;
    ca.B = p.B; ca.D = p.D; ca.m = p.m; ca.L = p.L;
    ca.aggA = aggA; ca.aggB = aggB; ca.carry = carry; ca.halo = halo; ca.rpart = rpart;
    ca.ctrl = ctrl; ca.mode = p.mode; ca.lam = c.lam; ca.undamped = c.lam == 1.0f;
    ca.band = p.band; ca.fpart = fpart; ca.tol = c.tol;
    ca.fc = p.fc;                    // kFcCarry or 0: the check stays a launch of its own
    // two sets of chunk maps only with kFcCarry (one set, read by the carry
    // launch, otherwise)
    ca.mstride = p.fc ? static_cast<int64_t>(p.B) * p.NC * p.D : 0;
    DiagArgs da{};                   // the channel-wise cell (m == D, float storage)
    da.a = c.params; da.xs = T * m; da.ss = T * D;
    da.B = p.B; da.D = p.D; da.L = p.L; da.cpb = p.cpb;
    da.aggA = aggA; da.aggB = aggB; da.carry = carry; da.halo = halo; da.rpart = rpart;
    da.ctrl = ctrl; da.mode = p.mode; da.lam = c.lam; da.undamped = c.lam == 1.0f;
    da.half = 0; da.rf = 1;
    da.hs = static_cast<int64_t>(p.B) * p.NC * p.D;
    da.fpart = fpart; da.tol = c.tol;
    CarryArgs cy{};
    cy.aggA = aggA; cy.aggB = aggB; cy.carry = carry; cy.B = p.B; cy.D = p.D; cy.do_check = 0;
    CheckArgs chk{};
    chk.rpart = rpart; chk.fpart = fpart; chk.advancing = 1; chk.max_iter = c.max_iter;
    chk.tol = c.tol; chk.ctrl = ctrl; chk.host = c.res->host_dev;
    volatile HostRec* hr = c.res->host;
    const int32_t epoch = ++c.res->epoch;
    chk.epoch = epoch;
    hr->iter = -1;

    int64_t a = 0, e = std::min<int64_t>(T, W);
    int Tw = 0;
    auto set_window = [&]() {
        Tw = static_cast<int>(e - a);
        const int NC = (Tw + p.L - 1) / p.L;
        ca.x = x + a * m;
        ca.s = out + a * D;
        ca.s0 = a == 0 ? s0 : out + (a - 1) * D;
        ca.s0s = a == 0 ? D : T * D;
        ca.Tw = Tw;
        ca.NC = NC;
        cy.s0 = ca.s0; cy.s0s = ca.s0s; cy.NC = NC;
        chk.nparts = p.B * NC;
        if (!p.matrix_cell) {
            da.x = ca.x; da.s = ca.s; da.s0 = ca.s0; da.s0s = ca.s0s;
            da.Tw = Tw; da.NC = NC; da.NCr = NC;
            chk.nparts = diag_tanh_nblocks(da);
        }
    };
    auto launch_pass = [&](int phase, int iter) -> hipError_t {
        if (!p.matrix_cell) {
            da.iter = iter;
            return launch_diag_tanh_pass(phase, da, c.st);
        }
        ca.iter = iter;
        if (p.mfma) return launch_dense_mfma_pass(p.kind, p.DP, phase, ca, c.st);
        return launch_cell_pass(p.kind, p.DP, p.dense, phase, ca, c.st);
    };

    // the initial iterate s0 on the first window, its maps and its check
    PN_HIP(launch_fill(out, T * D, s0, D, p.B, static_cast<int>(e), p.D, c.st));
    set_window();
    PN_HIP(launch_pass(kMaps, 0));
    chk.iter = 0;
    PN_HIP(launch_check(chk, c.st));
    int64_t ma = a, me = e;          // the window the chunk maps on the device belong to
    for (int i = 0;;) {
        {
            int rc = wait_record(c.res, hr, c.st, epoch, i);
            if (rc != PN_OK) return rc;
        }
        const uint32_t rb = hr->r_bits;
        const uint32_t first = hr->first;
        float r;
        std::memcpy(&r, &rb, sizeof(r));
        if (c.hist) c.hist->push_back(r);
        if (rb >= kNonFiniteBits) { *K = i; *status = PN_NONFINITE; break; }
        const int64_t acc = std::min<int64_t>(first, e - a);
        accepted->push_back(static_cast<int32_t>(acc));
        a += acc;
        if (a >= T) { *K = i; *status = PN_OK; break; }
        if (i == c.max_iter) { *K = i; *status = PN_NOT_CONVERGED; break; }
        const int64_t e_new = std::min<int64_t>(T, a + W);
        // steps entering the window start from its last state: the maps pass
        // of the matrix cells' kernels writes them itself
        const bool tile_fill = p.matrix_cell;
        if (e_new > e && !tile_fill)
            PN_HIP(launch_fill(out + e * D, T * D, out + (e - 1) * D, T * D, p.B,
                               static_cast<int>(e_new - e), p.D, c.st));
        const int fill_rows = tile_fill ? static_cast<int>(e_new - e) : 0;
        e = e_new;
        set_window();
        if (a != ma || e != me) {
            ca.fill_rows = fill_rows;
            PN_HIP(launch_pass(kMaps, i));
            ca.fill_rows = 0;
            ma = a;
            me = e;
        }
        if (!(p.fc & kFcCarry)) PN_HIP(p.dense ? launch_dense_carry(cy, c.st) : launch_diag_carry(cy, c.st));
        size_t e0 = 0, e1 = 0;
        const bool timed = c.tm->take();
        if (timed) { int rc = request_timing(c, &e0, &e1); if (rc) return rc; }
        PN_HIP(launch_pass(kSteady, i));
        if (timed) {
            int rc = check_timed_launch();
            if (rc) return rc;
            c.tm->apply.push_back({e0, e1});
            c.tm->apply_bytes.push_back(apply_bytes(p, Tw, false));
            c.tm->apply_flops.push_back(apply_flops(p, Tw));
        }
        ++i;
        chk.iter = i;
        PN_HIP(launch_check(chk, c.st));
    }
    if (e < T)
        PN_HIP(launch_fill(out + e * D, T * D, out + (e - 1) * D, T * D, p.B, static_cast<int>(T - e),
                           p.D, c.st));
    return PN_OK;
}

// The whole solve as one cooperative launch (matrix cells, diagonal modes).
// Returns PN_EUNSUPPORTED (no launch made) when the device cannot run it, so
// the caller falls back to the multi-launch driver.
int solve_persistent(SolveCtx& c, const float* x, const float* s0, float* out, int64_t T,
                     std::vector<int>* wit, int* total, int* overall) {
    const Plan& p = *c.p;
    int dev = 0, coop = 0;
    PN_HIP(hipGetDevice(&dev));
    PN_HIP(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
    if (!coop) return PN_EUNSUPPORTED;
    int nb_max = 0;
    PN_HIP(cell_persist_max_blocks(p.kind, p.DP, p.L, p.m, &nb_max));
    if (nb_max < 1) return PN_EUNSUPPORTED;
    const int nblocks = static_cast<int>(std::min<int64_t>(nb_max, static_cast<int64_t>(p.B) * p.NC));
    char* ws = c.ws;
    unsigned* bar = reinterpret_cast<unsigned*>(ws + p.off_sync);
    int32_t* winfo = reinterpret_cast<int32_t*>(ws + p.off_winfo);
    PN_HIP(hipMemsetAsync(ws + p.off_sync, 0, 256, c.st));
    PN_HIP(hipMemsetAsync(winfo, 0xff, sizeof(int32_t) * 2 * p.nwin, c.st));
    PersistArgs a{};
    CellArgs& g = a.g;
    g.w = reinterpret_cast<const float*>(ws + p.off_w);
    g.xs = T * p.m;
    g.ss = T * p.D;
    g.B = p.B; g.D = p.D; g.m = p.m; g.L = p.L;
    g.aggA = reinterpret_cast<float*>(ws + p.off_aggA);
    g.aggB = reinterpret_cast<float*>(ws + p.off_aggB);
    g.carry = reinterpret_cast<float*>(ws + p.off_carry);
    g.halo = reinterpret_cast<float*>(ws + p.off_halo);
    g.rpart = reinterpret_cast<uint32_t*>(ws + p.off_rpart);
    g.ctrl = nullptr;
    g.mode = p.mode; g.lam = c.lam; g.undamped = c.lam == 1.0f;
    a.x0 = x; a.s_base = out; a.s0_user = s0;
    a.T = T; a.W = static_cast<int32_t>(p.W); a.nwin = p.nwin;
    a.tol = c.tol; a.max_iter = c.max_iter;
    a.bar = bar; a.err = bar + 1;
    a.hist_len = reinterpret_cast<int32_t*>(bar + 2);
    a.win_iters = winfo; a.win_status = winfo + p.nwin;
    a.hist = reinterpret_cast<float*>(ws + p.off_hist);
    a.hist_cap = p.hist_cap;
    size_t e0 = 0, e1 = 0;
    if (c.tm->on) { int rc = record(c, &e0); if (rc) return rc; }
    {
        const hipError_t le = launch_cell_persist(p.kind, p.DP, nblocks, a, c.st);
        if (le == hipErrorCooperativeLaunchTooLarge) {
            (void)hipGetLastError();
            return PN_EUNSUPPORTED;
        }
        if (le != hipSuccess) return fail(PN_EHIP, "cooperative launch failed: %s", hipGetErrorString(le));
    }
    if (c.tm->on) { int rc = record(c, &e1); if (rc) return rc; }
    PN_HIP(hipStreamSynchronize(c.st));
    std::vector<int32_t> info(64 + 2 * p.nwin);
    PN_HIP(hipMemcpy(info.data(), bar, 256, hipMemcpyDeviceToHost));
    PN_HIP(hipMemcpy(info.data() + 64, winfo, sizeof(int32_t) * 2 * p.nwin, hipMemcpyDeviceToHost));
    if (info[1] != 0) return fail(PN_EHIP, "grid barrier of the persistent solver timed out");
    const int hlen = std::min(info[2], p.hist_cap);
    if (c.hist && hlen > 0) {
        c.hist->resize(hlen);
        PN_HIP(hipMemcpy(c.hist->data(), a.hist, sizeof(float) * hlen, hipMemcpyDeviceToHost));
    }
    *total = 0;
    *overall = PN_OK;
    double bytes = 0.0, flops = 0.0;
    for (int w = 0; w < p.nwin; ++w) {
        const int K = info[64 + w], st = info[64 + p.nwin + w];
        if (K < 0) break;
        const int Tw = static_cast<int>(std::min<int64_t>(p.W, T - static_cast<int64_t>(w) * p.W));
        wit->push_back(K);
        *total += K;
        if (K > 0) bytes += apply_bytes(p, Tw, true) + (K - 1) * apply_bytes(p, Tw, false);
        flops += K * apply_flops(p, Tw);
        if (st == PN_NONFINITE) { *overall = PN_NONFINITE; break; }
        if (st == PN_NOT_CONVERGED) *overall = PN_NOT_CONVERGED;
    }
    if (c.tm->on) {
        c.tm->apply.push_back({e0, e1});
        c.tm->apply_bytes.push_back(bytes);
        c.tm->apply_flops.push_back(flops);
    }
    return PN_OK;
}

// Where a solve's device memory and check records come from when the caller
// brings neither a workspace nor a pinned record ring: the library's static
// device scratch (pn_eval_noalloc).  Records then live in device memory and
// the host reads each one back with a copy after synchronising the stream.
struct Backing {
    char* ws;                // 256-byte aligned device memory for the plan's regions
    size_t bytes;
    ThreadRes* res;          // dev_ring set, host = a host shadow array
};

// Where a one-launch solver writes its per-window counts, statuses and
// residual history ([hist_len | win_iters, win_status | history | accepted
// steps], laid out as the workspace region off_sync .. off_info_end): straight to pinned
// host memory, or, for pn_eval_noalloc (records in device memory), to the
// workspace, copied back once after the launch.
struct OneLaunchInfo {
    size_t nbytes = 0;
    char* dev = nullptr;
    const char* host = nullptr;
    std::vector<char> copy;
};

int one_launch_info(SolveCtx& c, OneLaunchInfo* inf) {
    const Plan& p = *c.p;
    inf->nbytes = p.off_info_end - p.off_sync;
    inf->dev = c.ws + p.off_sync;
    if (!c.res->dev_ring) {
        char* h = nullptr;
        int rc = small_info_buffer(c.res, inf->nbytes, &h, &inf->dev);
        if (rc != PN_OK) return rc;
        inf->host = h;
    }
    return PN_OK;
}

// After the launch: bring the results to the host and fill counts, statuses,
// history and the profile entry of the launch.
int one_launch_results(SolveCtx& c, OneLaunchInfo* inf, int64_t T, std::vector<int>* wit, int* total,
                       int* overall, bool timed, size_t e0, size_t e1) {
    const Plan& p = *c.p;
    if (c.res->dev_ring) {
        inf->copy.resize(inf->nbytes);
        PN_HIP(hipMemcpyAsync(inf->copy.data(), inf->dev, inf->nbytes, hipMemcpyDeviceToHost, c.st));
        inf->host = inf->copy.data();
    }
    PN_HIP(hipStreamSynchronize(c.st));
    int32_t hlen = 0;
    std::memcpy(&hlen, inf->host, sizeof(hlen));
    const int32_t* wi = reinterpret_cast<const int32_t*>(inf->host + (p.off_winfo - p.off_sync));
    const float* hist = reinterpret_cast<const float*>(inf->host + (p.off_hist - p.off_sync));
    if (c.hist) c.hist->assign(hist, hist + std::min(hlen, p.hist_cap));
    *total = 0;
    *overall = PN_OK;
    double bytes = 0.0, flops = 0.0;
    for (int w = 0; w < p.nwin; ++w) {
        const int K = wi[w], st = wi[p.nwin + w];
        if (K < 0) break;
        const int Tw = static_cast<int>(std::min<int64_t>(p.W, T - static_cast<int64_t>(w) * p.W));
        wit->push_back(K);
        *total += K;
        if (K > 0) bytes += apply_bytes(p, Tw, true) + (K - 1) * apply_bytes(p, Tw, false);
        flops += K * apply_flops(p, Tw);
        if (st == PN_NONFINITE) { *overall = PN_NONFINITE; break; }
        if (st == PN_NOT_CONVERGED) *overall = PN_NOT_CONVERGED;
    }
    if (timed) {
        c.tm->apply.push_back({e0, e1});
        c.tm->apply_bytes.push_back(bytes);
        c.tm->apply_flops.push_back(flops);
    }
    return PN_OK;
}

// The whole solve in one launch of the one-workgroup solver.
int solve_small(SolveCtx& c, const float* x, const float* s0, float* out, int64_t T,
                std::vector<int>* wit, int* total, int* overall) {
    const Plan& p = *c.p;
    OneLaunchInfo inf;
    int rc = one_launch_info(c, &inf);
    if (rc != PN_OK) return rc;
    SmallArgs a{};
    a.params = c.params; a.x = x; a.s0 = s0; a.out = out; a.T = T;
    a.W = static_cast<int32_t>(p.W); a.nwin = p.nwin; a.B = p.B; a.D = p.D; a.m = p.m;
    a.mode = p.mode; a.band = p.band; a.max_iter = c.max_iter;
    a.undamped = c.lam == 1.0f; a.tol = c.tol; a.lam = c.lam;
    a.hist_len = reinterpret_cast<int32_t*>(inf.dev);
    a.win_iters = reinterpret_cast<int32_t*>(inf.dev + (p.off_winfo - p.off_sync));
    a.win_status = a.win_iters + p.nwin;
    a.hist = reinterpret_cast<float*>(inf.dev + (p.off_hist - p.off_sync));
    a.hist_cap = p.hist_cap;
    const bool timed = c.tm->take();
    size_t e0 = 0, e1 = 0;
    if (timed) { rc = request_timing(c, &e0, &e1); if (rc) return rc; }
    PN_HIP(launch_small_solve(p.kind, p.dense, a, c.st));
    if (timed) { rc = check_timed_launch(); if (rc) return rc; }
    return one_launch_results(c, &inf, T, wit, total, overall, timed, e0, e1);
}

// The whole solve as one cooperative launch of the resident solver.  Returns
// PN_EUNSUPPORTED (nothing launched) when the chunks do not all fit on the
// device at once.
int solve_resident(SolveCtx& c, const float* x, const float* s0, float* out, int64_t T,
                   std::vector<int>* wit, int* total, int* overall) {
    const Plan& p = *c.p;
    int dev = 0, coop = 0, nb = 0;
    PN_HIP(hipGetDevice(&dev));
    PN_HIP(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
    if (!coop) return PN_EUNSUPPORTED;
    // one chunk per workgroup, else (D padded to 16) four strided chunks per workgroup
    int cpw = 1;
    PN_HIP(cell_resident_max_blocks(p.kind, p.DP, p.L, p.m, 1, &nb));
    if (static_cast<int64_t>(p.B) * p.NC > nb) {
        cpw = 4;
        nb = 0;
        if (p.DP == 16) PN_HIP(cell_resident_max_blocks(p.kind, p.DP, p.L, p.m, cpw, &nb));
        if (static_cast<int64_t>(p.B) * ((p.NC + cpw - 1) / cpw) > nb) return PN_EUNSUPPORTED;
    }
    OneLaunchInfo inf;
    int rc = one_launch_info(c, &inf);
    if (rc != PN_OK) return rc;
    char* ws = c.ws;
    ResidentArgs a{};
    a.w = reinterpret_cast<const float*>(ws + p.off_w);
    a.x = x; a.out = out; a.s0 = s0; a.T = T;
    a.W = static_cast<int32_t>(p.W); a.nwin = p.nwin; a.B = p.B; a.D = p.D; a.m = p.m; a.L = p.L;
    a.NC = p.NC; a.mode = p.mode; a.undamped = c.lam == 1.0f; a.max_iter = c.max_iter;
    a.lam = c.lam; a.tol = c.tol;
    a.mapA = reinterpret_cast<float*>(ws + p.off_aggA);
    a.mapB = reinterpret_cast<float*>(ws + p.off_aggB);
    a.halo = reinterpret_cast<float*>(ws + p.off_halo);
    a.s0n = reinterpret_cast<float*>(ws + p.off_carry);
    Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + p.off_ctrl);
    a.err = &ctrl->bar_err;
    const size_t chunks = static_cast<size_t>(p.B) * p.NC;
    a.rword = reinterpret_cast<unsigned long long*>(ws + p.off_lag);
    a.ready = reinterpret_cast<unsigned*>(a.rword + 4 * chunks);
    a.s0ready = a.ready + chunks;
    a.hist_len = reinterpret_cast<int32_t*>(inf.dev);
    a.win_iters = reinterpret_cast<int32_t*>(inf.dev + (p.off_winfo - p.off_sync));
    a.win_status = a.win_iters + p.nwin;
    a.hist = reinterpret_cast<float*>(inf.dev + (p.off_hist - p.off_sync));
    a.hist_cap = p.hist_cap;
    // error flag, residual words, ready words and window-state words start at zero
    PN_HIP(hipMemsetAsync(ctrl, 0, sizeof(Ctrl), c.st));
    PN_HIP(hipMemsetAsync(a.rword, 0, sizeof(unsigned long long) * 4 * chunks + sizeof(unsigned) * (chunks + p.B),
                          c.st));
    const bool timed = c.tm->take();
    size_t e0 = 0, e1 = 0;
    if (timed) { rc = request_timing(c, &e0, &e1); if (rc) return rc; }
    {
        const hipError_t le = launch_cell_resident(p.kind, p.DP, cpw, a, c.st);
        if (le == hipErrorCooperativeLaunchTooLarge) {
            (void)hipGetLastError();
            g_launch_timing = LaunchTiming{};
            return PN_EUNSUPPORTED;
        }
        if (le != hipSuccess) return fail(PN_EHIP, "cooperative launch failed: %s", hipGetErrorString(le));
    }
    if (timed) { rc = check_timed_launch(); if (rc) return rc; }
    rc = one_launch_results(c, &inf, T, wit, total, overall, timed, e0, e1);
    if (rc != PN_OK) return rc;
    unsigned err = 0;
    PN_HIP(hipMemcpy(&err, a.err, sizeof(err), hipMemcpyDeviceToHost));
    if (err != 0) return fail(PN_EHIP, "grid barrier of the resident solver timed out");
    return PN_OK;
}

// The advancing window as one cooperative launch of cell_resident_adv: the
// shortest chunk (from the plan's on) whose B x ceil(W / L) workgroups are
// co-resident.  Returns PN_EUNSUPPORTED (nothing launched) when none fits.
int solve_advancing_resident(SolveCtx& c, const float* x, const float* s0, float* out, int64_t T, int* K,
                             int* status, std::vector<int32_t>* accepted) {
    const Plan& p = *c.p;
    int dev = 0, coop = 0;
    PN_HIP(hipGetDevice(&dev));
    PN_HIP(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
    if (!coop) return PN_EUNSUPPORTED;
    int L = 0, NC = 0;
    for (int64_t Lt = p.L; Lt <= 64; Lt *= 2) {
        const int nc = static_cast<int>((p.W + Lt - 1) / Lt);
        int nb = 0;
        PN_HIP(cell_resident_adv_max_blocks(p.kind, p.DP, static_cast<int>(Lt), p.m, &nb));
        if (static_cast<int64_t>(p.B) * nc <= nb) {
            L = static_cast<int>(Lt);
            NC = nc;
            break;
        }
        if (Lt >= p.W) break;
    }
    if (L == 0) return PN_EUNSUPPORTED;
    OneLaunchInfo inf;
    int rc = one_launch_info(c, &inf);
    if (rc != PN_OK) return rc;
    char* ws = c.ws;
    ResidentArgs a{};
    a.w = reinterpret_cast<const float*>(ws + p.off_w);
    a.x = x; a.out = out; a.s0 = s0; a.T = T;
    a.W = static_cast<int32_t>(p.W); a.nwin = 1; a.B = p.B; a.D = p.D; a.m = p.m; a.L = L;
    a.NC = NC; a.mode = p.mode; a.undamped = c.lam == 1.0f; a.max_iter = c.max_iter;
    a.lam = c.lam; a.tol = c.tol;
    a.mapA = reinterpret_cast<float*>(ws + p.off_aggA);
    a.mapB = reinterpret_cast<float*>(ws + p.off_aggB);
    Ctrl* ctrl = reinterpret_cast<Ctrl*>(ws + p.off_ctrl);
    a.rslot = &ctrl->rmax[0][0][0];
    a.bar = reinterpret_cast<unsigned*>(ws + p.off_rpart);   // one arrival word per workgroup
    a.err = &ctrl->bar_err;
    a.hist_len = reinterpret_cast<int32_t*>(inf.dev);
    a.win_iters = reinterpret_cast<int32_t*>(inf.dev + (p.off_winfo - p.off_sync));
    a.win_status = a.win_iters + p.nwin;
    a.hist = reinterpret_cast<float*>(inf.dev + (p.off_hist - p.off_sync));
    a.hist_cap = p.hist_cap;
    a.acc = reinterpret_cast<int32_t*>(inf.dev + (p.off_acc - p.off_sync));
    a.acc_cap = p.hist_cap;
    a.ready = reinterpret_cast<unsigned*>(ws + p.off_halo);   // the halo region, unused here
    // residual and first-step slots, arrival words, ready words and error flag start at zero
    PN_HIP(hipMemsetAsync(ctrl, 0, sizeof(Ctrl), c.st));
    PN_HIP(hipMemsetAsync(a.bar, 0, sizeof(unsigned) * p.B * NC, c.st));
    PN_HIP(hipMemsetAsync(a.ready, 0, sizeof(unsigned) * p.B * NC, c.st));
    const bool timed = c.tm->take();
    size_t e0 = 0, e1 = 0;
    if (timed) { rc = request_timing(c, &e0, &e1); if (rc) return rc; }
    {
        const hipError_t le = launch_cell_resident_adv(p.kind, p.DP, a, c.st);
        if (le == hipErrorCooperativeLaunchTooLarge) {
            (void)hipGetLastError();
            g_launch_timing = LaunchTiming{};
            return PN_EUNSUPPORTED;
        }
        if (le != hipSuccess) return fail(PN_EHIP, "cooperative launch failed: %s", hipGetErrorString(le));
    }
    if (timed) { rc = check_timed_launch(); if (rc) return rc; }
    if (c.res->dev_ring) {
        inf.copy.resize(inf.nbytes);
        PN_HIP(hipMemcpyAsync(inf.copy.data(), inf.dev, inf.nbytes, hipMemcpyDeviceToHost, c.st));
        inf.host = inf.copy.data();
    }
    PN_HIP(hipStreamSynchronize(c.st));
    unsigned err = 0;
    PN_HIP(hipMemcpy(&err, a.err, sizeof(err), hipMemcpyDeviceToHost));
    if (err != 0) return fail(PN_EHIP, "grid barrier of the resident solver timed out");
    int32_t hlen = 0;
    std::memcpy(&hlen, inf.host, sizeof(hlen));
    const int32_t* wi = reinterpret_cast<const int32_t*>(inf.host + (p.off_winfo - p.off_sync));
    const float* hist = reinterpret_cast<const float*>(inf.host + (p.off_hist - p.off_sync));
    const int32_t* acc = reinterpret_cast<const int32_t*>(inf.host + (p.off_acc - p.off_sync));
    *K = wi[0];
    *status = wi[p.nwin];
    if (c.hist) c.hist->assign(hist, hist + std::min(hlen, p.hist_cap));
    const int rounds = std::min(*status == PN_NONFINITE ? hlen - 1 : hlen, p.hist_cap);
    accepted->assign(acc, acc + std::max(rounds, 0));
    if (timed) {
        // the windows the updates ran on, from the accepted steps
        double bytes = 0.0, flops = 0.0;
        int64_t A = 0;
        for (int k = 0; k < *K && k < static_cast<int>(accepted->size()); ++k) {
            A += (*accepted)[k];
            const int Tw = static_cast<int>(std::min<int64_t>(T, A + p.W) - A);
            bytes += apply_bytes(p, Tw, false);
            flops += apply_flops(p, Tw);
        }
        c.tm->apply.push_back({e0, e1});
        c.tm->apply_bytes.push_back(bytes);
        c.tm->apply_flops.push_back(flops);
    }
    return PN_OK;
}

// Frees a workspace the library allocated for one call on every exit path.
struct OwnedWorkspace {
    void* p = nullptr;
    hipStream_t st = nullptr;
    ~OwnedWorkspace() {
        if (p) {
            (void)hipFreeAsync(p, st);
            (void)hipStreamSynchronize(st);
        }
    }
    hipError_t release() {
        void* q = p;
        p = nullptr;
        hipError_t e = hipFreeAsync(q, st);
        hipError_t e2 = hipStreamSynchronize(st);
        return e != hipSuccess ? e : e2;
    }
};

int eval_impl(const pn_cell* cell, const float* params, const float* x, const float* s0, int64_t B,
              int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter, float* out,
              int32_t* iters_out, const pn_opts* o, bool half = false, const Backing* bk = nullptr) {
    g_err.clear();
    g_launch_timing = LaunchTiming{};     // no request left over from a failed call
    int rc = validate(cell, params, x, s0, B, T, D, mode, tol, max_iter, out, iters_out, o, half ? 2 : 4);
    if (rc != PN_OK) return rc;
    if (half) {
        if (cell->kind != PN_CELL_DIAG_TANH)
            return fail(PN_EUNSUPPORTED, "binary16 storage supports the channel-wise cell only");
        if (o && ((o->window > 0 && o->window < T) || o->window_mode != PN_WINDOW_CONSECUTIVE))
            return fail(PN_EUNSUPPORTED, "binary16 storage solves the whole horizon as one window");
        if (o && o->switch_mode >= 0)
            return fail(PN_EUNSUPPORTED, "binary16 storage does not combine with switching");
    }
    if (o && o->profile) std::memset(o->profile, 0, sizeof(pn_profile));
    if (B == 0 || T == 0 || D == 0) {
        *iters_out = 0;
        if (o && o->window_iters_len > 0) o->window_iters[0] = 0;
        if (o && o->resid_hist_len > 0) o->resid_hist[0] = 0.0f;
        return PN_OK;
    }
    Plan p, p2;
    bool has2 = false;
    if (half) rc = make_plan(p, cell, B, T, D, mode, o, true);
    else rc = make_plans(p, p2, &has2, cell, B, T, D, mode, o);
    if (rc != PN_OK) return rc;
    if (o && o->workspace && o->workspace_bytes < p.total)
        return fail(PN_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                    o->workspace_bytes, p.total);
    if (bk && bk->bytes < p.total)
        return fail(PN_EWORKSPACE, "problem needs %zu bytes of scratch; the static scratch holds %zu",
                    p.total, bk->bytes);
    ThreadRes* res;
    if (bk) {
        res = bk->res;
    } else {
        rc = get_res(&res);
        if (rc != PN_OK) return rc;
    }
    hipStream_t st = o ? static_cast<hipStream_t>(o->stream) : nullptr;
    char* ws = nullptr;
    OwnedWorkspace own;
    if (bk) {
        ws = bk->ws;
    } else if (o && o->workspace) {
        ws = static_cast<char*>(o->workspace);
    } else {
        void* q = nullptr;
        PN_HIP(hipMallocAsync(&q, p.total, st));
        own.p = q;
        own.st = st;
        ws = static_cast<char*>(q);
    }
    Timing tm;
    tm.on = o && o->profile;
    tm.stride = (o && o->profile_stride > 1) ? o->profile_stride : 1;
    std::vector<float> hist;
    SolveCtx c{&p, st, ws, res, params, tol, o ? o->damping : 1.0f, max_iter, &tm, &hist,
               o ? o->switch_ratio : 0.0f, o ? o->switch_damping : 0.0f};
    // the one-workgroup solver reads the flat parameters itself; a cap of
    // more updates per window than kSmallMaxIter goes to the multi-launch
    // driver, whose host-side wait is bounded
    const bool small = p.small && max_iter <= kSmallMaxIter;
    if (p.matrix_cell && !small)
        PN_HIP(launch_prep_weights(p.kind, params, reinterpret_cast<float*>(ws + p.off_w), p.D, p.DP, p.m,
                                   !p.mfma || (has2 && !p2.mfma), st));
    size_t ev_first = 0;
    if (tm.on) { rc = record(c, &ev_first); if (rc) return rc; }
    int total = 0, overall = PN_OK;
    std::vector<int> wit;
    std::vector<int32_t> accepted, wsw;
    const int64_t m = p.m;
    bool persisted = false;
    const bool multi = o && (o->flags & (PN_FLAG_MULTI_LAUNCH | PN_FLAG_PERSISTENT));
    if (small) {
        rc = solve_small(c, x, s0, out, T, &wit, &total, &overall);
        if (rc != PN_OK) return rc;
        persisted = true;
    } else if (p.resident_ok && !multi && max_iter <= kSmallMaxIter) {
        rc = solve_resident(c, x, s0, out, T, &wit, &total, &overall);
        if (rc == PN_OK) persisted = true;
        else if (rc != PN_EUNSUPPORTED) return rc;
    }
    if (!persisted && p.persist_ok && o && (o->flags & PN_FLAG_PERSISTENT)) {
        rc = solve_persistent(c, x, s0, out, T, &wit, &total, &overall);
        if (rc == PN_OK) persisted = true;
        else if (rc != PN_EUNSUPPORTED) return rc;
    }
    if (p.advancing) {
        int K = 0, status = PN_OK;
        // one launch when the chunks fit at once and the history holds every check
        rc = PN_EUNSUPPORTED;
        if (p.adv_resident_ok && !multi && max_iter < p.hist_cap)
            rc = solve_advancing_resident(c, x, s0, out, T, &K, &status, &accepted);
        if (rc == PN_EUNSUPPORTED) {
            accepted.clear();
            if (c.hist) c.hist->clear();
            rc = solve_advancing(c, x, s0, out, T, &K, &status, &accepted);
        }
        if (rc != PN_OK) return rc;
        total = K;
        wit.push_back(K);
        overall = status;
        persisted = true;       // nothing left for the window loop below
    }
    for (int64_t w0 = 0; !persisted && w0 < T; w0 += p.W) {
        const int Tw = static_cast<int>(std::min<int64_t>(p.W, T - w0));
        const float* xw = x + w0 * m;
        float* sw = out + w0 * D;
        const float* s0w = w0 == 0 ? s0 : out + (w0 - 1) * D;
        const int64_t s0s = w0 == 0 ? D : T * D;
        int K = 0, status = PN_OK, swi = -1;
        rc = solve_window(c, xw, T * m, sw, T * D, s0w, s0s, Tw, &K, &status, has2 ? &p2 : nullptr, &swi);
        if (rc != PN_OK) return rc;
        total += K;
        wit.push_back(K);
        wsw.push_back(swi);
        if (status == PN_NONFINITE) { overall = PN_NONFINITE; break; }
        if (status == PN_NOT_CONVERGED) overall = PN_NOT_CONVERGED;
    }
    size_t ev_last = 0;
    if (tm.on) { rc = record(c, &ev_last); if (rc) return rc; }
    PN_HIP(hipStreamSynchronize(st));
    if (own.p) PN_HIP(own.release());
    *iters_out = total;
    if (o) {
        for (int64_t k = 0; k < o->window_iters_len && k < static_cast<int64_t>(wit.size()); ++k)
            o->window_iters[k] = wit[k];
        for (int32_t k = 0; k < o->resid_hist_len && k < static_cast<int32_t>(hist.size()); ++k)
            o->resid_hist[k] = hist[k];
        for (int64_t k = 0; o->accepted && k < o->accepted_len && k < static_cast<int64_t>(accepted.size()); ++k)
            o->accepted[k] = accepted[k];
        for (int64_t k = 0; o->window_switch && k < o->window_switch_len && k < static_cast<int64_t>(wsw.size()); ++k)
            o->window_switch[k] = wsw[k];
        if (o->profile) {
            pn_profile* pr = o->profile;
            for (size_t k = 0; k < tm.apply.size(); ++k) {
                float ms = 0.0f;
                PN_HIP(hipEventElapsedTime(&ms, res->timing[tm.apply[k].first], res->timing[tm.apply[k].second]));
                pr->apply_ms += ms;
                pr->apply_bytes += tm.apply_bytes[k];
                pr->apply_flops += tm.apply_flops[k];
            }
            pr->apply_launches = static_cast<int32_t>(tm.apply.size());
            float ms = 0.0f;
            PN_HIP(hipEventElapsedTime(&ms, res->timing[ev_first], res->timing[ev_last]));
            pr->total_ms = ms;
        }
    }
    return overall;
}

}  // namespace

namespace pn {
LaunchTiming& launch_timing() { return g_launch_timing; }
}  // namespace pn

extern "C" {

void pn_opts_init(pn_opts* o) {
    if (!o) return;
    std::memset(o, 0, sizeof(*o));
    o->damping = 1.0f;
    o->bandwidth = 1;
    o->switch_mode = -1;
    o->switch_ratio = 0.5f;
    o->switch_damping = 0.0f;
    o->profile_stride = 1;
}

int pn_eval_ex(const pn_cell* cell, const float* params, const float* x, const float* s0, int64_t B,
               int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter, float* out,
               int32_t* iters_out, const pn_opts* opts) {
    return eval_impl(cell, params, x, s0, B, T, D, mode, tol, max_iter, out, iters_out, opts);
}

int pn_eval(const pn_cell* cell, const float* params, const float* x, const float* s0, int64_t B,
            int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter, float* out,
            int32_t* iters_out) {
    return eval_impl(cell, params, x, s0, B, T, D, mode, tol, max_iter, out, iters_out, nullptr);
}

int pn_eval_f16(const pn_cell* cell, const float* params, const uint16_t* x, const float* s0,
                int64_t B, int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter,
                uint16_t* out, int32_t* iters_out, const pn_opts* opts) {
    // the kernels address x and out in binary16 elements; the float pointer
    // type below only carries the address
    if (D % 2 == 0 && ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) & 3) != 0) {
        g_err.clear();
        return fail(PN_EINVAL, "binary16 x and out must be 4-byte aligned");
    }
    return eval_impl(cell, params, reinterpret_cast<const float*>(x), s0, B, T, D, mode, tol, max_iter,
                     reinterpret_cast<float*>(out), iters_out, opts, true);
}

int pn_eval_noalloc(const pn_cell* cell, const float* params, const float* x, const float* s0,
                    int64_t B, int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter,
                    float* out, int32_t* iters_out, const pn_opts* opts) {
    g_err.clear();
    if (opts && (opts->workspace || opts->workspace_bytes))
        return fail(PN_EINVAL, "pn_eval_noalloc runs on the static scratch: opts->workspace must be NULL");
    if (opts && opts->profile)
        return fail(PN_EINVAL, "profiling creates timing events, which pn_eval_noalloc does not");
    int rc = validate(cell, params, x, s0, B, T, D, mode, tol, max_iter, out, iters_out, opts);
    if (rc != PN_OK) return rc;
    if (B == 0 || T == 0 || D == 0) return eval_impl(cell, params, x, s0, B, T, D, mode, tol, max_iter,
                                                     out, iters_out, opts);
    // the size check comes before any device call
    Plan p, p2;
    bool has2 = false;
    rc = make_plans(p, p2, &has2, cell, B, T, D, mode, opts);
    if (rc != PN_OK) return rc;
    if (p.total > kStaticScratchBytes - kStaticRingBytes)
        return fail(PN_EWORKSPACE, "problem needs %zu bytes of scratch; pn_eval_noalloc has %zu",
                    p.total, kStaticScratchBytes - kStaticRingBytes);
    void* base = nullptr;
    size_t bytes = 0;
    const hipError_t e = static_scratch(&base, &bytes);
    if (e != hipSuccess) return fail(PN_EHIP, "static scratch lookup failed: %s", hipGetErrorString(e));
    // check records go to the first kStaticRingBytes of the scratch; the
    // host reads each back into this shadow
    HostRec shadow[kHostRing];
    ThreadRes r;
    (void)hipGetDevice(&r.device);
    r.host = shadow;
    r.host_dev = static_cast<HostRec*>(base);
    r.dev_ring = true;
    r.epoch = g_static_epoch.fetch_add(1 << 16);
    Backing bk{static_cast<char*>(base) + kStaticRingBytes, bytes - kStaticRingBytes, &r};
    return eval_impl(cell, params, x, s0, B, T, D, mode, tol, max_iter, out, iters_out, opts, false, &bk);
}

size_t pn_workspace_bytes(const pn_cell* cell, int64_t B, int64_t T, int64_t D, int32_t mode,
                          const pn_opts* opts) {
    g_err.clear();
    int32_t dummy = 0;
    static const float kDummy = 0.0f;
    int rc = validate(cell, &kDummy, &kDummy, &kDummy, B, T, D, mode, 0.0f, 0, &kDummy, &dummy, opts, 0);
    if (rc != PN_OK) return 0;
    if (B == 0 || T == 0 || D == 0) return kAlign;
    Plan p, p2;
    bool has2 = false;
    if (make_plans(p, p2, &has2, cell, B, T, D, mode, opts) != PN_OK) return 0;
    size_t total = p.total;
    if (cell->kind == PN_CELL_DIAG_TANH) {
        // the same size also serves pn_eval_f16, whose chunking differs
        Plan h;
        if (make_plan(h, cell, B, T, D, mode, opts, true) == PN_OK) total = std::max(total, h.total);
    }
    return total;
}

size_t pn_affine_scan_workspace_bytes(int64_t B, int64_t T, int64_t D, int32_t dense,
                                      const pn_opts* opts) {
    g_err.clear();
    if (B < 0 || T < 0 || D < 0) { fail(PN_EINVAL, "negative size"); return 0; }
    if (dense && D > 64) { fail(PN_EUNSUPPORTED, "dense scan supports D <= 64"); return 0; }
    if (B == 0 || T == 0 || D == 0) return kAlign;
    if (!dense) {
        // one-pass look-back: chunk maps, end states, flags, ticket and error word
        const int64_t L = std::min<int64_t>(kLbChunk, T);
        const int64_t NC = (T + L - 1) / L;
        const int64_t nblk = (D + kLbChannels - 1) / kLbChannels;
        const size_t bnd = static_cast<size_t>(B) * NC * D;
        return 3 * align_up(sizeof(float) * bnd) + align_up(sizeof(uint32_t) * B * NC * nblk) + kAlign;
    }
    const int chunk = opts && opts->chunk > 0 ? opts->chunk : 32;
    const int64_t L = std::min<int64_t>(chunk, T);
    const int64_t NC = (T + L - 1) / L;
    const size_t bnd = static_cast<size_t>(B) * NC * D;
    return align_up(sizeof(float) * bnd * D) + 2 * align_up(sizeof(float) * bnd);
}

int pn_affine_scan(const float* A, const float* b, const float* s0, int64_t B, int64_t T, int64_t D,
                   int32_t dense, float* out, const pn_opts* opts) {
    g_err.clear();
    if (B < 0 || T < 0 || D < 0) return fail(PN_EINVAL, "negative size");
    if (dense != 0 && dense != 1) return fail(PN_EINVAL, "dense must be 0 or 1");
    if (opts && (opts->chunk < 0 || opts->chunk > (1 << 20))) return fail(PN_EINVAL, "chunk out of range");
    if (opts && opts->workspace && (reinterpret_cast<uintptr_t>(opts->workspace) % kAlign) != 0)
        return fail(PN_EWORKSPACE, "workspace must be 256-byte aligned");
    if (B == 0 || T == 0 || D == 0) return PN_OK;
    if (!A || !b || !s0 || !out) return fail(PN_EINVAL, "a device pointer is NULL");
    if (dense && D > 64) return fail(PN_EUNSUPPORTED, "dense scan supports D <= 64");
    if (B > 65535 || T >= (int64_t(1) << 31)) return fail(PN_EUNSUPPORTED, "size too large");
    const int64_t nout = B * T * D * 4;
    if (overlaps(out, nout, A, nout * (dense ? D : 1)) || overlaps(out, nout, b, nout) ||
        overlaps(out, nout, s0, B * D * 4))
        return fail(PN_EINVAL, "out overlaps an input");
    const size_t need = pn_affine_scan_workspace_bytes(B, T, D, dense, opts);
    hipStream_t st = opts ? static_cast<hipStream_t>(opts->stream) : nullptr;
    char* ws = nullptr;
    OwnedWorkspace own;
    if (opts && opts->workspace) {
        if (opts->workspace_bytes < need)
            return fail(PN_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                        opts->workspace_bytes, need);
        ws = static_cast<char*>(opts->workspace);
    } else {
        void* q = nullptr;
        PN_HIP(hipMallocAsync(&q, need, st));
        own.p = q;
        own.st = st;
        ws = static_cast<char*>(q);
    }
    if (!dense) {
        LookbackArgs a{};
        a.A = A; a.b = b; a.s0 = s0; a.out = out;
        a.B = static_cast<int>(B); a.T = static_cast<int>(T); a.D = static_cast<int>(D);
        a.L = static_cast<int>(std::min<int64_t>(kLbChunk, T));
        a.NC = static_cast<int>((T + a.L - 1) / a.L);
        a.nblk = static_cast<int>((D + kLbChannels - 1) / kLbChannels);
        const size_t bnd = static_cast<size_t>(B) * a.NC * D;
        size_t off = 0;
        a.aggA = reinterpret_cast<float*>(ws + off); off += align_up(sizeof(float) * bnd);
        a.aggB = reinterpret_cast<float*>(ws + off); off += align_up(sizeof(float) * bnd);
        a.yv = reinterpret_cast<float*>(ws + off); off += align_up(sizeof(float) * bnd);
        const size_t nflag = align_up(sizeof(uint32_t) * B * a.NC * a.nblk);
        a.flag = reinterpret_cast<uint32_t*>(ws + off);
        a.ticket = reinterpret_cast<uint32_t*>(ws + off + nflag);
        a.err = a.ticket + 1;
        PN_HIP(hipMemsetAsync(a.flag, 0, nflag + kAlign, st));
        PN_HIP(launch_scan_lookback(a, st));
        uint32_t err = 0;
        PN_HIP(hipMemcpyAsync(&err, a.err, sizeof(err), hipMemcpyDeviceToHost, st));
        PN_HIP(hipStreamSynchronize(st));
        if (own.p) PN_HIP(own.release());
        if (err != 0) return fail(PN_EHIP, "a look-back wait of the scan timed out");
        return PN_OK;
    }
    const int chunk = opts && opts->chunk > 0 ? opts->chunk : 32;
    const int L = static_cast<int>(std::min<int64_t>(chunk, T));
    const int NC = static_cast<int>((T + L - 1) / L);
    const size_t bnd = static_cast<size_t>(B) * NC * D;
    ScanArgs a{};
    a.A = A; a.b = b; a.out = out;
    a.B = static_cast<int>(B); a.T = static_cast<int>(T); a.D = static_cast<int>(D); a.L = L; a.NC = NC;
    a.aggA = reinterpret_cast<float*>(ws);
    a.aggB = reinterpret_cast<float*>(ws + align_up(sizeof(float) * bnd * D));
    float* carry = reinterpret_cast<float*>(reinterpret_cast<char*>(a.aggB) + align_up(sizeof(float) * bnd));
    a.carry = carry;
    const int DP = std::max(4, next_pow2(static_cast<int>(D)));
    PN_HIP(launch_scan_aggregate(true, DP, a, st));
    CarryArgs cy{};
    cy.aggA = a.aggA; cy.aggB = a.aggB; cy.carry = carry; cy.s0 = s0; cy.s0s = D;
    cy.B = a.B; cy.D = a.D; cy.NC = NC; cy.do_check = 0;
    PN_HIP(launch_dense_carry(cy, st));
    PN_HIP(launch_scan_apply(true, DP, a, st));
    PN_HIP(hipStreamSynchronize(st));
    if (own.p) PN_HIP(own.release());
    return PN_OK;
}

const char* pn_last_error(void) { return g_err.c_str(); }

const char* pn_version(void) { return "pn 0.1.0 gfx950"; }

}  // extern "C"
