/*
 * pn.h -- C interface of libpn, a GPU engine that evaluates nonlinear
 * recurrences s_t = f_t(s_{t-1}), t = 1..T, in parallel over time.
 *
 * Method: the web article "并行牛顿方法：加速非线性序列评估的计算革命" (a survey of
 * parallel Newton methods for nonlinear sequence evaluation; cited below as
 * [PN §x]).  The whole trajectory s = (s_1..s_T) is the unknown of a
 * fixed-point problem F(s) = 0 [PN §1.2] with
 *     F_t(s) = s_t - f_t(s_{t-1}),   s_0 given,
 * and is improved by s <- s - J~^{-1}(s) F(s), where J~ is I minus the
 * sub-diagonal of approximated state Jacobians A~_t ~ df_t/ds_{t-1}:
 *     Jacobi        A~_t = 0                      [PN §1.2]
 *     Picard        A~_t = I                      [PN §1.2, §2.2.3]
 *     quasi-Newton  A~_t = diag(df_t/ds_{t-1})    [PN §2.2.1]
 *     banded        A~_t = band_k(df_t/ds_{t-1})  [PN §2.2.2]
 *                   (entries with |i - j| <= k kept, the rest zero)
 *     Newton        A~_t = df_t/ds_{t-1} (dense)  [PN §1.2]
 * Applying J~^{-1} is the first-order linear recurrence
 *     s^_t = v_t + A~_t (s^_{t-1} - p_t),  p_t = s_{t-1},  v_t = f_t(p_t),
 * evaluated by an associative scan over affine maps [PN §2.1].
 *
 * Readings fixed by this library where the article is silent:
 *   - initial iterate s_t = s_0 for every t;
 *   - residual r = max over (b, t, d) of |F|, one stop rule for the batch;
 *   - stop at the first check with r non-finite (PN_NONFINITE), else with
 *     r <= tol (PN_OK), else when max_iter updates have been applied
 *     (PN_NOT_CONVERGED); the count reported is the number of updates;
 *   - damping lam in (0, 1] is step damping, s <- s + lam (s^ - s)
 *     [PN §4.3 suggests more damping when iterations stall];
 *   - windows [PN §1.3.1, §2.3]: consecutive blocks of W steps solved in
 *     order, window w starting from the last state of window w-1; or, with
 *     PN_WINDOW_ADVANCING, one window of W steps that slides past its
 *     converged prefix (below).
 *
 * Memory conventions (all functions):
 *   - float pointers named params, x, s0, out, A, b are DEVICE pointers to
 *     C-contiguous float32 arrays owned by the caller; the library never
 *     frees them.
 *   - x is [B, T, m]; s0 is [B, D]; out is [B, T, D] and receives s_1..s_T.
 *   - pointers named *_hist, *_iters, iters_out, profile are HOST pointers.
 *   - calls block until the result is complete on the device.
 *   - on a negative (error) status the message is available from
 *     pn_last_error() on the calling thread.  Argument, size and workspace
 *     errors are found before any device work and leave out untouched; once
 *     kernels have been enqueued (PN_EHIP from a failed launch, copy or
 *     wait), out is unspecified.
 *   - out must not share a byte with x, s0 or params (PN_EINVAL otherwise).
 *   - thread-safe when concurrent calls use distinct streams and workspaces.
 */
#ifndef PN_H
#define PN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Transition maps f(p, x) (p = previous state, x = input at this step).
 *  PN_CELL_DIAG_TANH  f = tanh(a * p + x), channel-wise; params a[D];
 *                     input_dim must equal D.  Any D >= 1.
 *  PN_CELL_TANH_RNN   f = tanh(W p + U x + b); params W[D*D] | U[D*m] | b[D]
 *                     (row-major, W[i*D+k] multiplies p_k into output i).
 *                     1 <= D <= 64.
 *  PN_CELL_GRU        gated recurrent unit with torch.nn.GRU's equations and
 *                     gate order (r, z, n); params W_ih[3D*m] | W_hh[3D*D] |
 *                     b_ih[3D] | b_hh[3D].  1 <= D <= 64.
 *  PN_CELL_EULER_TANH f = p + h * (tanh(W p + U x + b) - p): one explicit
 *                     Euler step (per-channel step sizes h) of the
 *                     continuous-time RNN ds/dt = -s + tanh(W s + U x + b);
 *                     params W[D*D] | U[D*m] | b[D] | h[D].  1 <= D <= 64.
 * The RNN cells are the application the article names [PN §1.3.2]; the
 * Euler cell is the small-step regime of [PN §1.3.1, §2.2.3], where the
 * dynamics Jacobian is close to the identity. */
enum { PN_CELL_DIAG_TANH = 0, PN_CELL_TANH_RNN = 1, PN_CELL_GRU = 2, PN_CELL_EULER_TANH = 3 };

/* Jacobian approximations (see above).  Every cell supports every mode.
 * PN_BANDED takes its half-bandwidth k from pn_opts.bandwidth; band_0 is the
 * diagonal and band_{D-1} the whole matrix, so k = 0 runs as PN_QUASI_NEWTON
 * and k >= D-1 as PN_NEWTON (for the channel-wise cell every k runs as
 * PN_QUASI_NEWTON: its Jacobian is diagonal). */
enum { PN_JACOBI = 0, PN_PICARD = 1, PN_QUASI_NEWTON = 2, PN_NEWTON = 3, PN_BANDED = 4 };

/* Status codes. */
enum {
    PN_OK = 0,              /* converged: final r <= tol                       */
    PN_NOT_CONVERGED = 1,   /* max_iter updates applied; out = last iterate     */
    PN_NONFINITE = 2,       /* r became NaN/Inf; out = the offending iterate     */
    PN_EINVAL = -1,         /* bad argument (null pointer, negative size, ...)  */
    PN_EUNSUPPORTED = -2,   /* valid but unsupported shape (e.g. D > 64 RNN)    */
    PN_EHIP = -3,           /* a HIP runtime call failed                         */
    PN_EWORKSPACE = -4      /* workspace missing, misaligned or too small        */
};

typedef struct pn_cell {
    int32_t kind;        /* PN_CELL_*                                        */
    int32_t input_dim;   /* m, the width of x (>= 1; == D for DIAG_TANH)      */
} pn_cell;

/* Optional per-call measurements of the library's own kernels, taken with
 * HIP events on the call's stream.  They cover the steady-state launches of
 * the fused per-iteration "apply" kernel (cell + Jacobian + scan replay +
 * damping + residual + next chunk maps) for iterations i >= 1, including the
 * last launches, which find the loop stopped and exit at once; with
 * pn_opts.profile_stride n > 1, only every n-th of them (each event pair
 * adds stream work between launches).  Algorithmic bytes of a launch that
 * runs: read x and s^(i), write s^(i+1); 0 for a launch that exits. */
typedef struct pn_profile {
    double apply_ms;          /* summed device time of apply launches       */
    int32_t apply_launches;   /* timed launches, including early-exit ones    */
    double apply_bytes;       /* summed algorithmic bytes of those launches   */
    double apply_flops;       /* summed algorithmic flops: matrix-cell
                                 evaluations and, for Newton and the banded
                                 mode, the chunk-map compose with A~_t (a
                                 band of 2k+1 diagonals costs that fraction
                                 of the dense product; 0 for the
                                 channel-wise cell)                           */
    double total_ms;          /* first launch to last completion              */
} pn_profile;

typedef struct pn_opts {
    float damping;            /* (0, 1]; 1 = plain update                      */
    int32_t chunk;            /* timesteps per tile; 0 = library choice         */
    int64_t window;           /* 0 = whole horizon, else W >= 1                 */
    void* stream;             /* hipStream_t; NULL = the null stream            */
    void* workspace;          /* device memory, 256-byte aligned; NULL = the
                                 library allocates (stream-ordered) per call   */
    size_t workspace_bytes;
    float* resid_hist;        /* host; receives r_0..r_K of each window in
                                 order (truncated to resid_hist_len)           */
    int32_t resid_hist_len;
    int32_t* window_iters;    /* host; updates per window (truncated)          */
    int64_t window_iters_len;
    pn_profile* profile;      /* host; NULL = no event timing                   */
    int32_t flags;            /* PN_FLAG_* bits, 0 = defaults                    */
    int32_t bandwidth;        /* PN_BANDED half-bandwidth k >= 0 (default 1)    */
    int32_t window_mode;      /* PN_WINDOW_CONSECUTIVE (default) or
                                 PN_WINDOW_ADVANCING                            */
    int32_t* accepted;        /* host; advancing window: steps accepted at each
                                 check with a finite residual, in order
                                 (truncated to accepted_len)                   */
    int64_t accepted_len;
    int32_t switch_mode;      /* -1 (default): off; else the mode a window
                                 moves to when its residual stalls (below)     */
    float switch_ratio;       /* rho >= 0 of the stall test (default 0.5)      */
    int32_t* window_switch;   /* host; per window: the check that switched, or
                                 -1 (truncated to window_switch_len)           */
    int64_t window_switch_len;
    float switch_damping;     /* 0 (default): the damping stays `damping` after
                                 a switch; else, in (0, 1], the step damping of
                                 the updates after it (below)                  */
    int32_t profile_stride;   /* with profile: time every n-th steady apply
                                 launch (0 or 1: every one)                    */
} pn_opts;

/* Residual-driven switching [PN §5.3]: start each window on the coarse
 * approximation `mode` and move to `switch_mode` once the residual stalls.
 * At each check i >= 1 of a window still on `mode`, r_i > switch_ratio *
 * r_{i-1} switches it: update i (already under way) keeps `mode`, updates
 * i+1, ... use `switch_mode` (its chunk maps are rebuilt at s^(i+1) by one
 * extra sweep when it differs from `mode`) and, if switch_damping > 0, the
 * step damping switch_damping instead of `damping` -- the other remedy the
 * article gives for a stalling curve.  switch_mode == mode with
 * switch_damping set switches the damping alone.  Consecutive windows, float
 * storage (pn_eval_ex); PN_EUNSUPPORTED with the advancing window or
 * pn_eval_f16.  A typical use is quasi-Newton first, then the banded or full
 * Jacobian. */

/* pn_opts.window_mode.
 * PN_WINDOW_CONSECUTIVE: windows of W steps solved one after another, each
 *   to tol; max_iter caps the updates of each window; window_iters and
 *   resid_hist hold one entry / one run per window.
 * PN_WINDOW_ADVANCING (every cell; float storage; the sliding window of
 *   [PN §1.3.1]): steps [0, a) are accepted and never change again; the
 *   window is [a, min(T, a + W)).  Each round checks the current iterate on
 *   the window, r_t = max over (b, d) of |F_t|, and r = max_t r_t (stored in
 *   resid_hist); r not finite stops with PN_NONFINITE; otherwise a moves to
 *   the first t with r_t > tol (past the window if none), a = T stops with
 *   PN_OK, and after max_iter updates in total the solve stops with
 *   PN_NOT_CONVERGED.  The window then slides to [a, min(T, a + W)), steps
 *   entering it start from its last state, and one update of the chosen mode
 *   is applied to it.  *iters_out and window_iters[0] count the updates; on
 *   exit, steps the window never reached hold its last state.  Damping and
 *   every mode apply; PN_FLAG_PERSISTENT is ignored. */
enum { PN_WINDOW_CONSECUTIVE = 0, PN_WINDOW_ADVANCING = 1 };

/* pn_opts.flags.  PN_FLAG_PERSISTENT runs a solve of a matrix cell in a
 * diagonal mode as one cooperative launch (all windows and iterations, with
 * grid-wide barriers between the carry and apply phases), when the device
 * supports cooperative launches and the weights fit in LDS; otherwise, and by
 * default, each phase is its own launch.  Results meet the same bar; on
 * MI355X a grid barrier costs more than a launch boundary, so the default is
 * the faster one for the shapes measured here. */
enum { PN_FLAG_PERSISTENT = 1 };

/* pn_opts.flags.  By default the library runs some solves in one launch:
 *  - a matrix cell with D <= 8 whose windows hold at most 1024 (D <= 4) or
 *    512 (D <= 8) (b, t) pairs, in one workgroup, every window, iteration
 *    and check included (float storage, consecutive windows, no switching,
 *    chunk 0, max_iter <= 16384);
 *  - a matrix cell in a diagonal mode (Jacobi, Picard, quasi-Newton) with D
 *    padded to 16, 32 or 64, float storage and no switching, as one
 *    cooperative launch of workgroups that each keep a chunk on chip, when
 *    all chunks fit on the device at once: consecutive windows of at most
 *    128 chunks (max_iter <= 16384), or the advancing window, whose
 *    acceptance decisions and window moves are then taken on the device
 *    (max_iter below ceil(T / W) * (W + 1) and below 65536, the capacity of
 *    its residual history).
 * PN_FLAG_MULTI_LAUNCH keeps such a solve on the launch-per-phase driver
 * instead.  Results meet the same bar either way. */
enum { PN_FLAG_MULTI_LAUNCH = 2 };

/* Fill *o with the defaults: damping 1, chunk 0, window 0, bandwidth 1,
 * switch_mode -1, switch_ratio 0.5, switch_damping 0, profile_stride 1,
 * everything else NULL / 0. */
void pn_opts_init(pn_opts* o);

/* Solve the recurrence for all B sequences [PN §1.1, §1.2].
 *   cell      host struct, read during the call only.
 *   params    device, float32, layout per cell kind (above).
 *   x         device [B, T, m];  s0 device [B, D].
 *   mode      PN_JACOBI .. PN_BANDED (PN_BANDED needs opts->bandwidth >= 0;
 *             pn_eval without options uses k = 1).
 *   tol       stop when r <= tol (tol >= 0; 0 runs to max_iter unless r == 0).
 *   max_iter  cap on updates per window (>= 0).
 *   out       device [B, T, D].  iters_out host int32: total updates applied
 *             over all windows.
 * Returns a status code.  B, T or D equal to 0 is an empty problem: PN_OK
 * with *iters_out = 0 and nothing written. */
int pn_eval(const pn_cell* cell, const float* params, const float* x, const float* s0,
            int64_t B, int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter,
            float* out, int32_t* iters_out);

/* pn_eval with options (opts may be NULL = defaults). */
int pn_eval_ex(const pn_cell* cell, const float* params, const float* x, const float* s0,
               int64_t B, int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter,
               float* out, int32_t* iters_out, const pn_opts* opts);

/* pn_eval_ex for callers that cannot allocate device memory (serving loops
 * and harnesses that forbid allocation during a call): the same solve, with
 * the same arguments, options and results, run on a static device scratch
 * that the library holds on each GPU it runs on until the process ends
 * (32 MiB, enough for every workload in this repository's benchmarks).  The
 * call itself allocates nothing: no device or pinned memory, no events.
 * opts->workspace must be NULL and opts->profile NULL (PN_EINVAL otherwise);
 * a problem whose workspace (pn_workspace_bytes) exceeds the scratch less
 * 256 bytes of check records returns PN_EWORKSPACE before any device work.
 * The host reads each convergence check back with a copy after draining the
 * stream, so iterations do not overlap the host's reading as in pn_eval_ex.
 * Every call on a GPU shares that GPU's scratch, which keeps the contents
 * of the last call (the library clears what must start at zero): calls that
 * overlap on one GPU, from any threads or streams, race and must not be
 * made. */
int pn_eval_noalloc(const pn_cell* cell, const float* params, const float* x, const float* s0,
                    int64_t B, int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter,
                    float* out, int32_t* iters_out, const pn_opts* opts);

/* Bytes of workspace pn_eval_ex (and pn_eval_f16) needs for this problem
 * with these options (opts may be NULL).  The size depends on the window and
 * also on the chunk, the mode switch and the bandwidth, so the whole option
 * block is taken rather than the window alone.  Returns 0 and sets the last
 * error for invalid or unsupported arguments. */
size_t pn_workspace_bytes(const pn_cell* cell, int64_t B, int64_t T, int64_t D,
                          int32_t mode, const pn_opts* opts);

/* pn_eval_ex with reduced-precision storage [PN §2.3, §4.2]: x and out hold
 * IEEE binary16 values (device, same shapes and layouts as pn_eval); params
 * and s0 stay float32 and all arithmetic is float32.  Every stored state is
 * rounded to nearest-even binary16, and the iteration continues from the
 * stored (rounded) states, so tol must lie above the binary16 resolution of
 * the states (about 2.4e-4 for |s| < 1).  Supported for PN_CELL_DIAG_TANH,
 * solved as one window (opts->window 0 or >= T, consecutive mode);
 * PN_EUNSUPPORTED otherwise.  With D even, x and out must be 4-byte aligned
 * (two channels move per access).  pn_workspace_bytes covers this entry
 * too.  It moves 6 bytes per state element and iteration instead of 12. */
int pn_eval_f16(const pn_cell* cell, const float* params, const uint16_t* x, const float* s0,
                int64_t B, int64_t T, int64_t D, int32_t mode, float tol, int32_t max_iter,
                uint16_t* out, int32_t* iters_out, const pn_opts* opts);

/* The scan step alone [PN §2.1]: out_t = A_t out_{t-1} + b_t, out_0 = s0,
 * for t = 1..T.  A is device [B, T, D] (dense = 0: diagonal A_t) or
 * [B, T, D, D] (dense = 1, row-major, 1 <= D <= 64); b device [B, T, D];
 * s0 device [B, D]; out device [B, T, D], sharing no byte with the inputs.
 * Diagonal A runs in one pass with a decoupled look-back over 32-step
 * chunks (A and b read once, out written once); dense A composes chunk
 * maps, scans their carries and replays (opts->chunk steps per chunk, 0 =
 * 32).  Uses opts->stream and opts->workspace (NULL: allocated per call);
 * returns PN_OK or an error code. */
int pn_affine_scan(const float* A, const float* b, const float* s0, int64_t B, int64_t T,
                   int64_t D, int32_t dense, float* out, const pn_opts* opts);

/* Workspace bytes for pn_affine_scan. */
size_t pn_affine_scan_workspace_bytes(int64_t B, int64_t T, int64_t D, int32_t dense,
                                      const pn_opts* opts);

/* Message of the last error on this thread ("" if none).  The pointer stays
 * valid until the next library call on the same thread. */
const char* pn_last_error(void);

/* Library version string, e.g. "pn 0.1.0 gfx950". */
const char* pn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PN_H */
