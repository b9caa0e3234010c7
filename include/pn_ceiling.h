/*
 * pn_ceiling.h -- measured ceilings of this GPU for the solver's access
 * patterns (libpn_ceiling.so, a measurement tool beside libpn).
 *
 * The data-sheet peaks (HBM 8 TB/s, FP32 matrix 157.3 TFLOP/s) are not what
 * any kernel attains; these microbenchmarks measure what plain streaming
 * kernels and a plain matrix-core loop do attain, so that a kernel's
 * achieved rate can be set against both.  The memory-access advice of the
 * parallel-Newton article (coalesced, contiguous access [PN §2.1]) is what
 * the patterns below follow.
 *
 * Every function allocates its own device buffers (hipMalloc) on the current
 * device, times `reps` launches with HIP events on a stream of its own after
 * one untimed launch, frees everything and returns 0, or -1 with a message
 * in pnc_last_error().
 */
#ifndef PN_CEILING_H
#define PN_CEILING_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Patterns; n = bytes per array, rate = bytes moved per launch / time:
 *  PNC_READ       sum of one array                               (n)
 *  PNC_WRITE      fill of one array                              (n)
 *  PNC_COPY       y = x                                          (2n)
 *  PNC_2R1W       s = x + 0.5 s, flat float4 grid stride         (3n)
 *  PNC_2R1W_ROWS  s = x + 0.5 s over [8, T, 256] float arrays in the access
 *                 order of the channel-wise apply kernel: one workgroup per
 *                 (batch row, 1024-step chunk), one channel per thread, rows
 *                 in order with 8-step register prefetch; T from n (3n).
 *  PNC_READ_ROWS  sum of x over [8, T, 256] in the access order of the
 *                 channel-wise sweeps that read only x: one workgroup per
 *                 (batch row, 512-step chunk), one channel per thread, 16
 *                 rows in flight while the previous 16 are summed (n). */
enum { PNC_READ = 0, PNC_WRITE = 1, PNC_COPY = 2, PNC_2R1W = 3, PNC_2R1W_ROWS = 4, PNC_READ_ROWS = 5 };

/* Best and median rate in GB/s (1e9 bytes/s) of `reps` launches. */
int pnc_hbm(int pattern, size_t bytes, int reps, double* best_gbs, double* median_gbs);

/* Best and median FP32 matrix-core rate in TFLOP/s: independent chains of
 * v_mfma_f32_32x32x2f32 on register operands, two wavefronts per SIMD. */
int pnc_mfma_f32(int reps, double* best_tflops, double* median_tflops);

/* The plain time loop of the channel-wise cell on the GPU, the baseline a
 * parallel-in-time solve has to beat: s_t = tanh(a[d] s_{t-1} + x[b,t,d])
 * for t = 1..T from s_0 = s0[b,d], one thread per (b, d), in time order.
 * x [B,T,D], a [D], s0 [B,D] and out [B,T,D] (receives s_1..s_T) are
 * caller-owned float32 device arrays.  Runs one untimed and `reps` timed
 * launches on a stream of its own; best and median milliseconds per launch.
 * Returns 0, or -1 (bad argument: null pointer, a size below 1, B > 65535,
 * reps < 1; or a HIP failure) with a message in pnc_last_error(). */
int pnc_sequential_tanh(const float* x, const float* a, const float* s0, float* out, int B, int T, int D,
                        int reps, double* best_ms, double* median_ms);

/* Message of the last failure on this thread ("" if none). */
const char* pnc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PN_CEILING_H */
