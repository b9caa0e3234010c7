// Matrix cells (tanh RNN, GRU): fused iteration kernel for every mode, the
// dense carry scan, and the weight preparation kernel.
//
// Work split per iteration is the same as for the channel-wise cell (see
// pn_diag.hip): a tiny carry scan over per-chunk affine maps, then one apply
// sweep per chunk that replays the recurrence of [PN §1.2] from the carry,
// stores s^(i+1) and, at the new iterate, produces the residual and the chunk
// maps of iteration i+1.  Differences:
//   * the cell couples channels (matrix-vector products), so a chunk is one
//     workgroup holding all D channels of L consecutive steps in LDS;
//   * the Jacobian of every matrix cell is a diagonal plus row-scaled copies
//     of the recurrent weight matrices:
//         tanh RNN: A_t = diag(1 - v^2) W
//         GRU     : A_t = diag(z) + diag(cz) W_hz + diag(cn) W_hn + diag(cr) W_hr
//         Euler   : A_t = diag(1 - h) + diag(h (1 - g^2)) W,  g = tanh(W p + U x + b)
//       (the explicit Euler step p + h (g - p) of ds/dt = -s + tanh(...))
//     so only D-vectors of coefficients per step are kept; the diagonal
//     modes use the diagonal of A_t (quasi-Newton [PN §2.2.1]), 1 (Picard) or
//     0 (Jacobi), and Newton uses A_t itself;
//   * the banded mode [PN §2.2.2] keeps the entries |i - k| <= band of A_t.
//     Row scaling keeps a band in place, so band(A_t) is the same sum with
//     every W restricted to the band: each product below only runs over the
//     2 band + 1 columns k of row i (Newton is band >= D);
//   * for Newton and the banded mode the chunk map is (prod A~_t, folded
//     offset), a D x D matrix chain [PN §2.1] (a product of banded factors
//     fills in, so the map itself is kept dense), and the replay is a
//     matrix-vector chain.
// The input projection U x_t (+ bias) does not depend on the iterate and is
// computed once per sweep.  D is padded to DP (a power of two <= 64) inside
// LDS; padded rows/columns are kept at zero.  For DP a multiple of 16 the
// cell is evaluated from matrix-core accumulators with the weights in
// registers (CellRegs).  In the diagonal modes with few chunks per window a
// sweep composes its own carries from the chunk maps and, with consecutive
// windows, takes its own check (CellArgs::fc), so an iteration is one launch.

#include "pn_device.hpp"
#include "pn_launch.hpp"

namespace pn {

constexpr int kCellTanhRnn = 1;
constexpr int kCellGru = 2;
constexpr int kCellEuler = 3;

template <int CELL> struct CellTraits;
template <> struct CellTraits<kCellTanhRnn> { static constexpr int NG = 1, NCO = 1; };
template <> struct CellTraits<kCellGru> { static constexpr int NG = 3, NCO = 4; };
template <> struct CellTraits<kCellEuler> { static constexpr int NG = 1, NCO = 2; };

__host__ __device__ size_t prepared_weight_floats(int kind, int DP, int m) {
    if (kind == kCellTanhRnn) return static_cast<size_t>(DP) * DP + static_cast<size_t>(m) * DP + 2 * DP;
    if (kind == kCellEuler) return static_cast<size_t>(DP) * DP + static_cast<size_t>(m) * DP + 3 * DP;
    return 3ull * DP * DP + 3ull * m * DP + 9ull * DP;
}

// Offset (a multiple of 4 floats) of the k-contiguous copy: WK[g][i][k] =
// WT[g][k][i] (DP x DP per gate), then UK[g][i][q] = UT[g][q][i] for
// q < m, 0 up to the row length K16 = m rounded up to 16.
__host__ __device__ inline size_t kcopy_offset(int kind, int DP, int m) {
    return (prepared_weight_floats(kind, DP, m) + 3) & ~size_t(3);
}

__host__ __device__ size_t prepared_total_floats(int kind, int DP, int m) {
    if (DP % 16 != 0) return prepared_weight_floats(kind, DP, m);
    const size_t NG = kind == kCellGru ? 3 : 1, K16 = (m + 15) & ~15;
    return kcopy_offset(kind, DP, m) + NG * DP * DP + NG * DP * K16;
}

// ---------------------------------------------------------------- weight prep
// tanh RNN: WT[k][i] = W[i][k] | UT[q][i] = U[i][q] | bias[i] | wdiag[i]
// Euler   : the tanh RNN layout, then h[i]
// GRU     : WhT[g][k][i] = W_hh[gD+i][k] | WiT[g][q][i] = W_ih[gD+i][q] |
//           bih[g][i] | bhh[g][i] | whdiag[g][i] = W_hh[gD+i][i]
__global__ __launch_bounds__(kThreads) void prep_weights_kernel(int kind, const float* __restrict__ p,
                                                                 float* __restrict__ w, int D, int DP,
                                                                 int m, int n) {
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) {
        float val = 0.0f;
        if (kind == kCellTanhRnn || kind == kCellEuler) {
            const float* W = p;
            const float* U = p + D * D;
            const float* bb = U + D * m;
            const float* hh = bb + D;
            if (e < DP * DP) {
                const int k = e / DP, i = e % DP;
                if (i < D && k < D) val = W[i * D + k];
            } else if (e < DP * DP + m * DP) {
                const int f = e - DP * DP, q = f / DP, i = f % DP;
                if (i < D) val = U[i * m + q];
            } else if (e < DP * DP + m * DP + DP) {
                const int i = e - DP * DP - m * DP;
                if (i < D) val = bb[i];
            } else if (e < DP * DP + m * DP + 2 * DP) {
                const int i = e - DP * DP - m * DP - DP;
                if (i < D) val = W[i * D + i];
            } else {
                const int i = e - DP * DP - m * DP - 2 * DP;
                if (i < D) val = hh[i];
            }
        } else {
            const float* Wih = p;
            const float* Whh = p + 3 * D * m;
            const float* bih = Whh + 3 * D * D;
            const float* bhh = bih + 3 * D;
            const int s1 = 3 * DP * DP, s2 = s1 + 3 * m * DP, s3 = s2 + 3 * DP, s4 = s3 + 3 * DP;
            if (e < s1) {
                const int g = e / (DP * DP), r = e % (DP * DP), k = r / DP, i = r % DP;
                if (i < D && k < D) val = Whh[(g * D + i) * D + k];
            } else if (e < s2) {
                const int f = e - s1, g = f / (m * DP), r = f % (m * DP), q = r / DP, i = r % DP;
                if (i < D) val = Wih[(g * D + i) * m + q];
            } else if (e < s3) {
                const int f = e - s2, g = f / DP, i = f % DP;
                if (i < D) val = bih[g * D + i];
            } else if (e < s4) {
                const int f = e - s3, g = f / DP, i = f % DP;
                if (i < D) val = bhh[g * D + i];
            } else {
                const int f = e - s4, g = f / DP, i = f % DP;
                if (i < D) val = Whh[(g * D + i) * D + i];
            }
        }
        w[e] = val;
    }
}

// The k-contiguous copy (prepared_total_floats), from the prepared layout
// written by prep_weights_kernel.
__global__ __launch_bounds__(kThreads) void prep_kcopy_kernel(int kind, float* __restrict__ w, int DP, int m,
                                                              int n) {
    const int NG = kind == kCellGru ? 3 : 1, K16 = (m + 15) & ~15;
    const float* WT = w;
    const float* UT = w + NG * DP * DP;
    float* WK = w + kcopy_offset(kind, DP, m);
    float* UK = WK + NG * DP * DP;
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) {
        if (e < NG * DP * DP) {
            const int g = e / (DP * DP), r = e % (DP * DP), i = r / DP, k = r % DP;
            WK[e] = WT[(g * DP + k) * DP + i];
        } else {
            const int f = e - NG * DP * DP, g = f / (DP * K16), r = f % (DP * K16), i = r / K16, q = r % K16;
            UK[f] = q < m ? UT[(g * m + q) * DP + i] : 0.0f;
        }
    }
}

hipError_t launch_prep_weights(int kind, const float* params, float* w, int D, int DP, int m, bool with_kcopy,
                               hipStream_t st) {
    const int n = static_cast<int>(prepared_weight_floats(kind, DP, m));
    const int blocks = std::min((n + kThreads - 1) / kThreads, 1024);
    prep_weights_kernel<<<blocks, kThreads, 0, st>>>(kind, params, w, D, DP, m, n);
    if (with_kcopy && DP % 16 == 0) {
        const int nk = static_cast<int>(prepared_total_floats(kind, DP, m) - kcopy_offset(kind, DP, m));
        prep_kcopy_kernel<<<std::min((nk + kThreads - 1) / kThreads, 1024), kThreads, 0, st>>>(kind, w, DP, m, nk);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- cell evaluation
typedef float v4f __attribute__((ext_vector_type(4)));

// C[j][o] = sum_{k<K} A[j][k] * bval(k, o) for rows j < nrows and columns
// o < NO (a multiple of 16), on the matrix cores: 16 x 16 output tiles of
// 16x16x4 FP32 MFMA steps, tiles spread over the workgroup's wavefronts.
// A is an LDS array of row stride lda, zero-padded to K (a multiple of 4).
// Lane layout of one step: A[l % 16][l / 16], B[l / 16][l % 16];
// the accumulator holds C[4 (l / 16) + r][l % 16], r < 4.
template <int KC, typename BFun>
__device__ __forceinline__ void rows_gemm(const float* A, int lda, int nrows, int K, int NO, BFun bval,
                                          float* C, int ldc) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c16 = lane & 15, kq = lane >> 4;
    const int RT = (nrows + 15) >> 4, CT = NO >> 4;
    const int KK = KC > 0 ? KC : K;
    for (int t = wave; t < RT * CT; t += kThreads / 64) {
        const int rt = t / CT, ct = t - rt * CT;
        const int row = rt * 16 + c16;
        const int col = ct * 16 + c16;
        const float* Ar = A + (row < nrows ? row : 0) * lda + kq;
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
        for (int k0 = 0; k0 < KK; k0 += 4) {
            const float a = row < nrows ? Ar[k0] : 0.0f;
            const float b = bval(k0 + kq, col);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int orow = rt * 16 + kq * 4 + r;
            if (orow < nrows) C[orow * ldc + col] = acc[r];
        }
    }
}

// The same product for K a multiple of 16, with the wavefronts on fixed
// column tiles: WC wavefront columns share the CT = NO / 16 column tiles
// (tile ct belongs to column ct % WC) and 4 / WC wavefront rows take the row
// tiles in turn.  Each lane loads its A values one float4 per 16 k and uses
// every load for all of its wavefront's column tiles.  The sum runs over k in
// a permuted order: in k block g, MFMA step s takes k = 16 g + 4 (l / 16) + s
// in lane l, for A and B alike.  With A's row stride lda = 4 (mod 8) floats
// (or 4 (mod 32) for 16-float rows) the 16 rows of one float4 load fall on
// distinct LDS banks.  A must be 16-byte aligned, lda a multiple of 4, and
// columns K of every row readable.
template <int NO, typename BFun>
__device__ __forceinline__ void rows_gemm16(const float* A, int lda, int nrows, int K, BFun bval,
                                            float* C, int ldc) {
    constexpr int CT = NO / 16;
    constexpr int NWAVE = kThreads / 64;
    constexpr int WC = CT % 4 == 0 ? 4 : (CT % 2 == 0 ? 2 : 1);
    constexpr int WR = NWAVE / WC;
    constexpr int NT = CT / WC;                       // column tiles per wavefront
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c16 = lane & 15, kq = lane >> 4;
    const int wc = wave % WC, wr = wave / WC;
    const int RT = (nrows + 15) >> 4;
    for (int rt = wr; rt < RT; rt += WR) {
        const int row = rt * 16 + c16;
        const bool rin = row < nrows;
        const float* Ar = A + (rin ? row : 0) * lda + 4 * kq;
        v4f acc[NT];
#pragma unroll
        for (int q = 0; q < NT; ++q) acc[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
        for (int g = 0; g < K; g += 16) {
            const float4 a4 = rin ? *reinterpret_cast<const float4*>(Ar + g) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k = g + 4 * kq + s;
#pragma unroll
                for (int q = 0; q < NT; ++q) {
                    const int col = (wc + q * WC) * 16 + c16;
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bval(k, col), acc[q], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < NT; ++q) {
            const int col = (wc + q * WC) * 16 + c16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int orow = rt * 16 + kq * 4 + r;
                if (orow < nrows) C[orow * ldc + col] = acc[q][r];
            }
        }
    }
}

// LDS row strides of the cell tile: the iterate rows (P, N) and the staged x
// rows carry 4 floats of padding (see rows_gemm16); x rows are zero-filled
// to a multiple of 16 columns.
template <int DP>
__host__ __device__ constexpr int iterate_stride() { return DP + 4; }
__host__ __device__ inline int x_stride(int m) { return ((m + 15) & ~15) + 4; }

// Columns of the gate pre-activation tables: NG gates of DP rows, padded to 16.
template <int CELL, int DP>
struct Gates {
    static constexpr int NG = CellTraits<CELL>::NG;
    static constexpr int NO = (NG * DP + 15) & ~15;
};

// Input projection XI[j][g*DP + i] = sum_q W_ig[i][q] x_j[q] (no bias), for the
// staged x rows X (row stride x_stride(m), zero beyond column m).
template <int CELL, int DP>
__device__ __forceinline__ void input_projection(const float* __restrict__ w, const float* X, int xs,
                                                 int Lc, int m, float* XI) {
    constexpr int NG = CellTraits<CELL>::NG, NO = Gates<CELL, DP>::NO;
    const float* UT = w + NG * DP * DP;
    rows_gemm16<NO>(X, xs, Lc, (m + 15) & ~15, [&](int q, int o) {
        const int gte = o / DP, i = o - gte * DP;
        return (gte < NG && q < m) ? UT[(gte * m + q) * DP + i] : 0.0f;
    }, XI, NO);
}

// For rows j < Lc of a chunk with p_t = Pin[j] (the state one step earlier;
// row stride iterate_stride<DP>()):
// V[j] = f_t(p_t) and the Jacobian coefficients CO.  The recurrent products
// W_g p_t go through the matrix cores into H (LDS); the gate nonlinearities
// are per element.  If Sres is given, also folds |Sres[j+1] - V[j]| (the
// residual of the trajectory held in Sres) into rb and, if fb is given, the
// first row j whose residual is not <= tol into *fb.  Callers synchronise
// the workgroup before and after.
template <int CELL, int DP, bool DENSE>
__device__ __forceinline__ void eval_rows(const float* __restrict__ w, const float* Pin,
                                          const float* XI, float* H, float* V, float* CO, int Lc,
                                          int L, int D, int m, int mode, const float* Sres,
                                          uint32_t& rb, uint32_t* fb = nullptr, float tol = 0.0f) {
    constexpr int NG = CellTraits<CELL>::NG, NO = Gates<CELL, DP>::NO;
    constexpr int NRG = kThreads / DP;
    constexpr int PS = iterate_stride<DP>();
    auto wval = [&](int k, int o) {
        const int gte = o / DP, i = o - gte * DP;
        return gte < NG ? w[(gte * DP + k) * DP + i] : 0.0f;
    };
    if constexpr (DP % 16 == 0) rows_gemm16<NO>(Pin, PS, Lc, DP, wval, H, NO);
    else rows_gemm<DP>(Pin, PS, Lc, DP, NO, wval, H, NO);
    __syncthreads();
    const int i = threadIdx.x % DP;
    const bool live = i < D;
    const float* bi = w + NG * DP * DP + NG * m * DP;     // input biases
    for (int j = threadIdx.x / DP; j < Lc; j += NRG) {
        const int o = j * DP + i;
        if (!live) {
            V[o] = 0.0f;
            if constexpr (DENSE) {
#pragma unroll
                for (int q = 0; q < CellTraits<CELL>::NCO; ++q) CO[q * L * DP + o] = 0.0f;
            } else {
                CO[o] = 0.0f;
            }
            continue;
        }
        const float* hj = H + j * NO;
        const float* xj = XI + j * NO;
        float v;
        if constexpr (CELL == kCellTanhRnn) {
            const float* wdiag = bi + DP;
            v = tanh_f(hj[i] + xj[i] + bi[i]);
            const float c1 = 1.0f - v * v;
            if constexpr (DENSE) {
                CO[o] = c1;
            } else {
                CO[o] = mode == kJacobi ? 0.0f : (mode == kPicard ? 1.0f : c1 * wdiag[i]);
            }
        } else if constexpr (CELL == kCellEuler) {
            const float* wdiag = bi + DP;
            const float hi = bi[2 * DP + i];
            const float gv = tanh_f(hj[i] + xj[i] + bi[i]);
            const float pi = Pin[j * PS + i];
            v = pi + hi * (gv - pi);
            const float c1 = hi * (1.0f - gv * gv);
            if constexpr (DENSE) {
                CO[o] = 1.0f - hi;
                CO[L * DP + o] = c1;
            } else {
                CO[o] = mode == kJacobi ? 0.0f : (mode == kPicard ? 1.0f : (1.0f - hi) + c1 * wdiag[i]);
            }
        } else {
            const float* bhh = bi + 3 * DP;
            const float* whd = bhh + 3 * DP;
            const float rr = sigmoid_f(xj[i] + bi[i] + hj[i] + bhh[i]);
            const float z = sigmoid_f(xj[DP + i] + bi[DP + i] + hj[DP + i] + bhh[DP + i]);
            const float gg = hj[2 * DP + i] + bhh[2 * DP + i];
            const float n = tanh_f(xj[2 * DP + i] + bi[2 * DP + i] + rr * gg);
            const float pi = Pin[j * PS + i];
            v = (1.0f - z) * n + z * pi;
            const float dn = (1.0f - z) * (1.0f - n * n);
            const float cz = (pi - n) * z * (1.0f - z);
            const float cn = dn * rr;
            const float cr = dn * gg * rr * (1.0f - rr);
            if constexpr (DENSE) {
                CO[o] = z;
                CO[L * DP + o] = cz;
                CO[2 * L * DP + o] = cn;
                CO[3 * L * DP + o] = cr;
            } else {
                const float jd = z + cz * whd[DP + i] + cn * whd[2 * DP + i] + cr * whd[i];
                CO[o] = mode == kJacobi ? 0.0f : (mode == kPicard ? 1.0f : jd);
            }
        }
        V[o] = v;
        if (Sres) {
            const float d = Sres[(j + 1) * PS + i] - v;
            rb = max(rb, abs_bits(d));
            if (fb && !(fabsf(d) <= tol)) *fb = min(*fb, static_cast<uint32_t>(j));
        }
    }
}

// (A~_t y)[i] for the dense or banded Jacobian, with y in LDS; row i only.
template <int CELL, int DP>
__device__ __forceinline__ float jac_row_apply(const float* __restrict__ w, const float* CO, int o,
                                               int L, int i, int D, int band, const float* y) {
    constexpr int NG = CellTraits<CELL>::NG;
    float acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = 0.0f;
    const int k1 = min(D, i + band + 1);
    for (int k = max(0, i - band); k < k1; ++k) {
        const float yk = y[k];
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g] += w[(g * DP + k) * DP + i] * yk;
    }
    if constexpr (CELL == kCellTanhRnn) {
        return CO[o] * acc[0];
    } else if constexpr (CELL == kCellEuler) {
        return CO[o] * y[i] + CO[L * DP + o] * acc[0];
    } else {
        return CO[o] * y[i] + CO[L * DP + o] * acc[1] + CO[2 * L * DP + o] * acc[2] +
               CO[3 * L * DP + o] * acc[0];
    }
}

// ---------------------------------------------------------------- register-resident evaluation
// For DP a multiple of 16 the cell is evaluated from the matrix-core
// accumulators.  Wavefront (wc, wr) of the workgroup, wc = wave % WC with
// WC = DP / 16, owns the state indices i = 16 wc + l % 16 (lane l) of every
// gate; wr = wave / WC takes the row tiles rt = wr, wr + WR, ... of the chunk.
// Accumulator g of a lane then holds gate g's pre-activation at rows
// 16 rt + 4 (l / 16) + r, r < 4, and index i, so the gate nonlinearities run
// on registers, and the input projection (with the biases folded in) stays in
// registers for both evaluations of a sweep.  The recurrent weights are the
// B operand, held in registers; the sums over k run in the permuted order of
// rows_gemm16.  Chunks are at most kMaxChunk steps.
constexpr int kMaxChunk = 64;

template <int CELL, int DP, int MAXC = kMaxChunk>
struct CellRegs {
    static constexpr int NG = CellTraits<CELL>::NG;
    static constexpr int WC = DP / 16;
    static constexpr int WR = (kThreads / 64) / WC;
    static constexpr int MAXRT = (MAXC / 16 + WR - 1) / WR;        // row tiles per wavefront
    static constexpr int KB = DP / 4;                              // B values per gate and lane
    static constexpr int PS = iterate_stride<DP>();
    static constexpr int KIN = DP;                                 // input widths held in registers
    int i, wr, kq;
    bool live;
    float wb[NG][KB];
    float ub[NG][KIN / 4];       // input weights, B operand (m <= KIN)
    v4f xi[MAXRT][NG];
    // per-index constants (biases, diagonals), kept as loaded: a use right
    // after the load would wait for every load issued before it
    float c0, c0b, c1, c1b, c2, c3, c4, c5, c6;

    // Weights: w the prepared layout (LDS or global), wg the whole prepared
    // region in global memory (its k-contiguous copy: one float4 per lane and
    // 16 k).
    __device__ __forceinline__ void load(const float* __restrict__ w, const float* __restrict__ wg, int D, int m) {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        i = (wave % WC) * 16 + (lane & 15);
        wr = wave / WC;
        kq = lane >> 4;
        live = i < D;
        const float* WK = wg + kcopy_offset(CELL, DP, m);
        const int K16 = (m + 15) & ~15;
        const float* UK = WK + NG * DP * DP;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
#pragma unroll
            for (int kb = 0; kb < DP / 16; ++kb) {
                const float4 v = *reinterpret_cast<const float4*>(WK + (g * DP + i) * DP + 16 * kb + 4 * kq);
                wb[g][kb * 4 + 0] = v.x;
                wb[g][kb * 4 + 1] = v.y;
                wb[g][kb * 4 + 2] = v.z;
                wb[g][kb * 4 + 3] = v.w;
            }
        }
        if (m <= KIN) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
#pragma unroll
                for (int kb = 0; kb < KIN / 16; ++kb) {
                    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    if (kb * 16 < K16) v = *reinterpret_cast<const float4*>(UK + (g * DP + i) * K16 + 16 * kb + 4 * kq);
                    ub[g][kb * 4 + 0] = v.x;
                    ub[g][kb * 4 + 1] = v.y;
                    ub[g][kb * 4 + 2] = v.z;
                    ub[g][kb * 4 + 3] = v.w;
                }
            }
        }
        const float* bi = w + NG * DP * DP + NG * m * DP;
        if constexpr (CELL == kCellGru) {
            c0 = bi[i];                                  // b_ir (+ b_hr)
            c0b = bi[3 * DP + i];
            c1 = bi[DP + i];                             // b_iz (+ b_hz)
            c1b = bi[4 * DP + i];
            c2 = bi[2 * DP + i];                         // b_in
            c3 = bi[5 * DP + i];                         // b_hn
            c4 = bi[6 * DP + i];                         // diag W_hr
            c5 = bi[7 * DP + i];                         // diag W_hz
            c6 = bi[8 * DP + i];                         // diag W_hn
        } else {
            c0 = bi[i];                                  // b
            c4 = bi[DP + i];                             // diag W
            if constexpr (CELL == kCellEuler) c5 = bi[2 * DP + i];   // h
        }
    }

    // Input projection of the staged x rows X (row stride xs, zero beyond
    // column m) plus the biases that add to it.
    __device__ __forceinline__ void project(const float* __restrict__ w, const float* X, int xs, int Lc, int m) {
        const float* UT = w + NG * DP * DP;
        const int RT = (Lc + 15) >> 4;
        const int K = (m + 15) & ~15;
#pragma unroll
        for (int u = 0; u < MAXRT; ++u) {
            const int rt = wr + WR * u;
            if (rt >= RT) break;
            const int row = rt * 16 + (threadIdx.x & 15);
            const bool rin = row < Lc;
            const float* Ar = X + (rin ? row : 0) * xs + 4 * kq;
            v4f acc[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            if (m <= KIN) {
                // B from the registers loaded with the recurrent weights
#pragma unroll
                for (int kb = 0; kb < KIN / 16; ++kb) {
                    if (kb * 16 >= K) break;
                    const float4 a4 = rin ? *reinterpret_cast<const float4*>(Ar + 16 * kb) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
#pragma unroll
                        for (int g = 0; g < NG; ++g)
                            acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], ub[g][kb * 4 + s], acc[g], 0, 0, 0);
                    }
                }
            } else {
#pragma unroll 4
                for (int q0 = 0; q0 < K; q0 += 16) {
                    const float4 a4 = rin ? *reinterpret_cast<const float4*>(Ar + q0) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int q = q0 + 4 * kq + s;
#pragma unroll
                        for (int g = 0; g < NG; ++g) {
                            const float b = q < m ? UT[(g * m + q) * DP + i] : 0.0f;
                            acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], b, acc[g], 0, 0, 0);
                        }
                    }
                }
            }
            if constexpr (CELL == kCellGru) {
                xi[u][0] = acc[0] + (c0 + c0b);
                xi[u][1] = acc[1] + (c1 + c1b);
                xi[u][2] = acc[2] + c2;
            } else {
                xi[u][0] = acc[0] + c0;
            }
        }
    }

    // V[j] = f_t(p_t), p_t = Pin[j] (row stride PS), and the Jacobian
    // coefficients CO for rows j < Lc; with Sres, the residual of the
    // trajectory held there (as eval_rows).
    template <bool DENSE>
    __device__ __forceinline__ void eval(const float* Pin, float* V, float* CO, int Lc, int L, int mode,
                                         const float* Sres, uint32_t& rb, uint32_t* fb, float tol) const {
        const int RT = (Lc + 15) >> 4;
#pragma unroll
        for (int u = 0; u < MAXRT; ++u) {
            const int rt = wr + WR * u;
            if (rt >= RT) break;
            const int row = rt * 16 + (threadIdx.x & 15);
            const bool rin = row < Lc;
            const float* Ar = Pin + (rin ? row : 0) * PS + 4 * kq;
            v4f acc[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[g] = xi[u][g];
            if constexpr (CELL == kCellGru) acc[2] = v4f{c3, c3, c3, c3};   // W_hn p + b_hn alone
#pragma unroll
            for (int kb = 0; kb < DP / 16; ++kb) {
                const float4 a4 = rin ? *reinterpret_cast<const float4*>(Ar + 16 * kb) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        acc[g] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], wb[g][kb * 4 + s], acc[g], 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = rt * 16 + 4 * kq + r;
                if (j >= Lc) continue;
                const int o = j * DP + i;
                if (!live) {
                    V[o] = 0.0f;
                    if constexpr (DENSE) {
#pragma unroll
                        for (int q = 0; q < CellTraits<CELL>::NCO; ++q) CO[q * L * DP + o] = 0.0f;
                    } else {
                        CO[o] = 0.0f;
                    }
                    continue;
                }
                float v;
                if constexpr (CELL == kCellTanhRnn) {
                    v = tanh_f(acc[0][r]);
                    const float d1 = 1.0f - v * v;
                    if constexpr (DENSE) CO[o] = d1;
                    else CO[o] = mode == kJacobi ? 0.0f : (mode == kPicard ? 1.0f : d1 * c4);
                } else if constexpr (CELL == kCellEuler) {
                    const float gv = tanh_f(acc[0][r]);
                    const float pi = Pin[j * PS + i];
                    v = pi + c5 * (gv - pi);
                    const float d1 = c5 * (1.0f - gv * gv);
                    if constexpr (DENSE) {
                        CO[o] = 1.0f - c5;
                        CO[L * DP + o] = d1;
                    } else {
                        CO[o] = mode == kJacobi ? 0.0f : (mode == kPicard ? 1.0f : (1.0f - c5) + d1 * c4);
                    }
                } else {
                    const float rr = sigmoid_f(acc[0][r]);
                    const float z = sigmoid_f(acc[1][r]);
                    const float gg = acc[2][r];
                    const float n = tanh_f(xi[u][2][r] + rr * gg);
                    const float pi = Pin[j * PS + i];
                    v = (1.0f - z) * n + z * pi;
                    const float dn = (1.0f - z) * (1.0f - n * n);
                    const float cz = (pi - n) * z * (1.0f - z);
                    const float cn = dn * rr;
                    const float cr = dn * gg * rr * (1.0f - rr);
                    if constexpr (DENSE) {
                        CO[o] = z;
                        CO[L * DP + o] = cz;
                        CO[2 * L * DP + o] = cn;
                        CO[3 * L * DP + o] = cr;
                    } else {
                        const float jd = z + cz * c5 + cn * c6 + cr * c4;
                        CO[o] = mode == kJacobi ? 0.0f : (mode == kPicard ? 1.0f : jd);
                    }
                }
                V[o] = v;
                if (Sres) {
                    const float d = Sres[(j + 1) * PS + i] - v;
                    rb = max(rb, abs_bits(d));
                    if (fb && !(fabsf(d) <= tol)) *fb = min(*fb, static_cast<uint32_t>(j));
                }
            }
        }
    }
};

// ---------------------------------------------------------------- the fused pass
// One tile (batch row b, chunk c) of one sweep.  `arr` is the LDS array
// region, `w` the prepared weights (LDS or global).  Returns the tile's
// residual bit-max through rb (the caller reduces it over the workgroup).
// Returns false when the sweep's own check (CellArgs::fc) stops the loop:
// the tile then writes nothing.
template <int CELL, int DP, bool DENSE, int PHASE>
__device__ __forceinline__ bool cell_tile(const CellArgs& g, int c, int b, float* arr,
                                          const float* w, uint32_t& rb, uint32_t* fb = nullptr) {
    constexpr int NG = CellTraits<CELL>::NG;
    constexpr int NCO = DENSE ? CellTraits<CELL>::NCO : 1;
    const int L = g.L, m = g.m, D = g.D;
    const int t0 = c * L;
    const int Lc = min(L, g.Tw - t0);
    const int tid = threadIdx.x;
    constexpr int NO = Gates<CELL, DP>::NO;
    constexpr int PS = iterate_stride<DP>();
    constexpr bool kRegs = DP % 16 == 0;     // register-resident evaluation (CellRegs)
    const int xs = x_stride(m);
    const int nxh = kRegs ? 0 : L * NO;
    float* P = arr;                          // [L+1][PS] rows t0-1 .. t1-1 of s^(i)
    float* N = P + (L + 1) * PS;             // [L+1][PS] the same rows of s^(i+1)
    float* XI = N + (L + 1) * PS;            // [L][NO] input projections (not with kRegs)
    float* H = XI + nxh;                     // [L][NO] recurrent pre-activations (not with kRegs)
    float* V = H + nxh;
    float* CO = V + L * DP;
    float* X = CO + NCO * L * DP;            // [L][xs]
    float* DL = X + L * xs;
    float* SCR = DL + DP;                    // [2][kThreads] carry segments (fc, diagonal modes)
    const size_t ci = static_cast<size_t>(b) * g.NC + c;        // chunk index
    const float* s0 = g.s0 + b * g.s0s;
    CellRegs<CELL, kRegs ? DP : 16> cr16;    // used when kRegs
    auto evaluate = [&](const float* Pin, const float* Sres, uint32_t* fbp) {
        if constexpr (kRegs) cr16.template eval<DENSE>(Pin, V, CO, Lc, L, g.mode, Sres, rb, fbp, g.tol);
        else eval_rows<CELL, DP, DENSE>(w, Pin, XI, H, V, CO, Lc, L, D, m, g.mode, Sres, rb, fbp, g.tol);
    };

    // ---- stage inputs: X rows and the rows of the iterate the sweep starts
    // from, with one wait; the carries of this chunk and the next (apply
    // sweeps) are fetched first, for the replay
    constexpr bool kApply = PHASE != kPrologue && PHASE != kMaps;
    const float* xg = g.x + b * g.xs + static_cast<int64_t>(t0) * m;
    const size_t HS = static_cast<size_t>(g.B) * g.NC * D;
    const bool has_next = c + 1 < g.NC;
    float c_first = 0.0f, c_next = 0.0f;
    // fc: r_i as the sweep before reduced it (every wavefront reads the
    // slots; reduced after the staging wait) and the control word
    uint32_t r_raw = 0;
    int stop_before = 0;
    const float* mA = g.aggA + (g.iter & 1) * g.mstride + static_cast<size_t>(b) * g.NC * D;
    const float* mB = g.aggB + (g.iter & 1) * g.mstride + static_cast<size_t>(b) * g.NC * D;
    float own_a = 0.0f, own_b = 0.0f;
    // fc: the chunk maps this thread folds, loaded before the staging loads
    // go out so that one memory round trip covers both (kFold per thread;
    // longer segments finish after staging)
    constexpr int kFold = (kFcMaxChunks + kThreads / DP - 1) / (kThreads / DP) < 16
                              ? (kFcMaxChunks + kThreads / DP - 1) / (kThreads / DP) : 16;
    float pa[kFold], pb[kFold];
    int k0 = 0, k1 = 0;
    if constexpr (kApply && !DENSE) {
        if (g.fc & kFcCheck) {
            const int lane = tid & 63;
            r_raw = lane < kRSlots ? g.ctrl->rmax[g.iter % 3][lane][0] : 0u;
            stop_before = g.ctrl->stop;
        }
        if (g.fc & kFcCarry) {
            // The carry of chunk c, composed here from the chunk maps of
            // iteration i: kThreads / DP segments of the chunks before c are
            // each folded into one affine map, then applied to s0 in order
            // (after the staging wait); the next chunk's carry is this
            // chunk's map applied to it.
            constexpr int NS = kThreads / DP;
            const int d = tid % DP, sg_ = tid / DP;
            const int per = (c + NS - 1) / NS;
            k0 = min(c, sg_ * per);
            k1 = d < D ? min(c, k0 + per) : k0;
#pragma unroll
            for (int u = 0; u < kFold; ++u) {
                const int k = k0 + u;
                pa[u] = k < k1 ? mA[k * D + d] : 1.0f;      // padding: the identity map
                pb[u] = k < k1 ? mB[k * D + d] : 0.0f;
            }
            if (tid < D && has_next) {
                own_a = mA[c * D + tid];
                own_b = mB[c * D + tid];
            }
        } else if (tid < D) {
            c_first = g.carry[ci * D + tid];
            if (has_next) c_next = g.carry[(ci + 1) * D + tid];
        }
    } else if (kApply && tid < D) {
        c_first = g.carry[ci * D + tid];
        if (has_next) c_next = g.carry[(ci + 1) * D + tid];
    }
    if constexpr (kRegs) cr16.load(w, g.w, D, m);
    copy_rows_to_lds<kThreads>(X, xs, xg, m, Lc, m);
    float* sg = g.s + b * g.ss + static_cast<int64_t>(t0) * D;
    if constexpr (PHASE == kPrologue) {
        // s^(0) = s0 everywhere: N holds rows t0-1 .. t1-1 of s^(0).
        for (int e = tid; e < (Lc + 1) * PS; e += kThreads) {
            const int i = e % PS;
            N[e] = i < D ? s0[i] : 0.0f;
        }
    } else if constexpr (PHASE == kMaps) {
        // N: rows t0-1 .. t1-1 of the iterate in s; its last row is the halo
        // the next apply reads.  Rows from ff on (window-relative) are new
        // steps: they start from the state before them, row ff-1 (or s0),
        // which this pass does not write, and are written to s here.
        const int ff = g.Tw - g.fill_rows;
        const float* sw = g.s + b * g.ss;                    // window row 0
        auto fillv = [&](int i) { return ff == 0 ? s0[i] : sw[static_cast<int64_t>(ff - 1) * D + i]; };
        if (tid < PS) N[tid] = tid < D ? (c == 0 ? s0[tid] : (t0 - 1 >= ff ? fillv(tid) : sg[tid - D])) : 0.0f;
        const int nld = max(0, min(Lc, ff - t0));           // rows already in s
        copy_rows_to_lds<kThreads>(N + PS, PS, sg, D, nld, D);
        for (int e = tid; e < (Lc - nld) * PS; e += kThreads) {
            const int j = nld + e / PS, i = e % PS;
            const float v = i < D ? fillv(i) : 0.0f;
            N[(j + 1) * PS + i] = v;
            if (i < D) sg[j * D + i] = v;
        }
    } else if constexpr (PHASE == kFirst) {
        // ---- P: rows t0-1 .. t1-1 of s^(i)
        for (int e = tid; e < (Lc + 1) * PS; e += kThreads) {
            const int i = e % PS;
            P[e] = i < D ? s0[i] : 0.0f;
        }
    } else {
        if (tid < PS) {
            P[tid] = tid < D ? ((c == 0) ? s0[tid] : g.halo[(g.iter & 1) * HS + (ci - 1) * D + tid]) : 0.0f;
        }
        copy_rows_to_lds<kThreads>(P + PS, PS, sg, D, Lc, D);
    }
    if constexpr (kApply && !DENSE) {
        if (g.fc & kFcCarry) {
            float fa = 1.0f, fbv = 0.0f;
#pragma unroll
            for (int u = 0; u < kFold; ++u) {
                fbv = pa[u] * fbv + pb[u];
                fa = pa[u] * fa;
            }
            for (int k = k0 + kFold; k < k1; ++k) {
                const int d = tid % DP;
                const float a = mA[k * D + d];
                fbv = a * fbv + mB[k * D + d];
                fa = a * fa;
            }
            SCR[tid] = fa;
            SCR[kThreads + tid] = fbv;
        }
    }
    __syncthreads();
    if constexpr (PHASE == kMaps) {
        if (tid < D) g.halo[(g.iter & 1) * HS + ci * D + tid] = N[Lc * PS + tid];
    }
    if constexpr (kApply && !DENSE) {
        if (g.fc & kFcCheck) {
            // the loop stopped at an earlier check: this launch was queued ahead
            if (stop_before) return false;
            // the check of iteration i, taken alike by every workgroup; block
            // 0 publishes it and clears the slot set of the sweep after next
            const uint32_t r_i = wave_max_u32(r_raw);
            CheckArgs chk{};
            chk.iter = g.iter;
            chk.max_iter = g.max_iter;
            chk.tol = g.tol;
            chk.ctrl = g.ctrl;
            chk.host = g.host + g.iter % kHostRing;
            chk.epoch = g.epoch;
            const int st = check_status(r_i, chk);
            if (c == 0 && b == 0) {
                if (tid < kRSlots)
                    __hip_atomic_store(&g.ctrl->rmax[(g.iter + 2) % 3][tid][0], 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                if (tid == 0) publish_check(chk, r_i, st, 0xffffffffu);
            }
            if (st >= 0) return false;
        }
        if ((g.fc & kFcCarry) && tid < D) {
            // the folded segments applied to s0 in order
            constexpr int NS = kThreads / DP;
            float x = s0[tid];
#pragma unroll
            for (int q = 0; q < NS; ++q) x = SCR[q * DP + tid] * x + SCR[kThreads + q * DP + tid];
            c_first = x;
            if (has_next) c_next = own_a * x + own_b;
        }
    }
    // ---- the input projection (iterate-free)
    if constexpr (kRegs) cr16.project(w, X, xs, Lc, m);
    else input_projection<CELL, DP>(w, X, xs, Lc, m, XI);

    if constexpr (kApply) {
        // ---- maps of iteration i at p_t = P[j]
        evaluate(P, nullptr, nullptr);
        __syncthreads();
        // ---- replay from the carry, damping, N = rows t0-1 .. t1-1 of s^(i+1)
        const float lam = g.lam;
        const bool und = g.undamped != 0;
        if constexpr (!DENSE) {
            if (g.mode == kJacobi) {
                // A~ = 0: row j of s^ is v_{j-1} itself, so the rows are
                // independent of one another.  Row 0 (the carry) and, with a
                // successor, row Lc (that chunk's carry) come from the values
                // thread i holds for state i.
                const int jl = has_next ? Lc - 1 : Lc;       // rows 1 .. jl from V
                for (int e = tid; e < jl * PS; e += kThreads) {
                    const int j = 1 + e / PS, i = e % PS;
                    float val = 0.0f;
                    if (i < D) {
                        const float sh = V[(j - 1) * DP + i], so = P[j * PS + i];
                        val = und ? sh : so + lam * (sh - so);
                    }
                    N[j * PS + i] = val;
                }
                if (tid < PS) {
                    const bool lv = tid < D;
                    N[tid] = lv ? (und ? c_first : P[tid] + lam * (c_first - P[tid])) : 0.0f;
                    if (has_next) {
                        const float so = P[Lc * PS + tid];
                        N[Lc * PS + tid] = lv ? (und ? c_next : so + lam * (c_next - so)) : 0.0f;
                    }
                }
            } else if (tid < D) {
                float shat = c_first;
                N[tid] = und ? shat : P[tid] + lam * (shat - P[tid]);
                // the last row of a chunk that has a successor is that
                // chunk's carry
                const int nrep = has_next ? Lc - 1 : Lc;
                // eight steps at a time: their LDS loads go out together,
                // ahead of the stores of N (which the compiler cannot tell
                // apart from the arrays read)
                int j = 0;
                for (; j + 8 <= nrep; j += 8) {
                    float v[8], co[8], pj[9];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        v[u] = V[(j + u) * DP + tid];
                        co[u] = CO[(j + u) * DP + tid];
                        pj[u] = P[(j + u) * PS + tid];
                    }
                    pj[8] = P[(j + 8) * PS + tid];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        shat = v[u] + co[u] * (shat - pj[u]);
                        N[(j + u + 1) * PS + tid] = und ? shat : pj[u + 1] + lam * (shat - pj[u + 1]);
                    }
                }
                for (; j < nrep; ++j) {
                    const int o = j * DP + tid;
                    shat = V[o] + CO[o] * (shat - P[j * PS + tid]);
                    const float so = P[(j + 1) * PS + tid];
                    N[(j + 1) * PS + tid] = und ? shat : so + lam * (shat - so);
                }
                if (has_next) {
                    const float so = P[Lc * PS + tid];
                    N[Lc * PS + tid] = und ? c_next : so + lam * (c_next - so);
                }
            } else if (tid < PS) {
                for (int j = 0; j <= Lc; ++j) N[j * PS + tid] = 0.0f;
            }
        } else {
            float shat = 0.0f;
            if (tid < D) {
                shat = c_first;
                N[tid] = und ? shat : P[tid] + lam * (shat - P[tid]);
            } else if (tid < PS) {
                for (int j = 0; j <= Lc; ++j) N[j * PS + tid] = 0.0f;
                if (tid < DP) DL[tid] = 0.0f;
            }
            for (int j = 0; j < Lc; ++j) {
                const int o = j * DP + tid;
                if (tid < D) DL[tid] = shat - P[j * PS + tid];
                __syncthreads();
                if (tid < D) {
                    shat = V[o] + jac_row_apply<CELL, DP>(w, CO, o, L, tid, D, g.band, DL);
                    if (j == Lc - 1 && has_next) shat = c_next;
                    const float so = P[(j + 1) * PS + tid];
                    N[(j + 1) * PS + tid] = und ? shat : so + lam * (shat - so);
                }
                __syncthreads();
            }
        }
        __syncthreads();
        // ---- store s^(i+1) rows t0 .. t1-1 and the halo for the next chunk
        for (int e = tid; e < Lc * D; e += kThreads) {
            const int j = e / D, i = e % D;
            sg[e] = N[(j + 1) * PS + i];
        }
        if (tid < D) g.halo[((g.iter + 1) & 1) * HS + ci * D + tid] = N[Lc * PS + tid];
    }
    // ---- maps of iteration i+1 at the new iterate, and its residual
    evaluate(N, N, fb);
    __syncthreads();
    if constexpr (!DENSE) {
        if (tid < D && g.mode == kJacobi) {
            // A~ = 0: the chunk map is y -> v at the chunk's last step
            const size_t mo = (PHASE == kPrologue ? 0 : PHASE == kMaps ? (g.iter & 1) : ((g.iter + 1) & 1)) *
                              g.mstride;
            g.aggA[mo + ci * D + tid] = 0.0f;
            g.aggB[mo + ci * D + tid] = V[(Lc - 1) * DP + tid];
        } else if (tid < D) {
            float A = 1.0f, Bc = 0.0f;
#pragma unroll 8
            for (int j = 0; j < Lc; ++j) {
                const int o = j * DP + tid;
                const float at = CO[o];
                const float bt = V[o] - at * N[j * PS + tid];
                Bc = at * Bc + bt;
                A = at * A;
            }
            // the maps of iteration i+1 (of iteration 0 in the prologue; a
            // maps pass launched with iter i writes those of iteration i)
            const size_t mo = (PHASE == kPrologue ? 0 : PHASE == kMaps ? (g.iter & 1) : ((g.iter + 1) & 1)) *
                              g.mstride;
            g.aggA[mo + ci * D + tid] = A;
            g.aggB[mo + ci * D + tid] = Bc;
        }
    } else {
        // chunk map y -> M y + bg, built step by step: M <- A~_j M, bg <- A~_j (bg - p_j) + v_j.
        // M rows are padded to MS = DP + 1 floats: in the banded mode the
        // lanes of a wave read M at rows k that follow their own row i.
        constexpr int MS = DP + 1;
        float* M0 = DL + DP;
        float* M1 = M0 + DP * MS;
        float* B0 = M1 + DP * MS;
        float* B1 = B0 + DP;
        for (int e = tid; e < DP * MS; e += kThreads) {
            const int i = e / MS, k = e % MS;
            M0[e] = (i == k && i < D) ? 1.0f : 0.0f;
            M1[e] = 0.0f;
        }
        if (tid < DP) {
            B0[tid] = 0.0f;
            B1[tid] = 0.0f;
        }
        __syncthreads();
        constexpr int NCG = kThreads / DP;
        const int i = tid % DP;
        const int cg = tid / DP;
        const int k0 = max(0, i - g.band), k1 = min(D, i + g.band + 1);
        for (int j = 0; j < Lc; ++j) {
            const int o = j * DP + i;
            if (i < D) {
                for (int col = cg; col < D; col += NCG) {
                    float acc[NG];
#pragma unroll
                    for (int q = 0; q < NG; ++q) acc[q] = 0.0f;
                    for (int k = k0; k < k1; ++k) {
                        const float mk = M0[k * MS + col];
#pragma unroll
                        for (int q = 0; q < NG; ++q) acc[q] += w[(q * DP + k) * DP + i] * mk;
                    }
                    float val;
                    if constexpr (CELL == kCellTanhRnn) {
                        val = CO[o] * acc[0];
                    } else if constexpr (CELL == kCellEuler) {
                        val = CO[o] * M0[i * MS + col] + CO[L * DP + o] * acc[0];
                    } else {
                        val = CO[o] * M0[i * MS + col] + CO[L * DP + o] * acc[1] +
                              CO[2 * L * DP + o] * acc[2] + CO[3 * L * DP + o] * acc[0];
                    }
                    M1[i * MS + col] = val;
                }
                if (cg == 0) {
                    // offset: A~_j (bg - p_j) + v_j, p_j = N[j]
                    float acc[NG];
#pragma unroll
                    for (int q = 0; q < NG; ++q) acc[q] = 0.0f;
                    for (int k = k0; k < k1; ++k) {
                        const float yk = B0[k] - N[j * PS + k];
#pragma unroll
                        for (int q = 0; q < NG; ++q) acc[q] += w[(q * DP + k) * DP + i] * yk;
                    }
                    float val;
                    if constexpr (CELL == kCellTanhRnn) {
                        val = CO[o] * acc[0];
                    } else if constexpr (CELL == kCellEuler) {
                        val = CO[o] * (B0[i] - N[j * PS + i]) + CO[L * DP + o] * acc[0];
                    } else {
                        val = CO[o] * (B0[i] - N[j * PS + i]) + CO[L * DP + o] * acc[1] +
                              CO[2 * L * DP + o] * acc[2] + CO[3 * L * DP + o] * acc[0];
                    }
                    B1[i] = V[o] + val;
                }
            }
            __syncthreads();
            float* t = M0; M0 = M1; M1 = t;
            t = B0; B0 = B1; B1 = t;
        }
        float* aA = g.aggA + ci * D * D;
        for (int e = tid; e < D * D; e += kThreads) aA[e] = M0[(e / D) * MS + (e % D)];
        if (tid < D) g.aggB[ci * D + tid] = B0[tid];
    }
    return true;
}

template <int CELL, int DP, bool DENSE, int PHASE, bool STAGE>
__global__ __launch_bounds__(kThreads) void cell_pass(CellArgs g) {
    if constexpr (PHASE != kPrologue && PHASE != kMaps) {   // apply launches enqueued ahead
        if (!(g.fc & kFcCheck) && g.ctrl->stop) return;      // (else read with the staging loads)
    }
    extern __shared__ __attribute__((aligned(16))) float lds[];
    // the prepared weights are staged once per workgroup in LDS when they fit
    const int nw = STAGE ? static_cast<int>(prepared_weight_floats(CELL, DP, g.m)) : 0;
    copy_to_lds<kThreads>(lds, g.w, nw);
    const float* w = STAGE ? lds : g.w;
    uint32_t rb = 0, fb = 0xffffffffu;
    if (!cell_tile<CELL, DP, DENSE, PHASE>(g, blockIdx.x, blockIdx.y, lds + ((nw + 3) & ~3), w, rb,
                                           g.fpart ? &fb : nullptr))
        return;                               // the sweep's own check stopped the loop
    rb = block_max_u32(rb);
    const size_t blk = static_cast<size_t>(blockIdx.y) * g.NC + blockIdx.x;
    if (threadIdx.x == 0) {
        if (g.fc & kFcCheck) {
            const int set = PHASE == kPrologue ? 0 : (g.iter + 1) % 3;
            __hip_atomic_fetch_max(&g.ctrl->rmax[set][blk % kRSlots][0], rb, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
            g.rpart[blk] = rb;
        }
    }
    if (g.fpart) {
        fb = ~block_max_u32(~fb);
        if (threadIdx.x == 0) g.fpart[blk] = fb == 0xffffffffu ? fb : blockIdx.x * g.L + fb;
    }
}

template <int CELL, int DP, bool DENSE, int PHASE, bool STAGE>
static hipError_t launch_one(const CellArgs& a, size_t lds, hipStream_t st) {
    auto k = cell_pass<CELL, DP, DENSE, PHASE, STAGE>;
    if (lds > 64 * 1024) {   // opt in to a larger LDS allocation
        const hipError_t attr = hipFuncSetAttribute(
            reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (attr != hipSuccess) return attr;
    }
    return launch_maybe_timed(k, dim3(a.NC, a.B), dim3(kThreads), lds, st, a);
}

template <int CELL, int DP, bool DENSE>
static hipError_t launch_phase(int phase, const CellArgs& a, hipStream_t st) {
    const bool stage = cell_pass_stages_weights(CELL, DP, DENSE, a.L, a.m);
    const size_t lds = cell_pass_lds_bytes(CELL, DP, DENSE, a.L, a.m);
    if (stage) {
        if (phase == kPrologue) return launch_one<CELL, DP, DENSE, kPrologue, true>(a, lds, st);
        if (phase == kFirst) return launch_one<CELL, DP, DENSE, kFirst, true>(a, lds, st);
        if (phase == kMaps) return launch_one<CELL, DP, DENSE, kMaps, true>(a, lds, st);
        return launch_one<CELL, DP, DENSE, kSteady, true>(a, lds, st);
    }
    if (phase == kPrologue) return launch_one<CELL, DP, DENSE, kPrologue, false>(a, lds, st);
    if (phase == kFirst) return launch_one<CELL, DP, DENSE, kFirst, false>(a, lds, st);
    if (phase == kMaps) return launch_one<CELL, DP, DENSE, kMaps, false>(a, lds, st);
    return launch_one<CELL, DP, DENSE, kSteady, false>(a, lds, st);
}

template <int CELL, bool DENSE>
static hipError_t launch_dp(int DP, int phase, const CellArgs& a, hipStream_t st) {
    switch (DP) {
        case 4: return launch_phase<CELL, 4, DENSE>(phase, a, st);
        case 8: return launch_phase<CELL, 8, DENSE>(phase, a, st);
        case 16: return launch_phase<CELL, 16, DENSE>(phase, a, st);
        case 32: return launch_phase<CELL, 32, DENSE>(phase, a, st);
        case 64: return launch_phase<CELL, 64, DENSE>(phase, a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cell_pass(int kind, int DP, bool dense, int phase, const CellArgs& a,
                            hipStream_t st) {
    if (a.L > kMaxChunk) return hipErrorInvalidValue;     // the register tiles hold at most kMaxChunk rows
    if (kind == kCellTanhRnn) {
        return dense ? launch_dp<kCellTanhRnn, true>(DP, phase, a, st)
                     : launch_dp<kCellTanhRnn, false>(DP, phase, a, st);
    }
    if (kind == kCellEuler) {
        return dense ? launch_dp<kCellEuler, true>(DP, phase, a, st)
                     : launch_dp<kCellEuler, false>(DP, phase, a, st);
    }
    return dense ? launch_dp<kCellGru, true>(DP, phase, a, st)
                 : launch_dp<kCellGru, false>(DP, phase, a, st);
}

static size_t cell_pass_array_floats(int kind, int DP, bool dense, int L, int m) {
    const size_t NG = kind == kCellGru ? 3 : 1;
    const size_t NCO = dense ? (kind == kCellTanhRnn ? 1 : kind == kCellEuler ? 2 : 4) : 1;
    const size_t NO = (NG * DP + 15) & ~size_t(15);
    const size_t PS = DP + 4, xs = x_stride(m);     // iterate_stride<DP>()
    const size_t nxh = DP % 16 == 0 ? 0 : static_cast<size_t>(L) * NO;   // XI, H (not with CellRegs)
    size_t f = 2ull * (L + 1) * PS + 2ull * nxh + static_cast<size_t>(L) * DP + NCO * L * DP +
               static_cast<size_t>(L) * xs + DP;
    if (dense) f += 2ull * DP * (DP + 1) + 2ull * DP;
    else f += 2ull * kThreads;                        // carry segments (CellArgs::fc)
    return f;
}

// The weights fit in LDS beside the tile arrays when the whole workgroup
// footprint stays within 150 KB (of the 160 KB per compute unit).
static bool weights_fit_lds(int kind, int DP, bool dense, int L, int m) {
    const size_t w = (prepared_weight_floats(kind, DP, m) + 3) & ~size_t(3);
    return (w + cell_pass_array_floats(kind, DP, dense, L, m)) * sizeof(float) <= 150 * 1024;
}

// A sweep stages the weights in LDS when they fit, except with the
// register-resident evaluation of the diagonal modes (DP a multiple of 16),
// which reads each weight once per tile into registers.
bool cell_pass_stages_weights(int kind, int DP, bool dense, int L, int m) {
    if (DP % 16 == 0 && !dense) return false;
    return weights_fit_lds(kind, DP, dense, L, m);
}

size_t cell_pass_lds_bytes(int kind, int DP, bool dense, int L, int m) {
    size_t f = cell_pass_array_floats(kind, DP, dense, L, m);
    if (cell_pass_stages_weights(kind, DP, dense, L, m))
        f += (prepared_weight_floats(kind, DP, m) + 3) & ~size_t(3);
    return f * sizeof(float);
}

int cell_pass_nblocks(const CellArgs& a) { return a.NC * a.B; }

// ---------------------------------------------------------------- persistent solver
// Grid-wide barrier over co-resident workgroups (cooperative launch): every
// block adds one arrival to a monotonically increasing counter and waits for
// epoch * nblocks arrivals.  Agent-scope fences before the arrival and after
// the wait publish this block's writes and make the others' visible.  The
// wait is bounded: on timeout, or when another block has timed out, the
// block sets the error flag and returns false, and every block then leaves
// the kernel, so a broken barrier cannot hang the device.
__device__ __forceinline__ bool grid_sync(const PersistArgs& a, unsigned& epoch) {
    __shared__ int ok;
    __syncthreads();
    ++epoch;
    if (threadIdx.x == 0) {
        ok = 1;
        __threadfence();
        atomicAdd(a.bar, 1u);
        const unsigned target = epoch * gridDim.x;
        unsigned spins = 0;
        while (__hip_atomic_load(a.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (__hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
                ++spins > (1u << 24)) {
                atomicExch(a.err, 1u);
                ok = 0;
                break;
            }
        }
        __threadfence();
    }
    __syncthreads();
    return ok != 0;
}

// Carries of one batch row for the diagonal modes (same recurrence as
// diag_carry_kernel): NSEG threads per channel compose contiguous runs of
// chunk maps, the runs are combined through LDS, each thread replays its run.
template <int DP>
__device__ __forceinline__ void carry_row(const CellArgs& g, int b, float* segA, float* segB) {
    constexpr int NSEG = kThreads / DP;
    constexpr int kPerR = 16;
    const int dl = threadIdx.x % DP, sg = threadIdx.x / DP;
    const int NC = g.NC, D = g.D;
    const int per = (NC + NSEG - 1) / NSEG;
    const int c0 = min(NC, sg * per), c1 = min(NC, c0 + per);
    const bool act = dl < D;
    const size_t base = static_cast<size_t>(b) * NC * D + dl;
    float A = 1.0f, Bc = 0.0f;
    float ra[kPerR], rbv[kPerR];
    const bool inreg = c1 - c0 <= kPerR;
    if (act) {
        if (inreg) {
#pragma unroll
            for (int k = 0; k < kPerR; ++k) {
                const bool in = c0 + k < c1;
                ra[k] = in ? g.aggA[base + static_cast<size_t>(c0 + k) * D] : 1.0f;
                rbv[k] = in ? g.aggB[base + static_cast<size_t>(c0 + k) * D] : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < kPerR; ++k) {
                Bc = ra[k] * Bc + rbv[k];
                A = ra[k] * A;
            }
        } else {
            for (int cc = c0; cc < c1; ++cc) {
                const float ac = g.aggA[base + static_cast<size_t>(cc) * D];
                const float bc = g.aggB[base + static_cast<size_t>(cc) * D];
                Bc = ac * Bc + bc;
                A = ac * A;
            }
        }
    }
    segA[sg * DP + dl] = A;
    segB[sg * DP + dl] = Bc;
    __syncthreads();
    if (act) {
        float y = g.s0[b * g.s0s + dl];
        for (int k = 0; k < sg; ++k) y = segA[k * DP + dl] * y + segB[k * DP + dl];
        float* cr = const_cast<float*>(g.carry);
        if (inreg) {
#pragma unroll
            for (int k = 0; k < kPerR; ++k) {
                if (c0 + k < c1) {
                    cr[base + static_cast<size_t>(c0 + k) * D] = y;
                    y = ra[k] * y + rbv[k];
                }
            }
        } else {
            for (int cc = c0; cc < c1; ++cc) {
                cr[base + static_cast<size_t>(cc) * D] = y;
                y = g.aggA[base + static_cast<size_t>(cc) * D] * y + g.aggB[base + static_cast<size_t>(cc) * D];
            }
        }
    }
    __syncthreads();
}

// One launch for the whole solve: per window, the iteration-0 chunk maps,
// then per iteration (identical stop decision in every block, from the same
// residual partials) a carry phase and an apply phase, each followed by a
// grid barrier.  The weights are staged in LDS once.
template <int CELL, int DP>
__global__ __launch_bounds__(kThreads) void cell_persist(PersistArgs a) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ float segA[kThreads], segB[kThreads];
    CellArgs g = a.g;
    const int nw = static_cast<int>(prepared_weight_floats(CELL, DP, g.m));
    copy_to_lds<kThreads>(lds, g.w, nw);
    const float* w = lds;
    float* arr = lds + ((nw + 3) & ~3);
    unsigned epoch = 0;
    int hist_pos = 0;
    const int B = g.B;
    for (int wi = 0; wi < a.nwin; ++wi) {
        const int64_t w0 = static_cast<int64_t>(wi) * a.W;
        const int Tw = static_cast<int>(a.T - w0 < a.W ? a.T - w0 : a.W);
        g.Tw = Tw;
        g.NC = (Tw + g.L - 1) / g.L;
        g.x = a.x0 + w0 * g.m;
        g.s = a.s_base + w0 * g.D;
        if (wi == 0) {
            g.s0 = a.s0_user;
            g.s0s = g.D;
        } else {
            g.s0 = a.s_base + (w0 - 1) * g.D;
            g.s0s = a.T * g.D;
        }
        const int ntiles = B * g.NC;
        for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
            uint32_t rb = 0;
            cell_tile<CELL, DP, false, kPrologue>(g, t % g.NC, t / g.NC, arr, w, rb);
            rb = block_max_u32(rb);
            if (threadIdx.x == 0) g.rpart[t] = rb;
        }
        if (!grid_sync(a, epoch)) return;
        int K = 0, status = -1;
        for (int i = 0;; ++i) {
            uint32_t mx = 0;
            for (int k = threadIdx.x; k < ntiles; k += kThreads) mx = max(mx, g.rpart[k]);
            mx = block_max_u32(mx);
            int st = -1;
            if (mx >= kNonFiniteBits) st = kStNonFinite;
            else if (__uint_as_float(mx) <= a.tol) st = kStOk;
            else if (i >= a.max_iter) st = kStNotConverged;
            if (blockIdx.x == 0 && threadIdx.x == 0 && hist_pos < a.hist_cap) a.hist[hist_pos] = __uint_as_float(mx);
            ++hist_pos;
            if (st >= 0) {
                K = i;
                status = st;
                break;
            }
            for (int bb = blockIdx.x; bb < B; bb += gridDim.x) carry_row<DP>(g, bb, segA, segB);
            if (!grid_sync(a, epoch)) return;
            g.iter = i;
            for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
                uint32_t rb = 0;
                if (i == 0) cell_tile<CELL, DP, false, kFirst>(g, t % g.NC, t / g.NC, arr, w, rb);
                else cell_tile<CELL, DP, false, kSteady>(g, t % g.NC, t / g.NC, arr, w, rb);
                rb = block_max_u32(rb);
                if (threadIdx.x == 0) g.rpart[t] = rb;
            }
            if (!grid_sync(a, epoch)) return;
        }
        if (K == 0) {
            // no update applied: the window's result is s0 repeated
            for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
                const int c = t % g.NC, b = t / g.NC;
                const int t0 = c * g.L, Lc = min(g.L, Tw - t0);
                float* sg = g.s + b * g.ss + static_cast<int64_t>(t0) * g.D;
                const float* s0 = g.s0 + b * g.s0s;
                for (int e = threadIdx.x; e < Lc * g.D; e += kThreads) sg[e] = s0[e % g.D];
            }
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.win_iters[wi] = K;
            a.win_status[wi] = status;
            *a.hist_len = hist_pos;
        }
        if (status == kStNonFinite) break;
        if (!grid_sync(a, epoch)) return;
    }
}

bool cell_persist_eligible(int kind, int DP, int L, int m) {
    return (kind == kCellTanhRnn || kind == kCellGru) && L <= kMaxChunk && weights_fit_lds(kind, DP, false, L, m);
}

template <int CELL, int DP>
static hipError_t persist_max_blocks_t(size_t lds, int* nb) {
    int per_cu = 0, dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (lds > 64 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(cell_persist<CELL, DP>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, cell_persist<CELL, DP>, kThreads, lds);
    if (e != hipSuccess) return e;
    *nb = per_cu * ncu;
    return hipSuccess;
}

// the persistent solver always stages the weights
static size_t persist_lds(int kind, int DP, int L, int m) {
    const size_t w = (prepared_weight_floats(kind, DP, m) + 3) & ~size_t(3);
    return (w + cell_pass_array_floats(kind, DP, false, L, m)) * sizeof(float);
}

hipError_t cell_persist_max_blocks(int kind, int DP, int L, int m, int* nb) {
    const size_t lds = persist_lds(kind, DP, L, m);
    if (kind == kCellTanhRnn) {
        switch (DP) {
            case 4: return persist_max_blocks_t<kCellTanhRnn, 4>(lds, nb);
            case 8: return persist_max_blocks_t<kCellTanhRnn, 8>(lds, nb);
            case 16: return persist_max_blocks_t<kCellTanhRnn, 16>(lds, nb);
            case 32: return persist_max_blocks_t<kCellTanhRnn, 32>(lds, nb);
            default: return persist_max_blocks_t<kCellTanhRnn, 64>(lds, nb);
        }
    }
    switch (DP) {
        case 4: return persist_max_blocks_t<kCellGru, 4>(lds, nb);
        case 8: return persist_max_blocks_t<kCellGru, 8>(lds, nb);
        case 16: return persist_max_blocks_t<kCellGru, 16>(lds, nb);
        case 32: return persist_max_blocks_t<kCellGru, 32>(lds, nb);
        default: return persist_max_blocks_t<kCellGru, 64>(lds, nb);
    }
}

template <int CELL, int DP>
static hipError_t launch_persist_t(int nblocks, const PersistArgs& a, size_t lds, hipStream_t st) {
    void* args[] = {const_cast<PersistArgs*>(&a)};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(cell_persist<CELL, DP>), dim3(nblocks),
                                      dim3(kThreads), args, static_cast<unsigned>(lds), st);
}

hipError_t launch_cell_persist(int kind, int DP, int nblocks, const PersistArgs& a, hipStream_t st) {
    const size_t lds = persist_lds(kind, DP, a.g.L, a.g.m);
    if (kind == kCellTanhRnn) {
        switch (DP) {
            case 4: return launch_persist_t<kCellTanhRnn, 4>(nblocks, a, lds, st);
            case 8: return launch_persist_t<kCellTanhRnn, 8>(nblocks, a, lds, st);
            case 16: return launch_persist_t<kCellTanhRnn, 16>(nblocks, a, lds, st);
            case 32: return launch_persist_t<kCellTanhRnn, 32>(nblocks, a, lds, st);
            default: return launch_persist_t<kCellTanhRnn, 64>(nblocks, a, lds, st);
        }
    }
    switch (DP) {
        case 4: return launch_persist_t<kCellGru, 4>(nblocks, a, lds, st);
        case 8: return launch_persist_t<kCellGru, 8>(nblocks, a, lds, st);
        case 16: return launch_persist_t<kCellGru, 16>(nblocks, a, lds, st);
        case 32: return launch_persist_t<kCellGru, 32>(nblocks, a, lds, st);
        default: return launch_persist_t<kCellGru, 64>(nblocks, a, lds, st);
    }
}

// ---------------------------------------------------------------- standalone check
__global__ __launch_bounds__(kThreads) void check_kernel(CheckArgs c) { run_check(c); }

hipError_t launch_check(const CheckArgs& c, hipStream_t st) {
    check_kernel<<<1, kThreads, 0, st>>>(c);
    return hipGetLastError();
}

// ---------------------------------------------------------------- dense carry scan
// carry[b][0] = s0[b]; carry[b][c+1] = M[b][c] carry[b][c] + bg[b][c].
// One wavefront per batch row; lane i owns row i of every chunk map and the
// i-th entry of the running carry.  The chain is serial, so what counts is
// the instruction count per chunk: each lane keeps the rows of the next AH
// chunks in registers (16-byte loads, issued AH chunks ahead, no per-element
// branches: lanes past D read row D-1 and drop the result), and the carry is
// broadcast through LDS (one write, DP/4 16-byte broadcast reads per chunk).
// D not a multiple of 4 takes a plain per-element loop.
// The register-ring chain; FULL: D == DP (no padded columns to clear).
template <int DP, bool FULL>
__device__ __forceinline__ void carry_chain(const CarryArgs& g, float* ys, float y) {
    constexpr int AH = DP <= 16 ? 8 : 4;         // chunk maps in flight
    constexpr int Q = DP / 4;                    // 16-byte pieces per row
    const int i = threadIdx.x, D = g.D;
    const bool live = i < D;
    const int ir = live ? i : D - 1;
    const size_t cb = static_cast<size_t>(blockIdx.x) * g.NC;
    const int steps = g.NC - 1;
    float4 ring[AH][Q];
    float ob[AH];
    auto load = [&](int c, float4 (&row)[Q], float& off) {
        const float4* M = reinterpret_cast<const float4*>(g.aggA + (cb + c) * D * D + static_cast<size_t>(ir) * D);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            if constexpr (FULL) row[q] = M[q];
            else row[q] = 4 * q < D ? M[q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        off = g.aggB[(cb + c) * D + ir];
    };
#pragma unroll
    for (int p = 0; p < AH; ++p) load(min(p, steps - 1), ring[p], ob[p]);
    const float4* y4 = reinterpret_cast<const float4*>(ys);
    for (int c0 = 0; c0 < steps; c0 += AH) {
#pragma unroll
        for (int p = 0; p < AH; ++p) {
            const int c = c0 + p;
            if (c < steps) {
                if (i < DP) ys[i] = y;
                __builtin_amdgcn_wave_barrier();
                float part[4] = {ob[p], 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const float4 yv = y4[q];
                    const float4 mv = ring[p][q];
                    part[q & 3] += mv.x * yv.x + mv.y * yv.y + mv.z * yv.z + mv.w * yv.w;
                }
                __builtin_amdgcn_wave_barrier();
                const float acc = (part[0] + part[1]) + (part[2] + part[3]);
                if constexpr (FULL) {
                    y = acc;
                    if (live) g.carry[(cb + c + 1) * D + i] = acc;
                } else {
                    y = live ? acc : 0.0f;
                    if (live) g.carry[(cb + c + 1) * D + i] = acc;
                }
                load(min(c + AH, steps - 1), ring[p], ob[p]);
            }
        }
    }
}

template <int DP>
__global__ __launch_bounds__(64) void dense_carry_kernel(CarryArgs g) {
    if (g.stop_on && g.stop_on->stop) return;     // queued ahead of a stop
    if (g.do_check && blockIdx.x == 0) run_check(g.chk);
    __shared__ __attribute__((aligned(16))) float ys[DP < 4 ? 4 : DP];
    const int b = blockIdx.x;
    const int i = threadIdx.x;
    const int D = g.D;
    const bool live = i < D;
    const int ir = live ? i : D - 1;
    const size_t cb = static_cast<size_t>(b) * g.NC;
    const int steps = g.NC - 1;                  // maps 0 .. NC-2 give carries 1 .. NC-1
    float y = live ? g.s0[b * g.s0s + i] : 0.0f;
    if (live) g.carry[cb * D + i] = y;
    if (steps <= 0) return;
    if (D % 4 != 0) {
        // plain chain: row i of each map straight from memory
        for (int c = 0; c < steps; ++c) {
            if (i < DP) ys[i] = y;
            __builtin_amdgcn_wave_barrier();
            const float* M = g.aggA + (cb + c) * D * D + static_cast<size_t>(ir) * D;
            float acc = g.aggB[(cb + c) * D + ir];
            for (int k = 0; k < D; ++k) acc += M[k] * ys[k];
            __builtin_amdgcn_wave_barrier();
            y = live ? acc : 0.0f;
            if (live) g.carry[(cb + c + 1) * D + i] = acc;
        }
        return;
    }
    // lanes past DP hold nothing; lanes in [D, DP) carry zeros
    if constexpr (DP >= 4) {
        if (D == DP) carry_chain<DP, true>(g, ys, y);
        else carry_chain<DP, false>(g, ys, y);
    }
}

// Wide form for D padded to 32 or 64 (D a multiple of 4): one workgroup of
// DP x DP/4 threads per batch row.  Thread (i, p) owns the 16-byte piece p of
// row i of every chunk map, so a chunk map arrives as one coalesced 16-byte
// load per thread and kKW chunks are in flight per workgroup (DP/4 times the
// bytes of the one-wavefront chain, whose time per chunk is the latency of
// its map loads).  The DP/4 partial dot products of a row sit in adjacent
// lanes of one 16-lane DPP row and are summed with DPP moves (swap neighbours,
// swap pairs, mirror within 8, mirror within 16); the new carry goes through
// a double-buffered LDS vector with one barrier per chunk.
// Every global access of the unrolled body is unconditional (clamped
// addresses and selects; threads of rows past D redo row D-1 and store the
// same value again), so the compiler can count the loads issued after each
// prefetch and wait for that one only.
constexpr int kKW = 16;                      // chunk maps in flight per thread

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int DP>
__global__ __launch_bounds__(DP * DP / 4) void dense_carry_wide(CarryArgs g) {
    if (g.stop_on && g.stop_on->stop) return;     // queued ahead of a stop
    if (g.do_check && blockIdx.x == 0) run_check(g.chk);
    constexpr int TPR = DP / 4;              // threads per map row
    __shared__ __attribute__((aligned(16))) float ys[2][DP];
    const int t = threadIdx.x;
    const int i = t / TPR, p = t % TPR;
    const int D = g.D;
    const bool live = i < D, pin = 4 * p < D;
    const int ir = live ? i : D - 1;
    const int pc = pin ? 4 * p : 0;          // clamped column of the piece
    const int b = blockIdx.x;
    const size_t cb = static_cast<size_t>(b) * g.NC;
    const int steps = g.NC - 1;
    if (p == 0) {
        const float y0 = live ? g.s0[b * g.s0s + i] : 0.0f;
        ys[0][i] = y0;
        if (live) g.carry[cb * D + i] = y0;
    }
    if (steps <= 0) return;
    const float* Mb = g.aggA + cb * D * D + static_cast<size_t>(ir) * D + pc;
    const float* Bb = g.aggB + cb * D + ir;
    float* Cb = g.carry + (cb + 1) * D + ir;
    const size_t DD = static_cast<size_t>(D) * D;
    float4 ring[kKW];
    float ob[kKW];
#pragma unroll
    for (int u = 0; u < kKW; ++u) {
        const int c = min(u, steps - 1);
        ring[u] = *reinterpret_cast<const float4*>(Mb + c * DD);
        ob[u] = Bb[static_cast<size_t>(c) * D];
    }
    __syncthreads();
    // one chunk: y_i = row i of M_c . y + bg_c
    auto step = [&](int c, const float4& m4, float off) {
        const float4 mv = pin ? m4 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float4 yv = *reinterpret_cast<const float4*>(&ys[c & 1][4 * p]);
        float part = (mv.x * yv.x + mv.y * yv.y) + (mv.z * yv.z + mv.w * yv.w);
        part = dpp_add<0xB1>(part);                          // quad_perm [1,0,3,2]
        part = dpp_add<0x4E>(part);                          // quad_perm [2,3,0,1]
        if constexpr (TPR >= 8) part = dpp_add<0x141>(part);   // row_half_mirror
        if constexpr (TPR >= 16) part = dpp_add<0x140>(part);  // row_mirror
        const float y = part + off;
        Cb[static_cast<size_t>(c) * D] = y;
        if (p == 0) ys[(c + 1) & 1][i] = live ? y : 0.0f;
    };
    int c0 = 0;
    for (; c0 + kKW <= steps; c0 += kKW) {
#pragma unroll
        for (int u = 0; u < kKW; ++u) {
            const int c = c0 + u;
            step(c, ring[u], ob[u]);
            const int cn = min(c + kKW, steps - 1);
            ring[u] = *reinterpret_cast<const float4*>(Mb + cn * DD);
            ob[u] = Bb[static_cast<size_t>(cn) * D];
            __syncthreads();
        }
    }
    // the last steps - c0 < kKW chunks are already in ring[0 ..]
#pragma unroll
    for (int u = 0; u < kKW; ++u) {
        if (c0 + u < steps) {
            step(c0 + u, ring[u], ob[u]);
            __syncthreads();
        }
    }
}

// D padded to 16 with at most kScanMaxChunks chunks per row: the carries as
// a two-level scan of the affine chunk maps (composing affine maps is
// associative [PN §2.1]) on the 16x16x4 FP32 matrix cores.  One workgroup per
// batch row, one wavefront per group of G <= kScanG consecutive chunks:
//  1. every group but the last composes its maps into one affine map (P, q);
//  2. wavefront 0 runs the group maps from s0: the carry entering each group;
//  3. every group runs its own maps from its entering carry and stores its
//     carries.
// That is 2 G + NC / G dependent map steps instead of NC - 1 (G about
// sqrt(NC / 2) minimises it).  A
// map step is four chained MFMAs: the A operand is the map as loaded (lane
// (i, h) holds M[i][4h .. 4h+3]), the B operand the running matrix or vector
// in the accumulator layout (register r of lane (j, h) holds entry (4h + r,
// j)), so each result is the next step's operand as it stands; a vector
// rides in every column.  Rows and columns past D are zero.
constexpr int kScanG = 8;
constexpr int kScanMaxChunks = 16 * kScanG;

// group size for NC chunks: the least G with 2 G^2 >= NC, at most kScanG
__host__ __device__ __forceinline__ int scan_group(int NC) {
    int G = 1;
    while (G < kScanG && 2 * G * G < NC) ++G;
    return G;
}

__device__ __forceinline__ v4f map_step16(const float4& A, const v4f& X, v4f C) {
    C = __builtin_amdgcn_mfma_f32_16x16x4f32(A.x, X[0], C, 0, 0, 0);
    C = __builtin_amdgcn_mfma_f32_16x16x4f32(A.y, X[1], C, 0, 0, 0);
    C = __builtin_amdgcn_mfma_f32_16x16x4f32(A.z, X[2], C, 0, 0, 0);
    C = __builtin_amdgcn_mfma_f32_16x16x4f32(A.w, X[3], C, 0, 0, 0);
    return C;
}

__global__ __launch_bounds__(64 * (kScanMaxChunks / kScanG)) void dense_carry_scan16(CarryArgs g) {
    if (g.stop_on && g.stop_on->stop) return;     // queued ahead of a stop
    if (g.do_check && blockIdx.x == 0) run_check(g.chk);
    __shared__ __attribute__((aligned(16))) float Pl[kScanMaxChunks / kScanG][256];   // group maps, row-major
    __shared__ __attribute__((aligned(16))) float ql[kScanMaxChunks / kScanG][16];    // group offsets
    __shared__ __attribute__((aligned(16))) float yl[kScanMaxChunks / kScanG][16];    // carries entering groups
    const int D = g.D, NC = g.NC;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = lane & 15, h = lane >> 4;
    const int G = scan_group(NC);
    const int nw = static_cast<int>(blockDim.x >> 6);     // ceil(NC / G)
    const size_t cb = static_cast<size_t>(blockIdx.x) * NC;
    const int c0 = w * G;
    const int nown = min(G, NC - c0);                     // carries of this group
    const int nmap = w < nw - 1 ? G : nown - 1;           // maps it runs
    const bool vec4 = (D & 3) == 0;
    // maps c0 .. c0 + nmap - 1 (at most NC - 2) in the A layout, offsets in
    // the accumulator layout.  Every load is unconditional (clamped chunk,
    // row and column; unused values are replaced by zeros), so all of them
    // are in flight at once.
    float4 Ma[kScanG], ba[kScanG];
    const float4 zero4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    const int ir = min(i, D - 1);
    if (vec4) {
        const bool colok = 4 * h < D;
        const int kc = colok ? 4 * h : 0;
#pragma unroll
        for (int u = 0; u < kScanG; ++u) {
            const size_t c = cb + min(c0 + u, NC - 1);
            const float4 mv = *reinterpret_cast<const float4*>(g.aggA + c * D * D + ir * D + kc);
            const float4 bb = *reinterpret_cast<const float4*>(g.aggB + c * D + kc);
            Ma[u] = (u < nmap && i < D && colok) ? mv : zero4;
            ba[u] = (u < nmap && colok) ? bb : zero4;
        }
    } else {
#pragma unroll
        for (int u = 0; u < kScanG; ++u) {
            const size_t c = cb + min(c0 + u, NC - 1);
            float mv[4], bb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k = 4 * h + s, kk = min(k, D - 1);
                const float m = g.aggA[c * D * D + ir * D + kk];
                const float o = g.aggB[c * D + kk];
                mv[s] = (u < nmap && i < D && k < D) ? m : 0.0f;
                bb[s] = (u < nmap && k < D) ? o : 0.0f;
            }
            Ma[u] = make_float4(mv[0], mv[1], mv[2], mv[3]);
            ba[u] = make_float4(bb[0], bb[1], bb[2], bb[3]);
        }
    }
    auto bvec = [](const float4& v) {
        v4f r;
        r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
        return r;
    };
    if (w < nw - 1) {
        // 1. (P, q) <- (M_c P, M_c q + b_c) over the group's maps
        v4f P, q = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < 4; ++r) P[r] = 4 * h + r == i ? 1.0f : 0.0f;
#pragma unroll
        for (int u = 0; u < kScanG; ++u) {
            if (u < G) {
                P = map_step16(Ma[u], P, v4f{0.0f, 0.0f, 0.0f, 0.0f});
                q = map_step16(Ma[u], q, bvec(ba[u]));
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) Pl[w][(4 * h + r) * 16 + i] = P[r];
        if (i == 0) *reinterpret_cast<float4*>(&ql[w][4 * h]) = make_float4(q[0], q[1], q[2], q[3]);
    }
    __syncthreads();
    if (w == 0) {
        // 2. the carry entering each group
        const float* s0b = g.s0 + static_cast<int64_t>(blockIdx.x) * g.s0s;
        v4f y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = 4 * h + r < D ? s0b[4 * h + r] : 0.0f;
        for (int v = 0; v < nw; ++v) {
            if (i == 0) *reinterpret_cast<float4*>(&yl[v][4 * h]) = make_float4(y[0], y[1], y[2], y[3]);
            if (v == nw - 1) break;
            const float4 A = *reinterpret_cast<const float4*>(&Pl[v][i * 16 + 4 * h]);
            y = map_step16(A, y, bvec(*reinterpret_cast<const float4*>(&ql[v][4 * h])));
        }
    }
    __syncthreads();
    // 3. the group's carries
    v4f y = bvec(*reinterpret_cast<const float4*>(&yl[w][4 * h]));
#pragma unroll
    for (int u = 0; u < kScanG; ++u) {
        if (u < nown) {
            if (i == 0) {
                float* cr = g.carry + (cb + c0 + u) * D;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (4 * h + r < D) cr[4 * h + r] = y[r];
            }
            if (u < nown - 1) y = map_step16(Ma[u], y, bvec(ba[u]));
        }
    }
}

hipError_t launch_dense_carry(const CarryArgs& a, hipStream_t st) {
    const int DP = a.D <= 4 ? 4 : a.D <= 8 ? 8 : a.D <= 16 ? 16 : a.D <= 32 ? 32 : 64;
    if (DP == 16 && a.NC >= 1 && a.NC <= kScanMaxChunks) {
        const int G = scan_group(a.NC);
        const int nw = (a.NC + G - 1) / G;
        dense_carry_scan16<<<a.B, 64 * nw, 0, st>>>(a);
        return hipGetLastError();
    }
    if (a.D % 4 == 0 && DP >= 16) {
        if (DP == 16) dense_carry_wide<16><<<a.B, 16 * 4, 0, st>>>(a);
        else if (DP == 32) dense_carry_wide<32><<<a.B, 32 * 8, 0, st>>>(a);
        else dense_carry_wide<64><<<a.B, 64 * 16, 0, st>>>(a);
        return hipGetLastError();
    }
    switch (DP) {
        case 4: dense_carry_kernel<4><<<a.B, 64, 0, st>>>(a); break;
        case 8: dense_carry_kernel<8><<<a.B, 64, 0, st>>>(a); break;
        case 16: dense_carry_kernel<16><<<a.B, 64, 0, st>>>(a); break;
        case 32: dense_carry_kernel<32><<<a.B, 64, 0, st>>>(a); break;
        default: dense_carry_kernel<64><<<a.B, 64, 0, st>>>(a); break;
    }
    return hipGetLastError();
}


// ---------------------------------------------------------------- resident solver
// The whole solve of a matrix cell in a diagonal mode as one cooperative
// launch, for shapes whose B x NC chunks are co-resident (one workgroup per
// chunk).  Unlike cell_persist, a workgroup keeps its chunk on chip for the
// whole window: the rows of the iterate in LDS, the input projections and the
// weights in registers (CellRegs), and the per-step coefficients of the last
// evaluation in LDS, which are the maps of the next update.  An iteration is
// therefore one evaluation (at the new iterate) instead of two, and the only
// traffic between workgroups is small: the chunk maps of the iteration, the
// last row of every chunk (the next chunk's halo), the residual maxima and the
// next window's initial state.  These go through relaxed device-scope atomic
// loads and stores, which are coherent across the XCDs' L2 caches without
// cache-wide fences; a grid barrier (one arrival word per workgroup, stored
// after every memory operation of the workgroup has completed) separates the
// iterations.  Every wait is bounded: on a timeout the error flag is set and
// every workgroup leaves, so a broken barrier cannot hang the device.
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier: the workgroup's memory operations complete (s_waitcnt 0),
// then the workgroup stores the barrier's epoch into its own arrival word (a
// store, not a read-modify-write: no two workgroups touch one word), and its
// first wavefront polls every arrival word, 64 per load instruction, until
// all hold at least this epoch.  The wait is bounded.
__device__ __forceinline__ bool resident_sync(const ResidentArgs& a, unsigned& epoch, unsigned nblocks) {
    __shared__ int ok;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    ++epoch;
    if (threadIdx.x < 64) {
        const unsigned blk = blockIdx.y * gridDim.x + blockIdx.x;
        if (threadIdx.x == 0) __hip_atomic_store(a.bar + blk, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned spins = 0;
        int good = 1;
        for (;;) {
            int done = 1;
            for (unsigned k = threadIdx.x; k < nblocks; k += 64)
                done &= __hip_atomic_load(a.bar + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= epoch;
            if (__all(done)) break;
            __builtin_amdgcn_s_sleep(1);
            if (++spins > (1u << 22) || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                if (threadIdx.x == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                good = 0;
                break;
            }
        }
        if (threadIdx.x == 0) ok = good;
    }
    __syncthreads();
    return ok != 0;
}

// CPW chunks per workgroup: chunk bx + k * gridDim.x of the batch row, k <
// CPW, so that more chunks than co-resident workgroups still fit (workload 2:
// 2048 chunks over 512 workgroups).  Each chunk keeps its own LDS region; the
// fold, the replay and the map composition of the CPW chunks run side by
// side on disjoint thread groups, the evaluations one chunk after another.
//
// No grid barrier per iteration.  A chunk's fold needs the maps (and the
// halo) of the chunks before it in its batch row only: after its own map
// stores have completed, each chunk stores the publication's tag into its
// ready word, and a workgroup waits for the ready words of its row's earlier
// chunks.  The stop decision needs every workgroup's residual, so it is taken
// one iteration late: iteration i replays s^(i+1) into the chunk's second row
// buffer and publishes its maps and r_{i+1} before it reads r_i, by then
// (almost always) complete, from one (tag, residual) word per workgroup.
// Each iteration first stores its rows of s^(i) to out (the last chunk of a
// row also its last row to s0n), so a stop at i finds the result in place;
// the work on s^(i+1) is dropped.
// Tags count publications alike in every workgroup (the decisions are
// alike), maps and halo rotate over three sets and the residual words over
// four, which no workgroup can overrun: to publish tag t + 3 a workgroup has
// seen every workgroup publish tag t + 1 (and t + 2 for the words), which
// each does only after its fold of tag t.  At a window's end every
// workgroup also waits for the iteration past the stop, before the next
// window reuses the sets.
template <int CELL, int DP, int CPW>
__global__ __launch_bounds__(kThreads, CPW > 1 ? 2 : 1) void cell_resident(ResidentArgs a) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int PS = iterate_stride<DP>();
    constexpr int TG = kThreads / CPW;           // threads per chunk in the fold
    constexpr int NS = TG / DP;                  // fold segments per channel
    static_assert(NS >= 1, "CPW x DP must not exceed the workgroup");
    const int L = a.L, m = a.m, D = a.D, B = a.B;
    const int xs = x_stride(m);
    const int bx = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int GX = gridDim.x;
    const int nblocks = gridDim.x * gridDim.y;
    const int blk = b * GX + bx;
    const bool lead = bx == 0 && b == 0;
    // One chunk per workgroup: two row buffers, s^(i) kept in one while the
    // replay writes s^(i+1) into the other.  Four: one buffer, replayed in
    // place (two would not leave two workgroups room on a compute unit), and
    // s^(i) stored to out at the start of each iteration instead.
    constexpr bool DB = CPW == 1;
    const int RB = (L + 1) * PS;                 // one row buffer
    const int per_chunk = (DB ? 2 : 1) * RB + 2 * L * DP + L * xs;
    float* SCR = lds + CPW * per_chunk;          // [2][kThreads] fold segments
    float* S0 = SCR + 2 * kThreads;              // [DP] initial state of the window
    int cur = 0;                                 // the row buffer holding s^(i) (DB)
    auto Sk = [&](int k) { return lds + k * per_chunk + (DB ? cur * RB : 0); };         // [L+1][PS] rows t0-1 .. t1-1
    auto Snx = [&](int k) { return lds + k * per_chunk + (DB ? (cur ^ 1) * RB : 0); };  // where the replay writes
    auto Vk = [&](int k) { return lds + k * per_chunk + (DB ? 2 : 1) * RB; };            // [L][DP]
    auto COk = [&](int k) { return Vk(k) + L * DP; };                   // [L][DP]
    auto Xk = [&](int k) { return COk(k) + L * DP; };                   // [L][xs]
    __shared__ uint32_t chk_r;
    __shared__ int sync_ok;
    CellRegs<CELL, DP> cr;
    cr.load(a.w, a.w, D, m);
    const size_t HS = static_cast<size_t>(B) * a.NC * D;   // set stride of maps and halo
    unsigned* rdy = a.ready + static_cast<size_t>(b) * a.NC;
    unsigned tag = 0;                            // publications so far
    int hist_pos = 0;
    // the thread's (chunk, channel) in the replay and the composition
    const int rk = tid / DP, ri = tid % DP;
    const bool rthr = rk < CPW && ri < D;
    float own_a = 1.0f, own_b = 0.0f;            // map of chunk (rk) of the current iteration, channel ri

    // Bounded waits of wavefront 0; on a timeout (or another workgroup's) the
    // error flag is set and the caller leaves.
    auto spin_fail = [&](unsigned& spins) -> bool {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1u << 22) || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            if (tid == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return true;
        }
        return false;
    };
    // every workgroup's word of set t % 4 carries tag t: their residual maximum to chk_r
    auto wait_all = [&](unsigned t) -> bool {
        if (tid < 64) {
            const unsigned long long* w = a.rword + static_cast<size_t>(t % 4) * nblocks;
            unsigned spins = 0;
            int good = 1;
            uint32_t mx = 0;
            for (;;) {
                int done = 1;
                mx = 0;
                for (int k = tid; k < nblocks; k += 64) {
                    const unsigned long long v = __hip_atomic_load(w + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    done &= static_cast<unsigned>(v >> 32) == t;
                    mx = max(mx, static_cast<uint32_t>(v));
                }
                if (__all(done)) break;
                if (spin_fail(spins)) {
                    good = 0;
                    break;
                }
            }
            mx = wave_max_u32(mx);
            if (tid == 0) {
                chk_r = mx;
                sync_ok = good;
            }
        }
        __syncthreads();
        return sync_ok != 0;
    };
    // the ready words of chunks [0, upto) of the row hold at least t
    auto wait_row = [&](unsigned t, int upto) -> bool {
        if (tid < 64) {
            int good = 1;
            unsigned spins = 0;
            for (;;) {
                int done = 1;
                for (int k = tid; k < upto; k += 64)
                    done &= __hip_atomic_load(rdy + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= t;
                if (__all(done)) break;
                if (spin_fail(spins)) {
                    good = 0;
                    break;
                }
            }
            if (tid == 0) sync_ok = good;
        }
        __syncthreads();
        return sync_ok != 0;
    };

    for (int wi = 0; wi < a.nwin; ++wi) {
        const int64_t w0 = static_cast<int64_t>(wi) * a.W;
        const int Tw = static_cast<int>(a.T - w0 < a.W ? a.T - w0 : a.W);
        const int NCw = (Tw + L - 1) / L;
        auto chunk = [&](int k) { return bx + k * GX; };
        auto active = [&](int k) { return chunk(k) < NCw; };
        auto rows = [&](int k) { return active(k) ? min(L, Tw - chunk(k) * L) : 0; };
        int upto = 0;                            // the fold waits for chunks [0, upto) of the row
#pragma unroll
        for (int k = 0; k < CPW; ++k)
            if (active(k)) upto = chunk(k);
        // the window's initial state: s0, or the last state of the row's previous window
        if (wi > 0) {
            if (tid < 64) {
                int good = 1;
                unsigned spins = 0;
                while (!__all(__hip_atomic_load(a.s0ready + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                              static_cast<unsigned>(wi))) {
                    if (spin_fail(spins)) {
                        good = 0;
                        break;
                    }
                }
                if (tid == 0) sync_ok = good;
            }
            __syncthreads();
            if (!sync_ok) return;
        }
        if (tid < DP)
            S0[tid] = tid < D ? (wi == 0 ? a.s0[static_cast<int64_t>(b) * D + tid] : ld_dev(a.s0n + b * D + tid)) : 0.0f;
        uint32_t rb = 0;
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            if (active(k))
                copy_rows_to_lds<kThreads>(Xk(k), xs, a.x + (static_cast<int64_t>(b) * a.T + w0 + chunk(k) * L) * m,
                                           m, rows(k), m);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            if (!active(k)) continue;
            float* S = Sk(k);
            for (int e = tid; e < (rows(k) + 1) * PS; e += kThreads) {
                const int i = e % PS;
                S[e] = i < DP ? S0[i] : 0.0f;
            }
        }
        __syncthreads();
        // the maps of iteration 0 at s^(0) = s0, and r_0 (one chunk after another)
#pragma unroll 1
        for (int k = 0; k < CPW; ++k) {
            if (!active(k)) continue;
            cr.project(a.w, Xk(k), xs, rows(k), m);
            cr.template eval<false>(Sk(k), Vk(k), COk(k), rows(k), L, a.mode, Sk(k), rb, nullptr, a.tol);
        }
        __syncthreads();
        // the chunk map of the iterate in the chunk's rows, composed and
        // published with its last row (the next chunk's halo) under tag t
        auto compose_publish = [&](unsigned t) {
            if (rthr && active(rk)) {
                const int Lc = rows(rk);
                const float* V = Vk(rk);
                const float* CO = COk(rk);
                const float* S = Sk(rk);
                float A = 1.0f, Bc = 0.0f;
                if (a.mode == kJacobi) {
                    A = 0.0f;
                    Bc = V[(Lc - 1) * DP + ri];
                } else {
#pragma unroll 8
                    for (int j = 0; j < Lc; ++j) {
                        const float at = CO[j * DP + ri];
                        Bc = at * Bc + (V[j * DP + ri] - at * S[j * PS + ri]);
                        A = at * A;
                    }
                }
                own_a = A;
                own_b = Bc;
                const size_t o = (t % 3) * HS + (static_cast<size_t>(b) * a.NC + chunk(rk)) * D + ri;
                st_dev(a.mapA + o, A);
                st_dev(a.mapB + o, Bc);
                st_dev(a.halo + o, S[Lc * PS + ri]);
            }
        };
        // once every memory operation of the workgroup has completed: the
        // ready words of its chunks and its (tag, residual) word
        auto post = [&](unsigned t, uint32_t rbv) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid < CPW && active(tid))
                __hip_atomic_store(rdy + chunk(tid), t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid == 0)
                __hip_atomic_store(a.rword + static_cast<size_t>(t % 4) * nblocks + blk,
                                   (static_cast<unsigned long long>(t) << 32) | rbv, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        };
        ++tag;
        compose_publish(tag);
        rb = block_max_u32(rb);
        post(tag, rb);
        int K = 0, status = kStOk;
        for (int i = 0;; ++i) {
            const unsigned tg = tag;             // tag of iteration i's maps and of r_i
            const int sel = static_cast<int>(tg % 3);
            // s^(i), the result should the check of iteration i stop: the
            // chunks' rows to out, the row's last state to s0n (one buffer)
#pragma unroll
            for (int k = 0; k < CPW; ++k) {
                if (DB || !active(k)) continue;
                const int c = chunk(k), Lc = rows(k);
                const float* S = Sk(k);
                float* o = a.out + (static_cast<int64_t>(b) * a.T + w0 + c * L) * D;
                for (int e = tid; e < Lc * D; e += kThreads) {
                    const int j = e / D, ii = e % D;
                    o[e] = S[(j + 1) * PS + ii];
                }
                if (c + 1 == NCw && tid < D) st_dev(a.s0n + b * D + tid, S[Lc * PS + tid]);
            }
            if (!wait_row(tg, upto)) return;
            // the carries: per chunk, NS segments of the maps of the chunks
            // before it, each folded into one map, applied to s0 after the barrier
            {
                const int fk = tid / TG, tl = tid % TG;
                const int d = tl % DP, sg_ = tl / DP;
                const int c = chunk(fk);
                const int cc = active(fk) ? c : 0;
                const int per = (cc + NS - 1) / NS;
                const int k0 = min(cc, sg_ * per);
                const int k1 = d < D ? min(cc, k0 + per) : k0;
                const float* mA = a.mapA + sel * HS + static_cast<size_t>(b) * a.NC * D;
                const float* mB = a.mapB + sel * HS + static_cast<size_t>(b) * a.NC * D;
                constexpr int kRF = (kFcMaxChunks + NS - 1) / NS < 16 ? (kFcMaxChunks + NS - 1) / NS : 16;
                float pa[kRF], pb[kRF];
#pragma unroll
                for (int u = 0; u < kRF; ++u) {
                    const int kk = k0 + u;
                    pa[u] = kk < k1 ? ld_dev(mA + kk * D + d) : 1.0f;
                    pb[u] = kk < k1 ? ld_dev(mB + kk * D + d) : 0.0f;
                }
                float fa = 1.0f, fbv = 0.0f;
#pragma unroll
                for (int u = 0; u < kRF; ++u) {
                    fbv = pa[u] * fbv + pb[u];
                    fa = pa[u] * fa;
                }
                for (int kk = k0 + kRF; kk < k1; ++kk) {
                    const float ak = ld_dev(mA + kk * D + d);
                    fbv = ak * fbv + ld_dev(mB + kk * D + d);
                    fa = ak * fa;
                }
                SCR[tid] = fa;
                SCR[kThreads + tid] = fbv;
            }
            // row t0-1 of s^(i): the window's s0 before the first chunk or
            // at i = 0, else the previous chunk's last row
            float hrow = 0.0f;
            if (rthr && active(rk)) {
                const int c = chunk(rk);
                hrow = (c == 0 || i == 0) ? S0[ri]
                                          : ld_dev(a.halo + sel * HS + (static_cast<size_t>(b) * a.NC + c - 1) * D + ri);
            }
            __syncthreads();
            // replay from the carry, damping: rows t0-1 .. t1-1 of s^(i+1) from
            // So into Sn (the same rows with one buffer: each old row is read
            // before the new one is written over it)
            const float lam = a.lam;
            const bool und = a.undamped != 0;
            if (rthr && active(rk)) {
                const int c = chunk(rk);
                const int Lc = rows(rk);
                const bool has_next = c + 1 < NCw;
                float xv = S0[ri];
#pragma unroll
                for (int sgi = 0; sgi < NS; ++sgi)
                    xv = SCR[rk * TG + sgi * DP + ri] * xv + SCR[kThreads + rk * TG + sgi * DP + ri];
                const float c_first = xv;
                const float c_next = own_a * xv + own_b;
                const float* So = Sk(rk);
                float* Sn = Snx(rk);
                const float* V = Vk(rk);
                const float* CO = COk(rk);
                float pold = hrow;                   // old value of the row before the current one
                float shat = c_first;
                Sn[ri] = und ? shat : pold + lam * (shat - pold);
                const int nrep = has_next ? Lc - 1 : Lc;
                if (a.mode == kJacobi) {
                    for (int j = 0; j < nrep; ++j) {
                        const float so = So[(j + 1) * PS + ri];
                        const float sh = V[j * DP + ri];
                        Sn[(j + 1) * PS + ri] = und ? sh : so + lam * (sh - so);
                    }
                } else {
                    int j = 0;
                    for (; j + 8 <= nrep; j += 8) {
                        float v[8], co[8], po[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            v[u] = V[(j + u) * DP + ri];
                            co[u] = CO[(j + u) * DP + ri];
                            po[u] = So[(j + u + 1) * PS + ri];
                        }
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            shat = v[u] + co[u] * (shat - pold);
                            pold = po[u];
                            Sn[(j + u + 1) * PS + ri] = und ? shat : pold + lam * (shat - pold);
                        }
                    }
                    for (; j < nrep; ++j) {
                        shat = V[j * DP + ri] + CO[j * DP + ri] * (shat - pold);
                        pold = So[(j + 1) * PS + ri];
                        Sn[(j + 1) * PS + ri] = und ? shat : pold + lam * (shat - pold);
                    }
                }
                if (has_next) {
                    const float so = So[Lc * PS + ri];
                    Sn[Lc * PS + ri] = und ? c_next : so + lam * (c_next - so);
                }
            }
            __syncthreads();
            if constexpr (DB) cur ^= 1;          // s^(i+1) is the current buffer now
            // the maps of iteration i+1 at s^(i+1), and r_{i+1}
            uint32_t rbn = 0;
#pragma unroll 1
            for (int k = 0; k < CPW; ++k) {
                if (!active(k)) continue;
                if (CPW > 1) cr.project(a.w, Xk(k), xs, rows(k), m);
                cr.template eval<false>(Sk(k), Vk(k), COk(k), rows(k), L, a.mode, Sk(k), rbn, nullptr, a.tol);
            }
            __syncthreads();
            ++tag;
            compose_publish(tag);
            rbn = block_max_u32(rbn);
            post(tag, rbn);
            // the check of iteration i (its residual words are in by now, as a rule)
            if (!wait_all(tg)) return;
            const uint32_t r_i = chk_r;
            int st = -1;
            if (r_i >= kNonFiniteBits) st = kStNonFinite;
            else if (__uint_as_float(r_i) <= a.tol) st = kStOk;
            else if (i >= a.max_iter) st = kStNotConverged;
            if (lead && tid == 0 && hist_pos < a.hist_cap) a.hist[hist_pos] = __uint_as_float(r_i);
            ++hist_pos;
            if (st >= 0) {
                K = i;
                status = st;
                if constexpr (DB) cur ^= 1;      // the result is s^(i)
                break;
            }
        }
        // every workgroup past the iteration after the stop before the sets
        // are reused; with one buffer out and s0n hold s^(K) since the start
        // of iteration K, with two they are stored now
        if (!wait_all(tag)) return;
        bool last = false;
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            if (!active(k)) continue;
            const int c = chunk(k), Lc = rows(k);
            if (c + 1 == NCw) last = true;
            if constexpr (DB) {
                const float* S = Sk(k);
                float* o = a.out + (static_cast<int64_t>(b) * a.T + w0 + c * L) * D;
                for (int e = tid; e < Lc * D; e += kThreads) {
                    const int j = e / D, ii = e % D;
                    o[e] = S[(j + 1) * PS + ii];
                }
                if (c + 1 == NCw && tid < D) st_dev(a.s0n + b * D + tid, S[Lc * PS + tid]);
            }
        }
        if (lead && tid == 0) {
            a.win_iters[wi] = K;
            a.win_status[wi] = status;
            *a.hist_len = hist_pos;
        }
        if (status == kStNonFinite) break;
        if (last) {
            __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();
        if (last && tid == 0)
            __hip_atomic_store(a.s0ready + b, static_cast<unsigned>(wi + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------- resident advancing window
// The advancing window [PN §1.3.1] of a matrix cell in a diagonal mode as one
// cooperative launch: workgroup (c, b) owns chunk c of batch row b of the
// current window [A, E), steps A + cL .. A + (c+1)L - 1.  A round is
//   check:  r_t of the current iterate on [A, E) and the first step over tol,
//           reduced over the grid (slot words 0 and 1), read alike by every
//           workgroup, which then all take the same decision;
//   slide:  A moves past the accepted prefix, E = min(T, A + W); when the
//           window moved, every workgroup stages its chunk of the new window
//           from the iterate in `out` (steps from the old E on start from the
//           old window's last state) and evaluates the cell there;
//   update: the chunk map, a wait for the maps of the chunks before it in
//           its row, the carry folded from those maps applied to the
//           accepted state s_{A-1}, the replay with damping, and the
//           evaluation at the new iterate, which is the next check; the
//           chunk's rows go back to `out`; a grid barrier ends the round.
// Rows travel between workgroups only through `out`, with device-scope
// loads and stores; the window never needs the host.
template <int CELL, int DP>
__global__ __launch_bounds__(kThreads, 1) void cell_resident_adv(ResidentArgs a) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    constexpr int PS = iterate_stride<DP>();
    constexpr int NS = kThreads / DP;            // fold segments per channel
    const int L = a.L, m = a.m, D = a.D;
    const int64_t T = a.T, W = a.W;
    const int xs = x_stride(m);
    const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int GX = gridDim.x;
    const unsigned nblocks = gridDim.x * gridDim.y;
    const bool lead = c == 0 && b == 0;
    float* S = lds;                              // [L+1][PS] rows t0-1 .. t0+L-1 of the iterate
    float* V = S + (L + 1) * PS;                 // [L][DP] f_t at the iterate
    float* CO = V + L * DP;                      // [L][DP] diagonal coefficients
    float* X = CO + L * DP;                      // [L][xs]
    float* SCR = X + L * xs;                     // [2][kThreads] fold segments
    float* S0 = SCR + 2 * kThreads;              // [DP] accepted state s_{A-1}
    float* outb = a.out + static_cast<int64_t>(b) * T * D;
    const float* s0b = a.s0 + static_cast<int64_t>(b) * D;
    CellRegs<CELL, DP> cr;
    cr.load(a.w, a.w, D, m);
    unsigned epoch = 0;
    const bool rthr = tid < D;                   // replay / composition thread of channel tid
    float own_a = 1.0f, own_b = 0.0f;
    __shared__ int row_ok;

    // the chunk of window [A, E) with the iterate's rows below Ev read from
    // out and the rest set to the fill value; returns the chunk's rows
    auto stage = [&](int64_t A, int64_t E, int64_t Ev) -> int {
        const int64_t t0 = A + static_cast<int64_t>(c) * L;
        const int Lc = t0 < E ? static_cast<int>(E - t0 < L ? E - t0 : L) : 0;
        if (tid < DP) S0[tid] = tid < D ? (A == 0 ? s0b[tid] : ld_dev(outb + (A - 1) * D + tid)) : 0.0f;
        if (Lc > 0) copy_rows_to_lds<kThreads>(X, xs, a.x + (static_cast<int64_t>(b) * T + t0) * m, m, Lc, m);
        // every element one load from its own source (kStageKB loads in
        // flight per thread before their LDS stores): row t of out below Ev,
        // the fill row Ev - 1 (s0 if Ev = 0) from Ev on, s0 before step 0
        constexpr int kStageKB = 8;
        const int n = (Lc + 1) * PS;
        for (int base = 0; base < n; base += kThreads * kStageKB) {
            float v[kStageKB];
#pragma unroll
            for (int u = 0; u < kStageKB; ++u) {
                const int e = base + u * kThreads + tid;
                const int r = e / PS, i = e - r * PS;
                const int64_t t = t0 - 1 + r;
                const bool live = e < n && i < D;
                const int ic = live ? i : 0;
                const int64_t tr = t < Ev ? t : Ev - 1;   // the row it reads
                const float* src = (tr < 0 || !live) ? s0b + ic : outb + tr * D + ic;
                const float x = ld_dev(src);
                v[u] = live ? x : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kStageKB; ++u) {
                const int e = base + u * kThreads + tid;
                if (e < n) S[e] = v[u];
            }
        }
        __syncthreads();
        return Lc;
    };
    // the chunk's rows of the iterate back to out
    auto write_rows = [&](int64_t t0, int Lc) {
        for (int e = tid; e < Lc * D; e += kThreads) {
            const int j = e / D, i = e - j * D;
            st_dev(outb + (t0 + j) * D + i, S[(j + 1) * PS + i]);
        }
    };
    // residual maximum and first step over tol of the chunk into check q's slots
    auto publish = [&](int q, uint32_t rb, uint32_t fb, int64_t rel0) {
        rb = block_max_u32(rb);
        const uint32_t nf = block_max_u32(fb == 0xffffffffu ? 0u : ~static_cast<uint32_t>(rel0 + fb));
        if (tid == 0) {
            uint32_t* sl = a.rslot + ((q % 3) * kRSlots + (b * GX + c) % kRSlots) * 64;
            __hip_atomic_fetch_max(sl, rb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_max(sl + 1, nf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    // round 0: the initial iterate s0 on [0, E), written out, and its check
    int64_t A = 0, E = T < W ? T : W;
    int Lc = stage(0, E, 0);
    {
        uint32_t rb = 0, fb = 0xffffffffu;
        if (Lc > 0) {
            cr.project(a.w, X, xs, Lc, m);
            cr.template eval<false>(S, V, CO, Lc, L, a.mode, S, rb, &fb, a.tol);
            write_rows(static_cast<int64_t>(c) * L, Lc);
        }
        publish(0, rb, fb, static_cast<int64_t>(c) * L);
    }
    if (!resident_sync(a, epoch, nblocks)) return;
    int K = 0, status = kStOk, hist_pos = 0;
    for (int i = 0, q = 0;; ++q) {
        // the check of round q (i updates so far), taken alike by every workgroup
        const int lane = tid & 63;
        const uint32_t* sl = a.rslot + ((q % 3) * kRSlots + (lane < kRSlots ? lane : 0)) * 64;
        const uint32_t rv = lane < kRSlots ? __hip_atomic_load(sl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        const uint32_t fv = lane < kRSlots ? __hip_atomic_load(sl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        const uint32_t r_q = wave_max_u32(rv);
        const uint32_t first = ~wave_max_u32(fv);
        if (lead) {
            if (tid == 0 && hist_pos < a.hist_cap) a.hist[hist_pos] = __uint_as_float(r_q);
            if (tid < kRSlots) {
                uint32_t* cl = a.rslot + (((q + 2) % 3) * kRSlots + tid) * 64;
                __hip_atomic_store(cl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(cl + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        ++hist_pos;
        if (r_q >= kNonFiniteBits) { K = i; status = kStNonFinite; break; }
        const int64_t acc = static_cast<int64_t>(first) < E - A ? static_cast<int64_t>(first) : E - A;
        if (lead && tid == 0 && q < a.acc_cap) a.acc[q] = static_cast<int32_t>(acc);
        A += acc;
        if (A >= T) { K = i; status = kStOk; break; }
        if (i >= a.max_iter) { K = i; status = kStNotConverged; break; }
        const int64_t En = T < A + W ? T : A + W;
        const int64_t t0 = A + static_cast<int64_t>(c) * L;
        if (acc != 0 || En != E) {
            // the moved window: stage the chunk at the current iterate and evaluate
            Lc = stage(A, En, E);
            if (Lc > 0) {
                uint32_t rb_unused = 0;
                cr.project(a.w, X, xs, Lc, m);
                cr.template eval<false>(S, V, CO, Lc, L, a.mode, nullptr, rb_unused, nullptr, a.tol);
            }
            __syncthreads();
        }
        E = En;
        const int NCw = static_cast<int>((E - A + L - 1) / L);
        const int par = i & 1;
        const size_t HS = static_cast<size_t>(a.B) * a.NC * D;
        float* mA = a.mapA + par * HS + static_cast<size_t>(b) * a.NC * D;
        float* mB = a.mapB + par * HS + static_cast<size_t>(b) * a.NC * D;
        // the chunk map of update i
        if (rthr && Lc > 0) {
            float Am = 1.0f, Bm = 0.0f;
            if (a.mode == kJacobi) {
                Am = 0.0f;
                Bm = V[(Lc - 1) * DP + tid];
            } else {
#pragma unroll 8
                for (int j = 0; j < Lc; ++j) {
                    const float at = CO[j * DP + tid];
                    Bm = at * Bm + (V[j * DP + tid] - at * S[j * PS + tid]);
                    Am = at * Am;
                }
            }
            own_a = Am;
            own_b = Bm;
            st_dev(mA + static_cast<size_t>(c) * D + tid, Am);
            st_dev(mB + static_cast<size_t>(c) * D + tid, Bm);
        }
        // The fold needs the maps of the chunks before this one in its row
        // only: once its own map stores have completed, the chunk stores the
        // update's tag (i + 1) into its ready word, and waits (bounded) for
        // the ready words of its row's earlier chunks instead of a grid
        // barrier.
        {
            const unsigned tag = static_cast<unsigned>(i + 1);
            unsigned* rdy = a.ready + static_cast<size_t>(b) * a.NC;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0 && Lc > 0) __hip_atomic_store(rdy + c, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (tid < 64) {
                int good = 1;
                if (Lc > 0 && c > 0) {
                    unsigned spins = 0;
                    for (;;) {
                        int done = 1;
                        for (int k = tid; k < c; k += 64)
                            done &= __hip_atomic_load(rdy + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= tag;
                        if (__all(done)) break;
                        __builtin_amdgcn_s_sleep(1);
                        if (++spins > (1u << 22) || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                            if (tid == 0) __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            good = 0;
                            break;
                        }
                    }
                }
                if (tid == 0) row_ok = good;
            }
            __syncthreads();
            if (!row_ok) return;
        }
        if (Lc > 0) {
            // the carry of chunk c: NS segments of the maps of the chunks before it
            {
                const int d = tid % DP, sg_ = tid / DP;
                const int per = (c + NS - 1) / NS;
                const int k0 = min(c, sg_ * per);
                const int k1 = d < D ? min(c, k0 + per) : k0;
                float fa = 1.0f, fbv = 0.0f;
                for (int kk = k0; kk < k1; ++kk) {
                    const float ak = ld_dev(mA + kk * D + d);
                    fbv = ak * fbv + ld_dev(mB + kk * D + d);
                    fa = ak * fa;
                }
                SCR[tid] = fa;
                SCR[kThreads + tid] = fbv;
            }
            __syncthreads();
            // replay from the carry, damping, in place: rows t0-1 .. t0+Lc-1 of the new iterate
            if (rthr) {
                const float lam = a.lam;
                const bool und = a.undamped != 0;
                const bool has_next = c + 1 < NCw;
                float xv = S0[tid];
#pragma unroll
                for (int sgi = 0; sgi < NS; ++sgi) xv = SCR[sgi * DP + tid] * xv + SCR[kThreads + sgi * DP + tid];
                const float c_next = own_a * xv + own_b;
                float pold = S[tid];
                float shat = xv;
                S[tid] = und ? shat : pold + lam * (shat - pold);
                const int nrep = has_next ? Lc - 1 : Lc;
                if (a.mode == kJacobi) {
                    for (int j = 0; j < nrep; ++j) {
                        const float so = S[(j + 1) * PS + tid];
                        const float sh = V[j * DP + tid];
                        S[(j + 1) * PS + tid] = und ? sh : so + lam * (sh - so);
                    }
                } else {
                    int j = 0;
                    for (; j + 8 <= nrep; j += 8) {
                        float v[8], co[8], po[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            v[u] = V[(j + u) * DP + tid];
                            co[u] = CO[(j + u) * DP + tid];
                            po[u] = S[(j + u + 1) * PS + tid];
                        }
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            shat = v[u] + co[u] * (shat - pold);
                            pold = po[u];
                            S[(j + u + 1) * PS + tid] = und ? shat : pold + lam * (shat - pold);
                        }
                    }
                    for (; j < nrep; ++j) {
                        shat = V[j * DP + tid] + CO[j * DP + tid] * (shat - pold);
                        pold = S[(j + 1) * PS + tid];
                        S[(j + 1) * PS + tid] = und ? shat : pold + lam * (shat - pold);
                    }
                }
                if (has_next) {
                    const float so = S[Lc * PS + tid];
                    S[Lc * PS + tid] = und ? c_next : so + lam * (c_next - so);
                }
            }
            __syncthreads();
        }
        // the check of the next round: the cell at the new iterate
        uint32_t rb = 0, fb = 0xffffffffu;
        if (Lc > 0) {
            cr.template eval<false>(S, V, CO, Lc, L, a.mode, S, rb, &fb, a.tol);
            write_rows(t0, Lc);
        }
        ++i;
        publish(q + 1, rb, fb, static_cast<int64_t>(c) * L);
        if (!resident_sync(a, epoch, nblocks)) return;
    }
    // steps the window never reached hold the last state of the window
    if (E < T) {
        const int64_t n = (T - E) * D;
        for (int64_t e = static_cast<int64_t>(c) * kThreads + tid; e < n; e += static_cast<int64_t>(GX) * kThreads) {
            const int i = static_cast<int>(e % D);
            outb[E * D + e] = ld_dev(outb + (E - 1) * D + i);
        }
    }
    if (lead && tid == 0) {
        a.win_iters[0] = K;
        a.win_status[0] = status;
        *a.hist_len = hist_pos;
    }
}

size_t resident_adv_lds_bytes(int DP, int L, int m) {
    const size_t PS = DP + 4, xs = x_stride(m);
    const size_t n = (L + 1) * PS + 2ull * L * DP + static_cast<size_t>(L) * xs + 2ull * kThreads + DP;
    return sizeof(float) * n;
}

template <int CELL, int DP>
static hipError_t resident_adv_blocks_t(size_t lds, int* nb) {
    int per_cu = 0, dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (lds > 64 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(cell_resident_adv<CELL, DP>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, cell_resident_adv<CELL, DP>, kThreads, lds);
    if (e != hipSuccess) return e;
    *nb = per_cu * ncu;
    return hipSuccess;
}

template <int CELL, int DP>
static hipError_t launch_resident_adv_t(const ResidentArgs& a, size_t lds, hipStream_t st) {
    void* args[] = {const_cast<ResidentArgs*>(&a)};
    LaunchTiming& t = launch_timing();
    if (t.start) {
        hipError_t e = hipEventRecord(t.start, st);
        if (e != hipSuccess) return e;
    }
    hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(cell_resident_adv<CELL, DP>),
                                              dim3(a.NC, a.B), dim3(kThreads), args, static_cast<unsigned>(lds), st);
    if (e != hipSuccess) return e;
    if (t.start) {
        e = hipEventRecord(t.stop, st);
        t = LaunchTiming{};
    }
    return e;
}

hipError_t cell_resident_adv_max_blocks(int kind, int DP, int L, int m, int* nb) {
    *nb = 0;
    const size_t lds = resident_adv_lds_bytes(DP, L, m);
    if (lds > 160 * 1024 || L > kMaxChunk) return hipSuccess;
#define PN_RES_CASE(K, DPV) if (kind == K && DP == DPV) return resident_adv_blocks_t<K, DPV>(lds, nb);
    PN_RES_CASE(kCellTanhRnn, 16) PN_RES_CASE(kCellTanhRnn, 32) PN_RES_CASE(kCellTanhRnn, 64)
    PN_RES_CASE(kCellGru, 16) PN_RES_CASE(kCellGru, 32) PN_RES_CASE(kCellGru, 64)
    PN_RES_CASE(kCellEuler, 16) PN_RES_CASE(kCellEuler, 32) PN_RES_CASE(kCellEuler, 64)
#undef PN_RES_CASE
    return hipSuccess;
}

hipError_t launch_cell_resident_adv(int kind, int DP, const ResidentArgs& a, hipStream_t st) {
    const size_t lds = resident_adv_lds_bytes(DP, a.L, a.m);
#define PN_RES_CASE(K, DPV) if (kind == K && DP == DPV) return launch_resident_adv_t<K, DPV>(a, lds, st);
    PN_RES_CASE(kCellTanhRnn, 16) PN_RES_CASE(kCellTanhRnn, 32) PN_RES_CASE(kCellTanhRnn, 64)
    PN_RES_CASE(kCellGru, 16) PN_RES_CASE(kCellGru, 32) PN_RES_CASE(kCellGru, 64)
    PN_RES_CASE(kCellEuler, 16) PN_RES_CASE(kCellEuler, 32) PN_RES_CASE(kCellEuler, 64)
#undef PN_RES_CASE
    return hipErrorInvalidValue;
}

size_t resident_lds_bytes(int DP, int L, int m, int cpw) {
    const size_t PS = DP + 4, xs = x_stride(m);
    const size_t per = (cpw == 1 ? 2 : 1) * (L + 1) * PS + 2ull * L * DP + static_cast<size_t>(L) * xs;
    return sizeof(float) * (cpw * per + 2ull * kThreads + DP);
}

template <int CELL, int DP, int CPW>
static hipError_t resident_blocks_t(size_t lds, int* nb) {
    int per_cu = 0, dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (lds > 64 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(cell_resident<CELL, DP, CPW>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, cell_resident<CELL, DP, CPW>, kThreads, lds);
    if (e != hipSuccess) return e;
    *nb = per_cu * ncu;
    return hipSuccess;
}

template <int CELL, int DP, int CPW>
static hipError_t launch_resident_t(const ResidentArgs& a, size_t lds, hipStream_t st) {
    void* args[] = {const_cast<ResidentArgs*>(&a)};
    LaunchTiming& t = launch_timing();
    if (t.start) {
        hipError_t e = hipEventRecord(t.start, st);
        if (e != hipSuccess) return e;
    }
    const int gx = (a.NC + CPW - 1) / CPW;
    hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(cell_resident<CELL, DP, CPW>),
                                              dim3(gx, a.B), dim3(kThreads), args, static_cast<unsigned>(lds), st);
    if (e != hipSuccess) return e;
    if (t.start) {
        e = hipEventRecord(t.stop, st);
        t = LaunchTiming{};
    }
    return e;
}

// Blocks of cell_resident with cpw chunks per workgroup that fit on the
// device at once (0 when the shape has no resident form: D padded to 16, 32
// or 64; cpw 1, or 4 at D padded to 16).
hipError_t cell_resident_max_blocks(int kind, int DP, int L, int m, int cpw, int* nb) {
    *nb = 0;
    const size_t lds = resident_lds_bytes(DP, L, m, cpw);
    if (lds > 160 * 1024 || L > kMaxChunk) return hipSuccess;
#define PN_RES_CASE(K, DPV, C) if (kind == K && DP == DPV && cpw == C) return resident_blocks_t<K, DPV, C>(lds, nb);
    PN_RES_CASE(kCellTanhRnn, 16, 1) PN_RES_CASE(kCellTanhRnn, 32, 1) PN_RES_CASE(kCellTanhRnn, 64, 1)
    PN_RES_CASE(kCellGru, 16, 1) PN_RES_CASE(kCellGru, 32, 1) PN_RES_CASE(kCellGru, 64, 1)
    PN_RES_CASE(kCellEuler, 16, 1) PN_RES_CASE(kCellEuler, 32, 1) PN_RES_CASE(kCellEuler, 64, 1)
    PN_RES_CASE(kCellTanhRnn, 16, 4) PN_RES_CASE(kCellGru, 16, 4) PN_RES_CASE(kCellEuler, 16, 4)
#undef PN_RES_CASE
    return hipSuccess;
}

hipError_t launch_cell_resident(int kind, int DP, int cpw, const ResidentArgs& a, hipStream_t st) {
    const size_t lds = resident_lds_bytes(DP, a.L, a.m, cpw);
#define PN_RES_CASE(K, DPV, C) if (kind == K && DP == DPV && cpw == C) return launch_resident_t<K, DPV, C>(a, lds, st);
    PN_RES_CASE(kCellTanhRnn, 16, 1) PN_RES_CASE(kCellTanhRnn, 32, 1) PN_RES_CASE(kCellTanhRnn, 64, 1)
    PN_RES_CASE(kCellGru, 16, 1) PN_RES_CASE(kCellGru, 32, 1) PN_RES_CASE(kCellGru, 64, 1)
    PN_RES_CASE(kCellEuler, 16, 1) PN_RES_CASE(kCellEuler, 32, 1) PN_RES_CASE(kCellEuler, 64, 1)
    PN_RES_CASE(kCellTanhRnn, 16, 4) PN_RES_CASE(kCellGru, 16, 4) PN_RES_CASE(kCellEuler, 16, 4)
#undef PN_RES_CASE
    return hipErrorInvalidValue;
}

}  // namespace pn
