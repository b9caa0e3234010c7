// Internal declarations shared by the host driver (pn_api.cpp) and the HIP
// kernel files.  Not part of the public interface (include/pn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pn {

constexpr int kThreads = 256;          // threads per workgroup of every tile kernel
constexpr uint32_t kNonFiniteBits = 0x7f800000u;

// Device-side control word of one solve, written by the check (block 0 of the
// carry kernel) and read by the next apply launch.
struct Ctrl {
    int32_t stop;      // 1: the iteration loop is over, apply launches exit at once
    int32_t status;    // PN_OK / PN_NOT_CONVERGED / PN_NONFINITE, or -1 (running)
    int32_t iter;      // iteration index i of the last check
    uint32_t r_bits;   // bit pattern of r_i = max |F| (non-negative float)
    // Sweeps that take their own check (CellArgs::fc): r_k is reduced into
    // the kRSlots words rmax[k % 3][q][0] by device-scope atomic max, each
    // workgroup of the sweep that produces it into slot (workgroup % kRSlots);
    // the sweep that reads set k % 3 (plain loads: the set is not written
    // while it is read) clears set (k + 2) % 3 for the sweep after it, with
    // device-scope atomic stores.  Each word has a 256-byte line of its own.
    // The resident solver's grid-barrier timeout flag.
    uint32_t bar_err;
    uint32_t pad_[59];
    uint32_t rmax[3][16][64];
};
constexpr int kRSlots = 16;

// Host-visible copy (pinned, mapped) of the same record.  The device writes
// the payload, then epoch, then iter; the host polls (epoch, iter).
struct HostRec {
    int32_t stop;
    int32_t status;
    uint32_t r_bits;
    uint32_t first;    // advancing window: first step (window-relative) with r_t > tol
    int32_t epoch;
    int32_t iter;
};

// Records of consecutive checks of a window go to kHostRing host records in
// turn (check i to record i % kHostRing): a sweep that runs ahead of the
// host's reading (CellArgs::fc) cannot overwrite a record not yet read.
constexpr int kHostRing = 4;

// Arguments of the per-check decision, evaluated on the device.
struct CheckArgs {
    const uint32_t* rpart;   // per-block residual maxima of the previous pass
    const uint32_t* fpart;   // per-block first step with r_t > tol (advancing window), or null
    int32_t advancing;       // 1: only reduce and publish; the host takes the decision
    int32_t nparts;
    int32_t iter;            // i: number of updates applied so far
    int32_t max_iter;
    float tol;
    Ctrl* ctrl;
    HostRec* host;           // device-usable pointer to pinned host memory
    int32_t epoch;           // call sequence number, echoed to the host record
};

// ---------------------------------------------------------------- elementwise cell
struct DiagArgs {
    const float* a;          // [D]
    const float* x;          // window base; row stride D (m == D), batch stride xs
    int64_t xs;
    float* s;                // window base of out; row stride D, batch stride ss
    int64_t ss;
    const float* s0;         // initial state of the window; batch stride s0s
    int64_t s0s;
    int32_t B, Tw, D, L, NC, cpb;
    float* aggA;             // [B][NC][D]
    float* aggB;             // [B][NC][D]
    const float* carry;      // [B][NC][D]
    const float* carryr[3];  // [B][NC][D] carries of iterations 0, 1, 2 (the recomputing passes)
    float* halo;             // [2][B][NC][D]
    uint32_t* rpart;         // one slot per workgroup
    const Ctrl* ctrl;
    int32_t mode, iter, undamped;
    float lam;
    int32_t half;            // x and s hold IEEE binary16 (strides in elements): 1 one
                             // channel per thread, 2 channel pairs (D even); 0 float
    int32_t force;           // run even when the control word says stop (the store of s^(1))
    // Carries and halo were written on a chunking rf times finer (NCr chunks
    // per batch row): this launch's chunk c reads them at chunk c * rf.
    int32_t rf, NCr;
    int64_t hs;              // halo parity stride in elements (B x the finest NC x D)
    uint32_t* fpart;         // advancing window: per-block first step with r_t > tol
                             // (window-relative; 0xffffffff if none), or null
    float tol;
};

// ---------------------------------------------------------------- matrix cells
// Prepared (transposed, zero-padded) weights live in the workspace:
//   tanh RNN: WT[DP][DP] | UT[m][DP] | bias[DP] | wdiag[DP]
//   GRU     : WhT[3][DP][DP] | WiT[3][m][DP] | bih[3][DP] | bhh[3][DP] | whdiag[3][DP]
struct CellArgs {
    const float* w;          // prepared weights
    const float* x;          // window base; row stride m, batch stride xs
    int64_t xs;
    float* s;                // window base of out; row stride D, batch stride ss
    int64_t ss;
    const float* s0;
    int64_t s0s;
    int32_t B, Tw, D, m, L, NC;
    float* aggA;             // diag: [B][NC][D]; dense: [B][NC][D][D] (row-major M)
    float* aggB;             // [B][NC][D]
    const float* carry;      // [B][NC][D]
    float* halo;             // [2][B][NC][D]
    uint32_t* rpart;
    Ctrl* ctrl;
    int32_t mode, iter, undamped;
    float lam;
    int32_t band;            // Jacobian half-bandwidth (dense modes; Newton: D)
    uint32_t* fpart;         // advancing window: per-block first step with r_t > tol
                             // (window-relative; 0xffffffff if none), or null
    float tol;
    // fc (diagonal modes with at most kFcMaxChunks chunks per row: both bits;
    // the matrix-core Newton and banded sweeps at D padded to 16 or 32:
    // kFcCheck alone), bits:
    // kFcCarry: no carry launch; every apply sweep composes the carry of its
    //   chunk from the chunk maps, which for iteration k are at aggA/aggB +
    //   (k & 1) * mstride (a maps pass launched with iter k writes set k & 1);
    // kFcCheck: every apply sweep also takes the check of its iteration from
    //   ctrl->rmax and publishes it (block 0) to ctrl and host.
    int32_t fc;
    // maps pass of the advancing window: the last fill_rows rows of the
    // window are new steps; the pass starts them from the state before them
    // (stored in s) and writes them (0: none)
    int32_t fill_rows;
    int32_t max_iter;
    int32_t epoch;
    int64_t mstride;
    HostRec* host;
};

constexpr int kFcMaxChunks = 128;
constexpr int kFcMaxBlocks = 16384;      // workgroups of one sweep (B x chunks)
constexpr int kFcCarry = 1, kFcCheck = 2;
// chunks (B x NC) up to which a matrix-core sweep runs two wavefronts per chunk
constexpr int kSplitMax = 1024;

struct CarryArgs {
    const float* aggA;
    const float* aggB;
    float* carry;
    const float* s0;
    int64_t s0s;
    int32_t B, D, NC;
    int32_t do_check;
    CheckArgs chk;
    // launches queued ahead of the check their sweep takes: with stop_on
    // set, a launch that finds its stop word set does nothing (null: never)
    const Ctrl* stop_on;
};

// kPrologue: iteration-0 chunk maps at s^(0) = s0 (implicit);  kFirst /
// kSteady: apply for i = 0 / i >= 1;  kMaps: chunk maps, residual and halo
// of the iterate stored in s (the advancing window, after it slides).
// Channel-wise cell only, the recomputing passes: the apply for i = 1, 2, 3
// that recomputes s^(1) .. s^(i) from the carries of iterations 0 .. i-1
// instead of reading s^(i) (kSecondR, kThirdR, kFourthR), and the passes
// that store nothing: kFirstNS (kFirst without the store of s^(1)), kSecondNS
// and kThirdNS (see pn_diag.hip).
enum Phase { kPrologue = 0, kFirst = 1, kSteady = 2, kMaps = 3, kFirstNS = 4, kSecondR = 5, kSecondNS = 6,
             kThirdR = 7, kThirdNS = 8, kFourthR = 9 };

// iterates a pass recomputes (0 for the passes that start from s0 or read s^(i))
__host__ __device__ constexpr int recompute_depth(int phase) {
    return phase == kSecondR || phase == kSecondNS ? 1 : phase == kThirdR || phase == kThirdNS ? 2
                                                       : phase == kFourthR ? 3 : 0;
}

// Timing request for the next steady apply launch of this thread: the
// launcher records these events around the kernel itself and clears them.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming& launch_timing();

// Launchers (return the hipError_t of the launch).
hipError_t launch_diag_tanh_pass(int phase, const DiagArgs& a, hipStream_t st);
int diag_tanh_nblocks(const DiagArgs& a);
hipError_t launch_diag_carry(const CarryArgs& a, hipStream_t st);
hipError_t launch_dense_carry(const CarryArgs& a, hipStream_t st);
hipError_t launch_check(const CheckArgs& c, hipStream_t st);
hipError_t launch_fill_half(void* out, int64_t ss, const float* s0, int64_t s0s, int B, int Tw, int D,
                            hipStream_t st);
hipError_t launch_fill(float* out, int64_t ss, const float* s0, int64_t s0s, int B, int Tw, int D,
                       hipStream_t st);

// with_kcopy: also write the k-contiguous copy (read by the tile kernel only)
hipError_t launch_prep_weights(int kind, const float* params, float* w, int D, int DP, int m, bool with_kcopy,
                               hipStream_t st);
__host__ __device__ size_t prepared_weight_floats(int kind, int DP, int m);
// The whole prepared region in the workspace: the layout above and, for DP a
// multiple of 16, a copy of the weight matrices with k contiguous per
// (gate, i) row, from which the register-resident evaluation loads float4s.
__host__ __device__ size_t prepared_total_floats(int kind, int DP, int m);
hipError_t launch_cell_pass(int kind, int DP, bool dense, int phase, const CellArgs& a,
                            hipStream_t st);
size_t cell_pass_lds_bytes(int kind, int DP, bool dense, int L, int m);
bool cell_pass_stages_weights(int kind, int DP, bool dense, int L, int m);
int cell_pass_nblocks(const CellArgs& a);
// Newton on the matrix cores (D padded to 16 or 32): one wavefront per chunk.
bool dense_mfma_supported(int kind, int DP, int m);
size_t dense_mfma_lds_bytes(int kind, int DP, int m);
hipError_t launch_dense_mfma_pass(int kind, int DP, int phase, const CellArgs& a, hipStream_t st);

// Persistent solver (matrix cells, diagonal modes): one cooperative launch runs
// every window and iteration with grid-wide barriers between phases.
struct PersistArgs {
    CellArgs g;              // per-window fields are filled in by the kernel
    const float* x0;         // x at t = 0
    float* s_base;           // out at t = 0
    const float* s0_user;    // s0 of the first window (batch stride D)
    int64_t T;
    int32_t W, nwin;
    float tol;
    int32_t max_iter;
    unsigned* bar;           // grid barrier arrival counter (zeroed before launch)
    unsigned* err;           // set when a barrier times out; every block then exits
    int32_t* win_iters;      // [nwin] updates per window (-1 = not reached)
    int32_t* win_status;     // [nwin]
    float* hist;             // residual history r_0..r_K of each window, appended
    int32_t hist_cap;
    int32_t* hist_len;
};
bool cell_persist_eligible(int kind, int DP, int L, int m);
hipError_t cell_persist_max_blocks(int kind, int DP, int L, int m, int* nblocks);
hipError_t launch_cell_persist(int kind, int DP, int nblocks, const PersistArgs& a, hipStream_t st);

// Static device scratch of pn_eval_noalloc (pn_static.hip): its device
// address on the current device (looked up once per device) and its size.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void** ptr, size_t* bytes);

// One-workgroup solver (pn_small.hip): matrix cells with D <= 8 whose window
// holds at most small_max_pairs_for(D) (b, t) pairs; every window, iteration
// and check in one launch.  Results go to device memory: per window the
// updates (-1: not reached) and status, and the residual history.
struct SmallArgs {
    const float* params;
    const float* x;          // [B][T][m]
    const float* s0;         // [B][D]
    float* out;              // [B][T][D]
    int64_t T;
    int32_t W, nwin, B, D, m, mode, band, max_iter, undamped;
    float tol, lam;
    int32_t* win_iters;      // [nwin]
    int32_t* win_status;     // [nwin]
    int32_t* hist_len;       // checks taken (the history keeps the first hist_cap)
    float* hist;
    int32_t hist_cap;
};
int small_max_pairs_for(int D);
hipError_t launch_small_solve(int kind, bool dense, const SmallArgs& a, hipStream_t st);

// Resident solver (pn_cell.hip, cell_resident): the whole solve of a matrix
// cell in a diagonal mode as one cooperative launch of B x NC co-resident
// workgroups that keep their chunk on chip; see the kernel's comment.
struct ResidentArgs {
    const float* w;          // prepared weights (global)
    const float* x;          // [B][T][m]
    float* out;              // [B][T][D]
    const float* s0;         // [B][D]
    int64_t T;
    int32_t W, nwin, B, D, m, L, NC, mode, undamped, max_iter;
    float lam, tol;
    float* mapA;             // [3][B][NC][D] chunk maps by publication (the
    float* mapB;             //   advancing window: [2][B][NC][D] by parity)
    float* halo;             // [3][B][NC][D] last row of every chunk, alike
    float* s0n;              // [B][D] initial state of the next window
    uint32_t* rslot;         // [3][kRSlots][64] residual maxima, one 256-byte line per slot
    unsigned* bar;           // [B * NC] grid barrier arrival words (zero at launch)
    unsigned* err;           // set on a barrier timeout
    int32_t* win_iters;      // [nwin] (-1: not reached)
    int32_t* win_status;
    int32_t* hist_len;
    float* hist;
    int32_t hist_cap;
    int32_t* acc;            // advancing window: steps accepted at each check
    int32_t acc_cap;
    unsigned* ready;         // [B * NC] chunk-map ready words (zero at launch)
    unsigned long long* rword;  // consecutive windows: [4][workgroups] (tag << 32 | residual bits)
    unsigned* s0ready;       // consecutive windows: [B] windows whose final state is in s0n
};

// cpw: chunks per workgroup (1, or 4 at D padded to 16); the grid is
// ceil(NC / cpw) x B workgroups
hipError_t cell_resident_max_blocks(int kind, int DP, int L, int m, int cpw, int* nb);
hipError_t launch_cell_resident(int kind, int DP, int cpw, const ResidentArgs& a, hipStream_t st);
// The advancing window as one cooperative launch: one chunk of L steps per
// workgroup, grid NC x B with NC = ceil(W / L).
hipError_t cell_resident_adv_max_blocks(int kind, int DP, int L, int m, int* nb);
hipError_t launch_cell_resident_adv(int kind, int DP, const ResidentArgs& a, hipStream_t st);

// Standalone affine scan.
struct ScanArgs {
    const float* A;          // diag [B][T][D] or dense [B][T][D][D]
    const float* b;          // [B][T][D]
    float* out;              // [B][T][D]
    int32_t B, T, D, L, NC;
    float* aggA;
    float* aggB;
    const float* carry;
};
hipError_t launch_scan_aggregate(bool dense, int DP, const ScanArgs& a, hipStream_t st);
hipError_t launch_scan_apply(bool dense, int DP, const ScanArgs& a, hipStream_t st);

// Diagonal scan in one pass with a decoupled look-back (pn_scan.hip).
constexpr int kLbChunk = 32;       // steps per chunk (held in registers)
constexpr int kLbChannels = 256;   // channels per workgroup (one per thread)
struct LookbackArgs {
    const float* A;          // [B][T][D]
    const float* b;          // [B][T][D]
    const float* s0;         // [B][D]
    float* out;              // [B][T][D]
    int32_t B, T, D, L, NC, nblk;
    float* aggA;             // [B][NC][D] chunk maps
    float* aggB;
    float* yv;               // [B][NC][D] state at the end of each chunk
    uint32_t* flag;          // [B][NC][nblk]: 0 nothing, 1 map published, 2 end state published
    uint32_t* ticket;        // workgroup order (zero at launch)
    uint32_t* err;           // set when a look-back wait times out
};
hipError_t launch_scan_lookback(const LookbackArgs& a, hipStream_t st);

}  // namespace pn
