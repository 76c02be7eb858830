// msscan_internal.h -- launch interface between the C ABI (api.cpp) and the
// HIP kernels (scan_lane, scan_tile, scan_kernels, decode, conv, scan_bwd).
// Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/msscan.h"

namespace msscan {

// The C ABI's shared pieces (api.cpp), for entry points in other files:
// the thread-local error text, and ms_scan_fwd's validation + launch.
void clear_error();
ms_status report(ms_status s, const char* text);  // sets the error text, returns s
ms_status scan_fwd_checked(const void* u, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* delta_bias,
                           uint32_t flags, void* y, const float* h0, float* h_last,
                           const ms_dims* dims, void* workspace, size_t workspace_bytes,
                           void* stream);

// How one ms_scan_fwd call is cut into work.  Lanes of a wave own 64
// consecutive channels; a workgroup holds `waves` waves that split the
// d_state states (`ns` per lane); the sequence is cut into `chunks` pieces of
// `chunk_len` steps each.  Pieces after the first start from a carried state
// computed by a separate pass (chunk summaries + carry propagation).
struct Plan {
    int tile_path;      // 3: scan_row kernels (a 16-lane row per channel, a state per lane);
                        // 2: scan_lane kernels (all states in a lane);
                        // 1: scan_tile kernels (waves split d_state); -1: none
    int ns;             // states per lane (compile-time variant)
    int waves;          // waves per workgroup = ceil(d_state / ns)
    int chunks;         // pieces along L
    int64_t chunk_len;  // steps per piece (last piece may be shorter)
    int tiles;          // channel tiles per batch row: ceil(d_inner / 64), or / (kRowCh / rows)
    int rows;           // row path: DPP rows per channel (1, 2, 4)
    size_t ws_floats;   // workspace floats (0 when chunks == 1)
    size_t bc_floats;   // tile path: fp32 B/C copy laid out per wave (0 if unused)
};

struct ScanArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* bias;
    const float* h0;
    float* h_last;
    void* y;
    float* agg;   // [batch][chunks-1][N][Dn]: chunk summaries, then carries
    float* sdt;   // [batch][chunks-1][Dn]: sum of dt over each chunk (exp-based A_bar)
    float* prod;  // [batch][chunks-1][N][Dn]: product of A_bar over each chunk (bilinear)
    float* bcw;   // tile path: [batch][waves][L][2*ns] fp32 B_t then C_t slices
    float* start0;  // several segments and h0 given: [batch][Dn][N] copy of h0 written by
                    // the carry pass; the first segment reads it instead of h0, so that
                    // h_last (written by the last segment in the same launch) may alias h0
    const void* dtx;  // fused dt projection: [batch][L][rank] low-rank input, io dtype
    const void* wdt;  // fused dt projection: [Dn][rank] weight, io dtype
    int rank;         // fused dt projection: columns of dtx and wdt (0: delta is given)
    int64_t L;
    int64_t chunk_len;
    int batch;
    int Dn;
    int N;
    int chunks;
    int softplus;
    int waves;    // tile path: waves per workgroup
    int tiles;    // row path: channel tiles (kRowCh channels each) per batch row
};

struct ConvArgs {
    const void* x;
    const float* w;      // [Dn][width]
    const float* bias;   // [Dn] or null
    const void* x_prev;  // [batch][width-1][Dn] or null
    void* u;
    int64_t L;
    int batch;
    int Dn;
    int width;
    int64_t tgroups, cgroups;  // set by launch_conv1d: workgroups along time and channels
};

struct StepArgs {
    float* h;
    const void* x;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* bias;
    void* y;
    int batch;
    int Dn;
    int N;
    int softplus;
};

// Each returns hipSuccess or the first launch error.
// disc: 0 Euler, 1 zero-order hold, 2 bilinear (kEuler / kZoh / kBilinear).
hipError_t launch_scan_tiles(const Plan& p, const ScanArgs& a, bool bf16, int disc, hipStream_t s);
// Segment carries: val[b][i][n][d] holds segment i's summary (state reached
// from zero); its decay is exp(A[d][n] * sdt[b][i][d]) or prod[b][i][n][d].
// Replaced in place by the composed state after slot i, taking the slots in
// order (reverse: last to first) from init[b][d][n] (null: zero).
struct CarryArgs {
    float* val;
    const float* sdt;
    const float* prod;
    const float* A;
    const float* init;
    float* start0;  // if set: receives init ([batch][Dn][N], zero when init is null)
    int batch;
    int km1;
    int N;
    int Dn;
};
constexpr int kCarryGroup = 8;         // slots whose loads one carry thread issues together
constexpr int kCarryLongChain = 1024;  // chains this long are split over several waves
hipError_t launch_carry(const CarryArgs& c, bool reverse, hipStream_t s);
hipError_t launch_carry(const ScanArgs& a, hipStream_t s);  // the forward summaries of a
bool tile_variant_exists(int ns, int waves);
// Row path (scan_row.hip, scan_row_wide.hip): a channel on 1, 2 or 4 16-lane
// DPP rows of one wave (d_state up to 16, 32 or 64; 128 with two states per
// lane); a workgroup is kRowWaves waves, kRowCh rows: kRowCh / rows channels.
constexpr int kRowWaves = 4;            // waves per workgroup
constexpr int kRowCh = 4 * kRowWaves;   // rows per workgroup (channels at one row each)
hipError_t launch_scan_rows(const Plan& p, const ScanArgs& a, bool bf16, int disc, hipStream_t s);
// several rows per channel (plan waves = kRowWaves * rows, ns = 16 * rows * states per lane)
hipError_t launch_scan_rows_wide(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                 hipStream_t s);
hipError_t launch_scan_lanes(const Plan& p, const ScanArgs& a, bool bf16, int disc, hipStream_t s);
bool lane_variant_exists(int n, int disc);
// Lane path with the low-rank dt projection fused in (a.dtx, a.wdt, a.rank).
hipError_t launch_scan_lanes_dtproj(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                    hipStream_t s);
bool dtproj_variant_exists(int n);
// The row kernel with the projection fused in (scan_row_dtproj.hip): a row
// plan with one row per channel; d_inner a multiple of 8 (bf16) or 4 (fp32).
hipError_t launch_scan_rows_dtproj(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                   hipStream_t s);
// The forward that also stores the backward's checkpoints into a.agg
// ([batch][ceil(L / 16)][Dn][N], scan_row_ckpt.hip): a row plan with one row
// per channel and one segment; d_inner a multiple of 8 (bf16) or 4 (fp32).
hipError_t launch_scan_rows_ckpt(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                 hipStream_t s);
hipError_t launch_bc_prepare(const ScanArgs& a, int np, bool bf16, hipStream_t s);  // rows np wide
// Causal depthwise conv1d (+ silu), width 1..8.  One-dimensional grid of
// conv_workgroups(a) workgroups, at most kMaxConvWorkgroups.
constexpr int64_t kMaxConvWorkgroups = 0x7fffffffLL;
int64_t conv_workgroups(const ConvArgs& a);
hipError_t launch_conv1d(const ConvArgs& a, bool bf16, bool silu, hipStream_t s);
// Decode step with 4 states per lane (d_state in {4, 8, ..., 128}).
bool step_quads_supported(int batch, int d_inner, int n);
hipError_t launch_step_quads(const StepArgs& a, bool bf16, int disc, hipStream_t s);

// Gradients (scan_bwd.hip).  f carries the forward inputs, with f.agg and
// f.sdt / f.prod holding the forward segment starts of a plan whose segments
// are bwd_segment_len() steps (computed first by launch_summary_carry).
struct BwdLaunch {
    ScanArgs f;
    const void* dy;
    const float* dh_last;
    void* du;
    void* ddelta;
    void* dz;
    float* dh0;
    float* dA;
    float* dB;
    float* dC;
    float* dD;
    float* dbias;
    float* mu;
    float* sdt_b;
    float* prod_b;
    float* pbc;
    float* pparam;
    float* pgroup;  // [kParamGroups][Dn][N+2]: first-level sums of pparam
    bool bf16;
    int disc;
    // fp32 [batch][L][Dn] or null: receives sum_n C h + D u of every element
    // (ypart_add: added to what it holds), from the gradient pass's recompute
    float* ypart = nullptr;
    int ypart_add = 0;
    // fp32 io only: du and ddelta are added to what their buffers hold
    int out_add = 0;
};
int bwd_segment_len();
constexpr int kParamGroups = 16;  // first-level groups of the parameter sums
constexpr int kBwdWaves = 4;  // backward segments per workgroup (one wave each)
hipError_t launch_scan_bwd(const BwdLaunch& L, hipStream_t s);
// The fixed-order sums that end every backward: dB | dC over `tiles` tile
// partials [tiles][batch][L][2N], dA | dD | dbias over the batch x
// ceil(f.chunks / kBwdWaves) rows of pparam [rows][Dn][N+2] (first in
// kParamGroups groups, into pgroup, then the groups in order).
hipError_t launch_bwd_reductions(const ScanArgs& f, float* pbc, int tiles, float* pparam,
                                 float* pgroup, float* dA, float* dB, float* dC, float* dD,
                                 float* dbias, hipStream_t s);
// Row-layout backward for d_state 9..16 (bwd_row.hip): a checkpointing
// forward walk, the reverse walk over 16-channel tiles, then the sums above.
// f.tiles = ceil(Dn / kRowCh); d_inner a multiple of 8 (bf16 io) or 4 (fp32).
struct BwdRowLaunch {
    ScanArgs f;
    const void* dy;
    const float* dh_last;
    void* du;
    void* ddelta;
    void* dz;
    float* dh0;
    float* dA;
    float* dB;
    float* dC;
    float* dD;
    float* dbias;
    float* ckpt;    // [batch][ceil(L / 16)][Dn][N]: the state before each 16-step block
    bool walk;      // compute ckpt first (false: it holds the forward's checkpoints; only read)
    float* pbc;     // [tiles][batch][L][2N]
    float* pparam;  // [batch][Dn][N+2]
    float* pgroup;  // [kParamGroups][Dn][N+2]
    bool bf16;
    int disc;
};
hipError_t launch_scan_bwd_rows(const BwdRowLaunch& L, hipStream_t s);

// Backward for d_state 17..128 (bwd_wide.hip): the state is differentiated
// in slices of kWideSlice states by the kernels above, run as fp32 problems
// with the gate and D taken out; these helpers prepare, gather, accumulate
// and combine.  Sizes: E = batch*L*Dn, BL = batch*L, BD = batch*Dn,
// BLN = batch*L*N.
constexpr int kWideSlice = 16;
constexpr int kWideGroups = 64;  // row groups of the dD partial sums
struct WideArgs {
    const void* u;
    const void* delta;
    const float* A;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const void* dy;
    const float* h0;
    const float* dh_last;
    int64_t E, BL, BD, BLN;
    int Dn, N;
    // workspace (fp32)
    float *g, *u32, *d32, *B32, *C32, *y32;
    int y32_add_du;  // y32 holds sum_n C h only: the combine adds D u
    float *As, *Bs, *Cs, *h0s, *dhls;
    float *du_s, *dv_s, *dAs, *dBs, *dCs, *dbias_s, *dh0s;
    float *du_acc, *dv_acc, *dbias_acc, *dD_part;
    // outputs
    void *du, *ddelta, *dz;
    float *dA, *dB, *dC, *dD, *dbias, *dh0;
};
hipError_t launch_wide_prep(const WideArgs& w, bool bf16, hipStream_t s);
hipError_t launch_wide_gather(const WideArgs& w, int n0, bool bf16, hipStream_t s);
hipError_t launch_wide_accumulate(const WideArgs& w, int n0, bool add_du, hipStream_t s);
hipError_t launch_wide_finish(const WideArgs& w, bool bf16, hipStream_t s);

// Kernel timing hooks (profile.cpp).  prof_call starts a new timed call;
// ProfScope records the phase's begin event at construction and its end
// event at destruction, around one kernel launch.  Both do nothing unless a
// profile is open.  Phase numbers are the ms_phase values of msscan.h.
void prof_call();
void prof_mark(hipStream_t s, int phase, int edge);
enum : int {
    kPhasePrep = 0,
    kPhaseSummary = 1,
    kPhaseCarry = 2,
    kPhaseMain = 3,
    kPhaseStep = 4,
    kPhaseConv = 5,
    kPhaseReduce = 6
};
struct ProfScope {
    hipStream_t s;
    int phase;
    ProfScope(hipStream_t s_, int phase_) : s(s_), phase(phase_) { prof_mark(s, phase, 0); }
    ~ProfScope() { prof_mark(s, phase, 1); }
    ProfScope(const ProfScope&) = delete;
    ProfScope& operator=(const ProfScope&) = delete;
};

}  // namespace msscan
