// msscan_internal.h -- launch interface between the C ABI (api.cpp) and the
// HIP kernels (scan_lane, scan_tile, scan_kernels, decode, conv, scan_bwd).
// Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msscan {

// How one ms_scan_fwd call is cut into work.  Lanes of a wave own 64
// consecutive channels; a workgroup holds `waves` waves that split the
// d_state states (`ns` per lane); the sequence is cut into `chunks` pieces of
// `chunk_len` steps each.  Pieces after the first start from a carried state
// computed by a separate pass (chunk summaries + carry propagation).
struct Plan {
    int tile_path;      // 2: scan_lane kernels (all states in a lane);
                        // 1: scan_tile kernels (waves split d_state); -1: none
    int ns;             // states per lane (compile-time variant)
    int waves;          // waves per workgroup = ceil(d_state / ns)
    int chunks;         // pieces along L
    int64_t chunk_len;  // steps per piece (last piece may be shorter)
    int tiles;          // ceil(d_inner / 64)
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
    int batch;
    int km1;
    int N;
    int Dn;
};
constexpr int kCarryGroup = 8;  // slots whose loads one carry thread issues together
hipError_t launch_carry(const CarryArgs& c, bool reverse, hipStream_t s);
hipError_t launch_carry(const ScanArgs& a, hipStream_t s);  // the forward summaries of a
bool tile_variant_exists(int ns, int waves);
hipError_t launch_scan_lanes(const Plan& p, const ScanArgs& a, bool bf16, int disc, hipStream_t s);
bool lane_variant_exists(int n, int disc);
// Lane path with the low-rank dt projection fused in (a.dtx, a.wdt, a.rank).
hipError_t launch_scan_lanes_dtproj(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                    hipStream_t s);
bool dtproj_variant_exists(int n);
hipError_t launch_bc_prepare(const ScanArgs& a, int np, bool bf16, hipStream_t s);  // rows np wide
// Causal depthwise conv1d (+ silu), width 1..8.
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
};
int bwd_segment_len();
constexpr int kParamGroups = 16;  // first-level groups of the parameter sums
constexpr int kBwdWaves = 4;  // backward segments per workgroup (one wave each)
hipError_t launch_scan_bwd(const BwdLaunch& L, hipStream_t s);

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
    kPhaseConv = 5
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
