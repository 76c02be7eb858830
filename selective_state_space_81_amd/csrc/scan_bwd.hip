// scan_bwd.hip -- gradients of the selective scan (ms_scan_bwd), for
// training, d_state <= 16.
//
// The reverse-mode derivative of the forward scan.  With lambda_t = dL/dh_t
// and g_t = dL/dy_pre_t (y_pre = sum_n C h + D u, before the gate),
//
//   lambda_t = C_t g_t + mu_t,   mu_t = A_bar_{t+1} lambda_{t+1}
//
// runs backwards in time, and every input collects its terms per step:
//   dC_t += g_t h_t          dB_t += lambda_t f_t u_t        du_t += lambda_t f_t B_t + g_t D
//   d(A_bar) = lambda_t h_{t-1},  d(f) = lambda_t B_t u_t  ->  ddt, dA
// (f is the B*u factor of the discretisation: dt, (e^{dt A}-1)/A or
// dt/(1-dt A/2)).  The pages train the model end to end (jsqmd page, section
// 4.2; lmnt page, section 4.2) but print no derivative; this is the chain rule
// applied to the forward recurrence.
//
// Parallel plan, mirroring the forward: the sequence is cut into segments of
// kSeg steps.
//   1. seg_summaries: per segment, from a zero state its forward end state
//      and, from mu = 0 at its end, the mu the adjoint passes left (beta),
//      with the segment decay; bf16 inputs are staged in LDS first;
//   2. carry_chain<false> composes the forward ones into every segment's
//      starting state, carry_chain<true> the adjoint ones (last segment first)
//      into the mu entering each segment from the right;
//   3. bwd_main (one wave per segment, kBwdWaves consecutive segments of
//      one 64-channel tile per workgroup): the forward states are recomputed from its
//      starting state (the start and the state half way kept in registers,
//      each sub-block's states recomputed from them), and the adjoint runs
//      back over the segment producing every gradient.  The
//      per-step sums over channels of dB and dC are reduced across the wave
//      through LDS and stored per 64-channel tile; the sums over time of dA,
//      dD and dbias are added over the workgroup's segments in LDS and
//      stored per workgroup;
//   4. small passes add those partials in a fixed order.
// No pass waits on another workgroup: the results are deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "dpp_common.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

#ifndef MSSCAN_SEGSUM_UNROLL
#define MSSCAN_SEGSUM_UNROLL 4  // steps per unrolled body of the summary walks
#endif
constexpr int kSeg = 16;  // timesteps per backward segment
// Timesteps per recomputed sub-block: 4, except 2 for ZOH and bilinear with
// fp32 io, whose per-state factors and unstaged inputs need more registers
// (half the recomputed states held, at the price of more recompute, instead
// of spilling).
template <int DISC, bool BF16>
constexpr int sub_len() { return (DISC == kEuler || BF16) ? 4 : 2; }

// Per-state derivatives of the discretisation: A_bar, the B*u factor f, and
// their partial derivatives w.r.t. dt and a (the continuous A), from
// t = dt*a*log2(e), invA = 1/a (0 at a = 0), a2 = a*log2(e).
template <int DISC>
struct Disc {
    float abar, f, dab_dt, dab_da, df_dt, df_da;
    __device__ __forceinline__ Disc(float dt, float t, float a2, float invA) {
        const float a = a2 * kLn2;
        if constexpr (DISC == kBilinear) {
            const float r = bilinear_r(t);
            const float r2 = r * r;
            abar = fmaf(2.f, r, -1.f);
            f = dt * r;
            dab_dt = a * r2;
            dab_da = dt * r2;
            df_dt = r2;
            df_da = 0.5f * dt * dt * r2;
        } else {
            abar = hw_exp2(t);
            dab_dt = a * abar;
            dab_da = dt * abar;
            if constexpr (DISC == kZoh) {
                f = zoh_factor(dt, t, abar, invA);
                df_dt = abar;
                // (dt A_bar - f)/a, or near a = 0 its series dt^2 (1/2 + x/3 + x^2/8)
                const float x = t * kLn2;
                const float ser = dt * dt * fmaf(x, fmaf(x, 0.125f, 1.f / 3.f), 0.5f);
                df_da = fabsf(t) < kZohSwitch ? ser : (dt * abar - f) * invA;
            } else {
                f = dt;
                df_dt = 1.f;
                df_da = 0.f;
            }
        }
    }
};

// Kernel arguments beyond the forward's.
struct BwdArgs {
    ScanArgs f;          // forward inputs; f.agg/f.sdt/f.prod: forward segment starts
    const void* dy;      // [batch][L][Dn] io
    const float* dh_last;
    void* du;            // [batch][L][Dn] io
    void* ddelta;        // [batch][L][Dn] io
    void* dz;            // [batch][L][Dn] io or null
    float* dh0;          // [batch][Dn][N] or null
    float* mu;           // [batch][K-1][N][Dn]: beta, then the mu entering each segment
    float* sdt_b;        // [batch][K-1][Dn] decay sums of segments 1..K-1 (exp-based)
    float* prod_b;       // [batch][K-1][N][Dn] decay products (bilinear)
    float* pbc;          // [tiles][batch][L][2N]: per-tile partial dB | dC
    float* pparam;       // [batch][ceil(K/kBwdWaves)][Dn][N+2]: partial dA | dD | dbias per group
    float* pgroup;       // [kParamGroups][Dn][N+2]: first-level sums of pparam
    float* ypart;        // [batch][L][Dn] fp32 or null: y_pre of each element, stored
    int ypart_add;       //   or (ypart_add) added to what the buffer holds
    int out_add;         // fp32 io: du and ddelta added to what their buffers hold
};

template <bool BF16>
__device__ __forceinline__ float ldio(const void* p, int64_t i) {
    return ld<BF16>(p, i);
}

// The softplus and z-gate options are wave-uniform flags.  Branching on them
// per step split the step loops into many small blocks; instead both forms
// are computed and one is kept by a mask (all ones: `on`, zero: `off`), so a
// step stays one straight-line block.
__device__ __forceinline__ float pick(uint32_t mask, float on, float off) {
    return __uint_as_float((__float_as_uint(on) & mask) | (__float_as_uint(off) & ~mask));
}
__device__ __forceinline__ float step_pick(float draw, float bias, uint32_t spm) {
    const float v = draw + bias;
    return pick(spm, softplus_f(v), v);
}

// Orders one wave's LDS accesses across its lanes.  Each wave of a workgroup
// works in LDS rows of its own, so no workgroup barrier is needed: the
// fences keep the compiler from moving LDS accesses across this point, and
// lgkmcnt(0) waits until the wave's LDS writes are done.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The raw bf16 inputs of steps [t0, t1) of one 64-channel tile, staged in
// LDS by one batch of loads: s_io[k][j][lane] for k = u, delta, z, dy and
// s_bc[k][j][state] for k = B, C (states past N zero; rows past t1 zero).
__device__ __forceinline__ void stage_segment(const BwdArgs& a, int64_t row0, int64_t t0,
                                              int64_t t1, int dd, int lane, uint16_t* s_io,
                                              uint16_t* s_bc) {
    const ScanArgs& f = a.f;
    using R = Io<true>;
    const int N = f.N;
    const uint32_t rowb = (uint32_t)f.Dn * 2u;
    const uint32_t nrows = (uint32_t)(t1 - t0);
    auto seg = [&](const void* p, uint32_t rb) {
        return make_rsrc(static_cast<const char*>(p) + (row0 + t0) * (int64_t)rb, nrows * rb);
    };
    const auto rU = seg(f.u, rowb), rD = seg(f.delta, rowb), rY = seg(a.dy, rowb);
    const auto rZ = f.z ? seg(f.z, rowb) : make_rsrc(f.u, 0u);
    const uint32_t off = (uint32_t)dd * 2u;
    uint16_t vu[kSeg], vd[kSeg], vz[kSeg], vy[kSeg];
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
        const uint32_t o = off + (uint32_t)j * rowb;
        vu[j] = R::load(rU, o);
        vd[j] = R::load(rD, o);
        vz[j] = R::load(rZ, o);
        vy[j] = R::load(rY, o);
    }
    // lane l takes state l & 15 of step 4k + (l >> 4)
    const uint32_t bcrow = (uint32_t)N * 2u;
    const auto rB = seg(f.B, bcrow), rC = seg(f.C, bcrow);
    const int st = lane & 15, sr = lane >> 4;
    uint16_t vb[kSeg / 4], vc[kSeg / 4];
#pragma unroll
    for (int k = 0; k < kSeg / 4; ++k) {
        const uint32_t o = st < N ? (uint32_t)(4 * k + sr) * bcrow + (uint32_t)st * 2u : kOutOfRange;
        vb[k] = R::load(rB, o);
        vc[k] = R::load(rC, o);
    }
#pragma unroll
    for (int j = 0; j < kSeg; ++j) {
        s_io[(0 * kSeg + j) * 64 + lane] = vu[j];
        s_io[(1 * kSeg + j) * 64 + lane] = vd[j];
        s_io[(2 * kSeg + j) * 64 + lane] = vz[j];
        s_io[(3 * kSeg + j) * 64 + lane] = vy[j];
    }
#pragma unroll
    for (int k = 0; k < kSeg / 4; ++k) {
        s_bc[(0 * kSeg + 4 * k + sr) * 16 + st] = vb[k];
        s_bc[(1 * kSeg + 4 * k + sr) * 16 + st] = vc[k];
    }
    wave_sync();
}

// ---- 1+2. segment summaries, forward and adjoint, in one pass -----------------
// Per 16-step segment s (blockIdx.y) of one 64-channel tile:
//   s < K-1 : the forward state at its end from a zero start (f.agg slot s)
//             and its decay (sum of dt, or the product of A_bar per state);
//   s >= 1  : from mu = 0 at its end, the adjoint run back over it gives the
//             mu passed left (beta, a.mu slot s-1) and the same decay.
// Both come from one walk of the segment in time order.
// The carries then compose them (forward: carry_chain<false>; adjoint:
// carry_chain<true>).
template <int NS, bool BF16, int DISC>
__global__ void __launch_bounds__(64, (BF16 && DISC != kZoh) ? 4 : 3) seg_summaries(BwdArgs a) {
    const ScanArgs& f = a.f;
    const int lane = threadIdx.x;
    const int b = blockIdx.z;
    const int s = blockIdx.y;
    const int d = blockIdx.x * 64 + lane;
    const bool dvalid = d < f.Dn;
    const int dd = dvalid ? d : f.Dn - 1;
    const int N = f.N;
    const int km1 = f.chunks - 1;
    const bool do_fwd = s < km1, do_bwd = s >= 1;
    const int jn = lane & (NS - 1);
    constexpr bool BIL = DISC == kBilinear;
    const uint32_t spm = f.softplus ? ~0u : 0u;
    const uint32_t zm = f.z ? ~0u : 0u;
    float A2[NS], invA[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        const float av = n < N ? f.A[(int64_t)dd * N + n] : 0.f;
        A2[n] = av * kLog2e;
        invA[n] = av != 0.f ? 1.f / av : 0.f;
    }
    const float bias = f.bias ? f.bias[dd] : 0.f;
    const int64_t t0 = (int64_t)s * kSeg;
    const int64_t t1 = min(f.L, t0 + kSeg);
    const int64_t row0 = (int64_t)b * f.L;
    constexpr bool STAGE = BF16;
    __shared__ uint16_t s_io[STAGE ? 4 * kSeg * 64 : 1];
    __shared__ uint16_t s_bc[STAGE ? 2 * kSeg * 16 : 1];
    if constexpr (STAGE) stage_segment(a, row0, t0, t1, dd, lane, s_io, s_bc);
    // input k (0 u, 1 delta, 2 z, 3 dy) and B (0) / C (1) of step j
    auto in = [&](int k, int j) -> float {
        const int64_t t = min(t0 + j, t1 - 1);
        if constexpr (STAGE)
            return __uint_as_float((uint32_t)s_io[(k * kSeg + (int)(t - t0)) * 64 + lane] << 16);
        if (k == 2 && !f.z) return 0.f;
        const void* p = k == 0 ? f.u : k == 1 ? f.delta : k == 2 ? f.z : a.dy;
        return ldio<BF16>(p, (row0 + t) * f.Dn + dd);
    };
    auto bc = [&](int k, int j) -> float {
        const int64_t t = min(t0 + j, t1 - 1);
        if constexpr (STAGE)
            return __uint_as_float((uint32_t)s_bc[(k * kSeg + (int)(t - t0)) * 16 + jn] << 16);
        return jn < N ? ldio<BF16>(k == 0 ? f.B : f.C, (row0 + t) * N + jn) : 0.f;
    };

    // The compensated sum of dt over the segment (its decay for the
    // exp-based forms).
    float ssum = 0.f, scomp = 0.f;
    auto kahan = [&](float v) {
        const float yk = v - scomp;
        const float tk = ssum + yk;
        scomp = (tk - ssum) - yk;
        ssum = tk;
    };
    float P[NS];  // running product of A_bar per state (the bilinear decay)
#pragma unroll
    for (int n = 0; n < NS; ++n) P[n] = 1.f;
    const int64_t base_f = (int64_t)b * km1 + s;      // forward slot
    const int64_t base_b = (int64_t)b * km1 + s - 1;  // adjoint slot

    // One walk in time order serves both summaries.  The forward one is the
    // recurrence from a zero state.  The adjoint one, run back from mu = 0 at
    // the segment end, equals sum_j (A_bar_0 ... A_bar_j) C_j g_j, so in time
    // order it needs the running product of A_bar (P, also the bilinear
    // decay) and one fma per state, sharing dt and A_bar with the forward
    // walk.  The walk is unrolled MSSCAN_SEGSUM_UNROLL ways, not fully: the
    // exponentials do not depend on the state, and fully unrolled the
    // compiler would form all of them at once and run out of registers.
    float h[NS], mu[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        h[n] = 0.f;
        mu[n] = 0.f;
    }
    auto walk_step = [&](int j, auto fwd_c, auto bwd_c) {
        constexpr bool FWD = decltype(fwd_c)::value, BWD = decltype(bwd_c)::value;
        const float dt = step_pick(in(1, j), bias, spm);
        kahan(dt);
        float uv = 0.f, bl = 0.f, g = 0.f, cl = 0.f;
        if constexpr (FWD) {
            uv = in(0, j);
            bl = bc(0, j);
        }
        if constexpr (BWD) {
            const float dyv = in(3, j);
            g = pick(zm, dyv * silu_f(in(2, j)), dyv);
            cl = bc(1, j);
        }
        const float xv = dt * uv;
        static_for(
            [&](auto nc) {
                constexpr int n = decltype(nc)::value;
                float abar;
                if constexpr (DISC == kEuler) {
                    abar = hw_exp2(dt * A2[n]);
                    if constexpr (FWD) h[n] = fmaf(abar, h[n], row_bcast<n>(bl) * xv);
                } else {
                    const Disc<DISC> q(dt, dt * A2[n], A2[n], invA[n]);
                    abar = q.abar;
                    if constexpr (FWD) h[n] = fmaf(q.abar, h[n], q.f * row_bcast<n>(bl) * uv);
                }
                if constexpr (BWD || BIL) P[n] *= abar;
                if constexpr (BWD) mu[n] = fmaf(row_bcast<n>(cl) * P[n], g, mu[n]);
            },
            std::make_integer_sequence<int, NS>{});
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    // fp32 io reads each step from memory: unrolled, its loads spill registers
    constexpr int kUnroll = BF16 ? MSSCAN_SEGSUM_UNROLL : 1;
    if (do_fwd && do_bwd) {  // a middle segment (full)
#pragma unroll kUnroll
        for (int j = 0; j < kSeg; ++j) walk_step(j, T_{}, T_{});
    } else if (do_fwd) {  // the first segment (full)
#pragma unroll kUnroll
        for (int j = 0; j < kSeg; ++j) walk_step(j, T_{}, F_{});
    } else {  // the last segment, possibly partial
        for (int j = 0; j < (int)(t1 - t0); ++j) walk_step(j, F_{}, T_{});
    }
    if (dvalid) {
        if (do_fwd) {
#pragma unroll
            for (int n = 0; n < NS; ++n)
                if (n < N) f.agg[(base_f * N + n) * f.Dn + d] = h[n];
            if constexpr (BIL) {
#pragma unroll
                for (int n = 0; n < NS; ++n)
                    if (n < N) f.prod[(base_f * N + n) * f.Dn + d] = P[n];
            } else {
                f.sdt[base_f * f.Dn + d] = ssum;
            }
        }
        if (do_bwd) {
#pragma unroll
            for (int n = 0; n < NS; ++n)
                if (n < N) a.mu[(base_b * N + n) * f.Dn + d] = mu[n];
            if constexpr (BIL) {
#pragma unroll
                for (int n = 0; n < NS; ++n)
                    if (n < N) a.prod_b[(base_b * N + n) * f.Dn + d] = P[n];
            } else {
                a.sdt_b[base_b * f.Dn + d] = ssum;
            }
        }
    }
}

// ---- 3. reverse carry ---------------------------------------------------------
// Slot s-1 of mu holds beta_s (from segment s, s = 1..K-1); carry_chain<true>
// replaces it by the mu entering segment s-1 from the right:
//   mu_in(K-1) = dh_last (or 0),  mu_in(s-1) = decay_s mu_in(s) + beta_s.

// ---- 4. per-segment gradients ---------------------------------------------------
// The segment's kSeg = 16 steps are walked back in sub-blocks of kSub steps
// (sub_len: 4, or 2 for fp32-io ZOH / bilinear).  Forward states come from two kept
// states, the segment start and the state after 8 steps (32 recomputed steps
// per segment with 4-step sub-blocks, 48 with 2-step ones), and each
// sub-block's inputs are read in one batch before its arithmetic.
template <int NS, bool BF16, int DISC>
__global__ void __launch_bounds__(64 * kBwdWaves, 2) bwd_main(BwdArgs a) {
    constexpr int kSub = sub_len<DISC, BF16>();
    static_assert(kSeg == 16 && (kSub == 4 || kSub == 2), "sub-blocks split the segment");
    const ScanArgs& f = a.f;
    // Per-step dB | dC contributions, [value][lane]; rows padded to 65 floats
    // so that the column sums below read distinct banks.
    __shared__ float red_w[kBwdWaves][2 * NS][65];
    // Wave w of the workgroup takes segment kBwdWaves * blockIdx.y + w of one
    // tile; a spare wave of the last group repeats the last segment and
    // stores nothing (so every wave runs the same code up to the final
    // workgroup barrier).
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // uniform
    float(*red)[65] = red_w[wave];
    const int lane = (int)(threadIdx.x & 63);
    const int b = blockIdx.z;
    const int s_raw = blockIdx.y * kBwdWaves + wave;
    const bool seg_ok = s_raw < f.chunks;
    const int s = seg_ok ? s_raw : f.chunks - 1;
    const int tile = blockIdx.x;
    const int d = tile * 64 + lane;
    const bool dvalid = d < f.Dn;
    const bool wvalid = dvalid && seg_ok;  // this lane stores results
    const int dd = dvalid ? d : f.Dn - 1;
    const int N = f.N;
    const int km1 = f.chunks - 1;
    const int jn = lane & (NS - 1);
    const float live = dvalid ? 1.f : 0.f;  // tail lanes repeat a channel: count it once
    const uint32_t spm = f.softplus ? ~0u : 0u;
    const uint32_t zm = f.z ? ~0u : 0u;
    // The mask form pays off with Euler and bf16 io.  ZOH and bilinear keep
    // branches: their steps hold more values, and straight-line steps spilled
    // registers there (measured 10% slower); so did the fp32-io Euler kernel.
    constexpr bool kMasks = DISC == kEuler && BF16;
    auto dt_of = [&](float v) {
        if constexpr (kMasks) return pick(spm, softplus_f(v), v);
        return f.softplus ? softplus_f(v) : v;
    };

    float A2[NS], invA[NS], mu[NS], h0s[NS], dA[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        const float av = n < N ? f.A[(int64_t)dd * N + n] : 0.f;
        A2[n] = av * kLog2e;
        invA[n] = av != 0.f ? 1.f / av : 0.f;
        dA[n] = 0.f;
        float h = 0.f, m = 0.f;
        if (n < N) {
            if (s == 0) {
                if (f.h0) h = f.h0[((int64_t)b * f.Dn + dd) * N + n];
            } else {
                h = f.agg[(((int64_t)b * km1 + (s - 1)) * N + n) * f.Dn + dd];
            }
            if (s == f.chunks - 1) {
                if (a.dh_last) m = a.dh_last[((int64_t)b * f.Dn + dd) * N + n];
            } else {
                m = a.mu[(((int64_t)b * km1 + s) * N + n) * f.Dn + dd];
            }
        }
        h0s[n] = h;
        mu[n] = m;
    }
    const float bias = f.bias ? f.bias[dd] : 0.f;
    const float Dd = f.D ? f.D[dd] : 0.f;
    const int64_t t0 = (int64_t)s * kSeg;
    const int64_t t1 = min(f.L, t0 + kSeg);
    const int64_t row0 = (int64_t)b * f.L;

    // bf16 io: the segment's inputs are staged in LDS by one batch of loads
    // at the start (raw 16-bit values: u, delta, z, dy per lane; B, C per
    // state), so the walk below never waits on HBM.  fp32 io reads them
    // from memory per sub-block.
    constexpr bool STAGE = BF16;
    __shared__ uint16_t s_io_w[kBwdWaves][STAGE ? 4 * kSeg * 64 : 1];  // [u|delta|z|dy][step][lane]
    __shared__ uint16_t s_bc_w[kBwdWaves][STAGE ? 2 * kSeg * 16 : 1];  // [B|C][step][state]
    uint16_t* s_io = s_io_w[wave];
    uint16_t* s_bc = s_bc_w[wave];
    if constexpr (STAGE) stage_segment(a, row0, t0, t1, dd, lane, s_io, s_bc);
    // bf16 io: du, ddelta and dz go out through buffer resources over the
    // segment's rows, so rows past t1 and tail lanes (offset out of range)
    // are dropped by the hardware, with no branch and 32-bit offsets.
    const uint32_t orowb = (uint32_t)f.Dn * 2u;
    auto out_rows = [&](void* p) {
        return make_rsrc(static_cast<char*>(p) + (row0 + t0) * (int64_t)orowb,
                         p ? (uint32_t)(t1 - t0) * orowb : 0u);
    };
    const auto rDu = out_rows(a.du), rDdl = out_rows(a.ddelta), rDz = out_rows(a.dz);
    const uint32_t ooff = wvalid ? (uint32_t)dd * 2u : kOutOfRange;
    auto wid = [](uint16_t v) { return __uint_as_float((uint32_t)v << 16); };

    // Inputs of the 4 steps from tb (indices clamped into the segment).
    struct Rows {
        float u[kSub], dl[kSub], z[kSub], dy[kSub], bl[kSub], cl[kSub];
    };
    auto load_rows = [&](Rows& r, int64_t tb, bool full) {
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
            const int64_t t = min(tb + j, t1 - 1);
            if constexpr (STAGE) {
                const int jj = (int)(t - t0);
                r.u[j] = wid(s_io[(0 * kSeg + jj) * 64 + lane]);
                r.dl[j] = wid(s_io[(1 * kSeg + jj) * 64 + lane]);
                r.bl[j] = wid(s_bc[(0 * kSeg + jj) * 16 + jn]);
                if (full) {
                    r.z[j] = wid(s_io[(2 * kSeg + jj) * 64 + lane]);
                    r.dy[j] = wid(s_io[(3 * kSeg + jj) * 64 + lane]);
                    r.cl[j] = wid(s_bc[(1 * kSeg + jj) * 16 + jn]);
                }
            } else {
                const int64_t e = (row0 + t) * f.Dn + dd;
                r.u[j] = ldio<BF16>(f.u, e);
                r.dl[j] = ldio<BF16>(f.delta, e);
                r.bl[j] = jn < N ? ldio<BF16>(f.B, (row0 + t) * N + jn) : 0.f;
                if (full) {
                    r.z[j] = f.z ? ldio<BF16>(f.z, e) : 0.f;
                    r.dy[j] = ldio<BF16>(a.dy, e);
                    r.cl[j] = jn < N ? ldio<BF16>(f.C, (row0 + t) * N + jn) : 0.f;
                }
            }
        }
    };
    // One forward step of all states (in place).
    auto fwd = [&](float (&h)[NS], float dl, float uv, float bl) {
        const float dt = dt_of(dl + bias);
        if constexpr (DISC == kEuler) {
            const float xv = dt * uv;  // B_bar u = B * (dt u)
            static_for(
                [&](auto nc) {
                    constexpr int n = decltype(nc)::value;
                    h[n] = fmaf(hw_exp2(dt * A2[n]), h[n], row_bcast<n>(bl) * xv);
                },
                std::make_integer_sequence<int, NS>{});
        } else {
            static_for(
                [&](auto nc) {
                    constexpr int n = decltype(nc)::value;
                    const Disc<DISC> q(dt, dt * A2[n], A2[n], invA[n]);
                    h[n] = fmaf(q.abar, h[n], q.f * row_bcast<n>(bl) * uv);
                },
                std::make_integer_sequence<int, NS>{});
        }
    };
    // Advance h over the 4 steps from tb.
    auto advance_sub = [&](float (&h)[NS], int64_t tb) {
        Rows r;
        load_rows(r, tb, false);
#pragma unroll
        for (int j = 0; j < kSub; ++j)
            if (tb + j < t1) fwd(h, r.dl[j], r.u[j], r.bl[j]);
    };

    float dbias = 0.f, dD = 0.f;
    // The tile's dB | dC partials of this segment's steps, [t - t0][2N] fp32,
    // through a buffer resource (rows past t1 dropped).
    const auto rPbc = make_rsrc(a.pbc + (((int64_t)tile * f.batch + b) * f.L + t0) * (2 * N),
                                (uint32_t)(t1 - t0) * (uint32_t)(2 * N) * 4u);

    // Gradients of the sub-block of 4 steps from tb, whose starting state is hb.
    auto sub_block = [&](int64_t tb, const float (&hb)[NS]) {
        if (tb >= t1) return;
        Rows r;
        load_rows(r, tb, true);
        // y_pre accumulated so far for these steps: loaded before the
        // recompute, so that the loads are in flight while it runs
        // (and, with out_add, the du and ddelta totals the results add to)
        float yprev[kSub], duprev[kSub], dvprev[kSub];
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
            yprev[j] = duprev[j] = dvprev[j] = 0.f;
            const int64_t ej = (row0 + tb + j) * f.Dn + dd;
            if (a.ypart && a.ypart_add && wvalid && tb + j < t1) yprev[j] = a.ypart[ej];
            if constexpr (!BF16) {
                if (a.out_add && wvalid && tb + j < t1) {
                    duprev[j] = static_cast<const float*>(a.du)[ej];
                    dvprev[j] = static_cast<const float*>(a.ddelta)[ej];
                }
            }
        }
        float hs[kSub][NS];  // hs[j] = state after step tb + j
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
#pragma unroll
            for (int n = 0; n < NS; ++n) hs[j][n] = j == 0 ? hb[n] : hs[j - 1][n];
            if (tb + j < t1) fwd(hs[j], r.dl[j], r.u[j], r.bl[j]);
        }
#pragma unroll
        for (int j = kSub - 1; j >= 0; --j) {
            const int64_t t = tb + j;
            if (t >= t1) continue;
            const int64_t e = (row0 + t) * f.Dn + dd;
            const float v = r.dl[j] + bias;
            const float dt = dt_of(v);
            const float uv = r.u[j];
            const float bl = r.bl[j];
            const float cl = r.cl[j];
            const float dyv = r.dy[j];
            // y_pre from the recomputed state, for the gate's derivative
            const float ypre = dpp_dot<NS>(Dd * uv, cl, hs[j]);
            if (a.ypart && wvalid) a.ypart[e] = yprev[j] + ypre;
            float g = dyv;
            if constexpr (kMasks) {
                const float zv = r.z[j];  // 0 when there is no gate
                const float sg = hw_rcp(1.f + hw_exp2(-zv * kLog2e));
                g = pick(zm, dyv * zv * sg, dyv);
                const float dzv = dyv * ypre * sg * fmaf(zv, 1.f - sg, 1.f);
                Io<true>::store(rDz, ooff + (uint32_t)(t - t0) * orowb, dzv);  // no z: size 0
            } else if (f.z) {
                const float zv = r.z[j];
                const float sg = hw_rcp(1.f + hw_exp2(-zv * kLog2e));
                g = dyv * zv * sg;
                const float dzv = dyv * ypre * sg * fmaf(zv, 1.f - sg, 1.f);
                if constexpr (BF16)
                    Io<true>::store(rDz, ooff + (uint32_t)(t - t0) * orowb, dzv);
                else if (wvalid)
                    st<BF16>(a.dz, e, dzv);
            }
            float du = g * Dd;
            dD = fmaf(g, uv, dD);
            float ddt = 0.f;
            dpp_axpy<NS>(mu, cl, g);  // mu[n] becomes l_n = C_n g + mu_n
            if constexpr (DISC == kEuler) {
                // f = dt for every state, so with s = sum_n l_n B_n:
                //   du   = g D + dt s,   d(dt) = sum_n l_n h_{n,t-1} A_bar_n a_n + u s,
                //   dA_n += l_n h_{n,t-1} A_bar_n dt,   dB_n = l_n dt u,  dC_n = g h_n.
                const float lg = live * g;
                const float fuv = live * dt * uv;
                const float sb = dpp_dot<NS>(0.f, bl, mu);
                float dta = 0.f;  // dta: sum_n (l h A_bar) A2_n
                static_for(
                    [&](auto nc) {
                        constexpr int n = decltype(nc)::value;
                        const float hp = j == 0 ? hb[n] : hs[j - 1][n];
                        const float abar = hw_exp2(dt * A2[n]);
                        const float l = mu[n];
                        red[NS + n][lane] = lg * hs[j][n];  // dC contribution
                        red[n][lane] = l * fuv;             // dB contribution
                        const float q = abar * l;           // the mu passed to step t-1
                        const float w = q * hp;
                        dta = fmaf(w, A2[n], dta);
                        dA[n] = fmaf(w, dt, dA[n]);
                        mu[n] = q;
                    },
                    std::make_integer_sequence<int, NS>{});
                du = fmaf(dt, sb, du);
                ddt = fmaf(dta, kLn2, uv * sb);
            } else if constexpr (DISC == kZoh) {
                // f_n = (A_bar_n - 1)/a_n (series near a = 0); with lb = l_n B_n:
                //   du    = g D + sum f lb,
                //   d(dt) = sum_n l h_{t-1} A_bar a + u sum_n A_bar lb,
                //   dA_n += l h_{t-1} A_bar dt + lb u df/da,
                //   df/da = (dt A_bar - f)/a, or near a = 0 dt^2 (1/2 + x/3 + x^2/8), x = t ln2.
                const float lg = live * g, luv = live * uv;
                const float dt2 = dt * dt;
                const float c0 = 0.5f * dt2, c1 = dt2 * (kLn2 / 3.f), c2 = dt2 * (kLn2 * kLn2 / 8.f);
                float sf = 0.f, dta = 0.f, dtb = 0.f;
                static_for(
                    [&](auto nc) {
                        constexpr int n = decltype(nc)::value;
                        const float hp = j == 0 ? hb[n] : hs[j - 1][n];
                        const float t2 = dt * A2[n];
                        const float abar = hw_exp2(t2);
                        const bool small = fabsf(t2) < kZohSwitch;
                        const float fz = small ? dt * fmaf(t2, fmaf(t2, kZohT2, kZohT1), 1.f)
                                               : fmaf(abar, invA[n], -invA[n]);
                        const float l = mu[n];
                        red[NS + n][lane] = lg * hs[j][n];  // dC contribution
                        red[n][lane] = (l * fz) * luv;      // dB contribution
                        const float lb = l * row_bcast<n>(bl);
                        sf = fmaf(fz, lb, sf);
                        const float q = abar * l;  // the mu passed to step t-1
                        const float w = q * hp;
                        dta = fmaf(w, A2[n], dta);
                        dtb = fmaf(abar, lb, dtb);
                        const float dfda = small ? fmaf(t2, fmaf(t2, c2, c1), c0)
                                                 : fmaf(dt, abar, -fz) * invA[n];
                        dA[n] = fmaf(lb * uv, dfda, fmaf(w, dt, dA[n]));
                        mu[n] = q;
                    },
                    std::make_integer_sequence<int, NS>{});
                du += sf;
                ddt = fmaf(dta, kLn2, uv * dtb);
            } else {
                static_assert(DISC == kBilinear, "three discretisations");
                // r = 1/(1 - dt a/2): A_bar = 2r - 1, f = dt r, and every
                // derivative carries r^2:  dA_bar/dt = a r^2, dA_bar/da = dt r^2,
                // df/dt = r^2, df/da = dt^2 r^2 / 2.  With lb = l_n B_n:
                //   d(dt) = sum r^2 (l h_{t-1} a + lb u),
                //   dA_n += r^2 (l h_{t-1} dt + lb u dt^2/2),  du = g D + sum f lb.
                const float lg = live * g, luv = live * uv;
                const float hdt2 = 0.5f * dt * dt;
                float sf = 0.f;
                static_for(
                    [&](auto nc) {
                        constexpr int n = decltype(nc)::value;
                        const float hp = j == 0 ? hb[n] : hs[j - 1][n];
                        const float r = bilinear_r(dt * A2[n]);
                        const float r2 = r * r;
                        const float abar = fmaf(2.f, r, -1.f);
                        const float fb = dt * r;
                        const float l = mu[n];
                        red[NS + n][lane] = lg * hs[j][n];  // dC contribution
                        red[n][lane] = (l * fb) * luv;      // dB contribution
                        const float lb = l * row_bcast<n>(bl);
                        sf = fmaf(fb, lb, sf);
                        const float dab = l * hp, dfac = lb * uv;
                        ddt = fmaf(r2, fmaf(dab, A2[n] * kLn2, dfac), ddt);
                        dA[n] = fmaf(r2, fmaf(dab, dt, dfac * hdt2), dA[n]);
                        mu[n] = abar * l;
                    },
                    std::make_integer_sequence<int, NS>{});
                du += sf;
            }
            float dv = ddt;
            if constexpr (kMasks)
                dv = pick(spm, ddt * hw_rcp(1.f + hw_exp2(-v * kLog2e)), ddt);
            else if (f.softplus)
                dv = ddt * hw_rcp(1.f + hw_exp2(-v * kLog2e));
            dbias += dv;
            if constexpr (BF16) {
                Io<true>::store(rDu, ooff + (uint32_t)(t - t0) * orowb, du);
                Io<true>::store(rDdl, ooff + (uint32_t)(t - t0) * orowb, dv);
            } else if (wvalid) {
                st<BF16>(a.du, e, du + duprev[j]);
                st<BF16>(a.ddelta, e, dv + dvprev[j]);
            }
            // Sum the 2N contributions of this step over the wave's channels:
            // lane l adds half (l & 1) of row l >> 1, the pair is combined
            // with a DPP add, and the even lane stores the tile's partial.
            wave_sync();
            {
                const int row = lane >> 1;
                const int half = lane & 1;
                // four partial sums (i mod 4) keep the add chain short
                float acc = 0.f;
                if (row < 2 * NS) {
                    float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 32; ++i) p4[i & 3] += red[row][32 * half + i];
                    acc = (p4[0] + p4[1]) + (p4[2] + p4[3]);
                }
                acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xf,
                                                               0xf, true));  // quad_perm 1,0,3,2
                const int n = row < NS ? row : row - NS;
                const bool keep = seg_ok && half == 0 && row < 2 * NS && n < N;
                const uint32_t po = (uint32_t)(t - t0) * (uint32_t)(2 * N) + (row < NS ? 0 : N) + n;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc), rPbc,
                                                      keep ? po * 4u : kOutOfRange, 0, 0);
            }
            wave_sync();
        }
    };

    float hm[NS];  // state after half the segment (8 steps)
#pragma unroll
    for (int n = 0; n < NS; ++n) hm[n] = h0s[n];
#pragma unroll
    for (int m = 0; m < kSeg / 2; m += kSub) advance_sub(hm, t0 + m);
    // Sub-blocks from the last to the first: each starts from the kept state
    // below it (the half-way state for the upper half, the segment start for
    // the lower) advanced to its first step.  One loop body keeps one
    // sub-block's registers live at a time.
    constexpr int kBlocks = kSeg / kSub;
#pragma unroll 1
    for (int k = kBlocks - 1; k >= 0; --k) {
        const bool upper = k >= kBlocks / 2;
        float hb[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) hb[n] = upper ? hm[n] : h0s[n];
#pragma unroll 1
        for (int m = upper ? kBlocks / 2 : 0; m < k; ++m) advance_sub(hb, t0 + kSub * m);
        sub_block(t0 + kSub * k, hb);
    }

    if (s == 0 && a.dh0 && wvalid) {
#pragma unroll
        for (int n = 0; n < NS; ++n)
            if (n < N) a.dh0[((int64_t)b * f.Dn + d) * N + n] = mu[n];
    }

    // The waves' partials of dA, dD and dbias are added in wave order through
    // LDS (each wave's own rows are free now), and wave 0 stores the group's.
    static_assert(NS >= 2, "N + 2 partial rows fit the 2 * NS rows of a wave");
    wave_sync();
#pragma unroll
    for (int n = 0; n < NS; ++n) red[n][lane] = seg_ok ? dA[n] : 0.f;
    red[NS][lane] = seg_ok ? dD : 0.f;
    red[NS + 1][lane] = seg_ok ? dbias : 0.f;
    __syncthreads();
    if (wave == 0 && dvalid) {
        const int groups = (f.chunks + kBwdWaves - 1) / kBwdWaves;
        float* pp = a.pparam + (((int64_t)b * groups + blockIdx.y) * f.Dn + d) * (N + 2);
        auto sum_w = [&](int row) {
            float acc = red_w[0][row][lane];
#pragma unroll
            for (int w = 1; w < kBwdWaves; ++w) acc += red_w[w][row][lane];
            return acc;
        };
#pragma unroll
        for (int n = 0; n < NS; ++n)
            if (n < N) pp[n] = sum_w(n);
        pp[N] = sum_w(NS);
        pp[N + 1] = sum_w(NS + 1);
    }
}

// ---- 5. fixed-order sums of the partials -----------------------------------------
__global__ void __launch_bounds__(256) reduce_bc(BwdArgs a, float* dB, float* dC, int tiles) {
    const ScanArgs& f = a.f;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (b, t, k), k < 2N
    const int64_t per = (int64_t)f.batch * f.L * 2 * f.N;
    if (idx >= per) return;
    // Tiles are added in order; each group of 8 loads is issued before its adds.
    float acc = 0.f;
    int tl = 0;
    for (; tl + 8 <= tiles; tl += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = a.pbc[(int64_t)(tl + i) * per + idx];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += v[i];
    }
    for (; tl < tiles; ++tl) acc += a.pbc[(int64_t)tl * per + idx];
    const int k = (int)(idx % (2 * f.N));
    const int64_t row = idx / (2 * f.N);
    if (k < f.N)
        dB[row * f.N + k] = acc;
    else
        dC[row * f.N + k - f.N] = acc;
}

// reduce_bc with four consecutive outputs per thread and 16-byte loads (when
// batch * L * 2N is a multiple of 4); each output's tiles are added in the
// same order, so the sums are the same.
constexpr int kBcBatch = 8;  // loads in flight per thread
// Thread `t` of the float4 range: the four outputs idx .. idx + 3 of dB | dC.
__device__ __forceinline__ void bc4_sum(const BwdArgs& a, float* dB, float* dC, int tiles,
                                        int64_t t) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const ScanArgs& f = a.f;
    const int64_t per = (int64_t)f.batch * f.L * 2 * f.N;
    const int64_t idx = t * 4;
    if (idx >= per) return;
    f4v acc = {0.f, 0.f, 0.f, 0.f};
    int tl = 0;
    for (; tl + kBcBatch <= tiles; tl += kBcBatch) {
        f4v v[kBcBatch];
#pragma unroll
        for (int i = 0; i < kBcBatch; ++i)
            v[i] = *reinterpret_cast<const f4v*>(a.pbc + (int64_t)(tl + i) * per + idx);
#pragma unroll
        for (int i = 0; i < kBcBatch; ++i) acc += v[i];
    }
    for (; tl < tiles; ++tl) acc += *reinterpret_cast<const f4v*>(a.pbc + (int64_t)tl * per + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t o = idx + i;
        const int k = (int)(o % (2 * f.N));
        const int64_t row = o / (2 * f.N);
        if (k < f.N)
            dB[row * f.N + k] = acc[i];
        else
            dC[row * f.N + k - f.N] = acc[i];
    }
}

__global__ void __launch_bounds__(256) reduce_bc4(BwdArgs a, float* dB, float* dC, int tiles) {
    bc4_sum(a, dB, dC, tiles, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// The dA | dD | dbias output of entry idx = (d, k), k < N + 2.
__device__ __forceinline__ void put_param(const ScanArgs& f, int64_t idx, float v, float* dA,
                                          float* dD, float* dbias) {
    const int k = (int)(idx % (f.N + 2));
    const int64_t d = idx / (f.N + 2);
    if (k < f.N)
        dA[d * f.N + k] = v;
    else if (k == f.N) {
        if (dD) dD[d] = v;
    } else if (dbias) {
        dbias[d] = v;
    }
}

// reduce_bc4 and the parameter sums in one launch, for pparam of at most
// kParamGroups rows (the row layout: one per batch row): blocks past
// bc_blocks add each entry's rows in increasing order, which gives the bits
// of the two-level sum below (each group holds one row; adding the empty
// groups' zeros changes nothing but the sign of a zero).
__global__ void __launch_bounds__(256) reduce_bc4_params(BwdArgs a, float* dB, float* dC,
                                                         int tiles, unsigned bc_blocks, float* dA,
                                                         float* dD, float* dbias) {
    if (blockIdx.x < bc_blocks) {
        bc4_sum(a, dB, dC, tiles, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
        return;
    }
    const ScanArgs& f = a.f;
    const int64_t idx = (int64_t)(blockIdx.x - bc_blocks) * blockDim.x + threadIdx.x;
    const int64_t per = (int64_t)f.Dn * (f.N + 2);
    if (idx >= per) return;
    const int64_t rows = (int64_t)f.batch * ((f.chunks + kBwdWaves - 1) / kBwdWaves);
    float acc = 0.f;
    for (int64_t r = 0; r < rows; ++r) acc += a.pparam[r * per + idx];
    put_param(f, idx, acc, dA, dD, dbias);
}

// Parameter sums over the batch x ceil(K/kBwdWaves) rows of pparam, in two fixed-order
// levels: group g (blockIdx.y) adds the rows r with r mod kParamGroups == g
// in increasing order, then reduce_param_groups adds the groups in order.
__global__ void __launch_bounds__(256) reduce_params(BwdArgs a) {
    const ScanArgs& f = a.f;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (d, k), k < N+2
    const int64_t per = (int64_t)f.Dn * (f.N + 2);
    if (idx >= per) return;
    const int g = blockIdx.y;
    const int64_t rows = (int64_t)f.batch * ((f.chunks + kBwdWaves - 1) / kBwdWaves);
    // The group's rows are added in increasing order; each batch of 8 loads is
    // issued before its adds.
    float acc = 0.f;
    int64_t r = g;
    for (; r + 7 * kParamGroups < rows; r += 8 * kParamGroups) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = a.pparam[(r + i * kParamGroups) * per + idx];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc += v[i];
    }
    for (; r < rows; r += kParamGroups) acc += a.pparam[r * per + idx];
    a.pgroup[(int64_t)g * per + idx] = acc;
}

__global__ void __launch_bounds__(256) reduce_param_groups(BwdArgs a, float* dA, float* dD,
                                                           float* dbias) {
    const ScanArgs& f = a.f;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per = (int64_t)f.Dn * (f.N + 2);
    if (idx >= per) return;
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < kParamGroups; ++g) acc += a.pgroup[(int64_t)g * per + idx];
    put_param(f, idx, acc, dA, dD, dbias);
}

template <int NS, bool BF16, int DISC>
hipError_t launch_bwd(const BwdArgs& a, float* dA, float* dB, float* dC, float* dD,
                      float* dbias, hipStream_t s) {
    const ScanArgs& f = a.f;
    const int tiles = (f.Dn + 63) / 64;
    const int K = f.chunks;
    hipError_t e;
    if (K > 1) {
        {
            ProfScope ps(s, kPhaseSummary);
            hipLaunchKernelGGL((seg_summaries<NS, BF16, DISC>), dim3(tiles, K, f.batch),
                               dim3(64), 0, s, a);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_carry(f, s)) != hipSuccess) return e;  // forward segment starts
        CarryArgs c{};
        c.val = a.mu;
        c.sdt = a.sdt_b;
        c.prod = a.prod_b;
        c.A = f.A;
        c.init = a.dh_last;
        c.batch = f.batch;
        c.km1 = K - 1;
        c.N = f.N;
        c.Dn = f.Dn;
        if ((e = launch_carry(c, true, s)) != hipSuccess) return e;  // adjoint mu entering
    }
    {
        ProfScope ps(s, kPhaseMain);
        hipLaunchKernelGGL((bwd_main<NS, BF16, DISC>),
                           dim3(tiles, (K + kBwdWaves - 1) / kBwdWaves, f.batch), dim3(64 * kBwdWaves),
                           0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_bwd_reductions(f, a.pbc, tiles, a.pparam, a.pgroup, dA, dB, dC, dD, dbias, s);
}

template <bool BF16, int DISC>
hipError_t launch_ns(const BwdArgs& a, float* dA, float* dB, float* dC, float* dD, float* dbias,
                     hipStream_t s) {
    const int N = a.f.N;
    if (N <= 4) return launch_bwd<4, BF16, DISC>(a, dA, dB, dC, dD, dbias, s);
    if (N <= 8) return launch_bwd<8, BF16, DISC>(a, dA, dB, dC, dD, dbias, s);
    if (N <= 16) return launch_bwd<16, BF16, DISC>(a, dA, dB, dC, dD, dbias, s);
    return hipErrorInvalidValue;
}

}  // namespace

int bwd_segment_len() { return kSeg; }

hipError_t launch_bwd_reductions(const ScanArgs& f, float* pbc, int tiles, float* pparam,
                                 float* pgroup, float* dA, float* dB, float* dC, float* dD,
                                 float* dbias, hipStream_t s) {
    BwdArgs a{};
    a.f = f;
    a.pbc = pbc;
    a.pparam = pparam;
    a.pgroup = pgroup;
    hipError_t e;
    const int64_t nbc = (int64_t)f.batch * f.L * 2 * f.N;
    const int64_t npar = (int64_t)f.Dn * (f.N + 2);
    const unsigned pblocks = (unsigned)((npar + 255) / 256);
    const int64_t prows = (int64_t)f.batch * ((f.chunks + kBwdWaves - 1) / kBwdWaves);
    if (nbc % 4 == 0 && prows <= kParamGroups) {
        const unsigned bc_blocks = (unsigned)((nbc / 4 + 255) / 256);
        ProfScope ps(s, kPhaseReduce);
        hipLaunchKernelGGL(reduce_bc4_params, dim3(bc_blocks + pblocks), dim3(256), 0, s, a, dB,
                           dC, tiles, bc_blocks, dA, dD, dbias);
        return hipGetLastError();
    }
    {
        ProfScope ps(s, kPhaseReduce);
        if (nbc % 4 == 0)
            hipLaunchKernelGGL(reduce_bc4, dim3((unsigned)((nbc / 4 + 255) / 256)), dim3(256), 0,
                               s, a, dB, dC, tiles);
        else
            hipLaunchKernelGGL(reduce_bc, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0, s, a,
                               dB, dC, tiles);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        ProfScope ps(s, kPhaseReduce);
        hipLaunchKernelGGL(reduce_params, dim3(pblocks, kParamGroups), dim3(256), 0, s, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        ProfScope ps(s, kPhaseReduce);
        hipLaunchKernelGGL(reduce_param_groups, dim3(pblocks), dim3(256), 0, s, a, dA, dD, dbias);
    }
    return hipGetLastError();
}

hipError_t launch_scan_bwd(const BwdLaunch& L, hipStream_t s) {
    BwdArgs a{};
    a.f = L.f;
    a.dy = L.dy;
    a.dh_last = L.dh_last;
    a.du = L.du;
    a.ddelta = L.ddelta;
    a.dz = L.dz;
    a.dh0 = L.dh0;
    a.mu = L.mu;
    a.sdt_b = L.sdt_b;
    a.prod_b = L.prod_b;
    a.pbc = L.pbc;
    a.pparam = L.pparam;
    a.pgroup = L.pgroup;
    a.ypart = L.ypart;
    a.ypart_add = L.ypart_add;
    a.out_add = L.out_add;
    switch (L.disc) {
#define MS_BWD_(DI)                                                                     \
    case DI:                                                                            \
        return L.bf16 ? launch_ns<true, DI>(a, L.dA, L.dB, L.dC, L.dD, L.dbias, s)      \
                      : launch_ns<false, DI>(a, L.dA, L.dB, L.dC, L.dD, L.dbias, s);
        MS_BWD_(kEuler)
        MS_BWD_(kZoh)
        MS_BWD_(kBilinear)
#undef MS_BWD_
        default: return hipErrorInvalidValue;
    }
}

}  // namespace msscan
