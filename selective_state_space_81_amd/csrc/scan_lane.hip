// scan_lane.hip -- selective scan (S6) kernel with every state of a channel
// in one lane, for d_state 8, 16 and 32 (64 with the Euler form) on gfx950;
// with PAD, any smaller d_state on the next of these sizes (the extra states
// get A = B = C = 0, stay zero and are never stored).
//
// A workgroup is a single wave: lane = one channel of a 64-channel tile, and
// the lane keeps all N states of its channel in VGPRs.  The wave walks one
// segment of the sequence timestep by timestep, doing the whole per-element
// pipeline in registers:
//   dt = softplus(delta + bias), x = dt*u                 (once per element)
//   for n: A_bar = exp(dt*A), h = A_bar*h + B_bar*u         (N recurrences)
//   y = sum_n C*h + D*u, times silu(z), rounded, stored    (once per element)
// There is no LDS, no barrier and no cross-wave exchange, so many waves fit
// a CU and the VALU stays busy; the sequence is cut into segments to supply
// those waves (the batch x tile count alone is too small for the chip).  A
// segment after the first starts from a carried state: a summary variant of
// this kernel (SUMMARY = true, no readout) computes each segment's end state
// from zero and its compensated sum of dt, and the carry pass composes them
// in order -- the scan is a composition of affine maps (jsqmd page,
// section 3.4).
//
// B_t and C_t (shared by all channels, lmnt page section 3.2) are read from
// the caller's [batch][L][d_state] tensors: lane l loads state (l mod N) and
// the DPP row_newbcast control hands state n to every lane as the first
// operand of v_mul / v_fmac, so the broadcast costs no extra instruction, no
// LDS traffic and no SGPRs (bf16 values are widened by one shift first).
//
// With DTP the raw step size is not read from HBM but projected from a
// low-rank input (the step is softplus of a linear map of the input plus a
// bias, jsqmd page section 2.2; the map is low-rank, a narrow slice of x_proj
// lifted to d_inner by dt_proj, lmnt page section 3.2):
//   delta[t][d] = sum_r W[d][r] * x[t][r],   r < rank <= 64.
// Every 16 timesteps the wave forms the 16 x 64 tile of delta on the matrix
// cores (one 16x16 output per 16 channels, K = rank in slices of 32) and turns
// it through LDS so that each lane holds its own channel's 16 values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "dpp_common.h"
#include "dtproj_frag.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

#ifndef MSSCAN_LANE_TB
#define MSSCAN_LANE_TB 4
#endif
#ifndef MSSCAN_LANE_DB
#define MSSCAN_LANE_DB 1
#endif
#ifndef MSSCAN_LANE_TB64
#define MSSCAN_LANE_TB64 4
#endif
#ifndef MSSCAN_LANE_DB64
#define MSSCAN_LANE_DB64 0
#endif
#ifndef MSSCAN_LANE_WPE
#define MSSCAN_LANE_WPE 1
#endif

constexpr int kPT = 16;   // timesteps per projected delta tile
constexpr int kPTS = 20;  // LDS row stride of the turned tile (floats; 16-byte rows)

typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));


template <int N, int TB, bool DB, bool BF16, int DISC, bool SP, bool SUMMARY, bool DTP = false,
          bool PAD = false>
__global__ void __launch_bounds__(64, N >= 32 ? 2 : MSSCAN_LANE_WPE) scan_lane(ScanArgs a) {
    static_assert(N == 8 || N == 16 || N == 32 || N == 64, "states per lane");
    constexpr bool ZOH = DISC == kZoh;
    constexpr bool BIL = DISC == kBilinear;
    // A bilinear summary keeps the product of A_bar per state (its segment
    // decay is not exp(A * sum dt)).
    constexpr bool PROD = SUMMARY && BIL;
    // B_t and C_t reach the lanes in groups of RW states, one DPP row each:
    // lane l holds state 16k + (l mod RW) of group k.
    constexpr int RW = N < 16 ? N : 16;
    constexpr int KB = N / RW;
    using R = Io<BF16>;
    using RT = typename R::T;

    const int lane = threadIdx.x;
    const int b = blockIdx.z;
    const int seg = blockIdx.y;
    const int d = blockIdx.x * 64 + lane;
    const bool dvalid = d < a.Dn;
    const int dd = dvalid ? d : a.Dn - 1;

    // PAD: the true d_state Nr = a.N is below N.  States Nr..N-1 get A = 0
    // and B = C = 0, so they stay zero and add nothing; they are never
    // stored, and every stride uses Nr.
    const int Nr = PAD ? a.N : N;
    float A2[N], invA[N], A2sq[N], h[N], P[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const float av = (!PAD || n < Nr) ? a.A[(int64_t)dd * Nr + n] : 0.f;
        A2[n] = av * kLog2e;
        if constexpr (ZOH) {
            invA[n] = (av != 0.f) ? 1.f / av : 0.f;
            A2sq[n] = A2[n] * A2[n];
        }
    }
    const int km1 = a.chunks - 1;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        float v = 0.f;
        if constexpr (!SUMMARY) {
            if (!PAD || n < Nr) {
                if (seg == 0) {
                    // several segments: the carry pass's copy of h0 (h_last may alias h0)
                    const float* h0 = a.chunks > 1 ? a.start0 : a.h0;
                    if (h0) v = h0[((int64_t)b * a.Dn + dd) * Nr + n];
                } else {
                    v = a.agg[(((int64_t)b * km1 + (seg - 1)) * Nr + n) * a.Dn + dd];
                }
            }
        }
        h[n] = v;
        P[n] = 1.f;
    }
    const float bias = a.bias ? a.bias[dd] : 0.f;
    const float Dd = a.D ? a.D[dd] : 0.f;
    const bool has_z = a.z != nullptr;

    const int64_t t0 = (int64_t)seg * a.chunk_len;
    const int64_t t1 = min(a.L, t0 + a.chunk_len);
    const int64_t row0 = (int64_t)b * a.L;

    const uint32_t rowb = (uint32_t)a.Dn * R::kSize;
    const uint32_t off0 = dvalid ? (uint32_t)d * R::kSize : kOutOfRange;
    auto block_rows = [&](int64_t tb) -> uint32_t {
        return (uint32_t)max((int64_t)0, min((int64_t)TB, t1 - tb));
    };  // rows of a block inside this segment (the prefetch past its end gets 0)
    auto block_base = [&](const void* p, int64_t tb) -> const void* {
        return static_cast<const char*>(p) + (row0 + tb) * (int64_t)rowb;
    };
    const uint32_t kBRow = (uint32_t)Nr * R::kSize;  // one timestep of B or C
    // Byte offset in a B/C row of the state lane `lane` holds in group k
    // (padded states read past the row: 0).
    uint32_t boff[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
        const int st = 16 * k + (lane & (RW - 1));
        boff[k] = (!PAD || st < Nr) ? (uint32_t)st * R::kSize : kOutOfRange;
    }
    auto bc_base = [&](const void* p, int64_t tb) -> const void* {
        return static_cast<const char*>(p) + (row0 + tb) * (int64_t)kBRow;
    };

    // Register buffers of one block's raw inputs (two when the next block is
    // prefetched while this one is computed).
    constexpr int NB = DB ? 2 : 1;
    RT ru[NB][TB], rd[NB][TB], rz[NB][TB], vb[NB][TB][KB], vc[NB][TB][KB];
    auto load_block = [&](int buf, int64_t tb) {
        const uint32_t nr = block_rows(tb);
        const auto rU = make_rsrc(block_base(a.u, tb), nr * rowb);
        const auto rD = make_rsrc(DTP ? a.u : block_base(a.delta, tb), DTP ? 0u : nr * rowb);
        const auto rZ = make_rsrc(has_z ? block_base(a.z, tb) : a.u, has_z ? nr * rowb : 0u);
        const auto rB = make_rsrc(bc_base(a.B, tb), nr * kBRow);
        const auto rC = make_rsrc(bc_base(a.C, tb), SUMMARY ? 0u : nr * kBRow);
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) {
            const uint32_t off = off0 + (uint32_t)tt * rowb;
            ru[buf][tt] = R::load(rU, off);
            if constexpr (!DTP) rd[buf][tt] = R::load(rD, off);
            if constexpr (!SUMMARY) rz[buf][tt] = R::load(rZ, off);
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const uint32_t o = (uint32_t)tt * kBRow + boff[k];
                vb[buf][tt][k] = R::load(rB, o);
                if constexpr (!SUMMARY) vc[buf][tt][k] = R::load(rC, o);
            }
        }
    };

    // SUMMARY: the sum of dt over the segment, compensated (Kahan) once per
    // block of TB steps; a block's own steps are added plainly.
    float s_sum = 0.f, s_comp = 0.f;
    auto kahan = [&](float v) {
        const float yk = v - s_comp;
        const float tk = s_sum + yk;
        s_comp = (tk - s_sum) - yk;
        s_sum = tk;
    };

    // One timestep: all N states of the lane's channel.
    auto step = [&](RT raw_u, float raw_d, RT raw_z, const RT (&raw_b)[KB], const RT (&raw_c)[KB],
                    float& y_out) {
        float vbt[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) vbt[k] = R::widen(raw_b[k]);
        const float uv = R::widen(raw_u);
        const float v = raw_d + bias;
        const float dt = SP ? softplus_f(v) : v;  // compile-time: no branch per step
        const float xv = ZOH ? uv : dt * uv;  // B is multiplied by u (ZOH) or dt*u
        float q1 = 0.f, q2 = 0.f;  // ZOH series coefficients for this dt
        if constexpr (ZOH) {
            const float dt2 = dt * dt;
            q1 = dt2 * kZohT1;
            q2 = dt2 * dt * kZohT2;
        }
        static_for(
            [&](auto nc) {
                constexpr int n = decltype(nc)::value;
                const float arg = dt * A2[n];
                float abar = 0.f, bx = 0.f;
                if constexpr (BIL) {
                    const float r = bilinear_r(arg);
                    const float ub = row_bcast<n % RW>(vbt[n / RW]) * xv;  // B * dt*u
                    if constexpr (PROD) {
                        abar = fmaf(2.f, r, -1.f);
                        bx = ub * r;
                    } else {
                        // (2r - 1) h + r (B dt u) = r (2h + B dt u) - h: two fma
                        h[n] = fmaf(r, fmaf(2.f, h[n], ub), -h[n]);
                    }
                } else {
                    abar = hw_exp2(arg);
                    const float bu = row_bcast<n % RW>(vbt[n / RW]) * xv;  // B*x (Euler) or B*u (ZOH)
                    if constexpr (ZOH)
                        bx = zoh_factor_q(dt, q1, q2, A2[n], A2sq[n], arg, abar, invA[n]) * bu;
                    else
                        bx = bu;
                }
                if constexpr (!BIL || PROD) h[n] = fmaf(abar, h[n], bx);
                if constexpr (PROD) P[n] *= abar;
                // With 32+ states the scheduler would otherwise start every
                // exponential before the first update and run out of VGPRs.
                if constexpr (N >= 32 && n % 8 == 7) __builtin_amdgcn_sched_barrier(0);
            },
            std::make_integer_sequence<int, N>{});
        if constexpr (SUMMARY && !PROD) {
            y_out = dt;  // summed by the caller
        } else if constexpr (!SUMMARY) {
            float y = DppReadout<RW>::run(R::widen(raw_c[0]), *reinterpret_cast<const float(*)[RW]>(h));
#pragma unroll
            for (int k = 1; k < KB; ++k) y = DppReadoutAcc16::run(y, R::widen(raw_c[k]), h + 16 * k);
            y = fmaf(Dd, uv, y);
            const float g = silu_f(R::widen(raw_z));
            y_out = y * (has_z ? g : 1.f);
        }
    };

    // DTP: the delta tile of timesteps [tp, tp + kPT), turned so that lane l
    // finds its channel's values at s_dt[l * kPTS + i].
    __shared__ __attribute__((aligned(16))) float s_dt[DTP ? 64 * kPTS : 4];
    auto project_tile = [&](int64_t tp) {
        if constexpr (DTP) {
            static_assert(kPT % TB == 0, "blocks inside a projected tile");
            const uint32_t xrow = (uint32_t)a.rank * R::kSize;
            const uint32_t nr = (uint32_t)max((int64_t)0, min((int64_t)kPT, a.L - tp));
            const auto rX = make_rsrc(static_cast<const char*>(a.dtx) + (row0 + tp) * (int64_t)xrow,
                                      nr * xrow);  // rows past L read 0
            const auto rW = make_rsrc(a.wdt, (uint32_t)a.Dn * xrow);  // channels past Dn read 0
            const bool vec = (a.rank % (BF16 ? 8 : 4)) == 0;
            const int m = lane & 15, q = lane >> 4;
            const uint32_t d0 = blockIdx.x * 64u;
            __syncthreads();  // the previous tile has been read
            f4 acc[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[g] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int kc = 0; kc < kMaxRank / 32; ++kc) {
                if (kc * 32 < a.rank) {  // uniform
                    const int k0 = kc * 32 + 8 * q;
                    Frag8<BF16> xf, wf[4];
                    // A operand: row m = timestep tp + m; B operand: column m
                    // of group g = channel d0 + 16 g + m; both take k0 .. k0+7.
                    xf.load(rX, (uint32_t)m * xrow, k0, a.rank, vec);
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        wf[g].load(rW, (d0 + 16u * g + (uint32_t)m) * xrow, k0, a.rank, vec);
#pragma unroll
                    for (int g = 0; g < 4; ++g) xf.mma(wf[g], acc[g]);
                }
            }
            // acc[g][i] is delta at timestep 4q + i, channel 16g + m.
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *reinterpret_cast<f4*>(&s_dt[(16 * g + m) * kPTS + 4 * q]) = acc[g];
            __syncthreads();
        }
    };
    auto block_delta = [&](int cur, int64_t tb, int tt) -> float {
        if constexpr (DTP)
            return s_dt[lane * kPTS + (int)((tb - t0) & (kPT - 1)) + tt];
        else
            return R::widen(rd[cur][tt]);
    };

    // A full block of TB timesteps, straight-line code.  The ragged end of
    // the last segment is left to a one-step loop below: a shared body with a
    // per-step guard would make every step a branch target and cost a copy of
    // every state per step.
    auto do_block = [&](auto cur_c, int blk) {
        constexpr int cur = decltype(cur_c)::value;
        const int64_t tb = t0 + (int64_t)blk * TB;
        if constexpr (DB)
            load_block(cur ^ 1, tb + TB);  // past the end it reads zeros
        else
            load_block(cur, tb);
        if constexpr (DTP) {
            if (((tb - t0) & (kPT - 1)) == 0) project_tile(tb);
        }
        const auto rY = make_rsrc(block_base(a.y, tb), (uint32_t)TB * rowb);
        float bsum = 0.f;
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) {
            float y = 0.f;
            step(ru[cur][tt], block_delta(cur, tb, tt), rz[cur][tt], vb[cur][tt], vc[cur][tt], y);
            if constexpr (!SUMMARY) R::store(rY, off0 + (uint32_t)tt * rowb, y);
            else bsum += y;
        }
        if constexpr (SUMMARY && !PROD) kahan(bsum);
    };

    const int nfull = (int)((t1 - t0) / TB);
    int blk = 0;
    if constexpr (DB) {
        load_block(0, t0);
        for (; blk + 1 < nfull; blk += 2) {
            do_block(std::integral_constant<int, 0>{}, blk);
            do_block(std::integral_constant<int, 1>{}, blk + 1);
        }
        if (blk < nfull) do_block(std::integral_constant<int, 0>{}, blk);
    } else {
        for (; blk < nfull; ++blk) do_block(std::integral_constant<int, 0>{}, blk);
    }
    // Ragged end (only the last segment can have one): one timestep at a time.
    for (int64_t t = t0 + (int64_t)nfull * TB; t < t1; ++t) {
        const auto rU = make_rsrc(block_base(a.u, t), rowb);
        const auto rD = make_rsrc(DTP ? a.u : block_base(a.delta, t), DTP ? 0u : rowb);
        const auto rZ = make_rsrc(has_z ? block_base(a.z, t) : a.u, has_z ? rowb : 0u);
        const RT xu = R::load(rU, off0);
        float xd;
        if constexpr (DTP) {
            if (((t - t0) & (kPT - 1)) == 0) project_tile(t);
            xd = s_dt[lane * kPTS + (int)((t - t0) & (kPT - 1))];
        } else {
            xd = R::widen(R::load(rD, off0));
        }
        const RT xz = SUMMARY ? RT{} : R::load(rZ, off0);
        RT xb[KB], xc[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const uint32_t o = boff[k];
            xb[k] = R::load(make_rsrc(bc_base(a.B, t), kBRow), o);
            xc[k] = SUMMARY ? RT{} : R::load(make_rsrc(bc_base(a.C, t), kBRow), o);
        }
        float y = 0.f;
        step(xu, xd, xz, xb, xc, y);
        if constexpr (!SUMMARY) R::store(make_rsrc(block_base(a.y, t), rowb), off0, y);
        if constexpr (SUMMARY && !PROD) kahan(y);
    }

    if (!dvalid) return;
    if constexpr (SUMMARY) {
        const int64_t base = (int64_t)b * km1 + seg;
#pragma unroll
        for (int n = 0; n < N; ++n)
            if (!PAD || n < Nr) a.agg[(base * Nr + n) * a.Dn + d] = h[n];
        if constexpr (PROD) {
#pragma unroll
            for (int n = 0; n < N; ++n)
                if (!PAD || n < Nr) a.prod[(base * Nr + n) * a.Dn + d] = P[n];
        } else {
            a.sdt[base * a.Dn + d] = s_sum;
        }
    } else {
        if (seg == a.chunks - 1 && a.h_last) {
#pragma unroll
            for (int n = 0; n < N; ++n)
                if (!PAD || n < Nr) a.h_last[((int64_t)b * a.Dn + d) * Nr + n] = h[n];
        }
    }
}

template <int N, bool BF16, int DISC, bool SP, bool DTP = false, bool PAD = false>
hipError_t launch_lanes(const Plan& p, const ScanArgs& a, hipStream_t s) {
    // 64 states (32 with the extra per-state values of ZOH or the bilinear
    // summary) leave room for one register block only: no prefetch.
    constexpr bool kBig = N >= 64 || (N >= 32 && DISC != kEuler);
    constexpr int TB = kBig ? MSSCAN_LANE_TB64 : MSSCAN_LANE_TB;
    constexpr bool DB = kBig ? MSSCAN_LANE_DB64 != 0 : MSSCAN_LANE_DB != 0;
    hipError_t e = hipSuccess;
    if (p.chunks > 1) {
        {
            ProfScope ps(s, kPhaseSummary);
            hipLaunchKernelGGL((scan_lane<N, TB, DB, BF16, DISC, SP, true, DTP, PAD>),
                               dim3(p.tiles, p.chunks - 1, a.batch), dim3(64), 0, s, a);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_carry(a, s);
        if (e != hipSuccess) return e;
    }
    {
        ProfScope ps(s, kPhaseMain);
        hipLaunchKernelGGL((scan_lane<N, TB, DB, BF16, DISC, SP, false, DTP, PAD>),
                           dim3(p.tiles, p.chunks, a.batch), dim3(64), 0, s, a);
    }
    return hipGetLastError();
}

template <bool BF16, int DISC>
hipError_t dispatch_dtp(const Plan& p, const ScanArgs& a, hipStream_t s) {
    switch (p.ns) {
        case 8: return a.softplus ? launch_lanes<8, BF16, DISC, true, true>(p, a, s)
                                  : launch_lanes<8, BF16, DISC, false, true>(p, a, s);
        case 16: return a.softplus ? launch_lanes<16, BF16, DISC, true, true>(p, a, s)
                                   : launch_lanes<16, BF16, DISC, false, true>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16, int DISC, bool SP, bool PAD>
hipError_t dispatch_n(const Plan& p, const ScanArgs& a, hipStream_t s) {
    switch (p.ns) {
        case 8: return launch_lanes<8, BF16, DISC, SP, false, PAD>(p, a, s);
        case 16: return launch_lanes<16, BF16, DISC, SP, false, PAD>(p, a, s);
        case 32: return launch_lanes<32, BF16, DISC, SP, false, PAD>(p, a, s);
        case 64:
            if constexpr (DISC == kEuler) return launch_lanes<64, BF16, DISC, SP, false, PAD>(p, a, s);
            return hipErrorInvalidValue;  // 64 ZOH/bilinear states do not fit a lane
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16, int DISC>
hipError_t dispatch(const Plan& p, const ScanArgs& a, hipStream_t s) {
    if (a.N != p.ns)  // d_state padded up to the variant's states
        return a.softplus ? dispatch_n<BF16, DISC, true, true>(p, a, s)
                          : dispatch_n<BF16, DISC, false, true>(p, a, s);
    return a.softplus ? dispatch_n<BF16, DISC, true, false>(p, a, s)
                      : dispatch_n<BF16, DISC, false, false>(p, a, s);
}

template <bool BF16>
hipError_t dispatch_disc(const Plan& p, const ScanArgs& a, int disc, hipStream_t s) {
    switch (disc) {
        case kEuler: return dispatch<BF16, kEuler>(p, a, s);
        case kZoh: return dispatch<BF16, kZoh>(p, a, s);
        case kBilinear: return dispatch<BF16, kBilinear>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scan_lanes_dtproj(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                    hipStream_t s) {
    if (a.rank < 1 || a.rank > kMaxRank) return hipErrorInvalidValue;
    switch (disc) {
        case kEuler: return bf16 ? dispatch_dtp<true, kEuler>(p, a, s) : dispatch_dtp<false, kEuler>(p, a, s);
        case kZoh: return bf16 ? dispatch_dtp<true, kZoh>(p, a, s) : dispatch_dtp<false, kZoh>(p, a, s);
        case kBilinear: return bf16 ? dispatch_dtp<true, kBilinear>(p, a, s)
                                    : dispatch_dtp<false, kBilinear>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

bool dtproj_variant_exists(int n) { return n == 8 || n == 16; }

bool lane_variant_exists(int n, int disc) {
    return n == 8 || n == 16 || n == 32 || (n == 64 && disc == kEuler);
}

hipError_t launch_scan_lanes(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                             hipStream_t s) {
    return bf16 ? dispatch_disc<true>(p, a, disc, s) : dispatch_disc<false>(p, a, disc, s);
}

}  // namespace msscan
