// scan_kernels.hip -- generic HIP kernels of the selective scan (S6) for
// gfx950 (any d_state the fast paths do not take), the carry pass every path
// shares, and the one-step decode fallback.
//
// Method (per batch b, channel d, state n; see include/msscan.h for the full
// statement and the passages it follows):
//   dt = softplus(delta + bias),  A_bar = exp(dt*A[d,n]),
//   h  = A_bar*h + B_bar*u  with B_bar = dt*B (Euler) or expm1(dt*A)/A*B (ZOH),
//   y  = sum_n C*h + D*u,  out = y*silu(z).
//
// Work mapping (CDNA4, wave64):
//   * lane  = one channel d of a 64-channel tile: u/delta/z/y rows are read and
//     written as 64 consecutive elements per wave (coalesced), and B_t/C_t --
//     shared by every channel (lmnt page section 3.2 broadcasts them over
//     channels) -- are wave-uniform, so they travel through scalar loads and
//     SGPR operands instead of per-lane registers;
//   * the lane's `NS` states live in VGPRs for the whole piece of sequence it
//     scans; a workgroup of `waves` waves covers d_state = waves*NS states and
//     sums their partial readouts through LDS;
//   * the sequence is cut into pieces ("chunks").  The scan is a composition
//     of affine maps h -> a*h + b (jsqmd page section 3.4), so a chunk is
//     summarised by (a, b) = (exp(A * sum dt), state reached from 0) -- for
//     the bilinear form a is the product of the chunk's A_bar.  Pass 1
//     (scan_summary) computes every chunk's b and sum dt, pass 2
//     (carry_chain) composes them in order to get each chunk's starting
//     state, pass 3 (scan_chunks) rescans every chunk from its true starting
//     state and writes y.  No pass waits on another workgroup, so there is no
//     spin-wait and the association order -- hence every output bit -- is
//     fixed by the plan alone.
//
// Arithmetic: fp32 throughout; bf16 io is widened exactly (bits << 16) and
// rounded back to nearest-even.  exp/log use the hardware base-2
// instructions with log2(e) folded into A once per (d, n).
#include <hip/hip_runtime.h>
#include <stdint.h>


#include "device_common.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

constexpr int kTB = 16;  // timesteps per LDS exchange when waves > 1

// Load the lane's A row slice (pre-multiplied by log2 e) and, for ZOH, 1/A.
template <int NS, bool ZOH>
__device__ __forceinline__ void load_a(const float* A, int dd, int N, int n0, int nvalid,
                                       float (&A2)[NS], float (&invA)[NS]) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        float av = (j < nvalid) ? A[(int64_t)dd * N + n0 + j] : 0.f;
        A2[j] = av * kLog2e;
        if constexpr (ZOH) invA[j] = (av != 0.f) ? 1.f / av : 0.f;
    }
}

// One timestep of the lane's NS states; returns the partial readout.  PROD
// multiplies each state's A_bar into P (the bilinear segment decay).
template <int NS, bool BF16, int DISC, bool READOUT, bool PROD = false>
__device__ __forceinline__ float advance(float (&h)[NS], float (&P)[NS], const float (&A2)[NS],
                                         const float (&invA)[NS], float dt, float uval,
                                         const void* B, const void* C, int64_t row,
                                         int nvalid) {
    float y = 0.f;
    const float x = dt * uval;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const bool ok = j < nvalid;
        const float bn = ok ? ld<BF16>(B, row + j) : 0.f;
        const float arg = dt * A2[j];
        float abar, bx;
        if constexpr (DISC == kBilinear) {
            const float r = bilinear_r(arg);
            abar = fmaf(2.f, r, -1.f);
            bx = (x * r) * bn;
        } else {
            abar = hw_exp2(arg);
            if constexpr (DISC == kZoh)
                bx = zoh_factor(dt, arg, abar, invA[j]) * (bn * uval);
            else
                bx = x * bn;
        }
        if constexpr (PROD) P[j] *= abar;
        h[j] = fmaf(abar, h[j], bx);
        if constexpr (READOUT) {
            const float cn = ok ? ld<BF16>(C, row + j) : 0.f;
            y = fmaf(cn, h[j], y);
        }
    }
    return y;
}

// ---- pass 1: chunk summaries --------------------------------------------------
// For every chunk but the last: the state reached from h = 0 over the chunk
// (the "b" of its affine summary) and the compensated sum of dt (the "a" is
// exp(A * sum dt), formed in pass 2) -- or, for the bilinear form, whose
// decay is not an exponential of sum dt, the product of A_bar per state.
template <int NS, bool BF16, int DISC>
__global__ void __launch_bounds__(256) scan_summary(ScanArgs a) {
    constexpr bool ZOH = DISC == kZoh;
    constexpr bool PROD = DISC == kBilinear;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = blockIdx.x;  // 0 .. chunks-2
    const int b = blockIdx.z;
    const int d = blockIdx.y * 64 + lane;
    const bool dvalid = d < a.Dn;
    const int dd = dvalid ? d : a.Dn - 1;
    const int n0 = w * NS;
    const int nvalid = min(NS, a.N - n0);

    float A2[NS], invA[NS], h[NS], P[NS];
    load_a<NS, ZOH>(a.A, dd, a.N, n0, nvalid, A2, invA);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        h[j] = 0.f;
        P[j] = 1.f;
    }
    const float bias = a.bias ? a.bias[dd] : 0.f;

    const int64_t t0 = (int64_t)c * a.chunk_len;
    const int64_t t1 = min(a.L, t0 + a.chunk_len);
    float s = 0.f, comp = 0.f;  // Kahan sum of dt
    for (int64_t t = t0; t < t1; ++t) {
        const int64_t e = ((int64_t)b * a.L + t) * a.Dn + dd;
        const float uval = ld<BF16>(a.u, e);
        const float dt = step_size(ld<BF16>(a.delta, e), bias, a.softplus);
        const float yk = dt - comp;
        const float tk = s + yk;
        comp = (tk - s) - yk;
        s = tk;
        advance<NS, BF16, DISC, false, PROD>(h, P, A2, invA, dt, uval, a.B, nullptr,
                                             ((int64_t)b * a.L + t) * a.N + n0, nvalid);
    }
    if (!dvalid) return;
    const int km1 = a.chunks - 1;
    const int64_t base = (int64_t)b * km1 + c;
#pragma unroll
    for (int j = 0; j < NS; ++j)
        if (j < nvalid) a.agg[(base * a.N + n0 + j) * a.Dn + d] = h[j];
    if constexpr (PROD) {
#pragma unroll
        for (int j = 0; j < NS; ++j)
            if (j < nvalid) a.prod[(base * a.N + n0 + j) * a.Dn + d] = P[j];
    } else {
        if (w == 0) a.sdt[base * a.Dn + d] = s;
    }
}

// ---- pass 2: compose chunk summaries in order --------------------------------
// One thread per (b, n, d).  Slot i of the summaries holds chunk i's map
// h -> a_i*h + b_i; it is replaced by the state at the start of chunk i+1:
// h_{i+1} = a_i*h_i + b_i, h_0 = the initial state or 0.  The decay a_i is
// exp(A * sum dt_i) or, when the summaries hold products of A_bar (bilinear),
// that product.  REV takes the slots last to first, which is the adjoint's
// carry in the backward.
//
// The kernel streams the summaries once in and once out (at the 130M layer's
// backward about 200 MB per call) and is bound by HBM bandwidth.  Loads of a
// group of slots are issued before its updates, so the chain waits on memory
// once per group, not once per slot.  A two-level form (waves of one
// workgroup folding runs of slots, then one barrier) and 16-byte accesses
// over four channels per thread both measured slower.
template <bool REV>
__global__ void __launch_bounds__(256) carry_chain(CarryArgs c) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)c.batch * c.N * c.Dn;
    if (idx >= total) return;
    const int d = (int)(idx % c.Dn);
    const int n = (int)((idx / c.Dn) % c.N);
    const int b = (int)(idx / ((int64_t)c.Dn * c.N));
    const bool prod = c.prod != nullptr;
    const float A2 = c.A[(int64_t)d * c.N + n] * kLog2e;
    float h = c.init ? c.init[((int64_t)b * c.Dn + d) * c.N + n] : 0.f;
    const int km1 = c.km1;
    for (int i0 = 0; i0 < km1; i0 += kCarryGroup) {
        float dv[kCarryGroup], gv[kCarryGroup];
#pragma unroll
        for (int j = 0; j < kCarryGroup; ++j) {
            dv[j] = 0.f;
            gv[j] = 0.f;
            const int i = i0 + j;
            if (i < km1) {
                const int64_t base = (int64_t)b * km1 + (REV ? km1 - 1 - i : i);
                dv[j] = prod ? c.prod[(base * c.N + n) * c.Dn + d] : c.sdt[base * c.Dn + d];
                gv[j] = c.val[(base * c.N + n) * c.Dn + d];
            }
        }
#pragma unroll
        for (int j = 0; j < kCarryGroup; ++j) {
            const int i = i0 + j;
            if (i < km1) {
                const int64_t base = (int64_t)b * km1 + (REV ? km1 - 1 - i : i);
                const float decay = prod ? dv[j] : hw_exp2(A2 * dv[j]);
                h = fmaf(decay, h, gv[j]);
                c.val[(base * c.N + n) * c.Dn + d] = h;
            }
        }
    }
}

// ---- pass 3: rescan every chunk from its true start, write y -----------------
template <int NS, bool BF16, int DISC, bool MULTI>
__global__ void __launch_bounds__(256) scan_chunks(ScanArgs a) {
    constexpr bool ZOH = DISC == kZoh;
    __shared__ float ypart[MULTI ? 4 : 1][MULTI ? kTB : 1][64];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int c = blockIdx.x;
    const int b = blockIdx.z;
    const int d = blockIdx.y * 64 + lane;
    const bool dvalid = d < a.Dn;
    const int dd = dvalid ? d : a.Dn - 1;
    const int n0 = w * NS;
    const int nvalid = min(NS, a.N - n0);

    float A2[NS], invA[NS], h[NS], P[NS];
    load_a<NS, ZOH>(a.A, dd, a.N, n0, nvalid, A2, invA);
    const int km1 = a.chunks - 1;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        float v = 0.f;
        if (j < nvalid) {
            if (c == 0) {
                if (a.h0) v = a.h0[((int64_t)b * a.Dn + dd) * a.N + n0 + j];
            } else {
                v = a.agg[(((int64_t)b * km1 + (c - 1)) * a.N + n0 + j) * a.Dn + dd];
            }
        }
        h[j] = v;
    }
    const float bias = a.bias ? a.bias[dd] : 0.f;
    const float Dd = a.D ? a.D[dd] : 0.f;

    const int64_t t0 = (int64_t)c * a.chunk_len;
    const int64_t t1 = min(a.L, t0 + a.chunk_len);
    if constexpr (!MULTI) {
        for (int64_t t = t0; t < t1; ++t) {
            const int64_t e = ((int64_t)b * a.L + t) * a.Dn + dd;
            const float uval = ld<BF16>(a.u, e);
            const float dt = step_size(ld<BF16>(a.delta, e), bias, a.softplus);
            float y = advance<NS, BF16, DISC, true>(h, P, A2, invA, dt, uval, a.B, a.C,
                                                   ((int64_t)b * a.L + t) * a.N + n0, nvalid);
            y = fmaf(Dd, uval, y);
            if (a.z) y *= silu_f(ld<BF16>(a.z, e));
            if (dvalid) st<BF16>(a.y, e, y);
        }
    } else {
        for (int64_t tb = t0; tb < t1; tb += kTB) {
            const int cnt = (int)min((int64_t)kTB, t1 - tb);
            for (int tt = 0; tt < cnt; ++tt) {
                const int64_t t = tb + tt;
                const int64_t e = ((int64_t)b * a.L + t) * a.Dn + dd;
                const float uval = ld<BF16>(a.u, e);
                const float dt = step_size(ld<BF16>(a.delta, e), bias, a.softplus);
                ypart[w][tt][lane] = advance<NS, BF16, DISC, true>(
                    h, P, A2, invA, dt, uval, a.B, a.C, ((int64_t)b * a.L + t) * a.N + n0, nvalid);
            }
            __syncthreads();
            for (int tt = w; tt < cnt; tt += nw) {
                const int64_t e = ((int64_t)b * a.L + tb + tt) * a.Dn + dd;
                float y = 0.f;
                for (int s = 0; s < nw; ++s) y += ypart[s][tt][lane];
                y = fmaf(Dd, ld<BF16>(a.u, e), y);
                if (a.z) y *= silu_f(ld<BF16>(a.z, e));
                if (dvalid) st<BF16>(a.y, e, y);
            }
            __syncthreads();
        }
    }
    if (c == a.chunks - 1 && a.h_last && dvalid) {
#pragma unroll
        for (int j = 0; j < NS; ++j)
            if (j < nvalid) a.h_last[((int64_t)b * a.Dn + d) * a.N + n0 + j] = h[j];
    }
}

// ---- decode step ---------------------------------------------------------------
// One thread per (b, d): the channel's N-state row (contiguous in h) is read,
// advanced one step and written back; B_t, C_t are uniform over the block's
// channels (one batch row per block).
template <bool BF16, int DISC>
__global__ void __launch_bounds__(256) state_step(StepArgs a) {
    const int d = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    if (d >= a.Dn) return;
    const int64_t e = (int64_t)b * a.Dn + d;
    const float xv = ld<BF16>(a.x, e);
    const float dt = step_size(ld<BF16>(a.delta, e), a.bias ? a.bias[d] : 0.f, a.softplus);
    const float dx = dt * xv;
    float* hrow = a.h + e * a.N;
    const float* arow = a.A + (int64_t)d * a.N;
    const int64_t brow = (int64_t)b * a.N;
    float y = 0.f;
    for (int n = 0; n < a.N; ++n) {
        const float an = arow[n];
        const float arg = dt * (an * kLog2e);
        const float bn = ld<BF16>(a.B, brow + n);
        float abar, bx;
        if constexpr (DISC == kBilinear) {
            const float r = bilinear_r(arg);
            abar = fmaf(2.f, r, -1.f);
            bx = (dx * r) * bn;
        } else {
            abar = hw_exp2(arg);
            if constexpr (DISC == kZoh)
                bx = zoh_factor(dt, arg, abar, an != 0.f ? 1.f / an : 0.f) * (bn * xv);
            else
                bx = dx * bn;
        }
        const float hn = fmaf(abar, hrow[n], bx);
        hrow[n] = hn;
        y = fmaf(ld<BF16>(a.C, brow + n), hn, y);
    }
    y = fmaf(a.D ? a.D[d] : 0.f, xv, y);
    if (a.z) y *= silu_f(ld<BF16>(a.z, e));
    st<BF16>(a.y, e, y);
}

template <int NS, bool BF16, int DISC>
hipError_t launch_ns(const Plan& p, const ScanArgs& a, hipStream_t s) {
    const dim3 block(64 * p.waves);
    if (p.chunks > 1) {
        {
            ProfScope ps(s, kPhaseSummary);
            hipLaunchKernelGGL((scan_summary<NS, BF16, DISC>), dim3(p.chunks - 1, p.tiles, a.batch),
                               block, 0, s, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_carry(a, s);
        if (e != hipSuccess) return e;
    }
    ProfScope ps(s, kPhaseMain);
    if (p.waves > 1) {
        if constexpr (NS == 32)
            hipLaunchKernelGGL((scan_chunks<NS, BF16, DISC, true>),
                               dim3(p.chunks, p.tiles, a.batch), block, 0, s, a);
        else
            return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((scan_chunks<NS, BF16, DISC, false>), dim3(p.chunks, p.tiles, a.batch),
                           block, 0, s, a);
    }
    return hipGetLastError();
}

template <bool BF16, int DISC>
hipError_t launch_io(const Plan& p, const ScanArgs& a, hipStream_t s) {
    switch (p.ns) {
        case 4: return launch_ns<4, BF16, DISC>(p, a, s);
        case 8: return launch_ns<8, BF16, DISC>(p, a, s);
        case 16: return launch_ns<16, BF16, DISC>(p, a, s);
        case 32: return launch_ns<32, BF16, DISC>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

template <bool BF16>
hipError_t launch_disc(const Plan& p, const ScanArgs& a, int disc, hipStream_t s) {
    switch (disc) {
        case kEuler: return launch_io<BF16, kEuler>(p, a, s);
        case kZoh: return launch_io<BF16, kZoh>(p, a, s);
        case kBilinear: return launch_io<BF16, kBilinear>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_scan(const Plan& p, const ScanArgs& a, bool bf16, int disc, hipStream_t s) {
    return bf16 ? launch_disc<true>(p, a, disc, s) : launch_disc<false>(p, a, disc, s);
}

hipError_t launch_carry(const CarryArgs& c, bool reverse, hipStream_t s) {
    if (c.km1 <= 0) return hipSuccess;
    const int64_t total = (int64_t)c.batch * c.N * c.Dn;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    ProfScope ps(s, kPhaseCarry);
    if (reverse)
        hipLaunchKernelGGL(carry_chain<true>, grid, block, 0, s, c);
    else
        hipLaunchKernelGGL(carry_chain<false>, grid, block, 0, s, c);
    return hipGetLastError();
}

hipError_t launch_carry(const ScanArgs& a, hipStream_t s) {
    CarryArgs c{};
    c.val = a.agg;
    c.sdt = a.sdt;
    c.prod = a.prod;
    c.A = a.A;
    c.init = a.h0;
    c.batch = a.batch;
    c.km1 = a.chunks - 1;
    c.N = a.N;
    c.Dn = a.Dn;
    return launch_carry(c, false, s);
}

hipError_t launch_step(const StepArgs& a, bool bf16, int disc, hipStream_t s) {
    const dim3 grid((a.Dn + 255) / 256, a.batch), block(256);
    ProfScope ps(s, kPhaseStep);
#define MS_STEP_(DI)                                                           \
    if (bf16)                                                                  \
        hipLaunchKernelGGL((state_step<true, DI>), grid, block, 0, s, a);      \
    else                                                                       \
        hipLaunchKernelGGL((state_step<false, DI>), grid, block, 0, s, a);
    switch (disc) {
        case kEuler: MS_STEP_(kEuler) break;
        case kZoh: MS_STEP_(kZoh) break;
        case kBilinear: MS_STEP_(kBilinear) break;
        default: return hipErrorInvalidValue;
    }
#undef MS_STEP_
    return hipGetLastError();
}

}  // namespace msscan
