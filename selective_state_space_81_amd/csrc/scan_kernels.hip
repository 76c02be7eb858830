// scan_kernels.hip -- the pieces every scan path shares, for gfx950: the
// carry pass that composes segment summaries, and the one-step decode
// fallback for d_state without a quad kernel.
//
// The scan is a composition of affine maps h -> a*h + b (jsqmd page section
// 3.4), so a segment of the sequence is summarised by (a, b) = (exp(A * sum
// dt), state reached from 0), or for the bilinear form by the product of its
// A_bar.  The summary passes of the lane and tile kernels write b and sum dt;
// the carry pass here composes them in order into each segment's starting
// state.  No pass waits on another workgroup, so there is no spin-wait and
// the association order -- hence every output bit -- is fixed by the plan.
#include <hip/hip_runtime.h>
#include <stdint.h>


#include "device_common.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

// ---- the carry: compose segment summaries in order --------------------------------
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

}  // namespace

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
