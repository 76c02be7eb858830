// scan_kernels.hip -- the carry pass every scan path shares, for gfx950: it
// composes the segment summaries in order.
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
// group of G slots are issued before its updates, so the chain waits on
// memory once per group, not once per slot.  With few (b, n, d) threads and
// long chains (the d_state 17-128 backward: 16-step segments, one 16-state
// slice of 1536 channels at a time) the loads in flight bound the rate, and
// G = 32 instead of 8 took the L 65536 backward's carries from 5.7 to 4.3 ms
// per call; for chains of a few hundred slots it measured no better.  A
// two-level form (waves of one workgroup folding runs of slots, then one
// barrier) and 16-byte accesses over four channels per thread both measured
// slower.
template <bool REV, int G>
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
    if (c.start0) c.start0[((int64_t)b * c.Dn + d) * c.N + n] = h;
    const int km1 = c.km1;
    for (int i0 = 0; i0 < km1; i0 += G) {
        float dv[G], gv[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
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
        for (int j = 0; j < G; ++j) {
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

}  // namespace

hipError_t launch_carry(const CarryArgs& c, bool reverse, hipStream_t s) {
    if (c.km1 <= 0) return hipSuccess;
    const int64_t total = (int64_t)c.batch * c.N * c.Dn;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    ProfScope ps(s, kPhaseCarry);
    const bool lng = c.km1 >= kCarryLongChain;
    if (reverse) {
        if (lng)
            hipLaunchKernelGGL((carry_chain<true, kCarryGroupLong>), grid, block, 0, s, c);
        else
            hipLaunchKernelGGL((carry_chain<true, kCarryGroup>), grid, block, 0, s, c);
    } else {
        if (lng)
            hipLaunchKernelGGL((carry_chain<false, kCarryGroupLong>), grid, block, 0, s, c);
        else
            hipLaunchKernelGGL((carry_chain<false, kCarryGroup>), grid, block, 0, s, c);
    }
    return hipGetLastError();
}

hipError_t launch_carry(const ScanArgs& a, hipStream_t s) {
    CarryArgs c{};
    c.val = a.agg;
    c.sdt = a.sdt;
    c.prod = a.prod;
    c.A = a.A;
    c.init = a.h0;
    c.start0 = a.start0;
    c.batch = a.batch;
    c.km1 = a.chunks - 1;
    c.N = a.N;
    c.Dn = a.Dn;
    return launch_carry(c, false, s);
}

}  // namespace msscan
