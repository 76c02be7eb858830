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
// memory once per group, not once per slot.  For chains of a few hundred
// slots, a two-level form (carry_parts below) and 16-byte accesses over four
// channels per thread both measured slower.  Chains of kCarryLongChain slots
// or more go to carry_parts.
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

// The same composition for long chains, split over P waves per 64 (b, n, d)
// columns: wave w takes the run of slots [w S, (w + 1) S), folds it into one
// map (the product of its decays, and the state its run reaches from 0),
// the waves' maps go through LDS, each wave composes those of the waves
// before it onto the initial state, and then walks its run again from that
// start, writing every slot as the chain does.  The summaries are read
// twice, but P times as many waves keep loads in flight: with few (b, n, d)
// columns and long chains (the d_state 17-128 backward: 16-step segments,
// one 16-state slice of 1536 channels at a time, 4095 slots at L 65536) the
// loads in flight bound the chain's rate.  There P = 16 took the backward's
// carries from 5.7 ms per call (the chain with groups of 8; 4.3 with groups
// of 32) to 3.0 ms; P = 4 gave 3.6 ms, and groups of 16 inside the parts no
// more than 2%.
#ifndef MSSCAN_CARRY_PARTS
#define MSSCAN_CARRY_PARTS 16
#endif
constexpr int kCarryParts = MSSCAN_CARRY_PARTS;
#ifndef MSSCAN_CARRY_PARTS_G
#define MSSCAN_CARRY_PARTS_G 8
#endif
constexpr int kCarryPartsGroup = MSSCAN_CARRY_PARTS_G;

template <bool REV, int P, int G>
__global__ void __launch_bounds__(64 * P) carry_parts(CarryArgs c) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t idx = (int64_t)blockIdx.x * 64 + lane;
    const int64_t total = (int64_t)c.batch * c.N * c.Dn;
    const bool valid = idx < total;
    const int64_t ci = valid ? idx : total - 1;  // lanes past the end compute, store nothing
    const int d = (int)(ci % c.Dn);
    const int n = (int)((ci / c.Dn) % c.N);
    const int b = (int)(ci / ((int64_t)c.Dn * c.N));
    const bool prod = c.prod != nullptr;
    const float A2 = c.A[(int64_t)d * c.N + n] * kLog2e;
    const int km1 = c.km1;
    const int S = (km1 + P - 1) / P;
    const int i0 = min(km1, w * S), i1 = min(km1, i0 + S);
    auto slot = [&](int i) -> int64_t { return (int64_t)b * km1 + (REV ? km1 - 1 - i : i); };
    // one run of slots: decays and values loaded G at a time, then f(decay, value, slot)
    auto walk = [&](auto f) __attribute__((always_inline)) {
        for (int g0 = i0; g0 < i1; g0 += G) {
            float dv[G], gv[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                dv[j] = 0.f;
                gv[j] = 0.f;
                if (g0 + j < i1) {
                    const int64_t base = slot(g0 + j);
                    dv[j] = prod ? c.prod[(base * c.N + n) * c.Dn + d] : c.sdt[base * c.Dn + d];
                    gv[j] = c.val[(base * c.N + n) * c.Dn + d];
                }
            }
#pragma unroll
            for (int j = 0; j < G; ++j)
                if (g0 + j < i1) f(prod ? dv[j] : hw_exp2(A2 * dv[j]), gv[j], slot(g0 + j));
        }
    };
    float pa = 1.f, pb = 0.f;  // this run as a map h -> pa h + pb
    walk([&](float decay, float v, int64_t) {
        pa *= decay;
        pb = fmaf(decay, pb, v);
    });
    __shared__ float s_a[P][64], s_b[P][64];
    s_a[w][lane] = pa;
    s_b[w][lane] = pb;
    __syncthreads();
    float h = c.init ? c.init[((int64_t)b * c.Dn + d) * c.N + n] : 0.f;
    if (w == 0 && valid && c.start0) c.start0[((int64_t)b * c.Dn + d) * c.N + n] = h;
    for (int v = 0; v < w; ++v) h = fmaf(s_a[v][lane], h, s_b[v][lane]);
    walk([&](float decay, float v, int64_t base) {
        h = fmaf(decay, h, v);
        if (valid) c.val[(base * c.N + n) * c.Dn + d] = h;
    });
}

}  // namespace

hipError_t launch_carry(const CarryArgs& c, bool reverse, hipStream_t s) {
    if (c.km1 <= 0) return hipSuccess;
    const int64_t total = (int64_t)c.batch * c.N * c.Dn;
    const dim3 grid((unsigned)((total + 255) / 256)), block(256);
    ProfScope ps(s, kPhaseCarry);
    if (c.km1 >= kCarryLongChain) {
        const dim3 pgrid((unsigned)((total + 63) / 64)), pblock(64 * kCarryParts);
        if (reverse)
            hipLaunchKernelGGL((carry_parts<true, kCarryParts, kCarryPartsGroup>), pgrid, pblock, 0, s, c);
        else
            hipLaunchKernelGGL((carry_parts<false, kCarryParts, kCarryPartsGroup>), pgrid, pblock, 0, s, c);
    } else if (reverse) {
        hipLaunchKernelGGL((carry_chain<true, kCarryGroup>), grid, block, 0, s, c);
    } else {
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
