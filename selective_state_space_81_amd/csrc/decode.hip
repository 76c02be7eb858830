// decode.hip -- one recurrent decode step (ms_state_update), any d_state up
// to 128 (4 * 2^k exactly, other sizes padded up to the next such).
//
// The step is one timestep of the scan with the state kept in HBM between
// calls (lmnt.cn page, section 5.3; the state cache of the jsqmd page,
// section 5.3): per (b, d) read x_t, delta_t, z_t, per n read and rewrite
// h[b, d, n].  Its bytes are dominated by the fp32 state (read and written
// once per step), so the kernel is laid out for that stream (see
// step_quads); the per-element work (softplus, gate) is repeated by the G
// lanes of a channel, which costs little next to the state traffic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

// Four consecutive io values as fp32.
template <bool BF16>
__device__ __forceinline__ float4 ld4(const void* p, int64_t i) {
    if constexpr (BF16) {
        const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
        return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                           __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
    } else {
        return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    }
}

#ifndef MSSCAN_STEP_ROWS
#define MSSCAN_STEP_ROWS 2
#endif

// The state is read once and written once per step: both are non-temporal
// accesses (measured 36 -> 32.5 us per step at batch 256, d_inner 5120,
// d_state 16; either one alone gained nothing).
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_state(const float* p) {
    const f4v t = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void store_state(float* p, const float (&v)[4]) {
    const f4v t = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(t, reinterpret_cast<f4v*>(p));
}

// Lane l of a wave owns one quad (4 consecutive states) of the d_inner * G
// quads of a batch row -- a wave's 16-byte state moves are one contiguous
// 1 KiB access -- and applies the step to that quad in BR batch rows: A's
// quad is loaded once for all of them and the BR state loads are in flight
// together (BR = 2 measured best of 1, 2, 4 and 8 rows, 128/256/512-lane
// blocks).  A channel's G quads sit on G neighbouring lanes (G divides 64),
// which sum their partial readouts with shuffles.
// Sum of v over each aligned group of G lanes (G a power of two, <= 64),
// left in every lane of the group.  Within a 16-lane row the partners come
// through DPP (quad_perm for xor 1 and 2; row_half_mirror and row_mirror
// pair each lane with one of the other half once its half holds one value);
// wider groups use shuffles.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    auto dpp = [](float x, auto ctrl) {
        return __int_as_float(
            __builtin_amdgcn_mov_dpp(__float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, true));
    };
    if constexpr (G >= 2) v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm 1,0,3,2
    if constexpr (G >= 4) v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm 2,3,0,1
    if constexpr (G >= 8) v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
    if constexpr (G >= 16) v += dpp(v, std::integral_constant<int, 0x140>{}); // row_mirror
    if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// PAD: the true d_state Nr = a.N is below 4 G (G the next power of two of
// its quads).  States past Nr load as 0 (A, B, C and h), so they stay 0 and
// add nothing to the readout; they are never stored.  When Nr is a multiple
// of 4, rows stay 16-byte aligned and a quad is wholly in or out, so quads
// move as vectors; otherwise states move one float at a time.
template <int G, int BR, bool BF16, int DISC, bool PAD = false>
__global__ void __launch_bounds__(256) step_quads(StepArgs a) {
    constexpr int NG = 4 * G;
    const int N = PAD ? a.N : NG;
    const int quads = a.Dn * G;
    const int qi = blockIdx.x * blockDim.x + threadIdx.x;
    // Quads past the row's end are clamped to its last quad (so every
    // shuffle has its partners) and store nothing; so are rows past the batch.
    const bool qvalid = qi < quads;
    const int qc = qvalid ? qi : quads - 1;
    const int d = qc / G;  // G is a power of two: a shift
    const int j = qc & (G - 1);
    const int n0 = 4 * j;
    const int b0 = blockIdx.y * BR;

    // Every load is issued here, before any arithmetic, so that a wave waits
    // on memory once.
    auto ld4s = [&](auto ld1) __attribute__((always_inline)) {  // the quad's 4 states, past N read as 0
        return make_float4(n0 < N ? ld1(n0) : 0.f, n0 + 1 < N ? ld1(n0 + 1) : 0.f,
                           n0 + 2 < N ? ld1(n0 + 2) : 0.f, n0 + 3 < N ? ld1(n0 + 3) : 0.f);
    };
    const bool vec = !PAD || (N & 3) == 0;  // whole quads, 16-byte aligned rows
    const bool qin = n0 < N;                // (for vec) this quad holds states
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 av = zero4;
    if (!vec)
        av = ld4s([&](int n) __attribute__((always_inline)) { return a.A[(int64_t)d * N + n]; });
    else if (qin)
        av = *reinterpret_cast<const float4*>(a.A + (int64_t)d * N + n0);
    const float bias = a.bias ? a.bias[d] : 0.f;
    const float Dd = a.D ? a.D[d] : 0.f;
    float4 hv[BR], bv[BR], cv[BR];
    float xv[BR], dr[BR], zv[BR];
#pragma unroll
    for (int r = 0; r < BR; ++r) {
        const int b = min(b0 + r, a.batch - 1);
        const int64_t e = (int64_t)b * a.Dn + d;
        hv[r] = bv[r] = cv[r] = zero4;
        if (vec) {
            if (qin) {
                hv[r] = load_state(a.h + e * N + n0);
                bv[r] = ld4<BF16>(a.B, (int64_t)b * N + n0);
                cv[r] = ld4<BF16>(a.C, (int64_t)b * N + n0);
            }
        } else {
            hv[r] = ld4s([&](int n) __attribute__((always_inline)) { return a.h[e * N + n]; });
            bv[r] = ld4s([&](int n) __attribute__((always_inline)) { return ld<BF16>(a.B, (int64_t)b * N + n); });
            cv[r] = ld4s([&](int n) __attribute__((always_inline)) { return ld<BF16>(a.C, (int64_t)b * N + n); });
        }
        if constexpr (G >= 4) {
            // x, delta and z of the channel: each lane of a quad (its j mod 4)
            // loads one of them, and the quad shares them below -- one load
            // instruction where there were three.
            const int q = j & 3;
            const void* src = q == 0 ? a.x : (q == 1 ? a.delta : (a.z ? a.z : a.x));
            xv[r] = ld<BF16>(src, e);
        } else {
            xv[r] = ld<BF16>(a.x, e);
            dr[r] = ld<BF16>(a.delta, e);
            zv[r] = a.z ? ld<BF16>(a.z, e) : 0.f;
        }
    }
    if constexpr (G >= 4) {
        auto quad_bcast = [](float v, auto ctrl) {  // DPP quad_perm: lane k of each quad
            return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v),
                                                           decltype(ctrl)::value, 0xf, 0xf, true));
        };
#pragma unroll
        for (int r = 0; r < BR; ++r) {
            const float v = xv[r];
            dr[r] = quad_bcast(v, std::integral_constant<int, 0x55>{});
            zv[r] = a.z ? quad_bcast(v, std::integral_constant<int, 0xAA>{}) : 0.f;
            xv[r] = quad_bcast(v, std::integral_constant<int, 0x00>{});
        }
    }
    const float A2[4] = {av.x * kLog2e, av.y * kLog2e, av.z * kLog2e, av.w * kLog2e};
    const float an[4] = {av.x, av.y, av.z, av.w};

#pragma unroll
    for (int r = 0; r < BR; ++r) {
        const float dt = step_size(dr[r], bias, a.softplus);
        const float dx = dt * xv[r];
        float hs[4] = {hv[r].x, hv[r].y, hv[r].z, hv[r].w};
        const float bs[4] = {bv[r].x, bv[r].y, bv[r].z, bv[r].w};
        const float cs[4] = {cv[r].x, cv[r].y, cv[r].z, cv[r].w};
        float y = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float arg = dt * A2[k];
            float abar, bx;
            if constexpr (DISC == kBilinear) {
                const float rb = bilinear_r(arg);
                abar = fmaf(2.f, rb, -1.f);
                bx = (dx * rb) * bs[k];
            } else {
                abar = hw_exp2(arg);
                if constexpr (DISC == kZoh)
                    bx = zoh_factor(dt, arg, abar, an[k] != 0.f ? 1.f / an[k] : 0.f) *
                         (bs[k] * xv[r]);
                else
                    bx = dx * bs[k];
            }
            hs[k] = fmaf(abar, hs[k], bx);
            y = fmaf(cs[k], hs[k], y);
        }
        y = group_sum<G>(y);
        const int b = b0 + r;
        if (!qvalid || b >= a.batch) continue;
        const int64_t e = (int64_t)b * a.Dn + d;
        if (vec) {
            if (qin) store_state(a.h + e * N + n0, hs);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (n0 + k < N) a.h[e * N + n0 + k] = hs[k];
        }
        if (j == 0) {
            y = fmaf(Dd, xv[r], y);
            if (a.z) y *= silu_f(zv[r]);
            st<BF16>(a.y, e, y);
        }
    }
}

// G: the next power of two of the d_state's quads; PAD when it holds more.
inline int quad_groups(int n) {
    int g = 1;
    while (4 * g < n) g *= 2;
    return g;
}

template <int BR, bool BF16, int DISC, bool PAD>
hipError_t launch_g(const StepArgs& a, hipStream_t s) {
    const int G = quad_groups(a.N);
    const int64_t quads = (int64_t)a.Dn * G;
    const dim3 grid((unsigned)((quads + 255) / 256), (unsigned)((a.batch + BR - 1) / BR)),
        block(256);
    switch (G) {
        case 1: hipLaunchKernelGGL((step_quads<1, BR, BF16, DISC, PAD>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((step_quads<2, BR, BF16, DISC, PAD>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((step_quads<4, BR, BF16, DISC, PAD>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((step_quads<8, BR, BF16, DISC, PAD>), grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL((step_quads<16, BR, BF16, DISC, PAD>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((step_quads<32, BR, BF16, DISC, PAD>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool BF16, bool PAD>
hipError_t launch_p(const StepArgs& a, int disc, hipStream_t s) {
    switch (disc) {
        case kEuler: return launch_g<MSSCAN_STEP_ROWS, BF16, kEuler, PAD>(a, s);
        case kZoh: return launch_g<MSSCAN_STEP_ROWS, BF16, kZoh, PAD>(a, s);
        case kBilinear: return launch_g<MSSCAN_STEP_ROWS, BF16, kBilinear, PAD>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool step_quads_supported(int batch, int d_inner, int n) {
    (void)batch;  // batch rows go to grid.y (<= 65535, checked by the caller)
    if (n < 1 || n > 128) return false;
    return (int64_t)d_inner * quad_groups(n) < (1LL << 30);  // quad index of a row fits int
}

hipError_t launch_step_quads(const StepArgs& a, bool bf16, int disc, hipStream_t s) {
    if (!step_quads_supported(a.batch, a.Dn, a.N)) return hipErrorInvalidValue;
    ProfScope ps(s, kPhaseStep);
    const bool pad = 4 * quad_groups(a.N) != a.N;
    if (pad) return bf16 ? launch_p<true, true>(a, disc, s) : launch_p<false, true>(a, disc, s);
    return bf16 ? launch_p<true, false>(a, disc, s) : launch_p<false, false>(a, disc, s);
}

}  // namespace msscan
