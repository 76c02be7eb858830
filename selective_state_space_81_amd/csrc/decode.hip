// decode.hip -- one recurrent decode step (ms_state_update) for d_state a
// multiple of 4, up to 128.
//
// The step is one timestep of the scan with the state kept in HBM between
// calls (lmnt.cn page, section 5.3; the state cache of the jsqmd page,
// section 5.3): per (b, d) read x_t, delta_t, z_t, per n read and rewrite
// h[b, d, n].  Its bytes are dominated by the fp32 state (read and written
// once per step), so the kernel is laid out for that stream: lane g of a
// channel owns states 4g .. 4g+3 and moves them as one 16-byte load and one
// 16-byte store, so a wave covers 1 KiB of consecutive state.  The G = N/4
// lanes of a channel sit in one wave (G divides 64) and sum their partial
// readouts with cross-lane shuffles; the per-element work (softplus, gate) is
// repeated by each of them, which costs little next to the state traffic.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

template <int G, bool BF16, bool ZOH>
__global__ void __launch_bounds__(256) step_quads(StepArgs a) {
    constexpr int N = 4 * G;
    const int64_t total = (int64_t)a.batch * a.Dn * G;
    const int64_t gl = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // Lanes past the end stay alive (clamped to the last lane) so that every
    // shuffle has all its partners; they store nothing.
    const bool valid = gl < total;
    const int64_t gc = valid ? gl : total - 1;
    const int q = (int)(gc % G);
    const int64_t e = gc / G;  // b * Dn + d
    const int d = (int)(e % a.Dn);
    const int b = (int)(e / a.Dn);

    const float xv = ld<BF16>(a.x, e);
    const float dt = step_size(ld<BF16>(a.delta, e), a.bias ? a.bias[d] : 0.f, a.softplus);
    const float dx = dt * xv;
    float* hp = a.h + e * N + 4 * q;
    float4 hv = *reinterpret_cast<const float4*>(hp);
    const float4 av = *reinterpret_cast<const float4*>(a.A + (int64_t)d * N + 4 * q);
    const float4 bv = ld4<BF16>(a.B, (int64_t)b * N + 4 * q);
    const float4 cv = ld4<BF16>(a.C, (int64_t)b * N + 4 * q);

    auto one = [&](float an, float bn, float cn, float& h, float& y) {
        const float arg = dt * (an * kLog2e);
        const float abar = hw_exp2(arg);
        float bx;
        if constexpr (ZOH)
            bx = zoh_factor(dt, arg, abar, an != 0.f ? 1.f / an : 0.f) * (bn * xv);
        else
            bx = dx * bn;
        h = fmaf(abar, h, bx);
        y = fmaf(cn, h, y);
    };
    float y = 0.f;
    one(av.x, bv.x, cv.x, hv.x, y);
    one(av.y, bv.y, cv.y, hv.y, y);
    one(av.z, bv.z, cv.z, hv.z, y);
    one(av.w, bv.w, cv.w, hv.w, y);
#pragma unroll
    for (int off = G / 2; off >= 1; off /= 2) y += __shfl_xor(y, off, 64);

    if (!valid) return;
    *reinterpret_cast<float4*>(hp) = hv;
    if (q == 0) {
        y = fmaf(a.D ? a.D[d] : 0.f, xv, y);
        if (a.z) y *= silu_f(ld<BF16>(a.z, e));
        st<BF16>(a.y, e, y);
    }
}

template <bool BF16, bool ZOH>
hipError_t launch_g(const StepArgs& a, hipStream_t s) {
    const int G = a.N / 4;
    const int64_t lanes = (int64_t)a.batch * a.Dn * G;
    const dim3 grid((unsigned)((lanes + 255) / 256)), block(256);
    switch (G) {
        case 1: hipLaunchKernelGGL((step_quads<1, BF16, ZOH>), grid, block, 0, s, a); break;
        case 2: hipLaunchKernelGGL((step_quads<2, BF16, ZOH>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((step_quads<4, BF16, ZOH>), grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL((step_quads<8, BF16, ZOH>), grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL((step_quads<16, BF16, ZOH>), grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL((step_quads<32, BF16, ZOH>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool step_quads_supported(int batch, int d_inner, int n) {
    if (n % 4 != 0 || n < 4 || n > 128 || ((n / 4) & (n / 4 - 1)) != 0) return false;
    return (int64_t)batch * d_inner * (n / 4) / 256 < 0x7fffffffLL;  // grid.x limit
}

hipError_t launch_step_quads(const StepArgs& a, bool bf16, bool zoh, hipStream_t s) {
    if (!step_quads_supported(a.batch, a.Dn, a.N)) return hipErrorInvalidValue;
    ProfScope ps(s, kPhaseStep);
    if (bf16) return zoh ? launch_g<true, true>(a, s) : launch_g<true, false>(a, s);
    return zoh ? launch_g<false, true>(a, s) : launch_g<false, false>(a, s);
}

}  // namespace msscan
