// bwd_wide.hip -- helper kernels of ms_scan_bwd for d_state 17..128.
//
// The backward kernels of scan_bwd.hip hold up to 16 states of a channel in
// one lane.  A wider state is differentiated in slices of 16 states: the
// recurrence is diagonal, so every state's adjoint lambda_t[n] = C_t[n] g_t +
// A_bar_{t+1}[n] lambda_{t+1}[n] involves its own state only, and the
// per-element gradients (du, ddelta before the softplus factor, which is a
// common factor) are sums over states, i.e. sums over slices.  Each slice is
// run as a 16-state fp32 problem with the gate and D taken out:
//   g = dy * silu(z)                 (dL/dy_pre, the slices' output gradient)
//   du     = sum_s du_s + g * D
//   ddelta = sum_s ddelta_s          (each already through the softplus)
//   dz     = dy * y_pre * sigma(z) * (1 + z (1 - sigma(z))),
//            y_pre = sum_n C h + D u: each slice's gradient pass adds its
//            states' sum_n C h from the states it recomputes (segment
//            layout; the combine adds D u), or, for row-layout slices, an
//            fp32 forward pass forms it
//   dD     = sum over batch and time of g * u
// while dA, dB, dC and dh0 are the slices' own, and dbias the slices' sum.
// The slices are added in order, so the result is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

__device__ __forceinline__ float sigmoid_f(float z) { return hw_rcp(1.f + hw_exp2(-z * kLog2e)); }

// g = dy * silu(z) (or dy), and fp32 copies of u and delta (bf16 io).
template <bool BF16>
__global__ void __launch_bounds__(256) wide_prep(WideArgs w) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < w.E; e += stride) {
        const float dy = ld<BF16>(w.dy, e);
        w.g[e] = w.z ? dy * silu_f(ld<BF16>(w.z, e)) : dy;
        if constexpr (BF16) {
            w.u32[e] = ld<true>(w.u, e);
            w.d32[e] = ld<true>(w.delta, e);
        }
    }
}

// fp32 copies of B and C (bf16 io), for the fp32 forward pass (row-layout
// slices).
__global__ void __launch_bounds__(256) wide_bc32(WideArgs w) {
    const int64_t n = w.BLN;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        w.B32[i] = ld<true>(w.B, i);
        w.C32[i] = ld<true>(w.C, i);
    }
}

// The inputs of slice n0 (states n0 .. n0+15, zero past d_state): A_s [Dn][16],
// B_s, C_s [batch][L][16] fp32, h0_s, dhl_s [batch][Dn][16].
template <bool BF16>
__global__ void __launch_bounds__(256) wide_gather(WideArgs w, int n0) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int N = w.N;
    for (int64_t i = i0; i < w.BL * kWideSlice; i += stride) {
        const int j = (int)(i % kWideSlice);
        const int64_t r = i / kWideSlice;
        const bool ok = n0 + j < N;
        w.Bs[i] = ok ? ld<BF16>(w.B, r * N + n0 + j) : 0.f;
        w.Cs[i] = ok ? ld<BF16>(w.C, r * N + n0 + j) : 0.f;
    }
    for (int64_t i = i0; i < (int64_t)w.Dn * kWideSlice; i += stride) {
        const int j = (int)(i % kWideSlice);
        const int64_t d = i / kWideSlice;
        w.As[i] = n0 + j < N ? w.A[d * N + n0 + j] : 0.f;
    }
    for (int64_t i = i0; i < w.BD * kWideSlice; i += stride) {
        const int j = (int)(i % kWideSlice);
        const int64_t r = i / kWideSlice;
        const bool ok = n0 + j < N;
        if (w.h0s) w.h0s[i] = (ok && w.h0) ? w.h0[r * N + n0 + j] : 0.f;
        if (w.dhls) w.dhls[i] = (ok && w.dh_last) ? w.dh_last[r * N + n0 + j] : 0.f;
    }
}

// Slice n0's results into the totals: du / ddelta partials added when the
// slice wrote them apart (add_du; otherwise its gradient pass wrote or added
// them into the totals itself), dbias added (first slice: copied), dA, dB,
// dC and dh0 scattered to their states.
__global__ void __launch_bounds__(256) wide_accumulate(WideArgs w, int n0, int add_du) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool first = n0 == 0;
    const int N = w.N;
    if (add_du) {
        for (int64_t e = i0; e < w.E; e += stride) {
            w.du_acc[e] += w.du_s[e];
            w.dv_acc[e] += w.dv_s[e];
        }
    }
    for (int64_t i = i0; i < w.BL * kWideSlice; i += stride) {
        const int j = (int)(i % kWideSlice);
        if (n0 + j >= N) continue;
        const int64_t r = i / kWideSlice;
        w.dB[r * N + n0 + j] = w.dBs[i];
        w.dC[r * N + n0 + j] = w.dCs[i];
    }
    for (int64_t i = i0; i < (int64_t)w.Dn * kWideSlice; i += stride) {
        const int j = (int)(i % kWideSlice);
        if (n0 + j >= N) continue;
        w.dA[(i / kWideSlice) * N + n0 + j] = w.dAs[i];
    }
    if (w.dh0) {
        for (int64_t i = i0; i < w.BD * kWideSlice; i += stride) {
            const int j = (int)(i % kWideSlice);
            if (n0 + j >= N) continue;
            w.dh0[(i / kWideSlice) * N + n0 + j] = w.dh0s[i];
        }
    }
    for (int64_t d = i0; d < w.Dn; d += stride)
        w.dbias_acc[d] = first ? w.dbias_s[d] : w.dbias_acc[d] + w.dbias_s[d];
}

// du = sum_s du_s + g D, ddelta = sum_s ddelta_s, dz from y_pre; io stores.
template <bool BF16>
__global__ void __launch_bounds__(256) wide_combine(WideArgs w) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < w.E; e += stride) {
        const int64_t d = e % w.Dn;
        const float g = w.g[e];
        st<BF16>(w.du, e, w.D ? fmaf(g, w.D[d], w.du_acc[e]) : w.du_acc[e]);
        st<BF16>(w.ddelta, e, w.dv_acc[e]);
        if (w.z) {
            const float zv = ld<BF16>(w.z, e);
            const float sg = sigmoid_f(zv);
            float ypre = w.y32[e];
            if (w.y32_add_du && w.D) ypre = fmaf(w.D[d], ld<BF16>(w.u, e), ypre);
            st<BF16>(w.dz, e, ld<BF16>(w.dy, e) * ypre * sg * fmaf(zv, 1.f - sg, 1.f));
        }
    }
}

// dD[d] = sum over batch and time of g * u: kWideGroups partial sums per
// channel over consecutive row ranges (rows in order, four independent
// accumulators added in a fixed order), then the groups added in order.
template <bool BF16>
__global__ void __launch_bounds__(256) wide_dD_part(WideArgs w) {
    const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= w.Dn || !w.dD) return;
    const int64_t per = (w.BL + kWideGroups - 1) / kWideGroups;
    const int64_t r0 = blockIdx.y * per, r1 = min(w.BL, r0 + per);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t r = r0;
    for (; r + 3 < r1; r += 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t e = (r + k) * w.Dn + d;
            acc[k] = fmaf(w.g[e], ld<BF16>(w.u, e), acc[k]);
        }
    }
    for (; r < r1; ++r) acc[0] = fmaf(w.g[r * w.Dn + d], ld<BF16>(w.u, r * w.Dn + d), acc[0]);
    w.dD_part[(int64_t)blockIdx.y * w.Dn + d] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

__global__ void __launch_bounds__(256) wide_dD_sum(WideArgs w) {
    const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (d >= w.Dn) return;
    if (w.dD) {
        float acc = 0.f;
        for (int gi = 0; gi < kWideGroups; ++gi) acc += w.dD_part[(int64_t)gi * w.Dn + d];
        w.dD[d] = acc;
    }
    if (w.dbias) w.dbias[d] = w.dbias_acc[d];
}

unsigned grid_of(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 16384 ? (b < 1 ? 1 : b) : 16384);
}

}  // namespace

hipError_t launch_wide_prep(const WideArgs& w, bool bf16, hipStream_t s) {
    ProfScope ps(s, kPhasePrep);
    if (bf16) {
        hipLaunchKernelGGL(wide_prep<true>, dim3(grid_of(w.E)), dim3(256), 0, s, w);
        hipLaunchKernelGGL(wide_bc32, dim3(grid_of(w.BLN)), dim3(256), 0, s, w);
    } else {
        hipLaunchKernelGGL(wide_prep<false>, dim3(grid_of(w.E)), dim3(256), 0, s, w);
    }
    return hipGetLastError();
}

hipError_t launch_wide_gather(const WideArgs& w, int n0, bool bf16, hipStream_t s) {
    ProfScope ps(s, kPhasePrep);
    const int64_t n = w.BL * kWideSlice;
    if (bf16)
        hipLaunchKernelGGL(wide_gather<true>, dim3(grid_of(n)), dim3(256), 0, s, w, n0);
    else
        hipLaunchKernelGGL(wide_gather<false>, dim3(grid_of(n)), dim3(256), 0, s, w, n0);
    return hipGetLastError();
}

hipError_t launch_wide_accumulate(const WideArgs& w, int n0, bool add_du, hipStream_t s) {
    ProfScope ps(s, kPhaseReduce);
    const int64_t n = add_du ? w.E : max(w.BL, w.BD) * kWideSlice;
    hipLaunchKernelGGL(wide_accumulate, dim3(grid_of(n)), dim3(256), 0, s, w, n0, add_du ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_wide_finish(const WideArgs& w, bool bf16, hipStream_t s) {
    ProfScope ps(s, kPhaseReduce);
    const unsigned gd = (unsigned)((w.Dn + 255) / 256);
    if (bf16) {
        hipLaunchKernelGGL(wide_combine<true>, dim3(grid_of(w.E)), dim3(256), 0, s, w);
        hipLaunchKernelGGL(wide_dD_part<true>, dim3(gd, kWideGroups), dim3(256), 0, s, w);
    } else {
        hipLaunchKernelGGL(wide_combine<false>, dim3(grid_of(w.E)), dim3(256), 0, s, w);
        hipLaunchKernelGGL(wide_dD_part<false>, dim3(gd, kWideGroups), dim3(256), 0, s, w);
    }
    hipLaunchKernelGGL(wide_dD_sum, dim3(gd), dim3(256), 0, s, w);
    return hipGetLastError();
}

}  // namespace msscan
