// device_common.h -- inline device helpers shared by the HIP kernels of
// libmsscan: bf16 io, the per-element activations (softplus, silu) and the
// zero-order-hold input factor.  Included only by .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msscan {
namespace dev {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---- io -------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    if constexpr (BF16)
        return __uint_as_float((uint32_t)(static_cast<const uint16_t*>(p)[i]) << 16);
    else
        return static_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void st(void* p, int64_t i, float v) {
    if constexpr (BF16)
        static_cast<uint16_t*>(p)[i] = f32_to_bf16_rne(v);
    else
        static_cast<float*>(p)[i] = v;
}

// ---- per-element activations ------------------------------------------------
// softplus(v) = log(1 + e^v) with the hardware base-2 exp/log:
// ln2 * log2(1 + 2^(v*log2 e)).  The exponent is clamped at 64 so 2^x stays
// finite; for v > 44 the result is v itself to fp32 precision, and max(v, .)
// returns it.  The rounding of 1 + w bounds the absolute error by about
// 2^-24 * ln2, which is what the step size needs (it scales B*u and the
// exponent dt*A).
__device__ __forceinline__ float softplus_f(float v) {
    const float w = hw_exp2(fminf(v * kLog2e, 64.f));
    return fmaxf(v, hw_log2(1.f + w) * kLn2);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu_f(float z) {
    return z * hw_rcp(1.f + hw_exp2(-z * kLog2e));
}

__device__ __forceinline__ float step_size(float draw, float bias, int softplus) {
    float v = draw + bias;
    return softplus ? softplus_f(v) : v;
}

// ZOH input factor expm1(x)/A with x = dt*A.  For |x| < 1/16 the series
// dt*(1 + x/2 + x^2/6 + x^3/24 + x^4/120) (relative error < 2e-9) avoids the
// cancellation of exp(x) - 1; it is also the A == 0 limit dt.  Otherwise
// (abar - 1) * (1/A), where abar = exp(x) is already computed.
__device__ __forceinline__ float zoh_factor(float dt, float x, float abar, float invA) {
    float ser = dt * (1.f + x * (0.5f + x * (1.f / 6.f + x * (1.f / 24.f + x * (1.f / 120.f)))));
    float big = (abar - 1.f) * invA;
    return fabsf(x) < 0.0625f ? ser : big;
}

}  // namespace dev
}  // namespace msscan
