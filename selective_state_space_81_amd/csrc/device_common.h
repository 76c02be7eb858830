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
// fp32 -> bf16 rounded to nearest even: the hardware conversion
// (v_cvt_pk_bf16_f32 on gfx950; NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
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

// Discretisations (ms_scan_fwd flags): Euler (A_bar = exp(dt A), B_bar =
// dt B), zero-order hold (B_bar = (exp(dt A) - 1)/A B) and bilinear
// (A_bar = (1 + dt A/2)/(1 - dt A/2), B_bar = dt/(1 - dt A/2) B).
enum : int { kEuler = 0, kZoh = 1, kBilinear = 2 };

// Bilinear factor r = 1/(1 - dt*A/2) from t = dt*A*log2(e) (the argument the
// other discretisations feed to exp2): A_bar = 2r - 1 and B_bar = dt*r*B.
__device__ __forceinline__ float bilinear_r(float t) {
    return hw_rcp(fmaf(t, -0.5f * kLn2, 1.f));
}

// ZOH input factor (exp(x) - 1)/A for x = dt*A, from t = x*log2(e) (the
// argument already formed for abar = 2^t).  For |x| < 1/32 the series
// dt*(1 + x/2 + x^2/6), written in t, avoids the cancellation of exp(x) - 1
// (truncation < 1.3e-6 relative) and is the A == 0 limit dt.  Otherwise
// abar*(1/A) - 1/A as one fma: only the rounding of abar is left, < 2e-6
// relative at the switch point.
constexpr float kZohT1 = 0.34657359027997264f;  // ln2 / 2
constexpr float kZohT2 = 0.08007550231970023f;  // ln2^2 / 6
constexpr float kZohSwitch = 0.045084220027780106f;  // (1/32) / ln2
// dB_bar/dA's series near A = 0, dt^2 (1/2 + x/3 + x^2/8) with x = t ln2:
// the coefficients of t and t^2
constexpr float kZohD1 = 0.23104906018664842f;  // ln2 / 3
constexpr float kZohD2 = 0.06005662673977517f;  // ln2^2 / 8
__device__ __forceinline__ float zoh_factor(float dt, float t, float abar, float invA) {
    const float ser = dt * fmaf(t, fmaf(t, kZohT2, kZohT1), 1.f);
    const float big = fmaf(abar, invA, -invA);
    return fabsf(t) < kZohSwitch ? ser : big;
}

// The same factor with the series expanded in powers of dt, for kernels that
// evaluate many states per dt:  dt + (c1 dt^2) a + (c2 dt^3) a^2  with
// a = A*log2(e), q1 = c1*dt^2 and q2 = c2*dt^3 formed once per timestep and
// a^2 once per channel (two fma per state instead of three operations).
__device__ __forceinline__ float zoh_factor_q(float dt, float q1, float q2, float a, float a_sq,
                                              float t, float abar, float invA) {
    const float ser = fmaf(q2, a_sq, fmaf(q1, a, dt));
    const float big = fmaf(abar, invA, -invA);
    return fabsf(t) < kZohSwitch ? ser : big;
}

// Workgroup id -> logical workgroup: XCD x (= id mod 8, the order in which
// the hardware deals workgroups to the 8 XCDs) gets a contiguous range of
// logical indices, in order, so that neighbouring logical workgroups share an
// L2.  A bijection on [0, G) for any G.
__device__ __forceinline__ uint32_t xcd_logical(uint32_t bid, uint32_t G) {
    const uint32_t q = G >> 3, rem = G & 7u, x = bid & 7u, i = bid >> 3;
    return x * q + (x < rem ? x : rem) + i;
}

}  // namespace dev
}  // namespace msscan
