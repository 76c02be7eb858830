// conv.hip -- causal depthwise conv1d (+ silu): the step that turns the x
// branch of the block input into the scan input u (lmnt.cn page, section
// 3.1: a depthwise 1D convolution of width about 4 ahead of the SSM; section
// 3.2: groups = d_inner, width-1 zeros of left padding, output cut to the
// first L steps, then silu):
//
//   u[b,t,d] = silu(bias[d] + sum_k w[d][k] * x[b, t-(W-1)+k, d])
//
// with x before t = 0 taken from x_prev (or zero).  The op moves 2 io values
// per element and does ~W+6 VALU ops, so it is HBM-bound.  A wave owns CH
// neighbouring channels per lane (64*CH channels: one 8-byte (bf16) or
// 16-byte (fp32) access per lane per timestep) and T consecutive timesteps;
// it walks them in order with the last W-1 inputs of each channel kept in
// registers, so every x is read once from HBM (plus W-1 halo rows per
// chunk, which the neighbouring chunk has just pulled into L2).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "dpp_common.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

#ifndef MSSCAN_CONV_T
#define MSSCAN_CONV_T 16
#endif
#ifndef MSSCAN_CONV_RB
#define MSSCAN_CONV_RB 4
#endif
constexpr int kConvT = MSSCAN_CONV_T;    // timesteps per wave
constexpr int kConvRB = MSSCAN_CONV_RB;  // rows loaded ahead

// CH io values at byte offset `off` of a buffer resource, widened to fp32.
template <int CH, bool BF16>
__device__ __forceinline__ void load_ch(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[CH]) {
    if constexpr (CH == 1) {
        v[0] = Io<BF16>::widen(Io<BF16>::load(r, off));
    } else if constexpr (BF16) {  // CH == 4: 8 bytes
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        const uint32_t lo = w[0], hi = w[1];
        v[0] = __uint_as_float(lo << 16);
        v[1] = __uint_as_float(lo & 0xffff0000u);
        v[2] = __uint_as_float(hi << 16);
        v[3] = __uint_as_float(hi & 0xffff0000u);
    } else {  // CH == 4: 16 bytes
        const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        v[0] = __uint_as_float(w[0]);
        v[1] = __uint_as_float(w[1]);
        v[2] = __uint_as_float(w[2]);
        v[3] = __uint_as_float(w[3]);
    }
}

// u is written once and not read back here: non-temporal stores (cache
// policy bit nt) measured 27.5 -> 21.7 us on the 130M-layer shape.  The
// loads stay cached: the W-1 halo rows of a chunk are read again by its
// neighbour.
constexpr int kStoreNt = 2;

template <int CH, bool BF16>
__device__ __forceinline__ void store_ch(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                         const float (&v)[CH]) {
    if constexpr (CH == 1) {
        Io<BF16>::store(r, off, v[0]);
    } else if constexpr (BF16) {
        auto bits = [](float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f); };
        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
        const u2 w = {bits(v[0]) | (bits(v[1]) << 16), bits(v[2]) | (bits(v[3]) << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, kStoreNt);
    } else {
        typedef uint32_t u4 __attribute__((ext_vector_type(4)));
        const u4 w = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, kStoreNt);
    }
}

#ifndef MSSCAN_CONV_WAVES
#define MSSCAN_CONV_WAVES 1
#endif
constexpr int kConvWaves = MSSCAN_CONV_WAVES;  // waves per workgroup, one time chunk each

template <int W, int CH, bool BF16, bool SILU>
__global__ void __launch_bounds__(64 * kConvWaves) conv1d_kernel(ConvArgs a) {
    constexpr int E = BF16 ? 2 : 4;
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.z;
    // time chunks on x (no limit on L): workgroup x holds kConvWaves of them
    const int64_t t0 = ((int64_t)blockIdx.x * kConvWaves + (threadIdx.x >> 6)) * kConvT;
    if (t0 >= a.L) return;  // a spare wave of the last workgroup: no rows, no history
    const int d0 = (blockIdx.y * 64 + lane) * CH;
    const bool dvalid = d0 < a.Dn;
    const int dd = dvalid ? d0 : 0;
    const uint32_t rowb = (uint32_t)a.Dn * E;
    const uint32_t off0 = dvalid ? (uint32_t)d0 * E : kOutOfRange;

    float w[CH][W], bias[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
        for (int k = 0; k < W; ++k) w[c][k] = a.w[(int64_t)min(dd + c, a.Dn - 1) * W + k];
        bias[c] = a.bias ? a.bias[min(dd + c, a.Dn - 1)] : 0.f;
    }

    // win[k][c]: x at t - (W-1) + k for k < W-1 (the history of the next step).
    float win[W > 1 ? W - 1 : 1][CH];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int64_t t = t0 - (W - 1) + k;
        float v[CH];
        if (t >= 0) {
            const auto r = make_rsrc(static_cast<const char*>(a.x) +
                                         ((int64_t)b * a.L + t) * (int64_t)rowb, rowb);
            load_ch<CH, BF16>(r, off0, v);
        } else if (a.x_prev) {
            const auto r = make_rsrc(static_cast<const char*>(a.x_prev) +
                                         ((int64_t)b * (W - 1) + (W - 1) + t) * (int64_t)rowb,
                                     rowb);
            load_ch<CH, BF16>(r, off0, v);
        } else {
#pragma unroll
            for (int c = 0; c < CH; ++c) v[c] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) win[k][c] = v[c];
    }

    const int64_t t1 = min(a.L, t0 + kConvT);
#pragma unroll 1
    for (int64_t tb = t0; tb < t1; tb += kConvRB) {
        const uint32_t nr = (uint32_t)min((int64_t)kConvRB, t1 - tb);
        const auto rx = make_rsrc(static_cast<const char*>(a.x) +
                                      ((int64_t)b * a.L + tb) * (int64_t)rowb, nr * rowb);
        const auto ru = make_rsrc(static_cast<char*>(a.u) +
                                      ((int64_t)b * a.L + tb) * (int64_t)rowb, nr * rowb);
        float xr[kConvRB][CH];
#pragma unroll
        for (int i = 0; i < kConvRB; ++i) load_ch<CH, BF16>(rx, off0 + (uint32_t)i * rowb, xr[i]);
#pragma unroll
        for (int i = 0; i < kConvRB; ++i) {
            float out[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                float pre = fmaf(w[c][W - 1], xr[i][c], bias[c]);
#pragma unroll
                for (int k = 0; k < W - 1; ++k) pre = fmaf(w[c][k], win[k][c], pre);
                out[c] = SILU ? silu_f(pre) : pre;
#pragma unroll
                for (int k = 0; k + 1 < W - 1; ++k) win[k][c] = win[k + 1][c];
                if constexpr (W > 1) win[W - 2][c] = xr[i][c];
            }
            store_ch<CH, BF16>(ru, off0 + (uint32_t)i * rowb, out);  // rows past L: dropped
        }
    }
}

template <int CH, bool BF16, bool SILU>
hipError_t launch_w(const ConvArgs& a, dim3 grid, hipStream_t s) {
    switch (a.width) {
#define MS_CONV_W_(W) \
    case W:                                                                             \
        hipLaunchKernelGGL((conv1d_kernel<W, CH, BF16, SILU>), grid, dim3(64 * kConvWaves), 0, s, a); \
        break;
        MS_CONV_W_(1) MS_CONV_W_(2) MS_CONV_W_(3) MS_CONV_W_(4)
        MS_CONV_W_(5) MS_CONV_W_(6) MS_CONV_W_(7) MS_CONV_W_(8)
#undef MS_CONV_W_
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int CH>
hipError_t launch_ch(const ConvArgs& a, bool bf16, bool silu, hipStream_t s) {
    const int64_t chunks = (a.L + kConvT - 1) / kConvT;
    const dim3 grid((unsigned)((chunks + kConvWaves - 1) / kConvWaves),
                    (unsigned)((a.Dn + 64 * CH - 1) / (64 * CH)), (unsigned)a.batch);
    if (bf16) return silu ? launch_w<CH, true, true>(a, grid, s) : launch_w<CH, true, false>(a, grid, s);
    return silu ? launch_w<CH, false, true>(a, grid, s) : launch_w<CH, false, false>(a, grid, s);
}

}  // namespace

hipError_t launch_conv1d(const ConvArgs& a, bool bf16, bool silu, hipStream_t s) {
    ProfScope ps(s, kPhaseConv);
    // Four channels per lane need rows whose byte size keeps 8/16-byte
    // accesses aligned: d_inner a multiple of 4.
    return (a.Dn % 4 == 0) ? launch_ch<4>(a, bf16, silu, s) : launch_ch<1>(a, bf16, silu, s);
}

}  // namespace msscan
