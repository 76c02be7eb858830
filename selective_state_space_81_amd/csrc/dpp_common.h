// dpp_common.h -- shared device pieces of the fast scan kernels: bounded
// buffer-resource io, the DPP row broadcast of B_t / C_t values, and the
// partial readout sum_n C_n * h_n with C_n delivered through DPP.
// Included only by .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace msscan {
namespace dev {

// Buffer-resource io.  A block's rows of u / delta / z / y (and of the
// prepared B/C rows) are addressed through a buffer descriptor whose size
// ends at the block's last valid row, so reads past it return 0 and writes
// past it are dropped by the hardware; tail channels get an offset beyond any
// size.  No branch is needed for ragged sequence ends or d_inner tails.
constexpr uint32_t kBufFlags = 0x00020000u;  // raw (untyped) access, gfx9 family
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kBufFlags);
}

template <bool BF16>
struct Io {
    static constexpr int kSize = BF16 ? 2 : 4;
    using T = typename std::conditional<BF16, uint16_t, float>::type;
    static __device__ __forceinline__ T load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        if constexpr (BF16)
            return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        else
            return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
    static __device__ __forceinline__ float widen(T v) {
        if constexpr (BF16)
            return __uint_as_float((uint32_t)v << 16);
        else
            return v;
    }
    // Round to the io type (bf16: hardware round-to-nearest-even) and store.
    static __device__ __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
        if constexpr (BF16)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v), r, off,
                                                  0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
    }
};

// DPP row_newbcast:n (gfx90a and later): every lane reads lane n of its own
// 16-lane row.  The compiler folds this move into the consuming VOP2
// instruction (v_mul_f32_dpp), so the broadcast costs nothing.
template <int n>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + n, 0xf, 0xf, true));
}

// Partial readout y = sum_j C[n0 + j] * h[j], with C[n0 + j] delivered by
// row_newbcast:j from vc.  Written as one asm block of v_mul/v_fmac with DPP
// sources because the compiler does not fold DPP moves into v_fmac.  The
// leading s_nop 1 provides the two wait states the hardware requires between
// a VALU write of vc and its read through DPP (the register allocator may
// place a copy of vc right before the block).
#define MS_DPP_(op, n, hop) op " %0, %1, " hop " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n"
template <int NS>
struct DppReadout;
template <>
struct DppReadout<2> {
    static __device__ __forceinline__ float run(float vc, const float (&h)[2]) {
        float y;
        asm("s_nop 1\n" MS_DPP_("v_mul_f32_dpp", 0, "%2") MS_DPP_("v_fmac_f32_dpp", 1, "%3")
            : "=&v"(y) : "v"(vc), "v"(h[0]), "v"(h[1]));
        return y;
    }
};
template <>
struct DppReadout<4> {
    static __device__ __forceinline__ float run(float vc, const float (&h)[4]) {
        float y;
        asm("s_nop 1\n" MS_DPP_("v_mul_f32_dpp", 0, "%2") MS_DPP_("v_fmac_f32_dpp", 1, "%3")
                MS_DPP_("v_fmac_f32_dpp", 2, "%4") MS_DPP_("v_fmac_f32_dpp", 3, "%5")
            : "=&v"(y) : "v"(vc), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]));
        return y;
    }
};
template <>
struct DppReadout<8> {
    static __device__ __forceinline__ float run(float vc, const float (&h)[8]) {
        float y;
        asm("s_nop 1\n" MS_DPP_("v_mul_f32_dpp", 0, "%2") MS_DPP_("v_fmac_f32_dpp", 1, "%3")
                MS_DPP_("v_fmac_f32_dpp", 2, "%4") MS_DPP_("v_fmac_f32_dpp", 3, "%5")
                    MS_DPP_("v_fmac_f32_dpp", 4, "%6") MS_DPP_("v_fmac_f32_dpp", 5, "%7")
                        MS_DPP_("v_fmac_f32_dpp", 6, "%8") MS_DPP_("v_fmac_f32_dpp", 7, "%9")
            : "=&v"(y)
            : "v"(vc), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]),
              "v"(h[6]), "v"(h[7]));
        return y;
    }
};
template <>
struct DppReadout<16> {
    static __device__ __forceinline__ float run(float vc, const float (&h)[16]) {
        float y;
        asm("s_nop 1\n" MS_DPP_("v_mul_f32_dpp", 0, "%2") MS_DPP_("v_fmac_f32_dpp", 1, "%3")
                MS_DPP_("v_fmac_f32_dpp", 2, "%4") MS_DPP_("v_fmac_f32_dpp", 3, "%5")
                    MS_DPP_("v_fmac_f32_dpp", 4, "%6") MS_DPP_("v_fmac_f32_dpp", 5, "%7")
                        MS_DPP_("v_fmac_f32_dpp", 6, "%8") MS_DPP_("v_fmac_f32_dpp", 7, "%9")
                            MS_DPP_("v_fmac_f32_dpp", 8, "%10") MS_DPP_("v_fmac_f32_dpp", 9, "%11")
                                MS_DPP_("v_fmac_f32_dpp", 10, "%12")
                                    MS_DPP_("v_fmac_f32_dpp", 11, "%13")
                                        MS_DPP_("v_fmac_f32_dpp", 12, "%14")
                                            MS_DPP_("v_fmac_f32_dpp", 13, "%15")
                                                MS_DPP_("v_fmac_f32_dpp", 14, "%16")
                                                    MS_DPP_("v_fmac_f32_dpp", 15, "%17")
            : "=&v"(y)
            : "v"(vc), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]),
              "v"(h[6]), "v"(h[7]), "v"(h[8]), "v"(h[9]), "v"(h[10]), "v"(h[11]), "v"(h[12]),
              "v"(h[13]), "v"(h[14]), "v"(h[15]));
        return y;
    }
};
// y + sum_j C[n0 + j] * h[j] for 16 states: the continuation of a readout
// chain for the second and later groups of 16 states of a lane.
struct DppReadoutAcc16 {
    static __device__ __forceinline__ float run(float y, float vc, const float* h) {
        asm("s_nop 1\n" MS_DPP_("v_fmac_f32_dpp", 0, "%2") MS_DPP_("v_fmac_f32_dpp", 1, "%3")
                MS_DPP_("v_fmac_f32_dpp", 2, "%4") MS_DPP_("v_fmac_f32_dpp", 3, "%5")
                    MS_DPP_("v_fmac_f32_dpp", 4, "%6") MS_DPP_("v_fmac_f32_dpp", 5, "%7")
                        MS_DPP_("v_fmac_f32_dpp", 6, "%8") MS_DPP_("v_fmac_f32_dpp", 7, "%9")
                            MS_DPP_("v_fmac_f32_dpp", 8, "%10") MS_DPP_("v_fmac_f32_dpp", 9, "%11")
                                MS_DPP_("v_fmac_f32_dpp", 10, "%12")
                                    MS_DPP_("v_fmac_f32_dpp", 11, "%13")
                                        MS_DPP_("v_fmac_f32_dpp", 12, "%14")
                                            MS_DPP_("v_fmac_f32_dpp", 13, "%15")
                                                MS_DPP_("v_fmac_f32_dpp", 14, "%16")
                                                    MS_DPP_("v_fmac_f32_dpp", 15, "%17")
            : "+&v"(y)
            : "v"(vc), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]),
              "v"(h[6]), "v"(h[7]), "v"(h[8]), "v"(h[9]), "v"(h[10]), "v"(h[11]), "v"(h[12]),
              "v"(h[13]), "v"(h[14]), "v"(h[15]));
        return y;
    }
};
#undef MS_DPP_

// The compiler folds a DPP move into v_mul but not into v_fma / v_fmac, so
// fmaf(row_bcast<n>(v), x, acc) costs a separate v_mov_b32_dpp.  The two
// helpers below issue v_fmac_f32_dpp with the broadcast operand directly (one
// instruction per state; same single rounding as fmaf), for the first NS
// states (NS = 4, 8 or 16, lane n of each row holding state n of v).
//   dpp_axpy: acc[n] += v_n * x for every n (in place)
//   dpp_dot:  y + sum_n v_n * h[n], accumulated in order n = 0, 1, ...
#define MS_AX_(n) "v_fmac_f32_dpp %" #n ", %[v], %[x] row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n"
#define MS_DT_(n, k) "v_fmac_f32_dpp %[y], %[v], %" #k " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n"
template <int NS>
__device__ __forceinline__ void dpp_axpy(float (&acc)[NS], float v, float x);
template <>
__device__ __forceinline__ void dpp_axpy<4>(float (&a)[4], float v, float x) {
    asm("s_nop 1\n" MS_AX_(0) MS_AX_(1) MS_AX_(2) MS_AX_(3)
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])
        : [v] "v"(v), [x] "v"(x));
}
template <>
__device__ __forceinline__ void dpp_axpy<8>(float (&a)[8], float v, float x) {
    asm("s_nop 1\n" MS_AX_(0) MS_AX_(1) MS_AX_(2) MS_AX_(3) MS_AX_(4) MS_AX_(5) MS_AX_(6)
            MS_AX_(7)
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
          "+v"(a[7])
        : [v] "v"(v), [x] "v"(x));
}
template <>
__device__ __forceinline__ void dpp_axpy<16>(float (&a)[16], float v, float x) {
    asm("s_nop 1\n" MS_AX_(0) MS_AX_(1) MS_AX_(2) MS_AX_(3) MS_AX_(4) MS_AX_(5) MS_AX_(6)
            MS_AX_(7) MS_AX_(8) MS_AX_(9) MS_AX_(10) MS_AX_(11) MS_AX_(12) MS_AX_(13) MS_AX_(14)
                MS_AX_(15)
        : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
          "+v"(a[7]), "+v"(a[8]), "+v"(a[9]), "+v"(a[10]), "+v"(a[11]), "+v"(a[12]),
          "+v"(a[13]), "+v"(a[14]), "+v"(a[15])
        : [v] "v"(v), [x] "v"(x));
}
template <int NS>
__device__ __forceinline__ float dpp_dot(float y, float v, const float (&h)[NS]);
template <>
__device__ __forceinline__ float dpp_dot<4>(float y, float v, const float (&h)[4]) {
    asm("s_nop 1\n" MS_DT_(0, 2) MS_DT_(1, 3) MS_DT_(2, 4) MS_DT_(3, 5)
        : [y] "+v"(y)
        : [v] "v"(v), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]));
    return y;
}
template <>
__device__ __forceinline__ float dpp_dot<8>(float y, float v, const float (&h)[8]) {
    asm("s_nop 1\n" MS_DT_(0, 2) MS_DT_(1, 3) MS_DT_(2, 4) MS_DT_(3, 5) MS_DT_(4, 6)
            MS_DT_(5, 7) MS_DT_(6, 8) MS_DT_(7, 9)
        : [y] "+v"(y)
        : [v] "v"(v), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]),
          "v"(h[6]), "v"(h[7]));
    return y;
}
template <>
__device__ __forceinline__ float dpp_dot<16>(float y, float v, const float (&h)[16]) {
    asm("s_nop 1\n" MS_DT_(0, 2) MS_DT_(1, 3) MS_DT_(2, 4) MS_DT_(3, 5) MS_DT_(4, 6)
            MS_DT_(5, 7) MS_DT_(6, 8) MS_DT_(7, 9) MS_DT_(8, 10) MS_DT_(9, 11) MS_DT_(10, 12)
                MS_DT_(11, 13) MS_DT_(12, 14) MS_DT_(13, 15) MS_DT_(14, 16) MS_DT_(15, 17)
        : [y] "+v"(y)
        : [v] "v"(v), "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "v"(h[4]), "v"(h[5]),
          "v"(h[6]), "v"(h[7]), "v"(h[8]), "v"(h[9]), "v"(h[10]), "v"(h[11]), "v"(h[12]),
          "v"(h[13]), "v"(h[14]), "v"(h[15]));
    return y;
}
#undef MS_AX_
#undef MS_DT_

template <typename F, int... Js>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, Js...>) {
    (f(std::integral_constant<int, Js>{}), ...);
}

}  // namespace dev
}  // namespace msscan
