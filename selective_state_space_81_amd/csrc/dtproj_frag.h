// dtproj_frag.h -- matrix-core fragments of the fused step projection,
// shared by the lane and row kernels.
//
// The raw step size is projected from a low-rank input (the step is
// softplus of a linear map of the input plus a bias, jsqmd page section 2.2;
// the map is low-rank, a narrow slice of x_proj lifted to d_inner by dt_proj,
// lmnt page section 3.2):  delta[t][d] = sum_r W[d][r] * x[t][r],  r < rank.
// A 16-step x 16-channel tile of it is one v_mfma_f32_16x16x32_bf16 per 32
// rank columns (fp32 io: eight v_mfma_f32_16x16x4f32): lane l supplies row
// l mod 16 of the A operand (timestep) and column l mod 16 of the B operand
// (channel), each over k = 8 (l / 16) .. +7 of the slice, and receives the
// output rows 4 (l / 16) .. +3 of column l mod 16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dpp_common.h"

namespace msscan {
namespace dev {

constexpr int kMaxRank = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float frag_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t frag_u4 __attribute__((ext_vector_type(4)));

// Eight consecutive io values k0 .. k0+7 of one row (row byte offset `row`,
// row length `rank`), zero at k >= rank and outside the resource.  `vec`:
// rows are 16-byte multiples, so whole 16-byte loads apply.
template <bool BF16>
struct Frag8;
template <>
struct Frag8<true> {
    frag_u4 v;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t row, int k0, int rank,
                                         bool vec) {
        if (vec) {
            v = __builtin_amdgcn_raw_buffer_load_b128(r, k0 < rank ? row + 2u * k0 : kOutOfRange,
                                                      0, 0);
        } else {
            uint32_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                e[j] = __builtin_amdgcn_raw_buffer_load_b16(
                    r, k0 + j < rank ? row + 2u * (k0 + j) : kOutOfRange, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = e[2 * j] | (e[2 * j + 1] << 16);
            __builtin_amdgcn_sched_barrier(0);  // one fragment's loads in flight at a time
        }
    }
    __device__ __forceinline__ void mma(const Frag8& w, frag_f4& acc) const {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v),
                                                      __builtin_bit_cast(bf16x8, w.v), acc, 0, 0, 0);
    }
};
template <>
struct Frag8<false> {
    float v[8];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t row, int k0, int rank,
                                         bool vec) {
        if (vec) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int k = k0 + 4 * h;
                const frag_u4 w = __builtin_amdgcn_raw_buffer_load_b128(
                    r, k < rank ? row + 4u * k : kOutOfRange, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) v[4 * h + j] = __uint_as_float(w[j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    r, k0 + j < rank ? row + 4u * (k0 + j) : kOutOfRange, 0, 0));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // Eight K=4 products; lane group q supplies element j as its k, on both
    // operands alike, so the pairing of x and W along r is exact.
    __device__ __forceinline__ void mma(const Frag8& w, frag_f4& acc) const {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[j], w.v[j], acc, 0, 0, 0);
    }
};

}  // namespace dev
}  // namespace msscan
