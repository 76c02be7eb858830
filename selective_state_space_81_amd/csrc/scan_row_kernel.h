// scan_row_kernel.h -- the selective scan (S6) row kernel: one 16-lane DPP
// row per channel and one state per lane for d_state 9..16, or several rows
// per channel for up to 128 states, on gfx950 (states past d_state get
// A = B = C = 0, stay zero and are never stored).  Instantiated by
// scan_row.hip (one row per channel) and scan_row_wide.hip (several).
//
// Why this layout.  With every state of a channel in one lane (scan_lane),
// a Mamba-130M layer has only batch x d_inner = 12288 lanes of work, 192
// waves for 1024 SIMDs, so the sequence must be cut into ~32 segments, and
// every segment but the last is walked twice (once from zero for its
// summary).  Here a channel's 16 states sit in the 16 lanes of one DPP row:
// the same layer is 3072 waves with the sequence whole, and the scan is done
// in one pass over the inputs with no summary and no carry.
//
// What each lane does, per block of 16 timesteps [tb, tb + 16):
//   per element  lane k of a row owns timestep tb + k of the row's channel:
//                dt = softplus(delta + bias), x = dt*u (Euler, bilinear)
//   per state    for j = 0..15, with dt_j and x_j broadcast from lane j by
//                DPP row_newbcast (folded into the consuming v_mul):
//                  A_bar = exp(dt_j*A[n]),  h = A_bar*h + x_j*B_j[n],
//                  p_j = C_j[n]*h
//   readout      y_j = sum over the row's 16 lanes of p_j, a reduce-scatter
//                whose result for timestep j lands in lane j (four DPP
//                stages, the first two with bank masks so that each half of
//                the row keeps its own timesteps without a select)
//   per element  lane k: y = (y + D*u) * silu(z), rounded, stored
// so the per-element work (softplus, gate, D, conversions) is done once per
// element, as in the naive loop of the lmnt page (section 3.2), and only the
// recurrence is spread over states.
//
// B_t and C_t (shared by all channels, lmnt page section 3.2) vary along
// the lanes of a row here, so they cannot come by broadcast: the workgroup
// loads the block's 16 x 16 tile of each once (one value per thread),
// widens it and writes it to LDS transposed ([state][time]); every lane then
// reads its state's 16 values with four 16-byte LDS reads.  One barrier per
// block (the LDS tiles alternate between two buffers).
//
// u, delta, z and y move one element per lane, a wave covering its 4
// channels over the block's 16 timesteps.  The L1 looks up the lines of a
// memory instruction quad by quad, so the loads and stores use the lane
// order in which a quad holds the 4 channels of one timestep (one line per
// quad), and ds_bpermute turns the values into the row order (lane k of
// row r: channel r, timestep k) and y back.  With the row order itself every
// quad would span 4 timesteps and 4 lines, and the L1 tag lookups, not the
// VALU, bounded the kernel.  The workgroup's 16 channels are a quarter of a
// 128-byte row segment, so workgroups are assigned to XCDs in contiguous
// ranges of tiles (the hardware deals workgroup ids to the 8 XCDs in turn):
// the tiles that share a cache line run on one XCD and share its L2.
//
// Wider states.  A channel of more than 16 states spreads over RPC = 2 or 4
// rows of one wave (up to 32 or 64 states), and with SPL = 2 states per lane
// up to 128.  Each row reduces its own states as above and the rows' partial
// sums are added across lanes 16 (and 32) apart with ds_bpermute; every row
// repeats its channel's per-element work, and the workgroup grows to 4 * RPC
// waves so that it still covers 16 channels with whole 16-byte io tiles.
//
// Segments.  When batch x channels alone do not fill the chip, the sequence
// is still cut into segments: a summary variant (SUMMARY) walks each segment
// but the last from zero and writes its end state and sum of dt (or the
// product of A_bar, bilinear), the shared carry pass composes them, and the
// main variant starts each segment from its carried state -- the scan is a
// composition of affine maps (jsqmd page, section 3.4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "dpp_common.h"
#include "dtproj_frag.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

constexpr int kRT = 16;        // timesteps per block = lanes of a DPP row
constexpr int kBcS = 20;       // LDS stride (floats) of one state's 16 timesteps
#ifndef MSSCAN_ROW_PF
#define MSSCAN_ROW_PF 4
#endif
constexpr int kRowPf = MSSCAN_ROW_PF;  // blocks between a block's loads and its staging
constexpr int kNb = 4;                 // LDS buffers of staged blocks (>= 3)
constexpr int kRowUnroll = 4;          // blocks per unrolled loop body
static_assert(kRowUnroll % kRowPf == 0 && kRowUnroll % kNb == 0,
              "block j uses load set j mod PF and buffer j mod NB");

typedef float f4 __attribute__((ext_vector_type(4)));

// Readout reduce-scatter, stages 1-2: p[j] (this lane's term for timestep
// j) -> r[m], the sum over 4 lanes for timestep 8*bit3 + 4*bit2 + m of the
// lane index within the row.
//   stage 1: lanes k and k^8 (row_ror:8); lanes 0-7 (banks 0,1) keep
//            timesteps 0-7, lanes 8-15 (banks 2,3) timesteps 8-15.
//   stage 2: lanes k and 7-k of each half (row_half_mirror); quad 0 of each
//            half (banks 0,2) keeps the half's first 4 timesteps, quad 1
//            (banks 1,3) the last 4.
// Each output is written by two instructions with complementary bank masks
// (lanes of a disabled bank keep the register's value).  The leading s_nop
// gives the two wait states a DPP read needs after a VALU write.
#define MS_S1_(m, a, b)                                                                   \
    "v_add_f32_dpp %" #m ", %" #a ", %" #a " row_ror:8 row_mask:0xf bank_mask:0x3\n"      \
    "v_add_f32_dpp %" #m ", %" #b ", %" #b " row_ror:8 row_mask:0xf bank_mask:0xc\n"
#define MS_S2_(m, a, b)                                                                       \
    "v_add_f32_dpp %" #m ", %" #a ", %" #a " row_half_mirror row_mask:0xf bank_mask:0x5\n"    \
    "v_add_f32_dpp %" #m ", %" #b ", %" #b " row_half_mirror row_mask:0xf bank_mask:0xa\n"
__device__ __forceinline__ void row_reduce_16_to_4(const float (&p)[16], float (&r)[4]) {
    float q[8];
    asm("s_nop 1\n" MS_S1_(0, 8, 16) MS_S1_(1, 9, 17) MS_S1_(2, 10, 18) MS_S1_(3, 11, 19)
            MS_S1_(4, 12, 20) MS_S1_(5, 13, 21) MS_S1_(6, 14, 22) MS_S1_(7, 15, 23)
        : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]),
          "=&v"(q[6]), "=&v"(q[7])
        : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]),
          "v"(p[7]), "v"(p[8]), "v"(p[9]), "v"(p[10]), "v"(p[11]), "v"(p[12]), "v"(p[13]),
          "v"(p[14]), "v"(p[15]));
    asm("s_nop 1\n" MS_S2_(0, 4, 8) MS_S2_(1, 5, 9) MS_S2_(2, 6, 10) MS_S2_(3, 7, 11)
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]),
          "v"(q[7]));
}
// Stage 1 for one register pair, p[m] = a and p[m + 8] = b: lets a caller
// that forms the 16 terms one at a time combine each pair as soon as both
// exist (with the rest of the reduce in row_reduce_finish).
__device__ __forceinline__ float row_reduce_pair(float a, float b) {
    float q;
    asm("s_nop 1\n" MS_S1_(0, 1, 2) : "=&v"(q) : "v"(a), "v"(b));
    return q;
}
// Stage 2 for one pair, q[m] = a and q[m + 4] = b.
__device__ __forceinline__ float row_reduce_pair2(float a, float b) {
    float r;
    asm("s_nop 1\n" MS_S2_(0, 1, 2) : "=&v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ void row_reduce_8_to_4(const float (&q)[8], float (&r)[4]) {
    asm("s_nop 1\n" MS_S2_(0, 4, 8) MS_S2_(1, 5, 9) MS_S2_(2, 6, 10) MS_S2_(3, 7, 11)
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]),
          "v"(q[7]));
}
#undef MS_S1_
#undef MS_S2_

// quad_perm DPP controls: [2,3,0,1] (lane k reads k^2) and [1,0,3,2] (k^1).
constexpr int kQpXor2 = 0x4e;
constexpr int kQpXor1 = 0xb1;
template <int CTRL>
__device__ __forceinline__ float qperm(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// The whole readout: lane k of each row receives sum over the row of p[k].
// Stages 3-4 pair lanes k, k^2 and k, k^1 inside a quad; a bank covers a
// whole quad, so there each lane sums both candidates and keeps one.
__device__ __forceinline__ float row_reduce_scatter(const float (&p)[16], bool bit1, bool bit0) {
    float r[4];
    row_reduce_16_to_4(p, r);
    const float t0 = r[0] + qperm<kQpXor2>(r[0]);
    const float t1 = r[1] + qperm<kQpXor2>(r[1]);
    const float t2 = r[2] + qperm<kQpXor2>(r[2]);
    const float t3 = r[3] + qperm<kQpXor2>(r[3]);
    const float s0 = bit1 ? t2 : t0;
    const float s1 = bit1 ? t3 : t1;
    const float u0 = s0 + qperm<kQpXor1>(s0);
    const float u1 = s1 + qperm<kQpXor1>(s1);
    return bit0 ? u1 : u0;
}

// Stages 3-4 of the readout (r[m] from stage 2).
__device__ __forceinline__ float row_reduce_quads(const float (&r)[4], bool bit1, bool bit0) {
    const float t0 = r[0] + qperm<kQpXor2>(r[0]);
    const float t1 = r[1] + qperm<kQpXor2>(r[1]);
    const float t2 = r[2] + qperm<kQpXor2>(r[2]);
    const float t3 = r[3] + qperm<kQpXor2>(r[3]);
    const float s0 = bit1 ? t2 : t0;
    const float s1 = bit1 ? t3 : t1;
    const float u0 = s0 + qperm<kQpXor1>(s0);
    const float u1 = s1 + qperm<kQpXor1>(s1);
    return bit0 ? u1 : u0;
}
// The rest of the readout after stage 1 (q[m] from row_reduce_pair).
__device__ __forceinline__ float row_reduce_finish(const float (&q)[8], bool bit1, bool bit0) {
    float r[4];
    row_reduce_8_to_4(q, r);
    return row_reduce_quads(r, bit1, bit0);
}

// out[i] = (v broadcast from lane J0 + i of the row) * x_i, as four
// v_mul_f32_dpp.  The compiler folds a broadcast into the consuming v_mul
// (row_bcast), but in the summary and checkpoint walks it scheduled the moves
// apart from their multiplies and left them unfolded: 32 extra moves per
// block.  The leading s_nop 1 gives the two wait states a DPP read needs.
template <int J0>
__device__ __forceinline__ void mul_bcast4(float* out, float v, float x0, float x1, float x2,
                                           float x3) {
    asm("s_nop 1\n"
        "v_mul_f32_dpp %0, %4, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %1, %4, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %2, %4, %7 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n"
        "v_mul_f32_dpp %3, %4, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf"
        : "=&v"(out[0]), "=&v"(out[1]), "=&v"(out[2]), "=&v"(out[3])
        : "v"(v), "v"(x0), "v"(x1), "v"(x2), "v"(x3), "n"(J0), "n"(J0 + 1), "n"(J0 + 2),
          "n"(J0 + 3));
}

// Sum over the 16 lanes of a row, in every lane.
__device__ __forceinline__ float row_allsum(float v) {
    v += qperm<kQpXor1>(v);
    v += qperm<kQpXor2>(v);
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, true));
    return v;
}

// A raw io value (bf16 bits zero-extended, or fp32 bits) moved to another
// lane of the wave (byte address 4 * lane), and widened to fp32.
template <typename T>
__device__ __forceinline__ uint32_t permute_bits(T v, int addr) {
    uint32_t bits;
    if constexpr (sizeof(T) == 2)
        bits = (uint32_t)v;
    else
        bits = __float_as_uint(v);
    return (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)bits);
}
template <bool BF16>
__device__ __forceinline__ float widen_bits(uint32_t bits) {
    return __uint_as_float(BF16 ? bits << 16 : bits);
}

// VB consecutive timesteps of one state, widened, into an LDS row.
template <int VB, typename RT, typename W>
__device__ __forceinline__ void put_bc(float* dst, const RT (&v)[VB], W widen) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    if constexpr (VB == 1) {
        dst[0] = widen(v[0]);
    } else if constexpr (VB == 2) {
        *reinterpret_cast<f2*>(dst) = f2{widen(v[0]), widen(v[1])};
    } else {
#pragma unroll
        for (int i = 0; i < VB; i += 4)
            *reinterpret_cast<f4*>(dst + i) =
                f4{widen(v[i]), widen(v[i + 1]), widen(v[i + 2]), widen(v[i + 3])};
    }
}

// RPC: DPP rows per channel (1, 2, 4); SPL: states per lane (1, 2).  A channel
// holds kRT * RPC * SPL states: lane n of the channel's row g holds states
// q * kRT * RPC + kRT * g + n for q < SPL.  A workgroup is 4 waves, 16 rows:
// CH = 16 / RPC channels, every row of a channel in one wave.
//
// CKPT (one row per channel, one segment): store the state before every
// block into a.agg as [batch][block][d_inner][d_state], from h0 (or zero)
// over the whole sequence.  With SUMMARY it is the backward's forward walk
// (no readout, no output); without, the forward pass saving the backward's
// checkpoints beside y.
//
// DTP (whole io tiles): the raw step is not read but projected,
// delta[t][d] = sum_r W[d][r] x[t][r] (dtproj_frag.h).  Wave 1, which would
// move the delta tile, loads the block's 16 x rank tile of x instead and, at
// staging, forms a 16-step x 16-channel delta tile on the matrix cores
// against W fragments it loaded once (the workgroup's CH channels first;
// with several rows per channel the rest of the 16 are computed and unused);
// the tile goes to LDS in fp32 (never rounded to the io type).  With two
// states per lane and bf16 io that variant asks for three waves per SIMD
// (168 registers, no spills), which the LDS of three workgroups allows; at
// the 200 it takes unasked, two fit, and a d_state 128 grid at batch 2 x
// d_inner 1536 ran in one and a half rounds (1.27 against 1.00 ms).
template <bool BF16, int DISC, bool SP, bool SUMMARY, bool COOP, int RPC, int SPL,
          bool CKPT = false, bool DTP = false>
__global__ void __launch_bounds__(64 * kRowWaves)
    __attribute__((amdgpu_waves_per_eu(DTP && SPL == 2 && BF16 ? 3 : 1))) scan_row(ScanArgs a) {
    static_assert(!CKPT || (RPC == 1 && SPL == 1), "checkpoints of one-row channels");
    static_assert(!DTP || (COOP && !CKPT), "projected step");
    static_assert(RPC == 1 || RPC == 2 || RPC == 4, "a channel's rows share one wave");
    static_assert(SPL == 1 || SPL == 2, "states per lane");
    static_assert(COOP || RPC == 1, "several rows per channel move io as whole tiles");
    constexpr int CH = kRowCh / RPC;             // channels per workgroup
    constexpr int kNS = kRT * RPC * SPL;         // states per channel, padded
    constexpr int kThreads = 64 * kRowWaves;
    constexpr int VB = kRT * kNS / kThreads;     // B (and C) tile values per thread
    // Two states per lane take twice as long per block, so half the blocks
    // in flight hide the same load latency, with half the load registers.
    // With the projection's x rows as well (bf16), one block ahead: that and
    // the register cap below keep three workgroups per CU, as without it.
    constexpr int PF = (SPL == 2 && DTP && BF16) ? 1 : (SPL == 2 || DTP) ? 2 : kRowPf;
    // Two states per lane make a 128-state B/C tile (20 KB per buffer): the
    // pipeline then runs on two buffers (NB2, below), which keeps the LDS of
    // three workgroups within a CU (three buffers allowed two).
    constexpr bool NB2 = SPL == 2;
    static_assert(!NB2 || COOP, "the two-buffer pipeline stages io tiles in LDS");
    constexpr int NB = NB2 ? 2 : kNb;
    constexpr int U = NB2 ? 2 : kRowUnroll;  // blocks per unrolled loop body
    static_assert(U % PF == 0 && U % NB == 0 && U % 2 == 0, "sets, buffers and y tiles cycle");
    constexpr bool ZOH = DISC == kZoh;
    constexpr bool BIL = DISC == kBilinear;
    constexpr bool PROD = SUMMARY && BIL && !CKPT;  // bilinear summary: product of A_bar
    using R = Io<BF16>;
    using RT = typename R::T;
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));

    // io tiles move in chunks of 16 bytes, or 8 when a tile row is 8 bytes
    // (4 bf16 channels)
    constexpr int kChB = CH * R::kSize < 16 ? CH * R::kSize : 16;
    using Chunk = std::conditional_t<kChB == 16, u4, u2>;
    static_assert(kChB == 16 || kChB == 8, "io chunk size");
    constexpr int kCw = kChB / R::kSize;  // channels per chunk
    constexpr int kCpr = CH / kCw;        // chunks per tile row
    constexpr int kIoS = CH + (BF16 ? 8 : 4);  // LDS row stride (elements) of an io tile
    constexpr int kIoT = SUMMARY ? 2 : 3; // io tiles staged: u, delta (, z)
    // LDS.  Block j is staged in buffer j mod NB: its B (and C) tile, widened,
    // [tensor][state][timestep]; with COOP also its u, delta (, z) tiles
    // [tensor][timestep][channel].  y tiles [timestep][channel] alternate
    // between two buffers (COOP).
    __shared__ __attribute__((aligned(16))) float s_bc[NB][SUMMARY ? 1 : 2][kNS][kBcS];
    __shared__ __attribute__((aligned(16))) RT s_io[COOP ? NB : 1][COOP ? kIoT : 1][kRT][kIoS];
    __shared__ __attribute__((aligned(16))) RT s_y[(COOP && !SUMMARY) ? 2 : 1][kRT][kIoS];
    // DTP: the projected delta tile of a staged block, [channel][step] fp32
    __shared__ __attribute__((aligned(16))) float s_dt[DTP ? NB : 1][DTP ? kRowCh : 1][kBcS];
    // ZOH main pass: each row's per-step (dt, x) of a block,
    // [parity][row][step][2]; every lane of the row reads them back as LDS
    // broadcasts, so the recurrence's products take plain VGPR operands (no
    // DPP source).  ZOH reads dt twice per state-step, and there this beat
    // the DPP broadcasts (3B layer 1.27 -> 1.21 ms); for Euler it lost (the
    // 130M layer 0.140 -> 0.147 ms).
    constexpr bool LDSB = !SUMMARY && ZOH;
    __shared__ __attribute__((aligned(16))) float s_dx[LDSB ? 2 : 1][LDSB ? kRowCh : 1][kRT][2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int n = lane & 15;  // this lane's state; also its timestep slot
    const int tiles = a.tiles;
    const int segs = (SUMMARY && !CKPT) ? a.chunks - 1 : a.chunks;
    const uint32_t l = xcd_logical(blockIdx.x, gridDim.x);
    const int tile = (int)(l % (uint32_t)tiles);
    const int seg = (int)((l / (uint32_t)tiles) % (uint32_t)segs);
    const int b = (int)(l / ((uint32_t)tiles * (uint32_t)segs));

    const int grow = tid >> 4;                 // the lane's row in the workgroup
    const int cl = grow / RPC;                 // the row's channel within the tile
    const int sg = grow % RPC;                 // the row's group of states
    const int c = tile * CH + cl;
    const bool cvalid = c < a.Dn;
    const int cc = cvalid ? c : a.Dn - 1;
    const int Nr = a.N;
    int st[SPL];       // this lane's states
    bool svalid[SPL];
    float A2[SPL], invA[SPL], h[SPL];
    const int km1 = a.chunks - 1;
#pragma unroll
    for (int q = 0; q < SPL; ++q) {
        st[q] = q * kRT * RPC + kRT * sg + n;
        svalid[q] = st[q] < Nr;
        const float av = svalid[q] ? a.A[(int64_t)cc * Nr + st[q]] : 0.f;
        A2[q] = av * kLog2e;
        invA[q] = 0.f;
        if constexpr (ZOH) invA[q] = av != 0.f ? 1.f / av : 0.f;
        h[q] = 0.f;
        if constexpr (!SUMMARY || CKPT) {
            if (svalid[q]) {
                if (seg == 0) {
                    // With several segments h0 is read from the carry pass's copy,
                    // so h_last (written by the last segment) may alias h0.
                    const float* h0 = a.chunks > 1 ? a.start0 : a.h0;
                    if (h0) h[q] = h0[((int64_t)b * a.Dn + cc) * Nr + st[q]];
                } else {
                    h[q] = a.agg[(((int64_t)b * km1 + (seg - 1)) * Nr + st[q]) * a.Dn + cc];
                }
            }
        }
    }
    const float bias = a.bias ? a.bias[cc] : 0.f;
    const float Dd = a.D ? a.D[cc] : 0.f;
    const bool has_z = a.z != nullptr;
    const bool bit1 = (n & 2) != 0, bit0 = (n & 1) != 0;

    const int64_t t0 = (int64_t)seg * a.chunk_len;
    const int64_t t1 = min(a.L, t0 + a.chunk_len);
    const int64_t row0 = (int64_t)b * a.L;
    const uint32_t rowb = (uint32_t)a.Dn * R::kSize;
    // Element io without COOP, in memory order: lane i of the wave holds the
    // wave's channel (i & 3) at timestep i >> 2 (one cache line per quad);
    // ds_bpermute moves values between that order and the row order.
    const int cm = tile * kRowCh + (tid >> 6) * 4 + (lane & 3);
    const uint32_t eoff =
        cm < a.Dn ? (uint32_t)(lane >> 2) * rowb + (uint32_t)cm * R::kSize : kOutOfRange;
    const int to_row = 4 * ((n << 2) | (lane >> 4));
    const int to_mem = 4 * (((lane & 3) << 4) | (lane >> 2));
    // COOP: wave w < kIoT moves io tile w (u, delta, z) with one chunk access
    // per lane (chunk cch of row crow); wave 3 stores the y tiles.  d_inner is
    // a multiple of kCw, so every chunk lies wholly inside or outside a row.
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int crow = lane / kCpr, cch = lane % kCpr;
    const int cchan = tile * CH + cch * kCw;
    const uint32_t coff = (lane < kRT * kCpr && cchan < a.Dn)
                              ? (uint32_t)crow * rowb + (uint32_t)cchan * R::kSize
                              : kOutOfRange;
    const int ntiles_io = SUMMARY ? 2 : (has_z ? 3 : 2);
    // DTP: this lane's operand row / column (m) and k quarter (q), the x and
    // W row strides, and the tile's W fragments (channels past d_inner read 0)
    const int fm = lane & 15, fq = lane >> 4;
    const uint32_t xrow = DTP ? (uint32_t)a.rank * R::kSize : 0u;
    const bool xvec = DTP && (a.rank % (BF16 ? 8 : 4)) == 0;
    Frag8<BF16> wfr[DTP ? 2 : 1];
    if constexpr (DTP) {
        if (wv == 1) {
            const auto rW = make_rsrc(a.wdt, (uint32_t)a.Dn * xrow);
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
                if (kc * 32 < a.rank)
                    wfr[kc].load(rW, (uint32_t)(tile * CH + fm) * xrow, kc * 32 + 8 * fq,
                                 a.rank, xvec);
        }
    }
    // CKPT: this lane's offset in a checkpoint slab [Dn][N]
    const uint32_t ck_off = (CKPT && cvalid && svalid[0])
                                ? ((uint32_t)c * (uint32_t)Nr + (uint32_t)st[0]) * 4u
                                : kOutOfRange;
    // this thread's elements of a block's B/C tile (kRT x kNS values): state
    // bs, timesteps VB * tq .. VB * tq + VB - 1.  Each load instruction covers
    // consecutive states of one timestep; the VB values of a state go to LDS
    // in one write (up to 16 bytes), which with the 20-float state stride
    // puts 8 lanes' 16-byte writes on distinct banks.
    const uint32_t kBRow = (uint32_t)Nr * R::kSize;
    const int bs = tid % kNS, tq = tid / kNS;
    const uint32_t boff =
        bs < Nr ? (uint32_t)(tq * VB) * kBRow + (uint32_t)bs * R::kSize : kOutOfRange;

    // Block starts are kept relative to t0 in 32 bits (a segment is < 2^31 steps).
    const int len = (int)(t1 - t0);
    // Rows of the block at rel inside the segment (0 past its end: loads there
    // read zeros and stores are dropped).  Wave-uniform; readfirstlane keeps
    // it in an SGPR, so the buffer descriptors built from it stay scalar.
    auto rows_of = [&](int rel) -> uint32_t {
        return (uint32_t)__builtin_amdgcn_readfirstlane(max(0, min(kRT, len - rel)));
    };
    auto base = [&](const void* p, int rel, uint32_t rb) -> const void* {
        return static_cast<const char*>(p) + (row0 + t0 + rel) * (int64_t)rb;
    };

    // Raw global data of one block, loaded PF blocks before it is staged.
    struct Raw {
        RT u, d, z;          // without COOP
        RT bb[VB], cb[VB];
        Chunk t;             // COOP: this lane's chunk of io tile wv
        Frag8<BF16> xf[DTP ? 2 : 1];  // DTP, wave 1: the block's x rows
    };
    auto load = [&](Raw& r, int rel) {
        // With one load set the compiler otherwise carries the block start
        // in a VGPR and wraps every load below in a waterfall loop.
        if constexpr (PF == 1) rel = __builtin_amdgcn_readfirstlane(rel);
        const uint32_t nr = rows_of(rel);
        if constexpr (COOP) {
            // DTP: wave 1's chunk load reads nothing (an empty range: zeros,
            // no memory access); the chunk path stays the same for every
            // wave, so its registers are the plain kernel's
            if (wv < ntiles_io) {
                const void* src = wv == 0 ? a.u : (wv == 1 ? (DTP ? a.u : a.delta) : a.z);
                const auto rs = make_rsrc(base(src, rel, rowb), (DTP && wv == 1) ? 0u : nr * rowb);
                if constexpr (kChB == 16)
                    r.t = __builtin_amdgcn_raw_buffer_load_b128(rs, coff, 0, 0);
                else
                    r.t = __builtin_amdgcn_raw_buffer_load_b64(rs, coff, 0, 0);
            }
            if constexpr (DTP) {
                if (wv == 1) {
                    const auto rX = make_rsrc(base(a.dtx, rel, xrow), nr * xrow);  // rows past L: 0
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc)
                        if (kc * 32 < a.rank)
                            r.xf[kc].load(rX, (uint32_t)fm * xrow, kc * 32 + 8 * fq, a.rank, xvec);
                }
            }
        } else {
            r.u = R::load(make_rsrc(base(a.u, rel, rowb), nr * rowb), eoff);
            r.d = R::load(make_rsrc(base(a.delta, rel, rowb), nr * rowb), eoff);
            if constexpr (!SUMMARY)
                r.z = has_z ? R::load(make_rsrc(base(a.z, rel, rowb), nr * rowb), eoff) : RT{};
        }
#pragma unroll
        for (int v = 0; v < VB; ++v) {
            r.bb[v] = R::load(make_rsrc(base(a.B, rel, kBRow), nr * kBRow), boff + v * kBRow);
            if constexpr (!SUMMARY)
                r.cb[v] = R::load(make_rsrc(base(a.C, rel, kBRow), nr * kBRow), boff + v * kBRow);
        }
    };
    // Without COOP the io values of a staged block wait in registers, in row order.
    struct Staged {
        uint32_t u = 0, d = 0, z = 0;
    };
    // Stage the block at rel (raw set r) into LDS buffer buf, then refill r
    // with the block PF ahead.
    auto stage = [&](Raw& r, int rel, int buf, Staged& sg) {
        const auto widen = [](RT x) { return R::widen(x); };
        put_bc<VB>(&s_bc[buf][0][bs][tq * VB], r.bb, widen);
        if constexpr (!SUMMARY) put_bc<VB>(&s_bc[buf][1][bs][tq * VB], r.cb, widen);
        if constexpr (COOP) {
            if (wv < ntiles_io && lane < kRT * kCpr)  // DTP: wave 1's zeros go unread
                *reinterpret_cast<Chunk*>(&s_io[buf][wv][crow][cch * kCw]) = r.t;
            if constexpr (DTP) {
                if (wv == 1) {
                    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kc = 0; kc < 2; ++kc)
                        if (kc * 32 < a.rank) r.xf[kc].mma(wfr[kc], acc);
                    // acc[i]: delta at step 4 fq + i of channel fm
                    *reinterpret_cast<f4*>(&s_dt[buf][fm][4 * fq]) = acc;
                }
            }
        } else {
            sg.u = permute_bits(r.u, to_row);
            sg.d = permute_bits(r.d, to_row);
            if constexpr (!SUMMARY) {
                if (has_z) sg.z = permute_bits(r.z, to_row);
            }
        }
        load(r, rel + PF * kRT);
    };
    // Per-element values of a staged block, in row order: lane k holds
    // timestep k of its row's channel.
    struct Elem {
        float dt, xv, u, z;
    };
    auto prologue = [&](int rel, int buf, const Staged& sg, int par) -> Elem {
        Elem e{};
        float draw;
        if constexpr (COOP) {
            e.u = R::widen(s_io[buf][0][n][cl]);
            if constexpr (DTP)
                draw = s_dt[buf][cl][n];
            else
                draw = R::widen(s_io[buf][1][n][cl]);
            if constexpr (!SUMMARY) {
                if (has_z) e.z = R::widen(s_io[buf][2][n][cl]);
            }
        } else {
            e.u = widen_bits<BF16>(sg.u);
            draw = widen_bits<BF16>(sg.d);
            if constexpr (!SUMMARY) e.z = widen_bits<BF16>(sg.z);
        }
        float dt = draw + bias;
        if constexpr (SP) dt = softplus_f(dt);
        e.dt = n < (int)rows_of(rel) ? dt : 0.f;  // steps past the end change nothing
        e.xv = ZOH ? e.u : e.dt * e.u;            // B is scaled by u (ZOH) or dt*u
        if constexpr (LDSB) {
            float2 v;
            v.x = e.dt;
            v.y = e.xv;
            *reinterpret_cast<float2*>(&s_dx[par][grow][n][0]) = v;
        }
        return e;
    };
    // COOP: wave 3 stores the y tile of the block at rel from buffer buf.
    auto store_y_tile = [&](int rel, int buf) {
        if constexpr (COOP && !SUMMARY) {
            if (wv == kRowWaves - 1 && lane < kRT * kCpr) {
                const Chunk v = *reinterpret_cast<const Chunk*>(&s_y[buf][crow][cch * kCw]);
                const auto rs = make_rsrc(base(a.y, rel, rowb), rows_of(rel) * rowb);
                if constexpr (kChB == 16)
                    __builtin_amdgcn_raw_buffer_store_b128(v, rs, coff, 0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b64(v, rs, coff, 0, 0);
            }
        }
    };

    float s_sum = 0.f, s_comp = 0.f;  // SUMMARY: Kahan sum of this lane's dt values
    float P[SPL];                     // PROD: product of A_bar
#pragma unroll
    for (int q = 0; q < SPL; ++q) P[q] = 1.f;

    // The recurrence over the block at rel (staged in buffer buf) and, unless
    // SUMMARY, its readout and output (y tile ybuf with COOP).
    auto compute = [&](int rel, int buf, int ybuf, const Elem& e) __attribute__((always_inline)) {
        if constexpr (CKPT) {
            // the block's [Dn][N] slab, addressed per block (wave-uniform
            // base), this lane's state at a fixed offset
            const int64_t slab = (int64_t)a.Dn * Nr;
            const float* ck = a.agg + ((int64_t)b * ((a.L + kRT - 1) / kRT) + rel / kRT) * slab;
            __builtin_amdgcn_raw_buffer_store_b32(
                __float_as_uint(h[0]), make_rsrc(ck, rel < len ? (uint32_t)slab * 4u : 0u),
                ck_off, 0, 0);
        }
        float p[16];
        static_for([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        // a second state's tiles are read only after the first state's work
        // (keeps one state's 32 B/C values live, not two)
        if constexpr (q > 0) __builtin_amdgcn_sched_barrier(0);
        f4 Bq[4], Cq[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Bq[i] = *reinterpret_cast<const f4*>(&s_bc[buf][0][st[q]][4 * i]);
            if constexpr (!SUMMARY)
                Cq[i] = *reinterpret_cast<const f4*>(&s_bc[buf][1][st[q]][4 * i]);
        }
        // the walks without a readout form the block's broadcast products
        // up front (mul_bcast4); the main pass leaves them to the compiler
        float argv[SUMMARY ? kRT : 1], ubv[SUMMARY ? kRT : 1];
        if constexpr (SUMMARY) {
            static_for(
                [&](auto gc) {
                    constexpr int g = decltype(gc)::value;
                    mul_bcast4<4 * g>(&argv[4 * g], e.dt, A2[q], A2[q], A2[q], A2[q]);
                    mul_bcast4<4 * g>(&ubv[4 * g], e.xv, Bq[g][0], Bq[g][1], Bq[g][2], Bq[g][3]);
                },
                std::make_integer_sequence<int, 4>{});
        }
        f4 dx[2];  // main pass: (dt, x) of steps 4g .. 4g + 3 of the current group
        static_for(
            [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const float bj = Bq[j / 4][j % 4];
                float arg, ub, dtj = 0.f;
                if constexpr (SUMMARY) {
                    arg = argv[j];
                    ub = ubv[j];
                } else if constexpr (!LDSB) {
                    arg = row_bcast<j>(e.dt) * A2[q];
                    ub = row_bcast<j>(e.xv) * bj;
                } else {
                    if constexpr (j % 4 == 0) {
                        dx[0] = *reinterpret_cast<const f4*>(&s_dx[ybuf][grow][j][0]);
                        dx[1] = *reinterpret_cast<const f4*>(&s_dx[ybuf][grow][j + 2][0]);
                    }
                    dtj = dx[(j % 4) / 2][2 * (j % 2)];
                    arg = dtj * A2[q];
                    ub = dx[(j % 4) / 2][2 * (j % 2) + 1] * bj;
                }
                float abar = 0.f, bx = 0.f;
                if constexpr (BIL) {
                    const float r = bilinear_r(arg);
                    if constexpr (PROD) {
                        abar = fmaf(2.f, r, -1.f);
                        bx = ub * r;
                    } else {
                        // (2r - 1) h + r ub = r (2h + ub) - h: two fmas
                        h[q] = fmaf(r, fmaf(2.f, h[q], ub), -h[q]);
                    }
                } else {
                    abar = hw_exp2(arg);
                    if constexpr (ZOH) {
                        const float dtb = LDSB ? dtj : row_bcast<j>(e.dt);
                        const float ser = dtb * fmaf(arg, fmaf(arg, kZohT2, kZohT1), 1.f);
                        const float big = fmaf(abar, invA[q], -invA[q]);
                        bx = (fabsf(arg) < kZohSwitch ? ser : big) * ub;
                    } else {
                        bx = ub;
                    }
                }
                if constexpr (!BIL || PROD) h[q] = fmaf(abar, h[q], bx);
                if constexpr (PROD) P[q] *= abar;
                if constexpr (!SUMMARY) {
                    if constexpr (q == 0)
                        p[j] = Cq[j / 4][j % 4] * h[q];
                    else
                        p[j] = fmaf(Cq[j / 4][j % 4], h[q], p[j]);
                }
            },
            std::make_integer_sequence<int, kRT>{});
        }, std::make_integer_sequence<int, SPL>{});
        if constexpr (SUMMARY) {
            if constexpr (!PROD && !CKPT) {
                const float yk = e.dt - s_comp;
                const float tk = s_sum + yk;
                s_comp = (tk - s_sum) - yk;
                s_sum = tk;
            }
        } else {
            float y = row_reduce_scatter(p, bit1, bit0);
            // the channel's other rows hold the rest of its states: lanes 16
            // (and 32) apart; every row ends with the same sum
            if constexpr (RPC >= 2)
                y += __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (lane ^ 16), __float_as_int(y)));
            if constexpr (RPC >= 4)
                y += __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (lane ^ 32), __float_as_int(y)));
            y = fmaf(Dd, e.u, y);
            if (has_z) y *= silu_f(e.z);
            if constexpr (COOP) {
                if (sg == 0) {
                    if constexpr (BF16)
                        s_y[ybuf][n][cl] = f32_to_bf16_rne(y);
                    else
                        s_y[ybuf][n][cl] = y;
                }
            } else {
                y = __int_as_float(__builtin_amdgcn_ds_bpermute(to_mem, __float_as_int(y)));
                R::store(make_rsrc(base(a.y, rel, rowb), rows_of(rel) * rowb), eoff, y);
            }
        }
    };

    // Software pipeline, one barrier per block j: stage block j + 1 (its raw
    // data loaded PF blocks earlier), barrier, store the y tile of block
    // j - 1, form the per-element values of block j + 1, and run block j's
    // recurrence with the values formed one block earlier.  Block j + 1 is
    // staged while slower waves may still read block j's buffer, and block
    // j + 2 only after every wave has passed block j + 1's barrier, so
    // NB >= 3 buffers suffice (NB2: two, below).  Blocks past the end stage
    // zeros, harmlessly.
    // NB2: barrier, store the y tile of block j - 1, form block j's
    // per-element values, stage block j + 1, run block j.  Every wave has
    // left block j - 1 (the other buffer) when it passes the barrier, so two
    // buffers suffice; the per-element values are formed just before their
    // block.
    const int nblk = (len + kRT - 1) / kRT;
    Raw r[PF];
    static_for([&](auto ic) { load(r[decltype(ic)::value], decltype(ic)::value * kRT); },
               std::make_integer_sequence<int, PF>{});
    Elem e;
    {
        Staged sg;
        stage(r[0], 0, 0, sg);
        if constexpr (!NB2) {
            __syncthreads();
            e = prologue(0, 0, sg, 0);
        }
    }
    auto do_block = [&](auto ic, int j) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;  // j mod U
        Staged sg;
        if constexpr (NB2) {
            __syncthreads();
            if (j > 0) store_y_tile((j - 1) * kRT, (i + 1) & 1);
            const Elem ej = prologue(j * kRT, i % NB, sg, i & 1);
            stage(r[(i + 1) % PF], (j + 1) * kRT, (i + 1) % NB, sg);
            compute(j * kRT, i % NB, i & 1, ej);
        } else {
            stage(r[(i + 1) % PF], (j + 1) * kRT, (i + 1) % NB, sg);
            __syncthreads();
            if (j > 0) store_y_tile((j - 1) * kRT, (i + 1) & 1);
            const Elem en = prologue((j + 1) * kRT, (i + 1) % NB, sg, (i + 1) & 1);
            compute(j * kRT, i % NB, i & 1, e);
            e = en;
        }
    };
    int blk = 0;
    for (; blk + U - 1 < nblk; blk += U)
        static_for([&](auto ic) { do_block(ic, blk + decltype(ic)::value); },
                   std::make_integer_sequence<int, U>{});
    static_for(
        [&](auto ic) {
            if (blk + decltype(ic)::value < nblk) do_block(ic, blk + decltype(ic)::value);
        },
        std::make_integer_sequence<int, U - 1>{});
    if constexpr (COOP && !SUMMARY) {  // the last block's y tile
        __syncthreads();
        store_y_tile((nblk - 1) * kRT, (nblk - 1) & 1);
    }

    if constexpr (SUMMARY && !CKPT) {
        const int64_t sb = (int64_t)b * km1 + seg;
        if constexpr (PROD) {
#pragma unroll
            for (int q = 0; q < SPL; ++q) {
                if (cvalid && svalid[q]) {
                    a.agg[(sb * Nr + st[q]) * a.Dn + c] = h[q];
                    a.prod[(sb * Nr + st[q]) * a.Dn + c] = P[q];
                }
            }
        } else {
            const float total = row_allsum(s_sum);
#pragma unroll
            for (int q = 0; q < SPL; ++q)
                if (cvalid && svalid[q]) a.agg[(sb * Nr + st[q]) * a.Dn + c] = h[q];
            if (cvalid && n == 0 && sg == 0) a.sdt[sb * a.Dn + c] = total;
        }
    } else if (!SUMMARY && seg == a.chunks - 1 && a.h_last && cvalid) {
#pragma unroll
        for (int q = 0; q < SPL; ++q)
            if (svalid[q]) a.h_last[((int64_t)b * a.Dn + c) * Nr + st[q]] = h[q];
    }
}

}  // namespace
}  // namespace msscan
