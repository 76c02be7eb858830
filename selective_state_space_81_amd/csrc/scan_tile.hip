// scan_tile.hip -- fast path of the selective scan (S6) for gfx950.
//
// One workgroup owns one 64-channel tile of one batch row over one segment of
// the sequence (the whole sequence when the batch x tile count fills the
// chip).  Its S waves split the d_state states (NS = d_state / S per lane), so
// every (channel, state) recurrence h = exp(dt*A)*h + B_bar*u runs in one lane
// with its state in a VGPR for the whole segment: no state is recomputed and
// no carry is exchanged inside a segment.
//
// The sequence is walked in blocks of TB timesteps, each in three phases:
//   A  per element (t, channel), spread over all threads of the workgroup:
//      widen u / delta, dt = softplus(delta + bias), x = dt*u, into LDS.  Each
//      element's activations are computed once, not once per state.
//   B  per wave: for each timestep, its NS states advance and their partial
//      readout sum_n C*h goes to LDS.
//   C  per element again: y = sum of the S partials + D*u, times silu(z),
//      rounded to the io type and stored (coalesced rows).
// The next block's global loads are issued before phase A of the current one
// (register double buffering) and the LDS buffers alternate between blocks,
// so each block needs two barriers.
//
// B_t and C_t are shared by every channel (the naive scan of the lmnt page,
// section 3.2, broadcasts them over channels).  They reach the VALU as DPP
// operands: a prepass widens them to fp32 rows [b][t][B row | C row]; each
// lane loads the value of state n0 + (lane mod NS) and the row_newbcast DPP
// control hands state n0 + j of the lane's 16-lane row to every lane as the
// first operand of v_mul / v_fmac.  No LDS bandwidth, no SGPRs and no extra
// instruction is spent per (state, timestep) on the broadcast.
//
// With several segments, a summary variant of the same kernel (no readout,
// SUMMARY = true) computes each segment's end state from zero and its
// compensated sum of dt; the shared carry pass composes them in order (the
// scan is a composition of affine maps, jsqmd page section 3.4) and the main
// variant starts every segment from its true state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "dpp_common.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

template <int NS, int S, int TB, bool BF16, int DISC, bool SUMMARY>
__global__ void __launch_bounds__(64 * S) scan_tile(ScanArgs a) {
    constexpr bool ZOH = DISC == kZoh;
    constexpr bool BIL = DISC == kBilinear;
    constexpr bool PROD = SUMMARY && BIL;  // bilinear: keep the product of A_bar
    constexpr int N = NS * S;
    constexpr int J = TB / S;  // timesteps per thread in phases A/C
    static_assert(TB % S == 0, "TB must be a multiple of S");
    static_assert(NS == 2 || NS == 4 || NS == 8 || NS == 16, "a wave's states fit one DPP row");
    using R = Io<BF16>;
    using RT = typename R::T;

    __shared__ float2 s_dx[2][TB][64];  // (dt, x) Euler and bilinear; (dt, u) ZOH
    __shared__ float s_y[SUMMARY ? 1 : 2][SUMMARY ? 1 : S][SUMMARY ? 1 : TB][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = blockIdx.z;
    const int seg = blockIdx.y;
    const int d = blockIdx.x * 64 + lane;
    const bool dvalid = d < a.Dn;
    const int dd = dvalid ? d : a.Dn - 1;
    const int n0 = w * NS;

    // The true d_state Nr may be below N: states Nr..N-1 get A = 0 and, in
    // the prepared B/C rows, B = C = 0, so they stay zero; they are never
    // stored, and every stride outside the prepared rows uses Nr.
    const int Nr = a.N;
    float A2[NS], invA[NS], h[NS], P[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        P[j] = 1.f;
        const float av = n0 + j < Nr ? a.A[(int64_t)dd * Nr + n0 + j] : 0.f;
        A2[j] = av * kLog2e;
        if constexpr (ZOH) invA[j] = (av != 0.f) ? 1.f / av : 0.f;
    }
    const int km1 = a.chunks - 1;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        float v = 0.f;
        if constexpr (!SUMMARY) {
            if (n0 + j < Nr) {
                if (seg == 0) {
                    // several segments: the carry pass's copy of h0 (h_last may alias h0)
                    const float* h0 = a.chunks > 1 ? a.start0 : a.h0;
                    if (h0) v = h0[((int64_t)b * a.Dn + dd) * Nr + n0 + j];
                } else {
                    v = a.agg[(((int64_t)b * km1 + (seg - 1)) * Nr + n0 + j) * a.Dn + dd];
                }
            }
        }
        h[j] = v;
    }
    const float bias = a.bias ? a.bias[dd] : 0.f;
    const float Dd = a.D ? a.D[dd] : 0.f;
    const bool has_z = a.z != nullptr;
    const bool use_sp = a.softplus != 0;

    const int64_t t0 = (int64_t)seg * a.chunk_len;
    const int64_t t1 = min(a.L, t0 + a.chunk_len);
    const int nblocks = (int)((t1 - t0 + TB - 1) / TB);
    const int64_t row0 = (int64_t)b * a.L;  // first row of this batch element

    // Byte offset of this thread's j-th element inside a block: row
    // (w*J + j), channel d.  Tail channels point past every buffer.
    const uint32_t rowb = (uint32_t)a.Dn * R::kSize;
    const uint32_t off0 = dvalid ? ((uint32_t)(w * J) * rowb + (uint32_t)d * R::kSize) : kOutOfRange;
    // Valid rows of the block starting at tb (0 past the segment end, so a
    // prefetch of a block that does not exist reads only zeros).
    auto block_rows = [&](int64_t tb) -> uint32_t {
        return (uint32_t)max((int64_t)0, min((int64_t)TB, t1 - tb));
    };
    auto block_base = [&](const void* p, int64_t tb) -> const void* {
        return static_cast<const char*>(p) + (row0 + tb) * (int64_t)rowb;
    };
    // Prepared B/C rows: 2N floats per timestep.  Lane l reads state
    // n0 + (l mod NS) of B (and, N floats further, of C).
    constexpr uint32_t kBCRow = 2u * N * 4u;
    const uint32_t bcoff = (uint32_t)(n0 + (lane & (NS - 1))) * 4u;

    // Register double buffer of the raw inputs of one block.
    RT ru[2][J], rd[2][J], rz[2][J];
    float vb[2][TB], vc[2][TB];
    auto load_block = [&](int buf, int64_t tb) __attribute__((always_inline)) {
        const uint32_t nr = block_rows(tb);
        const auto rU = make_rsrc(block_base(a.u, tb), nr * rowb);
        const auto rD = make_rsrc(block_base(a.delta, tb), nr * rowb);
        const auto rZ = make_rsrc(has_z ? block_base(a.z, tb) : a.u, has_z ? nr * rowb : 0u);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint32_t off = off0 + (uint32_t)j * rowb;
            ru[buf][j] = R::load(rU, off);
            rd[buf][j] = R::load(rD, off);
            if constexpr (!SUMMARY) rz[buf][j] = R::load(rZ, off);
        }
        const auto rBC = make_rsrc(a.bcw + (row0 + tb) * (2 * N), nr * kBCRow);
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) {
            vb[buf][tt] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rBC, (uint32_t)tt * kBCRow + bcoff, 0, 0));
            if constexpr (!SUMMARY)
                vc[buf][tt] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                    rBC, (uint32_t)tt * kBCRow + (uint32_t)N * 4u + bcoff, 0, 0));
        }
    };

    float uf[J];                      // widened u kept from phase A to phase C
    float s_sum = 0.f, s_comp = 0.f;  // Kahan sum of dt (wave 0, SUMMARY)

    // One timestep of this wave's NS states.
    auto step = [&](int cur, int tt, float2 dx, float vbt, float vct) __attribute__((always_inline)) {
        static_for(
            [&](auto jc) {
                constexpr int j = decltype(jc)::value;
                const float arg = dx.x * A2[j];
                float abar = 0.f, bx = 0.f;
                if constexpr (BIL) {
                    const float r = bilinear_r(arg);
                    const float ub = row_bcast<j>(vbt) * dx.y;  // B * dt*u
                    if constexpr (PROD) {
                        abar = fmaf(2.f, r, -1.f);
                        bx = ub * r;
                    } else {
                        // (2r - 1) h + r (B dt u) = r (2h + B dt u) - h: two fma
                        h[j] = fmaf(r, fmaf(2.f, h[j], ub), -h[j]);
                    }
                } else {
                    abar = hw_exp2(arg);
                    const float bu = row_bcast<j>(vbt) * dx.y;  // B*x (Euler) or B*u (ZOH)
                    if constexpr (ZOH)
                        bx = zoh_factor(dx.x, arg, abar, invA[j]) * bu;
                    else
                        bx = bu;
                }
                if constexpr (!BIL || PROD) h[j] = fmaf(abar, h[j], bx);
                if constexpr (PROD) P[j] *= abar;
                // With a block's steps unrolled, the scheduler would start the
                // exponentials of many steps ahead of their updates and spill.
                if constexpr (j % 8 == 7) __builtin_amdgcn_sched_barrier(0);
            },
            std::make_integer_sequence<int, NS>{});
        if constexpr (!SUMMARY) {
            s_y[cur][w][tt][lane] = DppReadout<NS>::run(vct, h);
        } else if constexpr (!PROD) {
            if (w == 0) {
                const float yk = dx.x - s_comp;
                const float tk = s_sum + yk;
                s_comp = (tk - s_sum) - yk;
                s_sum = tk;
            }
        }
    };

    // One block of TB timesteps; CUR (the buffer parity) is a compile-time
    // constant so the register double buffer is indexed statically.
    auto do_block = [&](auto cur_c, int blk) __attribute__((always_inline)) {
        constexpr int cur = decltype(cur_c)::value;
        const int64_t tb = t0 + (int64_t)blk * TB;
        const int cnt = (int)min((int64_t)TB, t1 - tb);
        load_block(cur ^ 1, tb + TB);  // unconditional: past the end it reads zeros

        // ---- phase A: per-element activations into LDS ----
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int tl = w * J + j;
            const float uv = R::widen(ru[cur][j]);
            const float v = R::widen(rd[cur][j]) + bias;
            const float sp = softplus_f(v);
            const float dt = use_sp ? sp : v;
            uf[j] = uv;
            s_dx[cur][tl][lane] = ZOH ? make_float2(dt, uv) : make_float2(dt, dt * uv);
        }
        __syncthreads();

        // ---- phase B: the recurrences of this wave's states ----
        if (cnt == TB) {
            float2 dxr[TB];
#pragma unroll
            for (int tt = 0; tt < TB; ++tt) dxr[tt] = s_dx[cur][tt][lane];
#pragma unroll
            for (int tt = 0; tt < TB; ++tt) step(cur, tt, dxr[tt], vb[cur][tt], vc[cur][tt]);
        } else {
#pragma unroll
            for (int tt = 0; tt < TB; ++tt)
                if (tt < cnt) step(cur, tt, s_dx[cur][tt][lane], vb[cur][tt], vc[cur][tt]);
        }

        // ---- phase C: combine partial readouts, skip term, gate, store ----
        if constexpr (!SUMMARY) {
            __syncthreads();
            float yp[J][S];
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int s = 0; s < S; ++s) yp[j][s] = s_y[cur][s][w * J + j][lane];
            const auto rY = make_rsrc(block_base(a.y, tb), (uint32_t)cnt * rowb);
#pragma unroll
            for (int j = 0; j < J; ++j) {
                float y = 0.f;
#pragma unroll
                for (int s = 0; s < S; ++s) y += yp[j][s];
                y = fmaf(Dd, uf[j], y);
                const float g = silu_f(R::widen(rz[cur][j]));
                y *= has_z ? g : 1.f;
                R::store(rY, off0 + (uint32_t)j * rowb, y);
            }
        }
    };

    load_block(0, t0);
    int blk = 0;
    for (; blk + 1 < nblocks; blk += 2) {
        do_block(std::integral_constant<int, 0>{}, blk);
        do_block(std::integral_constant<int, 1>{}, blk + 1);
    }
    if (blk < nblocks) do_block(std::integral_constant<int, 0>{}, blk);

    if (!dvalid) return;
    if constexpr (SUMMARY) {
        const int64_t base = (int64_t)b * km1 + seg;
#pragma unroll
        for (int j = 0; j < NS; ++j)
            if (n0 + j < Nr) a.agg[(base * Nr + n0 + j) * a.Dn + d] = h[j];
        if constexpr (PROD) {
#pragma unroll
            for (int j = 0; j < NS; ++j)
                if (n0 + j < Nr) a.prod[(base * Nr + n0 + j) * a.Dn + d] = P[j];
        } else {
            if (w == 0) a.sdt[base * a.Dn + d] = s_sum;
        }
    } else {
        if (seg == a.chunks - 1 && a.h_last) {
#pragma unroll
            for (int j = 0; j < NS; ++j)
                if (n0 + j < Nr) a.h_last[((int64_t)b * a.Dn + d) * Nr + n0 + j] = h[j];
        }
    }
}

// Widen B and C to fp32 rows [b][t][B_t row | C_t row] for the DPP delivery,
// each row np wide (np = the kernel's states; entries past d_state are 0).
// One thread per output float: reads and writes are both contiguous.
template <bool BF16>
__global__ void __launch_bounds__(256) bc_prepare(ScanArgs a, int np) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = i / (2 * np);
    if (row >= (int64_t)a.batch * a.L) return;
    const int k = (int)(i - row * 2 * np);
    const int n = k < np ? k : k - np;
    a.bcw[i] = n >= a.N ? 0.f : k < np ? ld<BF16>(a.B, row * a.N + n) : ld<BF16>(a.C, row * a.N + n);
}

template <int NS, int S, int TB, bool BF16, int DISC>
hipError_t launch_tiles(const Plan& p, const ScanArgs& a, hipStream_t s) {
    const dim3 block(64 * S);
    hipError_t e = launch_bc_prepare(a, NS * S, BF16, s);
    if (e != hipSuccess) return e;
    if (p.chunks > 1) {
        {
            ProfScope ps(s, kPhaseSummary);
            hipLaunchKernelGGL((scan_tile<NS, S, TB, BF16, DISC, true>),
                               dim3(p.tiles, p.chunks - 1, a.batch), block, 0, s, a);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_carry(a, s);
        if (e != hipSuccess) return e;
    }
    {
        ProfScope ps(s, kPhaseMain);
        hipLaunchKernelGGL((scan_tile<NS, S, TB, BF16, DISC, false>),
                           dim3(p.tiles, p.chunks, a.batch), block, 0, s, a);
    }
    return hipGetLastError();
}

template <bool BF16, int DISC>
hipError_t dispatch_io(const Plan& p, const ScanArgs& a, hipStream_t s) {
    constexpr int TB = 16;
    if (p.waves == 4) {
        switch (p.ns) {
            case 2: return launch_tiles<2, 4, TB, BF16, DISC>(p, a, s);
            case 4: return launch_tiles<4, 4, TB, BF16, DISC>(p, a, s);
            case 8: return launch_tiles<8, 4, TB, BF16, DISC>(p, a, s);
            case 16: return launch_tiles<16, 4, TB, BF16, DISC>(p, a, s);
            default: break;
        }
    } else if (p.waves == 8) {
        switch (p.ns) {
            case 2: return launch_tiles<2, 8, TB, BF16, DISC>(p, a, s);
            case 8: return launch_tiles<8, 8, TB, BF16, DISC>(p, a, s);
            case 16: return launch_tiles<16, 8, TB, BF16, DISC>(p, a, s);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bc_prepare(const ScanArgs& a, int np, bool bf16, hipStream_t s) {
    const int64_t total = (int64_t)a.batch * a.L * 2 * np;
    const dim3 grid((unsigned)((total + 255) / 256));
    ProfScope ps(s, kPhasePrep);
    if (bf16)
        hipLaunchKernelGGL((bc_prepare<true>), grid, dim3(256), 0, s, a, np);
    else
        hipLaunchKernelGGL((bc_prepare<false>), grid, dim3(256), 0, s, a, np);
    return hipGetLastError();
}

bool tile_variant_exists(int ns, int waves) {
    if (waves == 4) return ns == 2 || ns == 4 || ns == 8 || ns == 16;
    if (waves == 8) return ns == 2 || ns == 8 || ns == 16;
    return false;
}

template <bool BF16>
hipError_t dispatch_disc(const Plan& p, const ScanArgs& a, int disc, hipStream_t s) {
    switch (disc) {
        case kEuler: return dispatch_io<BF16, kEuler>(p, a, s);
        case kZoh: return dispatch_io<BF16, kZoh>(p, a, s);
        case kBilinear: return dispatch_io<BF16, kBilinear>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_scan_tiles(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                             hipStream_t s) {
    return bf16 ? dispatch_disc<true>(p, a, disc, s) : dispatch_disc<false>(p, a, disc, s);
}

}  // namespace msscan
