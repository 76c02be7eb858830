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
//      widen u / delta (/ z), dt = softplus(delta + bias), x = dt*u, and the
//      block's B_t / C_t rows widened to fp32 -- all into LDS.  Each element's
//      activations are computed exactly once, not once per state.
//   B  per wave: for each timestep, its NS states advance and their partial
//      readout sum_n C*h goes to LDS.  dt, x, B_t, C_t are read from LDS; the
//      B/C reads are wave-uniform broadcasts.
//   C  per element again: y = sum of the S partials + D*u, times silu(z),
//      rounded to the io type and stored (coalesced rows).
// The next block's global loads are issued before phase A of the current one
// (register double buffering), and the LDS buffers alternate between blocks,
// so each block needs two barriers.
//
// With several segments, a summary variant of the same kernel (no readout,
// SUMMARY = true) computes each segment's end state from zero and its
// compensated sum of dt; the generic carry pass composes them in order (the
// scan is a composition of affine maps, jsqmd page section 3.4) and the main
// variant starts every segment from its true state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "msscan_internal.h"

namespace msscan {
namespace {

using namespace dev;

// Buffer-resource io.  A block's rows of u / delta / z / y are addressed
// through a buffer descriptor whose size ends at the block's last valid row,
// so reads past it return 0 and writes past it are dropped by the hardware;
// tail channels get an offset beyond any size.  No branch is needed for
// ragged sequence ends or d_inner tails.
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

template <int NS, int S, int TB, bool BF16, bool ZOH, bool SUMMARY>
__global__ void __launch_bounds__(64 * S) scan_tile(ScanArgs a) {
    constexpr int N = NS * S;
    constexpr int NT = 64 * S;
    constexpr int J = TB / S;                    // timesteps per thread in phases A/C
    constexpr int BCN = (TB * N + NT - 1) / NT;  // B (and C) tile elements per thread
    static_assert(TB % S == 0, "TB must be a multiple of S");
    static_assert(NS % 2 == 0, "the B/C slice of a wave is read in 16-byte pieces");
    using R = Io<BF16>;
    using RT = typename R::T;

    __shared__ float2 s_dx[2][TB][64];           // (dt, x) Euler; (dt, u) ZOH
    // B_t / C_t of the block widened to fp32, grouped per wave: for timestep
    // tt and wave w, the NS values of B then the NS values of C.
    __shared__ __attribute__((aligned(16))) float s_bc[2][TB][S][2][NS];
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

    float A2[NS], invA[NS], h[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const float av = a.A[(int64_t)dd * N + n0 + j];
        A2[j] = av * kLog2e;
        if constexpr (ZOH) invA[j] = (av != 0.f) ? 1.f / av : 0.f;
    }
    const int km1 = a.chunks - 1;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        float v = 0.f;
        if constexpr (!SUMMARY) {
            if (seg == 0) {
                if (a.h0) v = a.h0[((int64_t)b * a.Dn + dd) * N + n0 + j];
            } else {
                v = a.agg[(((int64_t)b * km1 + (seg - 1)) * N + n0 + j) * a.Dn + dd];
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
    auto block_bytes = [&](int64_t tb) -> uint32_t {
        return (uint32_t)min((int64_t)TB, t1 - tb) * rowb;
    };
    auto block_base = [&](const void* p, int64_t tb) -> const void* {
        return static_cast<const char*>(p) + (row0 + tb) * (int64_t)rowb;
    };

    // Register double buffer of the raw inputs of one block.
    RT ru[2][J], rd[2][J], rz[2][J], rb[2][BCN], rc[2][BCN];
    auto load_block = [&](int buf, int64_t tb) {
        {
            const uint32_t nbc = (uint32_t)min((int64_t)TB, t1 - tb) * (uint32_t)(N * R::kSize);
            const auto rB = make_rsrc(static_cast<const char*>(a.B) + (row0 + tb) * N * R::kSize, nbc);
            const auto rC = make_rsrc(static_cast<const char*>(a.C) + (row0 + tb) * N * R::kSize, nbc);
#pragma unroll
            for (int k = 0; k < BCN; ++k) {
                const int i = tid + k * NT;
                const uint32_t off = (i < TB * N) ? (uint32_t)i * R::kSize : kOutOfRange;
                rb[buf][k] = R::load(rB, off);
                if constexpr (!SUMMARY) rc[buf][k] = R::load(rC, off);
            }
        }
        const uint32_t nb = block_bytes(tb);
        const auto rU = make_rsrc(block_base(a.u, tb), nb);
        const auto rD = make_rsrc(block_base(a.delta, tb), nb);
        const auto rZ = make_rsrc(has_z ? block_base(a.z, tb) : a.u, has_z ? nb : 0u);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const uint32_t off = off0 + (uint32_t)j * rowb;
            ru[buf][j] = R::load(rU, off);
            rd[buf][j] = R::load(rD, off);
            if constexpr (!SUMMARY) rz[buf][j] = R::load(rZ, off);
        }
    };

    float uf[J];                      // widened u kept from phase A to phase C
    float s_sum = 0.f, s_comp = 0.f;  // Kahan sum of dt (wave 0, SUMMARY)

    // One timestep of this wave's NS states; B and C come from LDS.
    auto step = [&](int cur, int tt, float2 dx) {
        float bc[2 * NS];
#pragma unroll
        for (int q = 0; q < 2 * NS; q += 4)
            *reinterpret_cast<float4*>(&bc[q]) =
                *reinterpret_cast<const float4*>(&s_bc[cur][tt][w][0][0] + q);
        float y = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const float arg = dx.x * A2[j];
            const float abar = hw_exp2(arg);
            const float bn = bc[j];
            float bx;
            if constexpr (ZOH)
                bx = zoh_factor(dx.x, arg * kLn2, abar, invA[j]) * (dx.y * bn);
            else
                bx = dx.y * bn;
            h[j] = fmaf(abar, h[j], bx);
            if constexpr (!SUMMARY) y = fmaf(bc[NS + j], h[j], y);
        }
        if constexpr (!SUMMARY) s_y[cur][w][tt][lane] = y;
        if constexpr (SUMMARY) {
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
    auto do_block = [&](auto cur_c, int blk) {
        constexpr int cur = decltype(cur_c)::value;
        const int64_t tb = t0 + (int64_t)blk * TB;
        const int cnt = (int)min((int64_t)TB, t1 - tb);
        if (blk + 1 < nblocks) load_block(cur ^ 1, tb + TB);

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
#pragma unroll
        for (int k = 0; k < BCN; ++k) {
            const int i = tid + k * NT;
            if (i < TB * N) {
                const int tt = i / N, n = i % N;
                s_bc[cur][tt][n / NS][0][n % NS] = R::widen(rb[cur][k]);
                if constexpr (!SUMMARY) s_bc[cur][tt][n / NS][1][n % NS] = R::widen(rc[cur][k]);
            }
        }
        __syncthreads();

        // ---- phase B: the recurrences of this wave's states ----
        if (cnt == TB) {
            float2 dxr[TB];
#pragma unroll
            for (int tt = 0; tt < TB; ++tt) dxr[tt] = s_dx[cur][tt][lane];
#pragma unroll
            for (int tt = 0; tt < TB; ++tt) step(cur, tt, dxr[tt]);
        } else {
            for (int tt = 0; tt < cnt; ++tt) step(cur, tt, s_dx[cur][tt][lane]);
        }

        // ---- phase C: combine partial readouts, skip term, gate, store ----
        if constexpr (!SUMMARY) {
            __syncthreads();
            float yp[J][S];
#pragma unroll
            for (int j = 0; j < J; ++j)
#pragma unroll
                for (int s = 0; s < S; ++s) yp[j][s] = s_y[cur][s][w * J + j][lane];
            const auto rY = make_rsrc(block_base(a.y, tb), block_bytes(tb));
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

    if (nblocks > 0) load_block(0, t0);
    for (int blk = 0; blk < nblocks; blk += 2) {
        do_block(std::integral_constant<int, 0>{}, blk);
        if (blk + 1 < nblocks) do_block(std::integral_constant<int, 1>{}, blk + 1);
    }

    if (!dvalid) return;
    if constexpr (SUMMARY) {
        const int64_t base = (int64_t)b * km1 + seg;
#pragma unroll
        for (int j = 0; j < NS; ++j) a.agg[(base * N + n0 + j) * a.Dn + d] = h[j];
        if (w == 0) a.sdt[base * a.Dn + d] = s_sum;
    } else {
        if (seg == a.chunks - 1 && a.h_last) {
#pragma unroll
            for (int j = 0; j < NS; ++j) a.h_last[((int64_t)b * a.Dn + d) * N + n0 + j] = h[j];
        }
    }
}

template <int NS, int S, int TB, bool BF16, bool ZOH>
hipError_t launch_tiles(const Plan& p, const ScanArgs& a, hipStream_t s) {
    const dim3 block(64 * S);
    if (p.chunks > 1) {
        hipLaunchKernelGGL((scan_tile<NS, S, TB, BF16, ZOH, true>),
                           dim3(p.tiles, p.chunks - 1, a.batch), block, 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_carry(a, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((scan_tile<NS, S, TB, BF16, ZOH, false>), dim3(p.tiles, p.chunks, a.batch),
                       block, 0, s, a);
    return hipGetLastError();
}

template <bool BF16, bool ZOH>
hipError_t dispatch_io(const Plan& p, const ScanArgs& a, hipStream_t s) {
    constexpr int TB = 16;
    if (p.waves == 4) {
        switch (p.ns) {
            case 2: return launch_tiles<2, 4, TB, BF16, ZOH>(p, a, s);
            case 4: return launch_tiles<4, 4, TB, BF16, ZOH>(p, a, s);
            case 8: return launch_tiles<8, 4, TB, BF16, ZOH>(p, a, s);
            case 16: return launch_tiles<16, 4, TB, BF16, ZOH>(p, a, s);
            case 32: return launch_tiles<32, 4, TB, BF16, ZOH>(p, a, s);
            default: break;
        }
    } else if (p.waves == 8) {
        switch (p.ns) {
            case 2: return launch_tiles<2, 8, TB, BF16, ZOH>(p, a, s);
            case 8: return launch_tiles<8, 8, TB, BF16, ZOH>(p, a, s);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool tile_variant_exists(int ns, int waves) {
    if (waves == 4) return ns == 2 || ns == 4 || ns == 8 || ns == 16 || ns == 32;
    if (waves == 8) return ns == 2 || ns == 8;
    return false;
}

hipError_t launch_scan_tiles(const Plan& p, const ScanArgs& a, bool bf16, bool zoh,
                             hipStream_t s) {
    if (bf16) return zoh ? dispatch_io<true, true>(p, a, s) : dispatch_io<true, false>(p, a, s);
    return zoh ? dispatch_io<false, true>(p, a, s) : dispatch_io<false, false>(p, a, s);
}

}  // namespace msscan
