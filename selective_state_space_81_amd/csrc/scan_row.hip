// scan_row.hip -- launchers of the row kernel (scan_row_kernel.h) with one
// DPP row per channel (d_state 9..16), and the row path's entry point, which
// hands channels of more states to scan_row_wide.hip.
#include "scan_row_kernel.h"

namespace msscan {
namespace {

template <bool BF16, int DISC, bool SP, bool COOP>
hipError_t launch_rows_c(const Plan& p, const ScanArgs& a, hipStream_t s) {
    const unsigned per_seg = (unsigned)a.batch * (unsigned)p.tiles;
    if (p.chunks > 1) {
        {
            ProfScope ps(s, kPhaseSummary);
            hipLaunchKernelGGL((scan_row<BF16, DISC, SP, true, COOP, 1, 1>),
                               dim3(per_seg * (p.chunks - 1)), dim3(64 * kRowWaves), 0, s, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_carry(a, s);
        if (e != hipSuccess) return e;
    }
    {
        ProfScope ps(s, kPhaseMain);
        hipLaunchKernelGGL((scan_row<BF16, DISC, SP, false, COOP, 1, 1>), dim3(per_seg * p.chunks),
                           dim3(64 * kRowWaves), 0, s, a);
    }
    return hipGetLastError();
}

// Tiles move through LDS with 16-byte accesses (COOP) when every 16-byte
// chunk of a row is wholly inside or outside it; else one element per lane.
template <bool BF16, int DISC, bool SP>
hipError_t launch_rows_t(const Plan& p, const ScanArgs& a, hipStream_t s) {
    if (a.Dn % (BF16 ? 8 : 4) == 0) return launch_rows_c<BF16, DISC, SP, true>(p, a, s);
    return launch_rows_c<BF16, DISC, SP, false>(p, a, s);
}

template <bool BF16, int DISC>
hipError_t launch_rows_d(const Plan& p, const ScanArgs& a, hipStream_t s) {
    return a.softplus ? launch_rows_t<BF16, DISC, true>(p, a, s)
                      : launch_rows_t<BF16, DISC, false>(p, a, s);
}

template <bool BF16>
hipError_t launch_rows_b(const Plan& p, const ScanArgs& a, int disc, hipStream_t s) {
    switch (disc) {
        case kEuler: return launch_rows_d<BF16, kEuler>(p, a, s);
        case kZoh: return launch_rows_d<BF16, kZoh>(p, a, s);
        case kBilinear: return launch_rows_d<BF16, kBilinear>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scan_rows(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                            hipStream_t s) {
    if (a.tiles != p.tiles || p.waves != kRowWaves) return hipErrorInvalidValue;
    if (p.rows > 1) return launch_scan_rows_wide(p, a, bf16, disc, s);
    if (a.N < 1 || a.N > kRT || p.ns != kRT) return hipErrorInvalidValue;
    return bf16 ? launch_rows_b<true>(p, a, disc, s) : launch_rows_b<false>(p, a, disc, s);
}

}  // namespace msscan
