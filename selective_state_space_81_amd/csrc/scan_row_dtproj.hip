// scan_row_dtproj.hip -- launchers of the row kernel (scan_row_kernel.h) with
// the step projection fused in (ms_scan_fwd_dtproj at d_state 9..128): one,
// two or four DPP rows per channel as in the plain forward, io tiles moved
// whole, the delta tile formed on the matrix cores from the low-rank input
// (dtproj_frag.h).
#include "scan_row_kernel.h"

namespace msscan {
namespace {

template <bool BF16, int DISC, bool SP>
hipError_t launch_dtp_rows(const Plan& p, const ScanArgs& a, hipStream_t s) {
    const unsigned per_seg = (unsigned)a.batch * (unsigned)p.tiles;
    if (p.chunks > 1) {
        {
            ProfScope ps(s, kPhaseSummary);
            hipLaunchKernelGGL((scan_row<BF16, DISC, SP, true, true, 1, 1, false, true>),
                               dim3(per_seg * (p.chunks - 1)), dim3(64 * kRowWaves), 0, s, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_carry(a, s);
        if (e != hipSuccess) return e;
    }
    {
        ProfScope ps(s, kPhaseMain);
        hipLaunchKernelGGL((scan_row<BF16, DISC, SP, false, true, 1, 1, false, true>),
                           dim3(per_seg * p.chunks), dim3(64 * kRowWaves), 0, s, a);
    }
    return hipGetLastError();
}

// Several rows per channel: the planner never cuts the sequence there.
template <bool BF16, int DISC, bool SP, int RPC, int SPL>
hipError_t launch_dtp_wide(const Plan& p, const ScanArgs& a, hipStream_t s) {
    if (p.chunks != 1) return hipErrorInvalidValue;
    ProfScope ps(s, kPhaseMain);
    hipLaunchKernelGGL((scan_row<BF16, DISC, SP, false, true, RPC, SPL, false, true>),
                       dim3((unsigned)a.batch * (unsigned)p.tiles), dim3(64 * kRowWaves), 0, s, a);
    return hipGetLastError();
}

template <bool BF16, int DISC, bool SP>
hipError_t launch_dtp_shape(const Plan& p, const ScanArgs& a, hipStream_t s) {
    const int spl = p.ns / (kRT * p.rows);
    if (p.rows == 1 && spl == 1) return launch_dtp_rows<BF16, DISC, SP>(p, a, s);
    if (p.rows == 2 && spl == 1) return launch_dtp_wide<BF16, DISC, SP, 2, 1>(p, a, s);
    if (p.rows == 4 && spl == 1) return launch_dtp_wide<BF16, DISC, SP, 4, 1>(p, a, s);
    if (p.rows == 4 && spl == 2) return launch_dtp_wide<BF16, DISC, SP, 4, 2>(p, a, s);
    return hipErrorInvalidValue;
}

template <bool BF16, int DISC>
hipError_t launch_dtp_d(const Plan& p, const ScanArgs& a, hipStream_t s) {
    return a.softplus ? launch_dtp_shape<BF16, DISC, true>(p, a, s)
                      : launch_dtp_shape<BF16, DISC, false>(p, a, s);
}

template <bool BF16>
hipError_t launch_dtp_b(const Plan& p, const ScanArgs& a, int disc, hipStream_t s) {
    switch (disc) {
        case kEuler: return launch_dtp_d<BF16, kEuler>(p, a, s);
        case kZoh: return launch_dtp_d<BF16, kZoh>(p, a, s);
        case kBilinear: return launch_dtp_d<BF16, kBilinear>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scan_rows_dtproj(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                   hipStream_t s) {
    // whole io tiles: chunks of kRowCh / rows channels, at most 16 bytes
    const int cw = bf16 ? (p.rows == 4 ? 4 : 8) : 4;
    if (p.tile_path != 3 || p.rows < 1 || a.tiles != p.tiles || a.N < 1 || a.N > p.ns ||
        a.rank < 1 || a.rank > kMaxRank || a.Dn % cw != 0)
        return hipErrorInvalidValue;
    return bf16 ? launch_dtp_b<true>(p, a, disc, s) : launch_dtp_b<false>(p, a, disc, s);
}

}  // namespace msscan
