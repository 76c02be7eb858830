// scan_row_wide.hip -- launchers of the row kernel (scan_row_kernel.h) with
// several DPP rows per channel: d_state 17..32 on 2 rows, 33..64 on 4, and
// 65..128 on 4 rows with 2 states per lane.  The planner takes this path only
// when batch x d_inner fills the chip without cutting the sequence and the
// io tiles move whole (d_inner a multiple of 8 for bf16 on 2 rows, else of
// 4), so the sequence is one segment here.
#include "scan_row_kernel.h"

namespace msscan {
namespace {

template <bool BF16, int DISC, bool SP, int RPC, int SPL>
hipError_t launch_wide_rows(const Plan& p, const ScanArgs& a, hipStream_t s) {
    // one segment: the planner never cuts the sequence on this path
    if (p.chunks != 1) return hipErrorInvalidValue;
    const unsigned per_seg = (unsigned)a.batch * (unsigned)p.tiles;
    ProfScope ps(s, kPhaseMain);
    hipLaunchKernelGGL((scan_row<BF16, DISC, SP, false, true, RPC, SPL>), dim3(per_seg),
                       dim3(64 * kRowWaves), 0, s, a);
    return hipGetLastError();
}

template <bool BF16, int DISC, bool SP>
hipError_t launch_wide_shape(const Plan& p, const ScanArgs& a, int rpc, int spl, hipStream_t s) {
    if (rpc == 2 && spl == 1) return launch_wide_rows<BF16, DISC, SP, 2, 1>(p, a, s);
    if (rpc == 4 && spl == 1) return launch_wide_rows<BF16, DISC, SP, 4, 1>(p, a, s);
    if (rpc == 4 && spl == 2) return launch_wide_rows<BF16, DISC, SP, 4, 2>(p, a, s);
    return hipErrorInvalidValue;
}

template <bool BF16, int DISC>
hipError_t launch_wide_d(const Plan& p, const ScanArgs& a, int rpc, int spl, hipStream_t s) {
    return a.softplus ? launch_wide_shape<BF16, DISC, true>(p, a, rpc, spl, s)
                      : launch_wide_shape<BF16, DISC, false>(p, a, rpc, spl, s);
}

template <bool BF16>
hipError_t launch_wide_b(const Plan& p, const ScanArgs& a, int disc, int rpc, int spl,
                         hipStream_t s) {
    switch (disc) {
        case kEuler: return launch_wide_d<BF16, kEuler>(p, a, rpc, spl, s);
        case kZoh: return launch_wide_d<BF16, kZoh>(p, a, rpc, spl, s);
        case kBilinear: return launch_wide_d<BF16, kBilinear>(p, a, rpc, spl, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scan_rows_wide(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                 hipStream_t s) {
    const int rpc = p.rows;
    const int spl = rpc > 0 ? p.ns / (kRT * rpc) : 0;
    // whole io tiles only (chunks of kRowCh / rpc channels, at most 16 bytes),
    // and the states must fit the channel's rows
    const int cw = bf16 ? (rpc == 4 ? 4 : 8) : 4;
    if (rpc < 2 || a.Dn % cw != 0 || p.ns != kRT * rpc * spl || a.N < 1 || a.N > p.ns)
        return hipErrorInvalidValue;
    return bf16 ? launch_wide_b<true>(p, a, disc, rpc, spl, s)
                : launch_wide_b<false>(p, a, disc, rpc, spl, s);
}

}  // namespace msscan
