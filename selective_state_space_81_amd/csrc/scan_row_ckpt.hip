// scan_row_ckpt.hip -- the forward pass that saves the backward's block-state
// checkpoints (ms_scan_fwd_checkpoint): the row kernel with one DPP row per
// channel (d_state 9..16), io tiles moved whole, the sequence in one segment,
// storing the state before every 16-step block beside its usual outputs.
#include "scan_row_kernel.h"

namespace msscan {
namespace {

template <bool BF16, int DISC, bool SP>
hipError_t launch_ckpt_rows(const Plan& p, const ScanArgs& a, hipStream_t s) {
    ProfScope ps(s, kPhaseMain);
    hipLaunchKernelGGL((scan_row<BF16, DISC, SP, false, true, 1, 1, true>),
                       dim3((unsigned)a.batch * (unsigned)p.tiles), dim3(64 * kRowWaves), 0, s, a);
    return hipGetLastError();
}

template <bool BF16, int DISC>
hipError_t launch_ckpt_d(const Plan& p, const ScanArgs& a, hipStream_t s) {
    return a.softplus ? launch_ckpt_rows<BF16, DISC, true>(p, a, s)
                      : launch_ckpt_rows<BF16, DISC, false>(p, a, s);
}

template <bool BF16>
hipError_t launch_ckpt_b(const Plan& p, const ScanArgs& a, int disc, hipStream_t s) {
    switch (disc) {
        case kEuler: return launch_ckpt_d<BF16, kEuler>(p, a, s);
        case kZoh: return launch_ckpt_d<BF16, kZoh>(p, a, s);
        case kBilinear: return launch_ckpt_d<BF16, kBilinear>(p, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_scan_rows_ckpt(const Plan& p, const ScanArgs& a, bool bf16, int disc,
                                 hipStream_t s) {
    if (p.tile_path != 3 || p.rows != 1 || p.ns != kRT || p.chunks != 1 || a.chunks != 1 ||
        a.tiles != p.tiles || p.waves != kRowWaves || a.N < 1 || a.N > kRT || !a.agg ||
        a.Dn % (bf16 ? 8 : 4) != 0)
        return hipErrorInvalidValue;
    return bf16 ? launch_ckpt_b<true>(p, a, disc, s) : launch_ckpt_b<false>(p, a, disc, s);
}

}  // namespace msscan
