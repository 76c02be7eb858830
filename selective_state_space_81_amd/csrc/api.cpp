// api.cpp -- the C ABI of libmsscan: argument validation, work planning and
// dispatch to the HIP kernels.  Declarations and the full contract are in
// include/msscan.h.
#include "../../include/msscan.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "device_common.h"
#include "msscan_internal.h"

namespace {

thread_local char g_err[512] = "";

ms_status fail(ms_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u); }

constexpr int kMaxState = 128;
constexpr int64_t kMaxLen = 0x7fffffffLL;

ms_status check_dims(const ms_dims* d) {
    if (!d) return fail(MS_ERR_NULL, "dims is NULL");
    if (d->batch < 1) return fail(MS_ERR_SHAPE, "batch=%d must be >= 1", d->batch);
    if (d->seqlen < 1 || d->seqlen > kMaxLen)
        return fail(MS_ERR_SHAPE, "seqlen=%lld must be in [1, 2^31-1]", (long long)d->seqlen);
    if (d->d_inner < 1) return fail(MS_ERR_SHAPE, "d_inner=%d must be >= 1", d->d_inner);
    if (d->d_state < 1 || d->d_state > kMaxState)
        return fail(MS_ERR_SHAPE, "d_state=%d must be in [1, %d]", d->d_state, kMaxState);
    if (d->io != MS_F32 && d->io != MS_BF16)
        return fail(MS_ERR_DTYPE, "io=%d is not MS_F32 (0) or MS_BF16 (1)", d->io);
    // grid limits: tiles and batch go to grid y/z
    if ((d->d_inner + 63) / 64 > 65535 || d->batch > 65535)
        return fail(MS_ERR_UNSUPPORTED, "d_inner/64 and batch must be <= 65535");
    // every buffer and workspace size (at most tens of bytes per element and
    // state) then stays far inside size_t
    const double states = (double)d->batch * (double)d->seqlen * (double)d->d_inner * d->d_state;
    if (states > 0x1p56)
        return fail(MS_ERR_SHAPE, "batch x seqlen x d_inner x d_state = %.3g exceeds 2^56",
                    states);
    return MS_OK;
}

constexpr uint32_t kKnownFlags = MS_SOFTPLUS | MS_ZOH | MS_BILINEAR;

ms_status check_flags(uint32_t flags) {
    if (flags & ~kKnownFlags)
        return fail(MS_ERR_FLAGS, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if ((flags & MS_ZOH) && (flags & MS_BILINEAR))
        return fail(MS_ERR_FLAGS, "MS_ZOH and MS_BILINEAR are exclusive");
    return MS_OK;
}

// Discretisation of the flags (kEuler / kZoh / kBilinear of the kernels).
int disc_of(uint32_t flags) {
    return (flags & MS_BILINEAR) ? msscan::dev::kBilinear
                                 : ((flags & MS_ZOH) ? msscan::dev::kZoh : msscan::dev::kEuler);
}

// Paths, in the order they are tried:
//   row path (below): a channel's states across the lanes of 1, 2 or 4 DPP
//     rows -- d_state 9..16 always, 17..128 when batch x d_inner alone fills
//     the chip (Euler at 33..64 excepted);
//   lane path (d_state 8, 16, 32; 64 with Euler): one wave per workgroup,
//     all states of a channel in one lane;
//   tile path (d_state 128, 64 with ZOH or bilinear): several waves split
//     d_state and share per-element work through LDS.
// The lane and tile paths map one 64-channel tile of one batch row to a
// workgroup and cut the sequence into segments until about kTargetWaves
// waves exist (many waves per CU keep the VALU issuing; a segment after the
// first costs a summary pass over it, so segments are not cut shorter than
// kMinSegment).
#ifndef MSSCAN_TILE_WAVES
#define MSSCAN_TILE_WAVES 4
#endif
#ifndef MSSCAN_TARGET_WAVES
#define MSSCAN_TARGET_WAVES 16384
#endif
constexpr int kTileWaves = MSSCAN_TILE_WAVES;
constexpr int64_t kTargetWaves = MSSCAN_TARGET_WAVES;
constexpr int64_t kSegmentQuantum = 16;  // whole register blocks of timesteps
#ifndef MSSCAN_MIN_SEGMENT
#define MSSCAN_MIN_SEGMENT 64  // 6144 waves (6 per SIMD) at the 130M layer
#endif
constexpr int64_t kMinSegment = MSSCAN_MIN_SEGMENT;

void cut_sequence(const ms_dims& d, int64_t waves_per_segment, msscan::Plan& p,
                  int64_t target_waves = kTargetWaves, int64_t min_segment = kMinSegment) {
    int64_t k = (target_waves + waves_per_segment - 1) / waves_per_segment;
    const int64_t kmax = (d.seqlen + min_segment - 1) / min_segment;
    if (k > kmax) k = kmax;
    if (k < 1) k = 1;
    int64_t len = (d.seqlen + k - 1) / k;
    len = (len + kSegmentQuantum - 1) / kSegmentQuantum * kSegmentQuantum;
    p.chunk_len = len;
    p.chunks = (int)((d.seqlen + len - 1) / len);
}

// Row path (d_state 9..16): a channel's states spread over one 16-lane DPP
// row, so there are 16x more waves than on the lane path and the sequence
// needs cutting only when batch x d_inner is small.  A segment after the
// first costs a summary walk over it (about as much as the scan itself), so
// the row path cuts only to about two waves per SIMD.
#ifndef MSSCAN_ROW_TARGET_WAVES
#define MSSCAN_ROW_TARGET_WAVES 2048
#endif
#ifndef MSSCAN_ROW_MIN_SEGMENT
#define MSSCAN_ROW_MIN_SEGMENT 256
#endif
// d_state 17..128 spreads a channel over 2 or 4 rows (with 2 states per lane
// past 64).  Each row repeats the channel's per-element work, so those shapes
// take the row path only when they need no cut at all (batch x d_inner x rows
// alone gives MSSCAN_ROW_WIDE_MIN_WAVES waves) and the io tiles move whole;
// otherwise the lane or tile path, whose summaries are cheaper per state,
// takes them.
#ifndef MSSCAN_ROW_WIDE_MIN_WAVES
#define MSSCAN_ROW_WIDE_MIN_WAVES 2048
#endif
static_assert(MSSCAN_ROW_WIDE_MIN_WAVES >= MSSCAN_ROW_TARGET_WAVES,
              "wide rows run the sequence as one segment");
#ifndef MSSCAN_ROW_EULER64_MIN_CHANNELS
#define MSSCAN_ROW_EULER64_MIN_CHANNELS 8192
#endif
// lane_euler: leave d_state 33..64 with Euler to the lane kernel (the plain
// forward; the fused projection has no lane kernel there).
bool row_plan(const ms_dims& d, int disc, msscan::Plan& p, bool lane_euler = true) {
    if (d.d_state <= 8) return false;
    // d_state 33..64 with Euler and few channels: the lane kernel (all 64
    // states in a lane) is as fast or faster there, summaries included
    // (batch 2, L 8192, d_inner 1536, d_state 64: 0.57 against 0.59 ms).
    // With more channels the rows win (batch 8, L 2048, d_inner 1536: 0.56
    // against 0.60 ms; batch 4, L 8192, d_inner 5120: 3.42 against 3.50).
    if (lane_euler && disc == msscan::dev::kEuler && d.d_state > 32 && d.d_state <= 64 &&
        (int64_t)d.batch * d.d_inner < MSSCAN_ROW_EULER64_MIN_CHANNELS &&
        msscan::lane_variant_exists(64, disc))
        return false;
    int rows = 1, spl = 1;
    if (d.d_state > 16) {
        rows = d.d_state <= 32 ? 2 : 4;
        spl = d.d_state <= 64 ? 1 : 2;
        // io tiles of 16 / rows channels move in whole chunks (16 bytes, or
        // 8 for 4 bf16 channels)
        const int cw = d.io == MS_BF16 ? (rows == 4 ? 4 : 8) : 4;
        if (d.d_inner % cw != 0) return false;
    }
    const int ch = msscan::kRowCh / rows;
    const int tiles = (d.d_inner + ch - 1) / ch;
    if (rows > 1 && (int64_t)d.batch * tiles * msscan::kRowWaves < MSSCAN_ROW_WIDE_MIN_WAVES)
        return false;
    p.tile_path = 3;
    p.ns = 16 * rows * spl;
    p.waves = msscan::kRowWaves;
    p.rows = rows;
    p.tiles = tiles;
    cut_sequence(d, (int64_t)d.batch * p.tiles * p.waves, p, MSSCAN_ROW_TARGET_WAVES,
                 MSSCAN_ROW_MIN_SEGMENT);
    return true;
}

bool lane_plan(const ms_dims& d, int disc, msscan::Plan& p) {
    // The smallest lane variant that holds d_state.  Other sizes run on it
    // with the extra states padded out (zero A, B and C; never stored): at up
    // to 8x the state work (d_state 1) it beat the generic kernels it replaced
    // by 2.5-6x at every size measured (1 to 48).
    int ns = 0;
    for (const int c : {8, 16, 32, 64})
        if (c >= d.d_state && msscan::lane_variant_exists(c, disc)) {
            ns = c;
            break;
        }
    if (ns == 0) return false;
    p.tile_path = 2;
    p.ns = ns;
    p.waves = 1;
    p.tiles = (d.d_inner + 63) / 64;
    cut_sequence(d, (int64_t)d.batch * p.tiles, p);
    return true;
}

bool tile_plan(const ms_dims& d, msscan::Plan& p) {
    // d_state 33-64 (the lane kernels take ZOH and bilinear up to 32) and
    // 65-128 run on the 64- and 128-state tile kernels, the extra states
    // padded out (zero A, B and C; never stored).
    const int N = d.d_state <= 64 ? (d.d_state > 32 ? 64 : d.d_state) : 128;
    int waves = kTileWaves;
    if (N % waves) return false;
    int ns = N / waves;
    if (ns > 16 && N % 8 == 0) {  // a wave's states must fit one 16-lane DPP row
        waves = 8;
        ns = N / 8;
    }
    if (!msscan::tile_variant_exists(ns, waves)) return false;
    p.tile_path = 1;
    p.ns = ns;
    p.waves = waves;
    p.tiles = (d.d_inner + 63) / 64;
    cut_sequence(d, (int64_t)d.batch * p.tiles * waves, p);
    return true;
}

// Which row plans make_plan may choose: none, those of the plain forward, or
// those of the fused step projection (which has no lane kernel above d_state
// 16, so it keeps the rows at d_state 33..64 with Euler too).
enum RowChoice { kNoRows, kForwardRows, kProjectionRows };

msscan::Plan make_plan(const ms_dims& d, uint32_t flags, RowChoice rows = kForwardRows) {
    msscan::Plan p{};
    const int N = d.d_state;
    // Per segment boundary and channel: N summary states, plus the segment
    // decay -- one sum of dt, or N products of A_bar for the bilinear form.
    const size_t per_channel = (size_t)N + ((flags & MS_BILINEAR) ? (size_t)N : 1);
    if ((rows != kNoRows && row_plan(d, disc_of(flags), p, rows == kForwardRows)) ||
        lane_plan(d, disc_of(flags), p) ||
        tile_plan(d, p)) {
        if (p.chunks > 1) {
            const size_t km1 = (size_t)(p.chunks - 1);
            p.ws_floats = km1 * (size_t)d.batch * (size_t)d.d_inner * per_channel;
        }
        // tile path: fp32 copy of B and C, rows [b][t][B_t | C_t], read as DPP
        // operands (the lane path reads B and C in place).
        if (p.tile_path == 1)  // B/C rows as wide as the tile kernels' states
            p.bc_floats = (size_t)d.batch * (size_t)d.seqlen * 2 * (size_t)(p.ns * p.waves);
        return p;
    }
    p.tile_path = -1;  // no kernel takes it (not reached for d_state 1..128)
    return p;
}

size_t round256(size_t bytes) { return (bytes + 255) / 256 * 256; }

// Workspace layout: [fp32 B/C rows][segment summaries + carries][sum of dt or
// product of A_bar][copy of h0 for the first segment], each region 256-byte
// aligned; the last three only when the sequence is cut into segments.
struct WsLayout {
    size_t bc, agg, decay, start0, total;  // byte offsets (total = size)
};

WsLayout ws_layout(const msscan::Plan& p, const ms_dims& d, uint32_t flags) {
    WsLayout w{};
    size_t off = round256(p.bc_floats * sizeof(float));
    w.bc = 0;
    if (p.chunks > 1) {
        const size_t km1 = (size_t)(p.chunks - 1);
        const size_t bdn = (size_t)d.batch * (size_t)d.d_inner * (size_t)d.d_state;
        w.agg = off;
        off += round256(km1 * bdn * sizeof(float));
        w.decay = off;
        off += round256(km1 * (size_t)d.batch * (size_t)d.d_inner *
                        ((flags & MS_BILINEAR) ? (size_t)d.d_state : 1) * sizeof(float));
        w.start0 = off;
        off += round256(bdn * sizeof(float));
    }
    w.total = off;
    return w;
}

size_t ws_bytes(const msscan::Plan& p, const ms_dims& d, uint32_t flags) {
    return ws_layout(p, d, flags).total;
}

// Points the workspace regions of a at `workspace` (laid out by ws_layout).
void bind_workspace(msscan::ScanArgs& a, const msscan::Plan& p, const ms_dims& d, uint32_t flags,
                    void* workspace) {
    const WsLayout w = ws_layout(p, d, flags);
    char* ws = static_cast<char*>(workspace);
    if (p.bc_floats) a.bcw = reinterpret_cast<float*>(ws + w.bc);
    if (p.chunks > 1) {
        a.agg = reinterpret_cast<float*>(ws + w.agg);
        float* decay = reinterpret_cast<float*>(ws + w.decay);
        if (flags & MS_BILINEAR)
            a.prod = decay;  // [batch][chunks-1][N][Dn], like the summaries
        else
            a.sdt = decay;  // [batch][chunks-1][Dn]
        if (a.h0) a.start0 = reinterpret_cast<float*>(ws + w.start0);
    }
}

// One forward scan: validation, plan, workspace binding and launch (the body
// of ms_scan_fwd and ms_scan_fwd_noalloc).
ms_status scan_fwd_impl(const void* u, const void* delta, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* delta_bias,
                        uint32_t flags, void* y, const float* h0, float* h_last,
                        const ms_dims* dims, void* workspace, size_t workspace_bytes,
                        void* stream) {
    ms_status st = check_dims(dims);
    if (st != MS_OK) return st;
    if ((st = check_flags(flags)) != MS_OK) return st;
    if (!u || !delta || !A || !B || !C || !y)
        return fail(MS_ERR_NULL, "u, delta, A, B, C and y are required");
    const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, y, h0, h_last, workspace};
    for (const void* p : ptrs)
        if (misaligned(p)) return fail(MS_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    const msscan::Plan p = make_plan(*dims, flags);
    if (p.tile_path < 0) return fail(MS_ERR_UNSUPPORTED, "no scan kernel for d_state %d", dims->d_state);
    const size_t need = ws_bytes(p, *dims, flags);
    if (need && (!workspace || workspace_bytes < need))
        return fail(MS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);

    msscan::ScanArgs a{};
    a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
    a.h0 = h0; a.h_last = h_last; a.y = y;
    a.L = dims->seqlen; a.chunk_len = p.chunk_len; a.batch = dims->batch; a.Dn = dims->d_inner;
    a.N = dims->d_state; a.chunks = p.chunks; a.softplus = (flags & MS_SOFTPLUS) ? 1 : 0;
    a.waves = p.waves;
    a.tiles = p.tiles;
    bind_workspace(a, p, *dims, flags, workspace);
    const bool bf16 = dims->io == MS_BF16;
    const int disc = disc_of(flags);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    msscan::prof_call();
    hipError_t e;
    if (p.tile_path == 3)
        e = msscan::launch_scan_rows(p, a, bf16, disc, hs);
    else if (p.tile_path == 2)
        e = msscan::launch_scan_lanes(p, a, bf16, disc, hs);
    else
        e = msscan::launch_scan_tiles(p, a, bf16, disc, hs);
    if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
}

}  // namespace

namespace msscan {
void clear_error() { g_err[0] = '\0'; }
ms_status report(ms_status s, const char* text) { return fail(s, "%s", text); }
ms_status scan_fwd_checked(const void* u, const void* delta, const float* A, const void* B,
                           const void* C, const float* D, const void* z, const float* delta_bias,
                           uint32_t flags, void* y, const float* h0, float* h_last,
                           const ms_dims* dims, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, flags, y, h0, h_last, dims,
                         workspace, workspace_bytes, stream);
}
}  // namespace msscan

extern "C" {

int ms_abi_version(void) { return MS_ABI_VERSION; }

const char* ms_last_error(void) { return g_err; }

const char* ms_status_string(ms_status s) {
    switch (s) {
        case MS_OK: return "ok";
        case MS_ERR_NULL: return "required pointer is NULL";
        case MS_ERR_SHAPE: return "size out of range";
        case MS_ERR_DTYPE: return "unsupported io dtype";
        case MS_ERR_FLAGS: return "unknown flag bits";
        case MS_ERR_ALIGN: return "pointer not 16-byte aligned";
        case MS_ERR_WORKSPACE: return "workspace missing or too small";
        case MS_ERR_UNSUPPORTED: return "unsupported request";
        case MS_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t ms_scan_workspace_bytes(const ms_dims* dims, uint32_t flags) {
    if (check_dims(dims) != MS_OK || check_flags(flags) != MS_OK) return (size_t)-1;
    return ws_bytes(make_plan(*dims, flags), *dims, flags);
}

// The fused step projection runs on the row kernel whenever a row plan with
// whole io tiles exists (d_state 9..16; 17..128 when batch x d_inner fills
// the chip uncut), else on the lane kernels (d_state 8 and 16).
static msscan::Plan dtproj_plan(const ms_dims& d, uint32_t flags) {
    const msscan::Plan p = make_plan(d, flags, kProjectionRows);
    if (p.tile_path == 3 && (p.rows > 1 || d.d_inner % (d.io == MS_BF16 ? 8 : 4) == 0)) return p;
    return make_plan(d, flags, kNoRows);
}

size_t ms_scan_dtproj_workspace_bytes(const ms_dims* dims, uint32_t flags) {
    if (check_dims(dims) != MS_OK || check_flags(flags) != MS_OK) return (size_t)-1;
    return ws_bytes(dtproj_plan(*dims, flags), *dims, flags);
}

ms_status ms_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      uint32_t flags, void* y, const float* h0, float* h_last,
                      const ms_dims* dims, void* workspace, size_t workspace_bytes,
                      void* stream) {
    g_err[0] = '\0';
    return scan_fwd_impl(u, delta, A, B, C, D, z, delta_bias, flags, y, h0, h_last, dims,
                         workspace, workspace_bytes, stream);
}

ms_status ms_scan_fwd_dtproj(const void* u, const void* dt_low, const void* W_dt,
                             int32_t dt_rank, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias,
                             uint32_t flags, void* y, const float* h0, float* h_last,
                             const ms_dims* dims, void* workspace, size_t workspace_bytes,
                             void* stream) {
    g_err[0] = '\0';
    ms_status st = check_dims(dims);
    if (st != MS_OK) return st;
    if ((st = check_flags(flags)) != MS_OK) return st;
    if (!u || !dt_low || !W_dt || !A || !B || !C || !y)
        return fail(MS_ERR_NULL, "u, dt_low, W_dt, A, B, C and y are required");
    if (dt_rank < 1 || dt_rank > 64)
        return fail(MS_ERR_SHAPE, "dt_rank=%d must be in [1, 64]", dt_rank);
    const void* ptrs[] = {u, dt_low, W_dt, A, B, C, D, z, delta_bias, y, h0, h_last, workspace};
    for (const void* p : ptrs)
        if (misaligned(p)) return fail(MS_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    const msscan::Plan p = dtproj_plan(*dims, flags);
    const bool rows = p.tile_path == 3;
    if (!rows &&
        (p.tile_path != 2 || p.ns != dims->d_state || !msscan::dtproj_variant_exists(dims->d_state)))
        return fail(MS_ERR_UNSUPPORTED,
                    "the fused dt projection needs d_state 8, 9..16, or 17..128 with "
                    "batch x d_inner filling the GPU uncut (got %d; all but 8 and 16 also need "
                    "d_inner a multiple of 8 for bf16, 4 for fp32)",
                    dims->d_state);
    const size_t need = ws_bytes(p, *dims, flags);
    if (need && (!workspace || workspace_bytes < need))
        return fail(MS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);

    msscan::ScanArgs a{};
    a.u = u; a.delta = nullptr; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
    a.h0 = h0; a.h_last = h_last; a.y = y;
    a.dtx = dt_low; a.wdt = W_dt; a.rank = dt_rank;
    a.L = dims->seqlen; a.chunk_len = p.chunk_len; a.batch = dims->batch; a.Dn = dims->d_inner;
    a.N = dims->d_state; a.chunks = p.chunks; a.softplus = (flags & MS_SOFTPLUS) ? 1 : 0;
    a.waves = p.waves;
    a.tiles = p.tiles;
    bind_workspace(a, p, *dims, flags, workspace);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    msscan::prof_call();
    const hipError_t e =
        rows ? msscan::launch_scan_rows_dtproj(p, a, dims->io == MS_BF16, disc_of(flags), hs)
             : msscan::launch_scan_lanes_dtproj(p, a, dims->io == MS_BF16, disc_of(flags), hs);
    if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
}

ms_status ms_state_update(float* h, const void* x_t, const void* delta_t, const float* A,
                          const void* B_t, const void* C_t, const float* D, const void* z_t,
                          const float* delta_bias, uint32_t flags, void* y_t, int32_t batch,
                          int32_t d_inner, int32_t d_state, int32_t io, void* stream) {
    g_err[0] = '\0';
    ms_dims dims{batch, 1, d_inner, d_state, io};
    ms_status st = check_dims(&dims);
    if (st != MS_OK) return st;
    if ((st = check_flags(flags)) != MS_OK) return st;
    if (!h || !x_t || !delta_t || !A || !B_t || !C_t || !y_t)
        return fail(MS_ERR_NULL, "h, x_t, delta_t, A, B_t, C_t and y_t are required");
    const void* ptrs[] = {h, x_t, delta_t, A, B_t, C_t, D, z_t, delta_bias, y_t};
    for (const void* p : ptrs)
        if (misaligned(p)) return fail(MS_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    msscan::StepArgs a{};
    a.h = h; a.x = x_t; a.delta = delta_t; a.A = A; a.B = B_t; a.C = C_t; a.D = D; a.z = z_t;
    a.bias = delta_bias; a.y = y_t; a.batch = batch; a.Dn = d_inner; a.N = d_state;
    a.softplus = (flags & MS_SOFTPLUS) ? 1 : 0;
    msscan::prof_call();
    const bool bf16 = io == MS_BF16;
    const int disc = disc_of(flags);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (!msscan::step_quads_supported(batch, d_inner, d_state))
        return fail(MS_ERR_UNSUPPORTED, "d_inner %d too large for the decode step", d_inner);
    hipError_t e = msscan::launch_step_quads(a, bf16, disc, hs);
    if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
}

namespace {
// Backward plan for d_state <= 16.
//   rows (d_state 9..16, whole 16-byte io chunks, and at least
//     MSSCAN_BWD_ROW_MIN_TILES 16-channel tiles over the batch): the row
//     layout of bwd_row.hip -- a checkpointing forward walk, one reverse walk
//     per tile over the whole sequence;
//   else segments of bwd_segment_len() steps, all states of a channel in one
//     lane (scan_bwd.hip).
#ifndef MSSCAN_BWD_ROW_MIN_TILES
#define MSSCAN_BWD_ROW_MIN_TILES 512
#endif
struct BwdPlan {
    msscan::Plan fwd;
    int64_t K, tiles;
    bool rows;
    size_t agg, fdecay, mu, bdecay, pbc, pparam, pgroup, ckpt;  // floats of each region
};

size_t pad64(size_t n) { return (n + 63) / 64 * 64; }

BwdPlan bwd_plan(const ms_dims& d, uint32_t flags) {
    BwdPlan q{};
    {
        const int64_t tiles = (d.d_inner + msscan::kRowCh - 1) / msscan::kRowCh;
        if (d.d_state > 8 && d.d_state <= 16 && d.d_inner % (d.io == MS_BF16 ? 8 : 4) == 0 &&
            (int64_t)d.batch * tiles >= MSSCAN_BWD_ROW_MIN_TILES) {
            const size_t B = (size_t)d.batch, D = (size_t)d.d_inner, N = (size_t)d.d_state;
            const size_t nblk = (size_t)((d.seqlen + 15) / 16);
            q.rows = true;
            q.K = 1;
            q.tiles = tiles;
            q.ckpt = B * nblk * D * N;
            q.pbc = (size_t)tiles * B * (size_t)d.seqlen * 2 * N;
            q.pparam = B * D * (N + 2);
            q.pgroup = (size_t)msscan::kParamGroups * D * (N + 2);
            msscan::Plan& p = q.fwd;
            p.tile_path = 3;
            p.ns = 16;
            p.waves = msscan::kRowWaves;
            p.rows = 1;
            p.tiles = (int)tiles;
            p.chunks = 1;
            p.chunk_len = d.seqlen;
            return q;
        }
    }
    const int64_t seg = msscan::bwd_segment_len();
    q.K = (d.seqlen + seg - 1) / seg;
    q.tiles = (d.d_inner + 63) / 64;
    const size_t B = (size_t)d.batch, D = (size_t)d.d_inner, N = (size_t)d.d_state;
    const size_t km1 = (size_t)(q.K - 1);
    const bool bil = (flags & MS_BILINEAR) != 0;
    q.agg = km1 * B * N * D;
    q.fdecay = km1 * B * D * (bil ? N : 1);
    q.mu = q.agg;
    q.bdecay = q.fdecay;
    q.pbc = (size_t)q.tiles * B * (size_t)d.seqlen * 2 * N;
    q.pparam = B * (size_t)((q.K + msscan::kBwdWaves - 1) / msscan::kBwdWaves) * D * (N + 2);
    q.pgroup = (size_t)msscan::kParamGroups * D * (N + 2);
    msscan::Plan& p = q.fwd;
    p.tile_path = 2;  // the backward's own segment plan (its kernels read ns)
    p.ns = d.d_state <= 4 ? 4 : (d.d_state <= 8 ? 8 : 16);
    p.waves = 1;
    p.tiles = (int)q.tiles;
    p.chunks = (int)q.K;
    p.chunk_len = seg;
    return q;
}

// with_ckpt: whether the workspace holds the checkpoints (not when the
// forward saved them).
size_t bwd_ws_floats(const BwdPlan& q, bool with_ckpt = true) {
    return pad64(q.agg) + pad64(q.fdecay) + pad64(q.mu) + pad64(q.bdecay) + pad64(q.pbc) +
           pad64(q.pparam) + pad64(q.pgroup) + (with_ckpt ? pad64(q.ckpt) : 0);
}

// Forward-saved checkpoints: offered where the backward runs on the row layout
// (bwd_plan's rows) and the forward's own plan is the uncut one-row kernel
// with whole io tiles, which the same conditions give.
bool ckpt_plan(const ms_dims& d, uint32_t flags, BwdPlan* q, msscan::Plan* p) {
    *q = bwd_plan(d, flags);
    *p = make_plan(d, flags);
    return q->rows && p->tile_path == 3 && p->rows == 1 && p->chunks == 1 &&
           d.d_inner % (d.io == MS_BF16 ? 8 : 4) == 0;
}

// Launches the 16-states-or-fewer backward kernels on one problem (the
// inputs in `f`, the workspace at ws laid out by bwd_plan).
// ckpt: the forward's checkpoints (row plans only; null: the backward walks
// the sequence for them, into the workspace).
hipError_t run_bwd_narrow(msscan::ScanArgs f, const BwdPlan& q, uint32_t flags, float* ws,
                          const void* dy, const float* dh_last, void* du, void* ddelta, void* dz,
                          float* dA, float* dB, float* dC, float* dD, float* dbias, float* dh0,
                          bool bf16, hipStream_t hs, const float* ckpt = nullptr,
                          float* ypart = nullptr, bool ypart_add = false, bool out_add = false) {
    f.chunk_len = q.fwd.chunk_len;
    f.chunks = q.fwd.chunks;
    if (q.rows) {
        f.tiles = (int)q.tiles;
        f.waves = msscan::kRowWaves;
        msscan::BwdRowLaunch L{};
        L.walk = ckpt == nullptr;
        if (ckpt) {
            L.ckpt = const_cast<float*>(ckpt);  // read only (no walk)
        } else {
            L.ckpt = ws;
            ws += pad64(q.ckpt);
        }
        L.pbc = ws;
        L.pparam = (ws += pad64(q.pbc));
        L.pgroup = ws + pad64(q.pparam);
        L.f = f;
        L.dy = dy; L.dh_last = dh_last; L.du = du; L.ddelta = ddelta; L.dz = f.z ? dz : nullptr;
        L.dh0 = dh0; L.dA = dA; L.dB = dB; L.dC = dC; L.dD = f.D ? dD : nullptr; L.dbias = dbias;
        L.bf16 = bf16;
        L.disc = disc_of(flags);
        // Checkpointing forward walk, reverse walk, fixed-order sums.
        return msscan::launch_scan_bwd_rows(L, hs);
    }
    f.waves = 1;
    const bool bil = (flags & MS_BILINEAR) != 0;
    f.agg = ws;
    ws += pad64(q.agg);
    if (bil) f.prod = ws; else f.sdt = ws;
    ws += pad64(q.fdecay);
    msscan::BwdLaunch L{};
    L.mu = ws;
    ws += pad64(q.mu);
    if (bil) L.prod_b = ws; else L.sdt_b = ws;
    ws += pad64(q.bdecay);
    L.pbc = ws;
    ws += pad64(q.pbc);
    L.pparam = ws;
    L.pgroup = ws + pad64(q.pparam);
    L.f = f;
    L.dy = dy; L.dh_last = dh_last; L.du = du; L.ddelta = ddelta; L.dz = f.z ? dz : nullptr;
    L.dh0 = dh0; L.dA = dA; L.dB = dB; L.dC = dC; L.dD = f.D ? dD : nullptr; L.dbias = dbias;
    L.bf16 = bf16;
    L.disc = disc_of(flags);
    L.ypart = ypart;  // the row layout above has no such output: callers check
    L.ypart_add = ypart_add ? 1 : 0;
    L.out_add = (out_add && !bf16) ? 1 : 0;
    // Segment summaries (forward and adjoint), both carries, the per-segment
    // gradients and the fixed-order sums.
    return msscan::launch_scan_bwd(L, hs);
}

// Backward for d_state 17..128: slices of 16 states (bwd_wide.hip).  The
// workspace holds, in order (fp32, each region padded to 64 floats):
//   g, u32, d32 (bf16 io), B32, C32 (bf16 io), y_pre, the fp32 forward's own
//   workspace (row-layout slices only), the slice inputs (A_s, B_s, C_s, h0_s, dh_last_s), the slice
//   outputs (du_s, ddelta_s, dA_s, dB_s, dC_s, dbias_s, dh0_s), the totals
//   (du, ddelta, dbias), the dD partials, and the 16-state backward's workspace.
struct WideLayout {
    ms_dims d16, dfwd;
    BwdPlan inner;
    msscan::Plan fwd;
    size_t off[32];
    size_t total;  // floats
};
enum : int {
    kWg, kWu32, kWd32, kWB32, kWC32, kWy32, kWfws, kWAs, kWBs, kWCs, kWh0s, kWdhls, kWdus,
    kWdvs, kWdAs, kWdBs, kWdCs, kWdbs, kWdh0s, kWduacc, kWdvacc, kWdbacc, kWdDp, kWinner,
    kWcount
};

WideLayout wide_layout(const ms_dims& d, uint32_t flags) {
    WideLayout w{};
    const size_t E = (size_t)d.batch * (size_t)d.seqlen * (size_t)d.d_inner;
    const size_t BL = (size_t)d.batch * (size_t)d.seqlen, BD = (size_t)d.batch * (size_t)d.d_inner;
    const size_t Dn = (size_t)d.d_inner, S = msscan::kWideSlice;
    const bool bf16 = d.io == MS_BF16;
    w.d16 = d;
    w.d16.d_state = msscan::kWideSlice;
    w.d16.io = MS_F32;
    w.dfwd = d;
    w.dfwd.io = MS_F32;
    w.inner = bwd_plan(w.d16, flags);
    w.fwd = make_plan(w.dfwd, flags);
    size_t n[kWcount] = {};
    n[kWg] = E;
    n[kWu32] = bf16 ? E : 0;
    n[kWd32] = bf16 ? E : 0;
    n[kWB32] = bf16 ? BL * (size_t)d.d_state : 0;
    n[kWC32] = n[kWB32];
    n[kWy32] = E;
    // the forward that forms y_pre runs only for row-layout slices
    n[kWfws] = w.inner.rows ? (ws_bytes(w.fwd, w.dfwd, flags) + 3) / 4 : 0;
    n[kWAs] = Dn * S;
    n[kWBs] = n[kWCs] = BL * S;
    n[kWh0s] = n[kWdhls] = BD * S;
    n[kWdus] = n[kWdvs] = E;
    n[kWdAs] = Dn * S;
    n[kWdBs] = n[kWdCs] = BL * S;
    n[kWdbs] = Dn;
    n[kWdh0s] = BD * S;
    n[kWduacc] = n[kWdvacc] = E;
    n[kWdbacc] = Dn;
    n[kWdDp] = (size_t)msscan::kWideGroups * Dn;
    n[kWinner] = bwd_ws_floats(w.inner);
    size_t off = 0;
    for (int i = 0; i < kWcount; ++i) {
        w.off[i] = off;
        off += pad64(n[i]);
    }
    w.total = off;
    return w;
}
}  // namespace

size_t ms_scan_bwd_workspace_bytes(const ms_dims* dims, uint32_t flags) {
    if (check_dims(dims) != MS_OK || check_flags(flags) != MS_OK) return (size_t)-1;
    if (dims->d_state > 16) return wide_layout(*dims, flags).total * sizeof(float);
    return bwd_ws_floats(bwd_plan(*dims, flags)) * sizeof(float);
}

ms_status ms_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      uint32_t flags, const float* h0, const void* dy, const float* dh_last,
                      void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD,
                      void* dz, float* dbias, float* dh0, const ms_dims* dims, void* workspace,
                      size_t workspace_bytes, void* stream) {
    g_err[0] = '\0';
    ms_status st = check_dims(dims);
    if (st != MS_OK) return st;
    if ((st = check_flags(flags)) != MS_OK) return st;
    if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC)
        return fail(MS_ERR_NULL, "u, delta, A, B, C, dy, du, ddelta, dA, dB and dC are required");
    if ((z && !dz) || (D && !dD))
        return fail(MS_ERR_NULL, "dz (dD) is required when z (D) is given");
    const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_last, du,
                          ddelta, dA, dB, dC, dD, dz, dbias, dh0, workspace};
    for (const void* p : ptrs)
        if (misaligned(p)) return fail(MS_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    const size_t need = ms_scan_bwd_workspace_bytes(dims, flags);
    if (!workspace || workspace_bytes < need)
        return fail(MS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    const bool bf16 = dims->io == MS_BF16;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    msscan::prof_call();

    msscan::ScanArgs a{};
    a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
    a.h0 = h0; a.L = dims->seqlen; a.batch = dims->batch; a.Dn = dims->d_inner;
    a.N = dims->d_state; a.softplus = (flags & MS_SOFTPLUS) ? 1 : 0;
    hipError_t e;
    if (dims->d_state <= 16) {
        e = run_bwd_narrow(a, bwd_plan(*dims, flags), flags, static_cast<float*>(workspace), dy,
                           dh_last, du, ddelta, dz, dA, dB, dC, dD, dbias, dh0, bf16, hs);
        if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        return MS_OK;
    }

    // d_state 17..128: slices of 16 states, each an fp32 problem with the
    // gate and D taken out (bwd_wide.hip).
    const WideLayout wl = wide_layout(*dims, flags);
    float* ws = static_cast<float*>(workspace);
    auto R = [&](int i) { return ws + wl.off[i]; };
    msscan::WideArgs w{};
    w.u = u; w.delta = delta; w.A = A; w.B = B; w.C = C; w.D = D; w.z = z; w.dy = dy;
    w.h0 = h0; w.dh_last = dh_last;
    w.E = (int64_t)dims->batch * dims->seqlen * dims->d_inner;
    w.BL = (int64_t)dims->batch * dims->seqlen;
    w.BD = (int64_t)dims->batch * dims->d_inner;
    w.BLN = w.BL * dims->d_state;
    w.Dn = dims->d_inner; w.N = dims->d_state;
    w.g = R(kWg); w.y32 = R(kWy32);
    w.u32 = bf16 ? R(kWu32) : nullptr; w.d32 = bf16 ? R(kWd32) : nullptr;
    w.B32 = bf16 ? R(kWB32) : nullptr; w.C32 = bf16 ? R(kWC32) : nullptr;
    w.As = R(kWAs); w.Bs = R(kWBs); w.Cs = R(kWCs);
    w.h0s = h0 ? R(kWh0s) : nullptr; w.dhls = dh_last ? R(kWdhls) : nullptr;
    w.du_s = R(kWdus); w.dv_s = R(kWdvs); w.dAs = R(kWdAs); w.dBs = R(kWdBs); w.dCs = R(kWdCs);
    w.dbias_s = R(kWdbs); w.dh0s = dh0 ? R(kWdh0s) : nullptr;
    w.du_acc = R(kWduacc); w.dv_acc = R(kWdvacc); w.dbias_acc = R(kWdbacc); w.dD_part = R(kWdDp);
    w.du = du; w.ddelta = ddelta; w.dz = z ? dz : nullptr;
    w.dA = dA; w.dB = dB; w.dC = dC; w.dD = D ? dD : nullptr; w.dbias = dbias; w.dh0 = dh0;
    if ((e = msscan::launch_wide_prep(w, bf16, hs)) != hipSuccess)
        return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    const float* u32 = bf16 ? w.u32 : static_cast<const float*>(u);
    const float* d32 = bf16 ? w.d32 : static_cast<const float*>(delta);
    // y_pre = sum_n C h + D u in fp32, for dz.  With the segment layout for
    // the slices, each slice's gradient pass adds its states' sum_n C h to
    // y32 from the states it recomputes anyway (in slice order, so the sum
    // is deterministic) and the combine adds D u; the row layout has no such
    // output, and there the forward scan without the gate forms y_pre.
    const bool fuse_ypre = z && !wl.inner.rows;
    w.y32_add_du = fuse_ypre ? 1 : 0;
    if (z && !fuse_ypre) {
        msscan::ScanArgs fa = a;
        fa.u = u32; fa.delta = d32; fa.z = nullptr; fa.y = w.y32; fa.h_last = nullptr;
        fa.B = bf16 ? w.B32 : B; fa.C = bf16 ? w.C32 : C;
        fa.chunk_len = wl.fwd.chunk_len; fa.chunks = wl.fwd.chunks; fa.waves = wl.fwd.waves;
        fa.tiles = wl.fwd.tiles;
        bind_workspace(fa, wl.fwd, wl.dfwd, flags, R(kWfws));
        const int disc = disc_of(flags);
        if (wl.fwd.tile_path == 3)
            e = msscan::launch_scan_rows(wl.fwd, fa, false, disc, hs);
        else if (wl.fwd.tile_path == 2)
            e = msscan::launch_scan_lanes(wl.fwd, fa, false, disc, hs);
        else
            e = msscan::launch_scan_tiles(wl.fwd, fa, false, disc, hs);
        if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    }
    for (int n0 = 0; n0 < dims->d_state; n0 += msscan::kWideSlice) {
        if ((e = msscan::launch_wide_gather(w, n0, bf16, hs)) != hipSuccess)
            return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        msscan::ScanArgs sa = a;
        sa.u = u32; sa.delta = d32; sa.A = w.As; sa.B = w.Bs; sa.C = w.Cs; sa.D = nullptr;
        sa.z = nullptr; sa.h0 = w.h0s; sa.N = msscan::kWideSlice;
        // du and ddelta go straight into the totals: written by the first
        // slice, added by the later ones' gradient passes (segment layout;
        // row-layout slices write their own and the accumulate adds them)
        const bool first = n0 == 0;
        const bool inplace = first || !wl.inner.rows;
        e = run_bwd_narrow(sa, wl.inner, flags, R(kWinner), w.g, w.dhls,
                           inplace ? w.du_acc : w.du_s, inplace ? w.dv_acc : w.dv_s, nullptr,
                           w.dAs, w.dBs, w.dCs, nullptr, w.dbias_s, w.dh0s, false, hs, nullptr,
                           fuse_ypre ? w.y32 : nullptr, !first, !first && inplace);
        if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
        if ((e = msscan::launch_wide_accumulate(w, n0, !inplace, hs)) != hipSuccess)
            return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    }
    if ((e = msscan::launch_wide_finish(w, bf16, hs)) != hipSuccess)
        return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
}

size_t ms_scan_checkpoint_bytes(const ms_dims* dims, uint32_t flags) {
    if (check_dims(dims) != MS_OK || check_flags(flags) != MS_OK) return (size_t)-1;
    BwdPlan q;
    msscan::Plan p;
    return ckpt_plan(*dims, flags, &q, &p) ? pad64(q.ckpt) * sizeof(float) : 0;
}

ms_status ms_scan_fwd_checkpoint(const void* u, const void* delta, const float* A,
                                 const void* B, const void* C, const float* D, const void* z,
                                 const float* delta_bias, uint32_t flags, void* y,
                                 const float* h0, float* h_last, float* checkpoint,
                                 const ms_dims* dims, void* stream) {
    g_err[0] = '\0';
    ms_status st = check_dims(dims);
    if (st != MS_OK) return st;
    if ((st = check_flags(flags)) != MS_OK) return st;
    if (!u || !delta || !A || !B || !C || !y || !checkpoint)
        return fail(MS_ERR_NULL, "u, delta, A, B, C, y and checkpoint are required");
    const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, y, h0, h_last, checkpoint};
    for (const void* p : ptrs)
        if (misaligned(p)) return fail(MS_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    BwdPlan q;
    msscan::Plan p;
    if (!ckpt_plan(*dims, flags, &q, &p))
        return fail(MS_ERR_UNSUPPORTED,
                    "no forward checkpoints for these dims (ms_scan_checkpoint_bytes is 0)");
    msscan::ScanArgs a{};
    a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
    a.h0 = h0; a.h_last = h_last; a.y = y; a.agg = checkpoint;
    a.L = dims->seqlen; a.chunk_len = p.chunk_len; a.batch = dims->batch; a.Dn = dims->d_inner;
    a.N = dims->d_state; a.chunks = p.chunks; a.softplus = (flags & MS_SOFTPLUS) ? 1 : 0;
    a.waves = p.waves;
    a.tiles = p.tiles;
    msscan::prof_call();
    const hipError_t e = msscan::launch_scan_rows_ckpt(p, a, dims->io == MS_BF16, disc_of(flags),
                                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
}

size_t ms_scan_bwd_checkpoint_workspace_bytes(const ms_dims* dims, uint32_t flags) {
    if (check_dims(dims) != MS_OK || check_flags(flags) != MS_OK) return (size_t)-1;
    BwdPlan q;
    msscan::Plan p;
    if (!ckpt_plan(*dims, flags, &q, &p)) return (size_t)-1;
    return bwd_ws_floats(q, false) * sizeof(float);
}

ms_status ms_scan_bwd_checkpoint(const void* u, const void* delta, const float* A,
                                 const void* B, const void* C, const float* D, const void* z,
                                 const float* delta_bias, uint32_t flags,
                                 const float* checkpoint, const void* dy, const float* dh_last,
                                 void* du, void* ddelta, float* dA, float* dB, float* dC,
                                 float* dD, void* dz, float* dbias, float* dh0,
                                 const ms_dims* dims, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    g_err[0] = '\0';
    ms_status st = check_dims(dims);
    if (st != MS_OK) return st;
    if ((st = check_flags(flags)) != MS_OK) return st;
    if (!u || !delta || !A || !B || !C || !checkpoint || !dy || !du || !ddelta || !dA || !dB ||
        !dC)
        return fail(MS_ERR_NULL,
                    "u, delta, A, B, C, checkpoint, dy, du, ddelta, dA, dB and dC are required");
    if ((z && !dz) || (D && !dD))
        return fail(MS_ERR_NULL, "dz (dD) is required when z (D) is given");
    const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, checkpoint, dy, dh_last, du,
                          ddelta, dA, dB, dC, dD, dz, dbias, dh0, workspace};
    for (const void* p : ptrs)
        if (misaligned(p)) return fail(MS_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    BwdPlan q;
    msscan::Plan p;
    if (!ckpt_plan(*dims, flags, &q, &p))
        return fail(MS_ERR_UNSUPPORTED,
                    "no forward checkpoints for these dims (ms_scan_checkpoint_bytes is 0)");
    const size_t need = bwd_ws_floats(q, false) * sizeof(float);
    if (!workspace || workspace_bytes < need)
        return fail(MS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    msscan::ScanArgs a{};
    a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
    a.L = dims->seqlen; a.batch = dims->batch; a.Dn = dims->d_inner;
    a.N = dims->d_state; a.softplus = (flags & MS_SOFTPLUS) ? 1 : 0;
    msscan::prof_call();
    const hipError_t e =
        run_bwd_narrow(a, q, flags, static_cast<float*>(workspace), dy, dh_last, du, ddelta, dz,
                       dA, dB, dC, dD, dbias, dh0, dims->io == MS_BF16,
                       static_cast<hipStream_t>(stream), checkpoint);
    if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
}

ms_status ms_conv1d_silu(const void* x, const float* weight, const float* bias,
                         const void* x_prev, int32_t width, int32_t silu, void* u,
                         int32_t batch, int64_t seqlen, int32_t d_inner, int32_t io,
                         void* stream) {
    g_err[0] = '\0';
    ms_dims dims{batch, seqlen, d_inner, 1, io};
    ms_status st = check_dims(&dims);
    if (st != MS_OK) return st;
    if (width < 1 || width > 8) return fail(MS_ERR_SHAPE, "width=%d must be in [1, 8]", width);
    if (!x || !weight || !u) return fail(MS_ERR_NULL, "x, weight and u are required");
    const void* ptrs[] = {x, weight, bias, x_prev, u};
    for (const void* p : ptrs)
        if (misaligned(p)) return fail(MS_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    msscan::ConvArgs a{};
    a.x = x; a.w = weight; a.bias = bias; a.x_prev = width > 1 ? x_prev : nullptr; a.u = u;
    a.L = seqlen; a.batch = batch; a.Dn = d_inner; a.width = width;
    if (msscan::conv_workgroups(a) > msscan::kMaxConvWorkgroups)
        return fail(MS_ERR_UNSUPPORTED, "batch x seqlen x d_inner needs more than 2^31-1 conv "
                                        "workgroups");
    msscan::prof_call();
    hipError_t e = msscan::launch_conv1d(a, io == MS_BF16, silu != 0,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
}

}  // extern "C"
