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

// Fast paths.  Both map one 64-channel tile of one batch row to a
// workgroup and cut the sequence into segments until about kTargetWaves
// waves exist (many waves per CU keep the VALU issuing; a segment after the
// first costs a summary pass over it, so segments are not cut shorter than
// kMinSegment).
//   lane path (d_state 8, 16, 32; 64 with Euler): one wave per workgroup,
//     all states of a channel in one lane;
//   tile path (d_state 128, 64 with ZOH or bilinear, or the others when the lane path is
//     compiled out): several waves split d_state and share per-element work
//     through LDS.
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

void cut_sequence(const ms_dims& d, int64_t waves_per_segment, msscan::Plan& p) {
    int64_t k = (kTargetWaves + waves_per_segment - 1) / waves_per_segment;
    const int64_t kmax = (d.seqlen + kMinSegment - 1) / kMinSegment;
    if (k > kmax) k = kmax;
    if (k < 1) k = 1;
    int64_t len = (d.seqlen + k - 1) / k;
    len = (len + kSegmentQuantum - 1) / kSegmentQuantum * kSegmentQuantum;
    p.chunk_len = len;
    p.chunks = (int)((d.seqlen + len - 1) / len);
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

msscan::Plan make_plan(const ms_dims& d, uint32_t flags) {
    msscan::Plan p{};
    const int N = d.d_state;
    // Per segment boundary and channel: N summary states, plus the segment
    // decay -- one sum of dt, or N products of A_bar for the bilinear form.
    const size_t per_channel = (size_t)N + ((flags & MS_BILINEAR) ? (size_t)N : 1);
    if (lane_plan(d, disc_of(flags), p) || tile_plan(d, p)) {
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

// Workspace layout: [fp32 B/C slices][chunk summaries + carries][sum of dt].
size_t ws_bytes(const msscan::Plan& p) {
    size_t n = round256(p.bc_floats * sizeof(float));
    if (p.ws_floats) n += round256(p.ws_floats * sizeof(float)) + 256;
    return n;
}

}  // namespace

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
    return ws_bytes(make_plan(*dims, flags));
}

ms_status ms_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z, const float* delta_bias,
                      uint32_t flags, void* y, const float* h0, float* h_last,
                      const ms_dims* dims, void* workspace, size_t workspace_bytes,
                      void* stream) {
    g_err[0] = '\0';
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
    const size_t need = ws_bytes(p);
    if (need && (!workspace || workspace_bytes < need))
        return fail(MS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);

    msscan::ScanArgs a{};
    a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
    a.h0 = h0; a.h_last = h_last; a.y = y;
    a.L = dims->seqlen; a.chunk_len = p.chunk_len; a.batch = dims->batch; a.Dn = dims->d_inner;
    a.N = dims->d_state; a.chunks = p.chunks; a.softplus = (flags & MS_SOFTPLUS) ? 1 : 0;
    a.waves = p.waves;
    float* ws = static_cast<float*>(workspace);
    if (p.bc_floats) {
        a.bcw = ws;
        ws += round256(p.bc_floats * sizeof(float)) / sizeof(float);
    }
    if (p.chunks > 1) {
        const size_t km1 = (size_t)(p.chunks - 1);
        a.agg = ws;
        const size_t agg_n = km1 * (size_t)dims->batch * (size_t)dims->d_state * (size_t)dims->d_inner;
        float* after = ws + ((agg_n + 63) / 64) * 64;
        if (flags & MS_BILINEAR)
            a.prod = after;  // [batch][chunks-1][N][Dn], like the summaries
        else
            a.sdt = after;
    }
    const bool bf16 = dims->io == MS_BF16;
    const int disc = disc_of(flags);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    msscan::prof_call();
    hipError_t e = p.tile_path == 2 ? msscan::launch_scan_lanes(p, a, bf16, disc, hs)
                                    : msscan::launch_scan_tiles(p, a, bf16, disc, hs);
    if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
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
    const msscan::Plan p = make_plan(*dims, flags);
    if (p.tile_path != 2 || p.ns != dims->d_state || !msscan::dtproj_variant_exists(dims->d_state))
        return fail(MS_ERR_UNSUPPORTED, "the fused dt projection needs d_state 8 or 16 (got %d)",
                    dims->d_state);
    const size_t need = ws_bytes(p);
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
    if (p.chunks > 1) {
        const size_t km1 = (size_t)(p.chunks - 1);
        float* ws = static_cast<float*>(workspace);
        a.agg = ws;
        const size_t agg_n = km1 * (size_t)dims->batch * (size_t)dims->d_state * (size_t)dims->d_inner;
        float* after = ws + ((agg_n + 63) / 64) * 64;
        if (flags & MS_BILINEAR)
            a.prod = after;
        else
            a.sdt = after;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    msscan::prof_call();
    const hipError_t e =
        msscan::launch_scan_lanes_dtproj(p, a, dims->io == MS_BF16, disc_of(flags), hs);
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
// Backward plan: segments of bwd_segment_len() steps, all states of a channel
// in one lane (d_state <= 16).
struct BwdPlan {
    msscan::Plan fwd;
    int64_t K, tiles;
    size_t agg, fdecay, mu, bdecay, pbc, pparam, pgroup;  // floats of each region
};

size_t pad64(size_t n) { return (n + 63) / 64 * 64; }

BwdPlan bwd_plan(const ms_dims& d, uint32_t flags) {
    BwdPlan q{};
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

size_t bwd_ws_floats(const BwdPlan& q) {
    return pad64(q.agg) + pad64(q.fdecay) + pad64(q.mu) + pad64(q.bdecay) + pad64(q.pbc) +
           pad64(q.pparam) + pad64(q.pgroup);
}
}  // namespace

size_t ms_scan_bwd_workspace_bytes(const ms_dims* dims, uint32_t flags) {
    if (check_dims(dims) != MS_OK || check_flags(flags) != MS_OK) return (size_t)-1;
    if (dims->d_state > 16) return (size_t)-1;
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
    if (dims->d_state > 16)
        return fail(MS_ERR_UNSUPPORTED, "ms_scan_bwd supports d_state <= 16 (got %d)",
                    dims->d_state);
    if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC)
        return fail(MS_ERR_NULL, "u, delta, A, B, C, dy, du, ddelta, dA, dB and dC are required");
    if ((z && !dz) || (D && !dD))
        return fail(MS_ERR_NULL, "dz (dD) is required when z (D) is given");
    const void* ptrs[] = {u, delta, A, B, C, D, z, delta_bias, h0, dy, dh_last, du,
                          ddelta, dA, dB, dC, dD, dz, dbias, dh0, workspace};
    for (const void* p : ptrs)
        if (misaligned(p)) return fail(MS_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    const BwdPlan q = bwd_plan(*dims, flags);
    const size_t need = bwd_ws_floats(q) * sizeof(float);
    if (!workspace || workspace_bytes < need)
        return fail(MS_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);

    msscan::ScanArgs a{};
    a.u = u; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.bias = delta_bias;
    a.h0 = h0; a.L = dims->seqlen; a.chunk_len = q.fwd.chunk_len; a.batch = dims->batch;
    a.Dn = dims->d_inner; a.N = dims->d_state; a.chunks = q.fwd.chunks;
    a.softplus = (flags & MS_SOFTPLUS) ? 1 : 0; a.waves = 1;
    const bool bil = (flags & MS_BILINEAR) != 0;
    float* ws = static_cast<float*>(workspace);
    a.agg = ws;
    ws += pad64(q.agg);
    if (bil) a.prod = ws; else a.sdt = ws;
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
    L.f = a;
    L.dy = dy; L.dh_last = dh_last; L.du = du; L.ddelta = ddelta; L.dz = z ? dz : nullptr;
    L.dh0 = dh0; L.dA = dA; L.dB = dB; L.dC = dC; L.dD = D ? dD : nullptr; L.dbias = dbias;
    L.bf16 = dims->io == MS_BF16;
    L.disc = disc_of(flags);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    msscan::prof_call();
    // Segment summaries (forward and adjoint), both carries, the per-segment
    // gradients and the fixed-order sums.
    const hipError_t e = msscan::launch_scan_bwd(L, hs);
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
    msscan::prof_call();
    hipError_t e = msscan::launch_conv1d(a, io == MS_BF16, silu != 0,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MS_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return MS_OK;
}

}  // extern "C"
