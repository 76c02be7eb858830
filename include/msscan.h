/*
 * msscan.h -- C ABI of libmsscan, the selective scan (S6) on AMD MI355X (gfx950).
 *
 * What is computed.  For every batch b, channel d (d_inner) and state n
 * (d_state), along the sequence t = 0..L-1:
 *
 *   dt    = softplus(delta[b,t,d] + delta_bias[d])    (MS_SOFTPLUS set)
 *         =          delta[b,t,d] + delta_bias[d]     (otherwise)
 *   A_bar = exp(dt * A[d,n])                           (Euler, MS_ZOH)
 *         = (1 + dt*A[d,n]/2) / (1 - dt*A[d,n]/2)      (MS_BILINEAR)
 *   B_bar = dt * B[b,t,n]                             (Euler, default)
 *         = (exp(dt*A[d,n]) - 1) / A[d,n] * B[b,t,n]  (MS_ZOH; dt*B when A == 0)
 *         = dt / (1 - dt*A[d,n]/2) * B[b,t,n]          (MS_BILINEAR)
 *   h[n]  = A_bar * h[n] + B_bar * u[b,t,d]           (h starts at h0, else 0)
 *   y     = sum_n C[b,t,n] * h[n]  +  D[d] * u[b,t,d]
 *   out[b,t,d] = y * z * sigmoid(z),  z = z[b,t,d]    (when z is given; else y)
 *
 * Passages followed (page titles as published, or the site where a page has
 * no title; section numbers are the pages'):
 *   - the per-timestep loop of the naive selective scan, with B and C shared by
 *     all channels and D*u added before the silu(z) gate: the lmnt.cn page
 *     (news/271401, untitled; opens with section 1 "从RNN到Mamba"), section
 *     3.2; the block data flow in section 3.1;
 *   - dt = softplus(W x + b): "Mamba架构原理与工业级长文本处理实战指南"
 *     (jsqmd.com), section 2.2;
 *   - zero-order hold A_bar = exp(dt A), B_bar = (A_bar - I) A^-1 B: "Mamba模型
 *     解析：从状态空间到序列建模实践" (intelliparadigm.com), section 3.2, and the
 *     integral form on the jsqmd page, section 2.3;
 *   - the bilinear transform named by the same page's section 3.2 code (printed
 *     garbled; the textbook form for a diagonal A is taken);
 *   - the scan as a composition of per-step affine maps, evaluated in parallel:
 *     jsqmd page section 3.4, lmnt page section 2.2;
 *   - single-token recurrent inference with one kept fp32 state: lmnt page,
 *     sections 2.2 and 5.3; the state cache of the jsqmd page, section 5.3.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers (HIP global memory) unless stated.
 *     The caller owns every buffer; the library never allocates or frees.
 *   - Layouts are contiguous row-major:
 *       u, delta, z, y : [batch][L][d_inner]      (io dtype)
 *       B, C           : [batch][L][d_state]      (io dtype)
 *       A              : [d_inner][d_state]       (fp32)
 *       D, delta_bias  : [d_inner]                (fp32)
 *       h0, h_last, h  : [batch][d_inner][d_state] (fp32)
 *   - Every base pointer must be 16-byte aligned (MS_ERR_ALIGN otherwise).
 *   - Validation is synchronous and host-only: on any error status nothing has
 *     been launched.  Work is enqueued on `stream` (a hipStream_t; NULL means
 *     the default stream) and outputs are valid once the stream reaches it.
 *     No call synchronises the host.
 *   - Data problems (NaN/Inf inputs, A > 0 growth) are computed as written and
 *     are not reported.  A NaN in one channel's inputs reaches only that
 *     channel's outputs (and state), from that timestep on.
 *   - Thread safety: calls may be made from several host threads; the last
 *     error text is thread-local.  Two calls that share an output buffer or a
 *     workspace and run concurrently (different streams) race.
 */
#ifndef MSSCAN_H
#define MSSCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MS_ABI_VERSION 1

typedef enum {
    MS_OK = 0,
    MS_ERR_NULL = 1,        /* a required pointer is NULL                       */
    MS_ERR_SHAPE = 2,       /* a size is out of range                           */
    MS_ERR_DTYPE = 3,       /* io is not MS_F32 or MS_BF16                      */
    MS_ERR_FLAGS = 4,       /* unknown flag bits, or MS_ZOH with MS_BILINEAR    */
    MS_ERR_ALIGN = 5,       /* a base pointer is not 16-byte aligned            */
    MS_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required       */
    MS_ERR_UNSUPPORTED = 7, /* valid request this library does not serve        */
    MS_ERR_HIP = 8          /* a HIP runtime call failed (text: ms_last_error)  */
} ms_status;

/* Element type of u, delta, z, B, C and y (x_t, delta_t, z_t, B_t, C_t, y_t). */
typedef enum { MS_F32 = 0, MS_BF16 = 1 } ms_dtype;

/* Flag bits. */
#define MS_SOFTPLUS (1u << 0) /* dt = softplus(delta + bias); else dt = delta + bias */
#define MS_ZOH (1u << 1)      /* zero-order hold B_bar; else Euler B_bar = dt * B     */
#define MS_BILINEAR (1u << 2) /* bilinear A_bar, B_bar (exclusive with MS_ZOH)        */

/*
 * Problem sizes.  Besides the per-field ranges (MS_ERR_SHAPE), batch and
 * ceil(d_inner / 64) must be <= 65535 (MS_ERR_UNSUPPORTED), and
 * batch * seqlen * d_inner * d_state must be <= 2^56 (MS_ERR_SHAPE), which
 * keeps every size the library computes inside size_t.
 */
typedef struct {
    int32_t batch;   /* >= 1                                   */
    int64_t seqlen;  /* L >= 1, any value (no power-of-two rule), <= 2^31 - 1 */
    int32_t d_inner; /* >= 1, any value (tails are masked)     */
    int32_t d_state; /* 1 .. 128                               */
    int32_t io;      /* ms_dtype                               */
} ms_dims;

/*
 * Bytes of device workspace ms_scan_fwd needs for these dims and flags (may
 * be 0).  Returns (size_t)-1 when the dims or flags are invalid.  Pure
 * function of its arguments; no device call.
 */
size_t ms_scan_workspace_bytes(const ms_dims* dims, uint32_t flags);

/*
 * Full-sequence selective scan (the formula at the top of this file).
 *
 *   u, delta, A, B, C, y, dims : required.
 *   D, z, delta_bias           : optional (NULL = term absent; a NULL bias is
 *                                identical to a zero bias).
 *   h0                         : optional initial state (NULL = zeros).
 *   h_last                     : optional; receives the state after step L-1.
 *                                h_last may equal h0: when the sequence is cut
 *                                into segments, the carry pass copies h0 into the
 *                                workspace before the pass that writes h_last,
 *                                and the first segment starts from that copy.
 *   workspace, workspace_bytes : device scratch of at least
 *                                ms_scan_workspace_bytes(dims, flags) bytes,
 *                                16-byte aligned; may be NULL when that is 0.
 *                                Its contents need no initialisation and are
 *                                undefined afterwards.
 *   stream                     : hipStream_t (NULL = default stream).
 *
 * y must not overlap any input.  Results are deterministic: the same inputs on
 * the same device give bit-identical outputs.
 */
ms_status ms_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z,
                      const float* delta_bias, uint32_t flags, void* y,
                      const float* h0, float* h_last, const ms_dims* dims,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * ms_scan_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * arguments and results are ms_scan_fwd's without the workspace: the scratch
 * that call takes as a workspace (ms_scan_workspace_bytes(dims, flags) bytes)
 * comes from a device array inside the library, MS_NOALLOC_MAX_BYTES per GPU,
 * held from the first call on that GPU until the process ends.  The call
 * allocates nothing (no hipMalloc, no allocating library routine).
 *
 *   - MS_ERR_UNSUPPORTED (nothing launched) when ms_scan_workspace_bytes
 *     exceeds MS_NOALLOC_MAX_BYTES; use ms_scan_fwd with a workspace then.
 *     Shapes that the library runs in one pass (e.g. d_state 9..16 with
 *     batch x d_inner >= 8192) need no scratch at all.
 *   - The scratch used is that of the calling thread's current device; the
 *     stream must belong to that device.
 *   - Every call on one GPU shares that GPU's array (its contents need no
 *     initialisation and are undefined afterwards): two calls that overlap in
 *     time on one GPU (different streams, or different host threads) race.
 *     Calls on one stream are ordered and do not.
 * Other statuses as for ms_scan_fwd; deterministic, with outputs bit-identical
 * to ms_scan_fwd's for the same inputs.
 */
#define MS_NOALLOC_MAX_BYTES ((size_t)64 << 20)
ms_status ms_scan_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                              const void* C, const float* D, const void* z,
                              const float* delta_bias, uint32_t flags, void* y,
                              const float* h0, float* h_last, const ms_dims* dims,
                              void* stream);

/*
 * ms_scan_fwd with the step size's low-rank projection fused into the scan.
 * The step size is softplus of a linear map of the input plus a bias (jsqmd
 * page, section 2.2); in the block that map is low-rank: x_proj yields a
 * narrow dt slice per timestep and dt_proj lifts it to d_inner (lmnt page,
 * section 3.2).  Here the raw step is
 *
 *   delta[b,t,d] = sum_{r < dt_rank} W_dt[d][r] * dt_low[b,t,r]
 *
 * accumulated in fp32 from the io values (exact products for bf16), never
 * rounded to the io type, and the scan then runs exactly as ms_scan_fwd with
 * that delta (bias, softplus flag, discretisation and outputs unchanged).
 *
 *   dt_low : [batch][seqlen][dt_rank] io dtype    (required)
 *   W_dt   : [d_inner][dt_rank] io dtype          (required; the layout of a
 *            linear layer's weight, out x in)
 *   dt_rank: 1 .. 64
 *   all other arguments as for ms_scan_fwd, except the workspace: at least
 *   ms_scan_dtproj_workspace_bytes(dims, flags) bytes (this call runs on
 *   kernels of its own, whose plan may need more than ms_scan_fwd's).
 *
 * Statuses as for ms_scan_fwd; MS_ERR_SHAPE for dt_rank outside 1..64;
 * MS_ERR_UNSUPPORTED unless one of these holds:
 *   d_state 8 or 16;
 *   d_state 9 .. 15 and d_inner a multiple of 8 (bf16 io) or 4 (fp32 io);
 *   d_state 17 .. 32, d_inner a multiple of 8 (bf16) or 4 (fp32) and
 *     batch * ceil(d_inner / 8) >= 512;
 *   d_state 33 .. 128, d_inner a multiple of 4 and
 *     batch * ceil(d_inner / 4) >= 512.
 * Deterministic.
 */
size_t ms_scan_dtproj_workspace_bytes(const ms_dims* dims, uint32_t flags);
ms_status ms_scan_fwd_dtproj(const void* u, const void* dt_low, const void* W_dt,
                             int32_t dt_rank, const float* A, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias,
                             uint32_t flags, void* y, const float* h0, float* h_last,
                             const ms_dims* dims, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * One recurrent decode step for a batch of sequences (one timestep of
 * ms_scan_fwd with the state kept by the caller between calls).
 *
 *   h          : in/out state [batch][d_inner][d_state] fp32, updated in place.
 *   x_t, delta_t, z_t, y_t : [batch][d_inner] io dtype (z_t optional).
 *   B_t, C_t   : [batch][d_state] io dtype.
 *   A, D, delta_bias, flags : as for ms_scan_fwd (D, delta_bias optional).
 *
 * y_t must not overlap any input or h.
 */
ms_status ms_state_update(float* h, const void* x_t, const void* delta_t, const float* A,
                          const void* B_t, const void* C_t, const float* D,
                          const void* z_t, const float* delta_bias, uint32_t flags,
                          void* y_t, int32_t batch, int32_t d_inner, int32_t d_state,
                          int32_t io, void* stream);

/*
 * Gradients of ms_scan_fwd, for training (reverse mode; any d_state 1..128).
 * Given dy = dL/dy ([batch][L][d_inner], io dtype) and optionally dh_last =
 * dL/dh_last ([batch][d_inner][d_state] fp32), returns dL/d of the inputs:
 *   du, ddelta, dz : [batch][L][d_inner] io dtype (ddelta is w.r.t. the raw
 *                    delta, i.e. through the softplus and bias)
 *   dA             : [d_inner][d_state] fp32
 *   dB, dC         : [batch][L][d_state] fp32 (sums over the channels)
 *   dD, dbias      : [d_inner] fp32 (sums over batch and time)
 *   dh0            : [batch][d_inner][d_state] fp32 (w.r.t. h0, or the zero
 *                    initial state when h0 is NULL)
 * The forward inputs, flags and dims are those of the ms_scan_fwd call being
 * differentiated (the forward states are recomputed, nothing is kept from
 * it).  The pages train the model end to end by gradient descent (jsqmd
 * page, section 4.2; lmnt page, section 4.2) and print no derivative: these
 * are the chain rule of the recurrence at the top of this file, run back in
 * time with lambda_t = dL/dh_t = C_t g_t + A_bar_{t+1} lambda_{t+1}.
 *
 *   required: u, delta, A, B, C, dy, du, ddelta, dA, dB, dC, dims, workspace;
 *   dz required when z is given, dD when D is given; dbias, dh0, dh_last,
 *   h0, D, z, delta_bias optional (NULL).  Outputs must not overlap inputs.
 *   workspace: ms_scan_bwd_workspace_bytes(dims, flags) bytes (never 0),
 *   16-byte aligned, no initialisation needed.
 * Statuses as for ms_scan_fwd.  Deterministic: partial sums are added in a
 * fixed order.  Above 16 states the state is differentiated in slices of 16
 * (the recurrence is diagonal, so the per-element gradients are sums over
 * slices), each an fp32 problem with the gate and D taken out, and the
 * workspace holds fp32 intermediates of the whole problem (about 40 bytes
 * per element).
 */
size_t ms_scan_bwd_workspace_bytes(const ms_dims* dims, uint32_t flags);
ms_status ms_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                      const void* C, const float* D, const void* z,
                      const float* delta_bias, uint32_t flags, const float* h0,
                      const void* dy, const float* dh_last, void* du, void* ddelta,
                      float* dA, float* dB, float* dC, float* dD, void* dz, float* dbias,
                      float* dh0, const ms_dims* dims, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Training pair with forward-saved checkpoints: the forward stores the state
 * before every 16-step block beside its outputs, and the backward reads them
 * instead of walking the sequence forward again to recompute them (the first
 * of ms_scan_bwd's passes where it runs on the one-row layout).  Same
 * recurrence and gradients as ms_scan_fwd / ms_scan_bwd (for training end to
 * end: jsqmd page, section 4.2; lmnt page, section 4.2); memory traded for
 * time: the checkpoints take
 * 4 * d_state / 16 bytes per element (4 for d_state 16), against 2 for a bf16
 * input tensor.
 *
 * ms_scan_checkpoint_bytes(dims, flags): bytes of the checkpoint buffer, a
 *   multiple of 256; 0 when this pair does not serve these dims and flags
 *   (then use ms_scan_fwd and ms_scan_bwd); (size_t)-1 for invalid dims or
 *   flags.  It serves d_state 9..16, d_inner a multiple of 8 (bf16 io) or 4
 *   (fp32 io), and batch * ceil(d_inner / 16) >= 512.
 *
 * ms_scan_fwd_checkpoint: ms_scan_fwd (same arguments, outputs and
 *   statuses; no workspace) that also fills
 *     checkpoint : [batch][ceil(seqlen / 16)][d_inner][d_state] fp32
 *                  (required; 16-byte aligned; must not overlap any other
 *                  argument): entry (b, k, d, n) is h[n] of channel d of
 *                  sequence b before step 16k -- h0 (or 0) at k = 0.
 *   MS_ERR_UNSUPPORTED when ms_scan_checkpoint_bytes is 0.  Deterministic.
 *
 * ms_scan_bwd_checkpoint: ms_scan_bwd for the same dims and flags, with the
 *   checkpoint filled by ms_scan_fwd_checkpoint on the same u, delta, A, B,
 *   delta_bias and h0 (read only; h0 itself is not an argument: its
 *   contribution is in the checkpoint), and a workspace of
 *   ms_scan_bwd_checkpoint_workspace_bytes(dims, flags) bytes ((size_t)-1
 *   when ms_scan_checkpoint_bytes is 0, or for invalid dims).  Other
 *   arguments, outputs and statuses as for ms_scan_bwd; MS_ERR_UNSUPPORTED
 *   when ms_scan_checkpoint_bytes is 0.  Deterministic; its gradients are
 *   those ms_scan_bwd computes from the states it recomputes.
 */
size_t ms_scan_checkpoint_bytes(const ms_dims* dims, uint32_t flags);
ms_status ms_scan_fwd_checkpoint(const void* u, const void* delta, const float* A,
                                 const void* B, const void* C, const float* D, const void* z,
                                 const float* delta_bias, uint32_t flags, void* y,
                                 const float* h0, float* h_last, float* checkpoint,
                                 const ms_dims* dims, void* stream);
size_t ms_scan_bwd_checkpoint_workspace_bytes(const ms_dims* dims, uint32_t flags);
ms_status ms_scan_bwd_checkpoint(const void* u, const void* delta, const float* A,
                                 const void* B, const void* C, const float* D, const void* z,
                                 const float* delta_bias, uint32_t flags,
                                 const float* checkpoint, const void* dy, const float* dh_last,
                                 void* du, void* ddelta, float* dA, float* dB, float* dC,
                                 float* dD, void* dz, float* dbias, float* dh0,
                                 const ms_dims* dims, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Causal depthwise conv1d over the sequence, optionally followed by silu: the
 * step of the block that turns the x branch into the scan input u (the
 * lmnt.cn page, section 3.1, puts a depthwise 1D convolution of width about 4
 * ahead of the SSM; its section 3.2 code uses groups = d_inner, width-1 zeros
 * of left padding, keeps the first L outputs and applies silu):
 *
 *   pre[b,t,d] = bias[d] + sum_{k<width} weight[d][k] * x[b, t-(width-1)+k, d]
 *   u[b,t,d]   = silu(pre) = pre * sigmoid(pre)   (silu != 0; else pre)
 *
 * where x at a time before 0 is x_prev[b][width-1 + time][d] when x_prev is
 * given (the width-1 inputs that precede this piece, oldest first, so a long
 * sequence can be processed in pieces or continued after a prefill) and 0
 * otherwise.
 *
 *   x      : [batch][L][d_inner] io dtype            (required)
 *   weight : [d_inner][width] fp32, width in 1..8    (required)
 *   bias   : [d_inner] fp32                          (NULL = no bias)
 *   x_prev : [batch][width-1][d_inner] io dtype      (NULL = zeros; ignored
 *            when width == 1)
 *   u      : [batch][L][d_inner] io dtype; must not overlap x or x_prev.
 *   batch, seqlen, d_inner, io : as in ms_dims (batch, d_inner/256 and the
 *            grid limits of ms_scan_fwd apply).
 * Statuses as for ms_scan_fwd (MS_ERR_SHAPE for a width outside 1..8).  All
 * pointers 16-byte aligned.  Deterministic.
 */
ms_status ms_conv1d_silu(const void* x, const float* weight, const float* bias,
                         const void* x_prev, int32_t width, int32_t silu, void* u,
                         int32_t batch, int64_t seqlen, int32_t d_inner, int32_t io,
                         void* stream);

/* Static text for a status code. */
const char* ms_status_string(ms_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* ms_last_error(void);

/* MS_ABI_VERSION of the loaded library. */
int ms_abi_version(void);

/*
 * Kernel timing, for benchmarks and profiling (not an operation of the
 * method).  Between ms_profile_begin and ms_profile_end, each of the next
 * `max_calls` successful calls of the library's entry points records a pair
 * of HIP events on its own stream around every kernel it launches (up to 64
 * per call), and ms_profile_end waits for those events and returns, per
 * phase, the number of timed launches and their summed kernel time (a call
 * that launches two kernels of one phase, like the backward's two carries,
 * counts two launches):
 *   MS_PHASE_PREP     B/C staging pass
 *   MS_PHASE_SUMMARY  per-segment end states (sequence cut into segments)
 *   MS_PHASE_CARRY    composition of segment summaries into start states
 *   MS_PHASE_MAIN     the scan that writes y (and h_last); the backward's
 *                     per-segment gradient pass
 *   MS_PHASE_STEP     ms_state_update's kernel
 *   MS_PHASE_CONV     ms_conv1d_silu's kernel
 *   MS_PHASE_REDUCE   the backward's fixed-order sums of partial gradients
 * A phase a call does not need records nothing.  Calls after the first
 * max_calls are not timed (out->calls counts the timed ones).  The event
 * records add a few microseconds per kernel to a call's wall time.
 *
 * ms_profile_begin: max_calls in [1, 1024]; creates the events on the current
 *   device (MS_ERR_SHAPE for a bad count, MS_ERR_HIP on event creation
 *   failure, MS_ERR_UNSUPPORTED when a profile is already open).
 * ms_profile_end: out may be NULL (results dropped).  Synchronises on the
 *   recorded events (blocks the host until they complete), frees them and
 *   closes the profile.  MS_ERR_UNSUPPORTED when no profile is open.
 * The profile is process-wide: open it, run the calls, close it from one
 * host thread.
 */
typedef enum {
    MS_PHASE_PREP = 0,
    MS_PHASE_SUMMARY = 1,
    MS_PHASE_CARRY = 2,
    MS_PHASE_MAIN = 3,
    MS_PHASE_STEP = 4,
    MS_PHASE_CONV = 5,
    MS_PHASE_REDUCE = 6,
    MS_PHASE_COUNT = 7
} ms_phase;

typedef struct {
    int32_t calls;                     /* calls timed                     */
    int32_t launches[MS_PHASE_COUNT];  /* kernel launches timed per phase */
    double total_ms[MS_PHASE_COUNT];   /* summed kernel time per phase    */
} ms_profile;

ms_status ms_profile_begin(int32_t max_calls);
ms_status ms_profile_end(ms_profile* out);

#ifdef __cplusplus
}
#endif

#endif /* MSSCAN_H */
