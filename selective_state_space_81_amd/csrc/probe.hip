// probe.hip -- hardware rate probes for the benchmark (libmsprobe.so, not
// part of libmsscan's C ABI): the rates the scan kernels' rooflines are
// judged against, measured on the GPU that runs them.
//
//   msprobe_exp  : v_exp_f32 issue rate.  Every lane runs kChains independent
//                  chains x <- 2^(-x) (the value settles near 0.64, so no
//                  chain overflows); one transcendental per step.
//   msprobe_fma  : plain fp32 VALU issue rate (v_fma_f32 chains, not packed).
//   msprobe_copy : device-to-device copy of n 16-byte words (read + write),
//                  and msprobe_read: a read-only pass (sum per thread).
// Each launches on the caller's stream and returns the HIP status; the
// caller times the launch with events.  Work counts:
//   exp / fma : blocks * 256 threads * kChains * iters lane-operations.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChains = 8;

__global__ void __launch_bounds__(256) exp_chains(float* out, int iters) {
    float x[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) x[k] = 0.1f * (float)(threadIdx.x & 7) + 0.01f * k;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += x[k];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) fma_chains(float* out, int iters) {
    float x[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) x[k] = 0.1f * (float)(threadIdx.x & 7) + 0.01f * k;
    const float m = 0.999f, c = 0.001f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k) x[k] = fmaf(x[k], m, c);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kChains; ++k) s += x[k];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Each workgroup copies one contiguous chunk of `per` words, kUnroll words
// per thread per pass with the pass's loads issued before its stores (of the
// shapes tried -- grid-stride passes of 1, 4 or 8 words per thread, cached or
// non-temporal, 1k to 16k workgroups -- the fastest on this GPU).
constexpr int kUnroll = 4;

__global__ void __launch_bounds__(256) copy16(const u4* __restrict__ src, u4* __restrict__ dst,
                                              int64_t n, int64_t per) {
    const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(n, b0 + per);
    for (int64_t i = b0 + threadIdx.x; i < b1; i += 256 * kUnroll) {
        u4 v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k)
            if (i + k * 256 < b1) v[k] = __builtin_nontemporal_load(&src[i + k * 256]);
#pragma unroll
        for (int k = 0; k < kUnroll; ++k)
            if (i + k * 256 < b1) __builtin_nontemporal_store(v[k], &dst[i + k * 256]);
    }
}

__global__ void __launch_bounds__(256) read16(const u4* __restrict__ src, uint32_t* out, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u4 v[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) v[k] = __builtin_nontemporal_load(&src[i + k * stride]);
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (; i < n; i += stride) {
        const u4 v = __builtin_nontemporal_load(&src[i]);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// out: blocks * 256 floats.  iters >= 1, blocks >= 1.
int msprobe_exp(float* out, int iters, int blocks, void* stream) {
    if (!out || iters < 1 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(exp_chains, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}

int msprobe_fma(float* out, int iters, int blocks, void* stream) {
    if (!out || iters < 1 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(fma_chains, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}

// src, dst: n 16-byte words each, 16-byte aligned, not overlapping.
int msprobe_copy(const void* src, void* dst, int64_t n, int blocks, void* stream) {
    if (!src || !dst || n < 1 || blocks < 1) return (int)hipErrorInvalidValue;
    const int64_t per = ((n + blocks - 1) / blocks + 255) / 256 * 256;
    hipLaunchKernelGGL(copy16, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u4*>(src), static_cast<u4*>(dst), n, per);
    return (int)hipGetLastError();
}

// out: blocks * 256 words.
int msprobe_read(const void* src, uint32_t* out, int64_t n, int blocks, void* stream) {
    if (!src || !out || n < 1 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read16, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const u4*>(src), out, n);
    return (int)hipGetLastError();
}

}  // extern "C"
