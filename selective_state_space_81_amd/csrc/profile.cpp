// profile.cpp -- HIP-event timing of the library's own kernel launches
// (ms_profile_begin / ms_profile_end).  Off by default: prof_mark then costs
// one relaxed atomic load.
#include "../../include/msscan.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>
#include <vector>

#include "msscan_internal.h"

namespace msscan {
namespace {

constexpr int kMaxCalls = 4096;

struct Profile {
    std::atomic<bool> on{false};
    std::mutex mu;
    int max_calls = 0;
    int call = -1;                 // index of the call being recorded
    std::vector<hipEvent_t> ev;    // [call][phase][edge]
    std::vector<unsigned char> used;  // [call][phase]
};

Profile& prof() {
    static Profile p;
    return p;
}

void release(Profile& p) {
    for (hipEvent_t e : p.ev)
        if (e) (void)hipEventDestroy(e);
    p.ev.clear();
    p.used.clear();
    p.max_calls = 0;
    p.call = -1;
}

}  // namespace

void prof_call() {
    Profile& p = prof();
    if (!p.on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> g(p.mu);
    if (p.call < p.max_calls) ++p.call;
}

void prof_mark(hipStream_t s, int phase, int edge) {
    Profile& p = prof();
    if (!p.on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> g(p.mu);
    if (p.call < 0 || p.call >= p.max_calls || phase < 0 || phase >= MS_PHASE_COUNT) return;
    const size_t k = (size_t)p.call * MS_PHASE_COUNT + (size_t)phase;
    if (hipEventRecord(p.ev[2 * k + (edge ? 1 : 0)], s) == hipSuccess && edge) p.used[k] = 1;
}

}  // namespace msscan

extern "C" {

ms_status ms_profile_begin(int32_t max_calls) {
    using namespace msscan;
    if (max_calls < 1 || max_calls > kMaxCalls) return MS_ERR_SHAPE;
    Profile& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (p.on.load()) return MS_ERR_UNSUPPORTED;
    const size_t n = (size_t)max_calls * MS_PHASE_COUNT;
    p.ev.assign(2 * n, nullptr);
    p.used.assign(n, 0);
    for (hipEvent_t& e : p.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            release(p);
            return MS_ERR_HIP;
        }
    }
    p.max_calls = max_calls;
    p.call = -1;
    p.on.store(true);
    return MS_OK;
}

ms_status ms_profile_end(ms_profile* out) {
    using namespace msscan;
    Profile& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.on.load()) return MS_ERR_UNSUPPORTED;
    p.on.store(false);
    ms_profile r{};
    ms_status st = MS_OK;
    const int calls = p.call < 0 ? 0 : (p.call < p.max_calls ? p.call + 1 : p.max_calls);
    r.calls = calls;
    for (int c = 0; c < calls; ++c) {
        for (int ph = 0; ph < MS_PHASE_COUNT; ++ph) {
            const size_t k = (size_t)c * MS_PHASE_COUNT + (size_t)ph;
            if (!p.used[k]) continue;
            float ms = 0.f;
            if (hipEventSynchronize(p.ev[2 * k + 1]) != hipSuccess ||
                hipEventElapsedTime(&ms, p.ev[2 * k], p.ev[2 * k + 1]) != hipSuccess) {
                st = MS_ERR_HIP;
                continue;
            }
            r.launches[ph] += 1;
            r.total_ms[ph] += ms;
        }
    }
    release(p);
    if (out) *out = r;
    return st;
}

}  // extern "C"
