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

constexpr int kMaxCalls = 1024;
constexpr int kMaxLaunchesPerCall = 64;  // event pairs kept per timed call (the d_state 17-128
                                         // backward launches ~40 kernels)

// One pair of events per kernel launch: a call may launch several kernels of
// one phase (the backward's two carries), and each launch is timed on its own.
struct Profile {
    std::atomic<bool> on{false};
    std::mutex mu;
    int max_calls = 0;
    int call = -1;                  // index of the call being recorded
    int launches_in_call = 0;       // pairs taken by the current call
    int open = -1;                  // pair whose end event is pending
    std::vector<hipEvent_t> ev;     // [pair][edge]
    std::vector<int> phase_of;      // [pair]: phase, or -1 (unused)
    std::vector<unsigned char> done;  // [pair]: end event recorded
    size_t next = 0;                // next free pair
};

Profile& prof() {
    static Profile p;
    return p;
}

void release(Profile& p) {
    for (hipEvent_t e : p.ev)
        if (e) (void)hipEventDestroy(e);
    p.ev.clear();
    p.phase_of.clear();
    p.done.clear();
    p.next = 0;
    p.max_calls = 0;
    p.call = -1;
    p.open = -1;
    p.launches_in_call = 0;
}

}  // namespace

void prof_call() {
    Profile& p = prof();
    if (!p.on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> g(p.mu);
    if (p.call < p.max_calls) ++p.call;
    p.launches_in_call = 0;
    p.open = -1;
}

void prof_mark(hipStream_t s, int phase, int edge) {
    Profile& p = prof();
    if (!p.on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> g(p.mu);
    if (p.call < 0 || p.call >= p.max_calls || phase < 0 || phase >= MS_PHASE_COUNT) return;
    if (edge == 0) {
        if (p.launches_in_call >= kMaxLaunchesPerCall || p.next >= p.phase_of.size()) return;
        const size_t k = p.next++;
        ++p.launches_in_call;
        if (hipEventRecord(p.ev[2 * k], s) != hipSuccess) return;
        p.phase_of[k] = phase;
        p.open = (int)k;
    } else if (p.open >= 0) {
        const size_t k = (size_t)p.open;
        p.open = -1;
        if (p.phase_of[k] == phase && hipEventRecord(p.ev[2 * k + 1], s) == hipSuccess)
            p.done[k] = 1;
    }
}

}  // namespace msscan

extern "C" {

ms_status ms_profile_begin(int32_t max_calls) {
    using namespace msscan;
    if (max_calls < 1 || max_calls > kMaxCalls) return MS_ERR_SHAPE;
    Profile& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (p.on.load()) return MS_ERR_UNSUPPORTED;
    const size_t pairs = (size_t)max_calls * kMaxLaunchesPerCall;
    p.ev.assign(2 * pairs, nullptr);
    p.phase_of.assign(pairs, -1);
    p.done.assign(pairs, 0);
    p.next = 0;
    for (hipEvent_t& e : p.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            release(p);
            return MS_ERR_HIP;
        }
    }
    p.max_calls = max_calls;
    p.call = -1;
    p.open = -1;
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
    r.calls = p.call < 0 ? 0 : (p.call < p.max_calls ? p.call + 1 : p.max_calls);
    for (size_t k = 0; k < p.next; ++k) {
        if (!p.done[k]) continue;
        float ms = 0.f;
        if (hipEventSynchronize(p.ev[2 * k + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, p.ev[2 * k], p.ev[2 * k + 1]) != hipSuccess) {
            st = MS_ERR_HIP;
            continue;
        }
        r.launches[p.phase_of[k]] += 1;
        r.total_ms[p.phase_of[k]] += ms;
    }
    release(p);
    if (out) *out = r;
    return st;
}

}  // extern "C"
