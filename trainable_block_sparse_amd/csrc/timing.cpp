// Kernel timing sessions (infv2_timing_start / infv2_timing_stop): a pair of HIP
// events per launch of one kernel family, stamped by the launch itself
// (launch_timed) or recorded on the stream around a scope (KernelTimer).
// Benchmark support only; the method's entry points never depend on it.
#include <hip/hip_runtime.h>

#include <mutex>
#include <utility>
#include <vector>

#include "../../include/infv2.h"
#include "kernels.hpp"

namespace {

struct Session {
    std::mutex mu;
    int kernel = -1;                                   // -1: no session open
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs;
    std::vector<hipEvent_t> pool;                      // reused events
};

Session& session() {
    static Session s;
    return s;
}

hipEvent_t take_event(Session& s) {
    if (!s.pool.empty()) {
        hipEvent_t e = s.pool.back();
        s.pool.pop_back();
        return e;
    }
    // timing only: no system-scope fence, so recording the event adds no L2
    // write-back and invalidation to the timed kernel
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

bool capturing(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;   // be conservative
    return cs != hipStreamCaptureStatusNone;
}

}  // namespace

namespace infv2 {

KernelTimer::KernelTimer(int kernel, hipStream_t st) : st_(st) {
    Session& s = session();
    std::lock_guard<std::mutex> lk(s.mu);
    if (s.kernel != kernel || capturing(st)) return;
    hipEvent_t a = take_event(s), b = take_event(s);
    if (!a || !b) return;
    hipEventRecord(a, st);
    s.pairs.emplace_back(a, b);
    stop_ = b;
}

KernelTimer::~KernelTimer() {
    if (stop_) hipEventRecord(static_cast<hipEvent_t>(stop_), st_);
}

void launch_events(int kernel, hipStream_t st, hipEvent_t* start, hipEvent_t* stop) {
    *start = *stop = nullptr;
    Session& s = session();
    std::lock_guard<std::mutex> lk(s.mu);
    if (s.kernel != kernel || capturing(st)) return;
    hipEvent_t a = take_event(s), b = take_event(s);
    if (!a || !b) {
        if (a) s.pool.push_back(a);
        if (b) s.pool.push_back(b);
        return;
    }
    s.pairs.emplace_back(a, b);
    *start = a;
    *stop = b;
}

}  // namespace infv2

extern "C" {

int32_t infv2_timing_start(int32_t kernel) {
    if (kernel < 0 || kernel >= INFV2_KERNEL_COUNT) return INFV2_ERR_SHAPE;
    Session& s = session();
    std::lock_guard<std::mutex> lk(s.mu);
    if (s.kernel >= 0) return INFV2_ERR_SHAPE;
    s.kernel = kernel;
    return INFV2_OK;
}

int32_t infv2_timing_stop(double* total_ms, int32_t* launches) {
    Session& s = session();
    std::lock_guard<std::mutex> lk(s.mu);
    if (s.kernel < 0) return INFV2_ERR_SHAPE;
    s.kernel = -1;
    double sum = 0.0;
    int32_t st = INFV2_OK;
    for (auto& pr : s.pairs) {
        float ms = 0.f;
        if (hipEventSynchronize(pr.second) != hipSuccess ||
            hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
            st = INFV2_ERR_DEVICE;
        sum += ms;
        s.pool.push_back(pr.first);
        s.pool.push_back(pr.second);
    }
    const int32_t n = static_cast<int32_t>(s.pairs.size());
    s.pairs.clear();
    if (total_ms) *total_ms = sum;
    if (launches) *launches = n;
    return st;
}

}  // extern "C"
