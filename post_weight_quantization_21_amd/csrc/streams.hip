// The side streams of the library, and optional event timing of kernel groups.
#include <mutex>
#include <vector>

#include "common.h"

namespace gptq {

hipError_t side_stream(SidePurpose purpose, SideStream *&out) {
    constexpr int kMaxDevices = 64;
    static SideStream ss[kSidePurposes][kMaxDevices];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    SideStream &s = ss[purpose][dev];
    if (!s.st) {
        hipStream_t st = nullptr, st2 = nullptr;
        if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return e;
        if ((e = hipStreamCreateWithFlags(&st2, hipStreamNonBlocking)) != hipSuccess) return e;
        for (int i = 0; i < SideStream::kEvents; ++i)
            if ((e = hipEventCreateWithFlags(&s.ev[i], hipEventDisableTiming)) != hipSuccess) return e;
        s.st2 = st2;
        s.st = st;
    }
    out = &s;
    return hipSuccess;
}

hipError_t signal_wait(hipEvent_t ev, hipStream_t from, hipStream_t to) {
    hipError_t e = hipEventRecord(ev, from);
    if (e != hipSuccess) return e;
    return hipStreamWaitEvent(to, ev, 0);
}

// ---------------------------------------------------------------------------
// Event timing: while enabled, each TimedScope records a start and a stop
// event on its stream; timing_read waits for them and sums the elapsed times.
// ---------------------------------------------------------------------------
namespace {
struct TimingState {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> pool;
    struct Rec {
        hipEvent_t start, stop;
        double work;
    };
    std::vector<Rec> pending[kTimedOps];
};
TimingState &timing() {
    static TimingState t;
    return t;
}
hipEvent_t take_event(TimingState &t) {
    if (!t.pool.empty()) {
        hipEvent_t ev = t.pool.back();
        t.pool.pop_back();
        return ev;
    }
    hipEvent_t ev = nullptr;
    return hipEventCreate(&ev) == hipSuccess ? ev : nullptr;
}
}  // namespace

void timing_set(bool on) {
    TimingState &t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    t.on = on;
}

TimedScope::TimedScope(TimedOp op, hipStream_t s, double work) : op_(op), s_(s), work_(work) {
    TimingState &t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    if (!t.on) return;
    start_ = take_event(t);
    stop_ = take_event(t);
    if (start_ && stop_ && hipEventRecord(start_, s_) == hipSuccess) return;
    if (start_) t.pool.push_back(start_);
    if (stop_) t.pool.push_back(stop_);
    start_ = stop_ = nullptr;
}

TimedScope::~TimedScope() {
    if (!start_) return;
    TimingState &t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    if (hipEventRecord(stop_, s_) == hipSuccess) {
        t.pending[op_].push_back({start_, stop_, work_});
    } else {
        t.pool.push_back(start_);
        t.pool.push_back(stop_);
    }
}

hipError_t timing_read(TimedOp op, double *ms, int64_t *count, double *work) {
    TimingState &t = timing();
    std::lock_guard<std::mutex> lock(t.mu);
    double sum = 0.0, w = 0.0;
    hipError_t err = hipSuccess;
    for (auto &r : t.pending[op]) {
        float el = 0.0f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&el, r.start, r.stop);
        if (e != hipSuccess && err == hipSuccess) err = e;
        sum += el;
        w += r.work;
        t.pool.push_back(r.start);
        t.pool.push_back(r.stop);
    }
    *ms = sum;
    *work = w;
    *count = (int64_t)t.pending[op].size();
    t.pending[op].clear();
    return err;
}

}  // namespace gptq
