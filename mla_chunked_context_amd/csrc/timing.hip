// Event bracketing of kernel launches for live per-kernel timing.
#include <atomic>
#include <map>
#include <mutex>
#include <vector>

#include "device.h"

namespace mla {

namespace {

struct Record {
    int kind;
    int device;
    hipEvent_t start, end;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Record> g_records;
// recycled events, per device: an event is recorded only on streams of the
// device that was current when it was created
std::map<int, std::vector<hipEvent_t>> g_free;

hipEvent_t take_event(int device) {
    // caller holds g_mu; `device` is the current device
    std::vector<hipEvent_t>& pool = g_free[device];
    if (!pool.empty()) {
        hipEvent_t e = pool.back();
        pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

TimedLaunch::TimedLaunch(int kind, hipStream_t stream) : kind_(kind), stream_(stream) {
    if (!g_enabled.load(std::memory_order_relaxed)) return;
    if (hipGetDevice(&device_) != hipSuccess) return;
    std::lock_guard<std::mutex> lock(g_mu);
    start_ = take_event(device_);
    if (start_ != nullptr && hipEventRecord(start_, stream_) != hipSuccess) {
        g_free[device_].push_back(start_);
        start_ = nullptr;
    }
}

TimedLaunch::~TimedLaunch() {
    if (start_ == nullptr) return;
    std::lock_guard<std::mutex> lock(g_mu);
    hipEvent_t end = take_event(device_);
    if (end == nullptr || hipEventRecord(end, stream_) != hipSuccess) {
        g_free[device_].push_back(start_);
        if (end != nullptr) g_free[device_].push_back(end);
        return;
    }
    g_records.push_back(Record{kind_, device_, start_, end});
}

}  // namespace mla

extern "C" {

int mla_kernel_timing_enable(int enable) {
    std::lock_guard<std::mutex> lock(mla::g_mu);
    mla::g_enabled.store(enable != 0);
    if (enable == 0) {
        for (auto& r : mla::g_records) {
            hipEventSynchronize(r.end);
            mla::g_free[r.device].push_back(r.start);
            mla::g_free[r.device].push_back(r.end);
        }
        mla::g_records.clear();
    }
    return MLA_OK;
}

int mla_kernel_timing_read(mla_kernel_time* times) {
    if (times == nullptr) return MLA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(mla::g_mu);
    int st = MLA_OK;
    for (auto& r : mla::g_records) {
        float ms = 0.f;
        if (hipEventSynchronize(r.end) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.end) != hipSuccess) {
            st = MLA_ERR_HIP;
        } else if (r.kind >= 0 && r.kind < MLA_KERNEL_KINDS) {
            times[r.kind].launches += 1;
            times[r.kind].total_ms += ms;
        }
        mla::g_free[r.device].push_back(r.start);
        mla::g_free[r.device].push_back(r.end);
    }
    mla::g_records.clear();
    return st;
}

}  // extern "C"
