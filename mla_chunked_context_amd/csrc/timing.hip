// Event bracketing of kernel launches for live per-kernel timing.
#include <atomic>
#include <mutex>
#include <vector>

#include "device.h"

namespace mla {

namespace {

struct Record {
    int kind;
    hipEvent_t start, end;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_free;

hipEvent_t take_event() {
    // caller holds g_mu
    if (!g_free.empty()) {
        hipEvent_t e = g_free.back();
        g_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

TimedLaunch::TimedLaunch(int kind, hipStream_t stream) : kind_(kind), stream_(stream) {
    if (!g_enabled.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lock(g_mu);
    start_ = take_event();
    if (start_ != nullptr && hipEventRecord(start_, stream_) != hipSuccess) {
        g_free.push_back(start_);
        start_ = nullptr;
    }
}

TimedLaunch::~TimedLaunch() {
    if (start_ == nullptr) return;
    std::lock_guard<std::mutex> lock(g_mu);
    hipEvent_t end = take_event();
    if (end == nullptr || hipEventRecord(end, stream_) != hipSuccess) {
        g_free.push_back(start_);
        if (end != nullptr) g_free.push_back(end);
        return;
    }
    g_records.push_back(Record{kind_, start_, end});
}

}  // namespace mla

extern "C" {

int mla_kernel_timing_enable(int enable) {
    std::lock_guard<std::mutex> lock(mla::g_mu);
    mla::g_enabled.store(enable != 0);
    if (enable == 0) {
        for (auto& r : mla::g_records) {
            hipEventSynchronize(r.end);
            mla::g_free.push_back(r.start);
            mla::g_free.push_back(r.end);
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
        mla::g_free.push_back(r.start);
        mla::g_free.push_back(r.end);
    }
    mla::g_records.clear();
    return st;
}

}  // extern "C"
