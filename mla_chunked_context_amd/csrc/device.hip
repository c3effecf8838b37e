// Device topology queries shared by the launchers: compute units (the key
// split rule and the persistent attention grid) and XCDs (how workgroups are
// grouped so that those sharing rows run under one L2).
#include <algorithm>
#include <mutex>

#include "device.h"

namespace mla {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_shape_mu;
DeviceShape g_shape[kMaxDevices];
bool g_known[kMaxDevices] = {};

}  // namespace

DeviceShape device_shape() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();  // no visible device: keep the defaults
        return DeviceShape{};
    }
    std::lock_guard<std::mutex> lock(g_shape_mu);
    if (!g_known[dev]) {
        DeviceShape s;
        int cus = 0, xcds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
            s.cus = cus;
        if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && xcds > 0)
            s.xcds = std::min(xcds, kMaxXcd);
        (void)hipGetLastError();
        g_shape[dev] = s;
        g_known[dev] = true;
    }
    return g_shape[dev];
}

}  // namespace mla
