// ev_api.hip -- status strings and the per-device facts the launchers need (gfx950 only).
#include <cstring>
#include <mutex>

#include "ev_internal.h"

namespace {
constexpr int kMaxDevices = 16;
std::mutex g_mu;
int g_checked[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
int g_cus[kMaxDevices];

void probe(int dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        g_checked[dev] = -1;
        return;
    }
    g_checked[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_cus[dev] = prop.multiProcessorCount;
}
}  // namespace

namespace ev {

int current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    return dev;
}

ev_status check_device() {
    const int dev = current_device();
    if (dev < 0 || dev >= kMaxDevices) return EV_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_checked[dev] == 0) probe(dev);
    return g_checked[dev] == 1 ? EV_OK : EV_ERR_DEVICE;
}

int device_cu_count() {
    const int dev = current_device();
    if (dev < 0 || dev >= kMaxDevices) return 1;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_checked[dev] == 0) probe(dev);
    return g_cus[dev] > 0 ? g_cus[dev] : 1;
}

}  // namespace ev

extern "C" const char *ev_status_string(ev_status status) {
    switch (status) {
        case EV_OK: return "EV_OK";
        case EV_ERR_NULL: return "EV_ERR_NULL: a required pointer is NULL";
        case EV_ERR_SHAPE: return "EV_ERR_SHAPE: unsupported or inconsistent sizes";
        case EV_ERR_DTYPE: return "EV_ERR_DTYPE: unsupported element type";
        case EV_ERR_ALIGN: return "EV_ERR_ALIGN: pointer, stride or row size breaks the 16-byte rules";
        case EV_ERR_WORKSPACE: return "EV_ERR_WORKSPACE: workspace missing or too small";
        case EV_ERR_DEVICE: return "EV_ERR_DEVICE: the current device is not gfx950";
        case EV_ERR_HIP: return "EV_ERR_HIP: a HIP runtime call or kernel launch failed";
    }
    return "EV_ERR_UNKNOWN";
}
