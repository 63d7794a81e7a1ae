// pa_device_cache.cpp -- per-device facts the launchers need (compute-unit
// count, LDS limit, resident workgroups of a kernel), queried from the HIP
// runtime once per device and kept for the life of the process, so that a
// launch costs no device query after the first one on that device.
#include <mutex>
#include <tuple>
#include <map>

#include "pa_internal.h"

namespace pa {
namespace {

struct DeviceFacts {
    bool known = false;
    DeviceInfo info{};
};

std::mutex g_mutex;
std::map<int, DeviceFacts> g_devices;
std::map<std::tuple<int, const void*, int, size_t>, int> g_occupancy;

}  // namespace

hipError_t current_device_info(int* device, DeviceInfo* info) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    *device = dev;
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceFacts& f = g_devices[dev];
    if (!f.known) {
        DeviceInfo d{};
        e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&d.max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess)
            return e;
        f.info = d;
        f.known = true;
    }
    *info = f.info;
    return hipSuccess;
}

hipError_t resident_workgroups_per_cu(int device, const void* kernel, int threads, size_t lds,
                                      int* per_cu) {
    const auto key = std::make_tuple(device, kernel, threads, lds);
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        const auto it = g_occupancy.find(key);
        if (it != g_occupancy.end()) {
            *per_cu = it->second;
            return hipSuccess;
        }
    }
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(g_mutex);
    g_occupancy[key] = n;
    *per_cu = n;
    return hipSuccess;
}

}  // namespace pa
