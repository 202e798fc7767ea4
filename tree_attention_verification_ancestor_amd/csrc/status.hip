// ABI version, status strings and device queries.

#include <map>
#include <mutex>
#include <utility>

#include "common.h"

namespace tav {

namespace {
std::mutex g_query_mu;
std::map<int, int> g_cus;                                      // device -> CUs
std::map<std::pair<int, std::pair<const void *, int>>, int> g_occ;   // (device, kernel, threads)
} // namespace

// Both queries are answered once per device (and kernel) and remembered:
// every launch plans its grid from them, and they do not change.
int device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    std::lock_guard<std::mutex> lock(g_query_mu);
    auto it = g_cus.find(dev);
    if (it != g_cus.end())
        return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    g_cus[dev] = cus;
    return cus;
}

int kernel_occupancy(const void *kernel, int threads)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    const auto key = std::make_pair(dev, std::make_pair(kernel, threads));
    std::lock_guard<std::mutex> lock(g_query_mu);
    auto it = g_occ.find(key);
    if (it != g_occ.end())
        return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess)
        return 0;
    g_occ[key] = n;
    return n;
}

} // namespace tav

extern "C" int32_t tav_abi_version(void) { return TAV_ABI_VERSION; }

extern "C" const char *tav_status_string(tav_status status)
{
    switch (status) {
    case TAV_OK:
        return "ok";
    case TAV_ERR_ARG:
        return "invalid argument (null or misaligned pointer, size out of range)";
    case TAV_ERR_UNSUPPORTED:
        return "unsupported shape";
    case TAV_ERR_WORKSPACE:
        return "workspace missing or too small";
    case TAV_ERR_LAUNCH:
        return "kernel launch failed";
    default:
        return "unknown status";
    }
}
