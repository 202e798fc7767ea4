// ABI version, status strings and device queries.

#include "common.h"

namespace tav {

int device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
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
