// device.hip -- per-device facts read once (see device.h).
#include "device.h"

namespace {
std::once_flag cu_once[MOE_MAX_DEVICES];
int cu_count[MOE_MAX_DEVICES];
hipError_t cu_err[MOE_MAX_DEVICES];

hipError_t current_device(int* dev) {
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return e;
    return (*dev >= 0 && *dev < MOE_MAX_DEVICES) ? hipSuccess : hipErrorInvalidDevice;
}
}  // namespace

hipError_t current_device_cus(int* ncu) {
    int dev = 0;
    hipError_t e = current_device(&dev);
    if (e != hipSuccess) return e;
    std::call_once(cu_once[dev], [dev] {
        cu_err[dev] = hipDeviceGetAttribute(&cu_count[dev], hipDeviceAttributeMultiprocessorCount, dev);
        if (cu_err[dev] == hipSuccess && cu_count[dev] <= 0) cu_err[dev] = hipErrorInvalidValue;
    });
    *ncu = cu_count[dev];
    return cu_err[dev];
}

hipError_t LdsLimit::ensure(const void* fn, int bytes) {
    int dev = 0;
    hipError_t e = current_device(&dev);
    if (e != hipSuccess) return e;
    std::call_once(once_[dev], [this, dev, fn, bytes] {
        err_[dev] = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    });
    return err_[dev];
}
