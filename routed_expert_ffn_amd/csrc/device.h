// device.h -- facts about each GPU read once per device, and the one-time
// raise of a kernel's dynamic LDS limit; both safe to call from any thread.
#pragma once
#include <hip/hip_runtime.h>

#include <mutex>

constexpr int MOE_MAX_DEVICES = 64;

// Number of compute units of the current device (read on the first call made
// with that device current, then cached).
hipError_t current_device_cus(int* ncu);

// Raises one kernel's dynamic LDS limit to `bytes` once per device; later calls
// return the first call's status.  Keep one LdsLimit per kernel instantiation
// (a function-local static in its launcher).
class LdsLimit {
  public:
    hipError_t ensure(const void* fn, int bytes);

  private:
    std::once_flag once_[MOE_MAX_DEVICES];
    hipError_t err_[MOE_MAX_DEVICES] = {};
};
