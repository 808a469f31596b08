// Runtime queries of the host dispatch: the compute-unit count of the current
// device, which sizes the split policy's grid (the kaispace blog, section 4.2,
// lists the grid dimensions as search parameters; here the rule fills the
// chip the call runs on).

#include <hip/hip_runtime_api.h>

#include <atomic>

#include "mga_internal.h"

namespace mga {

int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> per_device[kMaxDevices] = {};  // 0: not asked yet
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCUs;
    int n = per_device[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = kDefaultCUs;
    per_device[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace mga
