// device_info.cpp — properties of the current device that the launchers read on the host,
// looked up once per device.
#include <hip/hip_runtime.h>

#include <atomic>

#include "launchers.hpp"

namespace mi355 {

int device_cu_count() {
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace mi355
