// Runtime glue of libh3block: device architecture check and launch-status
// translation. The library keeps no other state.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>

#include "h3_runtime.h"

namespace h3 {

namespace {
constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture.
std::atomic<int> g_arch_state[kMaxDevices];
}  // namespace

// Failed HIP calls are reported on stderr (the status code alone cannot carry
// the runtime's reason).
static int hip_fail(hipError_t e, const char *what) {
    std::fprintf(stderr, "libh3block: %s failed: %s (%d)\n", what, hipGetErrorString(e), (int)e);
    return H3_ERR_HIP;
}

int device_check() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return H3_ERR_DEVICE;
    int s = g_arch_state[dev].load(std::memory_order_relaxed);
    if (s == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        s = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_state[dev].store(s, std::memory_order_relaxed);
    }
    return s == 1 ? H3_OK : H3_ERR_DEVICE;
}

int launch_status() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? H3_OK : hip_fail(e, "kernel launch");
}

}  // namespace h3
