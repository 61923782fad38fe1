// Host-side launch helpers shared by the libbq8 sources: device properties
// cached per device, and each kernel's opt-in to the device's full dynamic
// LDS, made once per kernel and device.  Safe to call from several host
// threads and with any device current.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace bq8 {

constexpr int HOST_MAX_DEVICES = 64;

// Index of the current device, or -1.
inline int host_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= HOST_MAX_DEVICES)
        return -1;
    return dev;
}

// Integer attribute A of the current device, queried once per device; -1
// without a device or when the query fails.
template <hipDeviceAttribute_t A> inline int64_t device_attr()
{
    static std::atomic<int64_t> cached[HOST_MAX_DEVICES];
    const int dev = host_device();
    if (dev < 0)
        return -1;
    const int64_t v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0)
        return v;
    int q = 0;
    if (hipDeviceGetAttribute(&q, A, dev) != hipSuccess || q <= 0)
        return -1;
    cached[dev].store(q, std::memory_order_relaxed);
    return q;
}

// Compute units of the current device, or -1.
inline int64_t device_cus()
{
    return device_attr<hipDeviceAttributeMultiprocessorCount>();
}

// Largest dynamic LDS a workgroup may use on the current device (160 KB on
// gfx950); 64 KB when the device cannot be queried.
inline int64_t device_lds_limit()
{
    const int64_t v = device_attr<hipDeviceAttributeMaxSharedMemoryPerBlock>();
    return v > 0 ? v : 65536;
}

// Lets `kernel` take up to `limit` bytes of dynamic LDS on the current
// device: hipFuncSetAttribute once per (kernel, device), later calls find
// the pair in a table.  False if the attribute cannot be set.
inline bool allow_dynamic_lds(const void *kernel, int64_t limit)
{
    struct Done {
        const void *kernel;
        int dev;
    };
    static std::mutex mu;
    static Done done[1024];
    static int ndone = 0;
    const int dev = host_device();
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < ndone; ++i)
        if (done[i].kernel == kernel && done[i].dev == dev)
            return true;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)limit) !=
        hipSuccess)
        return false;
    if (ndone < 1024)
        done[ndone++] = Done{kernel, dev};
    return true;
}

} // namespace bq8
