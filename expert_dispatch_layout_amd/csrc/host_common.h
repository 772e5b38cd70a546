// Host-side helpers shared by the entry points of libmep.so.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <tuple>
#include <type_traits>

#include "../../include/mep.h"

namespace mep {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Launch status of an entry point: the first failing return code of its own launches
// (hipExtLaunchKernel reports each launch's result), never an error that an earlier, unrelated
// call left in the runtime.  Kept per host thread: launch_begin() at the start of an entry
// point, launch_status() at its end (which also clears it).
inline thread_local hipError_t t_launch_error = hipSuccess;

inline void launch_begin() { t_launch_error = hipSuccess; }

inline int launch_status() {
    const hipError_t e = t_launch_error;
    t_launch_error = hipSuccess;
    return e == hipSuccess ? MEP_OK : MEP_ERR_DEVICE;
}

// Launches `kernel` with its arguments converted to the kernel's parameter types; start / stop
// (may be null) are events the launch itself records around the kernel.
template <typename... KArgs, typename... Args>
inline void launch_ext(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                       hipEvent_t start, hipEvent_t stop, uint32_t flags, Args&&... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<std::decay_t<KArgs>...> t{static_cast<std::decay_t<KArgs>>(args)...};
    const hipError_t e = std::apply(
        [&](auto&... v) {
            void* p[] = {static_cast<void*>(&v)...};
            return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, p, shmem, st, start, stop,
                                      (int)flags);
        },
        t);
    if (e != hipSuccess && t_launch_error == hipSuccess) t_launch_error = e;
}

template <typename... KArgs, typename... Args>
inline void launch_ggl(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t st,
                       Args&&... args) {
    launch_ext(kernel, grid, block, shmem, st, nullptr, nullptr, 0u, std::forward<Args>(args)...);
}

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (cached per device; 256 if the query fails).
inline int device_units() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace mep
