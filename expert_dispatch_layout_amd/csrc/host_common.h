// Host-side helpers shared by the entry points of libmep.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mep.h"

namespace mep {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? MEP_OK : MEP_ERR_DEVICE;
}

inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace mep
