// Host-side helpers shared by the C-ABI translation units: divisor
// constants for the kernels' multiply-shift division, integer logarithms and
// argument checks.
#pragma once

#include <stdint.h>

#include "msda.h"
#include "msda_device.hpp"

namespace msda_host {

inline msda::FastDiv make_fast_div(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d) ++l;
    const uint64_t shift = 31 + l;
    const uint64_t mul = ((uint64_t{1} << shift) + d - 1) / d;  // <= 2^32 - 1
    return msda::FastDiv{static_cast<uint32_t>(mul), static_cast<uint32_t>(shift)};
}

inline int floor_log2(int64_t x) {
    int r = 0;
    while ((int64_t{2} << r) <= x) ++r;
    return r;
}

inline int ceil_log2(int64_t x) {
    int r = 0;
    while ((int64_t{1} << r) < x) ++r;
    return r;
}

inline bool known_dtype(int dt) { return dt == MSDA_F32 || dt == MSDA_BF16; }

inline bool aligned(const void* ptr, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0;
}

// Compute units of the current device (0 if the query fails).
inline int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

}  // namespace msda_host
