// Internal helpers shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/winattn.h"

namespace winattn {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
inline bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

inline int element_bytes(int32_t dtype) {
    switch (dtype) {
        case WIN_DTYPE_BF16:
        case WIN_DTYPE_FP16:
            return 2;
        case WIN_DTYPE_FP32:
            return 4;
        default:
            return 0;
    }
}

// Status of the launch just enqueued.
inline int launch_status() { return hipGetLastError() == hipSuccess ? WIN_OK : WIN_EDEVICE; }

}  // namespace winattn
