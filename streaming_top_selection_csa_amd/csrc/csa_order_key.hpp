// csa_order_key.hpp -- the score <-> sortable-key map shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace csa {

// Monotone map float -> uint32 (larger float -> larger key), -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

}  // namespace csa
