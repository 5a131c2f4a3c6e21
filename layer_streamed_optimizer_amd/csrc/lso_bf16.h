// BF16 conversions used by the fused kernel (and by the probe that checks
// the rounding against the host definition over all 2^32 FP32 patterns).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lso {

// BF16 round to nearest, ties to even, from the FP32 bit pattern: adding
// 0x7FFF plus the lowest kept bit carries into the kept half exactly when
// the dropped half is above the midpoint, or at it with an odd kept half.
// A carry out of the significand bumps the exponent (next binade, or +-Inf
// on overflow).  NaN keeps sign and top payload bits and is made quiet.
// Subnormals round like any other value (no flush to zero).
__device__ __forceinline__ uint32_t bf16_rne(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const bool is_nan = (u & 0x7FFFFFFFu) > 0x7F800000u;
    return is_nan ? ((u >> 16) | 0x0040u) : rounded;
}

// BF16 is the upper half of an FP32 pattern: widening is exact.
__device__ __forceinline__ float bf16_widen(uint32_t h16) { return __uint_as_float(h16 << 16); }

}  // namespace lso
