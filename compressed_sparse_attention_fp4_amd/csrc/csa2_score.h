// Device helpers of the MXFP4 index-score kernels (the plain scoring kernel and the
// fused score + select kernel).
#pragma once

#include "csa2_device.h"

namespace csa2 {

// max(x, 0) for a float through its bit pattern: a signed-integer max with 0 keeps every
// x >= +0 and maps negative values and -0 to +0, in one instruction (a float max would
// first quiet possible signalling NaNs).
__device__ __forceinline__ float relu_bits(float x)
{
    const int b = __float_as_int(x);
    return __int_as_float(b > 0 ? b : 0);
}

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Loads with a constant byte offset (the offset folds into the instruction).  They are
// ordinary loads, so the compiler tracks them and waits for each register it reads; the
// code issues them early and in a fixed order, so the compiler's waits let the next key
// tiles stay in flight while the current ones are scored.
template <int OFF>
__device__ __forceinline__ u32x4_t gload_x4(const void* p)
{
    return *reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(p) + OFF);
}
template <int OFF>
__device__ __forceinline__ int gload_u8(const void* p)
{
    return static_cast<const uint8_t*>(p)[OFF];
}
template <int OFF>
__device__ __forceinline__ int gload_i32(const void* p)
{
    return *reinterpret_cast<const int32_t*>(static_cast<const uint8_t*>(p) + OFF);
}
template <int OFF>
__device__ __forceinline__ float gload_f32(const void* p)
{
    return *reinterpret_cast<const float*>(static_cast<const uint8_t*>(p) + OFF);
}

}  // namespace csa2
