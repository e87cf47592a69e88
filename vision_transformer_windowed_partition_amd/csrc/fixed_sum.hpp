// Sums of floats in LDS as 64-bit fixed point with 32 fraction bits.
//
// The backward's bias-gradient sums add many terms per table entry from
// every lane of a workgroup.  On gfx950, LDS fp32 atomic adds (ds_add_f32)
// cost about a hundred cycles per wavefront instruction; 64-bit integer ones
// (ds_add_u64) run at the LDS's own rate.  An integer sum is also exact and
// independent of the order the lanes arrive in.  Each term is truncated
// toward zero to a multiple of 2^-32 (an error below 2^-32 per term), and
// both the terms and the running sums must stay below 2^31 in magnitude.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swin {
namespace fixed {

typedef unsigned long long acc_t;

__device__ __forceinline__ acc_t to_fixed(float x)
{
    const float a = fabsf(x);
    const float hi = floorf(a);                                  // exact integer part
    const uint32_t lo = (uint32_t)((a - hi) * 4294967296.0f);    // a - hi is exact in fp32
    const acc_t m = ((acc_t)(uint32_t)hi << 32) | lo;
    return x < 0.0f ? 0ull - m : m;
}

__device__ __forceinline__ float from_fixed(acc_t v)
{
    return (float)((double)(long long)v * 0x1p-32);
}

// *p += x on an LDS accumulator
__device__ __forceinline__ void add(acc_t* p, float x) { atomicAdd(p, to_fixed(x)); }

}  // namespace fixed
}  // namespace swin
