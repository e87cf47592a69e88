// Cross-lane reductions of a wavefront without LDS traffic (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swin {
namespace lanes {

// v_permlane16_swap (v_permlane32_swap) exchanges the odd 16-lane rows
// (32-lane halves) of its first operand with the even ones of its second:
// given x twice, every lane gets back its own x and that of lane ^ 16 (^ 32),
// in one order or the other.
__device__ __forceinline__ float sum_x16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_x16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// DPP row_ror:N, a rotation within each row of 16 lanes
template <int N>
__device__ __forceinline__ float row_ror(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

enum class Op { Sum, Max, Min };
template <Op OP>
__device__ __forceinline__ float combine(float a, float b)
{
    return OP == Op::Sum ? a + b : OP == Op::Max ? fmaxf(a, b) : fminf(a, b);
}

// sum, maximum or minimum over the 64 lanes, in every lane
template <Op OP>
__device__ __forceinline__ float wave_reduce(float x)
{
    x = combine<OP>(x, row_ror<8>(x));
    x = combine<OP>(x, row_ror<4>(x));
    x = combine<OP>(x, row_ror<2>(x));
    x = combine<OP>(x, row_ror<1>(x));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = combine<OP>(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return combine<OP>(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace lanes
}  // namespace swin
