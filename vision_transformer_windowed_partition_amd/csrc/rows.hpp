// One head's 32 channels of a token as fp32 registers: loads and stores for
// fp32 and bf16 tensors (16-byte accesses).
#pragma once

#include "common.hpp"

namespace swin {

template <typename T> __device__ __forceinline__ void load_row32(const T* p, float* f);
template <> __device__ __forceinline__ void load_row32<float>(const float* p, float* f)
{
    const float4* v = (const float4*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 x = v[i];
        f[4 * i] = x.x; f[4 * i + 1] = x.y; f[4 * i + 2] = x.z; f[4 * i + 3] = x.w;
    }
}
template <> __device__ __forceinline__ void load_row32<uint16_t>(const uint16_t* p, float* f)
{
    const u32x4* v = (const u32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack_bf16x8(v[i], f + 8 * i);
}

template <typename T> __device__ __forceinline__ void store_row32(T* p, const float* f);
template <> __device__ __forceinline__ void store_row32<float>(float* p, const float* f)
{
    float4* v = (float4*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
}
template <> __device__ __forceinline__ void store_row32<uint16_t>(uint16_t* p, const float* f)
{
    bf16x8* v = (bf16x8*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack_bf16x8(f + 8 * i);
}

}  // namespace swin
