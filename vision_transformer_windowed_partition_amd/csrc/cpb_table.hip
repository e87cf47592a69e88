// Log-spaced continuous position bias table (SwinV2 card, Method item 3,
// eq. 3-4): for every relative offset (dy, dx) in [-(M-1), M-1]^2 the meta
// network G = W2 relu(W1 (f(dx), f(dy)) + b1) + b2 with f(x) = sign(x)
// ln(1+|x|) is evaluated once and stored, one column per head.
//
// One workgroup per offset: its threads evaluate the hidden layer into LDS,
// then each wavefront reduces the output-layer dot products of a subset of
// heads.  At most 41 MFLOP for a 47 x 47 offset grid: latency bound, run once
// per layer and window size, never inside the attention call.
#include "common.hpp"
#include "launch.hpp"

namespace swin {

__global__ void __launch_bounds__(256)
cpb_table_kernel(int M, int heads, int hidden, const float* __restrict__ w1,
                 const float* __restrict__ b1, const float* __restrict__ w2,
                 const float* __restrict__ b2, float* __restrict__ table)
{
    extern __shared__ float hid[];                 // hidden activations of this offset
    const int S = 2 * M - 1;
    const int row = blockIdx.x;                    // (dy + M-1)*S + (dx + M-1)
    const int dy = row / S - (M - 1);
    const int dx = row % S - (M - 1);
    const float fx = dx > 0 ? log1pf((float)dx) : (dx < 0 ? -log1pf((float)-dx) : 0.0f);
    const float fy = dy > 0 ? log1pf((float)dy) : (dy < 0 ? -log1pf((float)-dy) : 0.0f);
    for (int j = threadIdx.x; j < hidden; j += blockDim.x) {
        float a = fmaf(w1[2 * j], fx, fmaf(w1[2 * j + 1], fy, b1 ? b1[j] : 0.0f));
        hid[j] = a > 0.0f ? a : 0.0f;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwave = blockDim.x >> 6;
    for (int o = wave; o < heads; o += nwave) {
        const float* w = w2 + (size_t)o * hidden;
        float acc = 0.0f;
        for (int j = lane; j < hidden; j += 64) acc = fmaf(w[j], hid[j], acc);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
        if (lane == 0) table[(size_t)row * heads + o] = acc + (b2 ? b2[o] : 0.0f);
    }
}

hipError_t launch_cpb_table(int M, int heads, int hidden, const float* w1, const float* b1,
                            const float* w2, const float* b2, float* table, hipStream_t stream)
{
    const int S = 2 * M - 1;
    cpb_table_kernel<<<S * S, 256, (size_t)hidden * sizeof(float), stream>>>(
        M, heads, hidden, w1, b1, w2, b2, table);
    return hipGetLastError();
}

}  // namespace swin
