// Log-spaced continuous position bias table (SwinV2 card, Method item 3,
// eq. 3-4): for every relative offset (dy, dx) in [-(M-1), M-1]^2 the meta
// network G = W2 relu(W1 (f(dx), f(dy)) + b1) + b2 with f(x) = sign(x)
// ln(1+|x|) is evaluated once and stored, one column per head.  The
// released code's variants (SwinV2 card, Paper vs code) are flags of `mode`:
// CODE_NORM maps an offset x to u = 8 x / (norm_M - 1), then to
// sign(u) log2(1+|u|) / log2(8); SIGMOID16 bounds the output to
// 16 sigmoid(G).
//
// One wavefront per (offset, group of up to four heads): lane j evaluates
// hidden units j, j + 64, ... of its offset and accumulates their share of
// the group's output dot products, then a cross-lane sum finishes them.  All
// weights a wavefront needs are requested at once (one memory latency per
// 512 hidden units), and nothing is shared between wavefronts: no LDS, no
// barrier.  The hidden layer is recomputed per head group (2 of the ~2 + HG
// multiply-adds per unit).  At most 41 MFLOP for a 47 x 47 offset grid.
#include "common.hpp"
#include "lanes.hpp"
#include "launch.hpp"

namespace swin {

namespace {

constexpr int HG = 4;          // heads per wavefront
constexpr int UPL = 8;         // hidden units per lane and pass (512 per pass)

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kNoLoad = 0x80000000u;     // beyond every record count here: reads zero
__device__ __forceinline__ Rsrc rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float ld1(Rsrc r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 ld2(Rsrc r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

__device__ __forceinline__ float signed_log1p(int x)
{
    return x > 0 ? log1pf((float)x) : (x < 0 ? -log1pf((float)-x) : 0.0f);
}

// G's input for offset x under `mode`
__device__ __forceinline__ float cpb_input(int x, int mode, float norm_scale)
{
    if (!(mode & SWIN_CPB_CODE_NORM)) return signed_log1p(x);
    const float u = (float)x * norm_scale;          // 8 x / (norm_M - 1)
    const float a = log2f(1.0f + fabsf(u)) * (1.0f / 3.0f);
    return u > 0.0f ? a : (u < 0.0f ? -a : 0.0f);
}

__global__ void __launch_bounds__(256)
cpb_table_kernel(int M, int heads, int hidden, const float* __restrict__ w1, const float* __restrict__ b1,
                 const float* __restrict__ w2, const float* __restrict__ b2, float* __restrict__ table,
                 int items, int mode, float norm_scale)
{
    const int lane = threadIdx.x & 63;
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (item >= items) return;
    const int groups = (heads + HG - 1) / HG;
    const int row = item / groups;                 // (dy + M-1)*S + (dx + M-1)
    const int o0 = (item - row * groups) * HG;     // first head of the group
    const int S = 2 * M - 1;
    const float fx = cpb_input(row % S - (M - 1), mode, norm_scale);
    const float fy = cpb_input(row / S - (M - 1), mode, norm_scale);

    // null biases: an empty resource, whose loads read zero
    const Rsrc r1 = rsrc(w1, (uint32_t)hidden * 8u);
    const Rsrc rb1 = rsrc(b1, b1 ? (uint32_t)hidden * 4u : 0u);
    const Rsrc r2 = rsrc(w2, (uint32_t)(heads * hidden) * 4u);
    float acc[HG] = {};
    for (int u0 = 0; u0 < hidden; u0 += 64 * UPL) {
        u32x2 w[UPL];
        float bb[UPL], v2[HG][UPL];
#pragma unroll
        for (int k = 0; k < UPL; ++k) {
            const int u = u0 + k * 64 + lane;
            const bool ok = u < hidden;
            w[k] = ld2(r1, ok ? (uint32_t)u * 8u : kNoLoad);
            bb[k] = ld1(rb1, ok ? (uint32_t)u * 4u : kNoLoad);
#pragma unroll
            for (int o = 0; o < HG; ++o)
                v2[o][k] = ld1(r2, ok && o0 + o < heads ? (uint32_t)((o0 + o) * hidden + u) * 4u : kNoLoad);
        }
#pragma unroll
        for (int k = 0; k < UPL; ++k) {
            // input 0 is the column (width) offset, input 1 the row offset
            const float a = fmaf(__uint_as_float(w[k][0]), fx, fmaf(__uint_as_float(w[k][1]), fy, bb[k]));
            const float hk = fmaxf(a, 0.0f);
#pragma unroll
            for (int o = 0; o < HG; ++o) acc[o] = fmaf(v2[o][k], hk, acc[o]);
        }
    }
    float mine = 0.0f;
#pragma unroll
    for (int o = 0; o < HG; ++o) {
        const float s = lanes::wave_reduce<lanes::Op::Sum>(acc[o]);
        mine = lane == o ? s : mine;
    }
    if (lane < HG && o0 + lane < heads) {
        float g = mine + (b2 ? b2[o0 + lane] : 0.0f);
        if (mode & SWIN_CPB_SIGMOID16) g = 16.0f / (1.0f + expf(-g));
        table[(size_t)row * heads + o0 + lane] = g;
    }
}

}  // namespace

hipError_t launch_cpb_table(int M, int norm_M, int heads, int hidden, const float* w1, const float* b1,
                            const float* w2, const float* b2, int mode, float* table, hipStream_t stream)
{
    const int S = 2 * M - 1;
    const int items = S * S * ((heads + HG - 1) / HG);
    const float norm_scale = norm_M > 1 ? 8.0f / (float)(norm_M - 1) : 0.0f;
    cpb_table_kernel<<<(items + 3) / 4, 256, 0, stream>>>(M, heads, hidden, w1, b1, w2, b2, table, items, mode,
                                                          norm_scale);
    return hipGetLastError();
}

}  // namespace swin
