// Log-spaced continuous position bias table (SwinV2 card, Method item 3,
// eq. 3-4): for every relative offset (dy, dx) in [-(M-1), M-1]^2 the meta
// network G = W2 relu(W1 (f(dx), f(dy)) + b1) + b2 with f(x) = sign(x)
// ln(1+|x|) is evaluated once and stored, one column per head.  The
// released code's variants (SwinV2 card, Paper vs code) are flags of `mode`:
// CODE_NORM is the code's coordinate table, an offset x mapped to
// u = 8 x / (norm_M - 1), then to sign(u) log2(1+|u|) / log2(8), with the
// row offset as G's first input (the page leaves the order open; the SwinV2
// port in transformers stacks (row, column)); SIGMOID16 bounds the output to
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
#include "launch_bwd.hpp"

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

// G's two inputs for table row (dy + M-1)(2M-1) + (dx + M-1): (f(dx), f(dy))
// in the paper's form, (f(dy), f(dx)) in the code's coordinate table
__device__ __forceinline__ void cpb_inputs(int row, int M, int mode, float norm_scale, float& in0, float& in1)
{
    const int S = 2 * M - 1;
    const float fx = cpb_input(row % S - (M - 1), mode, norm_scale);
    const float fy = cpb_input(row / S - (M - 1), mode, norm_scale);
    const bool code = (mode & SWIN_CPB_CODE_NORM) != 0;
    in0 = code ? fy : fx;
    in1 = code ? fx : fy;
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
    float in0, in1;
    cpb_inputs(row, M, mode, norm_scale, in0, in1);

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
            const float a = fmaf(__uint_as_float(w[k][0]), in0, fmaf(__uint_as_float(w[k][1]), in1, bb[k]));
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

// Backward of the table: gradients of G's parameters from dtable.  Per table
// row, a = W1 x + b1, hid = relu(a); dg = dtable (SIGMOID16: times
// dT/dG = T (1 - T/16), T the forward table); dW2 += dg hid^T, db2 += dg,
// dhid = W2^T dg, da = dhid [a > 0], dW1 += da x^T, db1 += da.
// Thread = hidden unit, workgroup = (256 units, BR table rows, HB heads): it
// sums its rows in registers and adds them to the outputs with one atomic
// per value (the outputs start at zero).  dhid is linear in dg, so the head
// blocks' partial dW1 and db1 add up.
constexpr int BR = 64;         // table rows per workgroup
constexpr int HB = 16;         // heads per workgroup

__global__ void __launch_bounds__(256)
cpb_table_bwd_kernel(int M, int heads, int hidden, const float* __restrict__ w1, const float* __restrict__ b1,
                     const float* __restrict__ w2, const float* __restrict__ table,
                     const float* __restrict__ dtable, int mode, float norm_scale, float* __restrict__ dw1,
                     float* __restrict__ db1, float* __restrict__ dw2, float* __restrict__ db2)
{
    __shared__ float sdg[BR * HB];                 // dg of this block's rows and heads
    __shared__ float sin0[BR], sin1[BR];           // G's inputs for those rows
    const int u = blockIdx.x * 256 + threadIdx.x;
    const int S = 2 * M - 1;
    const int row0 = blockIdx.y * BR, row1 = min(row0 + BR, S * S);
    const int o0 = blockIdx.z * HB;
    // dg = dtable (times dT/dG for SIGMOID16) for the block, all loads at once
    for (int i = threadIdx.x; i < BR * HB; i += 256) {
        const int row = row0 + i / HB, o = o0 + i % HB;
        float dg = 0.0f;
        if (row < row1 && o < heads) {
            const size_t at = (size_t)row * heads + o;
            dg = dtable[at];
            if (mode & SWIN_CPB_SIGMOID16) { const float t = table[at]; dg *= t * (1.0f - t * (1.0f / 16.0f)); }
        }
        sdg[i] = dg;
    }
    if (threadIdx.x < BR) {
        const int row = min(row0 + (int)threadIdx.x, S * S - 1);
        cpb_inputs(row, M, mode, norm_scale, sin0[threadIdx.x], sin1[threadIdx.x]);
    }
    __syncthreads();
    const bool unit = u < hidden;
    float w10 = 0.0f, w11 = 0.0f, bb = 0.0f, w2c[HB];
#pragma unroll
    for (int o = 0; o < HB; ++o) w2c[o] = unit && o0 + o < heads ? w2[(size_t)(o0 + o) * hidden + u] : 0.0f;
    if (unit) { w10 = w1[2 * u]; w11 = w1[2 * u + 1]; bb = b1 ? b1[u] : 0.0f; }
    float gw2[HB], g0 = 0.0f, g1 = 0.0f, gb = 0.0f, gb2 = 0.0f;
#pragma unroll
    for (int o = 0; o < HB; ++o) gw2[o] = 0.0f;
    // db2 of head o0 + threadIdx.x, in the first unit block
    const bool own_b2 = blockIdx.x == 0 && threadIdx.x < HB && o0 + threadIdx.x < heads;
    for (int row = row0; row < row1; ++row) {
        const float x0 = sin0[row - row0], x1 = sin1[row - row0];
        const float a = fmaf(w10, x0, fmaf(w11, x1, bb));
        const float hid = fmaxf(a, 0.0f);
        float dh = 0.0f;
#pragma unroll
        for (int o = 0; o < HB; ++o) {
            const float dg = sdg[(row - row0) * HB + o];     // zero past the last head
            gw2[o] = fmaf(dg, hid, gw2[o]);
            dh = fmaf(w2c[o], dg, dh);
            if (own_b2 && o == (int)threadIdx.x) gb2 += dg;
        }
        const float da = a > 0.0f ? dh : 0.0f;
        g0 = fmaf(da, x0, g0);
        g1 = fmaf(da, x1, g1);
        gb += da;
    }
    if (unit) {
#pragma unroll
        for (int o = 0; o < HB; ++o)
            if (o0 + o < heads) unsafeAtomicAdd(&dw2[(size_t)(o0 + o) * hidden + u], gw2[o]);
        unsafeAtomicAdd(&dw1[2 * u], g0);
        unsafeAtomicAdd(&dw1[2 * u + 1], g1);
        if (db1) unsafeAtomicAdd(&db1[u], gb);
    }
    if (own_b2 && db2) unsafeAtomicAdd(&db2[o0 + threadIdx.x], gb2);
}

__global__ void zero4_kernel(float* a, int na, float* b, int nb, float* c, int nc, float* d, int nd)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (a && i < na) a[i] = 0.0f;
    if (b && i < nb) b[i] = 0.0f;
    if (c && i < nc) c[i] = 0.0f;
    if (d && i < nd) d[i] = 0.0f;
}

}  // namespace

hipError_t launch_cpb_table_bwd(int M, int norm_M, int heads, int hidden, const float* w1, const float* b1,
                                const float* w2, const float* table, const float* dtable, int mode, float* dw1,
                                float* db1, float* dw2, float* db2, hipStream_t stream)
{
    const int S = 2 * M - 1;
    const int n = max(max(2 * hidden, heads * hidden), heads);
    zero4_kernel<<<(n + 255) / 256, 256, 0, stream>>>(dw1, 2 * hidden, db1, hidden, dw2, heads * hidden, db2,
                                                       heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float norm_scale = norm_M > 1 ? 8.0f / (float)(norm_M - 1) : 0.0f;
    dim3 grid((hidden + 255) / 256, (S * S + BR - 1) / BR, (heads + HB - 1) / HB);
    cpb_table_bwd_kernel<<<grid, 256, 0, stream>>>(M, heads, hidden, w1, b1, w2, table, dtable, mode, norm_scale,
                                                   dw1, db1, dw2, db2);
    return hipGetLastError();
}

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

// ---- a Swin V1 bias table at a new window size: each head's (2Ms-1)^2
// table resampled bi-cubically to (2Md-1)^2 (SwinV2 card, Problem and tab. 1),
// by separable cubic convolution with Keys' kernel (a = -0.75), sample
// centres aligned and the border replicated.  One thread per output entry and
// head; weights and sums in fp32.
namespace {

__device__ __forceinline__ float keys_w(float t)
{
    constexpr float a = -0.75f;
    const float u = fabsf(t);
    if (u <= 1.0f) return ((a + 2.0f) * u - (a + 3.0f)) * u * u + 1.0f;
    if (u < 2.0f) return ((a * u - 5.0f * a) * u + 8.0f * a) * u - 4.0f * a;
    return 0.0f;
}

__global__ void __launch_bounds__(256)
table_resize_kernel(int Ss, int Sd, int heads, const float* src, float* dst)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= Sd * Sd * heads) return;
    const int h = i % heads, yx = i / heads, y = yx / Sd, x = yx - y * Sd;
    const float scale = (float)Ss / (float)Sd;
    const float sy = ((float)y + 0.5f) * scale - 0.5f, sx = ((float)x + 0.5f) * scale - 0.5f;
    const int y0 = (int)floorf(sy), x0 = (int)floorf(sx);
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int iy = min(max(y0 - 1 + m, 0), Ss - 1);
        const float wy = keys_w(sy - (float)(y0 - 1 + m));
        float row = 0.0f;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int ix = min(max(x0 - 1 + n, 0), Ss - 1);
            row = fmaf(keys_w(sx - (float)(x0 - 1 + n)), src[((size_t)iy * Ss + ix) * heads + h], row);
        }
        acc = fmaf(wy, row, acc);
    }
    dst[i] = acc;
}

}  // namespace

hipError_t launch_table_resize(int Ms, int Md, int heads, const float* src, float* dst, hipStream_t stream)
{
    const int Ss = 2 * Ms - 1, Sd = 2 * Md - 1;
    const int n = Sd * Sd * heads;
    table_resize_kernel<<<(n + 255) / 256, 256, 0, stream>>>(Ss, Sd, heads, src, dst);
    return hipGetLastError();
}

}  // namespace swin
