// Device helpers shared by the kernels of libswinattn.so: window geometry,
// token addressing for both partitions, shift-region intervals, bf16 moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swin_attn.h"

namespace swin {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Shape of one attention call, as the kernels see it.
struct Geometry {
    int B, H, W, C, heads, d;
    int M, shift, part, layout;
    int nwr, nwc;   // window rows (H/M) and columns (W/M) per image
    int N;          // tokens per window, M*M
    int nwin;       // windows in the batch, B*nwr*nwc
};

// Element offset of the first channel of local token (r, c) of window `win`.
// Cyclic partition ("Swin V1's" partition of the SwinV2 card, rolled by
// -shift): grid ((wr*M + r + shift) mod H, (wc*M + c + shift) mod W).
// Interleaved partition (Iwin): grid (wr + r*H/M, wc + c*W/M).
__device__ __forceinline__ int64_t token_offset(const Geometry& g, int win, int r, int c)
{
    if (g.layout == SWIN_LAYOUT_WINDOWS)
        return ((int64_t)win * g.N + r * g.M + c) * g.C;
    const int nW = g.nwr * g.nwc;
    const int b = win / nW;
    const int w = win - b * nW;
    const int wr = w / g.nwc;
    const int wc = w - wr * g.nwc;
    int gi, gj;
    if (g.part == SWIN_PART_INTERLEAVED) {
        gi = wr + r * g.nwr;
        gj = wc + c * g.nwc;
    } else {
        gi = wr * g.M + r + g.shift;
        if (gi >= g.H) gi -= g.H;
        gj = wc * g.M + c + g.shift;
        if (gj >= g.W) gj -= g.W;
    }
    return (((int64_t)b * g.H + gi) * g.W + gj) * g.C;
}

// Local positions [lo, hi) along one axis that a token at local position p of
// window index w (of nw along that axis) may attend to.  Only the last window
// of a shifted axis is split: rolled coordinates [L-M, L-s) and [L-s, L) are
// the two regions it holds, i.e. local [0, M-s) and [M-s, M).
__device__ __forceinline__ void region_interval(int w, int nw, int M, int s, int p, int& lo, int& hi)
{
    if (s == 0 || w != nw - 1) { lo = 0; hi = M; }
    else if (p < M - s)        { lo = 0; hi = M - s; }
    else                       { lo = M - s; hi = M; }
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ void unpack_bf16x8(const u32x4 w, float* f)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* f)
{
    f32x8 v = {f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]};
    return __builtin_convertvector(v, bf16x8);   // round to nearest even
}

__device__ __forceinline__ bf16x4 pack_bf16x4(float a, float b, float c, float d)
{
    f32x4 v = {a, b, c, d};
    return __builtin_convertvector(v, bf16x4);
}

}  // namespace swin
