// Launch entries of the kernels either side of the attention and of its
// alternatives (proj.hip, attn_fused.hip, dwconv.hip, window_linear.hip), called by api.hip
// after the host-side validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace swin {

struct ProjArgs {
    const void* x;             // QKV: input features; NORM: attention output o (T x C)
    const void* w;             // QKV: 3C x C; NORM: C x C (output rows, input columns)
    const float* b;            // bias per output row, or nullptr
    void *q, *k, *v;           // QKV outputs (T x C each)
    const void* resid;         // NORM: main path (T x C)
    const float *gamma, *beta; // NORM: per-channel scale and shift (C)
    float eps;                 // NORM: added to the variance inside the root
    void* y;                   // NORM output (T x C); may equal resid
    int64_t T;                 // tokens
    int C;                     // channels
    int dtype;                 // SWIN_DT_F32 or SWIN_DT_BF16
};

struct DwconvArgs {
    const void* v;             // (B, H, W, C) values
    const float* w;            // C x 3 x 3 taps
    const float* b;            // C bias, or nullptr
    void* out;                 // (B, H, W, C) attention output, updated in place
    int B, H, W, C;
    int dtype;
};

struct WlinArgs {
    const void* A;             // heads x N x N, the features' dtype
    const float* bias;         // heads x N, or nullptr
};

struct FusedArgs {
    const void* x;             // (B, H, W, C) features
    const void* w;             // 3C x C input-layer weight (rows q, k, v)
    const float* b;            // 3C bias, or nullptr
};

bool proj_supported(int C);
// window attention with the input layer fused in (attn_fused.hip): p holds
// the geometry, modes, tau, table and out (p.q, p.k, p.v unused)
bool attn_fused_supported(const AttnParams& p);
hipError_t launch_attn_fused(const AttnParams& p, const FusedArgs& a, hipStream_t stream);
bool dwconv_supported(int C, int dtype);
hipError_t launch_dwconv_add(const DwconvArgs& a, hipStream_t stream);
// p: geometry, dtype, v and out of the window mapping (launch.hpp)
hipError_t launch_window_linear(const AttnParams& p, const WlinArgs& la, hipStream_t stream);
hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t stream);
hipError_t launch_proj_norm(const ProjArgs& a, hipStream_t stream);

}  // namespace swin
