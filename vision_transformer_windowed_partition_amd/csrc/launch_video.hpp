// Attention over video (3D) windows and their three-offset bias table, used
// by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace swin {

// (B, T, H, W, C) channels-last grid, windows Mt x M x M, d = 32 channels a
// head.  Token (t, r, c) of a window is local slot (t*M + r)*M + c; windows
// run image, temporal, row, column.
struct VideoArgs {
    int B, T, H, W, C, heads;
    int Mt, M, shift_t, shift, part;
    int sim, pos, dtype;
    int nwt, nwr, nwc, N, nwin;
    float tau_min;
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const float* tau;
    const float* table;
};

// LDS bytes the kernel needs with kc keys staged at a time (0 if no kc fits).
size_t video_lds(const VideoArgs& a, int* kc);
hipError_t launch_attn_video(const VideoArgs& a, hipStream_t stream);

// The same on the matrix cores: bf16, M <= 22, no rotary positions.
bool video_mfma_supported(const VideoArgs& a);
hipError_t launch_attn_video_mfma(const VideoArgs& a, hipStream_t stream);
hipError_t launch_cpb_table3d(int Mt, int M, int heads, int hidden, const float* w1, const float* b1,
                              const float* w2, const float* b2, float* table, hipStream_t stream);

}  // namespace swin
