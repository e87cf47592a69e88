// Internal launch interface between the C-ABI layer (api.cpp) and the
// kernel translation units.  Arguments reaching these functions are already
// validated.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace swin {

struct AttnParams {
    Geometry g;
    int sim, pos, dtype;
    float tau_min, rope_base;
    const void* q;
    const void* k;
    const void* v;
    void* out;
    const float* tau;
    const float* table;
    const float* rope_freqs;
    // per (window, head, query slot) natural-log log-sum-exp of the
    // logits, fp32, n_windows x heads x N: written by a forward when not
    // NULL, read by a backward when not NULL (which then skips its own pass)
    float* lse = nullptr;
};

hipError_t launch_window_copy(const void* src, void* dst, const Geometry& g, int elem_size,
                              bool to_windows, hipStream_t stream);

hipError_t launch_cpb_table(int M, int norm_M, int heads, int hidden, const float* w1, const float* b1,
                            const float* w2, const float* b2, int mode, float* table, hipStream_t stream);
hipError_t launch_table_resize(int Ms, int Md, int heads, const float* src, float* dst, hipStream_t stream);

// fp32 (and any-shape fallback) attention on the vector ALUs.
hipError_t launch_attn_valu(const AttnParams& p, hipStream_t stream);

// bf16 attention on the matrix cores (d == 32), any window size.
hipError_t launch_attn_mfma(const AttnParams& p, hipStream_t stream);

// bf16 attention for windows of at most 256 key slots without rotary
// positions, each window-head's keys and values staged once in LDS.
bool attn_small_supported(const AttnParams& p);
hipError_t launch_attn_small(const AttnParams& p, hipStream_t stream);

// bf16 attention for windows of 16 < M <= 32 and for rotary positions at
// M <= 32: one workgroup per window-head, its keys and values staged in LDS
// once.
bool attn_large_supported(const AttnParams& p);
hipError_t launch_attn_large(const AttnParams& p, hipStream_t stream);

}  // namespace swin
