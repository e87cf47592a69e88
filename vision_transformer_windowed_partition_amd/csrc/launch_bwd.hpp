// Entry points of the backward kernels (vector ALUs and matrix cores) and
// of the CPB table's backward, used by the C-ABI layer.
#pragma once

#include "launch.hpp"

namespace swin {

hipError_t launch_cpb_table_bwd(int M, int norm_M, int heads, int hidden, const float* w1, const float* b1,
                                const float* w2, const float* table, const float* dtable, int mode, float* dw1,
                                float* db1, float* dw2, float* db2, hipStream_t stream);

// Backward of the window attention (vector ALUs; d = 32, M <= 64 where the
// statistics and table fit LDS; the matrix-core kernels take bf16 M <= 32).
bool attn_bwd_supported(const AttnParams& p);
hipError_t launch_attn_bwd(const AttnParams& p, const void* out, const void* dout, void* dq, void* dk, void* dv,
                           float* dtau, float* dtable, hipStream_t stream);

// Backward on the matrix cores (called by launch_attn_bwd after it zeroes
// dtau and dtable): bf16 windows of at most 256 key slots without rotary
// positions (small), else bf16 windows up to M = 32 whose staging fits LDS,
// rotary positions with DOT only (large).
bool attn_bwd_large_supported(const AttnParams& p);
hipError_t launch_attn_bwd_large(const AttnParams& p, const void* out, const void* dout, void* dq, void* dk,
                                 void* dv, float* dtau, float* dtable, hipStream_t stream);
bool attn_bwd_small_supported(const AttnParams& p);
hipError_t launch_attn_bwd_small(const AttnParams& p, const void* out, const void* dout, void* dq, void* dk,
                                 void* dv, float* dtau, float* dtable, hipStream_t stream);

}  // namespace swin
