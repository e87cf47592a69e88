// Window partition (gather) and reverse (scatter): a bit-exact copy of one
// C-channel row per token between the (B, H, W, C) grid and the
// (B*nW, M*M, C) window tensor.  Pure HBM traffic: every byte is read once
// and written once; consecutive lanes move consecutive 16-byte pieces of a
// row, and consecutive rows of a window row are consecutive grid tokens (up
// to one wrap of the cyclic roll), so both sides stay coalesced.
#include "common.hpp"
#include "launch.hpp"

namespace swin {

template <typename V>
__global__ void __launch_bounds__(256)
window_copy_kernel(const V* __restrict__ src, V* __restrict__ dst, Geometry g,
                   int vec_per_row, int64_t total_vec, int to_windows)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total_vec; i += stride) {
        const int64_t row = i / vec_per_row;              // window-tensor row = win*N + t
        const int piece = (int)(i - row * vec_per_row);
        const int win = (int)(row / g.N);
        const int t = (int)(row - (int64_t)win * g.N);
        const int r = t / g.M;
        const int c = t - r * g.M;
        const int64_t grid_vec = token_offset(g, win, r, c) / g.C * vec_per_row + piece;
        const int64_t win_vec = row * vec_per_row + piece;
        if (to_windows) dst[win_vec] = src[grid_vec];
        else            dst[grid_vec] = src[win_vec];
    }
}

hipError_t launch_window_copy(const void* src, void* dst, const Geometry& g, int elem_size,
                              bool to_windows, hipStream_t stream)
{
    const int64_t row_bytes = (int64_t)g.C * elem_size;
    const uintptr_t align = (uintptr_t)src | (uintptr_t)dst;
    int vb = 16;
    while (vb > 1 && ((row_bytes % vb) || (align % vb))) vb >>= 1;
    const int vec_per_row = (int)(row_bytes / vb);
    const int64_t total = (int64_t)g.nwin * g.N * vec_per_row;
    if (total == 0) return hipSuccess;
    const int threads = 256;
    int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    Geometry gg = g;
    gg.layout = SWIN_LAYOUT_GRID;
    switch (vb) {
    case 16: window_copy_kernel<u32x4><<<(int)blocks, threads, 0, stream>>>(
                 (const u32x4*)src, (u32x4*)dst, gg, vec_per_row, total, to_windows); break;
    case 8:  window_copy_kernel<u32x2><<<(int)blocks, threads, 0, stream>>>(
                 (const u32x2*)src, (u32x2*)dst, gg, vec_per_row, total, to_windows); break;
    case 4:  window_copy_kernel<uint32_t><<<(int)blocks, threads, 0, stream>>>(
                 (const uint32_t*)src, (uint32_t*)dst, gg, vec_per_row, total, to_windows); break;
    case 2:  window_copy_kernel<uint16_t><<<(int)blocks, threads, 0, stream>>>(
                 (const uint16_t*)src, (uint16_t*)dst, gg, vec_per_row, total, to_windows); break;
    default: window_copy_kernel<uint8_t><<<(int)blocks, threads, 0, stream>>>(
                 (const uint8_t*)src, (uint8_t*)dst, gg, vec_per_row, total, to_windows); break;
    }
    return hipGetLastError();
}

}  // namespace swin
