// LinMapper's aggregation inside each window ("What Makes for Hierarchical
// Vision Transformer?", abstract: self-attention replaced by a simple linear
// mapping layer inside each non-overlapped window, Swin's cross-window
// communication kept):
//   out[i] = bias_h[i] + sum_j A_h[i][j] v[j]
// per window and head over the head's d channels, A_h an N x N matrix shared
// by all windows, the pairs of a shifted window's different regions excluded
// as in the attention.  Windows, shift and interleaving as in the attention
// kernels: the partition is fused into the loads and stores.
//
// bf16, M = 8 or 16: the attention's second product with the weights given.
// A workgroup of four wavefronts serves one head (M = 16: four windows
// shared, query tiles rank + 4j; M = 8: a window per wavefront).  V rows go to LDS by
// LDS-DMA and come back as V^T fragments (ds_read_b64_tr_b16); the B operand
// of O^T = V^T A^T is 8 consecutive entries of one row of A_h, a 16-byte load
// that every window of the head finds in L2; in windows with shift regions
// the entries of excluded pairs are zeroed in registers.
// fp32, and other M: one thread per output, fp32.
#include "common.hpp"
#include "launch.hpp"
#include "launch_proj.hpp"
#include "tile_io.hpp"

namespace swin {

namespace {

using namespace tio;

template <int M>
__global__ void __launch_bounds__(256) wlin_kernel(AttnParams p, WlinArgs la, int units, int per_xcd)
{
    constexpr int N = M * M, NCH = N / 32, QW = M == 16 ? 4 : 1, WH = 4 / QW;
    constexpr int NQT = N / 16, SETS = 2 * NCH / QW, GPR = M / 8;
    __shared__ __attribute__((aligned(16))) __bf16 vst_all[WH * N * D];
    const Geometry& g = p.g;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    const int wh = wave / QW, rank = wave - wh * QW;
    // work ids window-block-major, head-minor; each XCD a contiguous range
    const int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (work >= units) return;                            // whole workgroup, before the barrier
    const int h = work % g.heads;
    const int wloc = (work / g.heads) * WH + wh;
    const bool active = wloc < g.nwin;
    const WinPlace wp = place_window(g, active ? wloc : 0);
    const WinGeo& wg = wp.wg;
    const uint32_t bytes = (uint32_t)(wp.span - h * D) * 2u;
    const RawRsrc vraw = raw_rsrc((const uint16_t*)p.v + wp.base + h * D, active ? bytes : 0u);
    const Rsrc orr = make_rsrc((const uint16_t*)p.out + wp.base + h * D, bytes);
    __bf16* vst = vst_all + wh * N * D;

    // V piece j (1 KB of LDS, this wave: j = rank + QW k): lane l fills 16
    // bytes at position 16 l, i.e. slot 16 j + l/4 (slot = token, M a
    // multiple of 8), LDS piece l%4, holding channel piece (l%4) ^ v_swizzle
#pragma unroll
    for (int k = 0; k < SETS; ++k) {
        const int j = rank + QW * k;
        const int s = 16 * j + (lane >> 2);
        const int gam = s >> 3;
        const int rj = gam / GPR, cj = 8 * (gam % GPR) + (s & 7);
        const int piece = (lane & 3) ^ v_swizzle(s);
        dma16(vraw, vst + (size_t)j * 512, wg.tok(rj, cj) + 16u * piece);
    }
    vm_wait_all();
    __syncthreads();
    if (!active) return;

    const bool needs_mask = wp.last_r || wp.last_c;
    const __bf16* Ah = (const __bf16*)la.A + (size_t)h * N * N;
    for (int t = rank; t < NQT; t += QW) {
        const int qi = 16 * t + li;                       // this lane's query (token)
        const int ri = qi / M, ci = qi - ri * M;
        int rlo = 0, rhi = M, clo = 0, chi = M;
        if (needs_mask) {
            region_interval(wp.last_r ? g.nwr - 1 : 0, g.nwr, M, g.shift, ri, rlo, rhi);
            region_interval(wp.last_c ? g.nwc - 1 : 0, g.nwc, M, g.shift, ci, clo, chi);
        }
        f32x4 o0 = {0.0f, 0.0f, 0.0f, 0.0f}, o1 = o0;
        const __bf16* arow = Ah + (size_t)qi * N + 8 * grp;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            u32x4 bw = *(const u32x4*)(arow + 32 * c);
            if (needs_mask) {
                // keys 32c + 8 grp + x: row rj, columns cj0 + x
                const int j0 = 32 * c + 8 * grp, rj = j0 / M, cj0 = j0 - rj * M;
                const bool rok = rj >= rlo && rj < rhi;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int x0 = cj0 + 2 * e;
                    const uint32_t lo = rok && x0 >= clo && x0 < chi ? 0x0000ffffu : 0u;
                    const uint32_t hi = rok && x0 + 1 >= clo && x0 + 1 < chi ? 0xffff0000u : 0u;
                    bw[e] &= lo | hi;
                }
            }
            const bf16x8 B = __builtin_bit_cast(bf16x8, bw);
            o0 = mfma(vt_frag(vst, c, 0, grp, li), B, o0);
            o1 = mfma(vt_frag(vst, c, 1, grp, li), B, o1);
        }
        // lane holds channels 4 grp..+3 and 16 + 4 grp..+3 of query qi
        const float b = la.bias ? la.bias[(size_t)h * N + qi] : 0.0f;
        const uint32_t off = wg.tok(ri, ci) + 8u * grp;
        store8(orr, off, pack_bf16x4(o0[0] + b, o0[1] + b, o0[2] + b, o0[3] + b));
        store8(orr, off + 32u, pack_bf16x4(o1[0] + b, o1[1] + b, o1[2] + b, o1[3] + b));
    }
}

// bf16, M = 16: a workgroup of four wavefronts serves one head and WPG
// windows, whose V rows all sit in LDS; a wavefront takes query tiles
// rank + 4j and, per 32-key chunk, loads the B operand (8 entries of a row
// of A_h) once for all WPG windows, so A_h crosses L2 once per WPG windows.
constexpr int WPG = 4;

__global__ void __launch_bounds__(256) wlin16_kernel(AttnParams p, WlinArgs la, int units, int per_xcd)
{
    constexpr int M = 16, N = 256, NCH = N / 32, NQT = N / 16, SETS = 2 * NCH / 4;
    __shared__ __attribute__((aligned(16))) __bf16 vst_all[WPG * N * D];
    const Geometry& g = p.g;
    const int tid = threadIdx.x, lane = tid & 63;
    const int rank = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    const int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (work >= units) return;                            // whole workgroup, before the barrier
    const int h = work % g.heads;
    const int w0 = (work / g.heads) * WPG;

    // V of each window: piece j (1 KB) of window w filled as in wlin_kernel
#pragma unroll
    for (int w = 0; w < WPG; ++w) {
        const int win = w0 + w;
        const bool act = win < g.nwin;
        const WinPlace wp = place_window(g, act ? win : 0);
        const uint32_t bytes = (uint32_t)(wp.span - h * D) * 2u;
        const RawRsrc vraw = raw_rsrc((const uint16_t*)p.v + wp.base + h * D, act ? bytes : 0u);
        __bf16* vst = vst_all + w * N * D;
#pragma unroll
        for (int k = 0; k < SETS; ++k) {
            const int j = rank + 4 * k;
            const int sl = 16 * j + (lane >> 2);
            const int rj = sl >> 4, cj = sl & 15;
            const int piece = (lane & 3) ^ v_swizzle(sl);
            dma16(vraw, vst + (size_t)j * 512, wp.wg.tok(rj, cj) + 16u * piece);
        }
    }
    vm_wait_all();
    __syncthreads();

    const __bf16* Ah = (const __bf16*)la.A + (size_t)h * N * N;
    for (int t = rank; t < NQT; t += 4) {
        const int qi = 16 * t + li;                       // this lane's query (token)
        const int ri = qi / M, ci = qi - ri * M;
        f32x4 o0[WPG], o1[WPG];
#pragma unroll
        for (int w = 0; w < WPG; ++w) { o0[w] = f32x4{0.0f, 0.0f, 0.0f, 0.0f}; o1[w] = o0[w]; }
        // shift regions: the last window row and column of a shifted grid
        int rlo[2], rhi[2], clo[2], chi[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            rlo[e] = 0; rhi[e] = M; clo[e] = 0; chi[e] = M;
            if (e == 1) {
                region_interval(g.nwr - 1, g.nwr, M, g.shift, ri, rlo[1], rhi[1]);
                region_interval(g.nwc - 1, g.nwc, M, g.shift, ci, clo[1], chi[1]);
            }
        }
        const __bf16* arow = Ah + (size_t)qi * N + 8 * grp;
#pragma unroll 2
        for (int c = 0; c < NCH; ++c) {
            const u32x4 bw = *(const u32x4*)(arow + 32 * c);
            const int j0 = 32 * c + 8 * grp, rj = j0 / M, cj0 = j0 - rj * M;
#pragma unroll
            for (int w = 0; w < WPG; ++w) {
                const int win = w0 + w;
                const WinPlace wp = place_window(g, win < g.nwin ? win : 0);
                u32x4 b = bw;
                if (wp.last_r || wp.last_c) {
                    const int lr = wp.last_r ? 1 : 0, lc = wp.last_c ? 1 : 0;
                    const bool rok = rj >= rlo[lr] && rj < rhi[lr];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int x0 = cj0 + 2 * e;
                        const uint32_t lo = rok && x0 >= clo[lc] && x0 < chi[lc] ? 0x0000ffffu : 0u;
                        const uint32_t hi = rok && x0 + 1 >= clo[lc] && x0 + 1 < chi[lc] ? 0xffff0000u : 0u;
                        b[e] &= lo | hi;
                    }
                }
                const bf16x8 B = __builtin_bit_cast(bf16x8, b);
                const __bf16* vst = vst_all + w * N * D;
                o0[w] = mfma(vt_frag(vst, c, 0, grp, li), B, o0[w]);
                o1[w] = mfma(vt_frag(vst, c, 1, grp, li), B, o1[w]);
            }
        }
        const float bias = la.bias ? la.bias[(size_t)h * N + qi] : 0.0f;
#pragma unroll
        for (int w = 0; w < WPG; ++w) {
            const int win = w0 + w;
            if (win >= g.nwin) continue;
            const WinPlace wp = place_window(g, win);
            const uint32_t bytes = (uint32_t)(wp.span - h * D) * 2u;
            const Rsrc orr = make_rsrc((const uint16_t*)p.out + wp.base + h * D, bytes);
            const uint32_t off = wp.wg.tok(ri, ci) + 8u * grp;
            store8(orr, off, pack_bf16x4(o0[w][0] + bias, o0[w][1] + bias, o0[w][2] + bias, o0[w][3] + bias));
            store8(orr, off + 32u, pack_bf16x4(o1[w][0] + bias, o1[w][1] + bias, o1[w][2] + bias, o1[w][3] + bias));
        }
    }
}

// Any dtype and M <= 64: one thread per (window, head, query, channel).
template <typename T>
__global__ void __launch_bounds__(256) wlin_valu_kernel(AttnParams p, WlinArgs la, int64_t total)
{
    const Geometry& g = p.g;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int M = g.M, N = g.N, d = g.d;
    const int e = (int)(idx % d);
    const int64_t r1 = idx / d;
    const int qi = (int)(r1 % N);
    const int64_t unit = r1 / N;
    const int h = (int)(unit % g.heads);
    const int win = (int)(unit / g.heads);
    const WinPlace wp = place_window(g, win);
    const int ri = qi / M, ci = qi - ri * M;
    int rlo = 0, rhi = M, clo = 0, chi = M;
    if (wp.last_r || wp.last_c) {
        region_interval(wp.last_r ? g.nwr - 1 : 0, g.nwr, M, g.shift, ri, rlo, rhi);
        region_interval(wp.last_c ? g.nwc - 1 : 0, g.nwc, M, g.shift, ci, clo, chi);
    }
    // token offsets of the geometry are bf16 bytes: elements = bytes / 2
    const T* v = (const T*)p.v + wp.base + h * d + e;
    const T* A = (const T*)la.A + ((size_t)h * N + qi) * N;
    float s = la.bias ? la.bias[(size_t)h * N + qi] : 0.0f;
    for (int rj = rlo; rj < rhi; ++rj)
        for (int cj = clo; cj < chi; ++cj) {
            const float a = (float)A[rj * M + cj];
            s = fmaf(a, (float)v[wp.wg.tok(rj, cj) / 2u], s);
        }
    ((T*)p.out)[wp.base + h * d + e + wp.wg.tok(ri, ci) / 2u] = (T)s;
}

}  // namespace

hipError_t launch_window_linear(const AttnParams& p, const WlinArgs& la, hipStream_t stream)
{
    const Geometry& g = p.g;
    if (g.nwin == 0) return hipSuccess;
    if (p.dtype == SWIN_DT_BF16 && g.d == D && (g.M == 8 || g.M == 16) &&
        (int64_t)g.H * g.W * g.C * 2 < ((int64_t)1 << 31) && (int64_t)g.W * g.C * 2 < ((int64_t)1 << 24)) {
        const int wh = g.M == 16 ? WPG : 4;
        const int64_t units = (int64_t)g.heads * ((g.nwin + wh - 1) / wh);
        if (units > INT32_MAX - 8) return hipErrorInvalidValue;
        const int per_xcd = (int)((units + 7) / 8);
        if (g.M == 16) wlin16_kernel<<<8 * per_xcd, 256, 0, stream>>>(p, la, (int)units, per_xcd);
        else wlin_kernel<8><<<8 * per_xcd, 256, 0, stream>>>(p, la, (int)units, per_xcd);
        return hipGetLastError();
    }
    const int64_t total = (int64_t)g.nwin * g.heads * g.N * g.d;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    if (p.dtype == SWIN_DT_F32) wlin_valu_kernel<float><<<(int)blocks, 256, 0, stream>>>(p, la, total);
    else wlin_valu_kernel<__bf16><<<(int)blocks, 256, 0, stream>>>(p, la, total);
    return hipGetLastError();
}

}  // namespace swin
