// Device helpers shared by the bf16 window-attention kernels: buffer-resource
// loads and stores with 32-bit offsets, LDS-DMA, window token addressing, the
// V-row swizzle and its transposed reads, and the 16x16x32 bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace swin {
namespace tio {

typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int D = 32;          // head dimension of every bf16 kernel

// Raw buffer access (gfx9 resource word 3 = 0x00020000: 32-bit data, no
// swizzle).  A raw load whose offset is at or past the record count returns
// zeros and a store there is dropped; tensors here stay below 2^31 bytes per
// image, so kNoLoad is always out of range.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kNoLoad = 0x80000000u;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 load16(Rsrc r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void store8(Rsrc r, uint32_t off, bf16x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
// kNoLoad unless ok (keeps the offset arithmetic unconditional: no branch)
__device__ __forceinline__ uint32_t masked(uint32_t off, bool ok) { return off | (ok ? 0u : kNoLoad); }

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds + 16 l (lds wave-uniform); out of range they are zeros.  Completion is
// counted by vmcnt; readers wait with vm_wait_all() and a barrier.  Issued
// from asm so that the compiler, which cannot tell this write from LDS reads
// elsewhere, adds no wait of its own before them; the asm has no output, and
// its inputs are read when it issues.
struct RawRsrc {
    u32x4 w;
};
__device__ __forceinline__ RawRsrc raw_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return RawRsrc{u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u}};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// lds: the LDS byte address (wave-uniform)
__device__ __forceinline__ void dma16_at(const RawRsrc& r, uint32_t lds, uint32_t off)
{
    // the resource and the LDS base are wave-uniform: pin them to scalar
    // registers, as the asm operands require
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_readfirstlane(r.w[i]);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(off), "s"(w) : "memory", "m0");
}
__device__ __forceinline__ void dma16(const RawRsrc& r, const void* lds, uint32_t off)
{
    dma16_at(r, lds_addr(lds), off);
}
__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// floor(a / b) for 0 <= a < 2^16, b <= 64, from a float reciprocal: the exact
// quotient of a + 1/2 sits at least 1/(2b) from an integer, far above the
// rounding error of the product.
__device__ __forceinline__ int qdiv(int a, float inv_b) { return (int)(((float)a + 0.5f) * inv_b); }

// Byte offset (within one image, or one window for the WINDOWS layout) of
// local token (r, c) is row(r) + col(c); all but (r, c) is wave-uniform:
// cyclic grid: origin (wr*M + shift, wc*M + shift), steps 1, wrap at H, W;
// interleaved: origin (wr, wc), steps (H/M, W/M), never wraps;
// windows tensor: origin 0, steps 1, an M x M "grid".
// The wrap is min(i, i - H) in unsigned arithmetic; products use the 24-bit
// multiplier (row and column strides stay below 2^24 bytes).
struct WinGeo {
    uint32_t r0, c0, rs, cs, Hm, Wm, rowb, colb;
    __device__ __forceinline__ uint32_t row(int r) const
    {
        const uint32_t gi = r0 + __umul24((uint32_t)r, rs);
        return __umul24(min(gi, gi - Hm), rowb);
    }
    __device__ __forceinline__ uint32_t col(int c) const
    {
        const uint32_t gj = c0 + __umul24((uint32_t)c, cs);
        return __umul24(min(gj, gj - Wm), colb);
    }
    __device__ __forceinline__ uint32_t tok(int r, int c) const { return row(r) + col(c); }
};

// Geometry of window `win` of the batch: its token addressing, the element
// offset of its image (or window) and the element count there, and whether it
// is in the last window row / column of a shifted grid.
struct WinPlace {
    WinGeo wg;
    int64_t base;
    int span;
    bool last_r, last_c;
};
__device__ __forceinline__ WinPlace place_window(const Geometry& g, int win)
{
    WinPlace w;
    const int M = g.M;
    const int nW = g.nwr * g.nwc;
    const int bimg = win / nW, wl = win - bimg * nW;
    const int wr = wl / g.nwc, wc = wl - wr * g.nwc;
    w.wg.colb = (uint32_t)g.C * 2u;
    if (g.layout == SWIN_LAYOUT_WINDOWS) {
        w.span = g.N * g.C;
        w.base = (int64_t)win * w.span;
        w.wg.r0 = w.wg.c0 = 0; w.wg.rs = w.wg.cs = 1; w.wg.Hm = w.wg.Wm = M;
    } else {
        w.span = g.H * g.W * g.C;
        w.base = (int64_t)bimg * w.span;
        w.wg.Hm = g.H; w.wg.Wm = g.W;
        if (g.part == SWIN_PART_INTERLEAVED) { w.wg.r0 = wr; w.wg.c0 = wc; w.wg.rs = g.nwr; w.wg.cs = g.nwc; }
        else { w.wg.r0 = wr * M + g.shift; w.wg.c0 = wc * M + g.shift; w.wg.rs = w.wg.cs = 1; }
    }
    w.wg.rowb = w.wg.Wm * w.wg.colb;
    const bool cyc_shift = g.part == SWIN_PART_CYCLIC && g.shift > 0;
    w.last_r = cyc_shift && wr == g.nwr - 1;
    w.last_c = cyc_shift && wc == g.nwc - 1;
    return w;
}

// Position (in 16-byte pieces) of piece p of V slot s in LDS rows of 64
// bytes is p ^ v_swizzle(s): of the transposed reads, the four 32-byte row
// halves a 16-lane group touches fall in distinct 128-byte bank windows, and
// the two groups of a half-wavefront in distinct 256-byte windows.
__device__ __forceinline__ int v_swizzle(int s) { return ((s >> 1) ^ (s >> 3)) & 1 ? 2 : 0; }

// V^T fragment (channels 16 dt..+15, slots 32c + 8 grp + 0..7) from V rows
// in LDS.  ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i%4 of the 4-element vectors addressed by lanes 4j + i/4,
// j = 0..3.  Transposed read h covers slots +4h..4h+3: lane li addresses
// slot + 4h + li/4, channels 16 dt + 4 (li%4) .. +3, and receives channel
// 16 dt + li of all four.
__device__ __forceinline__ bf16x8 vt_frag(const __bf16* vst, int c, int dt, int grp, int li)
{
    i16x4 half[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int s = 32 * c + 8 * grp + 4 * h + (li >> 2);
        const int m = li & 3;
        const __bf16* src = vst + s * D + (((2 * dt + (m >> 1)) ^ v_swizzle(s)) * 8) + 4 * (m & 1);
        half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)src);
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// The same with the lane's addresses taken apart: the swizzle of slot
// 32 c + 8 grp + 4 h + li/4 depends on neither c nor h, so the fragment of
// chunk c is read at vt_off(dt, grp, li) + 32 c D elements (the second
// transposed read 4 D further), and a loop over chunks needs one base.
__device__ __forceinline__ int vt_off(int dt, int grp, int li)
{
    const int s = 8 * grp + (li >> 2), m = li & 3;
    return s * D + (((2 * dt + (m >> 1)) ^ v_swizzle(s)) * 8) + 4 * (m & 1);
}
__device__ __forceinline__ bf16x8 vt_frag_at(const __bf16* p)
{
    i16x4 half[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
        half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * h * D));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
}
// Element offset of 16-byte piece `piece` of slot s in swizzled 64-byte
// rows; unchanged in its swizzle for s + 32 c, and for s + 4 when s % 8 < 4.
__device__ __forceinline__ int row_off(int s, int piece) { return s * D + ((piece ^ v_swizzle(s)) * 8); }

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace tio
}  // namespace swin
