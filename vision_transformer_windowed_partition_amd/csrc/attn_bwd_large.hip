// Backward of window attention on the gfx950 matrix cores for bf16 windows
// too large for the small-window backward: up to 32 x 32 tokens, with the
// window-local rotary positions (FlashSwin abstract) and the bias table of
// the SwinV2 card (eq. 3-4).
//
// Same gradient as the small-window backward (SwinV2 card eq. 1-2; with
// logit_ij = (q~_i . k~_j) a_i c_j + b_ij, q~, k~ the rotated operands):
//   dl_ij = p_ij (dout_i . v_j - D_i),  dv_j = sum_i p_ij dout_i,
//   G_i = sum_j dl_ij c_j k~_j,  H_j = sum_i dl_ij a_i q~_i,
//   COSINE: dq_i = a_i (G_i - q_i (q_i . G_i)/||q_i||^2), dk likewise with c_j;
//   DOT:    dq~ = G / sqrt(d) ... folded: a = c = 1/sqrt(d); ROPE2D: dq = R^T dq~.
//   dtable[offset(i, j)] += dl_ij (summed per workgroup in LDS as 64-bit
//   fixed point), dtau from sum dl_ij cos_ij.
// One workgroup of sixteen wavefronts (four per SIMD) per window-head, in two
// stages of LDS:
//   stage 1: K~ and V rows of every key slot (64-byte rows, XOR-swizzled
//     16-byte pieces), K rotated in fp32 and rounded once; per-slot scales
//     and D_i = dout_i . out_i.  Query-major passes over each wavefront's
//     query tiles (16 tokens; q~ and dout fragments straight from memory):
//     0: log-sum-exp per query; B: dP^T = V dout^T, dl, G^T += K~^T (dl c)^T
//     with K~^T read transposed; dq, dtau and the bias gradient.
//   stage 2: Q~ and dout rows replace them; key-major pass A over 16-key
//     tiles (k~, v fragments from memory): S = Q~ K~^T and dP = dout V^T with
//     permuted query rows, then dV^T += dout^T P and H^T += Q~^T (dl a).
// Rounding: for COSINE the operands are raw bf16 (exact) and the scales
// multiply in fp32; rotated operands are rounded to bf16 once, as in the
// forward, and for COSINE with rotation the score products take hi + lo
// pairs (the rotated rows' remainders in LDS, the tile's in registers), the
// cosine's normalisation being taken on the rotated operand (rotation keeps
// the norm).  All products are
// v_mfma_f32_16x16x32_bf16, fp32 accumulation.
#include "common.hpp"
#include "fixed_sum.hpp"
#include "lanes.hpp"
#include "launch.hpp"
#include "launch_bwd.hpp"
#include "tile_io.hpp"

namespace swin {

namespace {

using namespace tio;
using namespace lanes;

#ifndef LBWD_WAVES
#define LBWD_WAVES 16
#endif
constexpr int WAVES = LBWD_WAVES;
constexpr int NTHR = WAVES * 64;

struct LargeBwdLayout {
    int SR;                    // slots per key row: M rounded up to 8
    int GPR;                   // 8-slot groups per row
    int NS;                    // slots, padded to a multiple of 32
    int NQT;                   // query tiles of 16 tokens
    int units;                 // window-heads
    int P;                     // work ids per XCD slot
    float inv_M, inv_SR, inv_GPR;
};

struct BwdLargeArgs {
    const void* out;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* dtau;
    float* dtable;
};

__device__ __forceinline__ void rowstore(__bf16* rows, int s, int piece, const bf16x8& v)
{
    *(bf16x8*)(rows + s * D + ((piece ^ v_swizzle(s)) * 8)) = v;
}

__device__ __forceinline__ float quad_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
    return x;
}

// DPP row shifts within 16-lane rows (source outside the row reads zero)
template <int N>
__device__ __forceinline__ float row_shl(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xf, 0xf, true));
}
template <int N>
__device__ __forceinline__ float row_shr(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}

template <int V> struct Mode { static constexpr int value = V; };

__device__ __forceinline__ bf16x4 load8b(Rsrc r, uint32_t off)
{
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

template <int SIM, int POS>
__global__ void __launch_bounds__(NTHR)
attn_bwd_large_kernel(AttnParams p, BwdLargeArgs a, LargeBwdLayout L)
{
    extern __shared__ __attribute__((aligned(16))) float smem_f[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1, SR = L.SR, NS = L.NS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;

    const int work = (blockIdx.x & 7) * L.P + (blockIdx.x >> 3);
    if (work >= L.units) return;
    const int win = work / g.heads;
    const int h = work - win * g.heads;

    const int tabsz = POS == SWIN_POS_TABLE ? (S * S + 8 + 3) / 4 * 4 : 0;
    __bf16* rowA = (__bf16*)smem_f;                            // [NS][D] K~, later Q~
    __bf16* rowB = rowA + NS * D;                              // [NS][D] V, later dout
    float* ksc = (float*)(rowB + NS * D);                      // [NS] c_j
    float* qsc = ksc + NS;                                     // [NS] log2(e) a_i
    float* lse = qsc + NS;                                     // [NS]
    float* dd = lse + NS;                                      // [NS] D_i
    float* bias2 = dd + NS;                                    // [tabsz] reversed, log2 units
    // [tabsz] reversed, natural units, 64-bit fixed point
    fixed::acc_t* dtab = (fixed::acc_t*)(bias2 + tabsz);
    float* rtab = (float*)(dtab + tabsz);                      // [M][2][8] (cos, sin)  (ROPE2D)
    float* red = rtab + (POS == SWIN_POS_ROPE2D ? M * 32 : 0); // [WAVES]
    // COSINE with rotation: the remainders of the rounded rotated rows (K~,
    // later Q~), 16-byte aligned after red
    __bf16* rowL = (__bf16*)(((uintptr_t)(red + WAVES) + 15) & ~(uintptr_t)15);   // [NS][D]
    constexpr bool CR = SIM == SWIN_SIM_COSINE && POS == SWIN_POS_ROPE2D;

    const WinPlace wp = place_window(g, win);
    const WinGeo& wg = wp.wg;
    const uint32_t bytes = (uint32_t)(wp.span - h * D) * 2u;
    const int64_t off0 = wp.base + h * D;
    const Rsrc qr = make_rsrc((const uint16_t*)p.q + off0, bytes);
    const Rsrc kr = make_rsrc((const uint16_t*)p.k + off0, bytes);
    const Rsrc vr = make_rsrc((const uint16_t*)p.v + off0, bytes);
    const Rsrc gr = make_rsrc((const uint16_t*)a.dout + off0, bytes);
    const Rsrc orr = make_rsrc((const uint16_t*)a.out + off0, bytes);
    float tau = 1.0f;
    if (SIM == SWIN_SIM_COSINE) tau = fmaxf(p.tau[h], p.tau_min);
    const float inv_tau = 1.0f / tau;
    // COSINE with rotation: rounded rotated operands would move a logit by
    // up to 2^-8 / tau, which dtau (a sum that cancels over each query's
    // keys) does not absorb, so the score products take hi + lo pairs (three
    // products) from rowL and the query remainders
    const bool split = CR;
    const bool needs_mask = wp.last_r || wp.last_c || SR != M || NS != M * SR;
    // With no padded slot (M a multiple of 8) the exclusions of a shifted
    // window fall on whole 8-slot groups when the column split M - shift is
    // a multiple of 8: a lane's group (8 keys of one key row against one
    // query, or 8 queries of one query row against one key) is kept or
    // dropped as a whole, and a dropped group reads the table's -inf row (or
    // adds -inf without a table): mask mode 2, one select per group instead
    // of one per pair (mode 1).  When the row split lands on a chunk
    // boundary, the tiles of a last-row window see only the chunks of their
    // own region (c_lo, c_hi below) and need no row masks.
    const int rsplit = M - g.shift;
    const bool unpadded = SR == M && NS == M * SR;
    const bool half_rows = unpadded && wp.last_r && (rsplit * M) % 32 == 0;
    const bool group_masks = unpadded && (!wp.last_c || (rsplit & 7) == 0);
    const int mask_mode = !needs_mask ? 0 : (half_rows && !wp.last_c) ? 0 : group_masks ? 2 : 1;
    // chunk range of a tile whose first slot is s0 (query tile in pass B,
    // key tile in pass A)
    auto chunk_range = [&](int s0, int& c_lo, int& c_hi) {
        c_lo = 0;
        c_hi = NS / 32;
        if (half_rows) {
            if (s0 < rsplit * M) c_hi = rsplit * M / 32;
            else c_lo = rsplit * M / 32;
        }
    };
    const int negrow = S * S;
    // lane offsets of the chunk loops' LDS fragments (the swizzles do not
    // change from chunk to chunk: chunk c adds 32 c D elements)
    const int offA = row_off(8 * (li >> 2) + (li & 3), grp);   // A rows sA (and sA + 4: + 4 D)
    const int vo0 = vt_off(0, grp, li), vo1 = vt_off(1, grp, li);
    auto fragA = [&](const __bf16* rows, int c, int second) -> bf16x8 {
        return *(const bf16x8*)(rows + offA + (32 * c + 4 * second) * D);
    };
    constexpr float RS32 = 0.17677669529663687f;              // 1/sqrt(32)

    // rotate 8 channels 8 pc..8 pc+7 of a token at (r, c) by sgn * angle:
    // channels [0, 16) turn with the row, [16, 32) with the column
    auto rot8 = [&](float* f, int pc, int r, int c, float sgn) {
        const int half = pc >> 1, pos = half ? c : r;
        const float* cs = rtab + ((pos * 2 + half) * 8 + (pc & 1) * 4) * 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float co = cs[2 * e], si = sgn * cs[2 * e + 1];
            const float x0 = f[2 * e], x1 = f[2 * e + 1];
            f[2 * e] = x0 * co - x1 * si;
            f[2 * e + 1] = x0 * si + x1 * co;
        }
    };
    // rotation (sgn = 1) or its inverse (sgn = -1) of a lane's channels
    // 4 grp..+3 (half 0) and 16 + 4 grp..+3 (half 1): pairs k = 2 grp + m
    auto turn_lane = [&](float* g8, int r, int c, float sgn) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int pos = hh ? c : r;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int k = 2 * grp + m;
                const float co = rtab[((pos * 2 + hh) * 8 + k) * 2];
                const float si = sgn * rtab[((pos * 2 + hh) * 8 + k) * 2 + 1];
                const float x0 = g8[4 * hh + 2 * m], x1 = g8[4 * hh + 2 * m + 1];
                g8[4 * hh + 2 * m] = x0 * co - x1 * si;
                g8[4 * hh + 2 * m + 1] = x0 * si + x1 * co;
            }
        }
    };
    auto unrot_lane = [&](float* g8, int r, int c) { turn_lane(g8, r, c, -1.0f); };
    auto rot_lane = [&](float* g8, int r, int c) { turn_lane(g8, r, c, 1.0f); };

    // ---- tables
    if (POS == SWIN_POS_TABLE) {
        for (int i = tid; i < S * S; i += NTHR) {
            bias2[S * S - 1 - i] = p.table[(size_t)i * g.heads + h] * kLog2e;
            dtab[i] = 0ull;
        }
        if (tid < 8) bias2[S * S + tid] = -INFINITY;
    }
    if (POS == SWIN_POS_ROPE2D) {
        for (int i = tid; i < M * 16; i += NTHR) {
            const int k = i & 7, half = (i >> 3) & 1, pos = i >> 4;
            const float th = p.rope_freqs ? p.rope_freqs[((size_t)h * 2 + half) * 8 + k]
                                          : exp2f(-(float)k * 0.125f * log2f(p.rope_base));
            float s_, c_;
            sincosf((float)pos * th, &s_, &c_);
            rtab[i * 2] = c_;
            rtab[i * 2 + 1] = s_;
        }
    }
    __syncthreads();

    // ---- stage a tensor's rows (rotated when `rot`) for every slot; four
    // threads per slot, one 16-byte piece each.  Returns nothing; sq receives
    // the squared norm of the slot (same in all four threads).
    auto slot_of = [&](int s, int& r, int& c) { r = qdiv(s, L.inv_SR); c = s - r * SR; };
    auto stage_rows = [&](Rsrc src, __bf16* dst, bool rot, float* norm_out, bool cosine_scale, Rsrc src2,
                          __bf16* dst2) {
#pragma unroll 4
        for (int i0 = 0; i0 < NS * 4; i0 += NTHR) {
            const int i = i0 + tid;
            const int s = i >> 2, pc = i & 3;
            const bool in = s < NS;
            int r, c;
            slot_of(in ? s : 0, r, c);
            const bool ok = in && r < M && c < M;
            const uint32_t off = masked(wg.tok(r, c) + 16u * pc, ok);
            const u32x4 x = load16(src, off);
            const u32x4 x2 = load16(src2, off);
            float f[8];
            unpack_bf16x8(x, f);
            if (POS == SWIN_POS_ROPE2D && rot) rot8(f, pc, min(r, M - 1), min(c, M - 1), 1.0f);
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
            ss = quad_sum(ss);
            if (in) {
                const bf16x8 hi = (POS == SWIN_POS_ROPE2D && rot) ? pack_bf16x8(f) : __builtin_bit_cast(bf16x8, x);
                if (CR && split && rot) {
                    float lo[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) lo[e] = f[e] - (float)hi[e];
                    rowstore(rowL, s, pc, pack_bf16x8(lo));
                }
                rowstore(dst, s, pc, hi);
                rowstore(dst2, s, pc, __builtin_bit_cast(bf16x8, x2));
                if (norm_out && pc == 0)
                    norm_out[s] = cosine_scale ? 1.0f / fmaxf(sqrtf(ss), 1e-12f) : 1.0f;
            }
        }
    };

    // ---- stage 1: K~ and V rows, c_j; a_i and D_i
    stage_rows(kr, rowA, true, ksc, SIM == SWIN_SIM_COSINE, vr, rowB);
#pragma unroll 4
    for (int i0 = 0; i0 < NS * 4; i0 += NTHR) {
        const int i = i0 + tid;
        const int s = i >> 2, pc = i & 3;
        const bool in = s < NS;
        int r, c;
        slot_of(in ? s : 0, r, c);
        const bool ok = in && r < M && c < M;
        const uint32_t off = masked(wg.tok(r, c) + 16u * pc, ok);
        float qf[8], gf[8], of[8];
        unpack_bf16x8(load16(qr, off), qf);
        unpack_bf16x8(load16(gr, off), gf);
        unpack_bf16x8(load16(orr, off), of);
        float qq = 0.0f, go = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { qq = fmaf(qf[e], qf[e], qq); go = fmaf(gf[e], of[e], go); }
        qq = quad_sum(qq);
        go = quad_sum(go);
        if (in && pc == 0) {
            qsc[s] = SIM == SWIN_SIM_COSINE ? kLog2e * inv_tau / fmaxf(sqrtf(qq), 1e-12f) : kLog2e * RS32;
            dd[s] = go;
        }
    }
    __syncthreads();

    const int nch = NS / 32;
    float dtau_acc = 0.0f;
    const Rsrc dqr = make_rsrc((const uint16_t*)a.dq + off0, bytes);
    const Rsrc dkr = make_rsrc((const uint16_t*)a.dk + off0, bytes);
    const Rsrc dvr = make_rsrc((const uint16_t*)a.dv + off0, bytes);

    // ---- passes 0 and B over this wave's query tiles
    const bool diag8 = (M & 7) == 0;
    for (int t0 = wave; t0 < L.NQT; t0 += WAVES) {
        const int t = t0 * 16 + li;
        const bool tv = t < N;
        const int tt = tv ? t : 0;
        const int ri = qdiv(tt, L.inv_M), ci = tt - ri * M;
        const int qs_slot = ri * SR + ci;
        const uint32_t qoffb = masked(wg.tok(ri, ci) + 16u * grp, tv);
        float qv[8];
        unpack_bf16x8(load16(qr, qoffb), qv);
        if (POS == SWIN_POS_ROPE2D) rot8(qv, grp, ri, ci, 1.0f);
        const bf16x8 qf = pack_bf16x8(qv);
        bf16x8 qf_lo = qf;
        if (CR && split) {
            float lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) lo[e] = qv[e] - (float)qf[e];
            qf_lo = pack_bf16x8(lo);
        }
        // S^T for the 8 keys of this lane's group in chunk c (hi + lo when split)
        auto scores = [&](int c, f32x4& sa, f32x4& sb) {
            const bf16x8 ka = fragA(rowA, c, 0), kb = fragA(rowA, c, 1);
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            sa = mfma(ka, qf, z);
            sb = mfma(kb, qf, z);
            if (CR && split) {
                sa = mfma(fragA(rowL, c, 0), qf, sa);
                sb = mfma(fragA(rowL, c, 1), qf, sb);
                sa = mfma(ka, qf_lo, sa);
                sb = mfma(kb, qf_lo, sb);
            }
        };
        const bf16x8 gfr = __builtin_bit_cast(bf16x8, load16(gr, qoffb));
        const float qs = qsc[qs_slot], Dq = dd[qs_slot];
        const int qoff = (M - 1 - ri) * S + (M - 1 - ci);
        int rlo = 0, rhi = M, clo = 0, chi = M;
        if (wp.last_r) { if (ri < M - g.shift) rhi = M - g.shift; else rlo = M - g.shift; }
        if (wp.last_c) { if (ci < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
        // allowed key columns of this query, and those of a lane's 8-key group
        const uint32_t cmask = (chi >= 32 ? 0xffffffffu : (1u << chi) - 1u) & ~((1u << clo) - 1u);
        auto group_bits = [&](int rj, int cj0) -> uint32_t {
            return !needs_mask ? 0xffu : tv && rj >= rlo && rj < rhi && rj < M ? (cmask >> cj0) & 0xffu : 0u;
        };

        // pass 0: running maximum and sum, unless the forward's log-sum-exp
        // is given (natural log, to log2 units)
        float m = -INFINITY, l = 0.0f;
        const int nch0 = p.lse ? 0 : nch;
        for (int c = 0; c < nch0; ++c) {
            f32x4 sa, sb;
            scores(c, sa, sb);
            const f32x4 k0 = *(const f32x4*)(ksc + 32 * c + 8 * grp);
            const f32x4 k1 = *(const f32x4*)(ksc + 32 * c + 8 * grp + 4);
            const int gam = 4 * c + grp, rj = qdiv(gam, L.inv_GPR), cj0 = 8 * (gam - rj * L.GPR);
            const int boff = qoff + rj * S + cj0;
            const uint32_t bits = group_bits(rj, cj0);
            float x[8], cm = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float sv = e < 4 ? sa[e] : sb[e - 4];
                const float kv = e < 4 ? k0[e] : k1[e - 4];
                const bool ok = ((bits >> e) & 1u) != 0u;
                float b = 0.0f;
                if (POS == SWIN_POS_TABLE) b = bias2[ok ? boff + e : negrow];
                x[e] = ok ? fmaf(sv * qs, kv, b) : -INFINITY;
                cm = fmaxf(cm, x[e]);
            }
            cm = max_x32(max_x16(cm));
            const float mn = fmaxf(m, cm);
            const float mref = mn == -INFINITY ? 0.0f : mn;
            float ls = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ls += __builtin_amdgcn_exp2f(x[e] - mref);
            l = l * __builtin_amdgcn_exp2f(m - mref) + ls;
            m = mn;
        }
        float lq;
        if (p.lse) {
            lq = tv ? p.lse[((size_t)win * g.heads + h) * N + t] * kLog2e : 0.0f;
        } else {
            l = sum_x32(sum_x16(l));
            lq = m + __builtin_amdgcn_logf(l);
        }
        if (grp == 0 && tv) lse[qs_slot] = lq;

        // pass B: dq
        f32x4 G0 = {0.0f, 0.0f, 0.0f, 0.0f}, G1 = G0;
        float dts = 0.0f;                                  // sum over keys of dS~ s (dtau without a_i)
        // MASK false: no padded slot, shift region or tail query in the
        // window, so every pair is kept and the loop carries no selects
        // TM: bias-gradient sums, 0 none, 1 one LDS atomic per element,
        // 2 diagonal sums (M a multiple of 8)
        int cb_lo, cb_hi;
        chunk_range(16 * t0, cb_lo, cb_hi);
        auto pass_b = [&](auto mflag, auto tflag) {
            constexpr int MK = decltype(mflag)::value;
            constexpr bool MASK = MK == 1;
            constexpr int TM = decltype(tflag)::value;
            for (int c = cb_lo; c < cb_hi; ++c) {
                const bf16x8 va = fragA(rowB, c, 0), vb = fragA(rowB, c, 1);
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                f32x4 sa, sb;
                scores(c, sa, sb);
                const f32x4 pa = mfma(va, gfr, z), pb = mfma(vb, gfr, z);
                const f32x4 k0 = *(const f32x4*)(ksc + 32 * c + 8 * grp);
                const f32x4 k1 = *(const f32x4*)(ksc + 32 * c + 8 * grp + 4);
                const int gam = 4 * c + grp, rj = qdiv(gam, L.inv_GPR), cj0 = 8 * (gam - rj * L.GPR);
                const int boff = qoff + rj * S + cj0;
                const uint32_t bits = MASK ? (tv ? group_bits(rj, cj0) : 0u) : 0xffu;
                const bool gok = MK != 2 || (rj >= rlo && rj < rhi && ((cmask >> cj0) & 1u));
                const int bidx = MK == 2 && !gok ? negrow : boff;
                float ds[8], dlv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sv = e < 4 ? sa[e] : sb[e - 4];
                    const float dpv = e < 4 ? pa[e] : pb[e - 4];
                    const float kv = e < 4 ? k0[e] : k1[e - 4];
                    const bool ok = !MASK || ((bits >> e) & 1u) != 0u;
                    float b = 0.0f;
                    if (POS == SWIN_POS_TABLE) b = MASK ? bias2[ok ? boff + e : negrow] : bias2[bidx + e];
                    else if (MK == 2) b = gok ? 0.0f : -INFINITY;
                    // logit (log2 units) = s a_i c_j + b, a_i c_j = qs kv (DOT: kv = 1)
                    const float arg = fmaf(sv, SIM == SWIN_SIM_COSINE ? qs * kv : qs, b) - lq;
                    const float pr = __builtin_amdgcn_exp2f(!MASK || ok ? arg : -INFINITY);
                    const float dl = pr * (dpv - Dq);
                    // COSINE: dS~ = dl c_j (dq's a_i after the sum); DOT: dl (1/sqrt(d) after)
                    ds[e] = SIM == SWIN_SIM_COSINE ? dl * kv : dl;
                    dlv[e] = dl;
                    if (SIM == SWIN_SIM_COSINE) dts = fmaf(ds[e], sv, dts);
                    if (TM == 1 && (!MASK || ok)) fixed::add(&dtab[boff + e], dl);
                }
                if (TM == 2) {
                    // M a multiple of 8: each 8-lane half of the tile is 8
                    // consecutive columns of one window row, so (lane, element e)
                    // lands at boff(lane) + e with boff falling by one per lane.
                    // Sums along those diagonals inside each half: lane j = li % 8
                    // gathers d = -j from lanes j + k (element k) and, for j >= 1,
                    // d = 8 - j from lanes j - 8 + e; terms from the other half are
                    // dropped.  Masked pairs carry dl = 0.
                    // Element k of a lane at position j moves k lanes down for the
                    // first sum and 8 - k lanes up for the second; it stays in its
                    // half for the first when j >= k and for the second otherwise,
                    // so each lane splits it before the moves and the shifted
                    // values only add (a lane shifted in from outside the 16-lane
                    // row reads zero).  Every lane evaluates every row shift, so
                    // that no shift is made conditional.
                    const int j = li & 7;
                    float x[8], y[8];
#pragma unroll
                    for (int k = 1; k < 8; ++k) {
                        x[k] = j >= k ? dlv[k] : 0.0f;
                        y[k] = j >= k ? 0.0f : dlv[k];
                    }
                    float A = dlv[0];
                    A += row_shl<1>(x[1]);
                    A += row_shl<2>(x[2]);
                    A += row_shl<3>(x[3]);
                    A += row_shl<4>(x[4]);
                    A += row_shl<5>(x[5]);
                    A += row_shl<6>(x[6]);
                    A += row_shl<7>(x[7]);
                    float B = row_shr<7>(y[1]);
                    B += row_shr<6>(y[2]);
                    B += row_shr<5>(y[3]);
                    B += row_shr<4>(y[4]);
                    B += row_shr<3>(y[5]);
                    B += row_shr<2>(y[6]);
                    B += row_shr<1>(y[7]);
                    if (!MASK || tv) fixed::add(&dtab[boff], A);
                    // B is zero at j = 0 (every source is outside the half); the
                    // add is kept there so the sum is not branched around
                    if (!MASK || tv) fixed::add(&dtab[boff + 8], B);
                }
                const bf16x8 dsb = pack_bf16x8(ds);
                G0 = mfma(vt_frag_at(rowA + 32 * c * D + vo0), dsb, G0);
                G1 = mfma(vt_frag_at(rowA + 32 * c * D + vo1), dsb, G1);
            }
        };
        auto pass_b_masks = [&](auto tflag) {
            if (mask_mode == 1) pass_b(Mode<1>{}, tflag);
            else if (mask_mode == 2) pass_b(Mode<2>{}, tflag);
            else pass_b(Mode<0>{}, tflag);
        };
        if (POS != SWIN_POS_TABLE || !a.dtable) pass_b_masks(Mode<0>{});
        else if (diag8) pass_b_masks(Mode<2>{});
        else pass_b_masks(Mode<1>{});
        // sum dl (log2-unit logit without the bias) = qs sum dS~ s
        if (SIM == SWIN_SIM_COSINE) dtau_acc = fmaf(dts, qs, dtau_acc);
        const float gs = SIM == SWIN_SIM_COSINE ? 1.0f : RS32;
        float g8[8] = {G0[0] * gs, G0[1] * gs, G0[2] * gs, G0[3] * gs,
                       G1[0] * gs, G1[1] * gs, G1[2] * gs, G1[3] * gs};
        const uint32_t o8 = masked(wg.tok(ri, ci) + 8u * grp, tv);
        if (SIM == SWIN_SIM_COSINE) {
            const bf16x4 qa4 = load8b(qr, o8), qb4 = load8b(qr, o8 + 32u);
            float q8[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { q8[e] = (float)qa4[e]; q8[e + 4] = (float)qb4[e]; }
            if (CR) rot_lane(q8, ri, ci);                     // the normalised operand is the rotated q
            float qg = 0.0f, qq = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) { qg = fmaf(q8[e], g8[e], qg); qq = fmaf(q8[e], q8[e], qq); }
            qg = sum_x32(sum_x16(qg));
            qq = sum_x32(sum_x16(qq));
            const float nq = sqrtf(qq);
            const float ai = inv_tau / fmaxf(nq, 1e-12f);
            const float pj = nq > 1e-12f ? qg / qq : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) g8[e] = ai * (g8[e] - q8[e] * pj);
        }
        if (POS == SWIN_POS_ROPE2D) unrot_lane(g8, ri, ci);
        store8(dqr, o8, pack_bf16x4(g8[0], g8[1], g8[2], g8[3]));
        store8(dqr, o8 + 32u, pack_bf16x4(g8[4], g8[5], g8[6], g8[7]));
    }
    __syncthreads();

    // ---- stage 2: Q~ and dout rows
    stage_rows(qr, rowA, true, nullptr, false, gr, rowB);
    __syncthreads();

    // ---- pass A: dk, dv over this wave's 16-key tiles
    const int nkt = NS / 16;
    for (int kt = wave; kt < nkt; kt += WAVES) {
        const int sk = 16 * kt + li;
        int rj, cj;
        slot_of(sk, rj, cj);
        const bool kv_ok = rj < M && cj < M;
        const int rjc = min(rj, M - 1), cjc = min(cj, M - 1);
        const uint32_t koffb = masked(wg.tok(rjc, cjc) + 16u * grp, kv_ok);
        float kvv[8];
        unpack_bf16x8(load16(kr, koffb), kvv);
        if (POS == SWIN_POS_ROPE2D) rot8(kvv, grp, rjc, cjc, 1.0f);
        const bf16x8 kB = pack_bf16x8(kvv);
        bf16x8 kB_lo = kB;
        if (CR && split) {
            float lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) lo[e] = kvv[e] - (float)kB[e];
            kB_lo = pack_bf16x8(lo);
        }
        const bf16x8 vB = __builtin_bit_cast(bf16x8, load16(vr, koffb));
        const float cj_s = ksc[sk];
        int rlo = 0, rhi = M, clo = 0, chi = M;
        if (wp.last_r) { if (rj < M - g.shift) rhi = M - g.shift; else rlo = M - g.shift; }
        if (wp.last_c) { if (cj < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
        const uint32_t cmask = ((chi >= 32 ? 0xffffffffu : ((1u << chi) - 1u)) & ~((1u << clo) - 1u)) &
                               (M >= 32 ? 0xffffffffu : ((1u << M) - 1u));
        f32x4 V0 = {0.0f, 0.0f, 0.0f, 0.0f}, V1 = V0, H0 = V0, H1 = V0;
        int ca_lo, ca_hi;
        chunk_range(16 * kt, ca_lo, ca_hi);
        auto pass_a = [&](auto mflag) {
            constexpr int MK = decltype(mflag)::value;
            constexpr bool MASK = MK == 1;
            for (int c = ca_lo; c < ca_hi; ++c) {
                const bf16x8 qa = fragA(rowA, c, 0), qb = fragA(rowA, c, 1);
                const bf16x8 ga = fragA(rowB, c, 0), gb = fragA(rowB, c, 1);
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                f32x4 sa = mfma(qa, kB, z), sb = mfma(qb, kB, z);
                if (CR && split) {
                    sa = mfma(fragA(rowL, c, 0), kB, sa);
                    sb = mfma(fragA(rowL, c, 1), kB, sb);
                    sa = mfma(qa, kB_lo, sa);
                    sb = mfma(qb, kB_lo, sb);
                }
                const int qs0 = 32 * c + 8 * grp;
                const f32x4 dA = *(const f32x4*)(dd + qs0), dB = *(const f32x4*)(dd + qs0 + 4);
                const f32x4 pa = mfma(ga, vB, z), pb = mfma(gb, vB, z);
                const f32x4 qsA = *(const f32x4*)(qsc + qs0), qsB = *(const f32x4*)(qsc + qs0 + 4);
                const f32x4 lA = *(const f32x4*)(lse + qs0), lB = *(const f32x4*)(lse + qs0 + 4);
                const int gam = 4 * c + grp, ri = qdiv(gam, L.inv_GPR), ci0 = 8 * (gam - ri * L.GPR);
                // reversed table position of query (ri, ci0 + 7) against key (rj, cj)
                const int rev7 = S * S - 8 - ((ri - rj + M - 1) * S + (ci0 - cj + M - 1));
                const bool gok = MK != 2 || (ri >= rlo && ri < rhi && ((cmask >> ci0) & 1u));
                const float* brow = bias2 + (MK == 2 && !gok ? negrow : rev7);
                const bool rok = kv_ok && ri < M && ri >= rlo && ri < rhi;
                const uint32_t cbits = MASK ? (rok ? (cmask >> ci0) & 0xffu : 0u) : 0xffu;
                float pp[8], dsa[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sv = e < 4 ? sa[e] : sb[e - 4];
                    const float dpv = e < 4 ? pa[e] : pb[e - 4];
                    const float qv_ = e < 4 ? qsA[e] : qsB[e - 4];
                    const float lv = e < 4 ? lA[e] : lB[e - 4];
                    const bool ok = !MASK || ((cbits >> e) & 1u) != 0u;
                    float b = 0.0f;
                    if (POS == SWIN_POS_TABLE) b = MASK ? bias2[ok ? rev7 + (7 - e) : negrow] : brow[7 - e];
                    else if (MK == 2) b = gok ? 0.0f : -INFINITY;
                    const float arg = fmaf(sv * qv_, cj_s, b) - lv;
                    const float pr = __builtin_amdgcn_exp2f(!MASK || ok ? arg : -INFINITY);
                    pp[e] = pr;
                    const float dl = pr * (dpv - (e < 4 ? dA[e] : dB[e - 4]));
                    // dS~ = dl log2(e) a_i (COSINE) or dl (DOT); the constant after the sum
                    dsa[e] = SIM == SWIN_SIM_COSINE ? dl * qv_ : dl;
                }
                const bf16x8 pbf = pack_bf16x8(pp), dsb = pack_bf16x8(dsa);
                V0 = mfma(vt_frag_at(rowB + 32 * c * D + vo0), pbf, V0);
                V1 = mfma(vt_frag_at(rowB + 32 * c * D + vo1), pbf, V1);
                H0 = mfma(vt_frag_at(rowA + 32 * c * D + vo0), dsb, H0);
                H1 = mfma(vt_frag_at(rowA + 32 * c * D + vo1), dsb, H1);
            }
        };
        if (mask_mode == 1) pass_a(Mode<1>{});
        else if (mask_mode == 2) pass_a(Mode<2>{});
        else pass_a(Mode<0>{});
        const float hs = SIM == SWIN_SIM_COSINE ? 1.0f / kLog2e : RS32;
        float h8[8] = {H0[0] * hs, H0[1] * hs, H0[2] * hs, H0[3] * hs,
                       H1[0] * hs, H1[1] * hs, H1[2] * hs, H1[3] * hs};
        const uint32_t o8 = masked(wg.tok(rjc, cjc) + 8u * grp, kv_ok);
        if (SIM == SWIN_SIM_COSINE) {
            const bf16x4 ka4 = load8b(kr, o8), kb4 = load8b(kr, o8 + 32u);
            float k8[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { k8[e] = (float)ka4[e]; k8[e + 4] = (float)kb4[e]; }
            if (CR) rot_lane(k8, rjc, cjc);
            float kh = 0.0f, kk = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) { kh = fmaf(k8[e], h8[e], kh); kk = fmaf(k8[e], k8[e], kk); }
            kh = sum_x32(sum_x16(kh));
            kk = sum_x32(sum_x16(kk));
            const float nk = sqrtf(kk);
            const float pj = nk > 1e-12f ? kh / kk : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) h8[e] = cj_s * (h8[e] - k8[e] * pj);
        }
        if (POS == SWIN_POS_ROPE2D) unrot_lane(h8, rjc, cjc);
        store8(dkr, o8, pack_bf16x4(h8[0], h8[1], h8[2], h8[3]));
        store8(dkr, o8 + 32u, pack_bf16x4(h8[4], h8[5], h8[6], h8[7]));
        store8(dvr, o8, pack_bf16x4(V0[0], V0[1], V0[2], V0[3]));
        store8(dvr, o8 + 32u, pack_bf16x4(V1[0], V1[1], V1[2], V1[3]));
    }

    // ---- this window-head's share of dtau and of the table gradient
    if (SIM == SWIN_SIM_COSINE && a.dtau) {
        const float s = wave_reduce<Op::Sum>(dtau_acc);
        if (lane == 0) red[wave] = s;
    }
    __syncthreads();
    if (SIM == SWIN_SIM_COSINE && a.dtau && tid == 0 && p.tau[h] > p.tau_min) {
        float s = 0.0f;
        for (int w = 0; w < WAVES; ++w) s += red[w];
        unsafeAtomicAdd(&a.dtau[h], s * (-1.0f / (kLog2e * p.tau[h])));
    }
    if (POS == SWIN_POS_TABLE && a.dtable)
        for (int i = tid; i < S * S; i += NTHR)
            if (dtab[i] != 0ull)
                unsafeAtomicAdd(&a.dtable[(size_t)(S * S - 1 - i) * g.heads + h], fixed::from_fixed(dtab[i]));
}

size_t lds_bytes(const AttnParams& p, int NS)
{
    const int S = 2 * p.g.M - 1;
    size_t b = (size_t)NS * D * 2 * 2 + (size_t)4 * NS * 4 + (size_t)WAVES * 4 + 64;
    if (p.pos == SWIN_POS_TABLE) b += (size_t)3 * ((S * S + 8 + 3) / 4 * 4) * 4;   // bias2, dtab
    if (p.pos == SWIN_POS_ROPE2D) b += (size_t)p.g.M * 32 * 4;
    if (p.sim == SWIN_SIM_COSINE && p.pos == SWIN_POS_ROPE2D) b += 16 + (size_t)NS * D * 2;   // remainder rows
    return b;
}

int slots_of(const AttnParams& p)
{
    const int SR = (p.g.M + 7) / 8 * 8;
    return (p.g.M * SR + 31) / 32 * 32;
}

template <int SIM, int POS>
hipError_t launch_large(const AttnParams& p, const BwdLargeArgs& a, const LargeBwdLayout& L, size_t lds,
                        hipStream_t s)
{
    auto* fn = attn_bwd_large_kernel<SIM, POS>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<8 * L.P, NTHR, lds, s>>>(p, a, L);
    return hipGetLastError();
}

}  // namespace

bool attn_bwd_large_supported(const AttnParams& p)
{
    const Geometry& g = p.g;
    return p.dtype == SWIN_DT_BF16 && g.d == D && g.M <= 32 &&
           lds_bytes(p, slots_of(p)) <= 160 * 1024 &&
           (int64_t)g.H * g.W * g.C * 2 < ((int64_t)1 << 31) && (int64_t)g.W * g.C * 2 < ((int64_t)1 << 24);
}

hipError_t launch_attn_bwd_large(const AttnParams& p, const void* out, const void* dout, void* dq, void* dk,
                                 void* dv, float* dtau, float* dtable, hipStream_t stream)
{
    const Geometry& g = p.g;
    if (g.nwin == 0) return hipSuccess;
    BwdLargeArgs a{out, dout, dq, dk, dv, dtau, dtable};
    LargeBwdLayout L;
    L.SR = (g.M + 7) / 8 * 8;
    L.GPR = L.SR / 8;
    L.NS = slots_of(p);
    L.NQT = (g.N + 15) / 16;
    L.units = g.nwin * g.heads;
    L.P = (L.units + 7) / 8;
    L.inv_M = 1.0f / (float)g.M;
    L.inv_SR = 1.0f / (float)L.SR;
    L.inv_GPR = 1.0f / (float)L.GPR;
    const size_t lds = lds_bytes(p, L.NS);
    if (p.sim == SWIN_SIM_COSINE) {
        if (p.pos == SWIN_POS_TABLE) return launch_large<SWIN_SIM_COSINE, SWIN_POS_TABLE>(p, a, L, lds, stream);
        if (p.pos == SWIN_POS_ROPE2D) return launch_large<SWIN_SIM_COSINE, SWIN_POS_ROPE2D>(p, a, L, lds, stream);
        return launch_large<SWIN_SIM_COSINE, SWIN_POS_NONE>(p, a, L, lds, stream);
    }
    if (p.pos == SWIN_POS_TABLE) return launch_large<SWIN_SIM_DOT, SWIN_POS_TABLE>(p, a, L, lds, stream);
    if (p.pos == SWIN_POS_ROPE2D) return launch_large<SWIN_SIM_DOT, SWIN_POS_ROPE2D>(p, a, L, lds, stream);
    return launch_large<SWIN_SIM_DOT, SWIN_POS_NONE>(p, a, L, lds, stream);
}

}  // namespace swin
