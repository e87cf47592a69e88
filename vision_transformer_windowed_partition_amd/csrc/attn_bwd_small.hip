// Backward of window attention on the gfx950 matrix cores, bf16, windows of
// up to 256 tokens (M <= 16), no rotary positions.
//
// Gradient of the SwinV2 card's eq. 1-2 with the log-CPB table of eq. 3-4
// over cyclic-shift or interleaved windows, per (window, head); with
// logit_ij = (q_i . k_j) a_i c_j + b_ij (COSINE: a_i = 1/(tau' ||q_i||),
// c_j = 1/||k_j||; DOT: a_i = c_j = 1/sqrt(d)), p the softmax over the
// query's shift region and D_i = dout_i . out_i:
//   dl_ij = p_ij (dout_i . v_j - D_i)
//   dv_j  = sum_i p_ij dout_i
//   G_i   = sum_j dl_ij c_j k_j,   dq_i = a_i (G_i - q_i (q_i . G_i) / ||q_i||^2)
//   H_j   = sum_i dl_ij a_i q_i,   dk_j = c_j (H_j - k_j (k_j . H_j) / ||k_j||^2)
//   (DOT: no projection terms), dtable[offset(i, j)] += dl_ij,
//   dtau = -(1/tau) sum dl_ij cos_ij / tau while tau > tau_min.
// q, k, v, dout stay raw (exact bf16) in LDS; the scales a_i, c_j multiply
// in fp32, so nothing is rounded before the products but the weights.
//
// A workgroup of four wavefronts serves one head: for 9 <= M <= 16 one
// window shared by the four, for M <= 8 one window each.  LDS holds two of
// the window's tensors as 64-byte rows in key-slot order (8 slots per row
// segment, XOR-swizzled 16-byte pieces, filled by LDS-DMA): K and V for
// passes 0 and B, then Q and dout, staged into the same space, for pass A;
// a pass takes the fragments of its own tiles of the other two straight from
// memory.  Beside them: the per-slot scales, log-sum-exp and D, the head's
// bias table (reversed, log2 units) and the workgroup's bias-gradient
// accumulator (64-bit fixed point, integer LDS atomics).  Three passes:
//   0  query-major (like the forward): S^T = K Q^T per 32-key chunk, running
//      maximum and sum -> log-sum-exp of each query (skipped when the
//      forward's is given);
//   B  query-major: S^T and dP^T = V dout^T, dl, then
//      G^T += K^T (dl c)^T with K^T read transposed from the K rows
//      (ds_read_b64_tr_b16); dq, dtau and the bias gradient;
//   A  key-major, one 16-key tile at a time: S = Q K^T and dP = dout V^T with
//      the query rows permuted so each lane holds 8 consecutive query slots
//      of one key (the B-operand layout of P and dS), then
//      dV^T += dout^T P and H^T += Q^T (dl a), dout^T and Q^T read transposed.
// All products are v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
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

constexpr int WAVES = 4;

struct BwdLayout {
    int NSP;                   // key slots in use: M rows of M rounded up to 8
    int NQT;                   // query tiles of 16 tokens per window
    int wgs;                   // workgroups with work
    int P;                     // work ids per XCD slot
    float inv_M;
};

struct BwdSmallArgs {
    const void* out;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* dtau;
    float* dtable;
};

__device__ __forceinline__ bf16x8 rowfrag(const __bf16* rows, int s, int piece)
{
    return *(const bf16x8*)(rows + s * D + ((piece ^ v_swizzle(s)) * 8));
}

// quad reductions (lanes ^1, ^2) by DPP quad_perm
__device__ __forceinline__ float quad_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
    return x;
}

// DPP row shifts within 16-lane rows; lanes whose source falls outside the
// row read zero.  shl: lane i reads lane i + N; shr: lane i reads lane i - N.
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

// Slot s of a window: row (s >> 3) / GPR, column 8 ((s >> 3) % GPR) + (s & 7).
template <int GPR>
__device__ __forceinline__ void slot_rc(int s, int& r, int& c)
{
    const int gam = s >> 3;
    r = gam / GPR;
    c = 8 * (gam % GPR) + (s & 7);
}

template <bool B> struct Flag { static constexpr bool value = B; };
template <int V> struct Mode { static constexpr int value = V; };

// DIAG: M = 16 with a table (the bias gradient by diagonal sums).
// RT: M = 16, so a 16-slot piece, a query tile and a key tile are each one
// window row (row offsets scalar, the lane's column its own).
template <int SIM, int POS, int NCH, int QW, bool DIAG, bool RT>
__global__ void __launch_bounds__(256)
attn_bwd_small_kernel(AttnParams p, BwdSmallArgs a, BwdLayout L)
{
    constexpr int GPR = NCH <= 2 ? 1 : 2;
    constexpr int WH = WAVES / QW;
    constexpr int NS = NCH * 32;                   // slots per window (padded)
    constexpr int SETS = 2 * NCH / QW;             // 1 KB row pieces per tensor and wave
    extern __shared__ __attribute__((aligned(16))) float smem_f[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    const int wh = wave / QW, rank = wave - wh * QW;

    const int tabsz = POS == SWIN_POS_TABLE ? (S * S + 8 + 3) / 4 * 4 : 0;
    float* bias2 = smem_f;                                     // [S*S + 8] reversed, log2 units
    // [S*S] reversed, natural units, 64-bit fixed point
    fixed::acc_t* dtab = (fixed::acc_t*)(bias2 + tabsz);
    float* red = (float*)(dtab + tabsz);                       // [16]
    float* scal = red + 16 + wh * (4 * NS);                    // this window's per-slot scalars
    float* ksc = scal;                                         // [NS] c_j
    float* qsc = ksc + NS;                                     // [NS] log2(e) a_i
    float* lse = qsc + NS;                                     // [NS] log2-sum-exp of the logits
    float* dd = lse + NS;                                      // [NS] D_i
    // PHASED (one window shared by four wavefronts): two row buffers, K and V
    // for passes 0 and B, then Q and dout for pass A; else all four at once
    // (LDS is not what limits those workgroups)
    constexpr bool PHASED = QW > 1;
    constexpr int NROWS = PHASED ? 2 : 4;
    __bf16* rows = (__bf16*)(red + 16 + WH * 4 * NS) + wh * (NROWS * NS * D);
    __bf16* krow = rows;
    __bf16* vrow = rows + NS * D;
    __bf16* qrow = rows + (PHASED ? 0 : 2 * NS * D);
    __bf16* orow = rows + (PHASED ? NS * D : 3 * NS * D);

    const int work = (blockIdx.x & 7) * L.P + (blockIdx.x >> 3);
    if (work >= L.wgs) return;
    const int h = work % g.heads;
    const int wloc = (work / g.heads) * WH + wh;
    const bool active = wloc < g.nwin;
    const int win = active ? wloc : 0;
    float tau = 1.0f;
    if (SIM == SWIN_SIM_COSINE) tau = fmaxf(p.tau[h], p.tau_min);
    const WinPlace wp = place_window(g, win);
    const WinGeo& wg = wp.wg;
    const uint32_t bytes = active ? (uint32_t)(wp.span - h * D) * 2u : 0u;

    // ---- staging: the four tensors' rows by LDS-DMA; piece j of a tensor
    // is slots 16 j .. 16 j + 15, lane l filling LDS piece l%4 of slot
    // 16 j + l/4 with channel piece (l%4) ^ v_swizzle(slot)
    // RT: the lane's column offsets, as a query or key (li) and as a staging
    // lane (l / 4, with its swizzled piece)
    const uint32_t lcol = RT ? wg.col(li) : 0u;
    const uint32_t scol = RT ? wg.col(lane >> 2) + 16u * ((lane & 3) ^ v_swizzle(lane >> 2)) : 0u;
    auto stage_rows = [&](const void* t0, const void* t1, __bf16* dst) {
        const void* src[2] = {t0, t1};
#pragma unroll
        for (int tsr = 0; tsr < 2; ++tsr) {
            const RawRsrc rr = raw_rsrc((const uint16_t*)src[tsr] + wp.base + h * D, bytes);
#pragma unroll
            for (int k = 0; k < SETS; ++k) {
                const int j = rank + QW * k;
                const int s = 16 * j + (lane >> 2);
                int r, c;
                slot_rc<GPR>(s, r, c);
                const int piece = (lane & 3) ^ v_swizzle(s);
                if (RT)
                    dma16(rr, dst + (size_t)tsr * NS * D + (size_t)j * 512, wg.row(j) + scol);
                else
                    dma16(rr, dst + (size_t)tsr * NS * D + (size_t)j * 512,
                          masked(wg.tok(r, c) + 16u * piece, r < M && c < M));
            }
        }
    };
    stage_rows(p.k, p.v, krow);
    if (!PHASED) stage_rows(p.q, a.dout, qrow);
    // a row's 8-channel piece straight from memory (zeros for padded slots):
    // the fragments of the tensors not in LDS during a pass
    const Rsrc qg = make_rsrc((const uint16_t*)p.q + wp.base + h * D, bytes);
    const Rsrc dg = make_rsrc((const uint16_t*)a.dout + wp.base + h * D, bytes);
    const Rsrc kg = make_rsrc((const uint16_t*)p.k + wp.base + h * D, bytes);
    const Rsrc vg = make_rsrc((const uint16_t*)p.v + wp.base + h * D, bytes);
    auto gfrag = [&](const Rsrc& r, int s, int piece) -> bf16x8 {
        int rr, cc;
        slot_rc<GPR>(s, rr, cc);
        return __builtin_bit_cast(bf16x8, load16(r, masked(wg.tok(rr, cc) + 16u * piece, rr < M && cc < M)));
    };
    // channels 4 grp..+3 and 16 + 4 grp..+3 of slot s, as floats, from an
    // LDS row (piece (4 grp / 8), half grp & 1) or from memory
    auto lquad = [&](const __bf16* rw, int s, float* f) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int ch = 16 * hh + 4 * grp;
            const __bf16* src = rw + s * D + (((ch >> 3) ^ v_swizzle(s)) * 8) + (ch & 7);
#pragma unroll
            for (int e = 0; e < 4; ++e) f[4 * hh + e] = (float)src[e];
        }
    };
    // RT: the same from the token offset of the lane's row and column
    auto tfrag = [&](const Rsrc& r, uint32_t tok, int piece) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, load16(r, tok + 16u * piece));
    };
    auto gquad = [&](const Rsrc& r, int s, float* f) {
        const bf16x8 lo = gfrag(r, s, grp >> 1), hi = gfrag(r, s, 2 + (grp >> 1));
        const int o = 4 * (grp & 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) { f[e] = (float)lo[o + e]; f[4 + e] = (float)hi[o + e]; }
    };
    //   per-slot scalars: four lanes per slot (a 16-byte piece each), slots
    //   rank*16 + 16 QW it ...; norms of k and q, and dout . out
    {
        const Rsrc kr = make_rsrc((const uint16_t*)p.k + wp.base + h * D, bytes);
        const Rsrc qr = make_rsrc((const uint16_t*)p.q + wp.base + h * D, bytes);
        const Rsrc gr = make_rsrc((const uint16_t*)a.dout + wp.base + h * D, bytes);
        const Rsrc orr = make_rsrc((const uint16_t*)a.out + wp.base + h * D, bytes);
        const int piece = lane & 3;
        for (int s0 = 16 * rank; s0 < NS; s0 += 16 * QW) {
            const int s = s0 + (lane >> 2);
            int r, c;
            slot_rc<GPR>(s, r, c);
            const uint32_t off = RT ? wg.row(s0 >> 4) + wg.col(lane >> 2) + 16u * piece
                                    : masked(wg.tok(r, c) + 16u * piece, r < M && c < M);
            float kf[8], qf[8], gf[8], of[8];
            unpack_bf16x8(load16(kr, off), kf);
            unpack_bf16x8(load16(qr, off), qf);
            unpack_bf16x8(load16(gr, off), gf);
            unpack_bf16x8(load16(orr, off), of);
            float kk = 0.0f, qq = 0.0f, go = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kk = fmaf(kf[e], kf[e], kk);
                qq = fmaf(qf[e], qf[e], qq);
                go = fmaf(gf[e], of[e], go);
            }
            kk = quad_sum(kk);
            qq = quad_sum(qq);
            go = quad_sum(go);
            if (piece == 0) {
                if (SIM == SWIN_SIM_COSINE) {
                    ksc[s] = 1.0f / fmaxf(sqrtf(kk), 1e-12f);
                    qsc[s] = kLog2e / (tau * fmaxf(sqrtf(qq), 1e-12f));
                } else {
                    ksc[s] = 1.0f;
                    qsc[s] = kLog2e * 0.17677669529663687f;
                }
                dd[s] = go;
            }
        }
    }
    if (POS == SWIN_POS_TABLE) {
        for (int i = tid; i < S * S; i += 256) {
            bias2[S * S - 1 - i] = p.table[(size_t)i * g.heads + h] * kLog2e;
            dtab[i] = 0ull;
        }
        if (tid < 8) bias2[S * S + tid] = -INFINITY;
    }
    vm_wait_all();
    __syncthreads();

    const bool padded = 8 * GPR != M || NCH * 32 != L.NSP;
    const bool needs_mask = wp.last_r || wp.last_c || padded;
    // Exclusions of a shifted window fall on whole 8-slot groups when nothing
    // is padded and the column split M - shift is a multiple of 8: a lane's
    // group (8 keys of one key row against one query, or 8 queries of one
    // query row against one key) is then kept or dropped as a whole, and a
    // dropped group reads the table's -inf row (mask mode 2, one select per
    // group instead of one per pair; mode 1 masks every pair).  With M = 16
    // and shift 8 a tile is one row and a 32-slot chunk two rows, so in a
    // window of the last row every tile sees only one half of the chunks
    // (HALF: the loop runs over that half).
    const bool group_masks = POS == SWIN_POS_TABLE && !padded && (!wp.last_c || ((M - g.shift) & 7) == 0);
    const bool half_rows = NCH == 8 && M == 16 && !padded && wp.last_r && g.shift == 8;
    const int mask_mode = !needs_mask ? 0 : !group_masks ? 1 : (half_rows && !wp.last_c) ? 0 : 2;
    const int negrow = S * S;
    const int kbase = (grp / GPR) * S + 8 * (grp % GPR);   // bias offset of this lane's key group, chunk 0
    // lane offsets of the chunk loops' LDS fragments (the swizzles do not
    // change from chunk to chunk: chunk c adds 32 c D elements)
    const int offA = row_off(8 * (li >> 2) + (li & 3), grp);   // A rows sA (and sA + 4: + 4 D)
    const int vo0 = vt_off(0, grp, li), vo1 = vt_off(1, grp, li);
    auto fragA = [&](const __bf16* rows, int c, int second) -> bf16x8 {
        return *(const bf16x8*)(rows + offA + (32 * c + 4 * second) * D);
    };

    // ---- pass 0: log-sum-exp of this wave's queries, or the forward's
    // (natural log, to log2 units)
    if (active && p.lse) {
        const float* lin = p.lse + ((size_t)win * g.heads + h) * N;
        for (int t = rank * 64 + lane; t < N; t += 64 * QW) {
            const int ri = qdiv(t, L.inv_M), ci = t - ri * M;
            lse[ri * 8 * GPR + ci] = lin[t] * kLog2e;
        }
    } else if (active) {
        for (int t0 = rank; t0 < L.NQT; t0 += QW) {
            const int t = t0 * 16 + li;
            const bool tv = t < N;
            const int tt = tv ? t : 0;
            const int ri = qdiv(tt, L.inv_M), ci = tt - ri * M;
            const int qs_slot = ri * 8 * GPR + ci;
            const bf16x8 qf = PHASED ? gfrag(qg, qs_slot, grp) : rowfrag(qrow, qs_slot, grp);
            const float qs = qsc[qs_slot];
            const int qoff = (M - 1 - ri) * S + (M - 1 - ci) + kbase;
            int rlo = 0, rhi = M, clo = 0, chi = M;
            if (wp.last_r) { if (ri < M - g.shift) rhi = M - g.shift; else rlo = M - g.shift; }
            if (wp.last_c) { if (ci < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
            const uint32_t cmask = (((1u << chi) - 1u) & ~((1u << clo) - 1u));
            float m = -INFINITY, l = 0.0f;
#pragma unroll 2
            for (int c = 0; c < NCH; ++c) {
                const bf16x8 ka = fragA(krow, c, 0), kb = fragA(krow, c, 1);
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                const f32x4 sa = mfma(ka, qf, z), sb = mfma(kb, qf, z);
                const f32x4 k0 = *(const f32x4*)(ksc + 32 * c + 8 * grp);
                const f32x4 k1 = *(const f32x4*)(ksc + 32 * c + 8 * grp + 4);
                const int gam = 4 * c + grp, rj = gam / GPR, cj0 = 8 * (gam % GPR);
                const uint32_t bits = !needs_mask ? 0xffu
                                    : tv && rj >= rlo && rj < rhi && rj < M ? (cmask >> cj0) & 0xffu : 0u;
                float x[8];
                float cm = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sv = e < 4 ? sa[e] : sb[e - 4];
                    const float kv = e < 4 ? k0[e] : k1[e - 4];
                    const bool ok = ((bits >> e) & 1u) != 0u;
                    float b = 0.0f;
                    if (POS == SWIN_POS_TABLE) b = bias2[ok ? qoff + (4 / GPR) * c * S + e : negrow];
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
            l = sum_x32(sum_x16(l));
            if (grp == 0 && tv) lse[qs_slot] = m + __builtin_amdgcn_logf(l);
        }
    }
    __syncthreads();
    const float inv_tau = 1.0f / tau;
    float dtau_acc = 0.0f;
    const Rsrc dqr = make_rsrc((const uint16_t*)a.dq + wp.base + h * D, bytes);
    const Rsrc dkr = make_rsrc((const uint16_t*)a.dk + wp.base + h * D, bytes);
    const Rsrc dvr = make_rsrc((const uint16_t*)a.dv + wp.base + h * D, bytes);
    // ---- pass B: dq of this wave's queries (query-major); MASK: the
    // window has shift regions or padded slots (else every pair counts)
    auto pass_b = [&](auto mflag, auto hflag) {
        constexpr int MK = decltype(mflag)::value;
        constexpr bool MASK = MK == 1;
        constexpr bool HALF = decltype(hflag)::value;
        for (int t0 = rank; t0 < L.NQT; t0 += QW) {
            const int t = t0 * 16 + li;
            const bool tv = !MASK || t < N;
            const int tt = tv ? t : 0;
            const int ri = RT ? t0 : qdiv(tt, L.inv_M), ci = RT ? li : tt - ri * M;
            const int qs_slot = ri * 8 * GPR + ci;
            const uint32_t qtok = RT ? wg.row(t0) + lcol : 0u;
            const bf16x8 qf = RT ? tfrag(qg, qtok, grp) : PHASED ? gfrag(qg, qs_slot, grp) : rowfrag(qrow, qs_slot, grp);
            const bf16x8 gf = RT ? tfrag(dg, qtok, grp) : PHASED ? gfrag(dg, qs_slot, grp) : rowfrag(orow, qs_slot, grp);
            const float qs = qsc[qs_slot], lq = lse[qs_slot], Dq = dd[qs_slot];
            const int qoff = (M - 1 - ri) * S + (M - 1 - ci) + kbase;
            int rlo = 0, rhi = M, clo = 0, chi = M;
            if (wp.last_r) { if (ri < M - g.shift) rhi = M - g.shift; else rlo = M - g.shift; }
            if (wp.last_c) { if (ci < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
            const uint32_t cmask = (((1u << chi) - 1u) & ~((1u << clo) - 1u));
            f32x4 G0 = {0.0f, 0.0f, 0.0f, 0.0f}, G1 = G0;
            float dts = 0.0f;                              // sum over keys of dS~ s (dtau without a_i)
            // HALF: key rows [rlo, rhi) are chunks [rlo / 2, rhi / 2)
            const int c_beg = HALF ? rlo >> 1 : 0;
#pragma unroll 2
            for (int cc = 0; cc < (HALF ? NCH / 2 : NCH); ++cc) {
                const int c = c_beg + cc;
                const bf16x8 ka = fragA(krow, c, 0), kb = fragA(krow, c, 1);
                const bf16x8 va = fragA(vrow, c, 0), vb = fragA(vrow, c, 1);
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                const f32x4 sa = mfma(ka, qf, z), sb = mfma(kb, qf, z);
                const f32x4 pa = mfma(va, gf, z), pb = mfma(vb, gf, z);
                const f32x4 k0 = *(const f32x4*)(ksc + 32 * c + 8 * grp);
                const f32x4 k1 = *(const f32x4*)(ksc + 32 * c + 8 * grp + 4);
                const int gam = 4 * c + grp, rj = gam / GPR, cj0 = 8 * (gam % GPR);
                const int boff = qoff + (4 / GPR) * c * S;
                const float* brow = bias2 + (MK == 2 && !(rj >= rlo && rj < rhi && ((cmask >> cj0) & 1u)) ? negrow : boff);
                // allowed keys of this lane's 8-key group (bit e: key column cj0 + e)
                const uint32_t bits = !MASK ? 0xffu : tv && rj >= rlo && rj < rhi && rj < M ? (cmask >> cj0) & 0xffu
                                                                                             : 0u;
                float ds[8], dlv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sv = e < 4 ? sa[e] : sb[e - 4];
                    const float dpv = e < 4 ? pa[e] : pb[e - 4];
                    const float kv = e < 4 ? k0[e] : k1[e - 4];
                    const bool ok = !MASK || ((bits >> e) & 1u) != 0u;
                    float b = 0.0f;
                    if (POS == SWIN_POS_TABLE) b = MASK ? bias2[ok ? boff + e : negrow] : brow[e];   // -inf: excluded
                    // logit (log2 units) = s a_i c_j + b, a_i c_j = qs kv (DOT: kv = 1)
                    float arg = fmaf(sv, SIM == SWIN_SIM_COSINE ? qs * kv : qs, b) - lq;
                    if (POS != SWIN_POS_TABLE && MASK) arg = ok ? arg : -INFINITY;
                    const float pr = __builtin_amdgcn_exp2f(arg);
                    const float dl = pr * (dpv - Dq);
                    // COSINE: dS~ = dl c_j (dq's a_i after the sum); DOT: dl (1/sqrt(d) after)
                    ds[e] = SIM == SWIN_SIM_COSINE ? dl * kv : dl;
                    dlv[e] = dl;
                    if (SIM == SWIN_SIM_COSINE) dts = fmaf(ds[e], sv, dts);
                    if (POS == SWIN_POS_TABLE && !DIAG && a.dtable && ok) fixed::add(&dtab[boff + e], dl);
                }
                if (POS == SWIN_POS_TABLE && DIAG && a.dtable) {
                    // M == 16: the tile is one window row, lane li its column li,
                    // so (lane li, element e) lands at boff(0) - li + e.  Row sums
                    // along those diagonals: lane li gathers d = -li from lanes
                    // li + e (element e) and, for li = 1..7, d = 8 - li from lanes
                    // li - 8 + e; excluded pairs carry dl = 0.
                    float A = dlv[0] + row_shl<1>(dlv[1]) + row_shl<2>(dlv[2]) + row_shl<3>(dlv[3]) +
                              row_shl<4>(dlv[4]) + row_shl<5>(dlv[5]) + row_shl<6>(dlv[6]) + row_shl<7>(dlv[7]);
                    float B = row_shr<8>(dlv[0]) + row_shr<7>(dlv[1]) + row_shr<6>(dlv[2]) + row_shr<5>(dlv[3]) +
                              row_shr<4>(dlv[4]) + row_shr<3>(dlv[5]) + row_shr<2>(dlv[6]) + row_shr<1>(dlv[7]);
                    // The rows of lane groups 2p and 2p+1 hold the two column
                    // halves of one key row (positions b-15..b and b-7..b+15):
                    // group 2p keeps b - li (adding group 2p+1's A from lane
                    // li + 8), group 2p+1 takes b + 16 - li (its B for li < 8,
                    // else its A and group 2p's B from lane li - 8).  One
                    // atomic per lane, no two lanes of the wave on one address.
                    const bool even = (grp & 1) == 0;
                    const auto sA = __builtin_amdgcn_permlane16_swap(__float_as_uint(A), __float_as_uint(A), false,
                                                                     false);
                    const auto sB = __builtin_amdgcn_permlane16_swap(__float_as_uint(B), __float_as_uint(B), false,
                                                                     false);
                    const float pA = __uint_as_float(even ? sA[1] : sA[0]);
                    const float pB = __uint_as_float(even ? sB[1] : sB[0]);
                    const float te = A + row_shl<8>(pA);
                    const float to = row_shr<8>(A) + row_shr<8>(pB);
                    const float T = __builtin_unpredictable(even) ? te : (__builtin_unpredictable(li <= 7) ? B : to);
                    // T is zero for lane 0 of an odd group (every source of its
                    // B lies outside the row); its add is kept so that no part
                    // of the sum sits under a branch
                    fixed::add(&dtab[boff + (even ? 0 : 8)], T);
                }
                const bf16x8 dsb = pack_bf16x8(ds);
                G0 = mfma(vt_frag_at(krow + 32 * c * D + vo0), dsb, G0);
                G1 = mfma(vt_frag_at(krow + 32 * c * D + vo1), dsb, G1);
            }
            // sum dl (log2-unit logit without the bias) = qs sum dS~ s
            if (SIM == SWIN_SIM_COSINE) dtau_acc = fmaf(dts, qs, dtau_acc);
            // lane holds channels 4 grp..+3 and 16 + 4 grp..+3 of query li
            float q8[8], g8[8];
            {
                if (RT) {                                  // the query's raw channels
                    const bf16x8 lo = tfrag(qg, qtok, grp >> 1), hi = tfrag(qg, qtok, 2 + (grp >> 1));
                    const int o = 4 * (grp & 1);
#pragma unroll
                    for (int e = 0; e < 4; ++e) { q8[e] = (float)lo[o + e]; q8[4 + e] = (float)hi[o + e]; }
                } else if (PHASED) gquad(qg, qs_slot, q8);
                else lquad(qrow, qs_slot, q8);
                g8[0] = G0[0]; g8[1] = G0[1]; g8[2] = G0[2]; g8[3] = G0[3];
                g8[4] = G1[0]; g8[5] = G1[1]; g8[6] = G1[2]; g8[7] = G1[3];
            }
            float dqv[8];
            if (SIM == SWIN_SIM_COSINE) {
                float qg = 0.0f, qq = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) { qg = fmaf(q8[e], g8[e], qg); qq = fmaf(q8[e], q8[e], qq); }
                qg = sum_x32(sum_x16(qg));
                qq = sum_x32(sum_x16(qq));
                const float nq = sqrtf(qq);
                const float ai = inv_tau / fmaxf(nq, 1e-12f);
                const float pj = nq > 1e-12f ? qg / qq : 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) dqv[e] = ai * (g8[e] - q8[e] * pj);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) dqv[e] = g8[e] * 0.17677669529663687f;
            }
            const uint32_t off = RT ? qtok + 8u * grp : masked(wg.tok(ri, ci) + 8u * grp, tv);
            store8(dqr, off, pack_bf16x4(dqv[0], dqv[1], dqv[2], dqv[3]));
            store8(dqr, off + 32u, pack_bf16x4(dqv[4], dqv[5], dqv[6], dqv[7]));
        }
    };
    if (active) {
        if (mask_mode == 1) pass_b(Mode<1>{}, Flag<false>{});
        else if (half_rows) {
            if (mask_mode == 2) pass_b(Mode<2>{}, Flag<true>{});
            else pass_b(Mode<0>{}, Flag<true>{});
        } else if (mask_mode == 2) pass_b(Mode<2>{}, Flag<false>{});
        else pass_b(Mode<0>{}, Flag<false>{});
    }
    if (PHASED) {
        // ---- Q and dout rows replace K and V
        __syncthreads();
        stage_rows(p.q, a.dout, qrow);
        vm_wait_all();
        __syncthreads();
    }
    // ---- pass A: dk, dv of this wave's 16-key tiles (key-major)
    auto pass_a = [&](auto mflag, auto hflag) {
        constexpr int MK = decltype(mflag)::value;
        constexpr bool MASK = MK == 1;
        constexpr bool HALF = decltype(hflag)::value;
        const int nkt = (L.NSP + 15) / 16;
        for (int kt = rank; kt < nkt; kt += QW) {
            const int sk = 16 * kt + li;                   // this lane's key slot
            int rj, cj;
            slot_rc<GPR>(sk, rj, cj);
            if (RT) { rj = kt; cj = li; }
            const bool kv_ok = rj < M && cj < M;
            const uint32_t ktok = RT ? wg.row(kt) + lcol : 0u;
            const bf16x8 kB = RT ? tfrag(kg, ktok, grp) : PHASED ? gfrag(kg, sk, grp) : rowfrag(krow, sk, grp);
            const bf16x8 vB = RT ? tfrag(vg, ktok, grp) : PHASED ? gfrag(vg, sk, grp) : rowfrag(vrow, sk, grp);
            const float cj_s = ksc[sk];
            int rlo = 0, rhi = M, clo = 0, chi = M;
            if (wp.last_r) { if (rj < M - g.shift) rhi = M - g.shift; else rlo = M - g.shift; }
            if (wp.last_c) { if (cj < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
            const uint32_t cmask = ((chi >= 32 ? 0xffffffffu : ((1u << chi) - 1u)) & ~((1u << clo) - 1u)) &
                                   ((1u << M) - 1u);
            f32x4 V0 = {0.0f, 0.0f, 0.0f, 0.0f}, V1 = V0, H0 = V0, H1 = V0;
            // HALF: query rows [rlo, rhi) are chunks [rlo / 2, rhi / 2)
            const int c_beg = HALF ? rlo >> 1 : 0;
#pragma unroll 2
            for (int cc = 0; cc < (HALF ? NCH / 2 : NCH); ++cc) {
                const int c = c_beg + cc;
                const bf16x8 qa = fragA(qrow, c, 0), qb = fragA(qrow, c, 1);
                const bf16x8 ga = fragA(orow, c, 0), gb = fragA(orow, c, 1);
                // this lane's query slots: 32 c + 8 grp + e, a row segment
                const int qs0 = 32 * c + 8 * grp;
                const f32x4 dA = *(const f32x4*)(dd + qs0), dB = *(const f32x4*)(dd + qs0 + 4);
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                const f32x4 sa = mfma(qa, kB, z), sb = mfma(qb, kB, z);
                const f32x4 pa = mfma(ga, vB, z), pb = mfma(gb, vB, z);
                const f32x4 qsA = *(const f32x4*)(qsc + qs0), qsB = *(const f32x4*)(qsc + qs0 + 4);
                const f32x4 lA = *(const f32x4*)(lse + qs0), lB = *(const f32x4*)(lse + qs0 + 4);
                const int gam = 4 * c + grp, ri = gam / GPR, ci0 = 8 * (gam % GPR);
                // query (ri, ci0 + e) against key (rj, cj): table row
                // (ri - rj + M-1) S + (ci0 + e - cj + M-1), reversed position
                // S*S - 1 - that, decreasing in e
                const int rev7 = S * S - 8 - ((ri - rj + M - 1) * S + (ci0 - cj + M - 1));   // rev. pos. of e = 7
                const float* brow =
                    bias2 + (MK == 2 && !(ri >= rlo && ri < rhi && ((cmask >> ci0) & 1u)) ? negrow : rev7);
                const bool rok = kv_ok && ri < M && ri >= rlo && ri < rhi;
                const uint32_t cbits = rok ? (cmask >> ci0) & 0xffu : 0u;
                float pp[8], dsa[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float sv = e < 4 ? sa[e] : sb[e - 4];
                    const float dpv = e < 4 ? pa[e] : pb[e - 4];
                    const float qv = e < 4 ? qsA[e] : qsB[e - 4];
                    const float lv = e < 4 ? lA[e] : lB[e - 4];
                    const bool ok = !MASK || ((cbits >> e) & 1u) != 0u;
                    float b = 0.0f;
                    if (POS == SWIN_POS_TABLE) b = MASK ? bias2[ok ? rev7 + (7 - e) : negrow] : brow[7 - e];
                    // (the select also covers padded query slots, whose statistics are unset)
                    const float arg = fmaf(sv * qv, cj_s, b) - lv;
                    const float pr = __builtin_amdgcn_exp2f(!MASK || ok ? arg : -INFINITY);
                    pp[e] = pr;
                    const float dl = pr * (dpv - (e < 4 ? dA[e] : dB[e - 4]));
                    // dS~ = dl log2(e) a_i (COSINE) or dl (DOT); the constant after the sum
                    dsa[e] = SIM == SWIN_SIM_COSINE ? dl * qv : dl;
                }
                const bf16x8 pbf = pack_bf16x8(pp), dsb = pack_bf16x8(dsa);
                V0 = mfma(vt_frag_at(orow + 32 * c * D + vo0), pbf, V0);
                V1 = mfma(vt_frag_at(orow + 32 * c * D + vo1), pbf, V1);
                H0 = mfma(vt_frag_at(qrow + 32 * c * D + vo0), dsb, H0);
                H1 = mfma(vt_frag_at(qrow + 32 * c * D + vo1), dsb, H1);
            }
            // lane holds channels 4 grp..+3 and 16 + 4 grp..+3 of key slot sk
            float k8[8], h8[8], dkv[8];
            {
                if (RT) {                                  // the key's raw channels
                    const bf16x8 lo = tfrag(kg, ktok, grp >> 1), hi = tfrag(kg, ktok, 2 + (grp >> 1));
                    const int o = 4 * (grp & 1);
#pragma unroll
                    for (int e = 0; e < 4; ++e) { k8[e] = (float)lo[o + e]; k8[4 + e] = (float)hi[o + e]; }
                } else if (PHASED) gquad(kg, sk, k8);
                else lquad(krow, sk, k8);
                // the constant of dS~: 1/log2(e) (COSINE) or 1/sqrt(d) (DOT)
                const float hs = SIM == SWIN_SIM_COSINE ? 1.0f / kLog2e : 0.17677669529663687f;
                h8[0] = H0[0] * hs; h8[1] = H0[1] * hs; h8[2] = H0[2] * hs; h8[3] = H0[3] * hs;
                h8[4] = H1[0] * hs; h8[5] = H1[1] * hs; h8[6] = H1[2] * hs; h8[7] = H1[3] * hs;
            }
            if (SIM == SWIN_SIM_COSINE) {
                float kh = 0.0f, kk = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) { kh = fmaf(k8[e], h8[e], kh); kk = fmaf(k8[e], k8[e], kk); }
                kh = sum_x32(sum_x16(kh));
                kk = sum_x32(sum_x16(kk));
                const float nk = sqrtf(kk);
                const float pj = nk > 1e-12f ? kh / kk : 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) dkv[e] = cj_s * (h8[e] - k8[e] * pj);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) dkv[e] = h8[e];
            }
            const uint32_t off = RT ? ktok + 8u * grp : masked(wg.tok(rj, cj) + 8u * grp, kv_ok);
            store8(dkr, off, pack_bf16x4(dkv[0], dkv[1], dkv[2], dkv[3]));
            store8(dkr, off + 32u, pack_bf16x4(dkv[4], dkv[5], dkv[6], dkv[7]));
            store8(dvr, off, pack_bf16x4(V0[0], V0[1], V0[2], V0[3]));
            store8(dvr, off + 32u, pack_bf16x4(V1[0], V1[1], V1[2], V1[3]));
        }
    };
    if (active) {
        if (mask_mode == 1) pass_a(Mode<1>{}, Flag<false>{});
        else if (half_rows) {
            if (mask_mode == 2) pass_a(Mode<2>{}, Flag<true>{});
            else pass_a(Mode<0>{}, Flag<true>{});
        } else if (mask_mode == 2) pass_a(Mode<2>{}, Flag<false>{});
        else pass_a(Mode<0>{}, Flag<false>{});
        if (SIM == SWIN_SIM_COSINE && a.dtau) {
            const float s = wave_reduce<Op::Sum>(dtau_acc);
            if (lane == 0) red[wave] = s;
        }
    }
    if (SIM == SWIN_SIM_COSINE && a.dtau && !active && lane == 0) red[wave] = 0.0f;
    __syncthreads();
    // ---- this workgroup's share of dtau and of the table gradient
    if (SIM == SWIN_SIM_COSINE && a.dtau && tid == 0 && p.tau[h] > p.tau_min) {
        float s = 0.0f;
        for (int w = 0; w < WAVES; ++w) s += red[w];
        // sum dl cos / tau: xs = log2(e) cos / tau
        unsafeAtomicAdd(&a.dtau[h], s * (-1.0f / (kLog2e * p.tau[h])));
    }
    if (POS == SWIN_POS_TABLE && a.dtable)
        for (int i = tid; i < S * S; i += 256)
            if (dtab[i] != 0ull)
                unsafeAtomicAdd(&a.dtable[(size_t)(S * S - 1 - i) * g.heads + h], fixed::from_fixed(dtab[i]));
}

template <int SIM, int POS>
hipError_t launch_nch(const AttnParams& p, const BwdSmallArgs& a, const BwdLayout& L, int nch, int grid,
                      size_t lds, hipStream_t s)
{
    auto* fn = nch <= 2 ? attn_bwd_small_kernel<SIM, POS, 2, 1, false, false>
             : nch <= 6 ? attn_bwd_small_kernel<SIM, POS, 6, 4, false, false>
             : p.g.M == 16 ? (POS == SWIN_POS_TABLE ? attn_bwd_small_kernel<SIM, POS, 8, 4, true, true>
                                                    : attn_bwd_small_kernel<SIM, POS, 8, 4, false, true>)
                        : attn_bwd_small_kernel<SIM, POS, 8, 4, false, false>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<grid, WAVES * 64, lds, s>>>(p, a, L);
    return hipGetLastError();
}

}  // namespace

bool attn_bwd_small_supported(const AttnParams& p)
{
    const Geometry& g = p.g;
    const int SR = (g.M + 7) / 8 * 8;
    return p.dtype == SWIN_DT_BF16 && p.pos != SWIN_POS_ROPE2D && g.d == D && g.M * SR <= 256 &&
           (int64_t)g.H * g.W * g.C * 2 < ((int64_t)1 << 31) && (int64_t)g.W * g.C * 2 < ((int64_t)1 << 24);
}

hipError_t launch_attn_bwd_small(const AttnParams& p, const void* out, const void* dout, void* dq, void* dk,
                                 void* dv, float* dtau, float* dtable, hipStream_t stream)
{
    const Geometry& g = p.g;
    if (g.nwin == 0) return hipSuccess;
    BwdSmallArgs a{out, dout, dq, dk, dv, dtau, dtable};
    BwdLayout L;
    L.NSP = g.M * ((g.M + 7) / 8 * 8);
    L.NQT = (g.N + 15) / 16;
    L.inv_M = 1.0f / (float)g.M;
    const int nch_real = (L.NSP + 31) / 32;
    const int nch = nch_real <= 2 ? 2 : nch_real <= 6 ? 6 : 8;
    const int wh = nch <= 2 ? WAVES : 1;
    const int S = 2 * g.M - 1;
    const int64_t wgs = (int64_t)g.heads * ((g.nwin + wh - 1) / wh);
    if (wgs > INT32_MAX - 8) return hipErrorInvalidValue;
    L.wgs = (int)wgs;
    L.P = (int)((wgs + 7) / 8);
    const int64_t grid = 8 * (int64_t)L.P;
    const int ns = nch * 32;
    const int nrows = wh == 1 ? 2 : 4;                              // phased when four waves share a window
    size_t lds = (size_t)(16 + wh * 4 * ns) * sizeof(float) + (size_t)wh * nrows * ns * D * 2;
    if (p.pos == SWIN_POS_TABLE) lds += (size_t)3 * ((S * S + 8 + 3) / 4 * 4) * sizeof(float);   // bias2, dtab
    if (p.sim == SWIN_SIM_COSINE) {
        if (p.pos == SWIN_POS_TABLE) return launch_nch<SWIN_SIM_COSINE, SWIN_POS_TABLE>(p, a, L, nch, (int)grid, lds, stream);
        return launch_nch<SWIN_SIM_COSINE, SWIN_POS_NONE>(p, a, L, nch, (int)grid, lds, stream);
    }
    if (p.pos == SWIN_POS_TABLE) return launch_nch<SWIN_SIM_DOT, SWIN_POS_TABLE>(p, a, L, nch, (int)grid, lds, stream);
    return launch_nch<SWIN_SIM_DOT, SWIN_POS_NONE>(p, a, L, nch, (int)grid, lds, stream);
}

}  // namespace swin
