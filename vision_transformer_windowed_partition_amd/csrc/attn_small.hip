// Window attention for windows of up to 256 tokens (M <= 16) on the gfx950
// matrix cores, with each window-head's keys and values staged once in LDS.
//
// Same computation as the general kernel (SwinV2 card eq. 1-2 and its
// window-attention pseudocode, log-CPB table of eq. 3-4, cyclic-shift or
// interleaved windows; rotary positions go to the large-window kernel),
// organised for small windows.  A workgroup of four wavefronts serves one
// head: for 9 <= M <= 16 all four share one window (each takes every fourth
// query tile), for M <= 8 each takes a window of its own (without a table
// and with an even head count, two windows of a head pair instead, so the
// two 64-byte halves of each 128-byte line are read together on one CU).
// The wavefronts of
// a window stage it together and then meet at the workgroup's only barrier:
//   K^ (keys x d): A operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16); each
//      lane loads 16 contiguous bytes of one key, the four lanes of a key
//      unit-normalise it together, and the fragments go to LDS in operand
//      order (one 16-byte read per lane and tile later);
//   V  (keys x d): copied by LDS-DMA (buffer_load ... lds) into rows of 64
//      bytes whose 16-byte pieces are XOR-swizzled through the choice of
//      source address; A operand of O^T = V^T P^T, read back transposed by
//      ds_read_b64_tr_b16 per chunk of 32 keys;
//   the bias table of the head, reversed (consecutive keys read consecutive
//      floats), in log2 units less a per-head offset every wavefront knows
//      before the barrier; each wavefront writes a quarter and posts its
//      extrema.
// The score tile leaves the MFMA with each lane holding 8 consecutive key
// slots of one query, the B-operand layout of P^T, so the softmax runs in
// registers between the two products; row sums come from a third MFMA
// against an all-ones operand.  For COSINE, k^ carries the head's
// log2(e)/tau and q enters unit-normalised, and the table entries (or the
// constant -log2(e)/tau) start the accumulator of S^T: the products leave
// shifted logits in log2 units and each score costs one exp2 and half a
// pack, no FMA.
//
// Precision.  COSINE normally feeds the MFMA k^ log2(e)/tau and q / ||q||,
// each rounded to bf16; each rounding (2^-9 of the norm) is multiplied by
// 1/tau, so for tau < 0.1 a window feeds the raw bf16 q and k (exact) and
// scales each score by 1/(||q_i|| ||k_j|| tau) in fp32 instead.  The softmax
// uses a static shift (cos <= 1, or Cauchy-Schwarz for DOT) when the spread
// of the logits stays within 2^60, else the running maximum per 32-key
// chunk.
#include "common.hpp"
#include "launch.hpp"
#include "lanes.hpp"
#include "tile_io.hpp"
#include "small_core.hpp"

namespace swin {

namespace {

using namespace tio;
using namespace lanes;
using namespace core;

struct SmallLayout {
    int NSP;                   // key slots in use: M rows of M rounded up to 8
    int NQT;                   // query tiles of 16 per window
    int wgs;                   // workgroups with work: heads * window blocks
    int P;                     // work ids per XCD slot
    int hpair;                 // M <= 8, no table, even heads: a workgroup takes two windows of a head pair
    float inv_M;
};

// NCH chunks of 32 key slots per window; QW wavefronts per window.
// RT: query tiles that are whole window rows, so that a tile's row offsets
// are the same for every lane (scalar) and its columns the lane's own:
// 1 for M = 16 (tile tq is row tq, query column li), 2 for M = 8 (rows
// 2 tq and 2 tq + 1, column li % 8); 0 for other M.
template <int SIM, int POS, int NCH, int QW, int RT>
__global__ void __launch_bounds__(256)
attn_small_kernel(AttnParams p, SmallLayout L)
{
    // groups of 8 key slots per key row: M <= 8 gives 8 slots per row and
    // at most 2 chunks of 32, 9 <= M <= 16 gives 16 slots per row
    constexpr int GPR = NCH <= 2 ? 1 : 2;
    constexpr int WH = WAVES / QW;                 // windows per workgroup
    constexpr int SETS = 2 * NCH / QW;             // K tiles and 1 KB V pieces staged per wave
    constexpr int TQ = NCH <= 2 ? 1 : 4;           // table entries per lane and wave: (2M-1)^2 <= 256 TQ
    extern __shared__ __attribute__((aligned(16))) float smem_f[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: item math stays scalar
    const int grp = lane >> 4;       // 16-lane group: k-range of the operands
    const int li = lane & 15;        // row / column inside a 16 x 16 tile
    const int wh = wave / QW;        // window of this wave within the workgroup
    const int rank = wave - wh * QW; // rank among the waves of that window

    const int tabsz = POS == SWIN_POS_TABLE ? (S * S + 8 + 3) / 4 * 4 : 0;
    float* bias2 = smem_f;                                            // [S*S + 8] (TABLE)
    float* red = bias2 + tabsz;                                       // [3 * WAVES]
    float* kinv = red + 16 + wh * (NCH * 32);                         // [NCH*32] 1/||k|| (precise path)
    bf16x8* kst = (bf16x8*)(red + 16 + WH * NCH * 32) + wh * (NCH * 2 * 64);       // [NCH][2][64]
    __bf16* vst = (__bf16*)((bf16x8*)(red + 16 + WH * NCH * 32) + WH * NCH * 2 * 64) + wh * (NCH * 32 * D);

    // ---- item: one head (or head pair) per workgroup, window block-major.  Work ids run
    // window-block-major, head-minor, and each XCD takes a contiguous range
    // of them (consecutive blockIdx land on different XCDs): the heads of a
    // window run back to back on one XCD, so the 128-byte lines their
    // 64-byte head slices share are fetched once.
    const int work = (blockIdx.x & 7) * L.P + (blockIdx.x >> 3);
    if (work >= L.wgs) return;                            // whole workgroup, before the barrier
    int h, wloc;
    if (WH > 1 && L.hpair) {
        // two windows x heads 2j, 2j + 1: the wavefronts reading the two
        // 64-byte halves of each 128-byte line run together on one CU
        const int hp = g.heads >> 1;
        h = 2 * (work % hp) + (wh & 1);
        wloc = (work / hp) * 2 + (wh >> 1);
    } else {
        h = work % g.heads;
        wloc = (work / g.heads) * WH + wh;
    }
    const bool active = wloc < g.nwin;
    const int win = active ? wloc : 0;
    const float tau_eff = SIM == SWIN_SIM_COSINE ? fmaxf(p.tau[h], p.tau_min) : 1.0f;
    const float inv_tau = 1.0f / tau_eff;
    const bool precise = SIM == SWIN_SIM_COSINE && tau_eff < PRECISE_TAU;

    const WinPlace wp = place_window(g, win);
    const WinGeo& wg = wp.wg;
    const bool padded = 8 * GPR != M || NCH * 32 != L.NSP;
    const bool needs_mask = wp.last_r || wp.last_c || padded;
    // one buffer resource per tensor, starting at channel h*D of this image
    // (window); byte offsets are 32-bit and an offset of kNoLoad reads zero
    const uint32_t bytes = (uint32_t)(wp.span - h * D) * 2u;
    const Rsrc qr = make_rsrc((const uint16_t*)p.q + wp.base + h * D, bytes);
    const Rsrc kr = make_rsrc((const uint16_t*)p.k + wp.base + h * D, bytes);
    const Rsrc orr = make_rsrc((const uint16_t*)p.out + wp.base + h * D, bytes);
    const RawRsrc vraw = raw_rsrc((const uint16_t*)p.v + wp.base + h * D, active ? bytes : 0u);

    // RT: the lane's query column offset (its column within every tile), and
    // the byte offset of query tile tq's row for this lane
    const uint32_t qcol = RT == 1 ? wg.col(li) : RT == 2 ? wg.col(li & 7) : 0u;
    auto qrow_of = [&](int tq) -> uint32_t {
        if (RT == 1) return wg.row(tq);
        const uint32_t r0 = wg.row(2 * tq), r1 = wg.row(2 * tq + 1);
        return (li & 8) ? r1 : r0;
    };

    // ---- issue every load of the staging at once.  Key slot 8 gam + x is
    // token (gam / GPR, 8 (gam % GPR) + x).
    //   K tile f = 2c + t (this wave: f = rank + QW k): tile A of chunk c
    //   holds slots 32c + 8(r/4) + r%4, tile B the next 4 of each group of
    //   8, so that S^T hands a lane slots 32c + 8 grp + 0..7.
    u32x4 kraw[SETS];
    // RT 1: a K tile f = rank + QW k holds rows 2c, 2c + 1 (lanes li / 8) at
    // the lane's columns 8 ((li / 4) % 2) + li % 4 + 4 (f % 2), the same for
    // every k; a V piece j is row j at columns 8 (l / 32) + (l / 4) % 8
    const uint32_t kcol = RT == 1 ? wg.col(8 * ((li >> 2) & 1) + (li & 3) + 4 * (rank & 1)) + 16u * grp : 0u;
    const uint32_t vcol = RT == 1 ? wg.col(8 * (lane >> 5) + ((lane >> 2) & 7)) +
                                        16u * ((lane & 3) ^ v_swizzle(lane >> 2)) : 0u;
#pragma unroll
    for (int k = 0; k < SETS; ++k) {
        const int f = rank + QW * k, c = f >> 1, t = f & 1;
        const int gam = 4 * c + (li >> 2);
        const int rj = gam / GPR, cj = 8 * (gam % GPR) + (li & 3) + 4 * t;
        if (RT == 1) {
            // rows 2c and 2c + 1 (lanes li / 8), columns of the lane's group
            const uint32_t r0 = wg.row(2 * c), r1 = wg.row(2 * c + 1);
            kraw[k] = load16(kr, masked(((li & 8) ? r1 : r0) + kcol, active));
        } else
            kraw[k] = load16(kr, masked(wg.tok(rj, cj) + 16u * grp, active && rj < M && cj < M));
    }
    //   V piece j (1 KB of LDS, this wave: j = rank + QW k): lane l fills
    //   16 bytes at position 16 l, i.e. slot 16 j + l/4, LDS piece l%4,
    //   which holds channel piece (l%4) ^ v_swizzle(slot).
#pragma unroll
    for (int k = 0; k < SETS; ++k) {
        const int j = rank + QW * k;
        const int s = 16 * j + (lane >> 2);
        const int gam = s >> 3;
        const int rj = gam / GPR, cj = 8 * (gam % GPR) + (s & 7);
        const int piece = (lane & 3) ^ v_swizzle(s);
        if (RT == 1)
            dma16(vraw, vst + (size_t)j * 512, wg.row(j) + vcol);
        else
            dma16(vraw, vst + (size_t)j * 512, masked(wg.tok(rj, cj) + 16u * piece, rj < M && cj < M));
    }
    //   the first two query tiles of this wave: tiles rank + QW k
    u32x4 qpre[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tq = rank + QW * i;
        const int t = tq * 16 + li;
        const bool ok = active && tq < L.NQT && t < N;
        if (RT) {
            qpre[i] = load16(qr, masked(qrow_of(tq) + qcol + 16u * grp, active && tq < L.NQT));
        } else {
            const int tt = ok ? t : 0;
            const int ri = qdiv(tt, L.inv_M), ci = tt - ri * M;
            qpre[i] = load16(qr, masked(wg.tok(ri, ci) + 16u * grp, ok));
        }
    }
    //   this wave's quarter of the bias table of head h: rows (wave + 4k) 64
    //   + lane, the last row standing in for those past the end (extrema
    //   are unaffected, nothing is written for them)
    float tv[TQ], t0 = 0.0f;
    if (POS == SWIN_POS_TABLE) {
        const Rsrc tr = make_rsrc(p.table, (uint32_t)(S * S * g.heads) * 4u);
        t0 = load_f32(tr, (uint32_t)h * 4u);                // row 0: the table's offset in LDS
#pragma unroll
        for (int k = 0; k < TQ; ++k) {
            const int r = min((wave + WAVES * k) * 64 + lane, S * S - 1);
            tv[k] = load_f32(tr, (uint32_t)__umul24((uint32_t)r, (uint32_t)g.heads) * 4u + (uint32_t)h * 4u);
        }
    }
    vm_wait_all();

    // ---- bias table: this wave's quarter, reversed (row r at S*S - 1 - r),
    // in log2 units less boff (row 0, and for COSINE the largest cosine
    // logit log2(e)/tau), which every wave knows before the barrier; its
    // extrema go to red for all waves
    const float boff = kLog2e * (t0 + (SIM == SWIN_SIM_COSINE ? inv_tau : 0.0f));
    if (POS == SWIN_POS_TABLE) {
        float mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int k = 0; k < TQ; ++k) {
            const int r = (wave + WAVES * k) * 64 + lane;
            mx = fmaxf(mx, tv[k]);
            mn = fminf(mn, tv[k]);
            if (r < S * S) bias2[S * S - 1 - r] = fmaf(tv[k], kLog2e, -boff);
        }
        mx = wave_reduce<Op::Max>(mx);
        mn = wave_reduce<Op::Min>(mn);
        if (lane == 0) { red[WAVES + wave] = mx; red[2 * WAVES + wave] = mn; }
        if (wave == 0 && lane < 8) bias2[S * S + lane] = -INFINITY;
    }

    // ---- k: unit-normalise and scale by log2(e)/tau (COSINE), or keep raw
    // and record 1/||k|| (precise COSINE) or the largest ||k|| (DOT);
    // fragments to LDS in operand order, one 16-byte write per lane and tile
    float kmax = 0.0f;
#pragma unroll
    for (int k = 0; k < SETS; ++k) {
        const int f = rank + QW * k, c = f >> 1, t = f & 1;
        const float ss = sum_x32(sum_x16(sumsq8(kraw[k])));
        bf16x8 kfrag;
        if (SIM == SWIN_SIM_COSINE) {
            const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));   // 1 / max(||k||, 1e-12)
            if (precise) {
                if (grp == 0) kinv[32 * c + 8 * (li >> 2) + (li & 3) + 4 * t] = inv;
                kfrag = *(const bf16x8*)&kraw[k];
            } else {
                float kf[8];
                unpack_bf16x8(kraw[k], kf);
                const float ks = inv * (kLog2e * inv_tau);
#pragma unroll
                for (int e = 0; e < 8; ++e) kf[e] *= ks;
                kfrag = pack_bf16x8(kf);
            }
        } else {
            kmax = fmaxf(kmax, ss);
            kfrag = *(const bf16x8*)&kraw[k];
        }
        kst[f * 64 + lane] = kfrag;
    }
    if (SIM == SWIN_SIM_DOT) {
        kmax = wave_reduce<Op::Max>(kmax);
        if (lane == 0) red[wave] = kmax;
    }
    __syncthreads();                                      // K^, V, table and red complete
    if (!active) return;
    if (SIM == SWIN_SIM_DOT) {
        kmax = red[wh * QW];
#pragma unroll
        for (int r = 1; r < QW; ++r) kmax = fmaxf(kmax, red[wh * QW + r]);
        kmax = sqrtf(kmax);                               // largest ||k|| of the window
    }
    // table extrema (log2 units, as stored): the static shift puts the
    // largest possible logit at 0 or below (COSINE: cos <= 1, and the
    // table's offset already holds log2(e)/tau; DOT: Cauchy-Schwarz per
    // query)
    float bias_max = 0.0f, bias_range = 0.0f;
    if (POS == SWIN_POS_TABLE) {
        float mx = red[WAVES], mn = red[2 * WAVES];
#pragma unroll
        for (int r = 1; r < WAVES; ++r) { mx = fmaxf(mx, red[WAVES + r]); mn = fminf(mn, red[2 * WAVES + r]); }
        bias_max = fmaf(mx, kLog2e, -boff);
        bias_range = (mx - mn) * kLog2e;
    }

    // ---- this wave's query tiles rank + QW k, two at a time; the next
    // pair's query rows load while the current pair runs
    const int kbase = (grp / GPR) * S + 8 * (grp % GPR);  // bias offset of this lane's key group in chunk 0
    u32x4 qnext[2] = {qpre[0], qpre[1]};
    for (int k0 = 0; rank + QW * k0 < L.NQT; k0 += 2) {
        Tile T[2];
        int qt[2];
        bool qv[2];
        u32x4 qraw[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tq = rank + QW * (k0 + i);
            const int t = tq * 16 + li;
            qv[i] = tq < L.NQT && t < N;
            qt[i] = qv[i] ? t : 0;
            qraw[i] = qnext[i];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tq = rank + QW * (k0 + 2 + i);
            const int t = tq * 16 + li;
            const bool ok = tq < L.NQT && t < N;
            if (RT) {
                qnext[i] = load16(qr, masked(qrow_of(tq) + qcol + 16u * grp, tq < L.NQT));
            } else {
                const int tt = ok ? t : 0;
                const int ri = qdiv(tt, L.inv_M), ci = tt - ri * M;
                qnext[i] = load16(qr, masked(wg.tok(ri, ci) + 16u * grp, ok));
            }
        }
        bool any_exact = false, partial = false;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tq = qv[i] ? rank + QW * (k0 + i) : 0;
            const int ri = RT == 1 ? tq : RT == 2 ? 2 * tq + (li >> 3) : qdiv(qt[i], L.inv_M);
            const int ci = RT == 1 ? li : RT == 2 ? (li & 7) : qt[i] - ri * M;
            const u32x4 qw = qraw[i];
            T[i].qf = __builtin_bit_cast(bf16x8, qw);
            const float ss = sum_x32(sum_x16(sumsq8(qraw[i])));
            float spread, shift = 0.0f;
            if (SIM == SWIN_SIM_COSINE) {
                const float qinv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));   // 1 / max(||q||, 1e-12)
                T[i].qscale = kLog2e * inv_tau * qinv;
                T[i].negm = -kLog2e * inv_tau;
                spread = 2.0f * kLog2e * inv_tau + bias_range;
                if (!precise) {                                   // the MFMA takes q / ||q||
                    float qf[8];
                    unpack_bf16x8(qw, qf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) qf[e] *= qinv;
                    T[i].qf = pack_bf16x8(qf);
                }
            } else {
                T[i].qscale = kLog2e * 0.17677669529663687f;          // log2(e) / sqrt(32)
                const float c_i = sqrtf(ss) * kmax * T[i].qscale;
                T[i].negm = -c_i;
                spread = 2.0f * c_i + bias_range;
                shift = c_i + bias_max;
            }
            // DOT with a table: the shift enters through the accumulator of
            // S^T; no table: it is the added term.  COSINE outside the
            // precise path starts the accumulator from the stored table
            // (or -log2(e)/tau) instead; the precise path takes the running
            // maximum.  Spreads within RANGE_LIMIT keep every exp2 argument
            // of the static shift in [-60, 60].
            T[i].exact = precise || __any(!(spread <= RANGE_LIMIT)) != 0;
            T[i].cinit = SIM == SWIN_SIM_DOT && POS == SWIN_POS_TABLE ? -shift / T[i].qscale : 0.0f;
            any_exact = any_exact || T[i].exact;
            T[i].mrun = -INFINITY;
            T[i].qoff = (M - 1 - ri) * S + (M - 1 - ci) + kbase;
            T[i].colbits = 0xffu;
            T[i].gmask = 0xffffffffu;
            if (needs_mask) {
                int rlo = 0, rhi = M, clo = 0, chi = M;
                if (wp.last_r) { if (ri < M - g.shift) rhi = M - g.shift; else rlo = M - g.shift; }
                if (wp.last_c) { if (ci < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
                const uint32_t cmask = (chi >= 32 ? 0xffffffffu : ((1u << chi) - 1u)) & ~((1u << clo) - 1u);
                // this lane's key group in chunk c: row (4/GPR) c + grp/GPR, columns
                // 8 (grp % GPR) .. +7; allowed chunks are those whose row lies in
                // [rlo, rhi), if the columns are allowed at all
                constexpr int STEP = 4 / GPR, SH = STEP == 4 ? 2 : 1;
                const int rl = grp / GPR;
                T[i].colbits = (cmask >> (8 * (grp % GPR))) & 0xffu;
                const int cb = max(0, (rlo - rl + STEP - 1) >> SH);
                const int ce = min(NCH, (rhi - rl + STEP - 1) >> SH);
                const uint32_t rows = ce > cb ? ((ce >= 32 ? 0xffffffffu : (1u << ce) - 1u) & ~((1u << cb) - 1u)) : 0u;
                T[i].gmask = T[i].colbits ? rows : 0u;
                // groups split by a region edge or by padding
                partial = partial || (wp.last_c && ((M - g.shift) & 7)) || (M & 7);
            }
            T[i].o0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            T[i].o1 = T[i].o0;
            T[i].ls = T[i].o0;
        }
        const int negrow = S * S;
        if (any_exact || precise) {
            // the running maximum (rare): one tile at a time, so that its
            // registers do not set the occupancy of the common path
            run_pair<SIM, POS, GPR, 0, NCH, true, true, true, 1>(kst, vst, T, bias2, kinv, S, negrow, lane, true,
                                                                 precise);
            run_pair<SIM, POS, GPR, 0, NCH, true, true, true, 1>(kst, vst, T + 1, bias2, kinv, S, negrow, lane, true,
                                                                 precise);
        } else if (needs_mask) {
            run_masked_pair<SIM, POS, GPR, NCH>(kst, vst, T, bias2, kinv, S, negrow, lane, partial);
        } else
            run_pair<SIM, POS, GPR, 0, NCH, false, false, false, 2>(kst, vst, T, bias2, kinv, S, negrow, lane, false,
                                                                 false);

        // ---- normalise and store: lane holds channels 4 grp..+3 and
        // 16 + 4 grp..+3 of query li
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tq = rank + QW * (k0 + i);
            uint32_t off;
            if (RT) {
                off = masked(qrow_of(tq) + qcol + 8u * grp, tq < L.NQT);
            } else {
                const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
                off = masked(wg.tok(ri, ci) + 8u * grp, qv[i]);
            }
            const float inv = __builtin_amdgcn_rcpf(T[i].ls[0]);
            store8(orr, off, pack_bf16x4(T[i].o0[0] * inv, T[i].o0[1] * inv, T[i].o0[2] * inv, T[i].o0[3] * inv));
            store8(orr, off + 32u, pack_bf16x4(T[i].o1[0] * inv, T[i].o1[1] * inv, T[i].o1[2] * inv, T[i].o1[3] * inv));
            if (p.lse && grp == 0 && qv[i]) {
                // the exp2 arguments were the logits in log2 units less off:
                // the stored table's offset boff (COSINE), that and the
                // static shift c_i + bias_max (DOT with a table), or -negm;
                // plus the running maximum where it was used
                float off2 = POS == SWIN_POS_TABLE ? boff + (SIM == SWIN_SIM_DOT ? bias_max - T[i].negm : 0.0f)
                                                   : -T[i].negm;
                if (T[i].exact) off2 += T[i].mrun;
                p.lse[((size_t)win * g.heads + h) * N + qt[i]] =
                    (__builtin_amdgcn_logf(T[i].ls[0]) + off2) * kLn2;
            }
        }
    }
}

template <int SIM, int POS>
hipError_t launch_nch(const AttnParams& p, const SmallLayout& L, int nch, int grid, size_t lds, hipStream_t s)
{
    const int M = p.g.M;
    auto* fn = nch <= 2 ? (M == 8 ? attn_small_kernel<SIM, POS, 2, 1, 2> : attn_small_kernel<SIM, POS, 2, 1, 0>)
             : nch <= 6 ? attn_small_kernel<SIM, POS, 6, 4, 0>
             : M == 16  ? attn_small_kernel<SIM, POS, 8, 4, 1>
                        : attn_small_kernel<SIM, POS, 8, 4, 0>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<grid, WAVES * 64, lds, s>>>(p, L);
    return hipGetLastError();
}

}  // namespace

bool attn_small_supported(const AttnParams& p)
{
    const Geometry& g = p.g;
    const int SR = (g.M + 7) / 8 * 8;
    return p.dtype == SWIN_DT_BF16 && p.pos != SWIN_POS_ROPE2D && g.d == D && g.M * SR <= 256 &&
           (int64_t)g.H * g.W * g.C * 2 < ((int64_t)1 << 31) &&    // byte offsets of one image fit 31 bits
           (int64_t)g.W * g.C * 2 < ((int64_t)1 << 24);            // row stride fits the 24-bit multiplier
}

hipError_t launch_attn_small(const AttnParams& p, hipStream_t stream)
{
    const Geometry& g = p.g;
    if (g.nwin == 0) return hipSuccess;
    SmallLayout L;
    L.NSP = g.M * ((g.M + 7) / 8 * 8);
    L.NQT = (g.N + 15) / 16;
    L.inv_M = 1.0f / (float)g.M;
    const int nch_real = (L.NSP + 31) / 32;
    const int nch = nch_real <= 2 ? 2 : nch_real <= 6 ? 6 : 8;      // M <= 8, 9-12, 13-16
    const int wh = nch <= 2 ? WAVES : 1;                            // windows per workgroup
    const int S = 2 * g.M - 1;
    // M <= 8 without a table (whose LDS copy is one head's): head pairs
    L.hpair = wh > 1 && p.pos != SWIN_POS_TABLE && g.heads % 2 == 0 ? 1 : 0;
    const int64_t wgs = L.hpair ? (int64_t)(g.heads / 2) * ((g.nwin + 1) / 2)
                                : (int64_t)g.heads * ((g.nwin + wh - 1) / wh);
    if (wgs > INT32_MAX - 8) return hipErrorInvalidValue;
    L.wgs = (int)wgs;
    L.P = (int)((wgs + 7) / 8);
    const int64_t grid = 8 * (int64_t)L.P;
    size_t lds = (size_t)(16 + wh * nch * 32) * sizeof(float) + (size_t)wh * nch * 32 * D * 2 * 2;
    if (p.pos == SWIN_POS_TABLE) lds += (size_t)((S * S + 8 + 3) / 4 * 4) * sizeof(float);
    if (p.sim == SWIN_SIM_COSINE) {
        if (p.pos == SWIN_POS_TABLE) return launch_nch<SWIN_SIM_COSINE, SWIN_POS_TABLE>(p, L, nch, (int)grid, lds, stream);
        return launch_nch<SWIN_SIM_COSINE, SWIN_POS_NONE>(p, L, nch, (int)grid, lds, stream);
    }
    if (p.pos == SWIN_POS_TABLE) return launch_nch<SWIN_SIM_DOT, SWIN_POS_TABLE>(p, L, nch, (int)grid, lds, stream);
    return launch_nch<SWIN_SIM_DOT, SWIN_POS_NONE>(p, L, nch, (int)grid, lds, stream);
}

}  // namespace swin
