// Window attention for windows of up to 256 tokens (M <= 16) on the gfx950
// matrix cores, with the window's keys and values held in registers.
//
// Same computation as the general kernel (SwinV2 card eq. 1-2 and its
// window-attention pseudocode, log-CPB table of eq. 3-4, cyclic-shift or
// interleaved windows; rotary positions go to the general kernel), organised
// for small windows: one wavefront owns (window, head, part of the queries)
// and loads that window-head's keys and values into MFMA fragments it keeps
// in registers for all of its query tiles.
//   K  (keys x d): A operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16); each
//      lane loads 16 contiguous bytes of one key from HBM.
//   V^T (d x keys): A operand of O^T = V^T P^T; V rows are copied to a
//      wavefront-private LDS area with contiguous 16-byte writes and read
//      back transposed by ds_read_b64_tr_b16 (within each 16-lane group,
//      lane i receives element i%4 of the 4-element vectors addressed by
//      lanes 4j + i/4, j = 0..3), two reads per 8-key fragment.
// The score tile leaves the MFMA with each lane holding 8 consecutive key
// slots of one query, the B-operand layout of P^T, so the softmax runs in
// registers between the two products; row sums come from a third MFMA
// against an all-ones operand.  The four wavefronts of a workgroup share one
// head and its bias table in LDS; no workgroup barrier follows the table.
//
// Precision.  COSINE normally feeds the MFMA the unit-normalised k^ rounded
// to bf16; that rounding (2^-9 of the norm) is multiplied by 1/tau, so for
// tau < 0.1 a wavefront feeds the raw bf16 k (exact) and scales each score by
// 1/||k_j|| in fp32 instead.  The softmax uses a static shift (cos <= 1, or
// Cauchy-Schwarz for DOT) when the spread of the logits stays within 2^60,
// else the running maximum per 32-key chunk.
#include "common.hpp"
#include "launch.hpp"
#include "tile_io.hpp"

namespace swin {

namespace {

using namespace tio;

constexpr int WAVES = 4;
constexpr float RANGE_LIMIT = 60.0f;
constexpr float PRECISE_TAU = 0.1f;

typedef short i16x8 __attribute__((ext_vector_type(8)));

struct SmallLayout {
    int NSP;                   // key slots in use: M rows of M rounded up to 8
    int NQT;                   // query tiles per window-head
    int TPW;                   // query tiles per wavefront item
    int parts;                 // wavefront items per window-head
    int per_head;              // items per head, padded to a multiple of WAVES
    int wgs;                   // workgroups with work: heads * per_head / WAVES
    int P;                     // work ids per XCD slot
    float inv_M;
};

template <int NCH>
struct Frags {                 // this wave's window-head, in MFMA operand layout
    const bf16x8* k;           // LDS: k^ (or raw k: DOT, precise COSINE), [NCH][2][64 lanes]
    bf16x8 v[NCH][2];          // V^T, channels 0-15 and 16-31
    int koff[NCH];             // bias-table offset of this lane's key group: rj*S + c0
};

struct Tile {                  // one query tile of 16 queries
    bf16x8 qf;
    float qscale, negm, mrun;
    int qoff;
    uint32_t gmask;            // chunks whose key group of this lane is allowed (bit c)
    uint32_t colbits;          // allowed columns of this lane's key group (bit e)
    bool exact;
    f32x4 o0, o1, ls;
};

// One pair of query tiles against key chunks [CB, CE) of the window (the
// others are masked for both tiles).
//   MASK: shift regions / padded slots; PRECISE: scores scaled by 1/||k_j||
//   (raw k operand); EXACT: running maximum instead of the static shift.
template <int SIM, int POS, int NCH, int CB, int CE, bool MASK, bool PRECISE, bool EXACT>
__device__ __forceinline__ void run_pair(const Frags<NCH>& F, Tile (&T)[2], const float* bias2,
                                         const float* kinv, int negrow, int lane, bool partial_any,
                                         bool precise_rt)
{
    const int grp = lane >> 4;
    const bool prec = PRECISE && precise_rt;
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
#pragma unroll
    for (int c = CB; c < CE; ++c) {
        uint32_t bits[2] = {0xffu, 0xffu};
        if (MASK) {
#pragma unroll
            for (int i = 0; i < 2; ++i) bits[i] = (T[i].gmask >> c) & 1u ? T[i].colbits : 0u;
        }
        float kin[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
        if (prec) {
            const f32x4 a = *(const f32x4*)(kinv + 32 * c + 8 * grp);
            const f32x4 b = *(const f32x4*)(kinv + 32 * c + 8 * grp + 4);
            kin[0] = a[0]; kin[1] = a[1]; kin[2] = a[2]; kin[3] = a[3];
            kin[4] = b[0]; kin[5] = b[1]; kin[6] = b[2]; kin[7] = b[3];
        }
        float add[2][8];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (POS == SWIN_POS_TABLE) {
                const float* bp = bias2 + ((MASK && bits[i] == 0u) ? negrow : F.koff[c] + T[i].qoff);
#pragma unroll
                for (int e = 0; e < 8; ++e) add[i][e] = SIM == SWIN_SIM_COSINE ? bp[e] : bp[e] + T[i].negm;
            } else {
                const float a = (MASK && bits[i] == 0u) ? -INFINITY : T[i].negm;
#pragma unroll
                for (int e = 0; e < 8; ++e) add[i][e] = a;
            }
        }
        const bf16x8 ka = F.k[(c * 2 + 0) * 64 + lane];
        const bf16x8 kb = F.k[(c * 2 + 1) * 64 + lane];
        f32x4 sa[2], sb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            sa[i] = mfma(ka, T[i].qf, zero4);
            sb[i] = mfma(kb, T[i].qf, zero4);
        }
        bf16x8 pb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = sa[i][e]; x[e + 4] = sb[i][e]; }
            float sc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] = prec ? T[i].qscale * kin[e] : T[i].qscale;
            float pr[8];
            if (!EXACT || !T[i].exact) {
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(x[e], sc[e], add[i][e]));
                if (MASK && partial_any) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = (bits[i] >> e) & 1u ? pr[e] : 0.0f;
                }
            } else {
                float xs[8], cm = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xs[e] = fmaf(x[e], sc[e], add[i][e]);
                    if (MASK) xs[e] = (bits[i] >> e) & 1u ? xs[e] : -INFINITY;
                    cm = fmaxf(cm, xs[e]);
                }
                cm = fmaxf(cm, __shfl_xor(cm, 16));
                cm = fmaxf(cm, __shfl_xor(cm, 32));
                const float mnew = fmaxf(T[i].mrun, cm);
                const float mref = mnew == -INFINITY ? 0.0f : mnew;
                const float alpha = __builtin_amdgcn_exp2f(T[i].mrun - mref);
                T[i].o0 *= alpha; T[i].o1 *= alpha; T[i].ls *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(xs[e] - mref);
                T[i].mrun = mnew;
            }
            pb[i] = pack_bf16x8(pr);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            T[i].o0 = mfma(F.v[c][0], pb[i], T[i].o0);
            T[i].o1 = mfma(F.v[c][1], pb[i], T[i].o1);
            T[i].ls = mfma(ones, pb[i], T[i].ls);
        }
    }
}

template <int SIM, int POS, int NCH>
__global__ void __launch_bounds__(256)
attn_small_kernel(AttnParams p, SmallLayout L)
{
    // groups of 8 key slots per key row: M <= 8 gives 8 slots per row and
    // at most 2 chunks of 32, 9 <= M <= 16 gives 16 slots per row
    constexpr int GPR = NCH <= 2 ? 1 : 2;
    extern __shared__ __attribute__((aligned(16))) float smem_f[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: item math stays scalar
    const int grp = lane >> 4;       // 16-lane group: k-range of the operands
    const int li = lane & 15;        // row / column inside a 16 x 16 tile

    const int tabsz = POS == SWIN_POS_TABLE ? (S * S + 8 + 3) / 4 * 4 : 0;
    float* bias2 = smem_f;                                           // [S*S + 8] (TABLE)
    float* red = bias2 + tabsz;                                      // [16]
    float* kinv = red + 16 + wave * (NCH * 32);                      // [NCH*32] 1/||k|| (precise path)
    __bf16* vst = (__bf16*)(red + 16 + WAVES * NCH * 32) + wave * (NCH * 32 * D);   // [NCH*32][D] V rows

    // ---- item: one head per workgroup, one (window, query part) per wave.
    // Work ids run window-block-major, head-minor, and each XCD takes a
    // contiguous range of them (consecutive blockIdx land on different
    // XCDs): the heads of a window block run back to back on one XCD, so the
    // 128-byte lines their 64-byte head slices share are fetched once.
    const int work = (blockIdx.x & 7) * L.P + (blockIdx.x >> 3);
    if (work >= L.wgs) return;                            // whole workgroup, before any barrier
    const int h = work % g.heads;
    const int local = (work / g.heads) * WAVES + wave;
    const bool active = local < g.nwin * L.parts;
    const int win = active ? local / L.parts : 0;
    const int part = active ? local - win * L.parts : 0;
    const float tau_eff = SIM == SWIN_SIM_COSINE ? fmaxf(p.tau[h], p.tau_min) : 1.0f;
    const float inv_tau = 1.0f / tau_eff;

    // ---- bias table of head h: reversed (consecutive keys read consecutive
    // floats), in log2 units, shifted by its max (and by 1/tau for COSINE)
    float bias_range = 0.0f;
    if (POS == SWIN_POS_TABLE) {
        float mx = -INFINITY, mn = INFINITY;
        for (int i = tid; i < S * S; i += 256) {
            const float v = p.table[(size_t)(S * S - 1 - i) * g.heads + h] * kLog2e;
            bias2[i] = v;
            mx = fmaxf(mx, v);
            mn = fminf(mn, v);
        }
        if (tid < 8) bias2[S * S + tid] = -INFINITY;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            mx = fmaxf(mx, __shfl_xor(mx, off));
            mn = fminf(mn, __shfl_xor(mn, off));
        }
        if (lane == 0) { red[wave] = mx; red[4 + wave] = mn; }
        __syncthreads();
        mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        mn = fminf(fminf(red[4], red[5]), fminf(red[6], red[7]));
        bias_range = mx - mn;
        const float shift = SIM == SWIN_SIM_COSINE ? mx + kLog2e / tau_eff : mx;
        __syncthreads();
        for (int i = tid; i < S * S; i += 256) bias2[i] -= shift;
        __syncthreads();
    }
    if (!active) return;                                  // no workgroup barrier after this point

    // ---- window geometry (wave-uniform)
    WinGeo wg;
    const int nW = g.nwr * g.nwc;
    const int bimg = win / nW, wl = win - bimg * nW;
    const int wr = wl / g.nwc, wc = wl - wr * g.nwc;
    wg.colb = (uint32_t)g.C * 2u;
    int64_t base;
    int span;                                             // elements of the image (or window)
    if (g.layout == SWIN_LAYOUT_WINDOWS) {
        span = N * g.C;
        base = (int64_t)win * span;
        wg.r0 = wg.c0 = 0; wg.rs = wg.cs = 1; wg.Hm = wg.Wm = M;
    } else {
        span = g.H * g.W * g.C;
        base = (int64_t)bimg * span;
        wg.Hm = g.H; wg.Wm = g.W;
        if (g.part == SWIN_PART_INTERLEAVED) { wg.r0 = wr; wg.c0 = wc; wg.rs = g.nwr; wg.cs = g.nwc; }
        else { wg.r0 = wr * M + g.shift; wg.c0 = wc * M + g.shift; wg.rs = wg.cs = 1; }
    }
    wg.rowb = wg.Wm * wg.colb;
    const bool cyc_shift = g.part == SWIN_PART_CYCLIC && g.shift > 0;
    const bool last_r = cyc_shift && wr == g.nwr - 1;
    const bool last_c = cyc_shift && wc == g.nwc - 1;
    const bool padded = 8 * GPR != M || NCH * 32 != L.NSP;
    const bool needs_mask = last_r || last_c || padded;
    // one buffer resource per tensor, starting at channel h*D of this image
    // (window); byte offsets are 32-bit and an offset of kNoLoad reads zero
    const uint32_t bytes = (uint32_t)(span - h * D) * 2u;
    const Rsrc qr = make_rsrc((const uint16_t*)p.q + base + h * D, bytes);
    const Rsrc kr = make_rsrc((const uint16_t*)p.k + base + h * D, bytes);
    const Rsrc vr = make_rsrc((const uint16_t*)p.v + base + h * D, bytes);
    const Rsrc orr = make_rsrc((const uint16_t*)p.out + base + h * D, bytes);
    const bool precise = SIM == SWIN_SIM_COSINE && tau_eff < PRECISE_TAU;

    // ---- K fragments: tile A of chunk c holds slots 32c + 8(r/4) + r%4,
    // tile B the next 4 of each group of 8, so that S^T hands this lane slots
    // 32c + 8 grp + 0..7.  V rows go to LDS (16 bytes per lane, contiguous).
    // Key slot 8 gam + x is token (gam / GPR, 8 (gam % GPR) + x): a lane's
    // key row advances by a fixed step per chunk, its column stays put.
    Frags<NCH> F;
    u32x4 kraw[NCH][2];
    {
        const int rl = (li >> 2) / GPR;
        uint32_t colk[2];
        bool cok[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int cj = 8 * ((li >> 2) % GPR) + (li & 3) + 4 * t;
            colk[t] = wg.col(cj) + 16u * grp;
            cok[t] = cj < M;
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int rj = (4 / GPR) * c + rl;
            const uint32_t rowk = wg.row(rj);
#pragma unroll
            for (int t = 0; t < 2; ++t) kraw[c][t] = load16(kr, masked(rowk + colk[t], cok[t] && rj < M));
        }
    }
    {
        u32x4 vraw[2 * NCH];
        const int rl = (lane >> 5) / GPR;
        const int cj = 8 * ((lane >> 5) % GPR) + ((lane >> 2) & 7);
        const uint32_t colv = wg.col(cj) + 16u * (lane & 3);
        const bool cok = cj < M;
#pragma unroll
        for (int j = 0; j < 2 * NCH; ++j) {               // piece j*64 + lane: slot (.)/4, channels 8*(. % 4)
            const int rj = (2 / GPR) * j + rl;
            vraw[j] = load16(vr, masked(wg.row(rj) + colv, cok && rj < M));
        }
#pragma unroll
        for (int j = 0; j < 2 * NCH; ++j) {
            const int idx = j * 64 + lane, s = idx >> 2, piece = idx & 3;
            *(u32x4*)(vst + s * D + ((piece ^ v_swizzle(s)) * 8)) = vraw[j];
        }
    }

    // ---- V^T fragments from the wave's LDS rows: lane (li, grp) takes
    // channel 16 dt + li of slots 32c + 8 grp + 0..7.  Transposed read h
    // covers slots +4h..4h+3: lane li addresses slot + 4h + li/4, channels
    // 16 dt + 4 (li%4) .. +3, and receives channel 16 dt + li of all four.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
            i16x4 half[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int s = 32 * c + 8 * grp + 4 * h + (li >> 2);
                const int m = li & 3;
                const __bf16* src = vst + s * D + (((2 * dt + (m >> 1)) ^ v_swizzle(s)) * 8) + 4 * (m & 1);
                half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)src);
            }
            const i16x8 v = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
            F.v[c][dt] = __builtin_bit_cast(bf16x8, v);
        }
        const int gam = 4 * c + grp;
        const int rj = gam / GPR, c0 = (gam % GPR) * 8;
        F.koff[c] = rj * S + c0;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();                      // V rows consumed: the area takes K next
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- k: unit-normalise (COSINE), or keep raw and record 1/||k||
    // (precise COSINE) or the largest ||k|| (DOT); fragments to LDS in
    // operand order, one 16-byte write per lane and tile
    bf16x8* kst = (bf16x8*)vst;
    float kmax = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float kf[8];
            unpack_bf16x8(kraw[c][t], kf);
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(kf[e], kf[e], ss);
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            bf16x8 kfrag;
            if (SIM == SWIN_SIM_COSINE) {
                const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));   // 1 / max(||k||, 1e-12)
                if (precise) {
                    if (grp == 0) kinv[32 * c + 8 * (li >> 2) + (li & 3) + 4 * t] = inv;
                    kfrag = *(const bf16x8*)&kraw[c][t];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) kf[e] *= inv;
                    kfrag = pack_bf16x8(kf);
                }
            } else {
                kmax = fmaxf(kmax, ss);
                kfrag = *(const bf16x8*)&kraw[c][t];
            }
            kst[(c * 2 + t) * 64 + lane] = kfrag;
        }
    if (SIM == SWIN_SIM_DOT) {
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, off));
        kmax = sqrtf(kmax);                               // largest ||k|| of the window
    }
    F.k = kst;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- this wave's query tiles, two at a time
    const int tfirst = part * L.TPW;
    const int tlast = min(tfirst + L.TPW, L.NQT);
    for (int t0 = tfirst; t0 < tlast; t0 += 2) {
        Tile T[2];
        int qt[2];
        bool qv[2];
        u32x4 qraw[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = (t0 + i) * 16 + li;
            qv[i] = t0 + i < tlast && t < N;
            qt[i] = qv[i] ? t : 0;
            const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
            qraw[i] = load16(qr, masked(wg.tok(ri, ci) + 16u * grp, qv[i]));
        }
        bool any_exact = false, partial = false;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
            float qf[8];
            unpack_bf16x8(qraw[i], qf);
            T[i].qf = pack_bf16x8(qf);
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(qf[e], qf[e], ss);
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            float spread;
            if (SIM == SWIN_SIM_COSINE) {
                T[i].qscale = kLog2e * inv_tau * __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
                T[i].negm = POS == SWIN_POS_TABLE ? 0.0f : -kLog2e * inv_tau;
                spread = 2.0f * kLog2e * inv_tau + bias_range;
            } else {
                T[i].qscale = kLog2e * 0.17677669529663687f;          // log2(e) / sqrt(32)
                const float c_i = sqrtf(ss) * kmax * T[i].qscale;
                T[i].negm = -c_i;
                spread = 2.0f * c_i + bias_range;
            }
            T[i].exact = __any(!(spread <= RANGE_LIMIT)) != 0;
            any_exact = any_exact || T[i].exact;
            T[i].mrun = -INFINITY;
            T[i].qoff = (M - 1 - ri) * S + (M - 1 - ci);
            int rlo = 0, rhi = M, clo = 0, chi = M;
            if (last_r) { if (ri < M - g.shift) rhi = M - g.shift; else rlo = M - g.shift; }
            if (last_c) { if (ci < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
            const uint32_t cmask = (chi >= 32 ? 0xffffffffu : ((1u << chi) - 1u)) & ~((1u << clo) - 1u);
            // this lane's key group in chunk c: row (4/GPR) c + grp/GPR, columns
            // 8 (grp % GPR) .. +7; allowed chunks are those whose row lies in
            // [rlo, rhi), if the columns are allowed at all
            {
                constexpr int STEP = 4 / GPR, SH = STEP == 4 ? 2 : 1;
                const int rl = grp / GPR;
                T[i].colbits = (cmask >> (8 * (grp % GPR))) & 0xffu;
                const int cb = max(0, (rlo - rl + STEP - 1) >> SH);
                const int ce = min(NCH, (rhi - rl + STEP - 1) >> SH);
                const uint32_t rows = ce > cb ? ((ce >= 32 ? 0xffffffffu : (1u << ce) - 1u) & ~((1u << cb) - 1u)) : 0u;
                T[i].gmask = T[i].colbits ? rows : 0u;
            }
            // groups split by a region edge or by padding
            if (needs_mask) partial = partial || (last_c && ((M - g.shift) & 7)) || (M & 7);
            T[i].o0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            T[i].o1 = T[i].o0;
            T[i].ls = T[i].o0;
        }
        const int negrow = S * S;
        if (any_exact || precise)
            run_pair<SIM, POS, NCH, 0, NCH, true, true, true>(F, T, bias2, kinv, negrow, lane, true, precise);
        else if (needs_mask) {
            // chunks some lane of the pair may see: all, or one half of the key rows
            uint32_t live = T[0].gmask | T[1].gmask;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) live |= (uint32_t)__shfl_xor((int)live, o);
            live = (uint32_t)__builtin_amdgcn_readfirstlane((int)live);
            constexpr uint32_t lo_half = (1u << (NCH / 2)) - 1u;
            if ((live & ~lo_half) == 0u)
                run_pair<SIM, POS, NCH, 0, NCH / 2, true, false, false>(F, T, bias2, kinv, negrow, lane, partial, false);
            else if ((live & lo_half) == 0u)
                run_pair<SIM, POS, NCH, NCH / 2, NCH, true, false, false>(F, T, bias2, kinv, negrow, lane, partial,
                                                                          false);
            else
                run_pair<SIM, POS, NCH, 0, NCH, true, false, false>(F, T, bias2, kinv, negrow, lane, partial, false);
        } else
            run_pair<SIM, POS, NCH, 0, NCH, false, false, false>(F, T, bias2, kinv, negrow, lane, false, false);

        // ---- normalise and store: lane holds channels 4 grp..+3 and
        // 16 + 4 grp..+3 of query li
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
            const float inv = __builtin_amdgcn_rcpf(T[i].ls[0]);
            const uint32_t off = masked(wg.tok(ri, ci) + 8u * grp, qv[i]);
            store8(orr, off, pack_bf16x4(T[i].o0[0] * inv, T[i].o0[1] * inv, T[i].o0[2] * inv, T[i].o0[3] * inv));
            store8(orr, off + 32u, pack_bf16x4(T[i].o1[0] * inv, T[i].o1[1] * inv, T[i].o1[2] * inv, T[i].o1[3] * inv));
        }
    }
}

template <int SIM, int POS>
hipError_t launch_nch(const AttnParams& p, const SmallLayout& L, int nch, int grid, size_t lds, hipStream_t s)
{
    auto* fn = nch <= 2 ? attn_small_kernel<SIM, POS, 2>
             : nch <= 6 ? attn_small_kernel<SIM, POS, 6>
                        : attn_small_kernel<SIM, POS, 8>;
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
    L.TPW = L.NQT > 8 ? 8 : L.NQT;
    L.parts = (L.NQT + L.TPW - 1) / L.TPW;
    L.per_head = (g.nwin * L.parts + WAVES - 1) / WAVES * WAVES;
    L.inv_M = 1.0f / (float)g.M;
    const int nch_real = (L.NSP + 31) / 32;
    const int nch = nch_real <= 2 ? 2 : nch_real <= 6 ? 6 : 8;      // M <= 8, 9-12, 13-16
    const int S = 2 * g.M - 1;
    const int64_t wgs = (int64_t)g.heads * L.per_head / WAVES;
    if (wgs > INT32_MAX - 8) return hipErrorInvalidValue;
    L.wgs = (int)wgs;
    L.P = (int)((wgs + 7) / 8);
    const int64_t grid = 8 * (int64_t)L.P;
    size_t lds = (size_t)(16 + WAVES * nch * 32) * sizeof(float) + (size_t)WAVES * nch * 32 * D * 2;
    if (p.pos == SWIN_POS_TABLE) lds += (size_t)((S * S + 8 + 3) / 4 * 4) * sizeof(float);
    if (p.sim == SWIN_SIM_COSINE) {
        if (p.pos == SWIN_POS_TABLE) return launch_nch<SWIN_SIM_COSINE, SWIN_POS_TABLE>(p, L, nch, (int)grid, lds, stream);
        return launch_nch<SWIN_SIM_COSINE, SWIN_POS_NONE>(p, L, nch, (int)grid, lds, stream);
    }
    if (p.pos == SWIN_POS_TABLE) return launch_nch<SWIN_SIM_DOT, SWIN_POS_TABLE>(p, L, nch, (int)grid, lds, stream);
    return launch_nch<SWIN_SIM_DOT, SWIN_POS_NONE>(p, L, nch, (int)grid, lds, stream);
}

}  // namespace swin
