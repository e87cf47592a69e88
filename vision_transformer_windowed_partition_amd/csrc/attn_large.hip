// Window attention for large windows (16 < M <= 32, up to 1024 tokens), and
// for rotary positions at any M <= 32, on the gfx950 matrix cores: bf16 in,
// fp32 accumulate, bf16 out, d = 32.
//
// Same computation as the other attention kernels: the window attention of
// the SwinV2 card (eq. 1-2, the window-attention pseudocode) with the
// log-CPB table (eq. 3-4) or the FlashSwin abstract's window-local rotary
// positions, over cyclic-shift or interleaved windows; exact softmax, the
// N x N scores never stored.
//
// One workgroup of eight wavefronts per window-head.  The window's keys are
// staged once into LDS, rotated (ROPE2D), unit-normalised (COSINE) and
// rounded to bf16, in the register layout of the MFMA A operand:
//   K^ (keys x d) for S^T = K^ Q^T (v_mfma_f32_16x16x32_bf16), tile A of
//   chunk c holding slots 32c + 8(r/4) + r%4 and tile B the next 4 of each
//   group of 8, so that S^T hands lane (li, grp) the slots 32c + 8 grp + 0..7.
// The values go to LDS by LDS-DMA as rows of 64 bytes and come back as V^T
// fragments (A operand of O^T = V^T P^T) through transposed reads.  Each
// wavefront then takes query tiles wave + 8j, two at a time, through every
// key chunk: the score tile leaves the MFMA in the B-operand layout of P^T,
// so the softmax runs in registers between the two products; row sums come
// from a third MFMA against an all-ones operand.  For COSINE (outside the
// precise path below) and for DOT with rotation, the staged keys carry the
// logit scale (log2(e)/tau, or log2(e)/sqrt(d)), COSINE queries enter
// unit-normalised, and the bias term (table entry, or the constant shift)
// starts the accumulator of S^T: each score then costs one exp2 and half a
// pack, no FMA.
//
// Key slots.  Key (rj, cj) sits in slot rj*SR + cj, SR = M rounded up to 8,
// so each lane's 8 slots share one key row.  Padded slots and keys of another
// shift region are masked per 8-slot group (a group masked for a lane reads
// its bias from a row of -inf); a pair of tiles visits only the chunks whose
// key rows its queries may see.
//
// Precision.  COSINE without rotation feeds k^ log2(e)/tau and q / ||q||,
// each rounded to bf16 (error 2^-9 of the norm, multiplied by 1/tau); for
// tau < 0.1 it feeds the raw bf16 q and k instead, exactly, and scales each
// score by 1/(||q_i|| ||k_j|| tau) in fp32.  With
// rotation the rotated operands are rounded; when that error, amplified by
// 1/tau (COSINE, tau < 0.1) or by max||q|| max||k|| log2(e)/sqrt(d) > 20
// (DOT), would pass the bf16 tolerance, q and k are carried as hi + lo bf16
// pairs and every score takes three products (hi hi, lo hi, hi lo: lo lo is
// below 2^-18 of |q||k|, the order of the remainders' own rounding); the
// keys are then staged in two halves, each run by two tile pairs of every
// wavefront, and consecutive cycles of two pairs take the halves in opposite
// order, so the half a cycle ends with is staged once for the next as well.  The softmax uses a static shift (cos <= 1, or
// Cauchy-Schwarz for DOT) when the spread of a row's logits stays within
// 2^60, else the running maximum per 32-key chunk.
#include "common.hpp"
#include "launch.hpp"
#include "tile_io.hpp"

namespace swin {

namespace {

using namespace tio;

#ifndef LARGE_WAVES
#define LARGE_WAVES 8
#endif
constexpr int WAVES = LARGE_WAVES;     // wavefronts per workgroup (one workgroup per CU)
constexpr int NTHR = WAVES * 64;
constexpr int KPW = (32 + WAVES - 1) / WAVES;   // key chunks a wavefront stages, at most (1024 slots)
constexpr int QPW = (64 + WAVES - 1) / WAVES;   // query tiles of a wavefront, at most (1024 queries)
#ifndef LARGE_NT
#define LARGE_NT 2
#endif
constexpr int NT = LARGE_NT;           // query tiles a wavefront runs through the keys together
constexpr float RANGE_LIMIT = 60.0f;
constexpr float PRECISE_TAU = 0.1f;    // COSINE, no rotation: raw k and 1/||k|| below this tau
constexpr float SPLIT_TAU = 0.1f;      // COSINE with rotation: hi + lo below this tau
constexpr float SPLIT_BOUND = 20.0f;   // DOT with rotation: hi + lo past this logit bound (log2 units)

struct LargeLayout {
    int SR;                    // slots per key row: M rounded up to 8
    int GPR;                   // 8-slot groups per key row
    int NSP;                   // key slots, padded to a multiple of 32
    int NQT;                   // query tiles per window-head
    int rounds;                // passes of NT tiles per wavefront (same for all)
    int units;                 // window-heads
    int P;                     // work ids per XCD slot
    int kv_bytes;              // LDS bytes of the key/value area
    float inv_M, inv_SR, inv_GPR;
};

struct Tile {                  // one query tile of 16 queries
    bf16x8 qf, qf_lo;
    float qscale, negm, mrun;
    int qoff, rlo, rhi;
    uint32_t cmask;            // allowed key columns (bit c)
    bool exact;
    f32x4 o0, o1, ls;
};

// Views of one staged block of key slots in LDS.
struct Block {
    const bf16x8* k;           // [nch][2][64] k^ (or raw k) fragments
    const bf16x8* klo;         // remainders (split only)
    const __bf16* v;           // [nch*32][D] V rows, swizzled
    int s0;                    // first slot
    int nch;                   // 32-slot chunks
};

// The lane's 8-slot group of chunk c: key row rj, first column c0; a chunk
// spans 4 groups, so the walk advances 32 slots at a time.
struct GroupWalk {
    int rj, c0;
    __device__ __forceinline__ void start(int slot0, float inv_SR, int SR)
    {
        rj = qdiv(slot0, inv_SR);
        c0 = slot0 - rj * SR;
    }
    __device__ __forceinline__ void next(int SR, float inv_SR)
    {
        c0 += 32;                                         // < SR + 32 <= 64
        const int q = qdiv(c0, inv_SR);
        rj += q;
        c0 -= q * SR;
    }
};

// Whether a window-head runs with the scale folded into its staged keys:
// COSINE outside the precise path (q then enters unit-normalised), and DOT
// with rotation (the rotated operands are rounded in any case).
template <int SIM, int POS>
__device__ __forceinline__ bool folded(bool precise)
{
    return SIM == SWIN_SIM_COSINE ? !precise : POS == SWIN_POS_ROPE2D;
}

// One pair of query tiles against chunks [cb, ce) of a staged block.
//   MASK: shift regions / padded slots; GENERAL: running maximum for tiles
//   that need it, 1/||k_j|| scaling (precise), hi + lo products (split).
//   NU: tiles of the pair in use (1 for a wavefront's odd last tile).
template <int SIM, int POS, bool MASK, bool GENERAL, int NU>
__device__ __forceinline__ void run_pair(const Block& bk, Tile (&T)[NT], const float* bias2, const float* kinv,
                                         int S, int SR, float inv_SR, int cb, int ce, int lane,
                                         bool partial, bool precise, bool split)
{
    const int grp = lane >> 4, li = lane & 15;
    const int negrow = S * S;
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    // folded scale: the staged keys carry log2(e)/tau (COSINE) or
    // log2(e)/sqrt(d) (DOT with rotation), the bias term starts the
    // accumulator, and S^T holds the shifted logits in log2 units
    const bool fold = folded<SIM, POS>(GENERAL && precise);
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
    GroupWalk gw;
    gw.start(bk.s0 + 32 * cb + 8 * grp, inv_SR, SR);
#pragma unroll 2
    for (int c = cb; c < ce; ++c) {
        bool gok[NT];
        uint32_t bits[NT];
#pragma unroll
        for (int i = 0; i < NU; ++i) { gok[i] = true; bits[i] = 0xffu; }
        if (MASK) {
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                bits[i] = gw.rj >= T[i].rlo && gw.rj < T[i].rhi ? (T[i].cmask >> gw.c0) & 0xffu : 0u;
                gok[i] = bits[i] != 0u;
            }
        }
        float add[NT][8];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            if (POS == SWIN_POS_TABLE) {
                const float* bp = bias2 + ((MASK && !gok[i]) ? negrow : gw.rj * S + gw.c0 + T[i].qoff);
#pragma unroll
                for (int e = 0; e < 8; ++e) add[i][e] = SIM == SWIN_SIM_COSINE ? bp[e] : bp[e] + T[i].negm;
            } else {
                const float a = (MASK && !gok[i]) ? -INFINITY : T[i].negm;
#pragma unroll
                for (int e = 0; e < 8; ++e) add[i][e] = a;
            }
        }
        const bf16x8 ka = bk.k[(c * 2 + 0) * 64 + lane];
        const bf16x8 kb = bk.k[(c * 2 + 1) * 64 + lane];
        const bf16x8 v0 = vt_frag(bk.v, c, 0, grp, li);
        const bf16x8 v1 = vt_frag(bk.v, c, 1, grp, li);
        f32x4 sa[NT], sb[NT];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const f32x4 ia = {add[i][0], add[i][1], add[i][2], add[i][3]};
            const f32x4 ib = {add[i][4], add[i][5], add[i][6], add[i][7]};
            sa[i] = mfma(ka, T[i].qf, fold ? ia : zero4);
            sb[i] = mfma(kb, T[i].qf, fold ? ib : zero4);
        }
        float kin[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
        if (GENERAL) {
            if (split) {
                const bf16x8 ka_lo = bk.klo[(c * 2 + 0) * 64 + lane];
                const bf16x8 kb_lo = bk.klo[(c * 2 + 1) * 64 + lane];
#pragma unroll
                for (int i = 0; i < NU; ++i) {
                    sa[i] = mfma(ka_lo, T[i].qf, sa[i]);
                    sb[i] = mfma(kb_lo, T[i].qf, sb[i]);
                    sa[i] = mfma(ka, T[i].qf_lo, sa[i]);
                    sb[i] = mfma(kb, T[i].qf_lo, sb[i]);
                }
            }
            if (precise) {
                const f32x4 a = *(const f32x4*)(kinv + bk.s0 + 32 * c + 8 * grp);
                const f32x4 b = *(const f32x4*)(kinv + bk.s0 + 32 * c + 8 * grp + 4);
                kin[0] = a[0]; kin[1] = a[1]; kin[2] = a[2]; kin[3] = a[3];
                kin[4] = b[0]; kin[5] = b[1]; kin[6] = b[2]; kin[7] = b[3];
            }
        }
        bf16x8 pb[NT];
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = sa[i][e]; x[e + 4] = sb[i][e]; }
            float pr[8];
            if (!GENERAL || !T[i].exact) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pr[e] = __builtin_amdgcn_exp2f(
                        fold ? x[e] : fmaf(x[e], GENERAL ? T[i].qscale * kin[e] : T[i].qscale, add[i][e]));
                if (MASK && partial) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = (bits[i] >> e) & 1u ? pr[e] : 0.0f;
                }
            } else {
                float xs[8], cm = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xs[e] = fold ? x[e] : fmaf(x[e], T[i].qscale * kin[e], add[i][e]);
                    if (MASK && partial) xs[e] = (bits[i] >> e) & 1u ? xs[e] : -INFINITY;
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
        for (int i = 0; i < NU; ++i) {
            T[i].o0 = mfma(v0, pb[i], T[i].o0);
            T[i].o1 = mfma(v1, pb[i], T[i].o1);
            T[i].ls = mfma(ones, pb[i], T[i].ls);
        }
        gw.next(SR, inv_SR);
    }
}

template <int SIM, int POS>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu((WAVES + 3) / 4)))
attn_large_kernel(AttnParams p, LargeLayout L)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1, SR = L.SR;

    // XCD-aware order: consecutive blockIdx land on different XCDs, so each
    // XCD takes a contiguous range of work ids; window-major, so the heads of
    // one window share that XCD's L2.
    const int work = (blockIdx.x & 7) * L.P + (blockIdx.x >> 3);
    if (work >= L.units) return;
    const int win = work / g.heads;
    const int h = work - win * g.heads;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4;
    const int li = lane & 15;

    unsigned char* kv = smem;                                             // [kv_bytes]
    float* bias2 = (float*)(smem + L.kv_bytes);                            // [S*S + 8]   (TABLE)
    float* rtab = bias2 + (POS == SWIN_POS_TABLE ? (S * S + 8 + 3) / 4 * 4 : 0);   // [M][2][8] cos, sin (ROPE2D)
    float* kinv = rtab + (POS == SWIN_POS_ROPE2D ? M * 32 : 0);           // [NSP]       (COSINE)
    float* red = kinv + (SIM == SWIN_SIM_COSINE ? L.NSP : 0);             // [4 * WAVES]

    const WinPlace wp = place_window(g, win);
    const uint32_t bytes = (uint32_t)(wp.span - h * D) * 2u;
    const int64_t off = wp.base + h * D;
    const Rsrc qr = make_rsrc((const uint16_t*)p.q + off, bytes);
    const Rsrc kr = make_rsrc((const uint16_t*)p.k + off, bytes);
    const Rsrc orr = make_rsrc((const uint16_t*)p.out + off, bytes);
    const RawRsrc vr = raw_rsrc((const uint16_t*)p.v + off, bytes);

    const float tau_eff = SIM == SWIN_SIM_COSINE ? fmaxf(p.tau[h], p.tau_min) : 1.0f;
    const float inv_tau = 1.0f / tau_eff;
    const bool precise = SIM == SWIN_SIM_COSINE && POS != SWIN_POS_ROPE2D && tau_eff < PRECISE_TAU;
    bool split = SIM == SWIN_SIM_COSINE && POS == SWIN_POS_ROPE2D && tau_eff < SPLIT_TAU;
    const bool needs_mask = wp.last_r || wp.last_c || SR != M || L.NSP != M * SR;

    // Rotate 8 channels (8 grp..8 grp+7) of a token at local (r, c): the
    // first half of the head dims turns with the row, the second with the
    // column; pairs (2k, 2k+1), angle pos * theta_k.
    auto rotate = [&](float* f, int r, int c) {
        const int half = grp >> 1, pos = half ? c : r;
        const float* cs = rtab + ((pos * 2 + half) * 8 + (grp & 1) * 4) * 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float co = cs[2 * e], si = cs[2 * e + 1];
            const float x0 = f[2 * e], x1 = f[2 * e + 1];
            f[2 * e] = x0 * co - x1 * si;
            f[2 * e + 1] = x0 * si + x1 * co;
        }
    };

    // ---- stage key slots [s0, s0 + 32 nch): V rows by LDS-DMA, K through
    // registers (rotated, normalised, rounded; remainders when split).
    // Wavefront w takes chunks w, w + 8, ...  Returns the largest squared
    // key norm this lane saw.
    u32x4 raw[KPW][2];
    int rr[KPW][2], cc[KPW][2];
    auto stage_issue = [&](const Block& bk, __bf16* vdst) {
#pragma unroll
        for (int j = 0; j < KPW; ++j) {
            const int cb = wave + WAVES * j;
            if (cb >= bk.nch) break;                      // wave-uniform
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2) {
                const int sl = 32 * cb + 16 * j2 + (lane >> 2);            // slot within the block
                const int s = bk.s0 + sl;
                const int rj = qdiv(s, L.inv_SR), cj = s - rj * SR;
                const uint32_t piece = (uint32_t)((lane & 3) ^ v_swizzle(sl));
                dma16(vr, vdst + (32 * cb + 16 * j2) * D, masked(wp.wg.tok(rj, cj) + 16u * piece, rj < M && cj < M));
            }
        }
        // every key load of the stage in flight before the first is used
#pragma unroll
        for (int j = 0; j < KPW; ++j) {
            const int cb = wave + WAVES * j;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int s = bk.s0 + 32 * cb + 8 * (li >> 2) + (li & 3) + 4 * t;
                rr[j][t] = qdiv(s, L.inv_SR);
                cc[j][t] = s - rr[j][t] * SR;
                const bool ok = cb < bk.nch && rr[j][t] < M && cc[j][t] < M;
                raw[j][t] = load16(kr, masked(wp.wg.tok(rr[j][t], cc[j][t]) + 16u * grp, ok));
            }
        }
    };
    auto stage_process = [&](const Block& bk, bf16x8* kdst, bf16x8* klodst, bool with_lo) -> float {
        float kmax2 = 0.0f;
#pragma unroll
        for (int j = 0; j < KPW; ++j) {
            const int cb = wave + WAVES * j;
            if (cb >= bk.nch) break;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                float kf[8];
                unpack_bf16x8(raw[j][t], kf);
                if (POS == SWIN_POS_ROPE2D) rotate(kf, min(rr[j][t], M - 1), min(cc[j][t], M - 1));
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(kf[e], kf[e], ss);
                ss += __shfl_xor(ss, 16);
                ss += __shfl_xor(ss, 32);
                kmax2 = fmaxf(kmax2, ss);
                const int idx = (cb * 2 + t) * 64 + lane;
                if (SIM == SWIN_SIM_COSINE) {
                    const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));   // 1 / max(||k||, 1e-12)
                    if (precise) {
                        if (grp == 0) kinv[bk.s0 + 32 * cb + 8 * (li >> 2) + (li & 3) + 4 * t] = inv;
                        kdst[idx] = __builtin_bit_cast(bf16x8, raw[j][t]);
                        continue;
                    }
                    const float ks = inv * (kLog2e * inv_tau);
#pragma unroll
                    for (int e = 0; e < 8; ++e) kf[e] *= ks;
                } else if (POS == SWIN_POS_ROPE2D) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) kf[e] *= kLog2e * 0.17677669529663687f;   // log2(e) / sqrt(32)
                }
                const bf16x8 hi = pack_bf16x8(kf);
                kdst[idx] = hi;
                if (with_lo) {
                    float lo[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) lo[e] = kf[e] - (float)hi[e];
                    klodst[idx] = pack_bf16x8(lo);
                }
            }
        }
        return kmax2;
    };

    // ---- keys and values, all slots in one block unless split
    const int nch_all = L.NSP / 32;
    Block whole;
    whole.k = (const bf16x8*)kv;
    whole.klo = nullptr;
    whole.v = (const __bf16*)(kv + L.NSP * 64);
    whole.s0 = 0;
    whole.nch = nch_all;
    auto load_pair_q = [&](int r, u32x4 (&qr2)[NT]) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int t = (wave + WAVES * (NT * r + i)) * 16 + li;
            const bool ok = t < N;
            const int tc = ok ? t : 0;
            const int ri = qdiv(tc, L.inv_M), ci = tc - ri * M;
            qr2[i] = load16(qr, masked(wp.wg.tok(ri, ci) + 16u * grp, ok));
        }
    };
    float kmax = 0.0f;
    // ---- every load of the staging in flight first: keys (registers),
    // values (LDS-DMA), the queries of the DOT + rotation norm test and the
    // first pair of query tiles; the tables are set up meanwhile
    if (!split) stage_issue(whole, (__bf16*)(kv + L.NSP * 64));
    u32x4 qraw[SIM == SWIN_SIM_DOT && POS == SWIN_POS_ROPE2D ? QPW : 1];
    if (SIM == SWIN_SIM_DOT && POS == SWIN_POS_ROPE2D) {             // (split is only set below for DOT)
#pragma unroll
        for (int j = 0; j < QPW; ++j) {
            const int t = (wave + WAVES * j) * 16 + li;
            const bool ok = t < N;
            const int tc = ok ? t : 0;
            const int ri = qdiv(tc, L.inv_M), ci = tc - ri * M;
            qraw[j] = load16(qr, masked(wp.wg.tok(ri, ci) + 16u * grp, ok));
        }
    }
    // DOT with rotation keeps those query rows for the tiles (a second read
    // of Q would come partly from HBM again: the window's K, V and Q pass
    // the L2 between the norm test and the last pair); others load a pair
    // ahead
    constexpr bool QKEEP = SIM == SWIN_SIM_DOT && POS == SWIN_POS_ROPE2D;
    u32x4 qnext[NT];
    if (!QKEEP) load_pair_q(0, qnext);
    // ---- tables: bias (reversed so that consecutive keys read consecutive
    // floats, in log2 units, shifted by its max and, for COSINE, by 1/tau);
    // rotary cos / sin per local position, half and pair
    float bias_range = 0.0f, tab_shift = 0.0f;   // tab_shift: subtracted from the stored table (log2 units)
    if (POS == SWIN_POS_TABLE) {
        float mx = -INFINITY, mn = INFINITY;
        for (int i = tid; i < S * S; i += NTHR) {
            const float v = p.table[(size_t)(S * S - 1 - i) * g.heads + h] * kLog2e;
            bias2[i] = v;
            mx = fmaxf(mx, v);
            mn = fminf(mn, v);
        }
        if (tid < 8) bias2[S * S + tid] = -INFINITY;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            mx = fmaxf(mx, __shfl_xor(mx, o));
            mn = fminf(mn, __shfl_xor(mn, o));
        }
        if (lane == 0) { red[wave] = mx; red[WAVES + wave] = mn; }
        __syncthreads();
        mx = red[0]; mn = red[WAVES];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) { mx = fmaxf(mx, red[w]); mn = fminf(mn, red[WAVES + w]); }
        bias_range = mx - mn;
        const float sh = SIM == SWIN_SIM_COSINE ? mx + kLog2e * inv_tau : mx;
        for (int i = tid; i < S * S; i += NTHR) bias2[i] -= sh;
        tab_shift = sh;
    }
    if (POS == SWIN_POS_ROPE2D) {
        for (int i = tid; i < M * 16; i += NTHR) {
            const int k = i & 7, half = (i >> 3) & 1, pos = i >> 4;
            // fp32 is ample: the rotated operands are rounded to bf16
            const float th = p.rope_freqs ? p.rope_freqs[((size_t)h * 2 + half) * 8 + k]
                                          : exp2f(-(float)k * 0.125f * log2f(p.rope_base));
            float s_, c_;
            sincosf((float)pos * th, &s_, &c_);
            rtab[i * 2] = c_;
            rtab[i * 2 + 1] = s_;
        }
    }
    __syncthreads();

    if (!split) {
        float k2 = stage_process(whole, (bf16x8*)kv, nullptr, false);
        // DOT: the window's largest key norm (Cauchy-Schwarz shift, split test)
        if (SIM == SWIN_SIM_DOT) {
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) k2 = fmaxf(k2, __shfl_xor(k2, o));
            if (lane == 0) red[2 * WAVES + wave] = k2;
        }
        // DOT with rotation: the largest query norm too, from this wave's tiles
        if (SIM == SWIN_SIM_DOT && POS == SWIN_POS_ROPE2D) {
            float q2 = 0.0f;
#pragma unroll
            for (int j = 0; j < QPW; ++j) {
                float qv[8];
                unpack_bf16x8(qraw[j], qv);
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(qv[e], qv[e], ss);
                ss += __shfl_xor(ss, 16);
                ss += __shfl_xor(ss, 32);
                q2 = fmaxf(q2, ss);
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) q2 = fmaxf(q2, __shfl_xor(q2, o));
            if (lane == 0) red[3 * WAVES + wave] = q2;
        }
        vm_wait_all();
        __syncthreads();
        if (SIM == SWIN_SIM_DOT) {
            float k2m = red[2 * WAVES], q2m = red[3 * WAVES];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) {
                k2m = fmaxf(k2m, red[2 * WAVES + w]);
                if (POS == SWIN_POS_ROPE2D) q2m = fmaxf(q2m, red[3 * WAVES + w]);
            }
            kmax = sqrtf(k2m);
            if (POS == SWIN_POS_ROPE2D) split = kmax * sqrtf(q2m) * (kLog2e * 0.17677669529663687f) > SPLIT_BOUND;
        }
    } else if (SIM == SWIN_SIM_DOT) {
        kmax = 0.0f;                                      // (COSINE only reaches here)
    }
    // split: keys in two halves with their remainders, staged per cycle of
    // two tile pairs (below)
    const int half_ch = (nch_all + 1) / 2;

    // ---- this wavefront's query tiles, two at a time; the next pair's
    // queries load while the current pair runs
    const int qhalf = POS == SWIN_POS_ROPE2D ? 1 : 0;
    // groups split by a region edge or by padded columns need per-key masks
    const bool partial = (wp.last_c && ((M - g.shift) & 7)) || (M & 7);
    const bool partial_s = __builtin_amdgcn_readfirstlane((int)partial) != 0;   // uniform
    // One pair's tile state: the queries' rows (rotated, normalised, rounded),
    // scales, masks and accumulators; rlo_min / rhi_max: the key rows some
    // query of the pair may see (wave-uniform).
    struct Pair {
        Tile T[NT];
        int qt[NT];
        bool qv[NT];
        bool any_exact, live, two;
        int rlo_min, rhi_max;
    };
    auto setup = [&](int r, Pair& P) {
        Tile (&T)[NT] = P.T;
        int (&qt)[NT] = P.qt;
        bool (&qv)[NT] = P.qv;
        u32x4 qcur[NT];
        if (QKEEP) {
            // this round's rows are qraw[0..NT); the rest move down a pair
#pragma unroll
            for (int i = 0; i < NT; ++i) qcur[i] = qraw[i];
#pragma unroll
            for (int j = 0; j + NT < QPW; ++j) qraw[j] = qraw[j + NT];
        } else {
#pragma unroll
            for (int i = 0; i < NT; ++i) qcur[i] = qnext[i];
            if (r + 1 < L.rounds) load_pair_q(r + 1, qnext);
        }
        bool any_exact = false;
        int rlo_min = M, rhi_max = 0;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int t = (wave + WAVES * (NT * r + i)) * 16 + li;
            qv[i] = t < N;
            qt[i] = qv[i] ? t : 0;
            const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
            const u32x4 raw = qcur[i];
            float qf[8];
            unpack_bf16x8(raw, qf);
            if (POS == SWIN_POS_ROPE2D) rotate(qf, ri, ci);
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(qf[e], qf[e], ss);
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            const float qinv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));   // 1 / max(||q||, 1e-12)
            if (SIM == SWIN_SIM_COSINE && !precise) {
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[e] *= qinv;
            }
            T[i].qf = qhalf || (SIM == SWIN_SIM_COSINE && !precise) ? pack_bf16x8(qf) : __builtin_bit_cast(bf16x8, raw);
            {
                float lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) lo[e] = qf[e] - (float)T[i].qf[e];
                T[i].qf_lo = pack_bf16x8(lo);
            }
            float spread;
            if (SIM == SWIN_SIM_COSINE) {
                T[i].qscale = kLog2e * inv_tau * qinv;
                T[i].negm = POS == SWIN_POS_TABLE ? 0.0f : -kLog2e * inv_tau;
                spread = 2.0f * kLog2e * inv_tau + bias_range;
            } else {
                T[i].qscale = kLog2e * 0.17677669529663687f;          // log2(e) / sqrt(32)
                const float c_i = sqrtf(ss) * kmax * T[i].qscale;
                T[i].negm = -c_i;
                spread = 2.0f * c_i + bias_range;
            }
            // DOT with a split: kmax is not known (COSINE only splits), so
            // the running maximum is used
            T[i].exact = __any(!(spread <= RANGE_LIMIT)) != 0 || (SIM == SWIN_SIM_DOT && split);
            any_exact = any_exact || T[i].exact;
            T[i].mrun = -INFINITY;
            T[i].qoff = (M - 1 - ri) * S + (M - 1 - ci);
            T[i].rlo = 0; T[i].rhi = M;
            int clo = 0, chi = M;
            if (wp.last_r) { if (ri < M - g.shift) T[i].rhi = M - g.shift; else T[i].rlo = M - g.shift; }
            if (wp.last_c) { if (ci < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
            T[i].cmask = (chi >= 32 ? 0xffffffffu : ((1u << chi) - 1u)) & ~((1u << clo) - 1u);
            if (qv[i]) { rlo_min = min(rlo_min, T[i].rlo); rhi_max = max(rhi_max, T[i].rhi); }
            T[i].o0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            T[i].o1 = T[i].o0;
            T[i].ls = T[i].o0;
        }
        // key rows some query of the pair may see (wave-uniform)
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            rlo_min = min(rlo_min, __shfl_xor(rlo_min, o));
            rhi_max = max(rhi_max, __shfl_xor(rhi_max, o));
        }
        rlo_min = __builtin_amdgcn_readfirstlane(rlo_min);
        rhi_max = __builtin_amdgcn_readfirstlane(rhi_max);
        P.live = rhi_max > rlo_min;                       // some tile of the pair has queries
        // whether the pair's second tile holds queries (wave-uniform)
        P.two = NT == 2 && (wave + WAVES * (NT * r + 1)) * 16 < N;
        P.any_exact = any_exact;
        P.rlo_min = rlo_min;
        P.rhi_max = rhi_max;

    };
    // the pair against the chunks of block bk its queries can see
    auto run = [&](Pair& P, const Block& bk) {
        if (!P.live) return;
        const int s_lo = P.rlo_min * SR - bk.s0, s_hi = P.rhi_max * SR - bk.s0;
        const int cb = max(0, s_lo) >> 5;
        const int ce = min(bk.nch, (max(0, s_hi) + 31) >> 5);
        if (cb >= ce) return;
        if (P.any_exact || precise || split)
            run_pair<SIM, POS, true, true, NT>(bk, P.T, bias2, kinv, S, SR, L.inv_SR, cb, ce, lane, partial,
                                               precise, split);
        else if (!P.two) {
            // the wavefront's last tile is alone: run it by itself
            if (needs_mask && partial_s)
                run_pair<SIM, POS, true, false, 1>(bk, P.T, bias2, kinv, S, SR, L.inv_SR, cb, ce, lane, true,
                                                   false, false);
            else if (needs_mask)
                run_pair<SIM, POS, true, false, 1>(bk, P.T, bias2, kinv, S, SR, L.inv_SR, cb, ce, lane, false,
                                                   false, false);
            else
                run_pair<SIM, POS, false, false, 1>(bk, P.T, bias2, kinv, S, SR, L.inv_SR, cb, ce, lane, false,
                                                    false, false);
        } else if (needs_mask && partial_s)
            run_pair<SIM, POS, true, false, NT>(bk, P.T, bias2, kinv, S, SR, L.inv_SR, cb, ce, lane, true, false,
                                                false);
        else if (needs_mask)
            // region edges on 8-slot group boundaries: a loop without
            // per-key selects
            run_pair<SIM, POS, true, false, NT>(bk, P.T, bias2, kinv, S, SR, L.inv_SR, cb, ce, lane, false, false,
                                                false);
        else
            run_pair<SIM, POS, false, false, NT>(bk, P.T, bias2, kinv, S, SR, L.inv_SR, cb, ce, lane, false, false,
                                                 false);
    };
    auto store = [&](Pair& P) {
        Tile (&T)[NT] = P.T;
        int (&qt)[NT] = P.qt;
        bool (&qv)[NT] = P.qv;
        // ---- normalise and store: lane holds channels 4 grp..+3 and
        // 16 + 4 grp..+3 of query li
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
            const float inv = __builtin_amdgcn_rcpf(T[i].ls[0]);
            const uint32_t o = masked(wp.wg.tok(ri, ci) + 8u * grp, qv[i]);
            store8(orr, o, pack_bf16x4(T[i].o0[0] * inv, T[i].o0[1] * inv, T[i].o0[2] * inv, T[i].o0[3] * inv));
            store8(orr, o + 32u, pack_bf16x4(T[i].o1[0] * inv, T[i].o1[1] * inv, T[i].o1[2] * inv, T[i].o1[3] * inv));
            if (p.lse && grp == 0 && qv[i]) {
                // the exp2 arguments were the logits in log2 units less the
                // table's shift and -negm, plus the running maximum where used
                const float off2 = tab_shift - T[i].negm + (T[i].exact ? T[i].mrun : 0.0f);
                p.lse[((size_t)win * g.heads + h) * N + qt[i]] = (__builtin_amdgcn_logf(T[i].ls[0]) + off2) * kLn2;
            }
        }
    };

    if (!split) {
        for (int r = 0; r < L.rounds; ++r) {
            Pair P;
            setup(r, P);
            run(P, whole);
            store(P);
        }
    } else {
        // two pairs per staging cycle: cycle c runs pairs 2c and 2c + 1 over
        // the halves in the order 0, 1 (c even) or 1, 0 (c odd), so its
        // first half is still in LDS from cycle c - 1 (the online normaliser
        // does not depend on the order of the keys)
        for (int r = 0; r < L.rounds; r += 2) {
            const bool second = r + 1 < L.rounds;
            Pair P0, P1;
            setup(r, P0);
            if (second) setup(r + 1, P1);
            for (int bi = 0; bi < 2; ++bi) {
                const int b = ((r >> 1) & 1) ? 1 - bi : bi;
                Block bk = whole;
                bk.nch = b == 0 ? half_ch : nch_all - half_ch;
                bk.s0 = b * half_ch * 32;
                bk.k = (const bf16x8*)kv;
                bk.klo = (const bf16x8*)(kv + half_ch * 32 * 64);
                bk.v = (const __bf16*)(kv + 2 * half_ch * 32 * 64);
                if (r == 0 || bi == 1) {
                    // stage this half (every wave takes part), with remainders
                    __syncthreads();                      // the previous half is consumed
                    stage_issue(bk, (__bf16*)(kv + 2 * half_ch * 32 * 64));
                    stage_process(bk, (bf16x8*)kv, (bf16x8*)(kv + half_ch * 32 * 64), true);
                    vm_wait_all();
                    __syncthreads();
                }
                run(P0, bk);
                if (second) run(P1, bk);
            }
            store(P0);
            if (second) store(P1);
        }
    }
}

template <int SIM, int POS>
hipError_t launch_large(const AttnParams& p, const LargeLayout& L, size_t lds, hipStream_t s)
{
    auto* fn = attn_large_kernel<SIM, POS>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<8 * L.P, NTHR, lds, s>>>(p, L);
    return hipGetLastError();
}

size_t large_lds(const Geometry& g, int sim, int pos, LargeLayout* out)
{
    LargeLayout L;
    L.SR = (g.M + 7) / 8 * 8;
    L.GPR = L.SR / 8;
    L.NSP = (g.M * L.SR + 31) / 32 * 32;
    L.NQT = (g.N + 15) / 16;
    const int tpw = (L.NQT + WAVES - 1) / WAVES;
    L.rounds = (tpw + NT - 1) / NT;
    L.units = g.nwin * g.heads;
    L.P = (L.units + 7) / 8;
    const int nch = L.NSP / 32, half = (nch + 1) / 2;
    L.kv_bytes = max(L.NSP * 128, 3 * half * 32 * 64);
    L.inv_M = 1.0f / (float)g.M;
    L.inv_SR = 1.0f / (float)L.SR;
    L.inv_GPR = 1.0f / (float)L.GPR;
    const int S = 2 * g.M - 1;
    size_t lds = (size_t)L.kv_bytes;
    if (pos == SWIN_POS_TABLE) lds += (size_t)((S * S + 8 + 3) / 4 * 4) * sizeof(float);
    if (pos == SWIN_POS_ROPE2D) lds += (size_t)g.M * 32 * sizeof(float);
    if (sim == SWIN_SIM_COSINE) lds += (size_t)L.NSP * sizeof(float);
    lds += 4 * WAVES * sizeof(float);
    if (out) *out = L;
    return lds;
}

}  // namespace

bool attn_large_supported(const AttnParams& p)
{
    const Geometry& g = p.g;
    if (p.dtype != SWIN_DT_BF16 || g.d != D || g.M > 32) return false;
    if (!(g.M > 16 || p.pos == SWIN_POS_ROPE2D)) return false;
    if ((int64_t)g.H * g.W * g.C * 2 >= ((int64_t)1 << 31)) return false;   // 32-bit byte offsets
    if ((int64_t)g.W * g.C * 2 >= ((int64_t)1 << 24)) return false;          // 24-bit row stride
    if ((int64_t)g.nwin * g.heads > INT32_MAX - 8) return false;
    return large_lds(g, p.sim, p.pos, nullptr) <= 160 * 1024;
}

hipError_t launch_attn_large(const AttnParams& p, hipStream_t stream)
{
    const Geometry& g = p.g;
    if (g.nwin == 0) return hipSuccess;
    LargeLayout L;
    const size_t lds = large_lds(g, p.sim, p.pos, &L);
    if (p.sim == SWIN_SIM_COSINE) {
        switch (p.pos) {
        case SWIN_POS_NONE: return launch_large<SWIN_SIM_COSINE, SWIN_POS_NONE>(p, L, lds, stream);
        case SWIN_POS_TABLE: return launch_large<SWIN_SIM_COSINE, SWIN_POS_TABLE>(p, L, lds, stream);
        default: return launch_large<SWIN_SIM_COSINE, SWIN_POS_ROPE2D>(p, L, lds, stream);
        }
    }
    switch (p.pos) {
    case SWIN_POS_NONE: return launch_large<SWIN_SIM_DOT, SWIN_POS_NONE>(p, L, lds, stream);
    case SWIN_POS_TABLE: return launch_large<SWIN_SIM_DOT, SWIN_POS_TABLE>(p, L, lds, stream);
    default: return launch_large<SWIN_SIM_DOT, SWIN_POS_ROPE2D>(p, L, lds, stream);
    }
}

}  // namespace swin
