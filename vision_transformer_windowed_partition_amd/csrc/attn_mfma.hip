// Fused window attention on the gfx950 matrix cores (bf16 in, fp32
// accumulate, bf16 out), d = 32.
//
// What it computes is the window attention of the SwinV2 card (eq. 1-2, the
// window-attention pseudocode), with the log-CPB bias table (eq. 3-4), the
// rotary variant and exact, never-materialised softmax of the FlashSwin
// abstract, over cyclic-shift or interleaved (Iwin) windows.
//
// Work decomposition.  A workgroup owns one (window, head, block of up to 8
// query tiles of 16 queries); each wavefront owns NQ <= 2 query tiles.  The
// window-head's keys are staged through LDS in blocks of KB key slots,
// written there directly in the register layout of the MFMA operands:
//   K^  (keys x d)  as the A operand of  S^T = K^ Q^T   (v_mfma_f32_16x16x32_bf16)
//   V^T (d x keys)  as the A operand of  O^T = V^T P^T
// so that every operand read is one linear ds_read_b128 per lane.  Q is read
// straight from HBM as the B operand (16 contiguous bytes per lane).  The
// score tile S^T leaves the MFMA with each lane holding 8 consecutive key
// slots of one query, exactly the B-operand layout P^T needs: the softmax
// runs in registers and feeds the second product without any shuffle.  The
// row sums come from a third MFMA against an all-ones A operand, which keeps
// them off the vector ALU.  Per 32-key chunk a wavefront issues the score
// products of all its tiles, then their exponentials, then the value
// products, with no branch in between, so the matrix core, the LDS and the
// vector ALU overlap.
//
// Key slots.  Key (rj, cj) of the window sits in slot rj*SR + cj with SR = M
// rounded up to 8, so a lane's 8 slots share one key row; slots are padded to
// a multiple of 32.  Padded slots and keys of another shift region are
// masked per 8-slot group: a chunk masked for every lane is skipped, a group
// masked for one lane reads its bias from a row of -inf, and only groups
// split by a region edge pay a per-element select.
//
// Softmax normaliser.  Softmax is invariant to a per-row shift, so any c_i
// with c_i >= max_j logit_ij can replace the row max when no term can
// underflow.  COSINE: |cos| <= 1, so c_h = 1/tau_h + max bias (per head).
// DOT: Cauchy-Schwarz, c_i = ||q_i|| max_j ||k_j|| / sqrt(d) + max bias.
// When the spread 2 * (c_i - bias part) + bias range stays below 60 in base
// 2, every kept weight is at least 2^-60 of the largest and this static shift
// is exact; then each score costs one FMA and one exp2.  Otherwise the tile
// takes the online normaliser (running max per 32-key chunk, rescaling the
// accumulators), which has no range condition.
#include "common.hpp"
#include "launch.hpp"

namespace swin {

namespace {

constexpr int D = 32;
constexpr int QT_MAX = 2;      // query tiles per wavefront (register budget: 3 waves per SIMD)
constexpr int MAX_WAVES = 4;
constexpr int KB = 256;        // key slots staged per block
constexpr int SB = 4;          // staging loads in flight per thread and tensor
constexpr int TB = 8;          // bias-table loads in flight per thread
constexpr float RANGE_LIMIT = 60.0f;
// Precision split: with bf16 operands a rounded unit vector k^ (or a rotated
// q, k) errs by up to 2^-9 of its norm, and the logit multiplies that error
// by 1/tau (COSINE) or by ||q|| ||k|| / sqrt(d) (DOT after rotation).  Past
// these amplifications the rounded operand is carried as hi + lo, two bf16
// terms, and the score takes one more MFMA per extra product.
constexpr float SPLIT_TAU = 0.1f;      // COSINE: split when tau < 0.1
constexpr float SPLIT_BOUND = 20.0f;   // DOT + ROPE2D: split when max ||q|| ||k|| log2(e)/sqrt(d) > 20

struct Layout {                // derived sizes, identical for every workgroup
    int SR;                    // slots per key row (M rounded up to 8)
    int NSP;                   // key slots, padded to 32
    int GPR;                   // 8-slot groups per key row
    int NQT;                   // query tiles per window-head
    int nqb;                   // query blocks per window-head
    int nblk;                  // key blocks per window-head (unsplit)
    int total;                 // workgroups with work
    int P;                     // workgroups per XCD slot
};

// Per-wavefront query-tile state.
template <int NQ>
struct Tiles {
    bf16x8 qf[NQ], qf_lo[NQ];
    float qscale[NQ], negm[NQ], mrun[NQ];
    int qoff[NQ], rlo[NQ], rhi[NQ];
    uint64_t cmask[NQ];
    bool exact[NQ];
    f32x4 o0[NQ], o1[NQ], ls[NQ];
};

struct Stage {                 // LDS views of one staged key block
    const bf16x8* kfrag;
    const bf16x8* kfrag_lo;
    const bf16x8* vfrag;
    const float* bias2;
    int S;                     // 2M - 1
    int negrow;                // index of the -inf row of bias2
};

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ones8()
{
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)1.0f;
    return o;
}

// 8-slot group bookkeeping: the lane's group in chunk c of a block starting
// at slot s0 is s0/8 + 4c + grp; groups run along key rows of SR slots.
struct GroupWalk {
    int rj, c0, drow, dcol, SR;
    __device__ __forceinline__ GroupWalk(int s0, int grp, int GPR, int SR_) : SR(SR_)
    {
        const int gam = (s0 >> 3) + grp;
        rj = gam / GPR;
        c0 = (gam - rj * GPR) * 8;
        drow = 4 / GPR;
        dcol = (4 - drow * GPR) * 8;
    }
    __device__ __forceinline__ void next()
    {
        c0 += dcol;
        rj += drow;
        if (c0 >= SR) { c0 -= SR; ++rj; }
    }
};

template <int NQ>
__device__ __forceinline__ uint32_t group_bits(const Tiles<NQ>& T, int qi, int rj, int c0)
{
    const bool rok = rj >= T.rlo[qi] && rj < T.rhi[qi];
    return rok ? (uint32_t)(T.cmask[qi] >> c0) & 0xffu : 0u;
}

// Fast chunk loop: static shift, one bf16 product per score, no split.
template <int SIM, int POS, int NQ, bool MASK>
__device__ __forceinline__ void run_fast(const Stage& st, Tiles<NQ>& T, int s0, int cnt,
                                         int lane, int grp, int GPR, int SR)
{
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    const bf16x8 ones = ones8();
    GroupWalk gw(s0, grp, GPR, SR);
    const int nch = cnt >> 5;
    for (int c = 0; c < nch; ++c, gw.next()) {
        uint32_t bits[NQ];
        if (MASK) {
            uint32_t anyb = 0;
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                bits[qi] = group_bits(T, qi, gw.rj, gw.c0);
                anyb |= bits[qi];
            }
            if (!__any(anyb != 0u)) continue;                  // chunk masked for the whole wave
        }
        const bf16x8 ka = st.kfrag[(c * 2 + 0) * 64 + lane];
        const bf16x8 kb = st.kfrag[(c * 2 + 1) * 64 + lane];
        const bf16x8 va = st.vfrag[(c * 2 + 0) * 64 + lane];
        const bf16x8 vb = st.vfrag[(c * 2 + 1) * 64 + lane];
        const int koff = gw.rj * st.S + gw.c0;

        float add[NQ][8];
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            if (POS == SWIN_POS_TABLE) {
                const float* bp = st.bias2 + ((MASK && bits[qi] == 0u) ? st.negrow : koff + T.qoff[qi]);
#pragma unroll
                for (int e = 0; e < 8; ++e) add[qi][e] = SIM == SWIN_SIM_COSINE ? bp[e] : bp[e] + T.negm[qi];
            } else {
                const float a = (MASK && bits[qi] == 0u) ? -INFINITY : T.negm[qi];
#pragma unroll
                for (int e = 0; e < 8; ++e) add[qi][e] = a;
            }
        }
        f32x4 sa[NQ], sb[NQ];
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            sa[qi] = mfma(ka, T.qf[qi], zero4);
            sb[qi] = mfma(kb, T.qf[qi], zero4);
        }
        bool part = false;
        if (MASK) {
            uint32_t pp = 0;
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) pp |= (bits[qi] != 0u && bits[qi] != 0xffu);
            part = __any(pp != 0u);
        }
        bf16x8 pb[NQ];
        if (!part) {
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                float pr[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pr[e] = __builtin_amdgcn_exp2f(fmaf(sa[qi][e], T.qscale[qi], add[qi][e]));
                    pr[e + 4] = __builtin_amdgcn_exp2f(fmaf(sb[qi][e], T.qscale[qi], add[qi][e + 4]));
                }
                pb[qi] = pack_bf16x8(pr);
            }
        } else {
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                float pr[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pr[e] = __builtin_amdgcn_exp2f(fmaf(sa[qi][e], T.qscale[qi], add[qi][e]));
                    pr[e + 4] = __builtin_amdgcn_exp2f(fmaf(sb[qi][e], T.qscale[qi], add[qi][e + 4]));
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = (bits[qi] >> e) & 1u ? pr[e] : 0.0f;
                pb[qi] = pack_bf16x8(pr);
            }
        }
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            T.o0[qi] = mfma(va, pb[qi], T.o0[qi]);
            T.o1[qi] = mfma(vb, pb[qi], T.o1[qi]);
            T.ls[qi] = mfma(ones, pb[qi], T.ls[qi]);
        }
    }
}

// General chunk loop: any mask, hi + lo operands, and per tile either the
// static shift or the online normaliser.
template <int SIM, int POS, int NQ>
__device__ __forceinline__ void run_general(const Stage& st, Tiles<NQ>& T, int s0, int cnt,
                                            int lane, int grp, int GPR, int SR, bool needs_mask,
                                            bool split_k, bool split_q)
{
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    const bf16x8 ones = ones8();
    GroupWalk gw(s0, grp, GPR, SR);
    const int nch = cnt >> 5;
    for (int c = 0; c < nch; ++c, gw.next()) {
        const bf16x8 ka = st.kfrag[(c * 2 + 0) * 64 + lane];
        const bf16x8 kb = st.kfrag[(c * 2 + 1) * 64 + lane];
        bf16x8 ka_lo = ka, kb_lo = kb;
        if (split_k) {
            ka_lo = st.kfrag_lo[(c * 2 + 0) * 64 + lane];
            kb_lo = st.kfrag_lo[(c * 2 + 1) * 64 + lane];
        }
        const bf16x8 va = st.vfrag[(c * 2 + 0) * 64 + lane];
        const bf16x8 vb = st.vfrag[(c * 2 + 1) * 64 + lane];
        const int koff = gw.rj * st.S + gw.c0;
#pragma unroll
        for (int qi = 0; qi < NQ; ++qi) {
            uint32_t bits = 0xffu;
            if (needs_mask) {
                bits = group_bits(T, qi, gw.rj, gw.c0);
                if (!__any(bits != 0u)) continue;
            }
            f32x4 sa = mfma(ka, T.qf[qi], zero4);
            f32x4 sb = mfma(kb, T.qf[qi], zero4);
            if (split_k) {
                sa = mfma(ka_lo, T.qf[qi], sa);
                sb = mfma(kb_lo, T.qf[qi], sb);
            }
            if (split_q) {                                // lo lo (< 2^-18 |q||k|) is left out
                sa = mfma(ka, T.qf_lo[qi], sa);
                sb = mfma(kb, T.qf_lo[qi], sb);
            }
            const float x[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
            float add[8];
            if (POS == SWIN_POS_TABLE) {
                const float* bp = st.bias2 + (bits == 0u ? st.negrow : koff + T.qoff[qi]);
#pragma unroll
                for (int e = 0; e < 8; ++e) add[e] = SIM == SWIN_SIM_COSINE ? bp[e] : bp[e] + T.negm[qi];
            } else {
                const float a = bits == 0u ? -INFINITY : T.negm[qi];
#pragma unroll
                for (int e = 0; e < 8; ++e) add[e] = a;
            }
            const bool partial = needs_mask && __any(bits != 0u && bits != 0xffu);
            float pr[8];
            if (!T.exact[qi]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(x[e], T.qscale[qi], add[e]));
                if (partial) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = (bits >> e) & 1u ? pr[e] : 0.0f;
                }
            } else {
                float xs[8];
                float cm = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xs[e] = fmaf(x[e], T.qscale[qi], add[e]);
                    if (partial) xs[e] = (bits >> e) & 1u ? xs[e] : -INFINITY;
                    cm = fmaxf(cm, xs[e]);
                }
                cm = fmaxf(cm, __shfl_xor(cm, 16));
                cm = fmaxf(cm, __shfl_xor(cm, 32));
                const float mnew = fmaxf(T.mrun[qi], cm);
                const float mref = mnew == -INFINITY ? 0.0f : mnew;
                const float alpha = __builtin_amdgcn_exp2f(T.mrun[qi] - mref);
                T.o0[qi] *= alpha; T.o1[qi] *= alpha; T.ls[qi] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(xs[e] - mref);
                T.mrun[qi] = mnew;
            }
            const bf16x8 pb = pack_bf16x8(pr);
            T.o0[qi] = mfma(va, pb, T.o0[qi]);
            T.o1[qi] = mfma(vb, pb, T.o1[qi]);
            T.ls[qi] = mfma(ones, pb, T.ls[qi]);
        }
    }
}

template <int SIM, int POS, int NQ>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
attn_mfma_kernel(AttnParams p, Layout L)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1;

    // XCD-aware order: consecutive blockIdx land on different XCDs, so give
    // each XCD a contiguous range of work ids; the heads and query blocks of
    // one window then share that XCD's L2.
    const int work = (blockIdx.x & 7) * L.P + (blockIdx.x >> 3);
    if (work >= L.total) return;
    const int qb = work % L.nqb;
    const int wh = work / L.nqb;
    const int h = wh % g.heads;
    const int win = wh / g.heads;

    const int tid = threadIdx.x;
    const int nthr = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = nthr >> 6;
    const int grp = lane >> 4;       // 16-lane group: k-range of the operands
    const int li = lane & 15;        // row / column inside a 16 x 16 tile

    bf16x8* kfrag = (bf16x8*)smem;                       // [KB/32][2][64]
    bf16x8* vfrag = kfrag + KB * 4;                      // [KB/32][2][64]
    float* red = (float*)(vfrag + KB * 4);               // [16] reductions
    float* bias2 = red + 16;                             // [S*S + 8]   (TABLE)
    float* rcs = bias2 + (POS == SWIN_POS_TABLE ? S * S + 8 : 0);   // [M][2][8] (ROPE2D)
    float* rsn = rcs + (POS == SWIN_POS_ROPE2D ? M * 16 : 0);

    const uint16_t* qg = (const uint16_t*)p.q;
    const uint16_t* kg = (const uint16_t*)p.k;
    const uint16_t* vg = (const uint16_t*)p.v;
    uint16_t* og = (uint16_t*)p.out;

    const int nW = g.nwr * g.nwc;
    const int wloc = win % nW;
    const int wr = wloc / g.nwc, wc = wloc % g.nwc;
    const bool shifted = g.part == SWIN_PART_CYCLIC && g.shift > 0 &&
                         (wr == g.nwr - 1 || wc == g.nwc - 1);
    const bool needs_mask = shifted || L.SR != M || L.NSP != M * L.SR;
    const float tau_eff = SIM == SWIN_SIM_COSINE ? fmaxf(p.tau[h], p.tau_min) : 1.0f;

    // ---- this wavefront's query tiles
    const int qt0 = qb * L.NQT / L.nqb, qt1 = (qb + 1) * L.NQT / L.nqb;
    const int my0 = qt0 + wave * NQ;
    const int nq = max(0, min(NQ, qt1 - my0));            // wave-uniform

    // Every global load of the set-up is issued before its first use, so a
    // workgroup waits for one memory round trip, not one per item.
    // (1) this wave's query fragments (tiles past its share, or past N,
    //     read token 0 and are zeroed later; they are never stored)
    u32x4 qraw[NQ];
    int qri[NQ], qci[NQ];
    bool qvalid[NQ];
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        const int t = (my0 + qi) * 16 + li;
        qvalid[qi] = qi < nq && t < N;
        const int tc = qvalid[qi] ? t : 0;
        qri[qi] = tc / M;
        qci[qi] = tc - qri[qi] * M;
        qraw[qi] = *(const u32x4*)(qg + token_offset(g, win, qri[qi], qci[qi]) + h * D + grp * 8);
    }

    // (2) key/value staging, SB items of 16 bytes per thread per batch
    u32x4 kraw[SB], vraw[SB];
    auto kv_load = [&](int s0, int cnt, int b0) {
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int it = b0 + j * nthr + tid;
            kraw[j] = u32x4{0u, 0u, 0u, 0u};
            vraw[j] = kraw[j];
            if (it < cnt * 4) {
                const int s = s0 + (it >> 2), piece = it & 3;
                const int rj = s / L.SR, cj = s - rj * L.SR;
                if (rj < M && cj < M) {
                    const int64_t off = token_offset(g, win, rj, cj) + h * D + piece * 8;
                    kraw[j] = *(const u32x4*)(kg + off);
                    vraw[j] = *(const u32x4*)(vg + off);
                }
            }
        }
    };
    // turn the loaded batch into MFMA fragments: k rotated (ROPE2D), unit
    // normalised (COSINE), rounded to bf16 (and its remainder when split);
    // v scattered transposed.
    auto kv_store = [&](int s0, int cnt, int b0, bool split_k, bool track_kmax) {
        bf16x8* kfrag_lo = kfrag + (KB / 2) * 4;
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int it = b0 + j * nthr + tid;
            if (it >= cnt * 4) continue;                   // whole wavefronts drop out
            const int sl = it >> 2, piece = it & 3;
            const int s = s0 + sl;
            const int rj = s / L.SR, cj = s - rj * L.SR;
            float kf[8], vf[8];
            unpack_bf16x8(kraw[j], kf);
            unpack_bf16x8(vraw[j], vf);
            if (POS == SWIN_POS_ROPE2D && rj < M && cj < M) {
                const int half = piece >> 1, pos = half ? cj : rj;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = (piece & 1) * 4 + e;
                    const float co = rcs[(pos * 2 + half) * 8 + k], si = rsn[(pos * 2 + half) * 8 + k];
                    const float x0 = kf[2 * e], x1 = kf[2 * e + 1];
                    kf[2 * e] = x0 * co - x1 * si;
                    kf[2 * e + 1] = x0 * si + x1 * co;
                }
            }
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(kf[e], kf[e], ss);
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            if (SIM == SWIN_SIM_COSINE) {
                const float inv = 1.0f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
                for (int e = 0; e < 8; ++e) kf[e] *= inv;
            } else if (track_kmax && piece == 0) {
                atomicMax((unsigned int*)&red[8], __float_as_uint(sqrtf(ss)));
            }
            const int c = sl >> 5, u = sl & 31, gg = u >> 3, e8 = u & 7;
            const int kidx = (c * 2 + (e8 >> 2)) * 64 + piece * 16 + gg * 4 + (e8 & 3);
            const bf16x8 khi = pack_bf16x8(kf);
            kfrag[kidx] = khi;
            if (split_k) {
                float lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) lo[e] = kf[e] - (float)khi[e];
                kfrag_lo[kidx] = pack_bf16x8(lo);
            }
            __bf16* vb = (__bf16*)vfrag;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int dd = piece * 8 + t;
                vb[(((c * 2 + (dd >> 4)) * 64 + gg * 16 + (dd & 15)) << 3) + e8] = (__bf16)vf[t];
            }
            __builtin_amdgcn_sched_barrier(0);           // one item at a time: bounded registers
        }
    };

    // Block size: halved when k^ is carried as hi + lo.  The split for
    // COSINE depends only on tau and is known now; for DOT + ROPE2D it waits
    // for the norm pre-pass, which also runs before any staging.
    constexpr bool kPrepassRope = SIM == SWIN_SIM_DOT && POS == SWIN_POS_ROPE2D;
    const bool prepass = SIM == SWIN_SIM_DOT && (L.nblk > 1 || kPrepassRope);
    const bool cos_split = SIM == SWIN_SIM_COSINE && tau_eff < SPLIT_TAU;
    if (!prepass) kv_load(0, min(cos_split ? KB / 2 : KB, L.NSP), 0);

    // (3) tables: bias (reversed so that consecutive keys read consecutive
    // floats, scaled by log2 e, shifted by its max), rotary cos/sin.
    float bias_range = 0.0f;
    if (POS == SWIN_POS_TABLE) {
        float mx = -INFINITY, mn = INFINITY;
        for (int i0 = 0; i0 < S * S; i0 += TB * nthr) {
            float tv[TB];
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int i = i0 + j * nthr + tid;
                tv[j] = i < S * S ? p.table[(size_t)(S * S - 1 - i) * g.heads + h] * kLog2e : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < TB; ++j) {
                const int i = i0 + j * nthr + tid;
                if (i < S * S) {
                    bias2[i] = tv[j];
                    mx = fmaxf(mx, tv[j]);
                    mn = fminf(mn, tv[j]);
                }
            }
        }
        if (tid < 8) bias2[S * S + tid] = -INFINITY;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            mx = fmaxf(mx, __shfl_xor(mx, off));
            mn = fminf(mn, __shfl_xor(mn, off));
        }
        if (lane == 0) { red[wave] = mx; red[4 + wave] = mn; }
        __syncthreads();
        mx = red[0]; mn = red[4];
        for (int w = 1; w < nwaves; ++w) { mx = fmaxf(mx, red[w]); mn = fminf(mn, red[4 + w]); }
        bias_range = mx - mn;
        const float shift = SIM == SWIN_SIM_COSINE ? mx + kLog2e / tau_eff : mx;
        for (int i = tid; i < S * S; i += nthr) bias2[i] -= shift;
    }
    if (POS == SWIN_POS_ROPE2D) {
        for (int i = tid; i < M * 16; i += nthr) {
            const int k = i & 7, half = (i >> 3) & 1, pos = i >> 4;
            const double th = p.rope_freqs
                ? (double)p.rope_freqs[((size_t)h * 2 + half) * 8 + k]
                : pow((double)p.rope_base, -(double)k / 8.0);
            double s_, c_;
            sincos((double)pos * th, &s_, &c_);
            rcs[i] = (float)c_;
            rsn[i] = (float)s_;
        }
    }
    if (tid == 0) { red[8] = 0.0f; red[9] = 0.0f; }       // max key / query norm (DOT)
    __syncthreads();

    // (4) DOT over several key blocks, or after rotation: the largest key
    // norm (and, with rotation, query norm) before any block is staged;
    // loads in batches of SB per thread.
    if (prepass) {
        float kmax = 0.0f, qmax = 0.0f;
        const int qend = min(qt1 * 16, N) - qt0 * 16;
        const int nitems = (N + (kPrepassRope ? max(qend, 0) : 0)) * 4;
        for (int b0 = 0; b0 < nitems; b0 += SB * nthr) {
            u32x4 w[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int it = b0 + j * nthr + tid;
                w[j] = u32x4{0u, 0u, 0u, 0u};
                if (it < nitems) {
                    const bool isq = it >= N * 4;
                    const int t = isq ? qt0 * 16 + ((it - N * 4) >> 2) : it >> 2;
                    const int rj = t / M, cj = t - rj * M;
                    w[j] = *(const u32x4*)((isq ? qg : kg) + token_offset(g, win, rj, cj) + h * D + (it & 3) * 8);
                }
            }
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int it = b0 + j * nthr + tid;
                float f[8];
                unpack_bf16x8(w[j], f);
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
                ss += __shfl_xor(ss, 1);
                ss += __shfl_xor(ss, 2);
                if (it >= N * 4) qmax = fmaxf(qmax, sqrtf(ss));
                else             kmax = fmaxf(kmax, sqrtf(ss));
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            kmax = fmaxf(kmax, __shfl_xor(kmax, off));
            qmax = fmaxf(qmax, __shfl_xor(qmax, off));
        }
        if (lane == 0) {
            atomicMax((unsigned int*)&red[8], __float_as_uint(kmax));
            atomicMax((unsigned int*)&red[9], __float_as_uint(qmax));
        }
        __syncthreads();
    }
    bool split_k = cos_split, split_q = cos_split && POS == SWIN_POS_ROPE2D;
    if (kPrepassRope) split_k = split_q = red[8] * red[9] * (kLog2e / sqrtf((float)D)) > SPLIT_BOUND;
    const int kbs = split_k ? KB / 2 : KB;               // slots per staged block

    Tiles<NQ> T;
    bool general = false;
    const Stage st = {kfrag, kfrag + (KB / 2) * 4, vfrag, bias2, S, S * S};

    // ---- block 0 (its first batch is already in flight unless a pre-pass ran)
    {
        const int cnt = min(kbs, L.NSP);
        if (prepass) kv_load(0, cnt, 0);
        kv_store(0, cnt, 0, split_k, !prepass);
        for (int b0 = SB * nthr; b0 < cnt * 4; b0 += SB * nthr) {
            kv_load(0, cnt, b0);
            kv_store(0, cnt, b0, split_k, !prepass);
        }
    }
    __syncthreads();

    for (int s0 = 0; s0 < L.NSP; s0 += kbs) {
        const int cnt = min(kbs, L.NSP - s0);
        if (s0 > 0) {
            __syncthreads();                              // previous block consumed
            for (int b0 = 0; b0 < cnt * 4; b0 += SB * nthr) {
                kv_load(s0, cnt, b0);
                kv_store(s0, cnt, b0, split_k, !prepass);
            }
            __syncthreads();
        }

        // ---- per query tile set-up, once the first block (and the key
        // norm bound) is in place.
        if (s0 == 0) {
            const float kmax = red[8];
#pragma unroll
            for (int qi = 0; qi < NQ; ++qi) {
                float qv[8];
                unpack_bf16x8(qraw[qi], qv);
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[e] = qvalid[qi] ? qv[e] : 0.0f;
                if (POS == SWIN_POS_ROPE2D) {
                    const int half = grp >> 1, pos = half ? qci[qi] : qri[qi];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int k = (grp & 1) * 4 + j;
                        const float co = rcs[(pos * 2 + half) * 8 + k], si = rsn[(pos * 2 + half) * 8 + k];
                        const float x0 = qv[2 * j], x1 = qv[2 * j + 1];
                        qv[2 * j] = x0 * co - x1 * si;
                        qv[2 * j + 1] = x0 * si + x1 * co;
                    }
                }
                T.qf[qi] = pack_bf16x8(qv);
                float lo[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) lo[e] = qv[e] - (float)T.qf[qi][e];
                T.qf_lo[qi] = pack_bf16x8(lo);
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(qv[e], qv[e], ss);
                ss += __shfl_xor(ss, 16);
                ss += __shfl_xor(ss, 32);
                const float qn = sqrtf(ss);
                float spread;
                if (SIM == SWIN_SIM_COSINE) {
                    T.qscale[qi] = kLog2e / (tau_eff * fmaxf(qn, 1e-12f));
                    T.negm[qi] = POS == SWIN_POS_TABLE ? 0.0f : -kLog2e / tau_eff;
                    spread = 2.0f * kLog2e / tau_eff + bias_range;
                } else {
                    T.qscale[qi] = kLog2e / sqrtf((float)D);
                    const float c_i = qn * kmax * T.qscale[qi];
                    T.negm[qi] = -c_i;
                    spread = 2.0f * c_i + bias_range;
                }
                T.exact[qi] = __any(!(spread <= RANGE_LIMIT)) != 0;
                general = general || T.exact[qi];
                T.qoff[qi] = (M - 1 - qri[qi]) * S + (M - 1 - qci[qi]);
                T.rlo[qi] = 0; T.rhi[qi] = M;
                int clo = 0, chi = M;
                if (shifted) {
                    region_interval(wr, g.nwr, M, g.shift, qri[qi], T.rlo[qi], T.rhi[qi]);
                    region_interval(wc, g.nwc, M, g.shift, qci[qi], clo, chi);
                }
                const uint64_t hi_bits = chi >= 64 ? ~0ull : ((1ull << chi) - 1ull);
                T.cmask[qi] = hi_bits & ~((1ull << clo) - 1ull);
                T.mrun[qi] = -INFINITY;
                T.o0[qi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                T.o1[qi] = T.o0[qi];
                T.ls[qi] = T.o0[qi];
            }
            general = general || split_k || split_q;
        }

        // ---- the key chunks of this block
        if (nq > 0) {
            if (general)
                run_general<SIM, POS, NQ>(st, T, s0, cnt, lane, grp, L.GPR, L.SR, needs_mask, split_k, split_q);
            else if (needs_mask)
                run_fast<SIM, POS, NQ, true>(st, T, s0, cnt, lane, grp, L.GPR, L.SR);
            else
                run_fast<SIM, POS, NQ, false>(st, T, s0, cnt, lane, grp, L.GPR, L.SR);
        }
    }

    // ---- normalise and write back to the query tokens' grid positions
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
        if (!qvalid[qi]) continue;
        const float inv = 1.0f / T.ls[qi][0];
        uint16_t* dst = og + token_offset(g, win, qri[qi], qci[qi]) + h * D + grp * 4;
        *(bf16x4*)dst = pack_bf16x4(T.o0[qi][0] * inv, T.o0[qi][1] * inv, T.o0[qi][2] * inv, T.o0[qi][3] * inv);
        *(bf16x4*)(dst + 16) = pack_bf16x4(T.o1[qi][0] * inv, T.o1[qi][1] * inv, T.o1[qi][2] * inv, T.o1[qi][3] * inv);
    }
}

template <int SIM, int POS>
hipError_t launch_nq(const AttnParams& p, const Layout& L, int nq, int threads, size_t lds, hipStream_t s)
{
    auto* fn = nq == 1 ? attn_mfma_kernel<SIM, POS, 1> : attn_mfma_kernel<SIM, POS, 2>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<8 * L.P, threads, lds, s>>>(p, L);
    return hipGetLastError();
}

template <int SIM>
hipError_t launch_pos(const AttnParams& p, const Layout& L, int nq, int threads, size_t lds, hipStream_t s)
{
    switch (p.pos) {
    case SWIN_POS_NONE:  return launch_nq<SIM, SWIN_POS_NONE>(p, L, nq, threads, lds, s);
    case SWIN_POS_TABLE: return launch_nq<SIM, SWIN_POS_TABLE>(p, L, nq, threads, lds, s);
    default:             return launch_nq<SIM, SWIN_POS_ROPE2D>(p, L, nq, threads, lds, s);
    }
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, hipStream_t stream)
{
    const Geometry& g = p.g;
    if (g.nwin == 0) return hipSuccess;
    Layout L;
    L.SR = (g.M + 7) / 8 * 8;
    L.NSP = (g.M * L.SR + 31) / 32 * 32;
    L.GPR = L.SR / 8;
    L.NQT = (g.N + 15) / 16;
    L.nqb = (L.NQT + QT_MAX * MAX_WAVES - 1) / (QT_MAX * MAX_WAVES);
    L.nblk = (L.NSP + KB - 1) / KB;
    const int64_t total = (int64_t)g.nwin * g.heads * L.nqb;
    L.total = (int)total;
    L.P = (int)((total + 7) / 8);
    // tiles per query block (at most), waves per workgroup, tiles per wave
    const int per_block = (L.NQT + L.nqb - 1) / L.nqb;
    int nwaves = (per_block + QT_MAX - 1) / QT_MAX;
    if (nwaves > MAX_WAVES) nwaves = MAX_WAVES;
    const int nq = (per_block + nwaves - 1) / nwaves;
    const int S = 2 * g.M - 1;
    size_t lds = (size_t)KB * 4 * sizeof(bf16x8) * 2 + 16 * sizeof(float);
    if (p.pos == SWIN_POS_TABLE) lds += (size_t)(S * S + 8) * sizeof(float);
    if (p.pos == SWIN_POS_ROPE2D) lds += (size_t)g.M * 32 * sizeof(float);
    if (p.sim == SWIN_SIM_COSINE) return launch_pos<SWIN_SIM_COSINE>(p, L, nq, 64 * nwaves, lds, stream);
    return launch_pos<SWIN_SIM_DOT>(p, L, nq, 64 * nwaves, lds, stream);
}

}  // namespace swin
