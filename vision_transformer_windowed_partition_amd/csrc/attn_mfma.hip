// Fused window attention on the gfx950 matrix cores (bf16 in, fp32
// accumulate, bf16 out), d = 32.
//
// What it computes is the window attention of the SwinV2 card (eq. 1-2, the
// window-attention pseudocode), with the log-CPB bias table (eq. 3-4), the
// rotary variant and exact, never-materialised softmax of the FlashSwin
// abstract, over cyclic-shift or interleaved (Iwin) windows.
//
// Work decomposition.  A workgroup owns one (window, head, block of up to 16
// query tiles of 16 queries); each wavefront owns up to QT query tiles.  The
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
// them off the vector ALU.
//
// Key slots.  Key (rj, cj) of the window sits in slot rj*SR + cj with SR = M
// rounded up to 8, so a lane's 8 slots share one key row; slots are padded to
// a multiple of 32.  Padded slots and keys of another shift region are
// masked per 8-slot group; a group masked for every lane of a tile is
// skipped outright, a group masked for one lane reads its bias from a row of
// -inf, and only groups split by a region edge pay a per-element select.
//
// Softmax normaliser.  Softmax is invariant to a per-row shift, so any c_i
// with c_i >= max_j logit_ij can replace the row max when no term can
// underflow.  COSINE: |cos| <= 1, so c_h = 1/tau_h + max bias (per head).
// DOT: Cauchy-Schwarz, c_i = ||q_i|| max_j ||k_j|| / sqrt(d) + max bias.
// When the spread 2 * (c_i - bias-free part) + bias range stays below 2^60
// in base 2, every weight is at least 2^-60 of the largest and this static
// shift is exact; then each score costs one FMA and one exp2.  Otherwise the
// tile falls back to the online normaliser (running max per 32-key chunk,
// rescaling the accumulators), which has no range condition.
#include "common.hpp"
#include "launch.hpp"

namespace swin {

namespace {

constexpr int D = 32;
constexpr int QT = 4;          // query tiles per wavefront
constexpr int MAX_WAVES = 4;
constexpr int KB = 256;        // key slots staged per block
constexpr float RANGE_LIMIT = 60.0f;
// Precision split: with bf16 operands a rounded unit vector k^ (or a rotated
// q, k) errs by up to 2^-9 of its norm, and the logit multiplies that error
// by 1/tau (COSINE) or by ||q|| ||k|| / sqrt(d) (DOT after rotation).  Past
// these amplifications the rounded operand is carried as hi + lo, two bf16
// terms, and the score takes one more MFMA per split operand.
constexpr float SPLIT_TAU = 0.1f;      // COSINE: split when tau < 0.1
constexpr float SPLIT_BOUND = 20.0f;   // DOT + ROPE2D: split when max ||q|| ||k|| log2(e)/sqrt(d) > 20

struct Layout {                // derived sizes, identical for every workgroup
    int SR;                    // slots per key row (M rounded up to 8)
    int NSP;                   // key slots, padded to 32
    int GPR;                   // 8-slot groups per key row
    int NQT;                   // query tiles per window-head
    int nqb;                   // query blocks per window-head
    int nblk;                  // key blocks per window-head
    int total;                 // workgroups with work
    int P;                     // workgroups per XCD slot
};

template <int SIM, int POS>
__global__ void __launch_bounds__(256)
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
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int grp = lane >> 4;       // 16-lane group: k-range of the operands
    const int li = lane & 15;        // row / column inside a 16 x 16 tile

    bf16x8* kfrag = (bf16x8*)smem;                       // [KB/32][2][64]
    bf16x8* vfrag = kfrag + KB * 4;                      // [KB/32][2][64]
    float* red = (float*)(vfrag + KB * 4);               // [16] reductions
    float* bias2 = red + 16;                             // [S*S + 8]   (TABLE)
    float* rcs = bias2 + (POS == SWIN_POS_TABLE ? S * S + 8 : 0);   // [M][2][8] (ROPE2D)
    float* rsn = rcs + (POS == SWIN_POS_ROPE2D ? M * 16 : 0);

    const float tau_eff = SIM == SWIN_SIM_COSINE ? fmaxf(p.tau[h], p.tau_min) : 1.0f;

    // ---- tables: bias (reversed so that consecutive keys read consecutive
    // floats, scaled by log2 e, shifted by its max), rotary cos/sin.
    float bias_range = 0.0f;
    if (POS == SWIN_POS_TABLE) {
        float mx = -INFINITY, mn = INFINITY;
        for (int i = tid; i < S * S; i += blockDim.x) {
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
        mx = red[0]; mn = red[4];
        for (int w = 1; w < nwaves; ++w) { mx = fmaxf(mx, red[w]); mn = fminf(mn, red[4 + w]); }
        bias_range = mx - mn;
        const float shift = SIM == SWIN_SIM_COSINE ? mx + kLog2e / tau_eff : mx;
        for (int i = tid; i < S * S; i += blockDim.x) bias2[i] -= shift;
    }
    if (POS == SWIN_POS_ROPE2D) {
        for (int i = tid; i < M * 16; i += blockDim.x) {
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

    // ---- this wavefront's query tiles
    const int qt0 = qb * L.NQT / L.nqb, qt1 = (qb + 1) * L.NQT / L.nqb;
    const int per = (qt1 - qt0 + nwaves - 1) / nwaves;
    const int my0 = qt0 + wave * per;
    const int nq = max(0, min(per, qt1 - my0));           // wave-uniform, <= QT

    // ---- DOT over several key blocks, or after rotation: the largest key
    // norm (and, with rotation, query norm) before any block is staged.
    constexpr bool kPrepassRope = SIM == SWIN_SIM_DOT && POS == SWIN_POS_ROPE2D;
    const bool prepass = SIM == SWIN_SIM_DOT && (L.nblk > 1 || kPrepassRope);
    if (prepass) {
        float kmax = 0.0f, qmax = 0.0f;
        const int qend = min(qt1 * 16, N) - qt0 * 16;
        const int nitems = (N + (kPrepassRope ? max(qend, 0) : 0)) * 4;
        for (int it = tid; it < nitems; it += blockDim.x) {
            const bool isq = it >= N * 4;
            const int t = isq ? qt0 * 16 + ((it - N * 4) >> 2) : it >> 2;
            const int piece = it & 3;
            const int rj = t / M, cj = t - rj * M;
            const u32x4 w = *(const u32x4*)((isq ? qg : kg) + token_offset(g, win, rj, cj) + h * D + piece * 8);
            float f[8];
            unpack_bf16x8(w, f);
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
            ss += __shfl_xor(ss, 1);
            ss += __shfl_xor(ss, 2);
            if (isq) qmax = fmaxf(qmax, sqrtf(ss));
            else     kmax = fmaxf(kmax, sqrtf(ss));
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
    bool split_k = false, split_q = false;
    if (SIM == SWIN_SIM_COSINE) {
        split_k = tau_eff < SPLIT_TAU;
        split_q = split_k && POS == SWIN_POS_ROPE2D;
    } else if (kPrepassRope) {
        split_k = split_q = red[8] * red[9] * (kLog2e / sqrtf((float)D)) > SPLIT_BOUND;
    }
    const int kbs = split_k ? KB / 2 : KB;               // slots per staged block
    bf16x8* kfrag_lo = kfrag + (KB / 2) * 4;             // second half holds k^ lo terms

    bf16x8 qf[QT], qf_lo[QT];
    float qscale[QT], negm[QT], mrun[QT];
    int qoff[QT], rlo[QT], rhi[QT];
    uint64_t cmask[QT];
    bool exact[QT];
    f32x4 o0[QT], o1[QT], ls[QT];
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

    for (int s0 = 0; s0 < L.NSP; s0 += kbs) {
        const int cnt = min(kbs, L.NSP - s0);
        if (s0 > 0) __syncthreads();                      // previous block consumed

        // ---- stage key slots [s0, s0+cnt) as MFMA fragments
        for (int it = tid; it < cnt * 4; it += blockDim.x) {
            const int sl = it >> 2, piece = it & 3;
            const int s = s0 + sl;
            const int rj = s / L.SR, cj = s - rj * L.SR;
            const bool valid = rj < M && cj < M;
            float kf[8], vf[8];
            if (valid) {
                const int64_t off = token_offset(g, win, rj, cj) + h * D + piece * 8;
                unpack_bf16x8(*(const u32x4*)(kg + off), kf);
                unpack_bf16x8(*(const u32x4*)(vg + off), vf);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) { kf[e] = 0.0f; vf[e] = 0.0f; }
            }
            if (POS == SWIN_POS_ROPE2D && valid) {
                const int half = piece >> 1, pos = half ? cj : rj;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = (piece & 1) * 4 + j;
                    const float co = rcs[(pos * 2 + half) * 8 + k], si = rsn[(pos * 2 + half) * 8 + k];
                    const float x0 = kf[2 * j], x1 = kf[2 * j + 1];
                    kf[2 * j] = x0 * co - x1 * si;
                    kf[2 * j + 1] = x0 * si + x1 * co;
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
            } else if (!prepass && piece == 0) {
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
        }
        __syncthreads();

        // ---- per query tile set-up, once the first block (and the key
        // norm bound) is in place
        if (s0 == 0) {
            const float kmax = red[8];
#pragma unroll
            for (int qi = 0; qi < QT; ++qi) {
                o0[qi] = zero4; o1[qi] = zero4; ls[qi] = zero4;
                mrun[qi] = -INFINITY;
                qf[qi] = bf16x8{};
                qf_lo[qi] = bf16x8{};
                qscale[qi] = 0.0f; negm[qi] = 0.0f; qoff[qi] = 0;
                rlo[qi] = 0; rhi[qi] = M; cmask[qi] = 0; exact[qi] = false;
                if (qi >= nq) continue;
                const int t = (my0 + qi) * 16 + li;
                const bool valid = t < N;
                const int ri = valid ? t / M : 0, ci = valid ? t % M : 0;
                float qv[8];
                if (valid) {
                    unpack_bf16x8(*(const u32x4*)(qg + token_offset(g, win, ri, ci) + h * D + grp * 8), qv);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) qv[e] = 0.0f;
                }
                if (POS == SWIN_POS_ROPE2D) {
                    const int half = grp >> 1, pos = half ? ci : ri;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int k = (grp & 1) * 4 + j;
                        const float co = rcs[(pos * 2 + half) * 8 + k], si = rsn[(pos * 2 + half) * 8 + k];
                        const float x0 = qv[2 * j], x1 = qv[2 * j + 1];
                        qv[2 * j] = x0 * co - x1 * si;
                        qv[2 * j + 1] = x0 * si + x1 * co;
                    }
                }
                qf[qi] = pack_bf16x8(qv);
                if (split_q) {
                    float lo[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) lo[e] = qv[e] - (float)qf[qi][e];
                    qf_lo[qi] = pack_bf16x8(lo);
                }
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(qv[e], qv[e], ss);
                ss += __shfl_xor(ss, 16);
                ss += __shfl_xor(ss, 32);
                const float qn = sqrtf(ss);
                float spread;
                if (SIM == SWIN_SIM_COSINE) {
                    qscale[qi] = kLog2e / (tau_eff * fmaxf(qn, 1e-12f));
                    negm[qi] = POS == SWIN_POS_TABLE ? 0.0f : -kLog2e / tau_eff;
                    spread = 2.0f * kLog2e / tau_eff + bias_range;
                } else {
                    qscale[qi] = kLog2e / sqrtf((float)D);
                    const float c_i = qn * kmax * qscale[qi];
                    negm[qi] = -c_i;
                    spread = 2.0f * c_i + bias_range;
                }
                exact[qi] = __any(!(spread <= RANGE_LIMIT)) != 0;
                qoff[qi] = (M - 1 - ri) * S + (M - 1 - ci);
                if (needs_mask) {
                    int clo = 0, chi = M;
                    if (shifted) {
                        region_interval(wr, g.nwr, M, g.shift, ri, rlo[qi], rhi[qi]);
                        region_interval(wc, g.nwc, M, g.shift, ci, clo, chi);
                    }
                    const uint64_t hi_bits = chi >= 64 ? ~0ull : ((1ull << chi) - 1ull);
                    cmask[qi] = hi_bits & ~((1ull << clo) - 1ull);
                }
            }
        }

        // ---- the key chunks of this block
        for (int c = 0; c < cnt / 32; ++c) {
            const bf16x8 ka = kfrag[(c * 2 + 0) * 64 + lane];
            const bf16x8 kb = kfrag[(c * 2 + 1) * 64 + lane];
            bf16x8 ka_lo = ka, kb_lo = kb;
            if (split_k) {
                ka_lo = kfrag_lo[(c * 2 + 0) * 64 + lane];
                kb_lo = kfrag_lo[(c * 2 + 1) * 64 + lane];
            }
            const bf16x8 va = vfrag[(c * 2 + 0) * 64 + lane];
            const bf16x8 vb = vfrag[(c * 2 + 1) * 64 + lane];
            const int gam = (s0 >> 3) + c * 4 + grp;          // this lane's 8-slot group
            const int rj = gam / L.GPR;
            const int c0 = (gam - rj * L.GPR) * 8;
            const int koff = rj * S + c0;
#pragma unroll
            for (int qi = 0; qi < QT; ++qi) {
                if (qi >= nq) break;
                uint32_t bits = 0xffu;
                if (needs_mask) {
                    const bool rok = rj >= rlo[qi] && rj < rhi[qi];
                    bits = rok ? (uint32_t)(cmask[qi] >> c0) & 0xffu : 0u;
                    if (!__any(bits != 0u)) continue;             // whole chunk masked
                }
                f32x4 sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[qi], zero4, 0, 0, 0);
                f32x4 sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qf[qi], zero4, 0, 0, 0);
                if (split_k) {
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka_lo, qf[qi], sa, 0, 0, 0);
                    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb_lo, qf[qi], sb, 0, 0, 0);
                }
                if (split_q) {
                    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf_lo[qi], sa, 0, 0, 0);
                    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qf_lo[qi], sb, 0, 0, 0);
                }
                const float x[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
                float add[8];
                if (POS == SWIN_POS_TABLE) {
                    const float* bp = bias2 + (bits == 0u ? S * S : koff + qoff[qi]);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        add[e] = SIM == SWIN_SIM_COSINE ? bp[e] : bp[e] + negm[qi];
                } else {
                    const float a = bits == 0u ? -INFINITY : negm[qi];
#pragma unroll
                    for (int e = 0; e < 8; ++e) add[e] = a;
                }
                const bool partial = needs_mask && __any(bits != 0u && bits != 0xffu);
                float pr[8];
                if (!exact[qi]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(fmaf(x[e], qscale[qi], add[e]));
                    if (partial) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) pr[e] = (bits >> e) & 1u ? pr[e] : 0.0f;
                    }
                } else {
                    float xs[8];
                    float cm = -INFINITY;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        xs[e] = fmaf(x[e], qscale[qi], add[e]);
                        if (partial) xs[e] = (bits >> e) & 1u ? xs[e] : -INFINITY;
                        cm = fmaxf(cm, xs[e]);
                    }
                    cm = fmaxf(cm, __shfl_xor(cm, 16));
                    cm = fmaxf(cm, __shfl_xor(cm, 32));
                    const float mnew = fmaxf(mrun[qi], cm);
                    const float mref = mnew == -INFINITY ? 0.0f : mnew;
                    const float alpha = __builtin_amdgcn_exp2f(mrun[qi] - mref);
                    o0[qi] *= alpha; o1[qi] *= alpha; ls[qi] *= alpha;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(xs[e] - mref);
                    mrun[qi] = mnew;
                }
                const bf16x8 pb = pack_bf16x8(pr);
                o0[qi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o0[qi], 0, 0, 0);
                o1[qi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pb, o1[qi], 0, 0, 0);
                ls[qi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, ls[qi], 0, 0, 0);
            }
        }
    }

    // ---- normalise and write back to the query tokens' grid positions
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) {
        if (qi >= nq) break;
        const int t = (my0 + qi) * 16 + li;
        if (t >= N) continue;
        const int ri = t / M, ci = t % M;
        const float inv = 1.0f / ls[qi][0];
        uint16_t* dst = og + token_offset(g, win, ri, ci) + h * D + grp * 4;
        *(bf16x4*)dst = pack_bf16x4(o0[qi][0] * inv, o0[qi][1] * inv, o0[qi][2] * inv, o0[qi][3] * inv);
        *(bf16x4*)(dst + 16) = pack_bf16x4(o1[qi][0] * inv, o1[qi][1] * inv, o1[qi][2] * inv, o1[qi][3] * inv);
    }
}

template <int SIM>
hipError_t dispatch_pos(const AttnParams& p, const Layout& L, int threads, size_t lds, hipStream_t s)
{
    const int grid = 8 * L.P;
    auto* fn = p.pos == SWIN_POS_NONE  ? attn_mfma_kernel<SIM, SWIN_POS_NONE>
             : p.pos == SWIN_POS_TABLE ? attn_mfma_kernel<SIM, SWIN_POS_TABLE>
                                       : attn_mfma_kernel<SIM, SWIN_POS_ROPE2D>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<grid, threads, lds, s>>>(p, L);
    return hipGetLastError();
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
    L.nqb = (L.NQT + QT * MAX_WAVES - 1) / (QT * MAX_WAVES);
    L.nblk = (L.NSP + KB - 1) / KB;
    const int64_t total = (int64_t)g.nwin * g.heads * L.nqb;
    L.total = (int)total;
    L.P = (int)((total + 7) / 8);
    int nwaves = (L.NQT + QT - 1) / QT;
    if (nwaves > MAX_WAVES) nwaves = MAX_WAVES;
    const int S = 2 * g.M - 1;
    size_t lds = (size_t)KB * 4 * sizeof(bf16x8) * 2 + 16 * sizeof(float);
    if (p.pos == SWIN_POS_TABLE) lds += (size_t)(S * S + 8) * sizeof(float);
    if (p.pos == SWIN_POS_ROPE2D) lds += (size_t)g.M * 32 * sizeof(float);
    if (p.sim == SWIN_SIM_COSINE) return dispatch_pos<SWIN_SIM_COSINE>(p, L, 64 * nwaves, lds, stream);
    return dispatch_pos<SWIN_SIM_DOT>(p, L, 64 * nwaves, lds, stream);
}

}  // namespace swin
