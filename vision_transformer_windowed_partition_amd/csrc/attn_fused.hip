// Window attention with the attention branch's input projection fused in
// (SwinV2 card, Method item 1 and the block pseudocode: the block maps the
// features through one linear layer to q, k, v and attends within windows):
// q, k, v = split(x W^T + b), then the window attention of attn_small.hip,
// without q, k, v ever reaching HBM.
//
// bf16, d = 32, windows of 9 <= M <= 16 (16 key slots per key row), C a
// multiple of 32 up to 192.  One workgroup of eight wavefronts per
// window-head (two per SIMD, two workgroups a compute unit by LDS):
//   1. the head's 96 rows of W (its q, k and v outputs; C bf16 each) go to
//      LDS with their bias, and the head's column of the bias table as in
//      attn_small (reversed, log2 units less an offset);
//   2. wavefront w projects k and v for the window's key rows 2w and 2w+1:
//      per row of 16 slots, K^T = W_k X^T and V^T = W_v X^T on the
//      matrix cores (A: 16 rows of W from LDS, B: 8 channels of one token per
//      lane, loaded straight from x), fp32 accumulation; the bias is added,
//      k is unit-normalised and scaled by log2(e)/tau (COSINE) and both are
//      rounded once and written to LDS in the layouts the attention reads
//      (K^ in MFMA operand order, V as swizzled rows);
//   3. wavefront w projects q for its query tiles 2w and 2w+1 (Q^T = W_q X^T;
//      for M = 16 these are its key rows, projected in step 2 from the same
//      features), moves the result from the accumulator layout (4 channels
//      of a token per lane) to the B-operand layout (8 consecutive channels
//      per lane) with two lane-half swaps, and after the workgroup's second
//      barrier runs the pair through the keys as attn_small does.
// Precision.  q, k, v are the fp32 products of bf16 features and weights,
// rounded once.  Where the rounding of the MFMA operands would be amplified
// past the bf16 tolerance (COSINE with tau < 0.1; DOT with a logit bound
// above 20, log2 units), q and k are carried as hi + lo bf16 pairs and S^T
// takes three products, scaled per key by 1/||k|| (COSINE) in fp32.
#include "common.hpp"
#include "launch_proj.hpp"
#include "small_core.hpp"

namespace swin {

namespace {

using namespace tio;
using namespace lanes;
using namespace core;

constexpr int MAXCK = 6;               // 32-channel input steps: C <= 192
constexpr float SPLIT_BOUND = 20.0f;   // DOT: hi + lo past this logit bound (log2 units)

struct FusedLayout {
    int NQT;                   // query tiles of 16 per window
    int wgs;                   // work items: window-heads
    int P;                     // work ids per XCD slot
    int CK;                    // C / 32
    int wrow;                  // LDS row stride of W (bf16 elements): C + 8
    float inv_M;
};

// bf16 bits of (a, b), round to nearest even
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b16x2));
}

__device__ __forceinline__ float bf16_round(float a)
{
    return __uint_as_float(pack2(a, 0.0f) << 16);
}

// The accumulator layout of Q^T (lane (li, g): channels 4g..4g+3 in lo, 16+4g..+3
// in hi, as bf16 pairs lo0, lo1 / hi0, hi1) to the B-operand layout (lane (li, G):
// channels 8G..8G+7).  The 32-lane swap moves channels 0-15 of groups 2, 3 and
// 16-31 of groups 0, 1 across; the 16-lane swap then pairs neighbours.
__device__ __forceinline__ bf16x8 to_b_operand(uint32_t lo0, uint32_t lo1, uint32_t hi0, uint32_t hi1)
{
    u32x4 out;
    {
        const auto s32 = __builtin_amdgcn_permlane32_swap(lo0, hi0, false, false);
        const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
        out[0] = s16[0];
        out[2] = s16[1];
    }
    {
        const auto s32 = __builtin_amdgcn_permlane32_swap(lo1, hi1, false, false);
        const auto s16 = __builtin_amdgcn_permlane16_swap(s32[0], s32[1], false, false);
        out[1] = s16[0];
        out[3] = s16[1];
    }
    return __builtin_bit_cast(bf16x8, out);
}

constexpr int FW = 8;                  // wavefronts per workgroup (one query-tile pair each)

// Q16: M = 16, where key row r is also query tile r (16 tokens), so a
// wavefront projects q for the two rows it projects k and v for and keeps it.
template <int SIM, int POS, int NCH, bool Q16>
__global__ void __launch_bounds__(FW * 64)
attn_fused_kernel(AttnParams p, const __bf16* __restrict__ x, const __bf16* __restrict__ w,
                  const float* __restrict__ bqkv, FusedLayout L)
{
    constexpr int GPR = 2;                          // 16 key slots per key row
    constexpr int NTHR = FW * 64;
    constexpr int WLOADS = (96 * 4 * MAXCK + NTHR - 1) / NTHR;
    extern __shared__ __attribute__((aligned(16))) float smem_f[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1, C = g.C, CK = L.CK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;

    const int tabsz = POS == SWIN_POS_TABLE ? (S * S + 8 + 3) / 4 * 4 : 0;
    float* bias2 = smem_f;                                        // [S*S + 8]
    float* red = bias2 + tabsz;                                   // [32]
    float* kinv = red + 32;                                       // [NCH*32] 1/||k|| (precise, split)
    float* bsh = kinv + NCH * 32;                                 // [96] the head's q, k, v biases
    bf16x8* kst = (bf16x8*)(bsh + 96);                            // [NCH][2][64] K^ (hi)
    bf16x8* klo = kst + NCH * 2 * 64;                             // [NCH][2][64] remainders
    __bf16* vst = (__bf16*)(klo + NCH * 2 * 64);                  // [NCH*32][D]
    __bf16* wst = vst + NCH * 32 * D;                             // [96][wrow]

    const int work = (blockIdx.x & 7) * L.P + (blockIdx.x >> 3);
    if (work >= L.wgs) return;                                    // whole workgroup, before any barrier
    const int h = work % g.heads;
    const int win = work / g.heads;
    const float tau_eff = SIM == SWIN_SIM_COSINE ? fmaxf(p.tau[h], p.tau_min) : 1.0f;
    const float inv_tau = 1.0f / tau_eff;
    const bool precise = SIM == SWIN_SIM_COSINE && tau_eff < PRECISE_TAU;

    const WinPlace wp = place_window(g, win);
    const WinGeo& wg = wp.wg;
    const bool padded = 16 != M || NCH * 32 != M * 16;
    const bool needs_mask = wp.last_r || wp.last_c || padded;
    const uint32_t bytes = (uint32_t)wp.span * 2u;
    const Rsrc xr = make_rsrc(x + wp.base, bytes);                // the image's features, all channels
    const Rsrc orr = make_rsrc((const uint16_t*)p.out + wp.base + h * D, (uint32_t)(wp.span - h * D) * 2u);

    // One 16-row block of a projection for the 16 tokens of this lane group:
    // out^T (16 channels x 16 tokens) = W[row0 .. row0+15] X^T, fp32.
    auto project = [&](const u32x4* xf, int row0) -> f32x4 {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < MAXCK; ++kk) {
            if (kk < CK) {
                const bf16x8 a = *(const bf16x8*)(wst + (row0 + li) * L.wrow + kk * 32 + grp * 8);
                acc = mfma(a, __builtin_bit_cast(bf16x8, xf[kk]), acc);
            }
        }
        return acc;
    };
    // 8 channels of token (r, c) for each 32-channel step: the B operand X^T
    auto load_x = [&](u32x4* xf, int r, int c, bool ok) {
        const uint32_t base = wg.tok(r, c);
#pragma unroll
        for (int kk = 0; kk < MAXCK; ++kk)
            xf[kk] = load16(xr, masked(base + (uint32_t)(kk * 64 + grp * 16), ok && kk < CK));
    };
    // q of one tile from its projection blocks: the bias added, rounded (to
    // q / ||q|| for COSINE outside the precise path, else to hi + lo) and
    // moved to the B-operand layout; ss gets ||q||^2
    auto make_q = [&](const f32x4& q0, const f32x4& q1, bf16x8& qh_out, bf16x8& ql_out, float& ss) {
        float qf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[e] = q0[e] + bsh[4 * grp + e];
            qf[4 + e] = q1[e] + bsh[16 + 4 * grp + e];
        }
        ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(qf[e], qf[e], ss);
        ss = sum_x32(sum_x16(ss));
        float qh[8], ql[8];
        if (SIM == SWIN_SIM_COSINE && !precise) {
            const float qinv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
#pragma unroll
            for (int e = 0; e < 8; ++e) { qh[e] = qf[e] * qinv; ql[e] = 0.0f; }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) { qh[e] = bf16_round(qf[e]); ql[e] = qf[e] - qh[e]; }
        }
        qh_out = to_b_operand(pack2(qh[0], qh[1]), pack2(qh[2], qh[3]), pack2(qh[4], qh[5]), pack2(qh[6], qh[7]));
        ql_out = to_b_operand(pack2(ql[0], ql[1]), pack2(ql[2], ql[3]), pack2(ql[4], ql[5]), pack2(ql[6], ql[7]));
    };

    // key rows 2 wave and 2 wave + 1 (16 slots each, one token per lane); for
    // M = 16 they are also this wave's query tiles
    const int r0 = 2 * wave;
    const bool rows_here = r0 < 2 * NCH;                          // (M <= 12: rows 0-11 only)
    // the first key row's features, in flight with the staging below
    u32x4 xf[MAXCK];
    load_x(xf, r0, li, rows_here && r0 < M && li < M);

    // ---- the head's rows of W (q: h*32.., k: C + h*32.., v: 2C + h*32..) and
    // biases; the table share; all loads issued before the first is used
    const int pieces = 96 * 4 * CK;                               // 16-byte pieces of the 96 rows
    const Rsrc wr = make_rsrc(w, (uint32_t)(3 * C * C) * 2u);
    u32x4 wv[WLOADS];
#pragma unroll
    for (int k = 0; k < WLOADS; ++k) {
        const int i = tid + NTHR * k;
        const int row = i / (4 * CK), pc = i - row * (4 * CK);
        const int grow = (row >> 5) * C + h * D + (row & 31);
        wv[k] = load16(wr, masked((uint32_t)(grow * C + pc * 8) * 2u, i < pieces));
    }
    float bv = 0.0f;
    if (tid < 96) bv = bqkv ? bqkv[(tid >> 5) * C + h * D + (tid & 31)] : 0.0f;
    constexpr int TQ = 2;                                         // (2M-1)^2 <= 961 <= TQ * NTHR
    float tv[TQ], t0 = 0.0f;
    if (POS == SWIN_POS_TABLE) {
        const Rsrc tr = make_rsrc(p.table, (uint32_t)(S * S * g.heads) * 4u);
        t0 = load_f32(tr, (uint32_t)h * 4u);
#pragma unroll
        for (int k = 0; k < TQ; ++k) {
            const int r = min(tid + NTHR * k, S * S - 1);
            tv[k] = load_f32(tr, (uint32_t)__umul24((uint32_t)r, (uint32_t)g.heads) * 4u + (uint32_t)h * 4u);
        }
    }
    vm_wait_all();
#pragma unroll
    for (int k = 0; k < WLOADS; ++k) {
        const int i = tid + NTHR * k;
        if (i < pieces) {
            const int row = i / (4 * CK), pc = i - row * (4 * CK);
            *(u32x4*)(wst + row * L.wrow + pc * 8) = wv[k];
        }
    }
    if (tid < 96) bsh[tid] = bv;
    const float boff = kLog2e * (t0 + (SIM == SWIN_SIM_COSINE ? inv_tau : 0.0f));
    if (POS == SWIN_POS_TABLE) {
        float mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int k = 0; k < TQ; ++k) {
            const int r = tid + NTHR * k;
            mx = fmaxf(mx, tv[k]);
            mn = fminf(mn, tv[k]);
            if (r < S * S) bias2[S * S - 1 - r] = fmaf(tv[k], kLog2e, -boff);
        }
        mx = wave_reduce<Op::Max>(mx);
        mn = wave_reduce<Op::Min>(mn);
        if (lane == 0) { red[FW + wave] = mx; red[2 * FW + wave] = mn; }
        if (wave == 0 && lane < 8) bias2[S * S + lane] = -INFINITY;
    }
    __syncthreads();                                              // W, biases, table

    // ---- k and v of this wave's two key rows, and for M = 16 q of the same
    // tokens
    float kmax = 0.0f;
    bf16x8 qkeep[2], qlkeep[2];
    float qsskeep[2] = {0.0f, 0.0f};
    if (rows_here) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = r0 + j;                                 // key row, slots 16 r + li
            const f32x4 k0 = project(xf, 32), k1 = project(xf, 48);
            const f32x4 v0 = project(xf, 64), v1 = project(xf, 80);
            if (Q16) {
                const f32x4 q0 = project(xf, 0), q1 = project(xf, 16);
                make_q(q0, q1, qkeep[j], qlkeep[j], qsskeep[j]);
            }
            if (j == 0) load_x(xf, r + 1, li, r + 1 < M && li < M);
            float kf[8], vf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[e] = k0[e] + bsh[32 + 4 * grp + e];
                kf[4 + e] = k1[e] + bsh[48 + 4 * grp + e];
                vf[e] = v0[e] + bsh[64 + 4 * grp + e];
                vf[4 + e] = v1[e] + bsh[80 + 4 * grp + e];
            }
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(kf[e], kf[e], ss);
            ss = sum_x32(sum_x16(ss));                            // ||k||^2 of token li
            const int s = 16 * r + li;                            // key slot
            const int c = s >> 5, wi = s & 31;
            const int f = 2 * c + ((wi >> 2) & 1);                // K tile
            const int lr = 4 * (wi >> 3) + (wi & 3);              // operand row of the slot
            float kh[8], kl[8];
            if (SIM == SWIN_SIM_COSINE && !precise) {
                const float ks = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f)) * (kLog2e * inv_tau);
#pragma unroll
                for (int e = 0; e < 8; ++e) { kh[e] = kf[e] * ks; kl[e] = 0.0f; }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) { kh[e] = bf16_round(kf[e]); kl[e] = kf[e] - kh[e]; }
                if (grp == 0)
                    kinv[s] = SIM == SWIN_SIM_COSINE ? __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f)) : 1.0f;
            }
            if (SIM == SWIN_SIM_DOT && r < M && li < M) kmax = fmaxf(kmax, ss);
            // channels 4 grp..+3 -> operand piece grp/2, half grp%2; 16 + 4 grp.. -> piece 2 + grp/2
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int piece = 2 * hf + (grp >> 1);
                const int at = ((f * 64 + lr + 16 * piece) * 8 + (grp & 1) * 4);     // bf16 element
                const u32x2 hi = {pack2(kh[4 * hf], kh[4 * hf + 1]), pack2(kh[4 * hf + 2], kh[4 * hf + 3])};
                *(u32x2*)((__bf16*)kst + at) = hi;
                if (SIM == SWIN_SIM_DOT || precise) {
                    const u32x2 lo = {pack2(kl[4 * hf], kl[4 * hf + 1]), pack2(kl[4 * hf + 2], kl[4 * hf + 3])};
                    *(u32x2*)((__bf16*)klo + at) = lo;
                }
                const int vat = s * D + ((piece ^ v_swizzle(s)) * 8) + (grp & 1) * 4;
                const u32x2 vv = {pack2(vf[4 * hf], vf[4 * hf + 1]), pack2(vf[4 * hf + 2], vf[4 * hf + 3])};
                *(u32x2*)(vst + vat) = vv;
            }
        }
    }
    if (SIM == SWIN_SIM_DOT) {
        kmax = wave_reduce<Op::Max>(kmax);
        if (lane == 0) red[wave] = kmax;
    }
    // ---- q of this wave's query tiles 2 wave, 2 wave + 1 (M < 16: tokens of
    // the dense order r M + c, so projected here from their own features)
    Tile T[2];
    bf16x8 qlo[2];
    int qt[2];
    bool qv[2];
    float qss[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int tq = 2 * wave + i;
        const int t = tq * 16 + li;
        qv[i] = tq < L.NQT && t < N;
        qt[i] = qv[i] ? t : 0;
    }
    const bool has_pair = 2 * wave < L.NQT;
    if (Q16) {
#pragma unroll
        for (int i = 0; i < 2; ++i) { T[i].qf = qkeep[i]; qlo[i] = qlkeep[i]; qss[i] = qsskeep[i]; }
    } else if (has_pair) {
        u32x4 xq[2][MAXCK];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
            load_x(xq[i], ri, ci, qv[i]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const f32x4 q0 = project(xq[i], 0), q1 = project(xq[i], 16);
            make_q(q0, q1, T[i].qf, qlo[i], qss[i]);
        }
    }
    __syncthreads();                                              // K^, remainders, V, kinv, red
    if (!has_pair) return;                                        // after the last barrier
    if (SIM == SWIN_SIM_DOT) {
        kmax = red[0];
#pragma unroll
        for (int r = 1; r < FW; ++r) kmax = fmaxf(kmax, red[r]);
        kmax = sqrtf(kmax);
    }
    float bias_max = 0.0f, bias_range = 0.0f;
    if (POS == SWIN_POS_TABLE) {
        float mx = red[FW], mn = red[2 * FW];
#pragma unroll
        for (int r = 1; r < FW; ++r) { mx = fmaxf(mx, red[FW + r]); mn = fminf(mn, red[2 * FW + r]); }
        bias_max = fmaf(mx, kLog2e, -boff);
        bias_range = (mx - mn) * kLog2e;
    }

    // ---- the pair through the keys, as in attn_small
    const int kbase = (grp / GPR) * S + 8 * (grp % GPR);
    bool any_exact = false, partial = false, split = precise;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float ss = qss[i];
        const float qinv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
        float spread, shift = 0.0f;
        if (SIM == SWIN_SIM_COSINE) {
            T[i].qscale = kLog2e * inv_tau * qinv;
            T[i].negm = -kLog2e * inv_tau;
            spread = 2.0f * kLog2e * inv_tau + bias_range;
        } else {
            T[i].qscale = kLog2e * 0.17677669529663687f;          // log2(e) / sqrt(32)
            const float c_i = sqrtf(ss) * kmax * T[i].qscale;
            T[i].negm = -c_i;
            spread = 2.0f * c_i + bias_range;
            shift = c_i + bias_max;
            split = split || __any(c_i > SPLIT_BOUND) != 0;
        }
        T[i].exact = __any(!(spread <= RANGE_LIMIT)) != 0;
        T[i].cinit = SIM == SWIN_SIM_DOT && POS == SWIN_POS_TABLE ? -shift / T[i].qscale : 0.0f;
        any_exact = any_exact || T[i].exact;
        T[i].mrun = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
        // the running maximum on the precise and split paths, as in attn_small
        T[i].exact = T[i].exact || split;
        T[i].qoff = (M - 1 - ri) * S + (M - 1 - ci) + kbase;
        T[i].colbits = 0xffu;
        T[i].gmask = 0xffffffffu;
        if (needs_mask) {
            int rlo = 0, rhi = M, clo = 0, chi = M;
            if (wp.last_r) { if (ri < M - g.shift) rhi = M - g.shift; else rlo = M - g.shift; }
            if (wp.last_c) { if (ci < M - g.shift) chi = M - g.shift; else clo = M - g.shift; }
            const uint32_t cmask = (chi >= 32 ? 0xffffffffu : ((1u << chi) - 1u)) & ~((1u << clo) - 1u);
            const int rl = grp / GPR;
            T[i].colbits = (cmask >> (8 * (grp % GPR))) & 0xffu;
            const int cb = max(0, (rlo - rl + 1) >> 1);
            const int ce = min(NCH, (rhi - rl + 1) >> 1);
            const uint32_t rows = ce > cb ? ((1u << ce) - 1u) & ~((1u << cb) - 1u) : 0u;
            T[i].gmask = T[i].colbits ? rows : 0u;
            partial = partial || (wp.last_c && ((M - g.shift) & 7)) || (M & 7);
        }
        T[i].o0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        T[i].o1 = T[i].o0;
        T[i].ls = T[i].o0;
    }
    const int negrow = S * S;
    if (any_exact || split) {
        run_pair<SIM, POS, GPR, 0, NCH, true, true, true, 1, true>(kst, vst, T, bias2, kinv, S, negrow, lane,
                                                                   true, split, klo, qlo);
        run_pair<SIM, POS, GPR, 0, NCH, true, true, true, 1, true>(kst, vst, T + 1, bias2, kinv, S, negrow,
                                                                   lane, true, split, klo, qlo + 1);
    } else if (needs_mask) {
        run_masked_pair<SIM, POS, GPR, NCH>(kst, vst, T, bias2, kinv, S, negrow, lane, partial);
    } else
        run_pair<SIM, POS, GPR, 0, NCH, false, false, false, 2>(kst, vst, T, bias2, kinv, S, negrow, lane, false,
                                                             false);

    // ---- normalise and store
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ri = qdiv(qt[i], L.inv_M), ci = qt[i] - ri * M;
        const float inv = __builtin_amdgcn_rcpf(T[i].ls[0]);
        const uint32_t off = masked(wg.tok(ri, ci) + 8u * grp, qv[i]);
        store8(orr, off, pack_bf16x4(T[i].o0[0] * inv, T[i].o0[1] * inv, T[i].o0[2] * inv, T[i].o0[3] * inv));
        store8(orr, off + 32u, pack_bf16x4(T[i].o1[0] * inv, T[i].o1[1] * inv, T[i].o1[2] * inv, T[i].o1[3] * inv));
    }
}

template <int SIM, int POS>
hipError_t launch_fused_sp(const AttnParams& p, const FusedArgs& a, const FusedLayout& L, int nch, size_t lds,
                           hipStream_t s)
{
    auto* fn = nch <= 6 ? attn_fused_kernel<SIM, POS, 6, false>
             : p.g.M == 16 ? attn_fused_kernel<SIM, POS, 8, true> : attn_fused_kernel<SIM, POS, 8, false>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<8 * L.P, FW * 64, lds, s>>>(p, (const __bf16*)a.x, (const __bf16*)a.w, a.b, L);
    return hipGetLastError();
}

}  // namespace

bool attn_fused_supported(const AttnParams& p)
{
    const Geometry& g = p.g;
    return p.dtype == SWIN_DT_BF16 && p.pos != SWIN_POS_ROPE2D && g.layout == SWIN_LAYOUT_GRID && g.d == D &&
           g.M >= 9 && g.M <= 16 && g.C % 32 == 0 && g.C <= 32 * MAXCK &&
           (int64_t)g.H * g.W * g.C * 2 < ((int64_t)1 << 31) && (int64_t)g.W * g.C * 2 < ((int64_t)1 << 24);
}

size_t attn_fused_lds(const AttnParams& p)
{
    const Geometry& g = p.g;
    const int nch = g.M <= 12 ? 6 : 8;
    const int S = 2 * g.M - 1;
    const int tabsz = p.pos == SWIN_POS_TABLE ? (S * S + 8 + 3) / 4 * 4 : 0;
    return (size_t)(tabsz + 32 + nch * 32 + 96) * sizeof(float) + (size_t)nch * 2 * 64 * 16 * 2 +
           (size_t)nch * 32 * D * 2 + (size_t)96 * (g.C + 8) * 2;
}

hipError_t launch_attn_fused(const AttnParams& p, const FusedArgs& a, hipStream_t stream)
{
    const Geometry& g = p.g;
    if (g.nwin == 0) return hipSuccess;
    FusedLayout L;
    L.NQT = (g.N + 15) / 16;
    L.CK = g.C / 32;
    L.wrow = g.C + 8;
    L.inv_M = 1.0f / (float)g.M;
    const int64_t wgs = (int64_t)g.heads * g.nwin;
    if (wgs > INT32_MAX - 8) return hipErrorInvalidValue;
    L.wgs = (int)wgs;
    L.P = (int)((wgs + 7) / 8);
    const int nch = g.M <= 12 ? 6 : 8;
    const size_t lds = attn_fused_lds(p);
    if (p.sim == SWIN_SIM_COSINE) {
        if (p.pos == SWIN_POS_TABLE) return launch_fused_sp<SWIN_SIM_COSINE, SWIN_POS_TABLE>(p, a, L, nch, lds, stream);
        return launch_fused_sp<SWIN_SIM_COSINE, SWIN_POS_NONE>(p, a, L, nch, lds, stream);
    }
    if (p.pos == SWIN_POS_TABLE) return launch_fused_sp<SWIN_SIM_DOT, SWIN_POS_TABLE>(p, a, L, nch, lds, stream);
    return launch_fused_sp<SWIN_SIM_DOT, SWIN_POS_NONE>(p, a, L, nch, lds, stream);
}

}  // namespace swin
