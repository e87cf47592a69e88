// Video (3D) window attention on the gfx950 matrix cores: bf16 tensors, d = 32,
// windows Mt x M x M with M <= 22 (the reading of the video form is the
// one the vector-ALU kernel in attn_video.hip follows: the SwinV2 card's
// window attention, eq. 1-2 and the window-attention pseudocode, with a
// temporal axis treated like the other two and the bias G(dx, dy, dt) of
// eq. 3-4 from a (2Mt-1)(2M-1)^2 x heads table).
//
// A workgroup owns one (window, head, query frame) for 9 <= M <= 16 (four
// wavefronts) and 17 <= M <= 22 (eight), or (window, head, four query
// frames) for M <= 8, one frame a wavefront; either way each wavefront keeps
// four query tiles of 16 queries live for the whole window: their q
// fragments, their normaliser references and their fp32 accumulators for
// O^T and the row sums.  The workgroup then walks the window's key frames:
// per key frame it stages that frame's M x M keys (unit-normalised and scaled by log2(e)/tau for COSINE, raw otherwise)
// as MFMA A-fragments and its values by LDS-DMA, together with the table
// slice of the time offset between each query frame and the key frame (a
// (2M-1)^2 slice, in log2 units), and every wavefront runs its tiles over
// the frame's 32-key chunks: S^T = K^ Q^T (the slice entries, or the scale,
// enter as the accumulator or one FMA), the weights against the normaliser's
// reference (below), P^T rounded to bf16 and O^T += V^T P^T, row sums by a
// third product against ones.  A key
// frame in another temporal shift region than a wavefront's query frame is
// skipped by that wavefront; within a frame, spatial shift regions mask
// 8-key groups (and single keys where a region edge splits a group).
// Normaliser: each frame's logits are bounded above from the slice's largest
// entry and |cos| <= 1 (COSINE) or Cauchy-Schwarz with the frame's largest
// ||k|| (DOT); when that bound lies within 60 (base 2) of the lowest
// possible logit, the frame is exponentiated against it (the accumulators
// rescaled once if it raises the reference), else against a running maximum
// per 32-key chunk, which has no range condition.
#include "common.hpp"
#include "lanes.hpp"
#include "launch_video.hpp"
#include "tile_io.hpp"

namespace swin {

namespace {

using namespace tio;
using namespace lanes;

constexpr int TPW = 4;                 // query tiles a wavefront keeps live
constexpr float PRECISE_TAU = 0.1f;    // COSINE below this: raw k and 1/||k|| in fp32
constexpr float RANGE_LIMIT = 60.0f;   // widest logit spread (base 2) a fixed reference may take

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float sumsq8(const u32x4 w)
{
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t wi = w[i];
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wi), __builtin_bit_cast(bf16x2, wi), s,
                                            false);
    }
    return s;
}

__device__ __forceinline__ int axis_pos(int L, int M, int s, int part, int w, int r)
{
    return part == SWIN_PART_INTERLEAVED ? w + r * (L / M) : (w * M + r + s) % L;
}

struct VTile {
    bf16x8 qf;                 // q (unit for COSINE outside the precise path) as the B operand
    f32x4 o0, o1, ls;          // O^T channels 0-15 and 16-31, row sums
    float mrun;                // reference of the accumulators (running maximum or bound), log2 units
    float qscale;              // per-score scale when not folded into K^
    float qnorm;               // ||q||
    int qoff;                  // bias offset of this tile's query in a slice, with this lane's key group
                               // of chunk 0 when GPR divides 4 (the group's key offset added per chunk)
    uint32_t cbits;            // allowed key columns: of this lane's group when GPR divides 4, else all
    int rlo, rhi;              // allowed key rows (spatial shift regions)
};

// Key slots of a frame: key (r, c) at slot r SR + c, SR = 8, 16 or 24 the
// smallest of these >= M, so every 8-slot group lies in one key row (slots
// past M hold zeros and are masked); a chunk of 32 slots holds 4
// groups, group 4c + grp of the lane being row gam / GPR, columns
// 8 (gam % GPR) .. +7.
//
// One 32-key chunk c of the staged key frame for NU tiles (two, or one when
// the pair's second tile lies past the frame); exact (wave-uniform): the
// running maximum, else the tiles' fixed references.
template <int SIM, int POS, int SR, int NU>
__device__ __forceinline__ void chunk(const bf16x8* kst, const __bf16* vst, const float* bias2, const float* kinv,
                                      VTile* T, int c, int lane, int S, bool mask, bool fold, bool prec,
                                      bool exact)
{
    constexpr int GPR = SR / 8;
    constexpr bool ALIGNED = 4 % GPR == 0;                  // a lane's group keeps its columns in every chunk
    const int grp = lane >> 4, li = lane & 15;
    const int gam = 4 * c + grp;
    const int rj = gam / GPR, cj0 = 8 * (gam - rj * GPR);   // this lane's key group
    uint32_t bits[2];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        const uint32_t cb = ALIGNED ? T[i].cbits : (T[i].cbits >> cj0) & 0xffu;
        bits[i] = !mask ? 0xffu : (rj >= T[i].rlo && rj < T[i].rhi ? cb : 0u);
    }
    if (mask && !__any((bits[0] | (NU > 1 ? bits[1] : 0u)) != 0u)) return;   // chunk masked for the whole wave
    const bf16x8 ka = kst[(c * 2 + 0) * 64 + lane];
    const bf16x8 kb = kst[(c * 2 + 1) * 64 + lane];
    float kin[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
    if (prec) {
        const f32x4 x0 = *(const f32x4*)(kinv + 32 * c + 8 * grp);
        const f32x4 x1 = *(const f32x4*)(kinv + 32 * c + 8 * grp + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { kin[e] = x0[e]; kin[e + 4] = x1[e]; }
    }
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        float add[8];
        if (POS == SWIN_POS_TABLE) {
            const int boff = T[i].qoff + (ALIGNED ? (4 / GPR) * c * S : rj * S + cj0);
            const int idx = bits[i] == 0u ? S * S : boff;
#pragma unroll
            for (int e = 0; e < 8; ++e) add[e] = bias2[idx + e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) add[e] = bits[i] == 0u ? -INFINITY : 0.0f;
        }
        const f32x4 za = {add[0], add[1], add[2], add[3]}, zb = {add[4], add[5], add[6], add[7]};
        const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        const f32x4 sa = mfma(ka, T[i].qf, fold ? za : zero);
        const f32x4 sb = mfma(kb, T[i].qf, fold ? zb : zero);
        float x[8], cm = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float s = e < 4 ? sa[e] : sb[e - 4];
            x[e] = fold ? s : fmaf(s, T[i].qscale * kin[e], add[e]);
            if (mask) x[e] = (bits[i] >> e) & 1u ? x[e] : -INFINITY;
            cm = fmaxf(cm, x[e]);
        }
        float mref = T[i].mrun;
        if (exact) {
            cm = max_x32(max_x16(cm));
            const float mnew = fmaxf(T[i].mrun, cm);
            mref = mnew == -INFINITY ? 0.0f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(T[i].mrun - mref);
            T[i].o0 *= alpha; T[i].o1 *= alpha; T[i].ls *= alpha;
            T[i].mrun = mnew;
        }
        float pr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[e] = __builtin_amdgcn_exp2f(x[e] - mref);
        pb[i] = pack_bf16x8(pr);
    }
    const bf16x8 v0 = vt_frag(vst, c, 0, grp, li);
    const bf16x8 v1 = vt_frag(vst, c, 1, grp, li);
#pragma unroll
    for (int i = 0; i < NU; ++i) {
        T[i].o0 = mfma(v0, pb[i], T[i].o0);
        T[i].o1 = mfma(v1, pb[i], T[i].o1);
        T[i].ls = mfma(ones, pb[i], T[i].ls);
    }
}

// Shape of a kernel family: SR slots per key row (M <= SR), QF query frames a
// workgroup owns, WV wavefronts.  SR = 8 (M <= 8): four frames, one a wave;
// SR = 16 (9 <= M <= 16): one frame over four waves; SR = 24 (17 <= M <= 22):
// one frame over eight waves (31 query tiles at M = 22).  OCC: wavefronts a
// SIMD holds at M = SR (registers capped to fit them).
template <int SR> struct VShape;
template <> struct VShape<8> { static constexpr int QF = 4, WV = 4, OCC = 3; };
template <> struct VShape<16> { static constexpr int QF = 1, WV = 4, OCC = 3; };
template <> struct VShape<24> { static constexpr int QF = 1, WV = 8, OCC = 2; };

// LDS of a workgroup for window M (kernel family SR): K^ fragments and V rows
// of a frame's slots, 1/||k|| per slot, the table slices, the reductions.
__host__ __device__ constexpr int video_nch(int M, int SR) { return (M * SR + 31) / 32; }
__host__ __device__ constexpr int video_slice(int M) { return (2 * M - 1) * (2 * M - 1) + 8; }

// FIT: M = SR, known at compile time (registers capped to hold OCC
// wavefronts a SIMD); else M = a.M < SR, its slots padded.
template <int SIM, int POS, int SR, bool FIT>
__global__ void __launch_bounds__(VShape<SR>::WV * 64)
__attribute__((amdgpu_waves_per_eu(FIT ? VShape<SR>::OCC : 1)))
attn_video_mfma_kernel(VideoArgs a, int units, int per_xcd)
{
    constexpr int GPR = SR / 8;
    constexpr int QF = VShape<SR>::QF, WV = VShape<SR>::WV;
    const int M = FIT ? SR : a.M, S = 2 * M - 1, NQ = M * M;
    const int NCH = video_nch(M, SR);
    const int SLICE = video_slice(M);
    const int SETS = (2 * NCH + WV - 1) / WV;    // K tiles and 1 KB V pieces a wave stages
    constexpr int KS = (2 * video_nch(SR, SR) + WV - 1) / WV;       // ... at most, for M = SR
    extern __shared__ __attribute__((aligned(16))) float smem_f[];
    // (the V staging takes its LDS address as an integer from the array's
    // own: a cast of a derived generic pointer miscompiles there)
    const uint32_t vst_lds = lds_addr(smem_f) + (uint32_t)NCH * 2 * 64 * 16;
    bf16x8* kst = (bf16x8*)smem_f;                                   // [NCH][2][64]
    __bf16* vst = (__bf16*)(kst + NCH * 2 * 64);                     // [NCH*32][D]
    float* kinv = (float*)(vst + NCH * 32 * D);                      // [NCH*32]
    float* bias2 = kinv + NCH * 32;                                  // [QF][SLICE]
    float* red = bias2 + (POS == SWIN_POS_TABLE ? QF * SLICE : 0);   // per wave: slice extrema per frame, ||k||^2

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    const int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (work >= units) return;                   // whole workgroup, before any barrier
    const int Mt = a.Mt;
    const int fblocks = (Mt + QF - 1) / QF;
    const int fb = work % fblocks, wh = work / fblocks;
    const int h = wh % a.heads, win = wh / a.heads;
    const int nW = a.nwt * a.nwr * a.nwc;
    const int b = win / nW, wl = win - b * nW;
    const int wt = wl / (a.nwr * a.nwc), wr = (wl / a.nwc) % a.nwr, wc = wl % a.nwc;
    const bool cyc = a.part == SWIN_PART_CYCLIC;

    // frame addressing: rows and columns as in the 2D kernels, frames by base
    WinGeo wg;
    wg.colb = (uint32_t)a.C * 2u;
    wg.Hm = a.H; wg.Wm = a.W;
    if (cyc) { wg.r0 = wr * M + a.shift; wg.c0 = wc * M + a.shift; wg.rs = wg.cs = 1; }
    else { wg.r0 = wr; wg.c0 = wc; wg.rs = a.nwr; wg.cs = a.nwc; }
    wg.rowb = a.W * wg.colb;
    const int64_t frame_elems = (int64_t)a.H * a.W * a.C;
    const uint32_t bytes = (uint32_t)(frame_elems - h * D) * 2u;
    auto frame_base = [&](int t) -> int64_t {
        return ((int64_t)b * a.T + axis_pos(a.T, Mt, a.shift_t, a.part, wt, t)) * frame_elems + h * D;
    };
    const bool last_r = cyc && a.shift > 0 && wr == a.nwr - 1;
    const bool last_c = cyc && a.shift > 0 && wc == a.nwc - 1;
    const bool mask = last_r || last_c || M != SR;              // shift regions or padded slots

    const float tau_eff = SIM == SWIN_SIM_COSINE ? fmaxf(a.tau[h], a.tau_min) : 1.0f;
    const float inv_tau = 1.0f / tau_eff;
    const bool prec = SIM == SWIN_SIM_COSINE && tau_eff < PRECISE_TAU;
    const bool fold = SIM == SWIN_SIM_COSINE && !prec;
    const float inv_M = 1.0f / (float)M;

    // ---- this wave's query frame and tiles (tile tq: queries 16 tq .. +15
    // of the frame in dense order r M + c)
    const int ti = QF == 1 ? fb : fb * QF + wave;
    const bool active = ti < Mt;
    const int tiq = active ? ti : 0;
    int tlo = 0, thi = Mt;
    if (cyc) region_interval(wt, a.nwt, Mt, a.shift_t, tiq, tlo, thi);
    VTile T[TPW];
    bool tval[TPW];
    {
        const Rsrc qr = make_rsrc((const uint16_t*)a.q + frame_base(tiq), bytes);
        u32x4 qraw[TPW];
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tq = QF == 1 ? wave + WV * k : k;
            const int t = 16 * tq + li;
            tval[k] = active && t < NQ;
            const int tt = tval[k] ? t : 0;
            const int ri = qdiv(tt, inv_M), ci = tt - ri * M;
            qraw[k] = load16(qr, masked(wg.tok(ri, ci) + 16u * grp, tval[k]));
        }
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int tq = QF == 1 ? wave + WV * k : k;
            const int t = tval[k] ? 16 * tq + li : 0;
            const int ri = qdiv(t, inv_M), ci = t - ri * M;
            const float ss = sum_x32(sum_x16(sumsq8(qraw[k])));
            const float qinv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));       // 1 / max(||q||, 1e-12)
            T[k].qf = __builtin_bit_cast(bf16x8, qraw[k]);
            if (fold) {
                float qf[8];
                unpack_bf16x8(qraw[k], qf);
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[e] *= qinv;
                T[k].qf = pack_bf16x8(qf);
            }
            T[k].qscale = SIM == SWIN_SIM_COSINE ? kLog2e * inv_tau * qinv : kLog2e * 0.17677669529663687f;
            T[k].qnorm = sqrtf(ss);
            T[k].o0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            T[k].o1 = T[k].o0;
            T[k].ls = T[k].o0;
            T[k].mrun = -INFINITY;
            constexpr bool ALIGNED = 4 % GPR == 0;
            T[k].qoff = (M - 1 - ri) * S + (M - 1 - ci) + (ALIGNED ? (grp / GPR) * S + 8 * (grp % GPR) : 0);
            int clo = 0, chi = M;
            T[k].rlo = 0; T[k].rhi = M;
            if (last_r) { if (ri < M - a.shift) T[k].rhi = M - a.shift; else T[k].rlo = M - a.shift; }
            if (last_c) { if (ci < M - a.shift) chi = M - a.shift; else clo = M - a.shift; }
            const uint32_t cmask = ((1u << chi) - 1u) & ~((1u << clo) - 1u);
            T[k].cbits = ALIGNED ? (cmask >> (8 * (grp % GPR))) & 0xffu : cmask;
        }
    }
    if (POS == SWIN_POS_TABLE && tid < 8 * QF) bias2[(tid >> 3) * SLICE + S * S + (tid & 7)] = -INFINITY;

    // ---- key frames
    for (int tj = 0; tj < Mt; ++tj) {
        __syncthreads();                         // the previous frame's LDS is consumed
        const int64_t kb0 = frame_base(tj);
        const Rsrc kr = make_rsrc((const uint16_t*)a.k + kb0, bytes);
        const RawRsrc vraw = raw_rsrc((const uint16_t*)a.v + kb0, bytes);
        u32x4 kraw[KS];
        float kmax2 = 0.0f;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int f = wave + WV * k, c = f >> 1, t = f & 1;
            if (k >= SETS) break;
            const int gam = 4 * c + (li >> 2);
            const int rj = gam / GPR, cj = 8 * (gam - (gam / GPR) * GPR) + (li & 3) + 4 * t;
            kraw[k] = load16(kr, masked(wg.tok(rj, cj) + 16u * grp, f < 2 * NCH && rj < M && cj < M));
        }
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int j = wave + WV * k;
            if (k >= SETS) break;
            if (j < 2 * NCH) {                   // wave-uniform
                const int s = 16 * j + (lane >> 2);
                const int rj = s / SR, cj = s - rj * SR;
                const int piece = (lane & 3) ^ v_swizzle(s);
                dma16_at(vraw, vst_lds + (uint32_t)j * 1024u, masked(wg.tok(rj, cj) + 16u * piece, rj < M && cj < M));
            }
        }
        if (POS == SWIN_POS_TABLE) {
            // slices of the offsets ti - tj, reversed (row r at S*S - 1 - r),
            // log2 units, and their extrema
#pragma unroll
            for (int q = 0; q < QF; ++q) {
                const int tq = QF == 1 ? fb : min(fb * QF + q, Mt - 1);
                const float* trow = a.table + (size_t)(tq - tj + Mt - 1) * (S * S) * a.heads + h;
                float mx = -INFINITY, mn = INFINITY;
                for (int r = tid; r < S * S; r += WV * 64) {
                    const float val = trow[(size_t)r * a.heads] * kLog2e;
                    bias2[q * SLICE + S * S - 1 - r] = val;
                    mx = fmaxf(mx, val);
                    mn = fminf(mn, val);
                }
                mx = wave_reduce<Op::Max>(mx);
                mn = wave_reduce<Op::Min>(mn);
                if (lane == 0) { red[wave * (2 * QF + 1) + 2 * q] = mx; red[wave * (2 * QF + 1) + 2 * q + 1] = mn; }
            }
        }
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int f = wave + WV * k, c = f >> 1, t = f & 1;
            if (k >= SETS || f >= 2 * NCH) break;
            const float ss = sum_x32(sum_x16(sumsq8(kraw[k])));
            bf16x8 kfrag = __builtin_bit_cast(bf16x8, kraw[k]);
            if (SIM == SWIN_SIM_COSINE) {
                const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
                if (prec) {
                    if (grp == 0) kinv[32 * c + 8 * (li >> 2) + (li & 3) + 4 * t] = inv;
                } else {
                    float kf[8];
                    unpack_bf16x8(kraw[k], kf);
                    const float sc = inv * (kLog2e * inv_tau);
#pragma unroll
                    for (int e = 0; e < 8; ++e) kf[e] *= sc;
                    kfrag = pack_bf16x8(kf);
                }
            }
            kst[f * 64 + lane] = kfrag;
            kmax2 = fmaxf(kmax2, ss);
        }
        if (SIM == SWIN_SIM_DOT) {
            kmax2 = wave_reduce<Op::Max>(kmax2);
            if (lane == 0) red[wave * (2 * QF + 1) + 2 * QF] = kmax2;
        }
        vm_wait_all();
        __syncthreads();                         // K^, V, the slices and their extrema complete
        if (!active || tj < tlo || tj >= thi) continue;
        const float* slice = bias2 + (QF == 1 ? 0 : wave * SLICE);
        // this frame's bound on every logit of a query (log2 units) and the spread below it
        const int qs = QF == 1 ? 0 : wave;
        float bmx = 0.0f, bmn = 0.0f, kmax = 0.0f;
#pragma unroll
        for (int w = 0; w < WV; ++w) {
            if (POS == SWIN_POS_TABLE) {
                const float x = red[w * (2 * QF + 1) + 2 * qs], y = red[w * (2 * QF + 1) + 2 * qs + 1];
                bmx = w == 0 ? x : fmaxf(bmx, x);
                bmn = w == 0 ? y : fminf(bmn, y);
            }
            if (SIM == SWIN_SIM_DOT) kmax = fmaxf(kmax, red[w * (2 * QF + 1) + 2 * QF]);
        }
        kmax = sqrtf(kmax);
        bool wide = false;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const float c = SIM == SWIN_SIM_COSINE ? kLog2e * inv_tau : T[k].qnorm * kmax * T[k].qscale;
            wide = wide || !(2.0f * c + (bmx - bmn) <= RANGE_LIMIT);
        }
        const bool exact = __any(wide);
        if (!exact) {
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                // raise the reference to the frame's bound (rescale once)
                const float c = SIM == SWIN_SIM_COSINE ? kLog2e * inv_tau : T[k].qnorm * kmax * T[k].qscale;
                const float ref = fmaxf(T[k].mrun, c + bmx);
                const float alpha = __builtin_amdgcn_exp2f(T[k].mrun - ref);
                T[k].o0 *= alpha; T[k].o1 *= alpha; T[k].ls *= alpha;
                T[k].mrun = ref;
            }
        }
#pragma unroll
        for (int pp = 0; pp < TPW / 2; ++pp) {
            if (!__any(tval[2 * pp] || tval[2 * pp + 1])) continue;    // (SR = 24: tiles past the window)
            // (SR = 24: a lone tile past the frame's last runs by itself)
            if (SR != 24 || __any(tval[2 * pp + 1])) {
#pragma unroll 1
                for (int c = 0; c < NCH; ++c)
                    chunk<SIM, POS, SR, 2>(kst, vst, slice, kinv, T + 2 * pp, c, lane, S, mask, fold, prec, exact);
            } else {
#pragma unroll 1
                for (int c = 0; c < NCH; ++c)
                    chunk<SIM, POS, SR, 1>(kst, vst, slice, kinv, T + 2 * pp, c, lane, S, mask, fold, prec, exact);
            }
        }
    }

    // ---- normalise and store: lane holds channels 4 grp..+3 and 16 + 4 grp..+3 of query li
    if (!active) return;
    const Rsrc orr = make_rsrc((const uint16_t*)a.out + frame_base(tiq), bytes);
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        const int tq = QF == 1 ? wave + WV * k : k;
        const int t = tval[k] ? 16 * tq + li : 0;
        const int ri = qdiv(t, inv_M), ci = t - ri * M;
        const float inv = __builtin_amdgcn_rcpf(T[k].ls[0]);
        const uint32_t off = masked(wg.tok(ri, ci) + 8u * grp, tval[k]);
        store8(orr, off, pack_bf16x4(T[k].o0[0] * inv, T[k].o0[1] * inv, T[k].o0[2] * inv, T[k].o0[3] * inv));
        store8(orr, off + 32u, pack_bf16x4(T[k].o1[0] * inv, T[k].o1[1] * inv, T[k].o1[2] * inv, T[k].o1[3] * inv));
    }
}

size_t video_mfma_lds(int M, int SR, int pos, int QF, int WV)
{
    const int nch = video_nch(M, SR);
    size_t b = (size_t)nch * 2 * 64 * 16 + (size_t)nch * 32 * D * 2 + (size_t)nch * 32 * 4;
    if (pos == SWIN_POS_TABLE) b += (size_t)QF * video_slice(M) * 4;
    return b + (size_t)WV * (2 * QF + 1) * 4;
}

template <int SIM, int POS, int SR, bool FIT>
hipError_t launch_sr(const VideoArgs& a, int units, int per_xcd, hipStream_t s)
{
    auto* fn = attn_video_mfma_kernel<SIM, POS, SR, FIT>;
    const size_t lds = video_mfma_lds(a.M, SR, a.pos, VShape<SR>::QF, VShape<SR>::WV);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<8u * (unsigned)per_xcd, VShape<SR>::WV * 64, lds, s>>>(a, units, per_xcd);
    return hipGetLastError();
}

template <int SIM, int POS>
hipError_t launch_m(const VideoArgs& a, int units, int per_xcd, hipStream_t s)
{
    if (a.M == 8) return launch_sr<SIM, POS, 8, true>(a, units, per_xcd, s);
    if (a.M == 16) return launch_sr<SIM, POS, 16, true>(a, units, per_xcd, s);
    if (a.M < 8) return launch_sr<SIM, POS, 8, false>(a, units, per_xcd, s);
    if (a.M < 16) return launch_sr<SIM, POS, 16, false>(a, units, per_xcd, s);
    return launch_sr<SIM, POS, 24, false>(a, units, per_xcd, s);
}

}  // namespace

bool video_mfma_supported(const VideoArgs& a)
{
    return a.dtype == SWIN_DT_BF16 && a.M >= 1 && a.M <= 22 && a.C / a.heads == D &&
           (a.pos == SWIN_POS_NONE || a.pos == SWIN_POS_TABLE) &&
           (int64_t)a.H * a.W * a.C * 2 < ((int64_t)1 << 31) && (int64_t)a.W * a.C * 2 < ((int64_t)1 << 24);
}

hipError_t launch_attn_video_mfma(const VideoArgs& a, hipStream_t stream)
{
    if (a.nwin == 0) return hipSuccess;
    const int qf = a.M <= 8 ? 4 : 1;
    const int64_t units = (int64_t)a.nwin * a.heads * ((a.Mt + qf - 1) / qf);
    if (units > INT32_MAX - 8) return hipErrorInvalidValue;
    const int per_xcd = (int)((units + 7) / 8);
    if (a.sim == SWIN_SIM_COSINE)
        return a.pos == SWIN_POS_TABLE ? launch_m<SWIN_SIM_COSINE, SWIN_POS_TABLE>(a, (int)units, per_xcd, stream)
                                       : launch_m<SWIN_SIM_COSINE, SWIN_POS_NONE>(a, (int)units, per_xcd, stream);
    return a.pos == SWIN_POS_TABLE ? launch_m<SWIN_SIM_DOT, SWIN_POS_TABLE>(a, (int)units, per_xcd, stream)
                                   : launch_m<SWIN_SIM_DOT, SWIN_POS_NONE>(a, (int)units, per_xcd, stream);
}

}  // namespace swin
