// Device code shared by the small-window attention kernels (attn_small.hip,
// attn_fused.hip): the per-pair query tile state and the loop of a pair of
// query tiles over the key chunks of a window staged in LDS (the two
// products on the matrix cores, the softmax in registers between them).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "lanes.hpp"
#include "tile_io.hpp"

namespace swin {
namespace core {

using namespace tio;
using namespace lanes;

constexpr int WAVES = 4;
constexpr float RANGE_LIMIT = 60.0f;
constexpr float PRECISE_TAU = 0.1f;

__device__ __forceinline__ float load_f32(Rsrc r, uint32_t off)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum of squares of 8 bf16 values (v_dot2_f32_bf16: products exact in fp32)
__device__ __forceinline__ float sumsq8(const u32x4 w)
{
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t wi = w[i];         // bit_cast of the subscript itself reads element 0
        const bf16x2 v = __builtin_bit_cast(bf16x2, wi);
        s = __builtin_amdgcn_fdot2_f32_bf16(v, v, s, false);
    }
    return s;
}

struct Tile {                  // one query tile of 16 queries
    bf16x8 qf;
    float qscale, negm, mrun;
    float cinit;               // S^T accumulator start: qscale * cinit is the softmax shift
    int qoff;                  // bias-table offset of this lane's query and key group
    uint32_t gmask;            // chunks whose key group of this lane is allowed (bit c)
    uint32_t colbits;          // allowed columns of this lane's key group (bit e)
    bool exact;
    f32x4 o0, o1, ls;
};

// NT (one or two) query tiles against key chunks [CB, CE) of the window
// (the others are masked for all of them); K^ fragments and V rows come
// from LDS.
// The key group of a lane in chunk c starts (4 / GPR) c rows further down
// the window than in chunk 0: its bias row moves by that many table rows.
//   MASK: shift regions / padded slots; PRECISE: scores scaled by 1/||k_j||
//   (raw k operand); EXACT: running maximum instead of the static shift.
//   SPLIT (with PRECISE): q and k are hi + lo bf16 pairs (klo: the keys'
//   remainders in K^'s layout, qlo: the tiles' remainders), S^T takes the
//   three products hi hi, lo hi, hi lo.
template <int SIM, int POS, int GPR, int CB, int CE, bool MASK, bool PRECISE, bool EXACT, int NT, bool SPLIT = false>
__device__ __forceinline__ void run_pair(const bf16x8* kst, const __bf16* vst, Tile* T, const float* bias2,
                                         const float* kinv, int S, int negrow, int lane, bool partial_any,
                                         bool precise_rt, const bf16x8* klo = nullptr, const bf16x8* qlo = nullptr)
{
    const int grp = lane >> 4, li = lane & 15;
    const bool prec = PRECISE && precise_rt;
    // COSINE outside the precise path: k^ carries log2(e)/tau and q its unit
    // norm, the table (or -log2(e)/tau) starts the accumulator, so S^T holds
    // the shifted logits in log2 units and goes to exp2 as it is
    const bool fold = SIM == SWIN_SIM_COSINE && !prec;
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
    // the running-maximum variant stays rolled: its registers are not to
    // set the kernel's occupancy
    constexpr int UNROLL = EXACT ? 1 : CE - CB;
#pragma unroll UNROLL
    for (int c = CB; c < CE; ++c) {
        const bf16x8 ka = kst[(c * 2 + 0) * 64 + lane];
        const bf16x8 kb = kst[(c * 2 + 1) * 64 + lane];
        uint32_t bits[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) bits[i] = 0xffu;
        if (MASK) {
#pragma unroll
            for (int i = 0; i < NT; ++i) bits[i] = (T[i].gmask >> c) & 1u ? T[i].colbits : 0u;
        }
        float kin[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
        if (prec) {
            const f32x4 a = *(const f32x4*)(kinv + 32 * c + 8 * grp);
            const f32x4 b = *(const f32x4*)(kinv + 32 * c + 8 * grp + 4);
            kin[0] = a[0]; kin[1] = a[1]; kin[2] = a[2]; kin[3] = a[3];
            kin[4] = b[0]; kin[5] = b[1]; kin[6] = b[2]; kin[7] = b[3];
        }
        float add[NT][8];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            if (POS == SWIN_POS_TABLE) {
                const float* bp = bias2 + ((MASK && bits[i] == 0u) ? negrow : T[i].qoff + (4 / GPR) * c * S);
#pragma unroll
                for (int e = 0; e < 8; ++e) add[i][e] = bp[e];
            } else {
                const float a = (MASK && bits[i] == 0u) ? -INFINITY : T[i].negm;
#pragma unroll
                for (int e = 0; e < 8; ++e) add[i][e] = a;
            }
        }
        f32x4 sa[NT], sb[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const f32x4 c4 = {T[i].cinit, T[i].cinit, T[i].cinit, T[i].cinit};
            const f32x4 ia = {add[i][0], add[i][1], add[i][2], add[i][3]};
            const f32x4 ib = {add[i][4], add[i][5], add[i][6], add[i][7]};
            sa[i] = mfma(ka, T[i].qf, fold ? ia : c4);
            sb[i] = mfma(kb, T[i].qf, fold ? ib : c4);
            if (SPLIT && prec) {
                const bf16x8 ka_lo = klo[(c * 2 + 0) * 64 + lane];
                const bf16x8 kb_lo = klo[(c * 2 + 1) * 64 + lane];
                sa[i] = mfma(ka_lo, T[i].qf, sa[i]);
                sb[i] = mfma(kb_lo, T[i].qf, sb[i]);
                sa[i] = mfma(ka, qlo[i], sa[i]);
                sb[i] = mfma(kb, qlo[i], sb[i]);
            }
        }
        const bf16x8 v0 = vt_frag(vst, c, 0, grp, li);
        const bf16x8 v1 = vt_frag(vst, c, 1, grp, li);
        bf16x8 pb[NT];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[e] = sa[i][e]; x[e + 4] = sb[i][e]; }
            float sc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] = prec ? T[i].qscale * kin[e] : T[i].qscale;
            float pr[8];
            if (!EXACT || !T[i].exact) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pr[e] = __builtin_amdgcn_exp2f(fold ? x[e] : fmaf(x[e], sc[e], add[i][e]));
                if (MASK && partial_any) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) pr[e] = (bits[i] >> e) & 1u ? pr[e] : 0.0f;
                }
            } else {
                float xs[8], cm = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xs[e] = fold ? x[e] : fmaf(x[e], sc[e], add[i][e]);
                    if (MASK) xs[e] = (bits[i] >> e) & 1u ? xs[e] : -INFINITY;
                    cm = fmaxf(cm, xs[e]);
                }
                cm = max_x32(max_x16(cm));
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
        for (int i = 0; i < NT; ++i) {
            T[i].o0 = mfma(v0, pb[i], T[i].o0);
            T[i].o1 = mfma(v1, pb[i], T[i].o1);
            T[i].ls = mfma(ones, pb[i], T[i].ls);
        }
    }
}

// A pair of query tiles over a window with shift regions or padded slots:
// only the chunks some lane of the pair may see (all, or one half of the key
// rows), and a loop of its own for windows whose region edges fall on 8-slot
// group boundaries (partial false), which then needs no per-key selects.
// partial must be uniform over the wavefront.
template <int SIM, int POS, int GPR, int NCH>
__device__ __forceinline__ void run_masked_pair(const bf16x8* kst, const __bf16* vst, Tile* T, const float* bias2,
                                                const float* kinv, int S, int negrow, int lane, bool partial)
{
    uint32_t live = T[0].gmask | T[1].gmask;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) live |= (uint32_t)__shfl_xor((int)live, o);
    live = (uint32_t)__builtin_amdgcn_readfirstlane((int)live);
    constexpr uint32_t lo_half = (1u << (NCH / 2)) - 1u;
    auto go = [&](auto part) {
        constexpr bool PART = decltype(part)::value;
        if ((live & ~lo_half) == 0u)
            run_pair<SIM, POS, GPR, 0, NCH / 2, true, false, false, 2>(kst, vst, T, bias2, kinv, S, negrow, lane,
                                                                    PART, false);
        else if ((live & lo_half) == 0u)
            run_pair<SIM, POS, GPR, NCH / 2, NCH, true, false, false, 2>(kst, vst, T, bias2, kinv, S, negrow, lane,
                                                                      PART, false);
        else
            run_pair<SIM, POS, GPR, 0, NCH, true, false, false, 2>(kst, vst, T, bias2, kinv, S, negrow, lane, PART,
                                                                false);
    };
    if (__builtin_amdgcn_readfirstlane((int)partial))
        go(std::integral_constant<bool, true>());
    else
        go(std::integral_constant<bool, false>());
}

}  // namespace core
}  // namespace swin
