// Backward of window attention on the vector ALUs, any dtype, windows of up
// to 64 x 64 tokens whose per-query statistics and table fit LDS.
//
// The forward is the SwinV2 card's eq. 1-2 with the log-CPB table of eq. 3-4,
// cyclic-shift or interleaved windows, and the FlashSwin abstract's
// window-local rotary variant.  Its gradient, per (window, head), with
// p = softmax of the logits over the query's shift region:
//   dv_j  = sum_i p_ij dout_i
//   dl_ij = p_ij (dout_i . v_j - D_i),  D_i = dout_i . out_i
//   TABLE: dtable[offset(i, j)] += dl_ij
//   COSINE (logit = q^.k^ / tau' + b): dq^_i = sum_j dl_ij k^_j / tau',
//          dk^_j = sum_i dl_ij q^_i / tau', dtau += sum dl_ij cos_ij (-1/tau^2)
//          while tau > tau_min; through x^ = x / max(||x||, eps):
//          dx = (dx^ - x^ (x^ . dx^)) / ||x||;
//   DOT (logit = q.k / sqrt(d) + b): the same with the raw operands;
//   ROPE2D: dx = R(-pos) dx~ (the rotation is orthogonal).
// One workgroup per (window, head), 256 threads.  Queries, 256 at a time,
// one per thread: a first sweep over the keys finds the row maximum and sum
// (online), a second forms p and dl and accumulates dq, dtau and the bias
// gradient (LDS atomics into the workgroup's copy of the table column).
// Then keys, one per thread: a sweep over the queries accumulates dk and dv
// from the row statistics the first phase left in LDS.  Keys (or queries)
// and values (or output gradients) pass through LDS in blocks of 128 and are
// read by every thread as broadcasts.  All arithmetic is fp32.
#include "common.hpp"
#include "lanes.hpp"
#include "launch.hpp"
#include "launch_bwd.hpp"

namespace swin {

namespace {

constexpr int D = 32;
constexpr int BLK = 128;       // keys or queries per LDS block
constexpr int TPB = 256;       // threads: queries or keys per round

template <typename T> __device__ __forceinline__ void load_row(const T* p, float* f);
template <> __device__ __forceinline__ void load_row<float>(const float* p, float* f)
{
    const float4* v = (const float4*)p;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
        const float4 x = v[i];
        f[4 * i] = x.x; f[4 * i + 1] = x.y; f[4 * i + 2] = x.z; f[4 * i + 3] = x.w;
    }
}
template <> __device__ __forceinline__ void load_row<uint16_t>(const uint16_t* p, float* f)
{
    const u32x4* v = (const u32x4*)p;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) unpack_bf16x8(v[i], f + 8 * i);
}

template <typename T> __device__ __forceinline__ void store_row(T* p, const float* f);
template <> __device__ __forceinline__ void store_row<float>(float* p, const float* f)
{
    float4* v = (float4*)p;
#pragma unroll
    for (int i = 0; i < D / 4; ++i) v[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
}
template <> __device__ __forceinline__ void store_row<uint16_t>(uint16_t* p, const float* f)
{
    bf16x8* v = (bf16x8*)p;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) v[i] = pack_bf16x8(f + 8 * i);
}

// Rotate channel pairs by sgn * the window-local position: [0, D/2) by row r,
// [D/2, D) by column c; cs/sn tables are [pos][half][D/4].  sgn = -1 applies
// the transpose.
__device__ __forceinline__ void rope_apply(float* x, int r, int c, const float* cs, const float* sn, float sgn)
{
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int pos = half == 0 ? r : c;
#pragma unroll
        for (int k = 0; k < D / 4; ++k) {
            const float co = cs[(pos * 2 + half) * (D / 4) + k];
            const float si = sgn * sn[(pos * 2 + half) * (D / 4) + k];
            const float x0 = x[half * (D / 2) + 2 * k], x1 = x[half * (D / 2) + 2 * k + 1];
            x[half * (D / 2) + 2 * k] = x0 * co - x1 * si;
            x[half * (D / 2) + 2 * k + 1] = x0 * si + x1 * co;
        }
    }
}

// Operand of the logits for one token's head slice: rotated (ROPE2D), then
// unit-normalised (COSINE); nrm receives max(||x||, eps) of the rotated x.
template <typename T, int SIM, int POS>
__device__ __forceinline__ void operand(const T* src, int r, int c, const float* cs, const float* sn, float* x,
                                        float& nrm)
{
    load_row<T>(src, x);
    if (POS == SWIN_POS_ROPE2D) rope_apply(x, r, c, cs, sn, 1.0f);
    nrm = 1.0f;
    if (SIM == SWIN_SIM_COSINE) {
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < D; ++e) ss = fmaf(x[e], x[e], ss);
        nrm = fmaxf(sqrtf(ss), 1e-12f);
        const float inv = 1.0f / nrm;
#pragma unroll
        for (int e = 0; e < D; ++e) x[e] *= inv;
    }
}

// Gradient of the logit operand back to the token's input slice, in place:
// through the normalisation (COSINE) and the rotation (ROPE2D).
template <int SIM, int POS>
__device__ __forceinline__ void operand_bwd(float* g, const float* xh, float nrm, int r, int c, const float* cs,
                                            const float* sn)
{
    if (SIM == SWIN_SIM_COSINE) {
        float proj = 0.0f;
#pragma unroll
        for (int e = 0; e < D; ++e) proj = fmaf(xh[e], g[e], proj);
        const float inv = 1.0f / nrm;
        // below the floor the normalisation is x / eps: no projection
        const float pr = nrm > 1e-12f ? proj : 0.0f;
#pragma unroll
        for (int e = 0; e < D; ++e) g[e] = (g[e] - xh[e] * pr) * inv;
    }
    if (POS == SWIN_POS_ROPE2D) rope_apply(g, r, c, cs, sn, -1.0f);
}

struct BwdArgs {
    const void* out;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* dtau;               // heads, or NULL
    float* dtable;             // (2M-1)^2 x heads, or NULL
};

template <typename T, int SIM, int POS>
__global__ void __launch_bounds__(TPB)
attn_bwd_kernel(AttnParams p, BwdArgs a)
{
    extern __shared__ float sm[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1;
    const int h = blockIdx.y;
    const int win = blockIdx.x;
    const int tid = threadIdx.x;
    const bool want_table = POS == SWIN_POS_TABLE && a.dtable != nullptr;

    float* kb = sm;                                   // [BLK][D] key (query) operands
    float* vb = kb + BLK * D;                         // [BLK][D] values (output gradients)
    float* st_m = vb + BLK * D;                       // [N] row maximum of the logits
    float* st_il = st_m + N;                          // [N] 1 / row sum
    float* st_d = st_il + N;                          // [N] dout . out
    float* bias = st_d + N;                           // [S*S] (TABLE)
    float* dtab = bias + (POS == SWIN_POS_TABLE ? S * S : 0);     // [S*S] (TABLE)
    float* cs = dtab + (POS == SWIN_POS_TABLE ? S * S : 0);       // [M][2][D/4] (ROPE2D)
    float* sn = cs + (POS == SWIN_POS_ROPE2D ? M * D / 2 : 0);
    float* red = sn + (POS == SWIN_POS_ROPE2D ? M * D / 2 : 0);   // [TPB / 64]

    if (POS == SWIN_POS_TABLE)
        for (int i = tid; i < S * S; i += TPB) { bias[i] = p.table[(size_t)i * g.heads + h]; dtab[i] = 0.0f; }
    if (POS == SWIN_POS_ROPE2D) {
        for (int i = tid; i < M * 2 * (D / 4); i += TPB) {
            const int k = i % (D / 4), half = (i / (D / 4)) % 2, pos = i / (D / 2);
            const double th = p.rope_freqs
                ? (double)p.rope_freqs[((size_t)h * 2 + half) * (D / 4) + k]
                : pow((double)p.rope_base, -(double)k / (double)(D / 4));
            double s_, c_;
            sincos((double)pos * th, &s_, &c_);
            cs[i] = (float)c_;
            sn[i] = (float)s_;
        }
    }
    __syncthreads();

    const T* qg = (const T*)p.q;
    const T* kg = (const T*)p.k;
    const T* vg = (const T*)p.v;
    const T* og = (const T*)a.out;
    const T* dog = (const T*)a.dout;
    const int nW = g.nwr * g.nwc;
    const int wloc = win % nW;
    const int wr = wloc / g.nwc, wc = wloc % g.nwc;
    const bool shifted = g.part == SWIN_PART_CYCLIC && g.shift > 0;
    float tau = 1.0f, scale = 0.17677669529663687f;       // DOT: 1/sqrt(32)
    if (SIM == SWIN_SIM_COSINE) {
        tau = fmaxf(p.tau[h], p.tau_min);
        scale = 1.0f / tau;
    }
    float dtau_acc = 0.0f;

    // ---- queries: row statistics, then dq, dtau, dtable
    for (int q0 = 0; q0 < N; q0 += TPB) {
        const int i = q0 + tid;
        const bool valid = i < N;
        const int ri = valid ? i / M : 0, ci = valid ? i - (i / M) * M : 0;
        float qh[D], go[D], nq = 1.0f, Di = 0.0f;
        if (valid) {
            const int64_t off = token_offset(g, win, ri, ci) + h * D;
            operand<T, SIM, POS>(qg + off, ri, ci, cs, sn, qh, nq);
            float o[D];
            load_row<T>(og + off, o);
            load_row<T>(dog + off, go);
#pragma unroll
            for (int e = 0; e < D; ++e) Di = fmaf(go[e], o[e], Di);
        }
        int rlo = 0, rhi = M, clo = 0, chi = M;
        if (shifted) {
            region_interval(wr, g.nwr, M, g.shift, ri, rlo, rhi);
            region_interval(wc, g.nwc, M, g.shift, ci, clo, chi);
        }
        float m = -INFINITY, l = 0.0f;
        float dqh[D];
#pragma unroll
        for (int e = 0; e < D; ++e) dqh[e] = 0.0f;
        for (int sweep = 0; sweep < 2; ++sweep) {
            const float il = 1.0f / l;
            for (int j0 = 0; j0 < N; j0 += BLK) {
                const int cnt = min(BLK, N - j0);
                __syncthreads();
                if (tid < cnt) {
                    const int j = j0 + tid, rj = j / M, cj = j - rj * M;
                    float x[D], nk;
                    operand<T, SIM, POS>(kg + token_offset(g, win, rj, cj) + h * D, rj, cj, cs, sn, x, nk);
#pragma unroll
                    for (int e = 0; e < D; ++e) kb[tid * D + e] = x[e];
                } else if (sweep == 1 && tid >= BLK && tid - BLK < cnt) {
                    const int j = j0 + tid - BLK, rj = j / M, cj = j - rj * M;
                    float x[D];
                    load_row<T>(vg + token_offset(g, win, rj, cj) + h * D, x);
#pragma unroll
                    for (int e = 0; e < D; ++e) vb[(tid - BLK) * D + e] = x[e];
                }
                __syncthreads();
                if (!valid) continue;
                for (int jj = 0; jj < cnt; ++jj) {
                    const int j = j0 + jj, rj = j / M, cj = j - rj * M;
                    if (rj < rlo || rj >= rhi || cj < clo || cj >= chi) continue;
                    const float* kr = kb + jj * D;
                    float s = 0.0f;
#pragma unroll
                    for (int e = 0; e < D; ++e) s = fmaf(qh[e], kr[e], s);
                    const int bidx = (ri - rj + M - 1) * S + (ci - cj + M - 1);
                    float x = s * scale;
                    if (POS == SWIN_POS_TABLE) x += bias[bidx];
                    if (sweep == 0) {
                        if (x > m) { l = l * expf(m - x) + 1.0f; m = x; }
                        else l += expf(x - m);
                        continue;
                    }
                    const float pj = expf(x - m) * il;
                    const float* vr = vb + jj * D;
                    float dp = 0.0f;
#pragma unroll
                    for (int e = 0; e < D; ++e) dp = fmaf(go[e], vr[e], dp);
                    const float dl = pj * (dp - Di);
                    const float ds = dl * scale;
#pragma unroll
                    for (int e = 0; e < D; ++e) dqh[e] = fmaf(ds, kr[e], dqh[e]);
                    if (SIM == SWIN_SIM_COSINE) dtau_acc = fmaf(dl, s, dtau_acc);
                    if (want_table) atomicAdd(&dtab[bidx], dl);
                }
            }
        }
        if (valid) {
            operand_bwd<SIM, POS>(dqh, qh, nq, ri, ci, cs, sn);
            store_row<T>((T*)a.dq + token_offset(g, win, ri, ci) + h * D, dqh);
            st_m[i] = m;
            st_il[i] = 1.0f / l;
            st_d[i] = Di;
        }
    }

    // ---- keys: dk, dv from the row statistics
    for (int k0 = 0; k0 < N; k0 += TPB) {
        const int j = k0 + tid;
        const bool valid = j < N;
        const int rj = valid ? j / M : 0, cj = valid ? j - (j / M) * M : 0;
        float kh[D], vj[D], nk = 1.0f;
        if (valid) {
            const int64_t off = token_offset(g, win, rj, cj) + h * D;
            operand<T, SIM, POS>(kg + off, rj, cj, cs, sn, kh, nk);
            load_row<T>(vg + off, vj);
        }
        int rlo = 0, rhi = M, clo = 0, chi = M;
        if (shifted) {
            region_interval(wr, g.nwr, M, g.shift, rj, rlo, rhi);
            region_interval(wc, g.nwc, M, g.shift, cj, clo, chi);
        }
        float dkh[D], dvj[D];
#pragma unroll
        for (int e = 0; e < D; ++e) { dkh[e] = 0.0f; dvj[e] = 0.0f; }
        for (int i0 = 0; i0 < N; i0 += BLK) {
            const int cnt = min(BLK, N - i0);
            __syncthreads();
            if (tid < cnt) {
                const int i = i0 + tid, ri = i / M, ci = i - ri * M;
                float x[D], nq;
                operand<T, SIM, POS>(qg + token_offset(g, win, ri, ci) + h * D, ri, ci, cs, sn, x, nq);
#pragma unroll
                for (int e = 0; e < D; ++e) kb[tid * D + e] = x[e];
            } else if (tid >= BLK && tid - BLK < cnt) {
                const int i = i0 + tid - BLK, ri = i / M, ci = i - ri * M;
                float x[D];
                load_row<T>(dog + token_offset(g, win, ri, ci) + h * D, x);
#pragma unroll
                for (int e = 0; e < D; ++e) vb[(tid - BLK) * D + e] = x[e];
            }
            __syncthreads();
            if (!valid) continue;
            for (int ii = 0; ii < cnt; ++ii) {
                const int i = i0 + ii, ri = i / M, ci = i - ri * M;
                if (ri < rlo || ri >= rhi || ci < clo || ci >= chi) continue;
                const float* qr = kb + ii * D;
                const float* gr = vb + ii * D;
                float s = 0.0f, dp = 0.0f;
#pragma unroll
                for (int e = 0; e < D; ++e) { s = fmaf(qr[e], kh[e], s); dp = fmaf(gr[e], vj[e], dp); }
                float x = s * scale;
                if (POS == SWIN_POS_TABLE) x += bias[(ri - rj + M - 1) * S + (ci - cj + M - 1)];
                const float pj = expf(x - st_m[i]) * st_il[i];
                const float ds = pj * (dp - st_d[i]) * scale;
#pragma unroll
                for (int e = 0; e < D; ++e) { dvj[e] = fmaf(pj, gr[e], dvj[e]); dkh[e] = fmaf(ds, qr[e], dkh[e]); }
            }
        }
        if (valid) {
            operand_bwd<SIM, POS>(dkh, kh, nk, rj, cj, cs, sn);
            const int64_t off = token_offset(g, win, rj, cj) + h * D;
            store_row<T>((T*)a.dk + off, dkh);
            store_row<T>((T*)a.dv + off, dvj);
        }
    }

    // ---- this window's share of dtau and of the bias-table gradient
    if (SIM == SWIN_SIM_COSINE && a.dtau) {
        const float s = lanes::wave_reduce<lanes::Op::Sum>(dtau_acc);
        if ((tid & 63) == 0) red[tid >> 6] = s;
    }
    __syncthreads();
    if (SIM == SWIN_SIM_COSINE && a.dtau && tid == 0 && p.tau[h] > p.tau_min) {
        float s = 0.0f;
        for (int w = 0; w < TPB / 64; ++w) s += red[w];
        unsafeAtomicAdd(&a.dtau[h], s * (-1.0f / (p.tau[h] * p.tau[h])));
    }
    if (want_table)
        for (int i = tid; i < S * S; i += TPB)
            if (dtab[i] != 0.0f) unsafeAtomicAdd(&a.dtable[(size_t)i * g.heads + h], dtab[i]);
}

__global__ void zero_kernel(float* a, int n, float* b, int nb)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (a && i < n) a[i] = 0.0f;
    if (b && i < nb) b[i] = 0.0f;
}

template <typename T, int SIM>
hipError_t dispatch_pos(const AttnParams& p, const BwdArgs& a, dim3 grid, size_t lds, hipStream_t s)
{
    auto* fn = p.pos == SWIN_POS_NONE  ? attn_bwd_kernel<T, SIM, SWIN_POS_NONE>
             : p.pos == SWIN_POS_TABLE ? attn_bwd_kernel<T, SIM, SWIN_POS_TABLE>
                                       : attn_bwd_kernel<T, SIM, SWIN_POS_ROPE2D>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<grid, TPB, lds, s>>>(p, a);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_sim(const AttnParams& p, const BwdArgs& a, dim3 grid, size_t lds, hipStream_t s)
{
    if (p.sim == SWIN_SIM_COSINE) return dispatch_pos<T, SWIN_SIM_COSINE>(p, a, grid, lds, s);
    return dispatch_pos<T, SWIN_SIM_DOT>(p, a, grid, lds, s);
}

}  // namespace

// LDS of the vector-ALU kernel: two operand blocks, three per-query
// statistics, and the table and its gradient (TABLE) or the angles (ROPE2D)
size_t attn_bwd_lds(const AttnParams& p)
{
    const int S = 2 * p.g.M - 1;
    size_t lds = (size_t)(2 * BLK * D + 3 * p.g.N + TPB / 64) * sizeof(float);
    if (p.pos == SWIN_POS_TABLE) lds += (size_t)2 * S * S * sizeof(float);
    if (p.pos == SWIN_POS_ROPE2D) lds += (size_t)p.g.M * D * sizeof(float);
    return lds;
}

bool attn_bwd_supported(const AttnParams& p)
{
    return p.g.d == D && p.g.M <= 64 && attn_bwd_lds(p) <= 160 * 1024;
}

hipError_t launch_attn_bwd(const AttnParams& p, const void* out, const void* dout, void* dq, void* dk, void* dv,
                           float* dtau, float* dtable, hipStream_t stream)
{
    const Geometry& g = p.g;
    const int S = 2 * g.M - 1;
    BwdArgs a{out, dout, dq, dk, dv, p.sim == SWIN_SIM_COSINE ? dtau : nullptr,
              p.pos == SWIN_POS_TABLE ? dtable : nullptr};
    // the gradients that are sums over windows start from zero (a kernel,
    // not a memset, so that the call can be captured in a graph)
    const int nt = a.dtable ? S * S * g.heads : 0, nh = a.dtau ? g.heads : 0;
    if (nt || nh) {
        zero_kernel<<<(max(nt, nh) + 255) / 256, 256, 0, stream>>>(a.dtable, nt, a.dtau, nh);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (g.nwin == 0) return hipSuccess;
    if (attn_bwd_small_supported(p))
        return launch_attn_bwd_small(p, out, dout, dq, dk, dv, a.dtau, a.dtable, stream);
    if (attn_bwd_large_supported(p))
        return launch_attn_bwd_large(p, out, dout, dq, dk, dv, a.dtau, a.dtable, stream);
    const size_t lds = attn_bwd_lds(p);
    dim3 grid(g.nwin, g.heads);
    if (p.dtype == SWIN_DT_F32) return dispatch_sim<float>(p, a, grid, lds, stream);
    return dispatch_sim<uint16_t>(p, a, grid, lds, stream);
}

}  // namespace swin
