// Window attention on the vector ALUs for fp32 tensors.
//
// This is the path for SWIN_DT_F32, where bf16 matrix-core operands would
// not reach fp32 accuracy.  One workgroup per (window, head); its threads
// take up to 512 queries at a time, one query each, keeping q, the running
// row max, the running sum and the fp32 output accumulator in registers (the
// online normaliser of Milakov & Gimelshein) while key/value chunks are
// staged through LDS and read by every thread as broadcasts.  The N x N
// scores are never stored.  The similarity and the logit are evaluated in
// fp64 (q.k, the norms, 1/tau, the bias): with tau at its 0.01 floor a logit
// reaches 100, and an fp32 dot product would already err by ~1e-5 there.
// Exponentials, the value accumulation and all storage are fp32.  Steps, in the SwinV2 card's order (eq. 1-2 and its
// window-attention pseudocode; FlashSwin abstract for the rotary variant):
// rotate q, k by their window-local (row, column) for ROPE2D; unit-normalise
// q and k for COSINE and divide by max(tau, tau_min), or scale q.k by
// 1/sqrt(d) for DOT; add the relative-position bias for TABLE; drop keys of
// another shift region; softmax; weighted sum of v.
#include "common.hpp"
#include "launch.hpp"
#include "rows.hpp"

namespace swin {

namespace {

constexpr int D = 32;
constexpr int KC_MAX = 256;   // keys per LDS chunk

// Rotate channel pairs by the window-local position: [0, D/2) by row r,
// [D/2, D) by column c; cs/sn tables are [pos][half][D/4].
__device__ __forceinline__ void rope_apply(float* x, int r, int c, const float* cs, const float* sn)
{
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int pos = half == 0 ? r : c;
#pragma unroll
        for (int k = 0; k < D / 4; ++k) {
            const float co = cs[(pos * 2 + half) * (D / 4) + k];
            const float si = sn[(pos * 2 + half) * (D / 4) + k];
            const float x0 = x[half * (D / 2) + 2 * k], x1 = x[half * (D / 2) + 2 * k + 1];
            x[half * (D / 2) + 2 * k] = x0 * co - x1 * si;
            x[half * (D / 2) + 2 * k + 1] = x0 * si + x1 * co;
        }
    }
}

template <typename T, int SIM, int POS>
__global__ void __launch_bounds__(512)
attn_valu_kernel(AttnParams p, int kc)
{
    extern __shared__ double smem_d[];
    const Geometry& g = p.g;
    const int M = g.M, N = g.N, S = 2 * M - 1;
    const int h = blockIdx.y;
    const int win = blockIdx.x;
    const int tid = threadIdx.x;

    double* kinv = smem_d;                             // [kc] 1/||k|| (COSINE)
    float* ks = (float*)(kinv + kc);                   // [kc][D]
    float* vs = ks + kc * D;                           // [kc][D]
    float* bias = vs + kc * D;                         // [S*S]        (TABLE)
    float* cs = bias + (POS == SWIN_POS_TABLE ? S * S : 0);   // [M][2][D/4] (ROPE2D)
    float* sn = cs + (POS == SWIN_POS_ROPE2D ? M * D / 2 : 0);

    if (POS == SWIN_POS_TABLE)
        for (int i = tid; i < S * S; i += blockDim.x) bias[i] = p.table[(size_t)i * g.heads + h];
    if (POS == SWIN_POS_ROPE2D) {
        // angles pos * theta in double, rounded once to fp32 cos/sin
        for (int i = tid; i < M * 2 * (D / 4); i += blockDim.x) {
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
    T* og = (T*)p.out;
    const int nW = g.nwr * g.nwc;
    const int wloc = win % nW;
    const int wr = wloc / g.nwc, wc = wloc % g.nwc;
    const bool shifted = g.part == SWIN_PART_CYCLIC && g.shift > 0;

    for (int q0 = 0; q0 < N; q0 += blockDim.x) {
        const int t = q0 + tid;
        const bool valid = t < N;
        const int ri = valid ? t / M : 0, ci = valid ? t % M : 0;
        float q[D], acc[D];
        double scale = 0.0;
        if (valid) {
            load_row32<T>(qg + token_offset(g, win, ri, ci) + h * D, q);
            if (POS == SWIN_POS_ROPE2D) rope_apply(q, ri, ci, cs, sn);
            if (SIM == SWIN_SIM_COSINE) {
                double ss = 0.0;
#pragma unroll
                for (int e = 0; e < D; ++e) ss = fma((double)q[e], (double)q[e], ss);
                const double tau = fmax((double)p.tau[h], (double)p.tau_min);
                scale = 1.0 / (tau * fmax(sqrt(ss), 1e-12));
            } else {
                scale = 1.0 / sqrt((double)D);
            }
        }
        int rlo = 0, rhi = M, clo = 0, chi = M;
        if (shifted) {
            region_interval(wr, g.nwr, M, g.shift, ri, rlo, rhi);
            region_interval(wc, g.nwc, M, g.shift, ci, clo, chi);
        }
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] = 0.0f;
        double m = -INFINITY;
        float l = 0.0f;

        for (int j0 = 0; j0 < N; j0 += kc) {
            const int cnt = min(kc, N - j0);
            __syncthreads();
            if (tid < cnt) {
                const int j = j0 + tid, rj = j / M, cj = j % M;
                float kr[D], vr[D];
                const int64_t off = token_offset(g, win, rj, cj) + h * D;
                load_row32<T>(kg + off, kr);
                load_row32<T>(vg + off, vr);
                if (POS == SWIN_POS_ROPE2D) rope_apply(kr, rj, cj, cs, sn);
                if (SIM == SWIN_SIM_COSINE) {
                    double ss = 0.0;
#pragma unroll
                    for (int e = 0; e < D; ++e) ss = fma((double)kr[e], (double)kr[e], ss);
                    kinv[tid] = 1.0 / fmax(sqrt(ss), 1e-12);
                }
#pragma unroll
                for (int e = 0; e < D; ++e) { ks[tid * D + e] = kr[e]; vs[tid * D + e] = vr[e]; }
            }
            __syncthreads();
            if (valid) {
                for (int jj = 0; jj < cnt; ++jj) {
                    const int j = j0 + jj, rj = j / M, cj = j - rj * M;
                    if (rj < rlo || rj >= rhi || cj < clo || cj >= chi) continue;
                    const float* kr = ks + jj * D;
                    double s = 0.0;
#pragma unroll
                    for (int e = 0; e < D; ++e) s = fma((double)q[e], (double)kr[e], s);
                    double x = s * scale;
                    if (SIM == SWIN_SIM_COSINE) x *= kinv[jj];
                    if (POS == SWIN_POS_TABLE) x += (double)bias[(ri - rj + M - 1) * S + (ci - cj + M - 1)];
                    const float* vr = vs + jj * D;
                    if (x > m) {
                        const float a = expf((float)(m - x));      // 0 on the first key
                        l = fmaf(l, a, 1.0f);
#pragma unroll
                        for (int e = 0; e < D; ++e) acc[e] = fmaf(acc[e], a, vr[e]);
                        m = x;
                    } else {
                        const float pj = expf((float)(x - m));
                        l += pj;
#pragma unroll
                        for (int e = 0; e < D; ++e) acc[e] = fmaf(pj, vr[e], acc[e]);
                    }
                }
            }
        }
        if (valid) {
            const float inv = 1.0f / l;
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] *= inv;
            store_row32<T>(og + token_offset(g, win, ri, ci) + h * D, acc);
            if (p.lse) p.lse[((size_t)win * g.heads + h) * N + t] = (float)(m + log((double)l));
        }
    }
}

template <typename T, int SIM>
hipError_t dispatch_pos(const AttnParams& p, dim3 grid, int threads, int kc, size_t lds, hipStream_t s)
{
    auto* fn = p.pos == SWIN_POS_NONE  ? attn_valu_kernel<T, SIM, SWIN_POS_NONE>
             : p.pos == SWIN_POS_TABLE ? attn_valu_kernel<T, SIM, SWIN_POS_TABLE>
                                       : attn_valu_kernel<T, SIM, SWIN_POS_ROPE2D>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<grid, threads, lds, s>>>(p, kc);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_sim(const AttnParams& p, dim3 grid, int threads, int kc, size_t lds, hipStream_t s)
{
    if (p.sim == SWIN_SIM_COSINE) return dispatch_pos<T, SWIN_SIM_COSINE>(p, grid, threads, kc, lds, s);
    return dispatch_pos<T, SWIN_SIM_DOT>(p, grid, threads, kc, lds, s);
}

}  // namespace

hipError_t launch_attn_valu(const AttnParams& p, hipStream_t stream)
{
    const Geometry& g = p.g;
    if (g.nwin == 0) return hipSuccess;
    int threads = ((g.N + 63) / 64) * 64;
    if (threads > 512) threads = 512;
    const int kc = threads < KC_MAX ? threads : KC_MAX;
    const int S = 2 * g.M - 1;
    size_t lds = (size_t)kc * sizeof(double) + (size_t)2 * kc * D * sizeof(float);
    if (p.pos == SWIN_POS_TABLE) lds += (size_t)S * S * sizeof(float);
    if (p.pos == SWIN_POS_ROPE2D) lds += (size_t)g.M * D * sizeof(float);
    dim3 grid(g.nwin, g.heads);
    if (p.dtype == SWIN_DT_F32) return dispatch_sim<float>(p, grid, threads, kc, lds, stream);
    return dispatch_sim<uint16_t>(p, grid, threads, kc, lds, stream);
}

}  // namespace swin
