// Window attention over video (3D) windows, and the bias table of the meta
// network G over three offsets.
//
// The pages fine-tune SwinV2 on Kinetics-400 with 16^2 x 8 windows over
// 256^2 x 8 frames (appendix A2) and move Iwin's weights from 2D to 3D (Iwin
// abstract) without writing the 3D form down; here it is the 2D window
// attention of the SwinV2 card (eq. 1-2, the window-attention pseudocode,
// eq. 3-4 for the bias) with a temporal axis treated like the other two:
// windows of Mt x M x M tokens, a cyclic shift (or interleaving) on every
// axis, pairs of different shift regions on any axis excluded, and the bias
// G(log-spaced dx, dy, dt) from a (2Mt-1)(2M-1)^2 x heads table.
//
// Vector ALUs, fp32 or bf16 tensors: one workgroup per (window, head), one
// thread per query (up to 512 at a time) with q, the running maximum, the
// running sum and the output accumulator in registers; keys and values are
// staged through LDS in chunks and read as broadcasts, the head's bias table
// sits in LDS for the whole window.  Similarities and logits are fp64 (a
// cosine logit reaches 100 at tau's floor), exponentials and the value sums
// fp32.  The N x N scores are never stored.
#include "common.hpp"
#include "lanes.hpp"
#include "launch_video.hpp"
#include "rows.hpp"

namespace swin {

namespace {

constexpr int D = 32;
constexpr int KC_MAX = 256;   // keys per LDS chunk

__device__ __forceinline__ int axis_pos(int L, int M, int s, int part, int w, int r)
{
    return part == SWIN_PART_INTERLEAVED ? w + r * (L / M) : (w * M + r + s) % L;
}

template <typename T, int SIM, int POS>
__global__ void __launch_bounds__(512) attn_video_kernel(VideoArgs a, int kc)
{
    extern __shared__ double smem_d[];
    const int M = a.M, Mt = a.Mt, MM = M * M, N = a.N, S = 2 * M - 1;
    const int h = blockIdx.y;
    const int win = blockIdx.x;
    const int tid = threadIdx.x;

    double* kinv = smem_d;                             // [kc] 1/||k|| (COSINE)
    float* ks = (float*)(kinv + kc);                   // [kc][D]
    float* vs = ks + kc * D;                           // [kc][D]
    float* bias = vs + kc * D;                         // [(2Mt-1) S S] (TABLE)
    if (POS == SWIN_POS_TABLE) {
        const int S3 = (2 * Mt - 1) * S * S;
        for (int i = tid; i < S3; i += blockDim.x) bias[i] = a.table[(size_t)i * a.heads + h];
    }

    // window (b, wt, wr, wc) and the grid offset of local token (t, r, c)
    const int nW = a.nwt * a.nwr * a.nwc;
    const int b = win / nW, wl = win - b * nW;
    const int wt = wl / (a.nwr * a.nwc), wr = (wl / a.nwc) % a.nwr, wc = wl % a.nwc;
    auto tok = [&](int t, int r, int c) -> int64_t {
        const int gt = axis_pos(a.T, Mt, a.shift_t, a.part, wt, t);
        const int gi = axis_pos(a.H, M, a.shift, a.part, wr, r);
        const int gj = axis_pos(a.W, M, a.shift, a.part, wc, c);
        return ((((int64_t)b * a.T + gt) * a.H + gi) * a.W + gj) * a.C + (int64_t)h * D;
    };
    const bool cyc = a.part == SWIN_PART_CYCLIC;
    const T* qg = (const T*)a.q;
    const T* kg = (const T*)a.k;
    const T* vg = (const T*)a.v;
    T* og = (T*)a.out;
    __syncthreads();

    for (int q0 = 0; q0 < N; q0 += blockDim.x) {
        const int t = q0 + tid;
        const bool valid = t < N;
        const int tq = valid ? t : 0;
        const int ti = tq / MM, ri = (tq / M) % M, ci = tq % M;
        float q[D], acc[D];
        double scale = 0.0;
        if (valid) {
            load_row32<T>(qg + tok(ti, ri, ci), q);
            if (SIM == SWIN_SIM_COSINE) {
                double ss = 0.0;
#pragma unroll
                for (int e = 0; e < D; ++e) ss = fma((double)q[e], (double)q[e], ss);
                const double tau = fmax((double)a.tau[h], (double)a.tau_min);
                scale = 1.0 / (tau * fmax(sqrt(ss), 1e-12));
            } else {
                scale = 1.0 / sqrt((double)D);
            }
        }
        // keys of the query's shift region, per axis
        int tlo = 0, thi = Mt, rlo = 0, rhi = M, clo = 0, chi = M;
        if (cyc) {
            region_interval(wt, a.nwt, Mt, a.shift_t, ti, tlo, thi);
            region_interval(wr, a.nwr, M, a.shift, ri, rlo, rhi);
            region_interval(wc, a.nwc, M, a.shift, ci, clo, chi);
        }
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] = 0.0f;
        double m = -INFINITY;
        float l = 0.0f;

        for (int j0 = 0; j0 < N; j0 += kc) {
            const int cnt = min(kc, N - j0);
            __syncthreads();
            if (tid < cnt) {
                const int j = j0 + tid;
                float kr[D], vr[D];
                const int64_t off = tok(j / MM, (j / M) % M, j % M);
                load_row32<T>(kg + off, kr);
                load_row32<T>(vg + off, vr);
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
            if (!valid) continue;
            // key (tj, rj, cj) of slot j0, advanced slot by slot
            int tj = j0 / MM, rj = (j0 / M) % M, cj = j0 % M;
            for (int jj = 0; jj < cnt; ++jj) {
                const bool ok = tj >= tlo && tj < thi && rj >= rlo && rj < rhi && cj >= clo && cj < chi;
                if (ok) {
                    const float* kr = ks + jj * D;
                    double s = 0.0;
#pragma unroll
                    for (int e = 0; e < D; ++e) s = fma((double)q[e], (double)kr[e], s);
                    double x = s * scale;
                    if (SIM == SWIN_SIM_COSINE) x *= kinv[jj];
                    if (POS == SWIN_POS_TABLE)
                        x += (double)bias[((ti - tj + Mt - 1) * S + (ri - rj + M - 1)) * S + (ci - cj + M - 1)];
                    const float* vr = vs + jj * D;
                    if (x > m) {
                        const float al = expf((float)(m - x));       // 0 on the first key
                        l = fmaf(l, al, 1.0f);
#pragma unroll
                        for (int e = 0; e < D; ++e) acc[e] = fmaf(acc[e], al, vr[e]);
                        m = x;
                    } else {
                        const float pj = expf((float)(x - m));
                        l += pj;
#pragma unroll
                        for (int e = 0; e < D; ++e) acc[e] = fmaf(pj, vr[e], acc[e]);
                    }
                }
                if (++cj == M) { cj = 0; if (++rj == M) { rj = 0; ++tj; } }
            }
        }
        if (valid) {
            const float inv = 1.0f / l;
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] *= inv;
            store_row32<T>(og + tok(ti, ri, ci), acc);
        }
    }
}

template <typename T, int SIM>
hipError_t launch_pos(const VideoArgs& a, dim3 grid, int threads, int kc, size_t lds, hipStream_t s)
{
    auto* fn = a.pos == SWIN_POS_TABLE ? attn_video_kernel<T, SIM, SWIN_POS_TABLE>
                                       : attn_video_kernel<T, SIM, SWIN_POS_NONE>;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
    }
    fn<<<grid, threads, lds, s>>>(a, kc);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_sim(const VideoArgs& a, dim3 grid, int threads, int kc, size_t lds, hipStream_t s)
{
    if (a.sim == SWIN_SIM_COSINE) return launch_pos<T, SWIN_SIM_COSINE>(a, grid, threads, kc, lds, s);
    return launch_pos<T, SWIN_SIM_DOT>(a, grid, threads, kc, lds, s);
}

int video_threads(const VideoArgs& a) { return a.N >= 512 ? 512 : (a.N + 63) / 64 * 64; }

// G over the log-spaced offsets (dx, dy, dt) of one table row for a group of
// up to four heads: one wavefront, lane j evaluating hidden units j, j + 64,
// ... and accumulating their share of the group's output sums, which a
// cross-lane sum finishes; fp32.
constexpr int CPB_HG = 4;

__global__ void __launch_bounds__(256) cpb3d_kernel(int Mt, int M, int heads, int hidden, const float* w1,
                                                    const float* b1, const float* w2, const float* b2,
                                                    float* table, int items)
{
    const int lane = threadIdx.x & 63;
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (item >= items) return;
    const int groups = (heads + CPB_HG - 1) / CPB_HG;
    const int row = item / groups, h0 = (item - row * groups) * CPB_HG;
    const int S = 2 * M - 1;
    const int dx = row % S - (M - 1), dy = (row / S) % S - (M - 1), dt = row / (S * S) - (Mt - 1);
    const auto lg = [](int x) { return copysignf(log1pf(fabsf((float)x)), (float)x); };
    const float in0 = lg(dx), in1 = lg(dy), in2 = lg(dt);
    float acc[CPB_HG] = {};
    for (int j = lane; j < hidden; j += 64) {
        const float z = fmaxf(fmaf(w1[3 * j], in0, fmaf(w1[3 * j + 1], in1, fmaf(w1[3 * j + 2], in2,
                                                                                 b1 ? b1[j] : 0.0f))), 0.0f);
#pragma unroll
        for (int o = 0; o < CPB_HG; ++o)
            if (h0 + o < heads) acc[o] = fmaf(w2[(size_t)(h0 + o) * hidden + j], z, acc[o]);
    }
#pragma unroll
    for (int o = 0; o < CPB_HG; ++o) {
        const float g = lanes::wave_reduce<lanes::Op::Sum>(acc[o]);
        if (lane == 0 && h0 + o < heads) table[(size_t)row * heads + h0 + o] = g + (b2 ? b2[h0 + o] : 0.0f);
    }
}

}  // namespace

size_t video_lds(const VideoArgs& a, int* kc_out)
{
    const int S = 2 * a.M - 1;
    const size_t tab = a.pos == SWIN_POS_TABLE ? (size_t)(2 * a.Mt - 1) * S * S * sizeof(float) : 0;
    int kc = video_threads(a) < KC_MAX ? video_threads(a) : KC_MAX;
    for (; kc >= 64; kc /= 2) {
        const size_t lds = (size_t)kc * sizeof(double) + (size_t)2 * kc * D * sizeof(float) + tab;
        if (lds <= 160 * 1024) {
            if (kc_out) *kc_out = kc;
            return lds;
        }
    }
    return 0;
}

hipError_t launch_attn_video(const VideoArgs& a, hipStream_t stream)
{
    if (a.nwin == 0) return hipSuccess;
    int kc = 0;
    const size_t lds = video_lds(a, &kc);
    if (lds == 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.nwin, (unsigned)a.heads);
    const int threads = video_threads(a);
    if (a.dtype == SWIN_DT_F32) return launch_sim<float>(a, grid, threads, kc, lds, stream);
    return launch_sim<uint16_t>(a, grid, threads, kc, lds, stream);
}

hipError_t launch_cpb_table3d(int Mt, int M, int heads, int hidden, const float* w1, const float* b1,
                              const float* w2, const float* b2, float* table, hipStream_t stream)
{
    const int S = 2 * M - 1;
    const int64_t items = (int64_t)(2 * Mt - 1) * S * S * ((heads + CPB_HG - 1) / CPB_HG);
    if (items == 0) return hipSuccess;
    cpb3d_kernel<<<(unsigned)((items + 3) / 4), 256, 0, stream>>>(Mt, M, heads, hidden, w1, b1, w2, b2, table,
                                                                  (int)items);
    return hipGetLastError();
}

}  // namespace swin
