// The linear layers on either side of the window attention in a Swin V2
// block (SwinV2 card, Method item 1 "Residual post-norm" and the block
// pseudocode; the block keeps Swin's layout):
//   QKV:  [q | k | v] = x W^T + b, W: 3C x C, outputs in that order, each
//         written to its own (T, C) tensor in the grid layout the attention
//         reads;
//   NORM: y = resid + norm_1(o W^T + b), W: C x C, norm_1 a layer norm over
//         the C channels of each token (biased variance, eps inside the
//         root) with per-channel gamma and beta.
//
// bf16 path (v_mfma_f32_16x16x32_bf16, fp32 accumulation).  A workgroup of
// four wavefronts takes 64 consecutive tokens.  The products are taken
// transposed, out^T = W x^T: the A operand is 16 weight rows (output
// channels), the B operand 16 token rows, so each lane ends with 4
// consecutive output channels of one token.  The input channels go 32 at a
// time: that slice of the 64 token rows and of the pass's weight rows is
// staged in LDS (XOR-swizzled 16-byte pieces, so the 16 rows of a fragment
// read cover all banks), in two stages, the next slice's global loads in
// flight while the matrix cores read the current one.  The wavefronts split
// the pass's 16-channel output tiles; each weight fragment serves all four
// token tiles.  Results go through LDS once more and leave as whole 16-byte
// pieces of contiguous runs (one run per token row and output tensor):
// storing the 8-byte pieces straight from the lanes, several wavefronts
// sharing each line, measured 15-25% slower.
//   QKV takes the 3C outputs in passes of 192 channels, adds the bias and
//   rounds once.  NORM takes all C <= 512 outputs in one pass and keeps them
//   in registers, reduces each token's sum and then its sum of squared
//   deviations across lanes and wavefronts (two passes, exact), and writes
//   resid + gamma (z - mean) / sqrt(var + eps) + beta, rounded once.
//
// fp32 path: one thread per output (QKV), one wavefront per token (NORM),
// fp32 throughout.
#include "common.hpp"
#include "lanes.hpp"
#include "launch_proj.hpp"
#include "tile_io.hpp"

namespace swin {

namespace {

using namespace lanes;
using namespace tio;

constexpr int PW = 4;                  // wavefronts per workgroup
constexpr int BT = 64;                 // tokens per workgroup
constexpr int RT = BT / 16;            // token tiles
constexpr int KC = 32;                 // input channels per staged slice

// LDS slot of the 16-byte piece p of staged row r (64-byte rows): the piece
// index is XOR-ed with bits 2-3 of the row, so the 16 rows one fragment read
// touches cover all 64 banks.
__device__ __forceinline__ int slot(int r, int p) { return r * KC + 8 * (p ^ ((r >> 2) & 3)); }

// two stages of bf16 slices: BT token rows and up to 64 NTW weight rows
template <int NTW>
constexpr size_t pass_lds() { return (size_t)2 * (BT + PW * NTW * 16) * KC * 2; }

// Output tiles of one pass: the product of the workgroup's token rows with
// the weight rows n0 .. n0 + nb - 1 (nb a multiple of 16, at most 64 NTW), the
// input channels taken KC at a time.  Both operand slices go through LDS in
// two stages: while one is read by the matrix cores, the next one's global
// loads are in flight.  Wavefront w holds output tiles w + PW j (j < NTW) of
// the pass for all BT tokens: z[j][r] is tokens 16r + li, channels
// n0 + 16 (w + PW j) + 4 grp .. +3.
template <int NTW>
__device__ __forceinline__ void pass_product(const __bf16* x, int nt, const __bf16* w, int C, int n0, int nb,
                                             __bf16* lds, f32x4 (&z)[NTW][RT], int tid, int wave, int lane)
{
    constexpr int NP = PW * NTW * 16;                     // weight rows per stage
    const int grp = lane >> 4, li = lane & 15;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int r = 0; r < RT; ++r) z[j][r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int XP = BT * 4 / (PW * 64);                // x pieces per thread
    constexpr int WP = NP * 4 / (PW * 64);                // weight pieces per thread, at most
    u32x4 xr[XP], wr[WP];
    auto load = [&](int s) {
#pragma unroll
        for (int m = 0; m < XP; ++m) {
            const int i = tid + PW * 64 * m, r = i >> 2, p = i & 3;
            xr[m] = r < nt ? *(const u32x4*)(x + (size_t)r * C + KC * s + 8 * p) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int m = 0; m < WP; ++m) {
            const int i = tid + PW * 64 * m, r = i >> 2, p = i & 3;
            if (r < nb) wr[m] = *(const u32x4*)(w + (size_t)(n0 + r) * C + KC * s + 8 * p);
        }
    };
    auto store = [&](__bf16* sx) {                        // stage: x rows, then weight rows
        __bf16* sw = sx + BT * KC;
#pragma unroll
        for (int m = 0; m < XP; ++m) {
            const int i = tid + PW * 64 * m;
            *(u32x4*)(sx + slot(i >> 2, i & 3)) = xr[m];
        }
#pragma unroll
        for (int m = 0; m < WP; ++m) {
            const int i = tid + PW * 64 * m, r = i >> 2;
            if (r < nb) *(u32x4*)(sw + slot(r, i & 3)) = wr[m];
        }
    };
    const int ks = C / KC;
    load(0);
    store(lds);
    __syncthreads();
    for (int s = 0; s < ks; ++s) {
        if (s + 1 < ks) load(s + 1);
        const __bf16* sx = lds + (s & 1) * (BT + NP) * KC;
        const __bf16* sw = sx + BT * KC;
        bf16x8 B[RT];
#pragma unroll
        for (int r = 0; r < RT; ++r) B[r] = *(const bf16x8*)(sx + slot(16 * r + li, grp));
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int m = wave + PW * j;                  // output tile within the pass
            if (16 * m >= nb) break;                      // wave-uniform
            const bf16x8 A = *(const bf16x8*)(sw + slot(16 * m + li, grp));
#pragma unroll
            for (int r = 0; r < RT; ++r) z[j][r] = mfma(A, B[r], z[j][r]);
        }
        if (s + 1 < ks) store(lds + ((s + 1) & 1) * (BT + NP) * KC);
        __syncthreads();
    }
}

// Staged outputs (BT tokens x channels [n0, n0 + nb) of [q | k | v], row
// stride OS) to their tensors: each destination's channels of the pass form
// one run per token, whole rows when the pass covers the tensor, so that
// consecutive threads write consecutive 16-byte pieces and the memory sees
// whole lines.
__device__ __forceinline__ void copy_out(const __bf16* ob, int OS, int n0, int nb, int C, int64_t t0, int nt,
                                         const ProjArgs& a, int tid)
{
    for (int d = n0 / C; d * C < n0 + nb; ++d) {
        const int lo = max(n0, d * C), hi = min(n0 + nb, (d + 1) * C);   // channels of [q | k | v]
        const int run = (hi - lo) / 8;                                  // 16-byte pieces per token
        __bf16* dst = (__bf16*)(d == 0 ? a.q : d == 1 ? a.k : a.v) + (size_t)t0 * C + (lo - d * C);
        for (int i = tid; i < nt * run; i += PW * 64) {
            const int t = i / run, p = i - t * run;
            *(u32x4*)(dst + (size_t)t * C + 8 * p) = *(const u32x4*)(ob + t * OS + (lo - n0) + 8 * p);
        }
    }
}

// [q | k | v] = x W^T + b: 64 tokens per workgroup, output channels in
// passes of up to 64 NTW.
template <int NTW>
__global__ void __launch_bounds__(PW * 64) qkv_kernel(ProjArgs a)
{
    constexpr int NP = PW * NTW * 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int C = a.C;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    const int64_t t0 = (int64_t)blockIdx.x * BT;
    const int nt = (int)min((int64_t)BT, a.T - t0);
    const __bf16* x = (const __bf16*)a.x + t0 * C;
#pragma unroll 1
    for (int n0 = 0; n0 < 3 * C; n0 += NP) {
        const int nb = min(NP, 3 * C - n0);
        f32x4 z[NTW][RT];
        pass_product<NTW>(x, nt, (const __bf16*)a.w, C, n0, nb, (__bf16*)smem, z, tid, wave, lane);
        // the pass's outputs to LDS (the slice stages are free now), then
        // out to q, k, v as runs of whole 16-byte pieces per token row
        __bf16* ob = (__bf16*)smem;                       // [BT][nb + 8]
        const int OS = nb + 8;
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int m = wave + PW * j;
            if (16 * m >= nb) break;
            // lane holds channels cl .. cl+3 of the pass for tokens 16r + li
            const int cl = 16 * m + 4 * grp;
            const f32x4 bias = a.b ? *(const f32x4*)(a.b + n0 + cl) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < RT; ++r)
                *(bf16x4*)(ob + (16 * r + li) * OS + cl) =
                    pack_bf16x4(z[j][r][0] + bias[0], z[j][r][1] + bias[1], z[j][r][2] + bias[2],
                                z[j][r][3] + bias[3]);
        }
        __syncthreads();
        copy_out(ob, OS, n0, nb, C, t0, nt, a, tid);
        __syncthreads();                                  // ob is the next pass's first stage
    }
}

// y = resid + norm_1(o W^T + b): 64 tokens per workgroup, all C <= 64 NTW
// output channels in one pass, held in registers through the norm.
template <int NTW>
__global__ void __launch_bounds__(PW * 64) norm_kernel(ProjArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int C = a.C;
    float* red = (float*)(smem + pass_lds<NTW>());        // [PW][BT] per-wave partial sums
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = lane >> 4, li = lane & 15;
    const int64_t t0 = (int64_t)blockIdx.x * BT;
    const int nt = (int)min((int64_t)BT, a.T - t0);
    f32x4 z[NTW][RT];
    pass_product<NTW>((const __bf16*)a.x + t0 * C, nt, (const __bf16*)a.w, C, 0, C, (__bf16*)smem, z, tid, wave,
                      lane);
    const int ntile = C / 16;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int n = wave + PW * j;
        if (n >= ntile) break;
        const f32x4 bias = a.b ? *(const f32x4*)(a.b + 16 * n + 4 * grp) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < RT; ++r) z[j][r] += bias;
    }

    // per-token sums over this lane's channels, then over the 4 lanes of a
    // token (lanes li + 16 grp) and the 4 wavefronts
    auto token_sum = [&](float (&part)[RT], float (&out)[RT]) {
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const float s = sum_x32(sum_x16(part[r]));
            if (grp == 0) red[wave * BT + 16 * r + li] = s;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < PW; ++w) s += red[w * BT + 16 * r + li];
            out[r] = s;
        }
        __syncthreads();                                  // red is reused
    };
    float part[RT], mean[RT], var[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
            if (wave + PW * j < ntile) s += (z[j][r][0] + z[j][r][1]) + (z[j][r][2] + z[j][r][3]);
        part[r] = s;
    }
    token_sum(part, mean);
    const float inv_c = 1.0f / (float)C;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
        mean[r] *= inv_c;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
            if (wave + PW * j < ntile) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float dz = z[j][r][e] - mean[r];
                    s = fmaf(dz, dz, s);
                }
            }
        part[r] = s;
    }
    token_sum(part, var);
    float rstd[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) rstd[r] = 1.0f / sqrtf(fmaf(var[r], inv_c, a.eps));
    __bf16* ob = (__bf16*)smem;                           // [BT][C + 8] (the slice stages are free)
    const int OS = C + 8;

#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int n = wave + PW * j;
        if (n >= ntile) break;
        const int ch = 16 * n + 4 * grp;
        const f32x4 g = *(const f32x4*)(a.gamma + ch);
        const f32x4 be = *(const f32x4*)(a.beta + ch);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
            const int t = 16 * r + li;
            const size_t off = (size_t)(t0 + (t < nt ? t : 0)) * C + ch;
            const u32x2 rw = *(const u32x2*)((const __bf16*)a.resid + off);
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t h = (e & 1) ? (rw[e >> 1] & 0xffff0000u) : (rw[e >> 1] << 16);
                y[e] = __uint_as_float(h) + fmaf(g[e], (z[j][r][e] - mean[r]) * rstd[r], be[e]);
            }
            *(bf16x4*)(ob + t * OS + ch) = pack_bf16x4(y[0], y[1], y[2], y[3]);
        }
    }
    // the block's rows of y are one contiguous run: out as whole 16-byte pieces
    __syncthreads();
    const int run = nt * (C / 8);
    __bf16* dst = (__bf16*)a.y + (size_t)t0 * C;
    for (int i = tid; i < run; i += PW * 64) {
        const int t = i / (C / 8), p = i - t * (C / 8);
        *(u32x4*)(dst + (size_t)t * C + 8 * p) = *(const u32x4*)(ob + t * OS + 8 * p);
    }
}

// fp32: one thread per output of [q | k | v].
__global__ void __launch_bounds__(256) qkv_f32_kernel(ProjArgs a)
{
    const int C = a.C, C3 = 3 * C;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.T * C3) return;
    const int64_t t = i / C3;
    const int n = (int)(i - t * C3);
    const float* x = (const float*)a.x + t * C;
    const float* w = (const float*)a.w + (size_t)n * C;
    float s = a.b ? a.b[n] : 0.0f;
    for (int c = 0; c < C; ++c) s = fmaf(x[c], w[c], s);
    const int which = n / C;
    float* dst = (float*)(which == 0 ? a.q : which == 1 ? a.k : a.v);
    dst[t * C + (n - which * C)] = s;
}

// fp32: one wavefront per token; z staged in LDS for the two passes.
__global__ void __launch_bounds__(64) norm_f32_kernel(ProjArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    float* zs = (float*)smem;                         // [C]
    const int C = a.C, lane = threadIdx.x;
    const int64_t t = blockIdx.x;
    const float* x = (const float*)a.x + t * C;
    for (int n = lane; n < C; n += 64) {
        const float* w = (const float*)a.w + (size_t)n * C;
        float s = a.b ? a.b[n] : 0.0f;
        for (int c = 0; c < C; ++c) s = fmaf(x[c], w[c], s);
        zs[n] = s;
    }
    float s = 0.0f;
    for (int n = lane; n < C; n += 64) s += zs[n];
    const float mean = wave_reduce<Op::Sum>(s) / (float)C;
    float q = 0.0f;
    for (int n = lane; n < C; n += 64) q = fmaf(zs[n] - mean, zs[n] - mean, q);
    const float rstd = 1.0f / sqrtf(wave_reduce<Op::Sum>(q) / (float)C + a.eps);
    const float* res = (const float*)a.resid + t * C;
    float* y = (float*)a.y + t * C;
    for (int n = lane; n < C; n += 64) y[n] = res[n] + fmaf(a.gamma[n], (zs[n] - mean) * rstd, a.beta[n]);
}

template <typename K>
hipError_t launch(K kernel, int64_t blocks, int threads, size_t lds, const ProjArgs& a, hipStream_t s)
{
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    kernel<<<(int)blocks, threads, lds, s>>>(a);
    return hipGetLastError();
}

}  // namespace

bool proj_supported(int C) { return C >= 32 && C <= 512 && C % 32 == 0; }

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t stream)
{
    if (a.T == 0) return hipSuccess;
    if (a.dtype == SWIN_DT_F32)
        return launch(qkv_f32_kernel, (a.T * 3 * a.C + 255) / 256, 256, 0, a, stream);
    // passes of 192 output channels: 3 tiles per wavefront keep the
    // registers at 3 wavefronts per SIMD (measured faster than one pass)
    return launch(qkv_kernel<3>, (a.T + BT - 1) / BT, PW * 64, pass_lds<3>(), a, stream);
}

hipError_t launch_proj_norm(const ProjArgs& a, hipStream_t stream)
{
    if (a.T == 0) return hipSuccess;
    if (a.dtype == SWIN_DT_F32)
        return launch(norm_f32_kernel, a.T, 64, (size_t)a.C * sizeof(float), a, stream);
    const int64_t blocks = (a.T + BT - 1) / BT;
    const size_t red = (size_t)PW * BT * sizeof(float);
    switch ((a.C + 63) / 64) {                            // 16-channel tiles per wavefront
    case 1: return launch(norm_kernel<1>, blocks, PW * 64, pass_lds<1>() + red, a, stream);
    case 2: return launch(norm_kernel<2>, blocks, PW * 64, pass_lds<2>() + red, a, stream);
    case 3: return launch(norm_kernel<3>, blocks, PW * 64, pass_lds<3>() + red, a, stream);
    case 4: return launch(norm_kernel<4>, blocks, PW * 64, pass_lds<4>() + red, a, stream);
    case 5: return launch(norm_kernel<5>, blocks, PW * 64, pass_lds<5>() + red, a, stream);
    case 6: return launch(norm_kernel<6>, blocks, PW * 64, pass_lds<6>() + red, a, stream);
    case 7: return launch(norm_kernel<7>, blocks, PW * 64, pass_lds<7>() + red, a, stream);
    default: return launch(norm_kernel<8>, blocks, PW * 64, pass_lds<8>() + red, a, stream);
    }
}

}  // namespace swin
