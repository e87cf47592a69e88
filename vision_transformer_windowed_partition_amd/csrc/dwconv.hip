// Iwin's convolution branch (Iwin abstract: the block couples interleaved
// window attention with a depthwise convolution that links each token to its
// local neighbours): out[b][y][x][c] += bias[c] + sum over the 3 x 3
// neighbourhood of w[c][dy+1][dx+1] v[b][y+dy][x+dx][c], zero padding at the
// image border, added to the attention output in place.
//
// A workgroup takes a 16 x 16 tile of tokens and 128 bytes of channels (one
// line of each token's row).  It stages the tile's 18 x 18 neighbourhood of v
// (zeros outside the image), the nine taps of its channels transposed to
// [tap][channel] and the bias in LDS, having first read the output pieces it
// will update into registers; each thread then forms 16-byte pieces of the
// output (8 bf16 or 4 fp32 channels of one token): nine taps in fp32 from
// LDS added to the attention output, rounded once and written back.
#include "common.hpp"
#include "launch_proj.hpp"

namespace swin {

namespace {

constexpr int TT = 16;                 // tile edge (tokens)
constexpr int HALO = TT + 2;
constexpr int NTHR = 256;
constexpr int CB = 128;                // channel chunk per workgroup, bytes (one line per token)
constexpr int OPT = TT * TT * (CB / 16) / NTHR;   // output pieces per thread (8)

template <typename T>
struct Piece;                          // 16 bytes of channels
template <>
struct Piece<uint16_t> {
    static constexpr int N = 8;
    __device__ static void to_f32(const u32x4 p, float* f) { unpack_bf16x8(p, f); }
    __device__ static u32x4 from_f32(const float* f) { return __builtin_bit_cast(u32x4, pack_bf16x8(f)); }
};
template <>
struct Piece<float> {
    static constexpr int N = 4;
    __device__ static void to_f32(const u32x4 p, float* f)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(p[i]);
    }
    __device__ static u32x4 from_f32(const float* f)
    {
        return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
};

// One workgroup: a TT x TT tile of tokens and CB bytes of channels (a whole
// line of each token's row, or the rest of the row).  The output pieces it
// will update are read into registers before the staging barrier, so their
// latency overlaps the staging of v.
template <typename T>
__global__ void __launch_bounds__(NTHR) dwconv_add_kernel(DwconvArgs a)
{
    using P = Piece<T>;
    constexpr int CC = CB / (int)sizeof(T);           // channels per chunk
    constexpr int PP = CB / 16;                        // pieces per token and chunk
    __shared__ u32x4 vs[HALO * HALO * PP];
    __shared__ float ws[9 * CC];
    __shared__ float bs[CC];
    const int C = a.C, H = a.H, W = a.W;
    const int c0 = blockIdx.y * CC;
    const int pp = min(PP, (C - c0) / P::N);           // pieces of this chunk (the last may be short)
    // blockIdx.x = (image * tile rows + tile row) * tile columns + tile column
    const int tx_n = (W + TT - 1) / TT, ty_n = (H + TT - 1) / TT;
    const int bx = blockIdx.x;
    const int tile_x = bx % tx_n, rest = bx / tx_n;
    const int ty = rest % ty_n, img = rest / ty_n;
    const int y0 = ty * TT, x0 = tile_x * TT;
    const size_t img_off = (size_t)img * H * W * C;
    const T* v = (const T*)a.v + img_off;
    T* out = (T*)a.out + img_off;

    // this thread's output pieces: i = threadIdx.x + NTHR m over TT*TT*PP
    u32x4 ov[OPT];
#pragma unroll
    for (int m = 0; m < OPT; ++m) {
        const int i = threadIdx.x + NTHR * m, tok = i / PP, p = i - tok * PP;
        const int y = y0 + tok / TT, x = x0 + tok % TT;
        if (y < H && x < W && p < pp) ov[m] = *(const u32x4*)(out + ((size_t)y * W + x) * C + c0 + P::N * p);
    }
    for (int i = threadIdx.x; i < HALO * HALO * PP; i += NTHR) {
        const int tok = i / PP, p = i - tok * PP;
        const int yy = y0 - 1 + tok / HALO, xx = x0 - 1 + tok % HALO;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (yy >= 0 && yy < H && xx >= 0 && xx < W && p < pp)
            val = *(const u32x4*)(v + ((size_t)yy * W + xx) * C + c0 + P::N * p);
        vs[i] = val;
    }
    for (int i = threadIdx.x; i < 9 * CC; i += NTHR) {
        const int tap = i / CC, c = i - tap * CC;
        ws[i] = c0 + c < C ? a.w[(size_t)(c0 + c) * 9 + tap] : 0.0f;
    }
    for (int i = threadIdx.x; i < CC; i += NTHR) bs[i] = (a.b && c0 + i < C) ? a.b[c0 + i] : 0.0f;
    __syncthreads();

#pragma unroll
    for (int m = 0; m < OPT; ++m) {
        const int i = threadIdx.x + NTHR * m, tok = i / PP, p = i - tok * PP;
        const int ly = tok / TT, lx = tok % TT;
        const int y = y0 + ly, x = x0 + lx;
        if (y >= H || x >= W || p >= pp) continue;
        float acc[P::N];
#pragma unroll
        for (int e = 0; e < P::N; ++e) acc[e] = bs[P::N * p + e];
#pragma unroll
        for (int dy = 0; dy < 3; ++dy)
#pragma unroll
            for (int dx = 0; dx < 3; ++dx) {
                float f[P::N];
                P::to_f32(vs[((ly + dy) * HALO + lx + dx) * PP + p], f);
                const float* wt = ws + (dy * 3 + dx) * CC + P::N * p;
#pragma unroll
                for (int e = 0; e < P::N; ++e) acc[e] = fmaf(wt[e], f[e], acc[e]);
            }
        float f[P::N];
        P::to_f32(ov[m], f);
#pragma unroll
        for (int e = 0; e < P::N; ++e) f[e] += acc[e];
        *(u32x4*)(out + ((size_t)y * W + x) * C + c0 + P::N * p) = P::from_f32(f);
    }
}

}  // namespace

bool dwconv_supported(int C, int dtype) { return C >= 1 && C % (dtype == SWIN_DT_F32 ? 4 : 8) == 0; }

hipError_t launch_dwconv_add(const DwconvArgs& a, hipStream_t stream)
{
    if ((int64_t)a.B * a.H * a.W == 0) return hipSuccess;
    const int64_t tiles = (int64_t)a.B * ((a.H + TT - 1) / TT) * ((a.W + TT - 1) / TT);
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
    const int cc = CB / (a.dtype == SWIN_DT_F32 ? 4 : 2);
    const dim3 grid((unsigned)tiles, (a.C + cc - 1) / cc);
    if (a.dtype == SWIN_DT_F32) dwconv_add_kernel<float><<<grid, NTHR, 0, stream>>>(a);
    else dwconv_add_kernel<uint16_t><<<grid, NTHR, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace swin
