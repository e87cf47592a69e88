// C ABI of libswinattn.so (declared in include/swin_attn.h): argument
// validation on the host, then one asynchronous launch on the caller's
// stream.  Nothing is enqueued unless every argument passes.
#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "launch.hpp"
#include "launch_bwd.hpp"
#include "launch_proj.hpp"
#include "launch_video.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return SWIN_OK;
    return fail(SWIN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Shape rules shared by partition and attention.  Returns SWIN_OK or the
// failing status (with the detail recorded).
int check_grid(int32_t B, int32_t H, int32_t W, int32_t C, int32_t M, int32_t shift,
               int32_t partition)
{
    if (B < 0 || H < 1 || W < 1 || C < 1 || M < 1)
        return fail(SWIN_EINVAL, "bad shape B=%d H=%d W=%d C=%d M=%d", B, H, W, C, M);
    if (partition != SWIN_PART_CYCLIC && partition != SWIN_PART_INTERLEAVED)
        return fail(SWIN_EINVAL, "unknown partition %d", partition);
    if (shift < 0 || shift >= M)
        return fail(SWIN_EINVAL, "shift %d outside [0, M=%d)", shift, M);
    if (partition == SWIN_PART_INTERLEAVED && shift != 0)
        return fail(SWIN_EINVAL, "interleaved windows take no shift (shift=%d)", shift);
    if (M > H || M > W || H % M || W % M)
        return fail(SWIN_EUNSUPPORTED, "H=%d, W=%d must be multiples of M=%d (no padding is built)", H, W, M);
    const int64_t nwin = (int64_t)B * (H / M) * (W / M);
    if ((int64_t)B * H * W > ((int64_t)1 << 31) - 1 || nwin * 64 > ((int64_t)1 << 31) - 1)
        return fail(SWIN_EUNSUPPORTED, "grid too large (B*H*W=%lld)", (long long)B * H * W);
    return SWIN_OK;
}

swin::Geometry make_geometry(int32_t B, int32_t H, int32_t W, int32_t C, int32_t heads,
                             int32_t M, int32_t shift, int32_t partition, int32_t layout)
{
    swin::Geometry g;
    g.B = B; g.H = H; g.W = W; g.C = C; g.heads = heads; g.d = C / heads;
    g.M = M; g.shift = shift; g.part = partition; g.layout = layout;
    g.nwr = H / M; g.nwc = W / M; g.N = M * M;
    g.nwin = B * g.nwr * g.nwc;
    return g;
}

int window_copy(const void* src, void* dst, int32_t B, int32_t H, int32_t W, int32_t C,
                int32_t M, int32_t shift, int32_t partition, int32_t dtype, void* stream,
                bool to_windows)
{
    int st = check_grid(B, H, W, C, M, shift, partition);
    if (st) return st;
    if (dtype != SWIN_DT_F32 && dtype != SWIN_DT_BF16) return fail(SWIN_EINVAL, "unknown dtype %d", dtype);
    const size_t bytes = (size_t)B * H * W * C * (dtype == SWIN_DT_F32 ? 4 : 2);
    if (bytes == 0) return SWIN_OK;
    if (!src || !dst) return fail(SWIN_EINVAL, "NULL tensor pointer");
    if (overlaps(src, bytes, dst, bytes)) return fail(SWIN_EINVAL, "source and destination overlap");
    swin::Geometry g = make_geometry(B, H, W, C, 1, M, shift, partition, SWIN_LAYOUT_GRID);
    return hip_status(swin::launch_window_copy(src, dst, g, dtype == SWIN_DT_F32 ? 4 : 2, to_windows,
                                               (hipStream_t)stream),
                      to_windows ? "swin_window_partition launch" : "swin_window_reverse launch");
}

}  // namespace

extern "C" {

int swin_version(void) { return SWIN_ATTN_VERSION; }

const char* swin_status_string(int status)
{
    switch (status) {
    case SWIN_OK: return "SWIN_OK: success";
    case SWIN_EINVAL: return "SWIN_EINVAL: invalid argument";
    case SWIN_EUNSUPPORTED: return "SWIN_EUNSUPPORTED: defined by the method but not built here";
    case SWIN_EHIP: return "SWIN_EHIP: HIP runtime error";
    default: return "unknown status";
    }
}

const char* swin_last_error(void) { return g_last_error.c_str(); }

int swin_cpb_table_ex(int32_t M, int32_t norm_M, int32_t heads, int32_t hidden, const float* w1,
                      const float* b1, const float* w2, const float* b2, int32_t cpb_mode, float* table,
                      void* stream)
{
    if (cpb_mode < 0 || cpb_mode > (SWIN_CPB_CODE_NORM | SWIN_CPB_SIGMOID16))
        return fail(SWIN_EINVAL, "unknown cpb_mode %d", cpb_mode);
    if (M < 1 || M > 64) return fail(SWIN_EINVAL, "M=%d outside [1, 64]", M);
    if ((cpb_mode & SWIN_CPB_CODE_NORM) && (norm_M < 2 || norm_M > 4096))
        return fail(SWIN_EINVAL, "normalising window %d outside [2, 4096]", norm_M);
    if (heads < 1 || heads > 64) return fail(SWIN_EINVAL, "heads=%d outside [1, 64]", heads);
    if (hidden < 1 || hidden > 4096) return fail(SWIN_EINVAL, "hidden=%d outside [1, 4096]", hidden);
    if (!w1 || !w2 || !table) return fail(SWIN_EINVAL, "NULL w1, w2 or table");
    const size_t tb = (size_t)(2 * M - 1) * (2 * M - 1) * heads * sizeof(float);
    if (overlaps(table, tb, w1, (size_t)hidden * 2 * 4) || overlaps(table, tb, w2, (size_t)heads * hidden * 4) ||
        (b1 && overlaps(table, tb, b1, (size_t)hidden * 4)) || (b2 && overlaps(table, tb, b2, (size_t)heads * 4)))
        return fail(SWIN_EINVAL, "table overlaps a parameter tensor");
    return hip_status(swin::launch_cpb_table(M, norm_M, heads, hidden, w1, b1, w2, b2, cpb_mode, table,
                                             (hipStream_t)stream),
                      "swin_cpb_table launch");
}

int swin_cpb_table(int32_t M, int32_t heads, int32_t hidden, const float* w1, const float* b1,
                   const float* w2, const float* b2, int32_t cpb_mode, float* table, void* stream)
{
    return swin_cpb_table_ex(M, M, heads, hidden, w1, b1, w2, b2, cpb_mode, table, stream);
}

int swin_cpb_table_resize(int32_t M_src, int32_t M_dst, int32_t heads, const float* src, float* dst, void* stream)
{
    if (M_src < 1 || M_src > 64 || M_dst < 1 || M_dst > 64)
        return fail(SWIN_EINVAL, "windows %d -> %d outside [1, 64]", M_src, M_dst);
    if (heads < 1 || heads > 64) return fail(SWIN_EINVAL, "heads=%d outside [1, 64]", heads);
    if (!src || !dst) return fail(SWIN_EINVAL, "NULL src or dst");
    const size_t ns = (size_t)(2 * M_src - 1) * (2 * M_src - 1) * heads * sizeof(float);
    const size_t nd = (size_t)(2 * M_dst - 1) * (2 * M_dst - 1) * heads * sizeof(float);
    if (overlaps(dst, nd, src, ns)) return fail(SWIN_EINVAL, "dst overlaps src");
    return hip_status(swin::launch_table_resize(M_src, M_dst, heads, src, dst, (hipStream_t)stream),
                      "swin_cpb_table_resize launch");
}

int swin_window_partition(const void* x, void* xw, int32_t B, int32_t H, int32_t W, int32_t C,
                          int32_t M, int32_t shift, int32_t partition, int32_t dtype, void* stream)
{
    return window_copy(x, xw, B, H, W, C, M, shift, partition, dtype, stream, true);
}

int swin_window_reverse(const void* xw, void* x, int32_t B, int32_t H, int32_t W, int32_t C,
                        int32_t M, int32_t shift, int32_t partition, int32_t dtype, void* stream)
{
    return window_copy(xw, x, B, H, W, C, M, shift, partition, dtype, stream, false);
}

}  // extern "C"

namespace {

// Checks of the descriptor alone (no pointers); SWIN_OK or the failure.
int check_desc(const swin_attn_desc* d, bool rope_freqs_given)
{
    if (!d) return fail(SWIN_EINVAL, "NULL descriptor");
    int st = check_grid(d->B, d->H, d->W, d->C, d->M, d->shift, d->partition);
    if (st) return st;
    if (d->heads < 1 || d->C % d->heads)
        return fail(SWIN_EINVAL, "C=%d is not a multiple of heads=%d", d->C, d->heads);
    if (d->sim != SWIN_SIM_COSINE && d->sim != SWIN_SIM_DOT) return fail(SWIN_EINVAL, "unknown sim %d", d->sim);
    if (d->pos != SWIN_POS_NONE && d->pos != SWIN_POS_TABLE && d->pos != SWIN_POS_ROPE2D)
        return fail(SWIN_EINVAL, "unknown pos %d", d->pos);
    if (d->dtype != SWIN_DT_F32 && d->dtype != SWIN_DT_BF16) return fail(SWIN_EINVAL, "unknown dtype %d", d->dtype);
    if (d->layout != SWIN_LAYOUT_GRID && d->layout != SWIN_LAYOUT_WINDOWS)
        return fail(SWIN_EINVAL, "unknown layout %d", d->layout);
    if (!(d->tau_min > 0.0f) || !(d->tau_min < 3.0e38f)) return fail(SWIN_EINVAL, "tau_min must be positive and finite");
    if (d->pos == SWIN_POS_ROPE2D && !rope_freqs_given && !(d->rope_base > 0.0f && d->rope_base < 3.0e38f))
        return fail(SWIN_EINVAL, "rope_base must be positive and finite");
    if (d->C / d->heads != 32)
        return fail(SWIN_EUNSUPPORTED, "head dim %d: only 32 is built", d->C / d->heads);
    if (d->M > 64) return fail(SWIN_EUNSUPPORTED, "M=%d: windows above 64 are not built", d->M);
    return SWIN_OK;
}

swin::AttnParams params_of(const swin_attn_desc* d)
{
    swin::AttnParams p{};
    p.g = make_geometry(d->B, d->H, d->W, d->C, d->heads, d->M, d->shift, d->partition, d->layout);
    p.sim = d->sim; p.pos = d->pos; p.dtype = d->dtype;
    p.tau_min = d->tau_min; p.rope_base = d->rope_base;
    return p;
}

enum class Kernel { VALU, SMALL, LARGE, MFMA };

Kernel kernel_for(const swin::AttnParams& p)
{
    if (p.dtype == SWIN_DT_F32) return Kernel::VALU;
    if (swin::attn_small_supported(p)) return Kernel::SMALL;
    if (swin::attn_large_supported(p)) return Kernel::LARGE;
    return Kernel::MFMA;
}

int attn_fwd(const swin_attn_desc* d, const void* q, const void* k, const void* v, void* out, const float* tau,
             const float* table, const float* rope_freqs, float* lse, void* stream)
{
    int st = check_desc(d, rope_freqs != nullptr);
    if (st) return st;
    const size_t es = d->dtype == SWIN_DT_F32 ? 4 : 2;
    const size_t bytes = (size_t)d->B * d->H * d->W * d->C * es;
    if (bytes == 0) return SWIN_OK;
    if (!q || !k || !v || !out) return fail(SWIN_EINVAL, "NULL q, k, v or out");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15)
        return fail(SWIN_EINVAL, "q, k, v and out must be 16-byte aligned");
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
        return fail(SWIN_EINVAL, "out overlaps q, k or v");
    if (d->sim == SWIN_SIM_COSINE && !tau) return fail(SWIN_EINVAL, "COSINE needs tau");
    if (d->pos == SWIN_POS_TABLE && !table) return fail(SWIN_EINVAL, "POS_TABLE needs a table");
    if (lse) {
        const size_t lb = bytes / es / (size_t)(d->C / d->heads) * sizeof(float);   // windows x heads x N
        if ((uintptr_t)lse & 3) return fail(SWIN_EINVAL, "lse must be 4-byte aligned");
        if (overlaps(lse, lb, q, bytes) || overlaps(lse, lb, k, bytes) || overlaps(lse, lb, v, bytes) ||
            overlaps(lse, lb, out, bytes))
            return fail(SWIN_EINVAL, "lse overlaps q, k, v or out");
    }

    swin::AttnParams p = params_of(d);
    p.q = q; p.k = k; p.v = v; p.out = out;
    p.tau = tau; p.table = table; p.rope_freqs = rope_freqs;
    p.lse = lse;
    hipError_t e;
    Kernel kern = kernel_for(p);
    if (lse && kern == Kernel::MFMA) kern = Kernel::VALU;      // the general kernel exports none
    switch (kern) {
    case Kernel::VALU: e = swin::launch_attn_valu(p, (hipStream_t)stream); break;
    case Kernel::SMALL: e = swin::launch_attn_small(p, (hipStream_t)stream); break;
    case Kernel::LARGE: e = swin::launch_attn_large(p, (hipStream_t)stream); break;
    default: e = swin::launch_attn_mfma(p, (hipStream_t)stream); break;
    }
    return hip_status(e, "swin_window_attn_fwd launch");
}

int attn_bwd(const swin_attn_desc* d, const void* q, const void* k, const void* v, const void* out,
             const void* dout, const float* tau, const float* table, const float* rope_freqs, const float* lse,
             void* dq, void* dk, void* dv, float* dtau, float* dtable, void* stream)
{
    int st = check_desc(d, rope_freqs != nullptr);
    if (st) return st;
    if (d->C != d->heads * 32) return fail(SWIN_EUNSUPPORTED, "backward: head dim %d (32 only)", d->C / d->heads);
    if (!swin::attn_bwd_supported(params_of(d)))
        return fail(SWIN_EUNSUPPORTED, "backward: M=%d (up to 64, where the statistics and table fit LDS)", d->M);
    const size_t es = d->dtype == SWIN_DT_F32 ? 4 : 2;
    const size_t bytes = (size_t)d->B * d->H * d->W * d->C * es;
    if (d->sim == SWIN_SIM_COSINE && !tau) return fail(SWIN_EINVAL, "COSINE needs tau");
    if (d->pos == SWIN_POS_TABLE && !table) return fail(SWIN_EINVAL, "POS_TABLE needs a table");
    const void* in[5] = {q, k, v, out, dout};
    void* g[3] = {dq, dk, dv};
    if (bytes) {
        uintptr_t al = 0;
        for (const void* x : in) { if (!x) return fail(SWIN_EINVAL, "NULL q, k, v, out or dout"); al |= (uintptr_t)x; }
        for (void* x : g) { if (!x) return fail(SWIN_EINVAL, "NULL dq, dk or dv"); al |= (uintptr_t)x; }
        if (al & 15) return fail(SWIN_EINVAL, "tensors must be 16-byte aligned");
        for (void* x : g) {
            for (const void* y : in)
                if (overlaps(x, bytes, y, bytes)) return fail(SWIN_EINVAL, "a gradient overlaps an input");
            for (void* y : g)
                if (x != y && overlaps(x, bytes, y, bytes)) return fail(SWIN_EINVAL, "gradients overlap");
        }
    }
    const int S = 2 * d->M - 1;
    const size_t tb = (size_t)S * S * d->heads * sizeof(float);
    if (dtable && d->pos == SWIN_POS_TABLE && table && overlaps(dtable, tb, table, tb))
        return fail(SWIN_EINVAL, "dtable overlaps the table");
    if (lse && ((uintptr_t)lse & 3)) return fail(SWIN_EINVAL, "lse must be 4-byte aligned");

    swin::AttnParams p = params_of(d);
    p.q = q; p.k = k; p.v = v; p.out = nullptr;
    p.tau = tau; p.table = table; p.rope_freqs = rope_freqs;
    p.lse = const_cast<float*>(lse);                          // read only by a backward
    return hip_status(swin::launch_attn_bwd(p, out, dout, dq, dk, dv, dtau, dtable, (hipStream_t)stream),
                      "swin_window_attn_bwd launch");
}

}  // namespace

extern "C" {

int swin_window_attn_fwd(const swin_attn_desc* d, const void* q, const void* k, const void* v,
                         void* out, const float* tau, const float* table, const float* rope_freqs,
                         void* stream)
{
    return attn_fwd(d, q, k, v, out, tau, table, rope_freqs, nullptr, stream);
}

int swin_window_attn_fwd_lse(const swin_attn_desc* d, const void* q, const void* k, const void* v,
                             void* out, const float* tau, const float* table, const float* rope_freqs,
                             float* lse, void* stream)
{
    if (!lse && d && (int64_t)d->B * d->H * d->W * d->C > 0) return fail(SWIN_EINVAL, "NULL lse");
    return attn_fwd(d, q, k, v, out, tau, table, rope_freqs, lse, stream);
}

int swin_cpb_table3d(int32_t Mt, int32_t M, int32_t heads, int32_t hidden, const float* w1, const float* b1,
                     const float* w2, const float* b2, float* table, void* stream)
{
    if (M < 1 || M > 64) return fail(SWIN_EINVAL, "M=%d outside [1, 64]", M);
    if (Mt < 1 || Mt > 64) return fail(SWIN_EINVAL, "Mt=%d outside [1, 64]", Mt);
    if (heads < 1 || heads > 64) return fail(SWIN_EINVAL, "heads=%d outside [1, 64]", heads);
    if (hidden < 1 || hidden > 4096) return fail(SWIN_EINVAL, "hidden=%d outside [1, 4096]", hidden);
    if (!w1 || !w2 || !table) return fail(SWIN_EINVAL, "NULL w1, w2 or table");
    const size_t tb = (size_t)(2 * Mt - 1) * (2 * M - 1) * (2 * M - 1) * heads * sizeof(float);
    if (overlaps(table, tb, w1, (size_t)hidden * 3 * 4) || overlaps(table, tb, w2, (size_t)heads * hidden * 4) ||
        (b1 && overlaps(table, tb, b1, (size_t)hidden * 4)) || (b2 && overlaps(table, tb, b2, (size_t)heads * 4)))
        return fail(SWIN_EINVAL, "table overlaps a parameter tensor");
    return hip_status(swin::launch_cpb_table3d(Mt, M, heads, hidden, w1, b1, w2, b2, table, (hipStream_t)stream),
                      "swin_cpb_table3d launch");
}

int swin_window_attn3d_fwd(const swin_attn_desc* d, int32_t T, int32_t Mt, int32_t shift_t, const void* q,
                           const void* k, const void* v, void* out, const float* tau, const float* table,
                           void* stream)
{
    int st = check_desc(d, false);
    if (st) return st;
    if (d->pos == SWIN_POS_ROPE2D) return fail(SWIN_EUNSUPPORTED, "video windows: no rotary form");
    if (d->layout != SWIN_LAYOUT_GRID) return fail(SWIN_EUNSUPPORTED, "video windows: grid layout only");
    if (T < 1 || Mt < 1 || T % Mt) return fail(SWIN_EINVAL, "T=%d is not a positive multiple of Mt=%d", T, Mt);
    if (Mt > 64) return fail(SWIN_EUNSUPPORTED, "Mt=%d: temporal windows above 64 are not built", Mt);
    if (shift_t < 0 || shift_t >= Mt) return fail(SWIN_EINVAL, "shift_t=%d outside [0, Mt)", shift_t);
    if (d->partition == SWIN_PART_INTERLEAVED && shift_t != 0)
        return fail(SWIN_EINVAL, "interleaved windows take no shift");
    const size_t es = d->dtype == SWIN_DT_F32 ? 4 : 2;
    const size_t bytes = (size_t)d->B * T * d->H * d->W * d->C * es;
    if (d->sim == SWIN_SIM_COSINE && !tau) return fail(SWIN_EINVAL, "COSINE needs tau");
    if (d->pos == SWIN_POS_TABLE && !table) return fail(SWIN_EINVAL, "POS_TABLE needs a table");
    swin::VideoArgs a{};
    a.B = d->B; a.T = T; a.H = d->H; a.W = d->W; a.C = d->C; a.heads = d->heads;
    a.Mt = Mt; a.M = d->M; a.shift_t = shift_t; a.shift = d->shift; a.part = d->partition;
    a.sim = d->sim; a.pos = d->pos; a.dtype = d->dtype; a.tau_min = d->tau_min;
    a.nwt = T / Mt; a.nwr = d->H / d->M; a.nwc = d->W / d->M; a.N = Mt * d->M * d->M;
    const int64_t nwin = (int64_t)d->B * a.nwt * a.nwr * a.nwc;
    if (nwin > INT32_MAX) return fail(SWIN_EUNSUPPORTED, "too many windows");
    a.nwin = (int)nwin;
    const bool mfma = swin::video_mfma_supported(a);
    if (!mfma && swin::video_lds(a, nullptr) == 0)
        return fail(SWIN_EUNSUPPORTED, "Mt=%d, M=%d: the bias table does not fit LDS", Mt, d->M);
    if (bytes == 0) return SWIN_OK;
    if (!q || !k || !v || !out) return fail(SWIN_EINVAL, "NULL q, k, v or out");
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15)
        return fail(SWIN_EINVAL, "q, k, v and out must be 16-byte aligned");
    if (overlaps(out, bytes, q, bytes) || overlaps(out, bytes, k, bytes) || overlaps(out, bytes, v, bytes))
        return fail(SWIN_EINVAL, "out overlaps q, k or v");
    a.q = q; a.k = k; a.v = v; a.out = out; a.tau = tau; a.table = table;
    const hipError_t e = mfma ? swin::launch_attn_video_mfma(a, (hipStream_t)stream)
                              : swin::launch_attn_video(a, (hipStream_t)stream);
    return hip_status(e, "swin_window_attn3d_fwd launch");
}

const char* swin_window_attn3d_kernel(const swin_attn_desc* d, int32_t T, int32_t Mt)
{
    if (!d || T < 1 || Mt < 1 || d->heads < 1 || d->M < 1) return "";
    swin::VideoArgs a{};
    a.B = d->B; a.T = T; a.H = d->H; a.W = d->W; a.C = d->C; a.heads = d->heads;
    a.Mt = Mt; a.M = d->M; a.part = d->partition; a.sim = d->sim; a.pos = d->pos; a.dtype = d->dtype;
    return swin::video_mfma_supported(a) ? "attn_video_mfma_kernel" : "attn_video_kernel";
}

int swin_window_attn_bwd(const swin_attn_desc* d, const void* q, const void* k, const void* v,
                         const void* out, const void* dout, const float* tau, const float* table,
                         const float* rope_freqs, void* dq, void* dk, void* dv, float* dtau, float* dtable,
                         void* stream)
{
    return attn_bwd(d, q, k, v, out, dout, tau, table, rope_freqs, nullptr, dq, dk, dv, dtau, dtable, stream);
}

int swin_window_attn_bwd_lse(const swin_attn_desc* d, const void* q, const void* k, const void* v,
                             const void* out, const void* dout, const float* tau, const float* table,
                             const float* rope_freqs, const float* lse, void* dq, void* dk, void* dv,
                             float* dtau, float* dtable, void* stream)
{
    if (!lse && d && (int64_t)d->B * d->H * d->W * d->C > 0) return fail(SWIN_EINVAL, "NULL lse");
    return attn_bwd(d, q, k, v, out, dout, tau, table, rope_freqs, lse, dq, dk, dv, dtau, dtable, stream);
}

int swin_qkv_proj(const void* x, const void* w, const float* b, void* q, void* k, void* v, int64_t T,
                  int32_t C, int32_t dtype, void* stream)
{
    if (dtype != SWIN_DT_F32 && dtype != SWIN_DT_BF16) return fail(SWIN_EINVAL, "unknown dtype %d", dtype);
    if (T < 0 || C < 1) return fail(SWIN_EINVAL, "bad shape T=%lld C=%d", (long long)T, C);
    if (!swin::proj_supported(C)) return fail(SWIN_EUNSUPPORTED, "C=%d: multiples of 32 up to 512 are built", C);
    if (T > ((int64_t)1 << 40) / C) return fail(SWIN_EUNSUPPORTED, "T=%lld too large", (long long)T);
    if (T == 0) return SWIN_OK;
    if (!x || !w || !q || !k || !v) return fail(SWIN_EINVAL, "NULL x, w, q, k or v");
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)b | (uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15)
        return fail(SWIN_EINVAL, "x, w, b, q, k and v must be 16-byte aligned");
    const size_t es = dtype == SWIN_DT_F32 ? 4 : 2;
    const size_t nx = (size_t)T * C * es, nw = (size_t)3 * C * C * es, nb = b ? (size_t)3 * C * 4 : 0;
    void* outs[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(outs[i], nx, x, nx) || overlaps(outs[i], nx, w, nw) || (b && overlaps(outs[i], nx, b, nb)))
            return fail(SWIN_EINVAL, "an output overlaps an input");
        for (int j = 0; j < i; ++j)
            if (overlaps(outs[i], nx, outs[j], nx)) return fail(SWIN_EINVAL, "q, k and v overlap");
    }
    swin::ProjArgs a{};
    a.x = x; a.w = w; a.b = b; a.q = q; a.k = k; a.v = v;
    a.T = T; a.C = C; a.dtype = dtype;
    return hip_status(swin::launch_qkv_proj(a, (hipStream_t)stream), "swin_qkv_proj launch");
}

int swin_qkv_window_attn_fwd(const swin_attn_desc* d, const void* x, const void* w_qkv, const float* b_qkv,
                             void* out, const float* tau, const float* table, void* stream)
{
    int st = check_desc(d, false);
    if (st) return st;
    if (d->layout != SWIN_LAYOUT_GRID) return fail(SWIN_EUNSUPPORTED, "the fused input layer needs the GRID layout");
    swin::AttnParams p = params_of(d);
    if (!swin::attn_fused_supported(p))
        return fail(SWIN_EUNSUPPORTED, "fused input layer: bf16, 9 <= M <= 16, no rotary positions, "
                                       "C a multiple of 32 up to 192 are built");
    const size_t bytes = (size_t)d->B * d->H * d->W * d->C * 2;
    if (bytes == 0) return SWIN_OK;
    if (!x || !w_qkv || !out) return fail(SWIN_EINVAL, "NULL x, w_qkv or out");
    if (((uintptr_t)x | (uintptr_t)w_qkv | (uintptr_t)out) & 15)
        return fail(SWIN_EINVAL, "x, w_qkv and out must be 16-byte aligned");
    if ((uintptr_t)b_qkv & 3) return fail(SWIN_EINVAL, "b_qkv must be 4-byte aligned");
    if (d->sim == SWIN_SIM_COSINE && !tau) return fail(SWIN_EINVAL, "COSINE needs tau");
    if (d->pos == SWIN_POS_TABLE && !table) return fail(SWIN_EINVAL, "POS_TABLE needs a table");
    const size_t nw = (size_t)3 * d->C * d->C * 2, nb = (size_t)3 * d->C * 4;
    if (overlaps(out, bytes, x, bytes) || overlaps(out, bytes, w_qkv, nw) || (b_qkv && overlaps(out, bytes, b_qkv, nb)))
        return fail(SWIN_EINVAL, "out overlaps x, w_qkv or b_qkv");
    p.out = out;
    p.tau = tau; p.table = table;
    swin::FusedArgs a{x, w_qkv, b_qkv};
    return hip_status(swin::launch_attn_fused(p, a, (hipStream_t)stream), "swin_qkv_window_attn_fwd launch");
}

int swin_proj_post_norm(const void* o, const void* w, const float* b, const void* resid, const float* gamma,
                        const float* beta, float eps, void* y, int64_t T, int32_t C, int32_t dtype, void* stream)
{
    if (dtype != SWIN_DT_F32 && dtype != SWIN_DT_BF16) return fail(SWIN_EINVAL, "unknown dtype %d", dtype);
    if (T < 0 || C < 1) return fail(SWIN_EINVAL, "bad shape T=%lld C=%d", (long long)T, C);
    if (!(eps >= 0.0f) || eps == INFINITY) return fail(SWIN_EINVAL, "eps must be finite and >= 0");
    if (!swin::proj_supported(C)) return fail(SWIN_EUNSUPPORTED, "C=%d: multiples of 32 up to 512 are built", C);
    if (T > ((int64_t)1 << 40) / C) return fail(SWIN_EUNSUPPORTED, "T=%lld too large", (long long)T);
    if (T == 0) return SWIN_OK;
    if (!o || !w || !resid || !gamma || !beta || !y) return fail(SWIN_EINVAL, "NULL o, w, resid, gamma, beta or y");
    if (((uintptr_t)o | (uintptr_t)w | (uintptr_t)b | (uintptr_t)resid | (uintptr_t)gamma | (uintptr_t)beta |
         (uintptr_t)y) & 15)
        return fail(SWIN_EINVAL, "o, w, b, resid, gamma, beta and y must be 16-byte aligned");
    const size_t es = dtype == SWIN_DT_F32 ? 4 : 2;
    const size_t nx = (size_t)T * C * es, nw = (size_t)C * C * es, nc = (size_t)C * 4;
    if (overlaps(y, nx, o, nx) || overlaps(y, nx, w, nw) || (b && overlaps(y, nx, b, nc)) ||
        overlaps(y, nx, gamma, nc) || overlaps(y, nx, beta, nc))
        return fail(SWIN_EINVAL, "y overlaps an input other than resid");
    if (y != resid && overlaps(y, nx, resid, nx)) return fail(SWIN_EINVAL, "y overlaps resid without equalling it");
    swin::ProjArgs a{};
    a.x = o; a.w = w; a.b = b; a.resid = resid; a.gamma = gamma; a.beta = beta; a.eps = eps; a.y = y;
    a.T = T; a.C = C; a.dtype = dtype;
    return hip_status(swin::launch_proj_norm(a, (hipStream_t)stream), "swin_proj_post_norm launch");
}

int swin_dwconv_add(const void* v, const float* w, const float* b, void* out, int32_t B, int32_t H, int32_t W,
                    int32_t C, int32_t dtype, void* stream)
{
    if (dtype != SWIN_DT_F32 && dtype != SWIN_DT_BF16) return fail(SWIN_EINVAL, "unknown dtype %d", dtype);
    if (B < 0 || H < 1 || W < 1 || C < 1) return fail(SWIN_EINVAL, "bad shape B=%d H=%d W=%d C=%d", B, H, W, C);
    if (!swin::dwconv_supported(C, dtype))
        return fail(SWIN_EUNSUPPORTED, "C=%d: multiples of 16 bytes of channels are built", C);
    if ((int64_t)B * H * W > ((int64_t)1 << 31) - 1) return fail(SWIN_EUNSUPPORTED, "grid too large");
    if (B == 0) return SWIN_OK;
    if (!v || !w || !out) return fail(SWIN_EINVAL, "NULL v, w or out");
    if (((uintptr_t)v | (uintptr_t)out) & 15) return fail(SWIN_EINVAL, "v and out must be 16-byte aligned");
    if (((uintptr_t)w | (uintptr_t)b) & 3) return fail(SWIN_EINVAL, "w and b must be 4-byte aligned");
    const size_t es = dtype == SWIN_DT_F32 ? 4 : 2;
    const size_t n = (size_t)B * H * W * C * es;
    if (overlaps(out, n, v, n) || overlaps(out, n, w, (size_t)C * 36) || (b && overlaps(out, n, b, (size_t)C * 4)))
        return fail(SWIN_EINVAL, "out overlaps v, w or b");
    swin::DwconvArgs a{v, w, b, out, B, H, W, C, dtype};
    return hip_status(swin::launch_dwconv_add(a, (hipStream_t)stream), "swin_dwconv_add launch");
}

int swin_window_linear(const swin_attn_desc* d, const void* v, const void* A, const float* bias, void* out,
                       void* stream)
{
    int st = check_desc(d, true);
    if (st) return st;
    if (d->C != d->heads * 32) return fail(SWIN_EUNSUPPORTED, "window linear: head dim %d (32 only)", d->C / d->heads);
    const size_t es = d->dtype == SWIN_DT_F32 ? 4 : 2;
    const size_t bytes = (size_t)d->B * d->H * d->W * d->C * es;
    if (bytes == 0) return SWIN_OK;
    const size_t N = (size_t)d->M * d->M;
    const size_t abytes = (size_t)d->heads * N * N * es;
    if (!v || !A || !out) return fail(SWIN_EINVAL, "NULL v, A or out");
    if (((uintptr_t)v | (uintptr_t)out | (uintptr_t)A) & 15) return fail(SWIN_EINVAL, "v, A and out must be 16-byte aligned");
    if ((uintptr_t)bias & 3) return fail(SWIN_EINVAL, "bias must be 4-byte aligned");
    if (overlaps(out, bytes, v, bytes) || overlaps(out, bytes, A, abytes) ||
        (bias && overlaps(out, bytes, bias, (size_t)d->heads * N * 4)))
        return fail(SWIN_EINVAL, "out overlaps v, A or bias");
    swin::AttnParams p = params_of(d);
    p.v = v; p.out = out;
    const swin::WlinArgs la{A, bias};
    return hip_status(swin::launch_window_linear(p, la, (hipStream_t)stream), "swin_window_linear launch");
}

int swin_cpb_table_bwd(int32_t M, int32_t norm_M, int32_t heads, int32_t hidden, const float* w1,
                       const float* b1, const float* w2, const float* table, const float* dtable,
                       int32_t cpb_mode, float* dw1, float* db1, float* dw2, float* db2, void* stream)
{
    if (cpb_mode < 0 || cpb_mode > (SWIN_CPB_CODE_NORM | SWIN_CPB_SIGMOID16))
        return fail(SWIN_EINVAL, "unknown cpb_mode %d", cpb_mode);
    if (M < 1 || M > 64) return fail(SWIN_EINVAL, "M=%d outside [1, 64]", M);
    if ((cpb_mode & SWIN_CPB_CODE_NORM) && (norm_M < 2 || norm_M > 4096))
        return fail(SWIN_EINVAL, "normalising window %d outside [2, 4096]", norm_M);
    if (heads < 1 || heads > 64) return fail(SWIN_EINVAL, "heads=%d outside [1, 64]", heads);
    if (hidden < 1 || hidden > 4096) return fail(SWIN_EINVAL, "hidden=%d outside [1, 4096]", hidden);
    if (!w1 || !w2 || !dtable || !dw1 || !dw2) return fail(SWIN_EINVAL, "NULL w1, w2, dtable, dw1 or dw2");
    if ((cpb_mode & SWIN_CPB_SIGMOID16) && !table) return fail(SWIN_EINVAL, "SIGMOID16 needs the forward table");
    const size_t tb = (size_t)(2 * M - 1) * (2 * M - 1) * heads * sizeof(float);
    const void* in[5] = {w1, b1, w2, table, dtable};
    const size_t insz[5] = {(size_t)hidden * 8, (size_t)hidden * 4, (size_t)heads * hidden * 4, tb, tb};
    float* out[4] = {dw1, db1, dw2, db2};
    const size_t outsz[4] = {(size_t)hidden * 8, (size_t)hidden * 4, (size_t)heads * hidden * 4,
                             (size_t)heads * 4};
    for (int i = 0; i < 4; ++i) {
        if (!out[i]) continue;
        for (int j = 0; j < 5; ++j)
            if (in[j] && overlaps(out[i], outsz[i], in[j], insz[j]))
                return fail(SWIN_EINVAL, "a gradient overlaps an input");
        for (int j = 0; j < 4; ++j)
            if (j != i && out[j] && overlaps(out[i], outsz[i], out[j], outsz[j]))
                return fail(SWIN_EINVAL, "gradients overlap");
    }
    return hip_status(swin::launch_cpb_table_bwd(M, norm_M, heads, hidden, w1, b1, w2, table, dtable, cpb_mode,
                                                 dw1, db1, dw2, db2, (hipStream_t)stream),
                      "swin_cpb_table_bwd launch");
}

const char* swin_window_attn_kernel(const swin_attn_desc* d)
{
    if (check_desc(d, true) != SWIN_OK) return nullptr;
    switch (kernel_for(params_of(d))) {
    case Kernel::VALU: return "attn_valu_kernel";
    case Kernel::SMALL: return "attn_small_kernel";
    case Kernel::LARGE: return "attn_large_kernel";
    default: return "attn_mfma_kernel";
    }
}

const char* swin_window_attn_bwd_kernel(const swin_attn_desc* d)
{
    if (check_desc(d, true) != SWIN_OK) return nullptr;
    if (d->C != d->heads * 32) {
        fail(SWIN_EUNSUPPORTED, "backward: head dim %d (32 only)", d->C / d->heads);
        return nullptr;
    }
    if (!swin::attn_bwd_supported(params_of(d))) {
        fail(SWIN_EUNSUPPORTED, "backward: M=%d (up to 64, where the statistics and table fit LDS)", d->M);
        return nullptr;
    }
    const swin::AttnParams p = params_of(d);
    if (swin::attn_bwd_small_supported(p)) return "attn_bwd_small_kernel";
    if (swin::attn_bwd_large_supported(p)) return "attn_bwd_large_kernel";
    return "attn_bwd_kernel";
}

}  // extern "C"
