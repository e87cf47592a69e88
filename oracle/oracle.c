/*
 * oracle.c -- plain fp64 CPU reference for windowed multi-head self-attention
 * (forward and backward), the log-spaced continuous position bias table, the
 * window partition / reverse maps, the attention branch's projections and
 * residual post-norm, Iwin's depthwise convolution branch, and LinMapper's
 * in-window linear mapping.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only code that may load this library.
 * It shares no source, header, table or helper with the GPU library.
 *
 * Sources it follows (the pages, by title and section):
 *   [SwinV2]  "Swin Transformer V2: Scaling Up Capacity and Resolution", paper
 *             card: Method items 2-3, eq. 1 (softmax(QK^T/sqrt(d) + B) V),
 *             eq. 2 (cos(q_i,k_j)/tau + B_ij, tau kept at or above 0.01),
 *             eq. 3 (B = G(dx, dy)), eq. 4 (sign(x) log(1+|x|)), the
 *             window-attention and continuous-bias pseudocode, the
 *             Architecture table (G is a 2-layer ReLU MLP, 512 wide in code);
 *             Method item 1 (residual post-norm) and the block pseudocode.
 *   [Flash]   "FLASHSWIN: Unlocking Large Windows and Dense Tokens ...",
 *             abstract: exact softmax attention inside each window, and
 *             window-local 2D rotary position embedding in place of the bias.
 *   [Iwin]    "Iwin Transformer: Hierarchical Vision Transformer using
 *             Interleaved Windows", abstract: interleaved window attention.
 *   [What]    "What Makes for Hierarchical Vision Transformer?", abstract:
 *             self-attention replaced by linear mapping inside each window.
 *
 * Where the pages leave a step open, the reading taken is stated at the step.
 * Nothing here is blocked, fused or reordered: every window, head, query and
 * key is visited in the plain order of the definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Mode codes of this library (its Python wrapper maps names onto them). */
enum { OR_PART_CYCLIC = 0, OR_PART_INTERLEAVED = 1 };
enum { OR_SIM_COSINE = 0, OR_SIM_DOT = 1 };
enum { OR_POS_NONE = 0, OR_POS_TABLE = 1, OR_POS_ROPE2D = 2 };

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* [SwinV2] eq. 4: an offset x is mapped to sign(x) * log(1 + |x|), natural log
 * (the page's worked example, +-2.079 for offset 7 and +-2.773 for offset 15,
 * is ln 8 and ln 16). */
double oracle_log_offset(double x)
{
    double a = log1p(fabs(x));
    if (x > 0) return a;
    if (x < 0) return -a;
    return 0.0;
}

/* The released code's coordinate transform ([SwinV2] card, "Paper vs code",
 * CPB coordinate transform): the offset is divided by (norm_M - 1), where
 * norm_M is the pretrained window when one is set and the window itself
 * otherwise, multiplied by 8, and mapped to sign(u) log2(1 + |u|) / log2(8).
 * Reading: norm_M < 2 has no such transform (the divisor is zero); callers
 * reject it. */
double oracle_code_offset(double x, int norm_M)
{
    const double u = x / (double)(norm_M - 1) * 8.0;
    const double a = log2(1.0 + fabs(u)) / log2(8.0);
    if (u > 0) return a;
    if (u < 0) return -a;
    return 0.0;
}

/* CPB variants, as flags: 0 = the paper's form (eq. 3-4, output unbounded);
 * bit 0 = the code's coordinate table: the transform above, with the row
 * offset as G's first input; bit 1 = the code's bounded output
 * 16 * sigmoid(G) ([SwinV2] card, "Paper vs code", CPB output bounded).
 * 3 = the released code. */
enum { OR_CPB_CODE_NORM = 1, OR_CPB_SIGMOID16 = 2 };

/* G's two inputs for offset (dy, dx) under `mode`.  The paper writes
 * G(dx, dy) (eq. 3): the column offset first.  The page does not say in
 * which order the released code stacks its coordinate table; reading: the
 * row offset first, as the SwinV2 port importable beside this oracle
 * (transformers' Swinv2SelfAttention) builds its table from a row-major
 * meshgrid of (row, column) offsets. */
static void cpb_inputs(int dy, int dx, int mode, int norm_M, double* in0, double* in1)
{
    if (mode & OR_CPB_CODE_NORM) {
        *in0 = oracle_code_offset((double)dy, norm_M);
        *in1 = oracle_code_offset((double)dx, norm_M);
    } else {
        *in0 = oracle_log_offset((double)dx);
        *in1 = oracle_log_offset((double)dy);
    }
}

/* [SwinV2] eq. 3 + eq. 4, Method item 3: the bias for relative offset
 * (dy, dx) = (row offset, column offset) between query and key is the meta
 * network G applied to the log-spaced offset, G(x) = W2 relu(W1 x + b1) + b2.
 * Readings: the offset is query position minus key position; G's inputs are
 * ordered as cpb_inputs says (paper form: column offset first); W1 is hidden x 2
 * row-major, W2 is heads x hidden row-major; a NULL bias vector is zero.
 * The table is stored once per relative position (Method item 3), row
 * (dy + M-1)*(2M-1) + (dx + M-1), one column per head.  mode selects the
 * coordinate transform and output bound (flags above); norm_M is the window
 * whose size less one normalises the offsets under the code's transform. */
int oracle_cpb_table_mode(int M, int norm_M, int heads, int hidden,
                          const double* w1, const double* b1,
                          const double* w2, const double* b2, int mode, double* table)
{
    if (M < 1 || heads < 1 || hidden < 1 || !w1 || !w2 || !table) return 1;
    if (mode < 0 || mode > 3) return 1;
    if ((mode & OR_CPB_CODE_NORM) && norm_M < 2) return 1;
    const int S = 2 * M - 1;
    double* h = (double*)malloc((size_t)hidden * sizeof(double));
    if (!h) return 2;
    for (int dy = -(M - 1); dy <= M - 1; ++dy) {
        for (int dx = -(M - 1); dx <= M - 1; ++dx) {
            double in0, in1;
            cpb_inputs(dy, dx, mode, norm_M, &in0, &in1);
            for (int j = 0; j < hidden; ++j) {
                double a = w1[2 * j] * in0 + w1[2 * j + 1] * in1 + (b1 ? b1[j] : 0.0);
                h[j] = a > 0.0 ? a : 0.0;                 /* ReLU between the two layers */
            }
            double* row = table + ((size_t)(dy + M - 1) * S + (size_t)(dx + M - 1)) * heads;
            for (int o = 0; o < heads; ++o) {
                double acc = b2 ? b2[o] : 0.0;
                for (int j = 0; j < hidden; ++j) acc += w2[(size_t)o * hidden + j] * h[j];
                row[o] = (mode & OR_CPB_SIGMOID16) ? 16.0 / (1.0 + exp(-acc)) : acc;
            }
        }
    }
    free(h);
    return 0;
}

/* The paper's form (mode 0). */
int oracle_cpb_table(int M, int heads, int hidden,
                     const double* w1, const double* b1,
                     const double* w2, const double* b2, double* table)
{
    return oracle_cpb_table_mode(M, M, heads, hidden, w1, b1, w2, b2, 0, table);
}

/* Shape rule shared by every entry point here: windows tile the grid exactly. */
static int bad_shape(int B, int H, int W, int C, int M, int shift, int part)
{
    if (B < 0 || H < 1 || W < 1 || C < 1 || M < 1) return 1;
    if (H % M || W % M) return 1;
    if (shift < 0 || shift >= M) return 1;
    if (part != OR_PART_CYCLIC && part != OR_PART_INTERLEAVED) return 1;
    if (part == OR_PART_INTERLEAVED && shift != 0) return 1;
    return 0;
}

/* Grid position of local token (r, c) of window (wr, wc).
 * Cyclic ([SwinV2] "window partitioning is Swin V1's"; the shift is not shown
 * on the page).  Reading: the grid is rolled by -shift on both axes, then cut
 * into M x M windows in row-major window order, tokens row-major inside.
 * Interleaved ([Iwin] abstract; the rule itself is not on the page).  Reading:
 * window (wr, wc) gathers every (H/M)-th row starting at wr and every (W/M)-th
 * column starting at wc, so local (r, c) is grid (wr + r*H/M, wc + c*W/M). */
static void grid_pos(int H, int W, int M, int shift, int part,
                     int wr, int wc, int r, int c, int* gi, int* gj)
{
    if (part == OR_PART_INTERLEAVED) {
        *gi = wr + r * (H / M);
        *gj = wc + c * (W / M);
    } else {
        *gi = (wr * M + r + shift) % H;
        *gj = (wc * M + c + shift) % W;
    }
}

/* Region of a rolled coordinate p along an axis of length L (cyclic shift s > 0):
 * [0, L-M) -> 0, [L-M, L-s) -> 1, [L-s, L) -> 2.  Tokens rolled in from the far
 * edge (label 2) and the ones they land next to (label 1) never attend to each
 * other.  With s == 0 every token is region 0. */
static int axis_region(int p, int L, int M, int s)
{
    if (s == 0) return 0;
    if (p < L - M) return 0;
    if (p < L - s) return 1;
    return 2;
}

/* Byte-exact gather: xw[b*nW + wr*(W/M) + wc][r*M + c][:] = x[b][gi][gj][:]. */
int oracle_partition(const void* x, void* xw, int B, int H, int W, int C,
                     int M, int shift, int part, int elem_size)
{
    if (bad_shape(B, H, W, C, M, shift, part) || elem_size < 1) return 1;
    const int nwr = H / M, nwc = W / M, N = M * M;
    const size_t row = (size_t)C * elem_size;
    const char* src = (const char*)x;
    char* dst = (char*)xw;
    for (int b = 0; b < B; ++b)
        for (int wr = 0; wr < nwr; ++wr)
            for (int wc = 0; wc < nwc; ++wc)
                for (int r = 0; r < M; ++r)
                    for (int c = 0; c < M; ++c) {
                        int gi, gj;
                        grid_pos(H, W, M, shift, part, wr, wc, r, c, &gi, &gj);
                        size_t w = ((size_t)b * nwr + wr) * nwc + wc;
                        memcpy(dst + (w * N + (size_t)r * M + c) * row,
                               src + (((size_t)b * H + gi) * W + gj) * row, row);
                    }
    return 0;
}

/* Byte-exact scatter, the inverse of oracle_partition. */
int oracle_reverse(const void* xw, void* x, int B, int H, int W, int C,
                   int M, int shift, int part, int elem_size)
{
    if (bad_shape(B, H, W, C, M, shift, part) || elem_size < 1) return 1;
    const int nwr = H / M, nwc = W / M, N = M * M;
    const size_t row = (size_t)C * elem_size;
    const char* src = (const char*)xw;
    char* dst = (char*)x;
    for (int b = 0; b < B; ++b)
        for (int wr = 0; wr < nwr; ++wr)
            for (int wc = 0; wc < nwc; ++wc)
                for (int r = 0; r < M; ++r)
                    for (int c = 0; c < M; ++c) {
                        int gi, gj;
                        grid_pos(H, W, M, shift, part, wr, wc, r, c, &gi, &gj);
                        size_t w = ((size_t)b * nwr + wr) * nwc + wc;
                        memcpy(dst + (((size_t)b * H + gi) * W + gj) * row,
                               src + (w * N + (size_t)r * M + c) * row, row);
                    }
    return 0;
}

/* [Flash] abstract: window-local 2D rotary embedding (no formula on the page).
 * Reading: channels [0, d/2) turn with the local row, [d/2, d) with the local
 * column; inside each half, pair (2k, 2k+1), k < d/4, turns by pos * theta_k,
 * theta_k = base^(-k/(d/4)), or the caller's per-head frequency when given
 * (freqs = 2 x d/4: row half then column half). */
static void rope_rotate(double* x, int d, int r, int c,
                        const double* freqs, double base)
{
    const int q4 = d / 4;
    for (int half = 0; half < 2; ++half) {
        const int pos = half == 0 ? r : c;
        for (int k = 0; k < q4; ++k) {
            double theta = freqs ? freqs[half * q4 + k] : pow(base, -(double)k / (double)q4);
            double a = (double)pos * theta;
            double cs = cos(a), sn = sin(a);
            double* p = x + half * (d / 2) + 2 * k;
            double x0 = p[0], x1 = p[1];
            p[0] = x0 * cs - x1 * sn;
            p[1] = x0 * sn + x1 * cs;
        }
    }
}

/* [SwinV2] eq. 2 normalize(): x / max(||x||_2, 1e-12) (the page gives no epsilon). */
static void unit_normalize(double* x, int d)
{
    double ss = 0.0;
    for (int e = 0; e < d; ++e) ss += x[e] * x[e];
    double n = sqrt(ss);
    if (n < 1e-12) n = 1e-12;
    for (int e = 0; e < d; ++e) x[e] /= n;
}

/*
 * Windowed multi-head self-attention forward over (B, H, W, C) grids,
 * channels last, head h owning channels [h*d, (h+1)*d), d = C / heads.
 *
 * Per (batch, window, head), in the pages' order:
 *   1. gather the window's M*M tokens (grid_pos), local order t = r*M + c;
 *   2. ROPE2D: rotate q and k by their local (r, c)          [Flash];
 *   3. COSINE: q^ = q/max(||q||,eps), k^ likewise, logit = q^.k^ / max(tau_h, tau_min)
 *                                                             [SwinV2] eq. 2;
 *      DOT:    logit = q.k / sqrt(d)                          [SwinV2] eq. 1;
 *   4. TABLE:  logit += table[(ri-rj+M-1)*(2M-1) + (ci-cj+M-1)][h]  [SwinV2] eq. 2-3;
 *   5. cyclic shift: a key in another region than the query is excluded
 *      outright (weight exactly 0; a finite penalty would not block it,
 *      since |cos|/0.01 reaches 100 and the bias is unbounded);
 *   6. softmax over the remaining keys: subtract the row max, exponentiate,
 *      divide by the sum                                      [SwinV2] pseudocode;
 *   7. o_i = sum_j p_ij v_j, written back to query i's grid position.
 *
 * windows: optional list of global window ids (b*nW + wr*(W/M) + wc) to
 * compute; NULL means all.  Only those windows' tokens of `out` are written.
 * weights: optional n_windows x heads x N x N array of the softmax weights.
 * lse: optional n_windows x heads x N array: per query, the natural-log
 *      log-sum-exp of its row of logits over the keys it may attend to.
 * Returns 0, or 1 on a bad argument.
 */
int oracle_window_attn(int B, int H, int W, int C, int heads, int M, int shift,
                       int part, int sim, int pos, double tau_min, double rope_base,
                       const double* q, const double* k, const double* v,
                       const double* tau, const double* table, const double* rope_freqs,
                       const int64_t* windows, int64_t n_windows,
                       double* out, double* weights, double* lse)
{
    if (bad_shape(B, H, W, C, M, shift, part)) return 1;
    if (heads < 1 || C % heads) return 1;
    const int d = C / heads;
    if (sim != OR_SIM_COSINE && sim != OR_SIM_DOT) return 1;
    if (pos != OR_POS_NONE && pos != OR_POS_TABLE && pos != OR_POS_ROPE2D) return 1;
    if (sim == OR_SIM_COSINE && !tau) return 1;
    if (pos == OR_POS_TABLE && !table) return 1;
    if (pos == OR_POS_ROPE2D && d % 4) return 1;
    if (!q || !k || !v || !out) return 1;

    const int nwr = H / M, nwc = W / M, N = M * M;
    const int64_t nW = (int64_t)nwr * nwc;
    const int64_t total = windows ? n_windows : (int64_t)B * nW;
    if (windows) {
        for (int64_t i = 0; i < n_windows; ++i)
            if (windows[i] < 0 || windows[i] >= (int64_t)B * nW) return 1;
    }
    const int S = 2 * M - 1;
    const double dot_scale = 1.0 / sqrt((double)d);
    int failed = 0;

    #pragma omp parallel
    {
        double* qs = (double*)malloc((size_t)N * d * sizeof(double));
        double* ks = (double*)malloc((size_t)N * d * sizeof(double));
        double* vs = (double*)malloc((size_t)N * d * sizeof(double));
        double* lg = (double*)malloc((size_t)N * sizeof(double));
        char* allowed = (char*)malloc((size_t)N);
        int* gi = (int*)malloc((size_t)N * sizeof(int));
        int* gj = (int*)malloc((size_t)N * sizeof(int));
        int* region = (int*)malloc((size_t)N * sizeof(int));
        if (!qs || !ks || !vs || !lg || !allowed || !gi || !gj || !region) {
            #pragma omp atomic write
            failed = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < total * heads; ++u) {
                const int64_t wi = u / heads;
                const int h = (int)(u % heads);
                const int64_t gw = windows ? windows[wi] : wi;
                const int b = (int)(gw / nW);
                const int wr = (int)((gw % nW) / nwc);
                const int wc = (int)(gw % nwc);

                /* 1. gather, with region labels in rolled coordinates */
                for (int t = 0; t < N; ++t) {
                    const int r = t / M, c = t % M;
                    grid_pos(H, W, M, shift, part, wr, wc, r, c, &gi[t], &gj[t]);
                    region[t] = (part == OR_PART_CYCLIC)
                        ? 3 * axis_region(wr * M + r, H, M, shift) + axis_region(wc * M + c, W, M, shift)
                        : 0;
                    const size_t base = (((size_t)b * H + gi[t]) * W + gj[t]) * C + (size_t)h * d;
                    for (int e = 0; e < d; ++e) {
                        qs[(size_t)t * d + e] = q[base + e];
                        ks[(size_t)t * d + e] = k[base + e];
                        vs[(size_t)t * d + e] = v[base + e];
                    }
                    /* 2. rotary position, window-local */
                    if (pos == OR_POS_ROPE2D) {
                        const double* f = rope_freqs ? rope_freqs + (size_t)h * 2 * (d / 4) : NULL;
                        rope_rotate(qs + (size_t)t * d, d, r, c, f, rope_base);
                        rope_rotate(ks + (size_t)t * d, d, r, c, f, rope_base);
                    }
                    /* 3a. unit-normalise for the cosine */
                    if (sim == OR_SIM_COSINE) {
                        unit_normalize(qs + (size_t)t * d, d);
                        unit_normalize(ks + (size_t)t * d, d);
                    }
                }
                double inv_tau = 0.0;
                if (sim == OR_SIM_COSINE) {
                    double t_h = tau[h] > tau_min ? tau[h] : tau_min;   /* max(tau, 0.01) */
                    inv_tau = 1.0 / t_h;
                }

                for (int i = 0; i < N; ++i) {
                    const int ri = i / M, ci = i % M;
                    double mx = -INFINITY;
                    for (int j = 0; j < N; ++j) {
                        const int rj = j / M, cj = j % M;
                        double s = 0.0;
                        for (int e = 0; e < d; ++e) s += qs[(size_t)i * d + e] * ks[(size_t)j * d + e];
                        double l = (sim == OR_SIM_COSINE) ? s * inv_tau : s * dot_scale;
                        if (pos == OR_POS_TABLE)
                            l += table[((size_t)(ri - rj + M - 1) * S + (size_t)(ci - cj + M - 1)) * heads + h];
                        lg[j] = l;
                        allowed[j] = (char)(region[j] == region[i]);
                        if (allowed[j] && l > mx) mx = l;
                    }
                    double sum = 0.0;
                    for (int j = 0; j < N; ++j) {
                        lg[j] = allowed[j] ? exp(lg[j] - mx) : 0.0;
                        sum += lg[j];
                    }
                    for (int j = 0; j < N; ++j) lg[j] /= sum;
                    /* log-sum-exp of the row's logits (natural log): what a
                       backward needs to rebuild the weights */
                    if (lse) lse[((size_t)wi * heads + h) * N + i] = mx + log(sum);
                    if (weights) {
                        double* wrow = weights + (((size_t)wi * heads + h) * N + i) * (size_t)N;
                        for (int j = 0; j < N; ++j) wrow[j] = lg[j];
                    }
                    const size_t ob = (((size_t)b * H + gi[i]) * W + gj[i]) * C + (size_t)h * d;
                    for (int e = 0; e < d; ++e) {
                        double acc = 0.0;
                        for (int j = 0; j < N; ++j) acc += lg[j] * vs[(size_t)j * d + e];
                        out[ob + e] = acc;
                    }
                }
            }
        }
        free(qs); free(ks); free(vs); free(lg); free(allowed); free(gi); free(gj); free(region);
    }
    return failed ? 2 : 0;
}

/* Cosine similarities q^_i . k^_j of one (window, head), N x N, for range checks
 * ([SwinV2] eq. 2: cos lies in [-1, 1]). Same gather and rotation as above. */
int oracle_window_cosines(int B, int H, int W, int C, int heads, int M, int shift,
                          int part, int pos, double rope_base,
                          const double* q, const double* k, const double* rope_freqs,
                          int64_t window, int head, double* cosines)
{
    if (bad_shape(B, H, W, C, M, shift, part) || heads < 1 || C % heads) return 1;
    const int d = C / heads, nwr = H / M, nwc = W / M, N = M * M;
    const int64_t nW = (int64_t)nwr * nwc;
    if (window < 0 || window >= (int64_t)B * nW || head < 0 || head >= heads) return 1;
    if (pos == OR_POS_ROPE2D && d % 4) return 1;
    const int b = (int)(window / nW), wr = (int)((window % nW) / nwc), wc = (int)(window % nwc);
    double* qs = (double*)malloc((size_t)N * d * sizeof(double));
    double* ks = (double*)malloc((size_t)N * d * sizeof(double));
    if (!qs || !ks) { free(qs); free(ks); return 2; }
    for (int t = 0; t < N; ++t) {
        int r = t / M, c = t % M, i0, j0;
        grid_pos(H, W, M, shift, part, wr, wc, r, c, &i0, &j0);
        const size_t base = (((size_t)b * H + i0) * W + j0) * C + (size_t)head * d;
        for (int e = 0; e < d; ++e) { qs[(size_t)t * d + e] = q[base + e]; ks[(size_t)t * d + e] = k[base + e]; }
        if (pos == OR_POS_ROPE2D) {
            const double* f = rope_freqs ? rope_freqs + (size_t)head * 2 * (d / 4) : NULL;
            rope_rotate(qs + (size_t)t * d, d, r, c, f, rope_base);
            rope_rotate(ks + (size_t)t * d, d, r, c, f, rope_base);
        }
        unit_normalize(qs + (size_t)t * d, d);
        unit_normalize(ks + (size_t)t * d, d);
    }
    for (int i = 0; i < N; ++i)
        for (int j = 0; j < N; ++j) {
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += qs[(size_t)i * d + e] * ks[(size_t)j * d + e];
            cosines[(size_t)i * N + j] = s;
        }
    free(qs); free(ks);
    return 0;
}

/*
 * Backward of oracle_window_attn: given dout = dLoss/dout, the gradients of
 * the same loss with respect to q, k, v (same layout), tau (heads) and the
 * bias table ((2M-1)^2 x heads).  The chain rule applied to the forward steps
 * above, in reverse, per (batch, window, head):
 *   p = softmax over allowed keys (recomputed), o_i = sum_j p_ij v_j
 *   dv_j   = sum_i p_ij dout_i
 *   dp_ij  = dout_i . v_j,  D_i = sum_j p_ij dp_ij
 *   dl_ij  = p_ij (dp_ij - D_i)             (0 for excluded keys: p_ij = 0)
 *   TABLE:  dtable[offset(i, j)][h] += dl_ij
 *   COSINE: ds_ij = dl_ij / tau';  dtau_h += sum dl_ij * cos_ij * (-1/tau_h^2)
 *           when tau_h > tau_min (the floor max(tau, tau_min) passes no
 *           gradient below it); dq^_i = sum_j ds_ij k^_j, dk^_j = sum_i ds_ij q^_i;
 *           through x^ = x / max(||x||, eps): dx = (dx^ - x^ (x^ . dx^)) / ||x||
 *           when ||x|| > eps, else dx^ / eps;
 *   DOT:    dq_i = sum_j dl_ij k_j / sqrt(d), dk_j = sum_i dl_ij q_i / sqrt(d);
 *   ROPE2D: the rotation is orthogonal, so dq = R^T dq~ (rotate by -pos).
 * Each token belongs to one window, so dq, dk, dv are written, not summed;
 * dtau and dtable are sums over all windows.  Any of dtau (DOT) and dtable
 * (not TABLE) may be NULL.  Returns 0, or 1 on a bad argument.
 *
 * Given forward statistics (FLASHSWIN abstract: exact attention whose weights
 * are never stored, so a backward rebuilds them from what the forward kept):
 * when `out` (B, H, W, C, the forward's output as the caller holds it) is
 * given, D_i = dout_i . out_i replaces sum_j p_ij dp_ij (the two are equal for
 * the exact output); when `lse` (windows x heads x N, natural log, window-
 * local query order) is given, p_ij = exp(l_ij - lse_i) over the allowed keys
 * replaces the softmax (equal for the exact log-sum-exp).  These are the
 * gradients a backward computes from the statistics it is handed.
 */
int oracle_window_attn_bwd_given(int B, int H, int W, int C, int heads, int M, int shift,
                                 int part, int sim, int pos, double tau_min, double rope_base,
                                 const double* q, const double* k, const double* v, const double* dout,
                                 const double* tau, const double* table, const double* rope_freqs,
                                 const double* out, const double* lse,
                                 double* dq, double* dk, double* dv, double* dtau, double* dtable)
{
    if (bad_shape(B, H, W, C, M, shift, part)) return 1;
    if (heads < 1 || C % heads) return 1;
    const int d = C / heads;
    if (sim != OR_SIM_COSINE && sim != OR_SIM_DOT) return 1;
    if (pos != OR_POS_NONE && pos != OR_POS_TABLE && pos != OR_POS_ROPE2D) return 1;
    if (sim == OR_SIM_COSINE && !tau) return 1;
    if (pos == OR_POS_TABLE && !table) return 1;
    if (pos == OR_POS_ROPE2D && d % 4) return 1;
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;

    const int nwr = H / M, nwc = W / M, N = M * M, S = 2 * M - 1;
    const int64_t nW = (int64_t)nwr * nwc, total = (int64_t)B * nW;
    const double dot_scale = 1.0 / sqrt((double)d);
    if (dtau) for (int h = 0; h < heads; ++h) dtau[h] = 0.0;
    if (dtable) memset(dtable, 0, (size_t)S * S * heads * sizeof(double));
    int failed = 0;

    #pragma omp parallel
    {
        const size_t nd = (size_t)N * d;
        double* qx = (double*)malloc(nd * sizeof(double));    /* rotated, before normalising */
        double* kx = (double*)malloc(nd * sizeof(double));
        double* qs = (double*)malloc(nd * sizeof(double));    /* operands of the logits */
        double* ks = (double*)malloc(nd * sizeof(double));
        double* vs = (double*)malloc(nd * sizeof(double));
        double* gs = (double*)malloc(nd * sizeof(double));    /* dout */
        double* os = (double*)malloc(nd * sizeof(double));    /* the given forward output */
        double* gq = (double*)malloc(nd * sizeof(double));
        double* gk = (double*)malloc(nd * sizeof(double));
        double* gv = (double*)malloc(nd * sizeof(double));
        double* p = (double*)malloc((size_t)N * N * sizeof(double));
        double* dl = (double*)malloc((size_t)N * N * sizeof(double));
        int* gi = (int*)malloc((size_t)N * sizeof(int));
        int* gj = (int*)malloc((size_t)N * sizeof(int));
        int* region = (int*)malloc((size_t)N * sizeof(int));
        double* my_dtau = (double*)calloc((size_t)heads, sizeof(double));
        double* my_dtable = dtable ? (double*)calloc((size_t)S * S * heads, sizeof(double)) : NULL;
        if (!qx || !kx || !qs || !ks || !vs || !gs || !os || !gq || !gk || !gv || !p || !dl || !gi || !gj ||
            !region || !my_dtau || (dtable && !my_dtable)) {
            #pragma omp atomic write
            failed = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < total * heads; ++u) {
                const int64_t gw = u / heads;
                const int h = (int)(u % heads);
                const int b = (int)(gw / nW);
                const int wr = (int)((gw % nW) / nwc);
                const int wc = (int)(gw % nwc);
                const double* f = (pos == OR_POS_ROPE2D && rope_freqs) ? rope_freqs + (size_t)h * 2 * (d / 4) : NULL;

                /* forward recomputation: gather, rotate, normalise */
                for (int t = 0; t < N; ++t) {
                    const int r = t / M, c = t % M;
                    grid_pos(H, W, M, shift, part, wr, wc, r, c, &gi[t], &gj[t]);
                    region[t] = (part == OR_PART_CYCLIC)
                        ? 3 * axis_region(wr * M + r, H, M, shift) + axis_region(wc * M + c, W, M, shift)
                        : 0;
                    const size_t base = (((size_t)b * H + gi[t]) * W + gj[t]) * C + (size_t)h * d;
                    for (int e = 0; e < d; ++e) {
                        qx[(size_t)t * d + e] = q[base + e];
                        kx[(size_t)t * d + e] = k[base + e];
                        vs[(size_t)t * d + e] = v[base + e];
                        gs[(size_t)t * d + e] = dout[base + e];
                        os[(size_t)t * d + e] = out ? out[base + e] : 0.0;
                    }
                    if (pos == OR_POS_ROPE2D) {
                        rope_rotate(qx + (size_t)t * d, d, r, c, f, rope_base);
                        rope_rotate(kx + (size_t)t * d, d, r, c, f, rope_base);
                    }
                    for (int e = 0; e < d; ++e) {
                        qs[(size_t)t * d + e] = qx[(size_t)t * d + e];
                        ks[(size_t)t * d + e] = kx[(size_t)t * d + e];
                    }
                    if (sim == OR_SIM_COSINE) {
                        unit_normalize(qs + (size_t)t * d, d);
                        unit_normalize(ks + (size_t)t * d, d);
                    }
                }
                double t_h = 1.0, inv_tau = 0.0;
                if (sim == OR_SIM_COSINE) {
                    t_h = tau[h] > tau_min ? tau[h] : tau_min;
                    inv_tau = 1.0 / t_h;
                }
                const double scale = (sim == OR_SIM_COSINE) ? inv_tau : dot_scale;

                /* softmax weights, as in the forward */
                for (int i = 0; i < N; ++i) {
                    const int ri = i / M, ci = i % M;
                    double mx = -INFINITY;
                    double* pr = p + (size_t)i * N;
                    for (int j = 0; j < N; ++j) {
                        const int rj = j / M, cj = j % M;
                        double s = 0.0;
                        for (int e = 0; e < d; ++e) s += qs[(size_t)i * d + e] * ks[(size_t)j * d + e];
                        double l = s * scale;
                        if (pos == OR_POS_TABLE)
                            l += table[((size_t)(ri - rj + M - 1) * S + (size_t)(ci - cj + M - 1)) * heads + h];
                        pr[j] = (region[j] == region[i]) ? l : -INFINITY;
                        if (pr[j] > mx) mx = pr[j];
                    }
                    if (lse) {
                        /* the weights rebuilt from the given log-sum-exp */
                        const double li = lse[((size_t)gw * heads + h) * N + i];
                        for (int j = 0; j < N; ++j) pr[j] = exp(pr[j] - li);
                        continue;
                    }
                    double sum = 0.0;
                    for (int j = 0; j < N; ++j) {
                        pr[j] = exp(pr[j] - mx);              /* excluded keys: exp(-inf) = 0 */
                        sum += pr[j];
                    }
                    for (int j = 0; j < N; ++j) pr[j] /= sum;
                }

                /* dv, dp, D, dl */
                for (size_t x = 0; x < nd; ++x) { gv[x] = 0.0; gq[x] = 0.0; gk[x] = 0.0; }
                for (int i = 0; i < N; ++i) {
                    const double* pr = p + (size_t)i * N;
                    double* dr = dl + (size_t)i * N;
                    double Di = 0.0;
                    for (int j = 0; j < N; ++j) {
                        double dp = 0.0;
                        for (int e = 0; e < d; ++e) dp += gs[(size_t)i * d + e] * vs[(size_t)j * d + e];
                        dr[j] = dp;
                        Di += pr[j] * dp;
                        for (int e = 0; e < d; ++e) gv[(size_t)j * d + e] += pr[j] * gs[(size_t)i * d + e];
                    }
                    if (out) {
                        Di = 0.0;
                        for (int e = 0; e < d; ++e) Di += gs[(size_t)i * d + e] * os[(size_t)i * d + e];
                    }
                    for (int j = 0; j < N; ++j) dr[j] = pr[j] * (dr[j] - Di);
                }

                /* bias table, tau, and the logit operands */
                for (int i = 0; i < N; ++i) {
                    const int ri = i / M, ci = i % M;
                    for (int j = 0; j < N; ++j) {
                        const int rj = j / M, cj = j % M;
                        const double g = dl[(size_t)i * N + j];
                        if (pos == OR_POS_TABLE && my_dtable)
                            my_dtable[((size_t)(ri - rj + M - 1) * S + (size_t)(ci - cj + M - 1)) * heads + h] += g;
                        if (sim == OR_SIM_COSINE && tau[h] > tau_min) {
                            double cs = 0.0;
                            for (int e = 0; e < d; ++e) cs += qs[(size_t)i * d + e] * ks[(size_t)j * d + e];
                            my_dtau[h] += g * cs * (-1.0 / (tau[h] * tau[h]));
                        }
                        for (int e = 0; e < d; ++e) {
                            gq[(size_t)i * d + e] += g * scale * ks[(size_t)j * d + e];
                            gk[(size_t)j * d + e] += g * scale * qs[(size_t)i * d + e];
                        }
                    }
                }

                /* through the normalisation and the rotation, then scatter */
                for (int t = 0; t < N; ++t) {
                    const int r = t / M, c = t % M;
                    for (int which = 0; which < 2; ++which) {
                        double* g = (which == 0 ? gq : gk) + (size_t)t * d;
                        const double* x = (which == 0 ? qx : kx) + (size_t)t * d;
                        const double* xh = (which == 0 ? qs : ks) + (size_t)t * d;
                        if (sim == OR_SIM_COSINE) {
                            double ss = 0.0, proj = 0.0;
                            for (int e = 0; e < d; ++e) { ss += x[e] * x[e]; proj += xh[e] * g[e]; }
                            const double n = sqrt(ss);
                            if (n > 1e-12) { for (int e = 0; e < d; ++e) g[e] = (g[e] - xh[e] * proj) / n; }
                            else { for (int e = 0; e < d; ++e) g[e] = g[e] / 1e-12; }
                        }
                        if (pos == OR_POS_ROPE2D) rope_rotate(g, d, -r, -c, f, rope_base);
                    }
                    const size_t base = (((size_t)b * H + gi[t]) * W + gj[t]) * C + (size_t)h * d;
                    for (int e = 0; e < d; ++e) {
                        dq[base + e] = gq[(size_t)t * d + e];
                        dk[base + e] = gk[(size_t)t * d + e];
                        dv[base + e] = gv[(size_t)t * d + e];
                    }
                }
            }
            #pragma omp critical
            {
                if (dtau) for (int h = 0; h < heads; ++h) dtau[h] += my_dtau[h];
                if (dtable) for (size_t x = 0; x < (size_t)S * S * heads; ++x) dtable[x] += my_dtable[x];
            }
        }
        free(qx); free(kx); free(qs); free(ks); free(vs); free(gs); free(os); free(gq); free(gk); free(gv);
        free(p); free(dl); free(gi); free(gj); free(region); free(my_dtau); free(my_dtable);
    }
    return failed ? 2 : 0;
}

/* The backward with its own statistics: the softmax recomputed, D_i from it. */
int oracle_window_attn_bwd(int B, int H, int W, int C, int heads, int M, int shift,
                           int part, int sim, int pos, double tau_min, double rope_base,
                           const double* q, const double* k, const double* v, const double* dout,
                           const double* tau, const double* table, const double* rope_freqs,
                           double* dq, double* dk, double* dv, double* dtau, double* dtable)
{
    return oracle_window_attn_bwd_given(B, H, W, C, heads, M, shift, part, sim, pos, tau_min, rope_base,
                                        q, k, v, dout, tau, table, rope_freqs, NULL, NULL,
                                        dq, dk, dv, dtau, dtable);
}

/*
 * Backward of oracle_cpb_table_mode: given dtable ((2M-1)^2 x heads), the
 * gradients of G's parameters (dw1 hidden x 2, db1 hidden, dw2 heads x hidden,
 * db2 heads), written.  Per table row, recompute a = W1 x + b1, hid = relu(a),
 * g = W2 hid + b2; SIGMOID16: dg = dtable * 16 s (1 - s), s = sigmoid(g);
 * dW2 += dg hid^T, db2 += dg, dhid = W2^T dg, da = dhid [a > 0],
 * dW1 += da x^T, db1 += da.  db1/db2 may be NULL.  Returns 0 or 1.
 */
int oracle_cpb_table_bwd(int M, int norm_M, int heads, int hidden,
                         const double* w1, const double* b1, const double* w2, const double* b2,
                         int mode, const double* dtable,
                         double* dw1, double* db1, double* dw2, double* db2)
{
    if (M < 1 || heads < 1 || hidden < 1 || !w1 || !w2 || !dtable || !dw1 || !dw2) return 1;
    if (mode < 0 || mode > 3) return 1;
    if ((mode & OR_CPB_CODE_NORM) && norm_M < 2) return 1;
    const int S = 2 * M - 1;
    double* a = (double*)malloc((size_t)hidden * sizeof(double));
    double* dg = (double*)malloc((size_t)heads * sizeof(double));
    if (!a || !dg) { free(a); free(dg); return 2; }
    memset(dw1, 0, (size_t)hidden * 2 * sizeof(double));
    memset(dw2, 0, (size_t)heads * hidden * sizeof(double));
    if (db1) memset(db1, 0, (size_t)hidden * sizeof(double));
    if (db2) memset(db2, 0, (size_t)heads * sizeof(double));
    for (int dy = -(M - 1); dy <= M - 1; ++dy)
        for (int dx = -(M - 1); dx <= M - 1; ++dx) {
            double in0, in1;
            cpb_inputs(dy, dx, mode, norm_M, &in0, &in1);
            const double* grow = dtable + ((size_t)(dy + M - 1) * S + (size_t)(dx + M - 1)) * heads;
            for (int j = 0; j < hidden; ++j) a[j] = w1[2 * j] * in0 + w1[2 * j + 1] * in1 + (b1 ? b1[j] : 0.0);
            for (int o = 0; o < heads; ++o) {
                dg[o] = grow[o];
                if (mode & OR_CPB_SIGMOID16) {
                    double g = b2 ? b2[o] : 0.0;
                    for (int j = 0; j < hidden; ++j) g += w2[(size_t)o * hidden + j] * (a[j] > 0.0 ? a[j] : 0.0);
                    const double s = 1.0 / (1.0 + exp(-g));
                    dg[o] *= 16.0 * s * (1.0 - s);
                }
                if (db2) db2[o] += dg[o];
            }
            for (int j = 0; j < hidden; ++j) {
                const double hj = a[j] > 0.0 ? a[j] : 0.0;
                double dh = 0.0;
                for (int o = 0; o < heads; ++o) {
                    dw2[(size_t)o * hidden + j] += dg[o] * hj;
                    dh += w2[(size_t)o * hidden + j] * dg[o];
                }
                const double da = a[j] > 0.0 ? dh : 0.0;
                dw1[2 * j] += da * in0;
                dw1[2 * j + 1] += da * in1;
                if (db1) db1[j] += da;
            }
        }
    free(a); free(dg);
    return 0;
}

/* ---------------------------------------------------------------------------
 * The steps either side of the window attention in a Swin V2 block ([SwinV2]
 * Method item 1 "Residual post-norm" and the block pseudocode; the block keeps
 * Swin's layout, Method opening paragraph).  Readings: the attention branch
 * maps its input features through a linear layer to queries, keys and values
 * (C -> 3C, in that order along the output, each with a bias) and its output
 * through a linear layer C -> C with a bias; norm_1 is a layer norm over the C
 * channels of each token (biased variance, eps inside the square root) with a
 * per-channel scale and shift, applied to the branch output before it is added
 * to the main path.
 * ------------------------------------------------------------------------- */

/* y[t][n] = sum_c x[t][c] w[n][c] + b[n]  (x: T x in, w: out x in, b: out or
 * NULL, y: T x out), every product and sum in fp64 in index order. */
int oracle_linear(const double* x, const double* w, const double* b, double* y, int64_t T, int in, int out)
{
    if (T < 0 || in < 1 || out < 1 || (T > 0 && (!x || !w || !y))) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int n = 0; n < out; ++n) {
            double s = b ? b[n] : 0.0;
            for (int c = 0; c < in; ++c) s += x[t * in + c] * w[(size_t)n * in + c];
            y[t * out + n] = s;
        }
    return 0;
}

/* y[t] = resid[t] + gamma * (z[t] - mean(z[t])) / sqrt(var(z[t]) + eps) + beta,
 * mean and (biased) variance over the C channels of token t. */
int oracle_post_norm(const double* resid, const double* z, const double* gamma, const double* beta,
                     double eps, double* y, int64_t T, int C)
{
    if (T < 0 || C < 1 || !(eps >= 0.0) || (T > 0 && (!resid || !z || !gamma || !beta || !y))) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double* zt = z + t * C;
        double mean = 0.0;
        for (int c = 0; c < C; ++c) mean += zt[c];
        mean /= C;
        double var = 0.0;
        for (int c = 0; c < C; ++c) var += (zt[c] - mean) * (zt[c] - mean);
        var /= C;
        const double inv = 1.0 / sqrt(var + eps);
        for (int c = 0; c < C; ++c)
            y[t * C + c] = resid[t * C + c] + gamma[c] * (zt[c] - mean) * inv + beta[c];
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Iwin's convolution branch ([Iwin] abstract: the block couples interleaved
 * window attention with a depthwise convolution that links each token to its
 * local neighbours).  Reading: a 3 x 3 depthwise convolution of v over the
 * (H, W) grid of each image, zero padding, stride 1, per-channel weights
 * w[c][dy+1][dx+1] and an optional per-channel bias, added to the attention
 * output:  out[b][y][x][c] += b[c] + sum_{dy,dx in -1..1} w[c][dy+1][dx+1]
 * v[b][y+dy][x+dx][c] (terms outside the grid are 0).
 * ------------------------------------------------------------------------- */
int oracle_dwconv_add(const double* v, const double* w, const double* b, double* out, int B, int H, int W, int C)
{
    if (B < 0 || H < 1 || W < 1 || C < 1 || (B > 0 && (!v || !w || !out))) return 1;
    const size_t plane = (size_t)H * W * C;
    double* tmp = (double*)malloc(((size_t)B * plane + 1) * sizeof(double));
    if (!tmp) return 2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int bi = 0; bi < B; ++bi)
        for (int y = 0; y < H; ++y)
            for (int x = 0; x < W; ++x)
                for (int c = 0; c < C; ++c) {
                    double s = b ? b[c] : 0.0;
                    for (int dy = -1; dy <= 1; ++dy)
                        for (int dx = -1; dx <= 1; ++dx) {
                            const int yy = y + dy, xx = x + dx;
                            if (yy < 0 || yy >= H || xx < 0 || xx >= W) continue;
                            s += w[(size_t)c * 9 + (size_t)(dy + 1) * 3 + (size_t)(dx + 1)] *
                                 v[(size_t)bi * plane + ((size_t)yy * W + xx) * C + c];
                        }
                    tmp[(size_t)bi * plane + ((size_t)y * W + x) * C + c] = s;
                }
    for (size_t i = 0; i < (size_t)B * plane; ++i) out[i] += tmp[i];
    free(tmp);
    return 0;
}

/* ---------------------------------------------------------------------------
 * LinMapper's aggregation inside each window ([What] abstract: self-attention
 * replaced by a simple linear mapping layer inside each non-overlapped
 * window, with Swin's cross-window communication kept).  Reading: per head h
 * a learned N x N matrix A_h (N = M^2, shared by all windows) and an optional
 * per-position bias b_h maps the window's values,
 *   out[i] = b_h[i] + sum_j A_h[i][j] v[j],
 * over the head's d channels, with the pairs of a shifted window's different
 * regions excluded exactly as in the attention (region labels of the rolled
 * grid).  Windows, regions and grid positions as in oracle_window_attn.
 * A: heads x N x N, bias: heads x N or NULL.
 * ------------------------------------------------------------------------- */
int oracle_window_linear(int B, int H, int W, int C, int heads, int M, int shift, int part,
                         const double* v, const double* A, const double* bias, double* out)
{
    if (bad_shape(B, H, W, C, M, shift, part)) return 1;
    if (heads < 1 || C % heads) return 1;
    if (B > 0 && (!v || !A || !out)) return 1;
    const int d = C / heads, nwr = H / M, nwc = W / M, N = M * M;
    const int64_t total = (int64_t)B * nwr * nwc;
    memset(out, 0, (size_t)B * H * W * C * sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < total * heads; ++u) {
        const int64_t gw = u / heads;
        const int h = (int)(u % heads);
        const int b = (int)(gw / ((int64_t)nwr * nwc));
        const int wr = (int)((gw % ((int64_t)nwr * nwc)) / nwc), wc = (int)(gw % nwc);
        for (int i = 0; i < N; ++i) {
            int gi_i, gj_i;
            grid_pos(H, W, M, shift, part, wr, wc, i / M, i % M, &gi_i, &gj_i);
            const int reg_i = part == OR_PART_CYCLIC
                ? 3 * axis_region(wr * M + i / M, H, M, shift) + axis_region(wc * M + i % M, W, M, shift) : 0;
            double* o = out + (((size_t)b * H + gi_i) * W + gj_i) * C + (size_t)h * d;
            for (int e = 0; e < d; ++e) o[e] = bias ? bias[(size_t)h * N + i] : 0.0;
            for (int j = 0; j < N; ++j) {
                const int reg_j = part == OR_PART_CYCLIC
                    ? 3 * axis_region(wr * M + j / M, H, M, shift) + axis_region(wc * M + j % M, W, M, shift) : 0;
                if (reg_j != reg_i) continue;
                int gi_j, gj_j;
                grid_pos(H, W, M, shift, part, wr, wc, j / M, j % M, &gi_j, &gj_j);
                const double a = A[((size_t)h * N + i) * N + j];
                const double* vj = v + (((size_t)b * H + gi_j) * W + gj_j) * C + (size_t)h * d;
                for (int e = 0; e < d; ++e) o[e] += a * vj[e];
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Video (3D) windows.  [SwinV2] appendix A2 fine-tunes a video model on
 * Kinetics-400 with windows of 16^2 x 8 over 256^2 x 8 frames (and 20^2 x 8
 * at 320^2); [Iwin] abstract transfers its 2D weights to 3D.  Neither page
 * writes the 3D form down.  Reading: the 2D definition with a third,
 * temporal axis treated exactly like the other two --
 *   - tokens (B, T, H, W, C), windows of Mt x M x M, local order
 *     (t*M + r)*M + c, window order ((b*nwt + wt)*nwr + wr)*nwc + wc;
 *   - cyclic: every axis rolled by -its shift (shift_t on the temporal
 *     axis), regions per axis as in 2D, a pair allowed when all three
 *     region labels agree; interleaved: every axis interleaved, no shift;
 *   - the bias table of G over the log-spaced offsets (dx, dy, dt), G's
 *     first layer taking three inputs, (2Mt-1)(2M-1)^2 rows indexed
 *     ((dt + Mt-1)(2M-1) + dy + M-1)(2M-1) + dx + M-1.
 * With Mt = 1 (or T = Mt = 1) every step reduces to the 2D definition.
 * ------------------------------------------------------------------------ */

/* Grid coordinate of local position r in window w along one axis of length L. */
static int axis_pos(int L, int M, int s, int part, int w, int r)
{
    return part == OR_PART_INTERLEAVED ? w + r * (L / M) : (w * M + r + s) % L;
}

/* [SwinV2] eq. 3-4 extended to three offsets: G(log-spaced dx, dy, dt), w1 is
 * hidden x 3 (columns: dx, dy, dt), ReLU between the two layers. */
int oracle_cpb_table3d(int Mt, int M, int heads, int hidden, const double* w1, const double* b1,
                       const double* w2, const double* b2, double* table)
{
    if (Mt < 1 || M < 1 || heads < 1 || hidden < 1 || !w1 || !w2 || !table) return 1;
    const int S = 2 * M - 1;
    double* h = (double*)malloc((size_t)hidden * sizeof(double));
    if (!h) return 2;
    for (int dt = -(Mt - 1); dt <= Mt - 1; ++dt)
        for (int dy = -(M - 1); dy <= M - 1; ++dy)
            for (int dx = -(M - 1); dx <= M - 1; ++dx) {
                const double in0 = oracle_log_offset((double)dx);
                const double in1 = oracle_log_offset((double)dy);
                const double in2 = oracle_log_offset((double)dt);
                for (int j = 0; j < hidden; ++j) {
                    const double a = w1[3 * j] * in0 + w1[3 * j + 1] * in1 + w1[3 * j + 2] * in2 +
                                     (b1 ? b1[j] : 0.0);
                    h[j] = a > 0.0 ? a : 0.0;
                }
                double* row = table + (((size_t)(dt + Mt - 1) * S + (size_t)(dy + M - 1)) * S +
                                       (size_t)(dx + M - 1)) * heads;
                for (int o = 0; o < heads; ++o) {
                    double acc = b2 ? b2[o] : 0.0;
                    for (int j = 0; j < hidden; ++j) acc += w2[(size_t)o * hidden + j] * h[j];
                    row[o] = acc;
                }
            }
    free(h);
    return 0;
}

/* Windowed attention over (B, T, H, W, C) video grids, windows Mt x M x M
 * (reading above); logit, bias, exclusion and softmax as in
 * oracle_window_attn.  pos: NONE or TABLE (no rotary form in 3D).  windows:
 * optional list of global window ids to compute (NULL: all); only their
 * tokens of `out` are written. */
int oracle_window_attn3d(int B, int T, int H, int W, int C, int heads, int Mt, int M,
                         int shift_t, int shift, int part, int sim, int pos, double tau_min,
                         const double* q, const double* k, const double* v,
                         const double* tau, const double* table, const int64_t* windows, int64_t n_windows,
                         double* out)
{
    if (bad_shape(B, H, W, C, M, shift, part)) return 1;
    if (T < 1 || Mt < 1 || T % Mt || shift_t < 0 || shift_t >= Mt) return 1;
    if (part == OR_PART_INTERLEAVED && shift_t != 0) return 1;
    if (heads < 1 || C % heads) return 1;
    if (sim != OR_SIM_COSINE && sim != OR_SIM_DOT) return 1;
    if (pos != OR_POS_NONE && pos != OR_POS_TABLE) return 1;
    if (sim == OR_SIM_COSINE && !tau) return 1;
    if (pos == OR_POS_TABLE && !table) return 1;
    if (!q || !k || !v || !out) return 1;
    const int d = C / heads;
    const int nwt = T / Mt, nwr = H / M, nwc = W / M, N = Mt * M * M, S = 2 * M - 1;
    const int64_t nW = (int64_t)nwt * nwr * nwc, total = windows ? n_windows : (int64_t)B * nW;
    if (windows)
        for (int64_t i = 0; i < n_windows; ++i)
            if (windows[i] < 0 || windows[i] >= (int64_t)B * nW) return 1;
    const double dot_scale = 1.0 / sqrt((double)d);
    int failed = 0;

    #pragma omp parallel
    {
        double* qs = (double*)malloc((size_t)N * d * sizeof(double));
        double* ks = (double*)malloc((size_t)N * d * sizeof(double));
        double* vs = (double*)malloc((size_t)N * d * sizeof(double));
        double* lg = (double*)malloc((size_t)N * sizeof(double));
        size_t* gofs = (size_t*)malloc((size_t)N * sizeof(size_t));
        int* region = (int*)malloc((size_t)N * sizeof(int));
        if (!qs || !ks || !vs || !lg || !gofs || !region) {
            #pragma omp atomic write
            failed = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t u = 0; u < total * heads; ++u) {
                const int64_t wi = windows ? windows[u / heads] : u / heads;
                const int h = (int)(u % heads);
                const int b = (int)(wi / nW);
                const int wt = (int)((wi % nW) / ((int64_t)nwr * nwc));
                const int wr = (int)((wi % ((int64_t)nwr * nwc)) / nwc);
                const int wc = (int)(wi % nwc);
                /* gather, with region labels per axis in rolled coordinates */
                for (int i = 0; i < N; ++i) {
                    const int t = i / (M * M), r = (i / M) % M, c = i % M;
                    const int gt = axis_pos(T, Mt, shift_t, part, wt, t);
                    const int gi = axis_pos(H, M, shift, part, wr, r);
                    const int gj = axis_pos(W, M, shift, part, wc, c);
                    region[i] = part == OR_PART_CYCLIC
                        ? 9 * axis_region(wt * Mt + t, T, Mt, shift_t) + 3 * axis_region(wr * M + r, H, M, shift) +
                          axis_region(wc * M + c, W, M, shift)
                        : 0;
                    gofs[i] = ((((size_t)b * T + gt) * H + gi) * W + gj) * C + (size_t)h * d;
                    for (int e = 0; e < d; ++e) {
                        qs[(size_t)i * d + e] = q[gofs[i] + e];
                        ks[(size_t)i * d + e] = k[gofs[i] + e];
                        vs[(size_t)i * d + e] = v[gofs[i] + e];
                    }
                    if (sim == OR_SIM_COSINE) {
                        unit_normalize(qs + (size_t)i * d, d);
                        unit_normalize(ks + (size_t)i * d, d);
                    }
                }
                const double inv_tau = sim == OR_SIM_COSINE ? 1.0 / (tau[h] > tau_min ? tau[h] : tau_min) : 0.0;
                for (int i = 0; i < N; ++i) {
                    const int ti = i / (M * M), ri = (i / M) % M, ci = i % M;
                    double mx = -INFINITY;
                    for (int j = 0; j < N; ++j) {
                        const int tj = j / (M * M), rj = (j / M) % M, cj = j % M;
                        double s = 0.0;
                        for (int e = 0; e < d; ++e) s += qs[(size_t)i * d + e] * ks[(size_t)j * d + e];
                        double l = sim == OR_SIM_COSINE ? s * inv_tau : s * dot_scale;
                        if (pos == OR_POS_TABLE)
                            l += table[((((size_t)(ti - tj + Mt - 1) * S + (size_t)(ri - rj + M - 1)) * S) +
                                        (size_t)(ci - cj + M - 1)) * heads + h];
                        lg[j] = region[j] == region[i] ? l : -INFINITY;
                        if (lg[j] > mx) mx = lg[j];
                    }
                    double sum = 0.0;
                    for (int j = 0; j < N; ++j) {
                        lg[j] = lg[j] == -INFINITY ? 0.0 : exp(lg[j] - mx);
                        sum += lg[j];
                    }
                    for (int e = 0; e < d; ++e) {
                        double acc = 0.0;
                        for (int j = 0; j < N; ++j) acc += lg[j] * vs[(size_t)j * d + e];
                        out[gofs[i] + e] = acc / sum;
                    }
                }
            }
        }
        free(qs); free(ks); free(vs); free(lg); free(gofs); free(region);
    }
    return failed ? 2 : 0;
}

/* ---------------------------------------------------------------------------
 * Swin V1 bias table at a new window size ([SwinV2] Problem and tab. 1: the
 * earlier model's parameterised (2M-1)^2 x heads table, interpolated
 * bi-cubically when the window changes; log-CPB replaces it).  Reading (the
 * page names the method only): each head's table is an image, rows dy,
 * columns dx, resampled from (2Ms-1)^2 to (2Md-1)^2 by separable cubic
 * convolution with Keys' kernel, a = -0.75; output sample x sits at source
 * coordinate (x + 1/2) Ss / Sd - 1/2 (sample centres aligned), and taps
 * outside the table take its border value.
 * ------------------------------------------------------------------------- */
static double keys_cubic(double t)
{
    const double a = -0.75;
    const double u = fabs(t);
    if (u <= 1.0) return ((a + 2.0) * u - (a + 3.0)) * u * u + 1.0;
    if (u < 2.0) return ((a * u - 5.0 * a) * u + 8.0 * a) * u - 4.0 * a;
    return 0.0;
}

/* source taps i0 - 1 .. i0 + 2 of output sample o and their weights */
static void resize_taps(int o, int Ss, int Sd, int* idx, double* w)
{
    const double s = ((double)o + 0.5) * (double)Ss / (double)Sd - 0.5;
    const double f = floor(s);
    const int i0 = (int)f;
    for (int m = 0; m < 4; ++m) {
        const int i = i0 - 1 + m;
        idx[m] = i < 0 ? 0 : i > Ss - 1 ? Ss - 1 : i;
        w[m] = keys_cubic(s - (double)i);
    }
}

int oracle_table_resize(int Ms, int Md, int heads, const double* src, double* dst)
{
    if (Ms < 1 || Md < 1 || heads < 1 || !src || !dst) return 1;
    const int Ss = 2 * Ms - 1, Sd = 2 * Md - 1;
    for (int y = 0; y < Sd; ++y) {
        int iy[4], ix[4];
        double wy[4], wx[4];
        resize_taps(y, Ss, Sd, iy, wy);
        for (int x = 0; x < Sd; ++x) {
            resize_taps(x, Ss, Sd, ix, wx);
            for (int h = 0; h < heads; ++h) {
                double acc = 0.0;
                for (int m = 0; m < 4; ++m)
                    for (int n = 0; n < 4; ++n)
                        acc += wy[m] * wx[n] * src[((size_t)iy[m] * Ss + (size_t)ix[n]) * heads + h];
                dst[((size_t)y * Sd + (size_t)x) * heads + h] = acc;
            }
        }
    }
    return 0;
}
