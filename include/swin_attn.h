/*
 * swin_attn.h -- C ABI of libswinattn.so: shifted-window / interleaved-window
 * multi-head self-attention on one AMD Instinct MI355X (gfx950): forward
 * (optionally exporting the softmax statistics), backward, the CPB table,
 * video (3D) windows, and the steps around it in a block (projections,
 * residual post-norm, Iwin's convolution, LinMapper's window mapping).
 *
 * Pages defining the operations (cited by title and section):
 *   [SwinV2] "Swin Transformer V2: Scaling Up Capacity and Resolution",
 *            paper card: Method items 1-3, eq. 1-4, the window-attention,
 *            continuous-bias and block pseudocode, Architecture table,
 *            appendix A2 (video fine-tuning).
 *   [Flash]  "FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin
 *            Vision Transformers with Memory Efficient Attention", abstract.
 *   [What]   "What Makes for Hierarchical Vision Transformer?", abstract.
 *   [Iwin]   "Iwin Transformer: Hierarchical Vision Transformer using
 *            Interleaved Windows", abstract.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers, allocated and owned by the caller;
 *     the library allocates no device memory and keeps no state between calls
 *     beyond its loaded code.  `desc` is a HOST pointer, read during the call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; results are ready when the stream is.
 *   - Token grids are (B, H, W, C) row-major, channels last (video grids
 *     (B, T, H, W, C)); head h owns channels [h*d, (h+1)*d), d = C / heads.
 *   - Window order: window (b, wr, wc) has id b*nW + wr*(W/M) + wc,
 *     nW = (H/M)*(W/M); inside a window, token (r, c) is number r*M + c.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued.  A bad argument returns SWIN_EINVAL, a case the pages define
 *     but this library does not build returns SWIN_EUNSUPPORTED; in both cases
 *     nothing is written.  A failed kernel launch returns SWIN_EHIP.
 *     swin_status_string() names a status; swin_last_error() gives the detail
 *     of the calling thread's last failure.
 *   - All entry points are thread-safe; no exception crosses the ABI.
 */
#ifndef SWIN_ATTN_H
#define SWIN_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWIN_ATTN_VERSION 1

enum swin_status { SWIN_OK = 0, SWIN_EINVAL = 1, SWIN_EUNSUPPORTED = 2, SWIN_EHIP = 3 };

/* Window partitions.
 * CYCLIC ([SwinV2] Method: Swin V1's partition; its shift is not shown on the
 *   page): the grid is rolled by -shift on both axes and cut into M x M
 *   windows, so window (wr, wc) local (r, c) is grid
 *   ((wr*M + r + shift) mod H, (wc*M + c + shift) mod W).  With shift > 0,
 *   tokens that the roll brought from the far edge do not attend to the ones
 *   they now sit beside: along each axis the rolled coordinate p = w*M + r
 *   falls in region [0, L-M), [L-M, L-shift) or [L-shift, L), and a query
 *   attends only to keys of its own region pair.  Masked weights are exactly 0.
 * INTERLEAVED ([Iwin] abstract): window (wr, wc) holds every (H/M)-th row from
 *   wr and every (W/M)-th column from wc: local (r, c) is grid
 *   (wr + r*H/M, wc + c*W/M).  Requires shift == 0. */
enum swin_partition { SWIN_PART_CYCLIC = 0, SWIN_PART_INTERLEAVED = 1 };

/* Similarity.  COSINE ([SwinV2] eq. 2): cos(q_i, k_j) / max(tau_h, tau_min),
 * each vector divided by max(||x||, 1e-12).  DOT ([SwinV2] eq. 1):
 * q_i . k_j / sqrt(d). */
enum swin_sim { SWIN_SIM_COSINE = 0, SWIN_SIM_DOT = 1 };

/* Position information.
 * TABLE ([SwinV2] eq. 2-3): logit += table[(ri-rj+M-1)*(2M-1) + (ci-cj+M-1)][h],
 *   offsets taken query minus key in window-local coordinates.
 * ROPE2D ([Flash] abstract: window-local 2D rotary embedding): before the
 *   similarity, q and k channels [0, d/2) turn by the local row r and
 *   [d/2, d) by the local column c; within each half, pair (2k, 2k+1),
 *   k < d/4, turns by pos * theta_k, theta_k = rope_base^(-k/(d/4)) or the
 *   caller's rope_freqs[h][half][k]. */
enum swin_pos { SWIN_POS_NONE = 0, SWIN_POS_TABLE = 1, SWIN_POS_ROPE2D = 2 };

enum swin_dtype { SWIN_DT_F32 = 0, SWIN_DT_BF16 = 1 };

/* GRID: q, k, v, out are (B, H, W, C) and the partition is applied inside the
 * kernel (the hot path).  WINDOWS: they are (B*nW, M*M, C), already
 * partitioned (e.g. by swin_window_partition); the shift mask still follows
 * each window's place in the grid. */
enum swin_layout { SWIN_LAYOUT_GRID = 0, SWIN_LAYOUT_WINDOWS = 1 };

/* Log-CPB variants, as flags.  PAPER = 0 ([SwinV2] eq. 4): inputs
 * sign(x) ln(1+|x|) of the raw offsets, output unbounded.  The released
 * code's forms ([SwinV2] card, "Paper vs code"):
 *   CODE_NORM: the code's coordinate table: inputs sign(u) log2(1+|u|) /
 *              log2(8) of u = 8 x / (norm_M - 1), norm_M the pretrained
 *              window (or the window itself), with the row offset as G's
 *              first input (the page does not give the order; the SwinV2
 *              port in transformers stacks (row, column) offsets);
 *   SIGMOID16: output 16 * sigmoid(G), in (0, 16).
 * CODE_NORM | SIGMOID16 (= 3) is the released code's table, so trained
 * meta-network weights of that code load unchanged. */
enum swin_cpb_mode { SWIN_CPB_PAPER = 0, SWIN_CPB_CODE_NORM = 1, SWIN_CPB_SIGMOID16 = 2 };

typedef struct swin_attn_desc {
    int32_t B, H, W, C, heads;  /* C % heads == 0; d = C/heads must be 32        */
    int32_t M, shift;           /* H % M == W % M == 0; 0 <= shift < M;
                                   shift == 0 for INTERLEAVED                     */
    int32_t partition;          /* enum swin_partition                           */
    int32_t sim;                /* enum swin_sim                                 */
    int32_t pos;                /* enum swin_pos                                 */
    int32_t dtype;              /* enum swin_dtype: q, k, v and out share it     */
    int32_t layout;             /* enum swin_layout                              */
    float   tau_min;            /* floor of tau, 0.01 on the pages ([SwinV2]
                                   Method item 2); must be > 0                   */
    float   rope_base;          /* 10000 unless rope_freqs is given; > 0        */
} swin_attn_desc;

/* Log-spaced continuous position bias table ([SwinV2] eq. 3-4, Method item 3:
 * computed once per relative position and stored).
 *   table[(dy+M-1)*(2M-1) + (dx+M-1)][h] = (W2 relu(W1 (f(dx), f(dy)) + b1) + b2)[h],
 *   f(x) = sign(x) ln(1+|x|), dy, dx in [-(M-1), M-1] (query minus key; dx is
 *   the column offset and G's first input in the paper's form; CODE_NORM
 *   feeds (dy, dx) instead, see swin_cpb_mode).
 * w1: hidden x 2, b1: hidden (or NULL = 0), w2: heads x hidden, b2: heads (or
 * NULL = 0), all fp32 row-major on the device.  table: (2M-1)^2 x heads fp32.
 * 1 <= M <= 64, 1 <= heads <= 64, 1 <= hidden <= 4096, 0 <= cpb_mode <= 3;
 * under CODE_NORM the offsets are normalised by this window (M >= 2).
 * Errors: SWIN_EINVAL for a bad size or mode, a NULL w1/w2/table, or a table
 * overlapping a parameter; nothing is written then. */
int swin_cpb_table(int32_t M, int32_t heads, int32_t hidden,
                   const float* w1, const float* b1, const float* w2, const float* b2,
                   int32_t cpb_mode, float* table, void* stream);

/* The same table for window M with the CODE_NORM offsets normalised by
 * norm_M - 1 instead ([SwinV2] card, Method item 3: a model trained at one
 * window size runs at another; "Paper vs code": the code divides by the
 * pretrained window less one).  2 <= norm_M <= 4096 when cpb_mode has
 * CODE_NORM; otherwise norm_M is ignored.  Same arguments, layout, ownership
 * and errors as swin_cpb_table. */
int swin_cpb_table_ex(int32_t M, int32_t norm_M, int32_t heads, int32_t hidden,
                      const float* w1, const float* b1, const float* w2, const float* b2,
                      int32_t cpb_mode, float* table, void* stream);

/* A parameterised (Swin V1) bias table carried to another window size by
 * bicubic interpolation, the transfer log-CPB replaces ([SwinV2] card,
 * Problem and tab. 1).  Each head's (2*M_src-1) x (2*M_src-1) table, rows
 * dy and columns dx in the layout swin_cpb_table writes, is resampled to
 * (2*M_dst-1) x (2*M_dst-1): separable cubic convolution with Keys' kernel,
 * a = -0.75, output sample x at source coordinate (x + 1/2) S_src/S_dst - 1/2,
 * taps past the border taking the border value (the page names the method
 * only; this is the common reading).  Weights and sums in fp32.
 * src: (2*M_src-1)^2 x heads fp32, dst: (2*M_dst-1)^2 x heads fp32, device
 * memory owned by the caller, dst not overlapping src; 1 <= M_src, M_dst <= 64,
 * 1 <= heads <= 64.  Errors: SWIN_EINVAL for a bad size, a NULL pointer or an
 * overlap (nothing is written then). */
int swin_cpb_table_resize(int32_t M_src, int32_t M_dst, int32_t heads, const float* src, float* dst,
                          void* stream);

/* Window partition (gather) of a (B, H, W, C) grid into (B*nW, M*M, C), and
 * its inverse (scatter).  A bit-exact copy of C elements per token; dtype
 * gives the element size.  x and xw must not overlap. */
int swin_window_partition(const void* x, void* xw, int32_t B, int32_t H, int32_t W,
                          int32_t C, int32_t M, int32_t shift, int32_t partition,
                          int32_t dtype, void* stream);
int swin_window_reverse(const void* xw, void* x, int32_t B, int32_t H, int32_t W,
                        int32_t C, int32_t M, int32_t shift, int32_t partition,
                        int32_t dtype, void* stream);

/* Windowed multi-head self-attention forward ([SwinV2] eq. 1-2 and the
 * window-attention pseudocode; [Flash] exact softmax attention inside the
 * window, never materialising the N x N scores, N = M*M):
 *   out_i = sum_j softmax_j(logit_ij) v_j over the keys j of query i's window
 *   (and shift region), logit as set by desc->sim and desc->pos.
 * q, k, v, out: device tensors of desc->dtype in desc->layout.  out must not
 * overlap q, k or v.  All must be 16-byte aligned.
 * tau: heads fp32 (required for COSINE, else ignored).
 * table: (2M-1)^2 x heads fp32 (required for POS_TABLE, else ignored).
 * rope_freqs: heads x 2 x (d/4) fp32, or NULL for the rope_base schedule
 * (POS_ROPE2D only).
 * Arithmetic: fp32 throughout for SWIN_DT_F32; for SWIN_DT_BF16 the two
 * contractions run on bf16 matrix cores with fp32 accumulation and the
 * softmax in fp32, output rounded to nearest even. */
int swin_window_attn_fwd(const swin_attn_desc* desc, const void* q, const void* k,
                         const void* v, void* out, const float* tau, const float* table,
                         const float* rope_freqs, void* stream);

/* swin_window_attn_fwd that also exports, per window, head and query, the
 * log-sum-exp of the query's logits over the keys it attends to ([Flash]
 * Abstract: training with exact attention and no score matrix; the
 * per-query softmax statistic is what lets a backward rebuild the weights
 * without a pass of its own):
 *   lse[(w*heads + h)*N + i] = log sum_j exp(logit_ij), natural log,
 * w the global window id (image-major, window rows, then columns), i the
 * query's local slot r*M + c.  lse: device fp32, n_windows x heads x N,
 * 4-byte aligned, written; it must not overlap q, k, v or out (SWIN_EINVAL,
 * also for NULL with a non-empty batch).  For SWIN_DT_BF16 it is formed
 * from the same rounded weights that normalise out (the softmax's fp32 sum
 * of bf16 weights), so the two agree; windows above M = 32 run the fp32
 * vector kernel when lse is requested. */
int swin_window_attn_fwd_lse(const swin_attn_desc* desc, const void* q, const void* k,
                             const void* v, void* out, const float* tau, const float* table,
                             const float* rope_freqs, float* lse, void* stream);

/* Backward of swin_window_attn_fwd: the gradients of a loss L given
 * dout = dL/dout, by the chain rule through the same steps ([SwinV2] eq. 1-2,
 * eq. 3-4 for the table, [Flash] for the rotary variant):
 *   p = the forward's softmax weights, D_i = dout_i . out_i,
 *   dv_j = sum_i p_ij dout_i,  dl_ij = p_ij (dout_i . v_j - D_i),
 *   dtable[offset(i, j)][h] += dl_ij (summed over all windows),
 *   COSINE: dtau_h = sum dl_ij cos_ij (-1/tau_h^2) while tau_h > tau_min
 *           (the floor passes no gradient), and dq, dk through the unit
 *           normalisation; DOT: dq, dk from dl / sqrt(d);
 *   ROPE2D: dq, dk rotated back by the window-local positions.
 * q, k, v, tau, table, rope_freqs: as given to the forward; out: the
 * forward's output for them; dout: dL/dout.  All (B,H,W,C)-shaped tensors
 * share desc->dtype and desc->layout and are 16-byte aligned.
 * dq, dk, dv (outputs, same shape and dtype): written; they must not overlap
 * an input or each other.  dtau: heads fp32 (COSINE; NULL skips it), dtable:
 * (2M-1)^2 x heads fp32 (POS_TABLE; NULL skips it): both written (sums over
 * the windows, accumulated with fp32 atomics, so the last bits depend on
 * order).  Requires d = 32 and M <= 64, with the per-query statistics and
 * (POS_TABLE) the table and its gradient fitting the vector kernel's LDS:
 * POS_TABLE up to M = 55 (SWIN_EUNSUPPORTED otherwise).
 * Arithmetic: SWIN_DT_F32 runs in fp32 on the vector ALUs.  SWIN_DT_BF16
 * runs its contractions on bf16 matrix cores with fp32 accumulation: the
 * stored bf16 inputs enter as they are, the softmax weights p and the score
 * gradients dl (and rotated q, k under ROPE2D) are rounded to bf16 as
 * operands, scales, softmax and sums stay fp32 (COSINE with ROPE2D runs the
 * fp32 vector path instead).  bf16 gradients are rounded to nearest even
 * once at the end. */
int swin_window_attn_bwd(const swin_attn_desc* desc, const void* q, const void* k,
                         const void* v, const void* out, const void* dout, const float* tau,
                         const float* table, const float* rope_freqs, void* dq, void* dk,
                         void* dv, float* dtau, float* dtable, void* stream);

/* swin_window_attn_bwd given the forward's log-sum-exp ([Flash]
 * Abstract, as for swin_window_attn_fwd_lse): lse as written by
 * swin_window_attn_fwd_lse for the same inputs (device fp32, n_windows x
 * heads x N, natural log, 4-byte aligned, read only).  The matrix-core paths
 * rebuild p_ij = exp(logit_ij - lse_i) from it and skip their own pass over
 * the keys; the fp32 vector path (SWIN_DT_F32, and COSINE with ROPE2D)
 * recomputes the statistics and does not read it.  Other arguments, results
 * and errors as swin_window_attn_bwd; NULL lse with a non-empty batch is
 * SWIN_EINVAL. */
int swin_window_attn_bwd_lse(const swin_attn_desc* desc, const void* q, const void* k,
                             const void* v, const void* out, const void* dout, const float* tau,
                             const float* table, const float* rope_freqs, const float* lse, void* dq,
                             void* dk, void* dv, float* dtau, float* dtable, void* stream);

/* Bias table of video (3D) windows Mt x M x M ([SwinV2] eq. 3-4 with a third
 * offset; appendix A2 fine-tunes on video with 16^2 x 8 windows, the page
 * gives no 3D form): row ((dt + Mt-1)(2M-1) + dy + M-1)(2M-1) + dx + M-1 of
 * table ((2Mt-1)(2M-1)^2 x heads fp32, written) holds
 *   G(x) = W2 relu(W1 x + b1) + b2,  x = sign(d) log(1 + |d|) of (dx, dy, dt),
 * w1: hidden x 3 (columns dx, dy, dt), b1: hidden or NULL, w2: heads x hidden,
 * b2: heads or NULL; device fp32, the table must not overlap them.  Each
 * value is a fp32 sum over hidden (64 partial sums, then across them).  1 <= Mt, M <= 64, 1 <= heads <= 64,
 * 1 <= hidden <= 4096 (SWIN_EINVAL otherwise). */
int swin_cpb_table3d(int32_t Mt, int32_t M, int32_t heads, int32_t hidden, const float* w1,
                     const float* b1, const float* w2, const float* b2, float* table, void* stream);

/* Window attention over video (3D) windows: swin_window_attn_fwd's logit,
 * bias, exclusion and softmax ([SwinV2] eq. 1-2 and the window-attention
 * pseudocode) over (B, T, H, W, C) grids, channels last, windows of
 * Mt x M x M tokens.  desc gives B, H, W, C, heads, M, shift, partition, sim,
 * pos (NONE or TABLE; ROPE2D is SWIN_EUNSUPPORTED), dtype and tau_min, with
 * layout GRID; T frames, temporal window Mt (T % Mt == 0) and temporal shift
 * shift_t (0 <= shift_t < Mt, 0 for interleaved windows) come as arguments.
 * Reading ([SwinV2] appendix A2, [Iwin] abstract: video models, no 3D form on
 * the pages): the temporal axis is rolled (or interleaved) like the other
 * two, pairs whose shift regions differ on any axis are excluded, and the
 * bias is swin_cpb_table3d's table, indexed by the offsets (dt, dy, dx).
 * q, k, v, out: device tensors of desc->dtype, 16-byte aligned, out not
 * overlapping q, k or v; tau: heads fp32 (COSINE); table: as written by
 * swin_cpb_table3d (TABLE).  bf16 with M <= 22 runs on the matrix cores
 * (the products on bf16 operands with fp32 accumulation, COSINE's unit q and
 * k scaled by 1/tau rounded to bf16 unless tau < 0.1, the weights rounded to
 * bf16 before P V, softmax in fp32 with a running maximum); everything else
 * on the vector ALUs (similarities and logits in fp64, exponentials and sums
 * in fp32), where the head's whole table must fit LDS next to a 64-key
 * chunk (SWIN_EUNSUPPORTED otherwise).  The output is rounded once. */
int swin_window_attn3d_fwd(const swin_attn_desc* desc, int32_t T, int32_t Mt, int32_t shift_t,
                           const void* q, const void* k, const void* v, void* out, const float* tau,
                           const float* table, void* stream);

/* Name of the kernel swin_window_attn3d_fwd runs for desc and the temporal
 * sizes ("attn_video_mfma_kernel" or "attn_video_kernel"; "" for a NULL or
 * malformed descriptor).  A static string; no device work. */
const char* swin_window_attn3d_kernel(const swin_attn_desc* desc, int32_t T, int32_t Mt);

/* Backward of swin_cpb_table_ex ([SwinV2] eq. 3-4, card "Paper vs code"):
 * from dtable ((2M-1)^2 x heads fp32) the gradients of the meta network's
 * parameters, dw1 (hidden x 2), db1 (hidden, or NULL to skip), dw2
 * (heads x hidden), db2 (heads, or NULL), written, fp32, device memory:
 *   a = W1 x + b1, hid = relu(a), dg = dtable (SIGMOID16: times
 *   T (1 - T/16), the derivative of T = 16 sigmoid(G)),
 *   dW2 = sum dg hid^T, db2 = sum dg, dW1 = sum (W2^T dg)[a > 0] x^T,
 *   db1 = sum (W2^T dg)[a > 0], over the table rows x.
 * table: the forward's table (required with SIGMOID16, else may be NULL).
 * Sizes and modes as swin_cpb_table_ex; outputs must not overlap an input or
 * each other.  Sums use fp32 atomics (order-dependent last bits). */
int swin_cpb_table_bwd(int32_t M, int32_t norm_M, int32_t heads, int32_t hidden,
                       const float* w1, const float* b1, const float* w2, const float* table,
                       const float* dtable, int32_t cpb_mode, float* dw1, float* db1,
                       float* dw2, float* db2, void* stream);

/* The attention branch's input layer ([SwinV2] Method opening paragraph: the
 * block keeps Swin's layout; block pseudocode): one linear layer C -> 3C whose
 * outputs are queries, keys and values in that order,
 *   [q | k | v][t] = w x[t] + b,  w: 3C x C (output rows, input columns).
 * x: T x C (any (B, H, W, C) grid flattened), q, k, v: T x C each (outputs,
 * written), all of `dtype` (SWIN_DT_F32 or SWIN_DT_BF16), device memory,
 * 16-byte aligned; w of the same dtype; b: 3C fp32 or NULL (no bias).
 * Requires C a multiple of 32, 32 <= C <= 512 (SWIN_EUNSUPPORTED otherwise);
 * T = 0 is a no-op.  q, k, v must not overlap x, w, b or each other
 * (SWIN_EINVAL).  Arithmetic: bf16 products on the matrix cores with fp32
 * accumulation, bias added in fp32, rounded once to nearest even; fp32
 * throughout for SWIN_DT_F32. */
int swin_qkv_proj(const void* x, const void* w, const float* b, void* q, void* k, void* v,
                  int64_t T, int32_t C, int32_t dtype, void* stream);

/* The attention branch's input layer fused into the window attention
 * ([SwinV2] Method item 1 and the block pseudocode: window_attention(features)
 * maps the features through one linear layer to q, k, v and attends within
 * windows): q, k, v = split(x w_qkv^T + b_qkv) as swin_qkv_proj computes
 * them, then swin_window_attn_fwd over them, without q, k, v leaving the
 * chip.  desc as for swin_window_attn_fwd, GRID layout; x, out: (B, H, W, C)
 * bf16; w_qkv: 3C x C bf16 (rows: q, k, v outputs); b_qkv: 3C fp32 or NULL;
 * tau, table as for swin_window_attn_fwd.  Device memory; x, w_qkv, out
 * 16-byte aligned; out must not overlap x, w_qkv or b_qkv (SWIN_EINVAL).
 * Built for bf16, 9 <= M <= 16, no rotary positions, d = 32 and C a multiple
 * of 32 up to 192; other descriptors return SWIN_EUNSUPPORTED (use
 * swin_qkv_proj and swin_window_attn_fwd).  Arithmetic: q, k, v in fp32 from
 * bf16 products, rounded once to bf16 for the matrix-core attention (as
 * hi + lo pairs where a rounded operand would pass the bf16 tolerance:
 * COSINE with tau < 0.1, DOT with a logit bound above 20 in log2 units). */
int swin_qkv_window_attn_fwd(const swin_attn_desc* desc, const void* x, const void* w_qkv, const float* b_qkv,
                             void* out, const float* tau, const float* table, void* stream);

/* The attention branch's output layer and residual post-norm ([SwinV2]
 * Method item 1: the layer norm moves to the output of the residual branch,
 * before the add; block pseudocode):
 *   z[t] = w o[t] + b,   y[t] = resid[t] + gamma * (z[t] - mean) / sqrt(var + eps) + beta,
 * mean and biased variance over the C channels of token t.
 * o (the attention output), resid (the main path) and y (output, written):
 * T x C of `dtype`; w: C x C of `dtype`; b (C or NULL), gamma, beta (C): fp32.
 * All device memory, 16-byte aligned.  y may be resid itself (in place) but
 * must not overlap any other input (SWIN_EINVAL); eps >= 0 and finite.  Same
 * C rule as swin_qkv_proj.  Arithmetic: z in fp32 from bf16 products (or fp32),
 * mean and variance in fp32 by two passes, y rounded once. */
int swin_proj_post_norm(const void* o, const void* w, const float* b, const void* resid,
                        const float* gamma, const float* beta, float eps, void* y,
                        int64_t T, int32_t C, int32_t dtype, void* stream);

/* Iwin's convolution branch ([Iwin] abstract: the block couples interleaved
 * window attention with a depthwise convolution that links each token to its
 * local neighbours).  Reading: a 3 x 3 depthwise convolution of v over the
 * (H, W) grid of each image, zero padding, added to the attention output:
 *   out[b][y][x][c] += b[c] + sum_{dy,dx = -1..1} w[c][dy+1][dx+1] v[b][y+dy][x+dx][c].
 * v, out: (B, H, W, C) of `dtype`, device memory, 16-byte aligned; out is read
 * and written (in place) and must not overlap v, w or b.  w: C x 3 x 3 fp32,
 * b: C fp32 or NULL.  Requires C a multiple of 8 (bf16) or 4 (fp32)
 * (SWIN_EUNSUPPORTED otherwise); B = 0 is a no-op.  Arithmetic: fp32; a bf16
 * out is rounded once more after the add. */
int swin_dwconv_add(const void* v, const float* w, const float* b, void* out, int32_t B, int32_t H,
                    int32_t W, int32_t C, int32_t dtype, void* stream);

/* LinMapper's aggregation inside each window ([What] abstract: the
 * self-attention of each non-overlapped window replaced by a linear mapping,
 * Swin's cross-window communication kept).  Reading: per head h an N x N
 * matrix A_h (N = M^2, shared by all windows) and an optional bias b_h:
 *   out[i] = b_h[i] + sum_j A_h[i][j] v[j]
 * over the head's channels, i, j window-local token indices (r M + c), the
 * pairs of a shifted window's different regions excluded as in the
 * attention.  desc as for swin_window_attn_fwd (sim, pos, tau_min and
 * rope_base are not used).  v, out: (B, H, W, C) (or the WINDOWS layout) of
 * desc->dtype; A: heads x N x N of the same dtype, row-major (A_h[i][j] at
 * (h N + i) N + j); bias: heads x N fp32 or NULL.  v, A, out 16-byte aligned,
 * out overlapping none of the inputs.  d = 32 (SWIN_EUNSUPPORTED otherwise).
 * Arithmetic: bf16 on the matrix cores with fp32 accumulation for M = 8 and
 * 16, fp32 on the vector ALUs otherwise; the output rounded once. */
int swin_window_linear(const swin_attn_desc* desc, const void* v, const void* A, const float* bias,
                       void* out, void* stream);

/* Name of the kernel that swin_window_attn_fwd launches for desc (static
 * storage), for matching profiler output:
 *   "attn_valu_kernel"  SWIN_DT_F32;
 *   "attn_small_kernel" SWIN_DT_BF16, M * roundup8(M) <= 256 key slots,
 *                       no rotary positions;
 *   "attn_large_kernel" SWIN_DT_BF16, M <= 32 otherwise (larger windows,
 *                       or rotary positions);
 *   "attn_mfma_kernel"  every other SWIN_DT_BF16 case.
 * Only the descriptor is read; rope_base is not required (the caller may
 * pass rope_freqs).  NULL if swin_window_attn_fwd would reject the
 * descriptor itself; swin_last_error() then says why.  Enqueues nothing. */
const char* swin_window_attn_kernel(const swin_attn_desc* desc);

/* Name of the kernel that swin_window_attn_bwd launches for desc (static
 * storage), beside the fill kernel that clears dtau and dtable:
 *   "attn_bwd_small_kernel" SWIN_DT_BF16, M * roundup8(M) <= 256 key slots,
 *                           no rotary positions;
 *   "attn_bwd_large_kernel" SWIN_DT_BF16, M <= 32 otherwise, when the
 *                           window's rows fit LDS (COSINE with ROPE2D, which
 *                           also stages the remainders, up to M = 24);
 *   "attn_bwd_kernel"       SWIN_DT_F32 and every other case.
 * NULL if swin_window_attn_bwd would reject the descriptor itself (also
 * d != 32, M > 64 or LDS); swin_last_error() then says why.  Enqueues
 * nothing. */
const char* swin_window_attn_bwd_kernel(const swin_attn_desc* desc);

/* Text for a status code (static storage). */
const char* swin_status_string(int status);

/* Detail of the calling thread's last non-OK return ("" if none). */
const char* swin_last_error(void);

/* SWIN_ATTN_VERSION of the built library. */
int swin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWIN_ATTN_H */
