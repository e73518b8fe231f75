/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer-quantization library.
 *
 * GPTQ quantizes one linear layer W (d_out x d_in) at a time so that W X stays
 * close to W_hat X on calibration activations X (page "LLM 量化方法原理与实现
 * 详解", §4.1 GPTQ, objective and Hessian; page "量化经典：LLM.int8 / GPTQ /
 * AWQ", §二 "方法核心").  The library runs the four steps on one GPU:
 *
 *   gptq_hessian_accumulate  H += 2 X X^T                       (step 1)
 *   gptq_prepare_hinv        order, damping, U = chol(H_d^-1)   (steps 2-3)
 *   gptq_quantize_layer      greedy column pass with error feedback and
 *                            lazy batch updates                 (step 4)
 *   gptq_rtn_quantize        round-to-nearest baseline (no feedback)
 *   gptq_layer_loss          ||W X - W_hat X||_F^2 through H, the check
 *
 * Conventions shared by every entry point
 *   - All pointers except `cfg` and `out` arguments of gptq_workspace_bytes
 *     are DEVICE pointers on the current HIP device.  The caller owns every
 *     buffer; the library never allocates: scratch memory is the `ws`
 *     argument, sized by gptq_workspace_bytes().
 *   - Matrices are row-major and densely packed unless a leading dimension is
 *     given.  Device pointers must be 16-byte aligned.
 *   - Calls are asynchronous and ordered on `stream`; the library never
 *     synchronizes the device.  Argument errors are reported synchronously by
 *     the return value (nothing is launched then); a failed kernel launch
 *     returns GPTQ_ERR_HIP.  gptq_last_error() gives a message for the calling
 *     thread's last failure.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics).
 *
 * Quantization grid (page "LLM 量化方法原理与实现详解", §2.2 and §2.3):
 *   symmetric:  qmax = 2^(b-1)-1, scale = max|x| / qmax,
 *               q = clamp(rint(x / scale), -qmax, qmax), stored code = q + 2^(b-1),
 *               stored zero = 2^(b-1);
 *   asymmetric: lo = min(min x, 0), hi = max(max x, 0), scale = (hi-lo)/(2^b-1),
 *               zero = clamp(rint(-lo/scale), 0, 2^b-1),
 *               code = clamp(rint(x/scale + zero), 0, 2^b-1);
 *   a group whose scale would be 0 gets scale 1 (and zero 0 when asymmetric).
 *   Decisions are made in fp32 with round-half-to-even.  Dequantized value:
 *   w_hat = (code - zero) * scale.  Groups are `group_size` consecutive input
 *   columns of one output row (in processing order); group_size 0 = one group
 *   per row.  scales/zeros are [d_out][n_groups] fp32, codes [d_out][d_in] u8.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define GPTQ_API __attribute__((visibility("default")))
#else
#define GPTQ_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GPTQ_OK = 0,
    GPTQ_ERR_INVALID_ARG = -1, /* bad pointer, size, alignment or config value */
    GPTQ_ERR_UNSUPPORTED = -2, /* valid but not implemented (see each call) */
    GPTQ_ERR_WORKSPACE = -3,   /* ws NULL or smaller than gptq_workspace_bytes() */
    GPTQ_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} gptq_status;

typedef enum { GPTQ_DT_F32 = 0, GPTQ_DT_BF16 = 1, GPTQ_DT_F16 = 2 } gptq_dtype;

typedef enum {
    GPTQ_OP_HESSIAN = 0,
    GPTQ_OP_PREPARE = 1,
    GPTQ_OP_QUANTIZE = 2,
    GPTQ_OP_LOSS = 3,
    GPTQ_OP_W4A16 = 4, /* n_tok = M, the rows of X */
    GPTQ_OP_HESSIAN_TOKENS = 5,
    GPTQ_OP_SMOOTH = 6, /* gptq_smooth_scales */
    GPTQ_OP_AWQ = 7,    /* gptq_awq_search (cfg: bits, symmetric, group_size) */
    GPTQ_OP_CALIBRATE = 8 /* gptq_calibrate_hessian (d_in, n_tok) */
} gptq_op;

/*
 * When the grids are fitted (page "LLM 量化方法原理与实现详解", §2.3 names the
 * granularities; when they are fitted is a choice of the quantizer):
 *   GPTQ_GRID_DYNAMIC  each group's grid when the pass reaches the group's
 *                      first column, from the weights as they are then;
 *                      groups follow the processing order.
 *   GPTQ_GRID_STATIC   every group's grid from the ORIGINAL weights, before
 *                      the pass; groups keep the original column order (under
 *                      act-order too), each column uses its own group's grid.
 *   GPTQ_GRID_TENSOR   one grid for the whole matrix, fitted on the original
 *                      weights; group_size must be 0; scales and zeros keep the
 *                      [d_out][1] layout, every row holding the same values.
 */
typedef enum { GPTQ_GRID_DYNAMIC = 0, GPTQ_GRID_STATIC = 1, GPTQ_GRID_TENSOR = 2 } gptq_grid;

typedef struct {
    int32_t bits;       /* 2..8 */
    int32_t symmetric;  /* 1: symmetric grid, 0: asymmetric grid (see above) */
    int32_t group_size; /* 0 (one group per row) or a divisor of d_in */
    int32_t block_size; /* lazy batch width B: 1 (the unblocked update) or a
                           multiple of 32.  Every B gives the same sums in
                           another fp32 order; the batch kernel runs batches of
                           the largest of 128, 96, 64, 32 dividing B (128 for
                           B = 1), and B > 128 forms blocks of such batches. */
    float damp_rel;     /* lambda = damp_rel * mean(diag H), >= 0 */
    int32_t act_order;  /* 1: process columns by descending diag(H) */
    int32_t grid;       /* gptq_grid: when the grids are fitted */
    int32_t super_cols; /* columns per superblock of the two-level lazy update
                           (0: 1024).  Batches of one superblock update only the
                           rest of it; the superblock's stacked errors update
                           every later column when it ends.  Rounded down to a
                           multiple of block_size (and of group_size when a
                           dynamic group spans batches), at least one of them;
                           >= d_in gives the one-level update.  The results
                           are the same sums in another fp32 order. */
} gptq_config;

/*
 * Step 1 -- Hessian accumulation (page "LLM 量化方法原理与实现详解", §4.1: the
 * Hessian of the layer objective is 2 X X^T; page "量化经典" §二 step 1).
 *
 *   H      [d_in][d_in] fp32, in/out.  Only the upper triangle (i <= j) is
 *          read and written: H[i][j] += 2 * sum_t X[i][t] X[j][t].
 *          Repeated calls accumulate token chunks.
 *   hdiag  [d_in] fp64, in/out, may be NULL: hdiag[i] += 2 * sum_t X[i][t]^2
 *          accumulated in fp64 (the exact-enough ordering key for act-order).
 *   X      [d_in][ldx] activations, one row per input channel, n_tok tokens
 *          used per row; bf16 (raw 16-bit patterns) or fp32 per x_dtype.
 *          ldx * element size must be a multiple of 16 bytes.
 *   ws     scratch of gptq_workspace_bytes(GPTQ_OP_HESSIAN, 0, d_in, n_tok, NULL).
 * n_tok == 0 is a no-op.  bf16 inputs are multiplied exactly and summed in
 * fp32 by matrix-core (MFMA) instructions.
 */
GPTQ_API gptq_status gptq_hessian_accumulate(float *H, double *hdiag, const void *X, gptq_dtype x_dtype,
                                    int64_t d_in, int64_t n_tok, int64_t ldx,
                                    void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Step 1 from token-major activations, as a layer's inputs arrive during
 * calibration (page "量化经典：LLM.int8 / GPTQ / AWQ", §二 step 1; page "LLM
 * 量化方法原理与实现详解", §4.1: H = 2 X X^T over all calibration tokens).
 * The SYRK reads the token-major tiles itself (no transposed copy of X).
 *
 *   H      [d_in][d_in] fp32 in/out, upper triangle: H[i][j] += 2 sum_t X[t][i] X[t][j].
 *   hdiag  [d_in] fp64 in/out or NULL, as in gptq_hessian_accumulate.
 *   X      [n_tok][ldx] one row per token, d_in channels used per row, ldx >= d_in;
 *          bf16 (raw 16-bit patterns): 8-byte aligned, ldx a multiple of 4;
 *          fp32: 4-byte aligned.
 *   ws     scratch of gptq_workspace_bytes(GPTQ_OP_HESSIAN_TOKENS, 0, d_in, n_tok, NULL),
 *          the same size as gptq_hessian_accumulate's (may be NULL when 0).
 * For bf16, H equals, bit for bit, that of gptq_hessian_accumulate called with
 * the same tokens in channel-major layout (hdiag: to fp64 rounding, summed in
 * another order).  Repeated calls accumulate further chunks.
 */
GPTQ_API gptq_status gptq_hessian_accumulate_tokens(float *H, double *hdiag, const void *X, gptq_dtype x_dtype,
                                                    int64_t d_in, int64_t n_tok, int64_t ldx, void *ws,
                                                    size_t ws_bytes, hipStream_t stream);

/*
 * The forward of a linear layer that produces the next layer's calibration
 * inputs (page "量化经典：LLM.int8 / GPTQ / AWQ", §二 step 1: the calibration
 * set is run through the model layer by layer and each layer's inputs are
 * recorded; page "LLM 量化方法原理与实现详解", §3.1: the PTQ flow runs the
 * calibration data through the model).  On the bf16 matrix cores:
 *
 *   Y[t][o] = bf16( sum_i X[t][i] W[o][i] )   (fp32 sums, rounded to nearest even)
 *
 *   X  [n_tok][ldx] bf16, token-major; W [d_out][ldw] bf16 (the layer's weight,
 *      one row per output channel); both 16-byte aligned with ldx, ldw
 *      multiples of 8 and >= d_prev.
 *   Y  [n_tok][ldy] bf16 out, ldy >= d_out (2-byte aligned).
 * No workspace.  n_tok == 0 or d_out == 0 is a no-op.
 */
GPTQ_API gptq_status gptq_linear_forward(void *Y, int64_t ldy, const void *X, int64_t ldx, const void *W, int64_t ldw,
                                         int64_t n_tok, int64_t d_prev, int64_t d_out, hipStream_t stream);

/*
 * Step 1 fed by that forward, chunk by chunk: for each chunk of
 * gptq_calibrate_chunk_tokens(d_in) tokens, Y = gptq_linear_forward(X chunk, W)
 * into the workspace, then gptq_hessian_accumulate_tokens(H, hdiag, Y), so the
 * layer inputs never exist in full (page "量化经典", §二 step 1; page "LLM
 * 量化方法原理与实现详解", §4.1).
 *
 *   H, hdiag  as in gptq_hessian_accumulate (d_in channels), accumulated.
 *   X, W      as in gptq_linear_forward with d_out = d_in (W is [d_in][ldw]).
 *   ws        scratch of gptq_workspace_bytes(GPTQ_OP_CALIBRATE, 0, d_in, n_tok, NULL):
 *             one chunk of Y plus the SYRK's scratch.
 * The result equals those two calls made chunk by chunk.
 */
GPTQ_API gptq_status gptq_calibrate_hessian(float *H, double *hdiag, const void *X, int64_t ldx, const void *W,
                                            int64_t ldw, int64_t n_tok, int64_t d_prev, int64_t d_in, void *ws,
                                            size_t ws_bytes, hipStream_t stream);

/* Tokens per chunk of gptq_calibrate_hessian for d_in channels (about 128 MiB
 * of bf16 layer inputs, a multiple of 1024 in [1024, 65536]). */
GPTQ_API int64_t gptq_calibrate_chunk_tokens(int64_t d_in);

/*
 * Steps 2-3 -- column order, damping and the inverse-Hessian factor.
 * The GPTQ update spreads a column's rounding error with the matching row of
 * the inverse Hessian of the not-yet-quantized columns (page "PTQ 权重量化：
 * 从 GPTQ 到 AWQ", GPTQ section); those rows are, up to a per-row scale, the
 * rows of the upper Cholesky factor of H_d^-1 (page "LLM 量化方法原理与实现
 * 详解", §4.1 sketch: the inverse is obtained with a Cholesky factorization).
 *
 *   H        [d_in][d_in] fp32 upper triangle (from step 1); not modified.
 *   hdiag    [d_in] fp64 or NULL; ordering key when cfg->act_order (if NULL
 *            the fp32 diagonal of H is used).
 *   cfg      host pointer; uses damp_rel and act_order.
 *   U        [d_in][d_in] fp32 out: upper triangle = U with U^T U = H_d^-1,
 *            H_d = P H P^T + lambda I, lambda = damp_rel * mean(diag H);
 *            strictly lower triangle = 0.
 *   perm     [d_in] int32 out (may be NULL when !act_order): processing
 *            position k holds original column perm[k]; identity if !act_order.
 *            Order: descending key, ties by lower original index.
 *   info_dev device int32 out: 0 on success, j+1 if the j-th pivot (processing
 *            order) of the factorization of H_d was not positive (then U is
 *            not meaningful).  Read it after synchronizing the stream.
 *   ws       scratch of gptq_workspace_bytes(GPTQ_OP_PREPARE, 0, d_in, 0, cfg).
 * Part of the inverse's assembly runs on a second stream of the library's own
 * (one per device, created on first use, default priority), forked from and
 * joined back to `stream` with events, so the call stays ordered on `stream`.
 * Calls on one device from several host threads share that stream: each call
 * enqueues its fork, side work and join under a per-device lock, so the calls'
 * side work runs one after the other, each after its own stream's earlier
 * work, and each caller's stream waits for its own side work.
 */
GPTQ_API gptq_status gptq_prepare_hinv(const float *H, const double *hdiag, int64_t d_in, const gptq_config *cfg,
                              float *U, int32_t *perm, int32_t *info_dev,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Step 4 -- the greedy column pass with error feedback and lazy batches
 * (page "PTQ 权重量化：从 GPTQ 到 AWQ", GPTQ section: update formula and the
 * 128-column lazy batch; page "量化经典" §二 steps 3-4).  For each column j in
 * processing order, for every row: fit the group grid when j starts a group
 * (from the current weights; with cfg->grid STATIC or TENSOR all grids are
 * fitted on the original W before the pass instead), quantize w_j,
 * e = (w_j - w_hat_j) / U[j][j], and w_k -= e * U[j][k] for the later
 * columns -- inside the current batch at once, for columns beyond it when the
 * batch of block_size columns ends.
 *
 *   W       [d_out][d_in] fp32, in/out (working storage).  On entry the
 *           layer in ORIGINAL column order.  On return W[r][k] holds, for
 *           processing position k, the weight's value when it was quantized.
 *   U, perm from gptq_prepare_hinv (perm may be NULL when !cfg->act_order).
 *   codes   [d_out][d_in] u8 out, ORIGINAL column order.
 *   scales, zeros [d_out][n_groups] fp32 out, groups in processing order
 *           (DYNAMIC) or in original column order (STATIC); [d_out][1] (TENSOR).
 *   g_idx   [d_in] int32 out or NULL: group of each ORIGINAL column.
 *   ws      scratch of gptq_workspace_bytes(GPTQ_OP_QUANTIZE, d_out, d_in, 0, cfg).
 * GPTQ_ERR_UNSUPPORTED when block_size is neither 1 nor a multiple of 32,
 * when group_size (0 counts as d_in) is neither a divisor in {32, 64, 128} of
 * the batch width w (the largest of 128, 96, 64, 32 dividing block_size; 128
 * for block_size 1) nor a multiple of w nor d_in (one group per row), or when
 * d_out > 2^21.
 * GPTQ_ERR_INVALID_ARG for an unknown grid, or TENSOR with group_size != 0.
 */
GPTQ_API gptq_status gptq_quantize_layer(float *W, int64_t d_out, int64_t d_in, const float *U, const int32_t *perm,
                                const gptq_config *cfg, uint8_t *codes, float *scales, float *zeros,
                                int32_t *g_idx, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * gptq_quantize_layer for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid device allocation.  It
 * takes no workspace: its scratch memory is a fixed array of
 * GPTQ_NOALLOC_SCRATCH_BYTES in the library's device image, one per device
 * (placed by the runtime when the library first runs on that device, held
 * until the process ends); it calls no allocator.  Arguments, results and
 * kernels are those of gptq_quantize_layer (the same bits), without ws.
 *   Returns GPTQ_ERR_WORKSPACE, launching nothing, when the layer needs more
 *   scratch than the array holds: gptq_workspace_bytes(GPTQ_OP_QUANTIZE, ...)
 *   > GPTQ_NOALLOC_SCRATCH_BYTES (e.g. 4096 x 4096 or 8192 x 8192 layers in
 *   natural order fit: 16 and 32 MiB; act-order adds d_out x d_in bytes).
 *   Nothing in the array needs to start at zero.  Every call on one device
 *   shares that device's array: calls that overlap in time on one device (on
 *   different streams, or from several host threads) race and give wrong
 *   results; calls on one stream are ordered and safe.
 */
#define GPTQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
GPTQ_API gptq_status gptq_quantize_layer_noalloc(float *W, int64_t d_out, int64_t d_in, const float *U,
                                                 const int32_t *perm, const gptq_config *cfg, uint8_t *codes,
                                                 float *scales, float *zeros, int32_t *g_idx, hipStream_t stream);

/*
 * Round-to-nearest baseline (page "PTQ 权重量化：从 GPTQ 到 AWQ", section on
 * RTN's limits: every weight rounded on its own): same grids as above fitted
 * on the original W, no error feedback, natural column order.  Uses bits,
 * symmetric, group_size and grid of cfg (DYNAMIC and STATIC are the same
 * here; TENSOR rounds on the one grid of the whole matrix, scales and zeros
 * [d_out][1]).
 */
GPTQ_API gptq_status gptq_rtn_quantize(const float *W, int64_t d_out, int64_t d_in, const gptq_config *cfg,
                              uint8_t *codes, float *scales, float *zeros, hipStream_t stream);

/*
 * Layer loss ||W X - W_hat X||_F^2 = 1/2 sum_r D_r H D_r^T with D = W_hat - W
 * (page "LLM 量化方法原理与实现详解", §4.1 objective; H = 2 X X^T undamped).
 *
 *   W         [d_out][d_in] original fp32 weights, ORIGINAL column order.
 *   codes     [d_out][d_in] u8, ORIGINAL column order.
 *   scales, zeros [d_out][n_groups]; g_idx [d_in] group of each original
 *             column, or NULL for column c in group c / group_size.
 *   H         [d_in][d_in] fp32, upper triangle read (original order).
 *   loss_dev  device double out.
 *   ws        scratch of gptq_workspace_bytes(GPTQ_OP_LOSS, d_out, d_in, 0, NULL).
 * Products are fp32 on matrix cores; tile sums are reduced in fp64.
 */
GPTQ_API gptq_status gptq_layer_loss(const float *W, const uint8_t *codes, const float *scales, const float *zeros,
                            const int32_t *g_idx, const float *H, int64_t d_out, int64_t d_in,
                            int32_t group_size, double *loss_dev, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * Per-channel scaling before the pass (page "LLM 量化方法原理与实现详解", §4.2
 * AWQ and §4.3 SmoothQuant).  Both pick s[d_in] > 0 and hand GPTQ (or RTN)
 * the equivalent problem W' = W diag(s), H' = diag(s)^-1 H diag(s)^-1; at
 * inference the activations are divided by s (folded into the previous op).
 *
 * gptq_channel_stats: per input channel of X [d_in][ldx] (bf16 bit patterns
 *   or fp32, n_tok tokens): absmax[c] = max(absmax[c], max_t |x|) (fp32) and
 *   abssum[c] += sum_t |x| (fp64), both device arrays, accumulating over
 *   calls (start them at 0).
 * gptq_smooth_scales: s_j = max(act_absmax_j^alpha / max_r |W[r][j]|^(1-alpha), 1e-5)
 *   (s_j = 1 when the denominator is 0), 0 <= alpha <= 1.
 *   ws: gptq_workspace_bytes(GPTQ_OP_SMOOTH, d_out, d_in, 0, NULL).
 * gptq_awq_search: for alpha = i / n_grid, i = 0 .. n_grid - 1, the scales
 *   s_j = max((a_j / w_j)^alpha, 1e-5) with a_j = act_abssum_j / n_tok and
 *   w_j = mean_r |W[r][j]| (s_j = 1 when w_j = 0); W' is rounded to the
 *   nearest grid point (bits, symmetric, group_size of cfg, grids fitted on W')
 *   and losses[i] = ||Q(W') diag(s)^-1 X - W X||^2, measured through H'
 *   (H: the undamped upper triangle).  best = the first smallest loss; s gets
 *   its scales.  All outputs are device pointers; nothing synchronizes.
 *   1 <= n_grid <= 64.  ws: gptq_workspace_bytes(GPTQ_OP_AWQ, d_out, d_in, 0, cfg).
 * gptq_scale_layer: in place, W <- W diag(s) (may be NULL), H <- diag(s)^-1 H
 *   diag(s)^-1 on the upper triangle (may be NULL), hdiag <- hdiag / s^2 (may
 *   be NULL).
 */
GPTQ_API gptq_status gptq_channel_stats(const void *X, gptq_dtype x_dtype, int64_t d_in, int64_t n_tok, int64_t ldx,
                                        float *absmax, double *abssum, hipStream_t stream);
GPTQ_API gptq_status gptq_smooth_scales(const float *act_absmax, const float *W, int64_t d_out, int64_t d_in,
                                        float alpha, float *s, void *ws, size_t ws_bytes, hipStream_t stream);
GPTQ_API gptq_status gptq_awq_search(const float *W, int64_t d_out, int64_t d_in, const float *H,
                                     const double *act_abssum, int64_t n_tok, const gptq_config *cfg, int32_t n_grid,
                                     float *s, double *losses, int32_t *best, void *ws, size_t ws_bytes,
                                     hipStream_t stream);
GPTQ_API gptq_status gptq_scale_layer(float *W, int64_t d_out, int64_t d_in, float *H, double *hdiag, const float *s,
                                      hipStream_t stream);

/*
 * Packed codes (after the pass; page "量化经典：LLM.int8 / GPTQ / AWQ", GPTQ
 * section: 3/4-bit weights plus scales -- the pages print no storage format).
 * Each row becomes one little-endian bit stream: packed column k is
 * codes[o][perm ? perm[k] : k] at bits [bits*k, bits*k + bits) of the row's
 * stream, in 32-bit words (word w = stream bits 32w .. 32w+31), the tail
 * padded with zero bits.
 *   codes   [d_out][d_in] u8, ORIGINAL column order; codes are masked to bits.
 *   perm    [d_in] int32 or NULL: the order the groups run in.  Pass the
 *           act-order permutation when the grids are DYNAMIC (groups in
 *           processing order), NULL for STATIC, TENSOR or natural order.
 *   packed  [d_out][ceil(d_in*bits/32)] u32 out.
 * bits: 2..8.  Integer work: bit-exact.
 */
GPTQ_API gptq_status gptq_pack_codes(const uint8_t *codes, int64_t d_out, int64_t d_in, int32_t bits,
                                     const int32_t *perm, uint32_t *packed, hipStream_t stream);

/*
 * W4A16 product (page "LLM 量化方法原理与实现详解", §6.2: 4-bit weights, 16-bit
 * activations; §2.2: dequantized weight (q - z) s):
 *   Y[m][o] = sum_k X[m][kperm ? kperm[k] : k] * (q[o][k] - z[o][k/g]) * s[o][k/g]
 * with q[o][k] packed column k of row o (4-bit, from gptq_pack_codes) and g =
 * group_size (0: d_in).  Groups are contiguous in packed order.
 *   X       fp16 [M][ldx] activations, one row per token (x_dtype must be
 *           GPTQ_DT_F16); 16-byte aligned, ldx a multiple of 8.
 *   kperm   [d_in] int32 or NULL: the perm the codes were packed with.
 *   packed  [d_out][d_in/8] u32; scales, zeros [d_out][d_in/g] fp32, zeros
 *           integers in 0..15 (as the quantizer stores them).
 *   Y       fp32 [M][ldy] out.
 *   ws      scratch of gptq_workspace_bytes(GPTQ_OP_W4A16, d_out, d_in, M, NULL).
 * Products are exact (integer weights times fp16 on fp16 matrix cores); sums
 * are fp32, added over K splits in a fixed order (deterministic).  g must be
 * a multiple of 32 (else GPTQ_ERR_UNSUPPORTED); packed 16-byte aligned.
 */
GPTQ_API gptq_status gptq_w4a16_gemm(const void *X, gptq_dtype x_dtype, int64_t M, int64_t d_in, int64_t ldx,
                                     const int32_t *kperm, const uint32_t *packed, const float *scales,
                                     const float *zeros, int32_t group_size, int64_t d_out, float *Y, int64_t ldy,
                                     void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Kernel timing for benchmarks (off by default).  While enabled, the column
 * pass records a pair of HIP events around each of its kernel launches of the
 * kinds below, on the stream the kernel runs on:
 *   GPTQ_TIMED_LAZY        the trailing-update products of the lazy batches
 *                          that run on the fp32 matrix cores;
 *   GPTQ_TIMED_BATCH       the batch kernels of the column pass;
 *   GPTQ_TIMED_LAZY_SPLIT  the trailing-update products that run on the bf16
 *                          matrix cores through the exact three-term split of
 *                          their fp32 operands (six bf16 products per fp32 one).
 * gptq_timing_read(op, ms, count, flops) waits for the recorded events of that
 * kind, returns their summed elapsed milliseconds, how many launches they
 * cover and, if `flops` is not NULL, the floating-point operations those
 * launches perform as fp32 arithmetic (2 M N K per product; 0 for the batch
 * kernels), all through host pointers, and forgets them.  Launches that run
 * beside each other on different streams are timed each on its own.
 * Process-wide; recording adds two event records per launch.
 */
typedef enum { GPTQ_TIMED_LAZY = 0, GPTQ_TIMED_BATCH = 1, GPTQ_TIMED_LAZY_SPLIT = 2 } gptq_timed_op;
GPTQ_API gptq_status gptq_timing_enable(int32_t on);
GPTQ_API gptq_status gptq_timing_read(int32_t op, double *ms, int64_t *count, double *flops);

/* Scratch bytes needed by `op` for these sizes (cfg may be NULL for
 * GPTQ_OP_HESSIAN and GPTQ_OP_LOSS).  `out` is a host pointer. */
GPTQ_API gptq_status gptq_workspace_bytes(int op, int64_t d_out, int64_t d_in, int64_t n_tok, const gptq_config *cfg,
                                 size_t *out);

/* Static text for a status code. */
GPTQ_API const char *gptq_status_string(gptq_status status);
/* Message of the calling thread's last failed call ("" if none). */
GPTQ_API const char *gptq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
