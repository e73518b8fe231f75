/*
 * gptq_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct CPU reference of GPTQ's column pass and of
 * the round-to-nearest (RTN) baseline.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load this file's library; the product
 * path never does.  It shares no code with the GPU library.
 *
 * Sources (the pages are the authority):
 *  - quantizer grids: page "LLM 量化方法原理与实现详解", §2.2 (symmetric and
 *    asymmetric integer quantization, with the printed reference code) and
 *    §2.3 (per-group granularity along in_features);
 *  - column pass: page "PTQ 权重量化：从 GPTQ 到 AWQ", section "GPTQ：Hessian
 *    引导的误差补偿" (update of the not-yet-quantized weights by the scaled
 *    column of the inverse Hessian), and page "量化经典：LLM.int8 / GPTQ /
 *    AWQ", §二 "方法核心" steps 3-4 (error compensation, lazy batch update).
 *
 * Precision.  The weight trajectory, the error terms and the inverse-Hessian
 * factor are binary64.  The grid itself (scale, zero point, code) is taken in
 * binary32: scales are stored as fp32, so the dequantized weight the layer
 * actually gets is (code - zero) * scale rounded to fp32, and the rounding
 * decision is made in the same precision as on the GPU.
 *
 * Readings of points the pages leave open:
 *  - symmetric grid: q in [-qmax, qmax], qmax = 2^(b-1)-1, scale = max|x|/qmax,
 *    stored code = q + 2^(b-1) with zero point 2^(b-1);
 *  - asymmetric grid: lo = min(min x, 0), hi = max(max x, 0),
 *    scale = (hi-lo)/(2^b-1), zero = clamp(rint(-lo/scale)), code =
 *    clamp(rint(x/scale + zero));  a zero-width group gets scale 1, zero 0;
 *  - rint rounds half to even (the pages' code uses torch.round);
 *  - a group's scale is fitted when its first column is reached, from the
 *    weights as they are at that moment (after earlier error feedback);
 *    the static variant fits every group from the original weights before
 *    the pass, and the per-tensor variant one grid from the whole matrix;
 *  - update sign: remaining weights -= (w - w_hat) / U[j][j] * U[j][k], where
 *    U is the upper Cholesky factor of the damped inverse Hessian
 *    (U^T U = H^-1), i.e. the scaled row of H_F^-1 on the remaining set F.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (see oracle/build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Grid of one group, decided in binary32 from the group's current values. */
static void grid_params(const double *w, int64_t n, int bits, int sym, float *scale, float *zero)
{
    if (sym) {
        float amax = 0.0f;
        for (int64_t i = 0; i < n; ++i) {
            float a = fabsf((float)w[i]);
            if (a > amax) amax = a;
        }
        float qmax = (float)((1 << (bits - 1)) - 1);
        float s = amax / qmax;
        if (s == 0.0f) s = 1.0f;
        *scale = s;
        *zero = (float)(1 << (bits - 1));
    } else {
        float lo = 0.0f, hi = 0.0f;
        for (int64_t i = 0; i < n; ++i) {
            float v = (float)w[i];
            if (v < lo) lo = v;
            if (v > hi) hi = v;
        }
        float maxq = (float)((1 << bits) - 1);
        float s = (hi - lo) / maxq;
        float z;
        if (s == 0.0f) {
            s = 1.0f;
            z = 0.0f;
        } else {
            z = rintf(-lo / s);
            if (z < 0.0f) z = 0.0f;
            if (z > maxq) z = maxq;
        }
        *scale = s;
        *zero = z;
    }
}

/* Stored code of one value on a given grid (binary32 decision). */
static float code_of(float x, float s, float z, int bits, int sym)
{
    if (sym) {
        float qmax = (float)((1 << (bits - 1)) - 1);
        float q = rintf(x / s);
        if (q < -qmax) q = -qmax;
        if (q > qmax) q = qmax;
        return q + (float)(1 << (bits - 1));
    } else {
        float maxq = (float)((1 << bits) - 1);
        float q = rintf(x / s + z);
        if (q < 0.0f) q = 0.0f;
        if (q > maxq) q = maxq;
        return q;
    }
}

/* Dequantized value (code - zero) * scale, in binary32 like the stored format. */
static float dequant(float code, float s, float z)
{
    return (code - z) * s;
}

/*
 * Round-to-nearest baseline: every group's grid from the original weights,
 * no error feedback.  W, codes: [d_out][d_in]; scales, zeros: [d_out][n_groups].
 * group == 0 means one group per row.
 */
int oracle_rtn(int64_t d_out, int64_t d_in, const float *W, int bits, int sym, int64_t group,
               uint8_t *codes, float *scales, float *zeros)
{
    int64_t g = group > 0 ? group : d_in;
    if (bits < 2 || bits > 8 || d_in % g != 0) return -1;
    int64_t ng = d_in / g;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < d_out; ++r) {
        double *buf = (double *)malloc(sizeof(double) * (size_t)g);
        for (int64_t gi = 0; gi < ng; ++gi) {
            const float *w = W + r * d_in + gi * g;
            for (int64_t i = 0; i < g; ++i) buf[i] = (double)w[i];
            float s, z;
            grid_params(buf, g, bits, sym, &s, &z);
            scales[r * ng + gi] = s;
            zeros[r * ng + gi] = z;
            for (int64_t i = 0; i < g; ++i)
                codes[r * d_in + gi * g + i] = (uint8_t)code_of(w[i], s, z, bits, sym);
        }
        free(buf);
    }
    return 0;
}

/*
 * GPTQ column pass over independent rows, in processing order.
 *
 *   W      [n_rows][ldw]  fp64 weights (already in processing order; not modified)
 *   U      [d][d]         fp64 upper factor, U^T U = damped H^-1 (lower part ignored)
 *   block  0: unblocked, every error is pushed onto all later columns at once;
 *          B > 0: lazy batches of at most B columns -- inside a batch errors go
 *          onto the batch's later columns, and the batch's accumulated error
 *          goes onto all later columns when the batch ends.  A batch is cut
 *          short at a group start whose group would cross its end, so every
 *          group is fitted from fully updated weights.
 * Outputs (processing order):
 *   codes  [n_rows][d], scales/zeros [n_rows][d/g],
 *   w_at_q [n_rows][d]  the weight's value when its column was quantized (may be NULL),
 *   err    [n_rows][d]  e_j = (w_j - w_hat_j) / U[j][j] (may be NULL).
 */
int oracle_gptq_pass(int64_t n_rows, int64_t d, const double *W, int64_t ldw, const double *U,
                     int bits, int sym, int64_t group, int64_t block,
                     uint8_t *codes, float *scales, float *zeros, double *w_at_q, double *err)
{
    int64_t g = group > 0 ? group : d;
    if (bits < 2 || bits > 8 || d % g != 0 || block < 0) return -1;
    int64_t ng = d / g;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        double *w = (double *)malloc(sizeof(double) * (size_t)d);
        double *e = (double *)malloc(sizeof(double) * (size_t)d);
        if (!w || !e) {
            status = -2;
            free(w);
            free(e);
            continue;
        }
        memcpy(w, W + r * ldw, sizeof(double) * (size_t)d);
        float s = 1.0f, z = 0.0f;
        int64_t c0 = 0;
        while (c0 < d) {
            int64_t c1 = d;
            if (block > 0) {
                c1 = c0 + block < d ? c0 + block : d;
                for (int64_t j = c0 + 1; j < c1; ++j)
                    if (j % g == 0 && j + g > c1) {
                        c1 = j;
                        break;
                    }
            }
            for (int64_t j = c0; j < c1; ++j) {
                if (j % g == 0) {
                    grid_params(w + j, g, bits, sym, &s, &z);
                    scales[r * ng + j / g] = s;
                    zeros[r * ng + j / g] = z;
                }
                float code = code_of((float)w[j], s, z, bits, sym);
                double wh = (double)dequant(code, s, z);
                double ej = (w[j] - wh) / U[j * d + j];
                codes[r * d + j] = (uint8_t)code;
                if (w_at_q) w_at_q[r * d + j] = w[j];
                e[j] = ej;
                if (err) err[r * d + j] = ej;
                int64_t kend = block > 0 ? c1 : d;
                for (int64_t k = j + 1; k < kend; ++k) w[k] -= ej * U[j * d + k];
            }
            if (block > 0) {
                for (int64_t k = c1; k < d; ++k) {
                    double acc = 0.0;
                    for (int64_t j = c0; j < c1; ++j) acc += e[j] * U[j * d + k];
                    w[k] -= acc;
                }
            }
            c0 = c1;
        }
        free(w);
        free(e);
    }
    return status;
}

/*
 * Column pass on grids fixed before it starts (page "LLM 量化方法原理与实现详解",
 * §2.3 granularity: static groups, whose scales come from the original
 * weights, and a single grid for the whole tensor).  The updates are those of
 * oracle_gptq_pass; only the grid of each column differs: processing column j
 * of row r is quantized on grid col_grid[j] of that row, i.e. on
 * (gscales[r][col_grid[j]], gzeros[r][col_grid[j]]), and no grid is refitted
 * during the pass.  Lazy batches (block > 0) are plain runs of `block`
 * columns: with no refit, no batch has to be cut short.
 *   col_grid [d]              grid index of each processing column, in [0, ngrid)
 *   gscales, gzeros [n_rows][ngrid]
 * Outputs as in oracle_gptq_pass (codes, w_at_q, err; the latter two may be NULL).
 */
int oracle_gptq_pass_fixed(int64_t n_rows, int64_t d, const double *W, int64_t ldw, const double *U,
                           int bits, int sym, const int64_t *col_grid, int64_t ngrid, const float *gscales,
                           const float *gzeros, int64_t block, uint8_t *codes, double *w_at_q, double *err)
{
    if (bits < 2 || bits > 8 || block < 0 || ngrid < 1) return -1;
    for (int64_t j = 0; j < d; ++j)
        if (col_grid[j] < 0 || col_grid[j] >= ngrid) return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        double *w = (double *)malloc(sizeof(double) * (size_t)d);
        double *e = (double *)malloc(sizeof(double) * (size_t)d);
        if (!w || !e) {
            status = -2;
            free(w);
            free(e);
            continue;
        }
        memcpy(w, W + r * ldw, sizeof(double) * (size_t)d);
        int64_t step = block > 0 ? block : d;
        for (int64_t c0 = 0; c0 < d; c0 += step) {
            int64_t c1 = c0 + step < d ? c0 + step : d;
            for (int64_t j = c0; j < c1; ++j) {
                float s = gscales[r * ngrid + col_grid[j]];
                float z = gzeros[r * ngrid + col_grid[j]];
                float code = code_of((float)w[j], s, z, bits, sym);
                double wh = (double)dequant(code, s, z);
                double ej = (w[j] - wh) / U[j * d + j];
                codes[r * d + j] = (uint8_t)code;
                if (w_at_q) w_at_q[r * d + j] = w[j];
                e[j] = ej;
                if (err) err[r * d + j] = ej;
                for (int64_t k = j + 1; k < c1; ++k) w[k] -= ej * U[j * d + k];
            }
            for (int64_t k = c1; k < d; ++k) {
                double acc = 0.0;
                for (int64_t j = c0; j < c1; ++j) acc += e[j] * U[j * d + k];
                w[k] -= acc;
            }
        }
        free(w);
        free(e);
    }
    return status;
}

/* Sampled entries of H = 2 X X^T in fp64 (X bf16 bit patterns or fp32). */
static double widen(const void *X, int is_bf16, int64_t idx)
{
    if (is_bf16) {
        uint32_t u = (uint32_t)((const uint16_t *)X)[idx] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)X)[idx];
}

int oracle_hessian_entries(const void *X, int is_bf16, int64_t d_in, int64_t n_tok, int64_t ldx,
                           int64_t n_pairs, const int64_t *rows, const int64_t *cols, double *out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < n_pairs; ++p) {
        int64_t i = rows[p], j = cols[p];
        double acc = 0.0;
        if (i >= 0 && j >= 0 && i < d_in && j < d_in)
            for (int64_t t = 0; t < n_tok; ++t) acc += widen(X, is_bf16, i * ldx + t) * widen(X, is_bf16, j * ldx + t);
        out[p] = 2.0 * acc;
    }
    return 0;
}
