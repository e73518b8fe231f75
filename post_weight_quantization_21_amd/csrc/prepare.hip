// Steps 2-3 of GPTQ: column order, damping and U = upper Cholesky factor of
// H_d^-1 (U^T U = H_d^-1).
//
// The column pass needs, for every column j, row j of the inverse Hessian of
// the columns not yet quantized (page "PTQ 权重量化：从 GPTQ 到 AWQ", GPTQ
// section).  Those rows, scaled by their diagonal's square root, are the rows
// of U.  Route (2/3 d^3 flops, fp32):
//   1. H_d = P H P^T + lambda I           (gather + one-workgroup damping)
//   2. UL-Cholesky H_d = T T^T, T upper   (blocked on two levels, from the
//      bottom-right corner: panels of 512 columns, each factored in steps of
//      64, one launch per step -- the step's column of T by back substitution,
//      the rank-64 update of the panel's remaining columns on matrix cores, the
//      next diagonal block factored by one workgroup -- then one rank-512
//      update of the whole leading block by the fp32 matrix-core GEMM)
//   3. U = T^-1                           (the diagonal blocks are inverted
//      all at once after the factorization; the off-diagonal blocks are merged
//      pairwise by the block formula inv([[A, B], [0, C]]) =
//      [[A^-1, -A^-1 B C^-1], [0, C^-1]], one batched matrix-core product
//      pair per level.)
// Indeed T T^T = H_d gives H_d^-1 = T^-T T^-1 = U^T U with U = T^-1 upper.
#include "common.h"
#include "quad.h"

#include <algorithm>

namespace gptq {
namespace {

constexpr int NB = 64;  // diagonal block edge
constexpr int kThreads = 256;

// perm[rank] = column; rank by descending key, ties by lower index (stable).
// NaN keys sort last, so the ranks always form a permutation.
__device__ __forceinline__ double order_key(const double *hdiag, const float *H, int64_t d, int64_t i) {
    const double k = hdiag ? hdiag[i] : (double)H[i * d + i];
    return k == k ? k : -__builtin_inf();
}

// Ranks over slices of kKeySlice keys: workgroup (x, y) ranks keys
// 256x .. 256x+255 against the keys of slice y (staged in LDS; every lane reads
// the same key, a broadcast) and adds the partial counts to rank[] (zeroed
// beforehand); scatter_rank_kernel then writes perm.
constexpr int kKeySlice = 1024;
__global__ __launch_bounds__(kThreads) void rank_kernel(const double *__restrict__ hdiag, const float *__restrict__ H,
                                                        int64_t d, int32_t *__restrict__ rank) {
    __shared__ double keys[kKeySlice];
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t j0 = (int64_t)blockIdx.y * kKeySlice;
    const int n = (int)(d - j0 < kKeySlice ? d - j0 : kKeySlice);
    for (int jj = threadIdx.x; jj < n; jj += kThreads) keys[jj] = order_key(hdiag, H, d, j0 + jj);
    const double ki = i < d ? order_key(hdiag, H, d, i) : 0.0;
    __syncthreads();
    int32_t r = 0;
    for (int jj = 0; jj < n; ++jj) {
        const double kj = keys[jj];
        r += (kj > ki) || (kj == ki && j0 + jj < i);
    }
    if (i < d && r > 0) atomicAdd(&rank[i], r);
}

__global__ __launch_bounds__(kThreads) void scatter_rank_kernel(const int32_t *__restrict__ rank, int64_t d,
                                                                int32_t *__restrict__ perm) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < d) perm[rank[i]] = (int32_t)i;
}

// A[a][b] = S[pa][pb] for a <= b (upper triangle of P S P^T), S with row
// stride lds: one workgroup per row a (grid-stride), its threads along b, so
// the writes are coalesced and the reads fall in one row of S (a row of H's
// upper triangle when there is no permutation: pa = a <= b = pb).
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const float *__restrict__ S, int64_t lds,
                                                               const int32_t *__restrict__ perm, int64_t d, int64_t lda,
                                                               float *__restrict__ A) {
    for (int64_t a = blockIdx.x; a < d; a += gridDim.x) {
        const int64_t pa = perm ? min(max((int64_t)perm[a], (int64_t)0), d - 1) : a;
        const float *__restrict__ src = S + pa * lds;
        float *__restrict__ dst = A + a * lda;
        for (int64_t b = a + threadIdx.x; b < d; b += kThreads)
            dst[b] = src[perm ? min(max((int64_t)perm[b], (int64_t)0), d - 1) : b];
    }
}

// The same under a column order for rows of at most kStagedRowMax entries:
// row pa of S is staged in LDS with 16-byte loads (S's rows are 16-byte
// aligned: lds a multiple of 4, S aligned), and the permuted picks read LDS.
constexpr int64_t kStagedRowMax = 16384;
__global__ __launch_bounds__(kThreads) void gather_perm_rows_kernel(const float *__restrict__ S, int64_t lds,
                                                                    const int32_t *__restrict__ perm, int64_t d,
                                                                    int64_t lda, float *__restrict__ A) {
    extern __shared__ float4 row4[];
    const float *row = reinterpret_cast<const float *>(row4);
    const int64_t n4 = (d + 3) / 4;  // within the row's padding (lds >= 4 n4)
    for (int64_t a = blockIdx.x; a < d; a += gridDim.x) {
        const int64_t pa = min(max((int64_t)perm[a], (int64_t)0), d - 1);
        const float4 *__restrict__ src = reinterpret_cast<const float4 *>(S + pa * lds);
        __syncthreads();  // the previous row's picks are done
        for (int64_t i = threadIdx.x; i < n4; i += kThreads) row4[i] = src[i];
        __syncthreads();
        float *__restrict__ dst = A + a * lda;
        for (int64_t b = a + threadIdx.x; b < d; b += kThreads) dst[b] = row[min(max((int64_t)perm[b], (int64_t)0), d - 1)];
    }
}

// S = H + H^T - diag(H) from H's upper triangle (both triangles of S written),
// by 64 x 64 tiles (ti <= tj) through LDS so that the mirrored tile is also
// written along rows.  Grid (nt, nt); the blocks below the diagonal exit.
constexpr int kSymTile = 64;
__global__ __launch_bounds__(kThreads) void symmetrize_kernel(const float *__restrict__ H, int64_t d, int64_t lds,
                                                              float *__restrict__ S) {
    const int ti = blockIdx.y, tj = blockIdx.x;
    if (ti > tj) return;
    __shared__ float t[kSymTile][kSymTile + 1];
    const int64_t r0 = (int64_t)ti * kSymTile, c0 = (int64_t)tj * kSymTile;
    const int cx = threadIdx.x % kSymTile, ry = threadIdx.x / kSymTile;  // 4 rows per pass
    for (int r = ry; r < kSymTile; r += kThreads / kSymTile) {
        const int64_t i = r0 + r, j = c0 + cx;
        t[r][cx] = (i < d && j < d && i <= j) ? H[i * d + j] : 0.0f;
    }
    __syncthreads();
    for (int r = ry; r < kSymTile; r += kThreads / kSymTile) {
        // S[r0 + r][c0 + cx] (the tile itself; on a diagonal tile its lower part mirrored)
        const int64_t i = r0 + r, j = c0 + cx;
        if (i < d && j < d) S[i * lds + j] = (ti < tj || r <= cx) ? t[r][cx] : t[cx][r];
        // S[c0 + r][r0 + cx] = H[r0 + cx][c0 + r] (the mirror of an off-diagonal tile)
        const int64_t i2 = c0 + r, j2 = r0 + cx;
        if (ti < tj && i2 < d && j2 < d) S[i2 * lds + j2] = t[cx][r];
    }
}

// lambda = damp_rel * mean(diag A) (fp64, fixed tree); A[i][i] += lambda.  One workgroup.
__global__ __launch_bounds__(kThreads) void damp_kernel(float *__restrict__ A, int64_t d, int64_t lda, float damp_rel) {
    __shared__ double red[kThreads];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < d; i += kThreads) s += (double)A[i * lda + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    const float lam = (float)((double)damp_rel * red[0] / (double)d);
    for (int64_t i = threadIdx.x; i < d; i += kThreads) A[i * lda + i] += lam;
}

__global__ __launch_bounds__(kThreads) void fill_kernel(float *__restrict__ p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) p[i] = v;
}

__global__ void zero_int_kernel(int32_t *p) { *p = 0; }

__global__ __launch_bounds__(kThreads) void iota_kernel(int32_t *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = (int32_t)i;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Rows past nb (and columns past nb) of a block row become the identity; the
// strictly lower part is cleared.
__device__ __forceinline__ void mask_block_row(float (&c)[NB], int lane, int nb) {
#pragma unroll
    for (int m = 0; m < NB; ++m) {
        const bool in = lane < nb && m < nb;
        c[m] = in ? (m >= lane ? c[m] : 0.0f) : (m == lane ? 1.0f : 0.0f);
    }
}

// UL-Cholesky of one diagonal block on the four waves of a workgroup.  For
// j = NB-1..0:  t_jj = sqrt(c_jj);  t_ij = c_ij / t_jj (i < j);
// c_ii' -= t_ij t_i'j (i' < j).  Wave w holds columns 16w .. 16w+15 of every row
// (lane i = row i) in cw (upper part, zero below the diagonal, the identity past
// nb).  The columns are factored from the right in four panels of 16:
//  * the panel's owner wave factors its 16 columns alone: the pivot comes from
//    its lane by readlane, t = c_j rsq(c_jj) on every lane (lane j gets t_jj;
//    lanes past j only change entries below their diagonal, which no later step
//    reads and which are stored as zero); the next pivot's column is updated at
//    once from a readlane of t, the panel's other columns one step later from
//    t's copy in LDS (col), so the pivot chain waits for neither; each column of
//    T also goes to LDS (pt);
//  * then every wave left of the panel subtracts the panel's rank-16 product
//    from its own 16 columns, reading its row's panel entries and the panel
//    rows of its columns (broadcasts) from LDS, four panel columns at a time
//    into 16 independent sums.
// A non-positive pivot sets t_jj = 1, and *info = kb + j + 1 for the first one
// in processing order (the first over all blocks wins).  T goes into the
// factor's diagonal block Tf[kb:kb+nb, kb:kb+nb] (upper part).
constexpr int kFCols = NB / 4;  // columns per wave
struct FactorSmem {
    float pt[NB][kFCols + 4];  // pt[i][m] = T[i][16 w + m] of the current panel w
    float col[2][NB];          // the owner's last two columns of T, by row
    int32_t badj[4];           // per wave: highest bad pivot column below nb, or -1
};
static_assert(sizeof(FactorSmem) <= sizeof(float) * NB * (NB + 4), "the factor's LDS reuses one 64 x 68 panel buffer");

// Row `lane` of the block, wave w's columns, masked: zero below the diagonal,
// the identity past nb.
__device__ __forceinline__ void mask_block_cols(float (&cw)[kFCols], int lane, int wave, int nb) {
#pragma unroll
    for (int m = 0; m < kFCols; ++m) {
        const int c = kFCols * wave + m;
        const bool in = lane < nb && c < nb;
        cw[m] = in ? (c >= lane ? cw[m] : 0.0f) : (c == lane ? 1.0f : 0.0f);
    }
}

__device__ __forceinline__ void factor_block(float (&cw)[kFCols], int wave, int nb, int64_t kb, float *__restrict__ Tf,
                                             int64_t lda, int32_t *__restrict__ info, FactorSmem &fs) {
    const int lane = (int)__lane_id();
    wave = __builtin_amdgcn_readfirstlane(wave);  // uniform: the panel branches are scalar
    // The masks of the block's loading (lanes and columns against nb) are not
    // reused here: kept live across the steps, they would take the scalar
    // registers.
    asm volatile("" : "+s"(nb));
    uint32_t bad_mask = 0;  // bad pivots of this wave's panel (bit m: column 16 wave + m)
#pragma unroll
    for (int w = 3; w >= 0; --w) {
        if (wave == w) {
            float tp = 0.0f;            // the previous step's column of T (this lane's entry)
            float4 cv[kFCols / 4] = {};  // ... and its panel rows, read at the end of that step
#pragma unroll
            for (int m = kFCols - 1; m >= 0; --m) {
                const int j = kFCols * w + m;
                const float p0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cw[m]), j));  // pivot
                const bool bad = !(p0 > 0.0f);
                // (bad is the same on every lane; the ballot keeps the mask scalar)
                bad_mask |= __builtin_amdgcn_ballot_w64(bad) ? (1u << m) : 0u;
                // hardware reciprocal square root (about 1 ulp): the factor
                // only has to be accurate
                const float t = cw[m] * __builtin_amdgcn_rsqf(bad ? 1.0f : p0);
                cw[m] = t;
                fs.pt[lane][m] = t;
                // step m+1's update of columns 0 .. m-1 (its column m was updated then)
                if (m + 1 < kFCols) {
#pragma unroll
                    for (int m2 = 0; m2 < m; ++m2) cw[m2] = fmaf(-tp, cv[m2 / 4][m2 % 4], cw[m2]);
                }
                // this step's update of the next pivot's column
                if (m >= 1) {
                    const float tm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), j - 1));
                    cw[m - 1] = fmaf(-t, tm, cw[m - 1]);
                }
                // this column's panel rows for the next step (LDS operations
                // of a wave complete in order: the reads see the write)
                if (m >= 2) {
                    fs.col[m & 1][lane] = t;
#pragma unroll
                    for (int q = 0; q < (m - 1 + 3) / 4; ++q)
                        cv[q] = *reinterpret_cast<const float4 *>(&fs.col[m & 1][kFCols * w + 4 * q]);
                }
                tp = t;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (w == 0) break;
        __syncthreads();  // the panel is in LDS
        if (wave < w) {
            // c_i,c -= sum_m T[i][16w+m] T[c][16w+m] for this wave's 16 columns c,
            // panel columns taken in pivot order (right to left)
            float4 pr[kFCols / 4];  // this row's entries of the panel
#pragma unroll
            for (int q = 0; q < kFCols / 4; ++q) pr[q] = *reinterpret_cast<const float4 *>(&fs.pt[lane][4 * q]);
#pragma unroll
            for (int q = kFCols / 4 - 1; q >= 0; --q) {
                float4 qv[kFCols];  // panel columns 4q..4q+3 of this wave's columns' rows (broadcasts)
#pragma unroll
                for (int m2 = 0; m2 < kFCols; ++m2)
                    qv[m2] = *reinterpret_cast<const float4 *>(&fs.pt[kFCols * wave + m2][4 * q]);
#pragma unroll
                for (int m2 = 0; m2 < kFCols; ++m2) cw[m2] = fmaf(-pr[q].w, qv[m2].w, cw[m2]);
#pragma unroll
                for (int m2 = 0; m2 < kFCols; ++m2) cw[m2] = fmaf(-pr[q].z, qv[m2].z, cw[m2]);
#pragma unroll
                for (int m2 = 0; m2 < kFCols; ++m2) cw[m2] = fmaf(-pr[q].y, qv[m2].y, cw[m2]);
#pragma unroll
                for (int m2 = 0; m2 < kFCols; ++m2) cw[m2] = fmaf(-pr[q].x, qv[m2].x, cw[m2]);
            }
        }
        __syncthreads();  // pt is rewritten by the next panel
    }
    // The lane masks of what follows are formed here, not hoisted above the
    // steps (where they would be kept live in scalar registers).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint32_t in_nb_bits = bad_mask & (kFCols * wave + kFCols <= nb ? 0xFFFFu
                                            : (kFCols * wave >= nb ? 0u : ((1u << (nb - kFCols * wave)) - 1u)));
    if (bad_mask != 0) {  // uniform, rarely taken: t_jj = 1
#pragma unroll
        for (int m = 0; m < kFCols; ++m)
            if ((bad_mask >> m) & 1) cw[m] = ln == kFCols * wave + m ? 1.0f : cw[m];
    }
    if (ln == 0) fs.badj[wave] = in_nb_bits ? kFCols * wave + (31 - __builtin_clz(in_nb_bits)) : -1;
    __syncthreads();
    if (wave == 0 && ln == 0) {
        int jb = -1;
#pragma unroll
        for (int v = 0; v < 4; ++v) jb = fs.badj[v] > jb ? fs.badj[v] : jb;
        if (jb >= 0) atomicCAS(info, 0, (int32_t)(kb + jb + 1));
    }
    if (ln < nb) {
        float *dst = Tf + (kb + ln) * lda + kb + kFCols * wave;
#pragma unroll
        for (int q = 0; q < kFCols / 4; ++q) {
            const int c0 = kFCols * wave + 4 * q;
            if (c0 + 3 < ln) continue;  // wholly below the diagonal
            float4 v;
            v.x = (c0 + 0 >= ln) ? cw[4 * q + 0] : 0.0f;
            v.y = (c0 + 1 >= ln) ? cw[4 * q + 1] : 0.0f;
            v.z = (c0 + 2 >= ln) ? cw[4 * q + 2] : 0.0f;
            v.w = (c0 + 3 >= ln) ? cw[4 * q + 3] : 0.0f;
            if (c0 + 3 < nb) {
                *reinterpret_cast<float4 *>(dst + 4 * q) = v;
            } else {
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + e < nb) dst[4 * q + e] = vv[e];
            }
        }
    }
}

// The first (bottom-right) diagonal block A[k0:k0+nb, k0:k0+nb], read from the
// working matrix and factored by four waves.
__global__ __launch_bounds__(kThreads) void panel_kernel(const float *__restrict__ A, float *__restrict__ Tf, int64_t lda,
                                                        int64_t k0, int nb, int32_t *__restrict__ info) {
    __shared__ __attribute__((aligned(16))) FactorSmem fs;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Row `lane` of the block, this wave's 16 columns (16-byte loads; chunks
    // past nb are not read: lda is a multiple of 4, so a chunk that starts
    // below nb ends inside the row).
    float cw[kFCols];
    const float *src = A + (k0 + (lane < nb ? lane : 0)) * lda + k0 + kFCols * wave;
#pragma unroll
    for (int q = 0; q < kFCols / 4; ++q) {
        const int c = kFCols * wave + 4 * q;
        const float4 v = c < nb ? *reinterpret_cast<const float4 *>(src + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
        cw[4 * q + 0] = v.x;
        cw[4 * q + 1] = v.y;
        cw[4 * q + 2] = v.z;
        cw[4 * q + 3] = v.w;
    }
    mask_block_cols(cw, lane, wave, nb);
    factor_block(cw, wave, nb, k0, Tf, lda, info, fs);
}

// V = T_bb^-1 of the diagonal blocks b = kb0, kb0+NB, ... (one wave each, once
// their factors exist): lane c holds column c of V.  For i = NB-1..0:
//   V_ic = -(1/t_ii) sum_{m>i} t_im V_mc (c > i), V_ii = 1/t_ii,
// reading row i of T from LDS with wave-uniform addresses.  V goes into U's
// diagonal block (zero below the diagonal).
__global__ __launch_bounds__(kWave) void invert_blocks_kernel(const float *__restrict__ Tf, float *__restrict__ U,
                                                              int64_t d, int64_t lda, int64_t kb0) {
    __shared__ __attribute__((aligned(16))) float tr[NB][NB + 4];
    const int64_t kb = kb0 + (int64_t)blockIdx.x * NB;
    const int nb = (int)(d - kb < NB ? d - kb : NB);
    const int lane = threadIdx.x;
    {
        float c[NB];
        const float *src = Tf + (kb + (lane < nb ? lane : 0)) * lda + kb;
#pragma unroll
        for (int q = 0; q < NB / 4; ++q) {
            const float4 v = 4 * q < nb ? *reinterpret_cast<const float4 *>(src + 4 * q)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
            c[4 * q + 0] = v.x;
            c[4 * q + 1] = v.y;
            c[4 * q + 2] = v.z;
            c[4 * q + 3] = v.w;
        }
        mask_block_row(c, lane, nb);
#pragma unroll
        for (int q = 0; q < NB / 4; ++q)
            *reinterpret_cast<float4 *>(&tr[lane][4 * q]) = make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
    }
    wave_sync_lds();
    float v[NB];
#pragma unroll
    for (int i = NB - 1; i >= 0; --i) {
        // row i of T, from its first 16-byte chunk that holds column i
        float4 trow[NB / 4];
#pragma unroll
        for (int q = i / 4; q < NB / 4; ++q) trow[q] = *reinterpret_cast<const float4 *>(&tr[i][4 * q]);
        const float rii = __builtin_amdgcn_rcpf(trow[i / 4][i % 4]);
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
        for (int m = i + 1; m < NB; ++m) {
            const float prod = trow[m / 4][m % 4] * v[m];
            if ((m & 3) == 0) s0 += prod;
            else if ((m & 3) == 1) s1 += prod;
            else if ((m & 3) == 2) s2 += prod;
            else s3 += prod;
        }
        float x = -rii * ((s0 + s1) + (s2 + s3));
        x = lane == i ? rii : x;
        v[i] = lane < i ? 0.0f : x;
    }
    // Column `lane` of V into U's block: each store instruction writes one row,
    // lanes along the columns.
    if (lane < nb) {
        float *dst = U + kb * d + kb + lane;
#pragma unroll
        for (int m = 0; m < NB; ++m)
            if (m < nb) dst[m * d] = v[m];
    }
}

// The panel solve of one step, P = panel T_kk^-T (so that P P^T is the
// update), row by row on four lanes per row: lane q of a quad holds columns
// q + 4t (t = 0..15) of its row.  Back substitution over the columns c =
// NB-1..0 on the unscaled values: with n_c'c = -t_c'c / t_cc,
//   a_c' += n_c'c a_c  (c' < c),  and at the end p_c = a_c / t_cc,
// which is p_c = (a_c - sum_{m>c} t_cm p_m) / t_cc.  Each update is one FMA
// whose a_c comes straight from its quad lane (DPP); the next column's operands
// are read from LDS one step ahead.
//   nq[c][p][q][i] = n_c'c for c' = q + 16p + 4i < c (zero on and below the
//   diagonal), rq[q][t] = 1 / t_cc for c = q + 4t; columns past nb are the
//   identity.
struct TkkSmem {
    float nq[NB][NB / 16][4][4];
    float rq[4][NB / 4];
};

// All kFThreads threads: T_kk (upper, Tf's diagonal block at k0) into the
// layout above; thread tid takes column tid % NB.  Global reads are row-wise
// (coalesced).
constexpr int kFThreads = 256;
__device__ __forceinline__ void load_tkk(TkkSmem &s, const float *__restrict__ Tf, int64_t lda, int64_t k0, int nb,
                                         int tid) {
    constexpr int kPer = NB * NB / kFThreads;
    const int c = tid % NB, rb = tid / NB;  // rows rb + 4u
    float tv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int r = rb + 4 * u;
        tv[u] = (r < c && c < nb) ? Tf[(k0 + r) * lda + k0 + c] : 0.0f;
    }
    const float rc = c < nb ? 1.0f / Tf[(k0 + c) * lda + k0 + c] : 1.0f;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int r = rb + 4 * u;
        s.nq[c][r / 16][r % 4][(r / 4) % 4] = r < c ? -tv[u] * rc : 0.0f;
    }
    if (rb == 0) s.rq[c % 4][c / 4] = rc;
}

// One row (TWO: two rows, a and b, sharing each step's reads of T_kk).
template <bool TWO>
__device__ __forceinline__ void trsm_rows(float (&a)[NB / 4], float (&b)[NB / 4], int q, const TkkSmem &s) {
    float4 nu[2][NB / 16];
    auto load_col = [&](int c, float4(&dst)[NB / 16]) {
#pragma unroll
        for (int p = 0; p <= (c >> 2) / 4; ++p) dst[p] = *reinterpret_cast<const float4 *>(&s.nq[c][p][q][0]);
    };
    load_col(NB - 1, nu[(NB - 1) & 1]);
#pragma unroll
    for (int c = NB - 1; c >= 0; --c) {
        const int qo = c & 3, to = c >> 2, cur = c & 1;
        if (c > 0) load_col(c - 1, nu[cur ^ 1]);
        const float pa = quad_bcast(a[to], qo);
        const float pb = TWO ? quad_bcast(b[to], qo) : 0.0f;
        auto upd = [&](int t) {
            const float4 u4 = nu[cur][t / 4];
            const float u = (t % 4 == 0) ? u4.x : (t % 4 == 1) ? u4.y : (t % 4 == 2) ? u4.z : u4.w;
            a[t] = fmaf(pa, u, a[t]);
            if constexpr (TWO) b[t] = fmaf(pb, u, b[t]);
        };
        // the next column's element first: it is the next step's pivot
        const int tn = c > 0 ? (c - 1) >> 2 : 0;
        upd(tn);
#pragma unroll
        for (int t = 0; t <= to; ++t)
            if (t != tn) upd(t);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int p = 0; p < NB / 16; ++p) {
        const float4 r4 = *reinterpret_cast<const float4 *>(&s.rq[q][4 * p]);
        const float rr[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[4 * p + i] *= rr[i];
            if constexpr (TWO) b[4 * p + i] *= rr[i];
        }
    }
}

// Row r0 + (tid / 4) of the panel A[:, k0:k0+nb], lane q's columns (zero past nb
// and past the leading rows k0).
__device__ __forceinline__ void load_panel_row(float (&a)[NB / 4], const float *__restrict__ A, int64_t lda, int64_t k0,
                                               int nb, int64_t row, int q) {
#pragma unroll
    for (int t = 0; t < NB / 4; ++t) {
        const int c = q + 4 * t;
        a[t] = (row < k0 && c < nb) ? A[row * lda + k0 + c] : 0.0f;
    }
}

// One step of the blocked factorization, fused.  Block k0 (columns k0..k0+nb)
// has been factored: T_kk sits in Tf's diagonal block.  Each workgroup takes
// one 64 x 64 upper tile (i, j) of the leading matrix A[0:k0, 0:k0]:
//   P_i = A[rows i, k0:k0+nb] T_kk^-T    (back substitution, above)
//   A[i, j] -= P_i P_j^T                  (upper part, fp32 matrix cores)
// and a diagonal tile also writes P_i into the factor T (Tf[rows i, k0:k0+nb]).
// The workgroup of the last diagonal tile, which holds the next block
// A[k0-NB:k0, k0-NB:k0], is dispatched first; after its update it factors
// that block from its updated values, so the next step's T_kk exists when the
// kernel ends, with no launch and no HBM round trip in between.  The inverses
// of the diagonal blocks are not on this chain (invert_blocks_kernel).
// PRE: P was formed once per row block by p_kernel; the tiles load P_i^T and
// P_j^T from its k-major copy Pt instead.
// The update runs on fp32 matrix cores in transposed form, D[col][row], so each
// lane's accumulators hold four consecutive columns of one row of A.
constexpr int FT = 64;   // tile edge
constexpr int FLD = FT + 4;

struct StepSmem {
    float pi[NB][FLD];  // P_i^T (k-major)
    float pj[NB][FLD];  // P_j^T (k-major); later the next block
    TkkSmem tk;
};

// Upper tiles (ti <= tj) of tile columns tj_lo .. nt-1, column by column, rows
// top to bottom: t -> (ti, tj).  Column tj holds tj + 1 tiles.
__device__ __forceinline__ void tile_upper_cols(int64_t t, int tj_lo, int nt, int &ti, int &tj) {
    int j = tj_lo;
    while (j < nt - 1 && t >= (int64_t)(j + 1)) {
        t -= j + 1;
        ++j;
    }
    tj = j;
    ti = (int)t;
}

// Tiles of a step restricted to tile columns tj_lo .. nt-1.
__host__ __device__ inline int64_t step_tiles(int tj_lo, int nt) {
    return ((int64_t)nt * (nt + 1) - (int64_t)tj_lo * (tj_lo + 1)) / 2;
}

template <bool PRE>
__global__ __launch_bounds__(kFThreads) void step_kernel(float *__restrict__ A, float *__restrict__ Tf,
                                                         const float *__restrict__ Pt, int64_t lda, int64_t k0, int nb,
                                                         int nt, int tj_lo, int32_t *__restrict__ info) {
    // Tiles in reverse order: workgroup 0 takes the last diagonal tile, whose
    // factorization of the next block is the step's longest chain.  Only the
    // tile columns tj_lo .. nt-1 (the rest of the current panel) are
    // updated; the columns left of the panel get the panel's whole product later.
    int ti, tj;
    tile_upper_cols(step_tiles(tj_lo, nt) - 1 - blockIdx.x, tj_lo, nt, ti, tj);
    const bool diag = ti == tj;
    const bool last = diag && ti == nt - 1;
    const int64_t r0 = (int64_t)ti * FT, s0 = (int64_t)tj * FT;
    __shared__ __attribute__((aligned(16))) StepSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hi = lane >> 5, lo = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int q = tid & 3, rr = tid >> 2;  // quad lane and row of the panel solve

    // Every global load is issued before the first LDS store.
    // (1) This tile's A values in the transposed accumulator layout: for
    //     g = 0..3, A[r][s .. s+3] with r = r0 + wm*32 + lo, s = s0 + wn*32 + 8g + 4*hi.
    float4 cold[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t r = r0 + wm * 32 + lo;
        const int64_t sc = s0 + wn * 32 + 8 * g + 4 * hi;
        cold[g] = (r < k0 && sc < k0) ? *reinterpret_cast<const float4 *>(A + r * lda + sc)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // (2) the rows of P (PRE: k-major P^T, float4 along the rows) or of the panel.
    float ai[NB / 4], aj[NB / 4];
    constexpr int kPer = FT * NB / 4 / kFThreads;
    float4 pv[kPer], qv[kPer];
    if constexpr (PRE) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e4 = tid + u * kFThreads;
            const int c = e4 / (FT / 4), r = (e4 % (FT / 4)) * 4;  // k0 is a multiple of FT: rows in range
            pv[u] = *reinterpret_cast<const float4 *>(Pt + c * lda + r0 + r);
            qv[u] = diag ? make_float4(0.f, 0.f, 0.f, 0.f) : *reinterpret_cast<const float4 *>(Pt + c * lda + s0 + r);
        }
    } else {
        load_panel_row(ai, A, lda, k0, nb, r0 + rr, q);
        if (!diag) load_panel_row(aj, A, lda, k0, nb, s0 + rr, q);
        load_tkk(sm.tk, Tf, lda, k0, nb, tid);
    }
    if constexpr (PRE) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int e4 = tid + u * kFThreads;
            const int c = e4 / (FT / 4), r = (e4 % (FT / 4)) * 4;
            *reinterpret_cast<float4 *>(&sm.pi[c][r]) = pv[u];
            if (!diag) *reinterpret_cast<float4 *>(&sm.pj[c][r]) = qv[u];
        }
        __syncthreads();
    } else {
        __syncthreads();  // T_kk in LDS
        if (diag)
            trsm_rows<false>(ai, aj, q, sm.tk);
        else
            trsm_rows<true>(ai, aj, q, sm.tk);
#pragma unroll
        for (int t = 0; t < NB / 4; ++t) {
            sm.pi[q + 4 * t][rr] = ai[t];
            if (!diag) sm.pj[q + 4 * t][rr] = aj[t];
        }
        if (tj == nt - 1 && r0 + rr < k0) {  // this row block's P goes into the factor (one tile per row block)
#pragma unroll
            for (int t = 0; t < NB / 4; ++t)
                if (q + 4 * t < nb) Tf[(r0 + rr) * lda + k0 + q + 4 * t] = ai[t];
        }
        __syncthreads();
    }
    float(*pjs)[FLD] = diag ? sm.pi : sm.pj;

    // A[r][s] -= sum_c P_i[r][c] P_j[s][c], as D[s][r] = sum_c P_j^T[c][s] P_i^T[c][r].
    floatx16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll 8
    for (int c = 0; c < NB; c += 2)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(pjs[c + hi][wn * 32 + lo], sm.pi[c + hi][wm * 32 + lo], acc, 0, 0, 0);
    if (last) __syncthreads();  // pj is about to hold the next block: every wave is done reading it
    const int64_t nb0 = k0 - NB;  // the next block's first row/column
    float(*blk)[NB + 4] = reinterpret_cast<float(*)[NB + 4]>(&sm.pj[0][0]);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t r = r0 + wm * 32 + lo;
        const int64_t sc = s0 + wn * 32 + 8 * g + 4 * hi;
        if (r >= k0 || sc >= k0) continue;
        float4 v = cold[g];
        v.x -= acc[4 * g + 0];
        v.y -= acc[4 * g + 1];
        v.z -= acc[4 * g + 2];
        v.w -= acc[4 * g + 3];
        if (last && r >= nb0 && sc >= nb0) {
            // the next block: kept in LDS for this workgroup's factorization
            *reinterpret_cast<float4 *>(&blk[r - nb0][sc - nb0]) = v;
            continue;
        }
        float *dst = A + r * lda + sc;
        if (!diag || r <= sc) {
            *reinterpret_cast<float4 *>(dst) = v;
        } else {  // diagonal tile: keep only r <= s
            if (r <= sc + 0) dst[0] = v.x;
            if (r <= sc + 1) dst[1] = v.y;
            if (r <= sc + 2) dst[2] = v.z;
            if (r <= sc + 3) dst[3] = v.w;
        }
    }
    if (!last) return;
    __syncthreads();  // the next block is complete in LDS
    float cw[kFCols];
#pragma unroll
    for (int q = 0; q < kFCols / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4 *>(&blk[lane][kFCols * wave + 4 * q]);
        cw[4 * q + 0] = v.x;
        cw[4 * q + 1] = v.y;
        cw[4 * q + 2] = v.z;
        cw[4 * q + 3] = v.w;
    }
    mask_block_cols(cw, lane, wave, NB);
    // P_i^T is dead: its space holds the factor's panel
    factor_block(cw, wave, NB, nb0, Tf, lda, info, *reinterpret_cast<FactorSmem *>(&sm.pi[0][0]));
}

// P = panel T_kk^-T for one 64-row block [r0, r0+64) of the leading rows
// [0, k0): the block's rows of the factor, T[rows, k0:k0+nb] (the step's panel
// solve, done once per row block), and P^T [NB][k0] (row stride lda), which
// the tiles of the step load as k-major operands.
__global__ __launch_bounds__(kFThreads) void p_kernel(const float *__restrict__ A, float *__restrict__ Tf,
                                                      float *__restrict__ Pt, int64_t lda, int64_t k0, int nb) {
    __shared__ __attribute__((aligned(16))) TkkSmem tk;
    const int64_t r0 = (int64_t)blockIdx.x * NB;
    const int tid = threadIdx.x, q = tid & 3, rr = tid >> 2;
    float a[NB / 4];
    load_panel_row(a, A, lda, k0, nb, r0 + rr, q);
    load_tkk(tk, Tf, lda, k0, nb, tid);
    __syncthreads();
    trsm_rows<false>(a, a, q, tk);
    const int64_t r = r0 + rr;  // < k0: k0 is a multiple of NB
#pragma unroll
    for (int t = 0; t < NB / 4; ++t) {
        const int c = q + 4 * t;
        Pt[c * lda + r] = a[t];  // zero past nb
        if (c < nb) Tf[r * lda + k0 + c] = a[t];
    }
}

// Wide products with K of 512 and more (the leading block's products of a
// panel, the inverse's merges and row-block solves): on the bf16 matrix cores
// through the exact three-term split when they have enough 256 x 256 tiles to
// fill the chip, else on the fp32 ones.
hipError_t launch_wide_product(const GemmDesc &g, hipStream_t s) {
    const int64_t gx = ceil_div(g.N, 256);
    const int64_t tiles = g.upper_only ? gx * (gx + 1) / 2 : ceil_div(g.M, 256) * gx;
    if (g.K >= 512 && tiles >= 64 && gemm_split_supported(g)) return launch_gemm_split(g, s);
    return launch_gemm_f32(g, s);
}

// Pairwise merges of inverted blocks: inv([[A, B], [0, C]]) = [[A^-1, -A^-1 B C^-1], [0, C^-1]],
// i.e. U12 = -U11 T12 U22 for the node [i0, i0 + ni + nj) with children
// [i0, j0 = i0 + ni) and [j0, j0 + nj).  Two products:
//   merge_right: Tw[i0:j0, j0:] = T12 U22    (needs the right child and T12)
//   merge_left:  U[i0:j0, j0:]  = -U11 Tw    (needs the left child as well)
// so the first can run as soon as the factorization has passed j0.  Batched
// over `npairs` nodes of one level (`stride` apart along the diagonal).
hipError_t merge_right(const float *Tf, float *U, float *Tw, int64_t d, int64_t lda, int64_t i0, int64_t ni, int64_t nj,
                       int64_t npairs, int64_t stride, hipStream_t st, int wgs) {
    const int64_t j0 = i0 + ni;
    GemmDesc g;
    g.max_wgs = wgs;
    g.batch = (int)npairs;
    g.M = ni;
    g.N = nj;
    g.K = nj;
    g.A = Tf + i0 * lda + j0;  // T12
    g.lda = lda;
    g.B = U + j0 * d + j0;  // U22 (upper triangular)
    g.ldb = d;
    g.b_upper = 1;
    g.C = Tw + i0 * lda + j0;
    g.ldc = lda;
    g.strideA = g.strideC = stride * (lda + 1);
    g.strideB = stride * (d + 1);
    return launch_wide_product(g, st);
}

hipError_t merge_left(float *U, const float *Tw, int64_t d, int64_t lda, int64_t i0, int64_t ni, int64_t nj,
                      int64_t npairs, int64_t stride, hipStream_t st, int wgs) {
    const int64_t j0 = i0 + ni;
    GemmDesc h;
    h.max_wgs = wgs;
    h.batch = (int)npairs;
    h.M = ni;
    h.N = nj;
    h.K = ni;
    h.A = U + i0 * d + i0;  // U11 (upper triangular, lower part zero)
    h.lda = d;
    h.a_upper = 1;
    h.B = Tw + i0 * lda + j0;
    h.ldb = lda;
    h.C = U + i0 * d + j0;
    h.ldc = d;
    h.alpha = -1.0f;
    h.beta = 0.0f;
    h.strideA = h.strideC = stride * (d + 1);
    h.strideB = stride * (lda + 1);
    return launch_wide_product(h, st);
}

// Columns per region of the inverse's assembly: once the factorization has
// passed a region, its diagonal inverses and the merges inside it run on a
// second stream, beside the rest of the factorization.
constexpr int64_t kRegion = 512;


// Workgroups of each product launched on a side stream while the
// factorization's chain runs on the caller's stream (0: one per tile): fewer
// than the chip holds, so the chain's launches find free compute units.
constexpr int kSideWgs = 0;

// U over the region [x, min(x + kRegion, d)): the diagonal inverses, then the
// merges level by level (full nodes batched, the last node possibly partial).
hipError_t assemble_region(const float *Tf, float *U, float *Tw, int64_t d, int64_t lda, int64_t x, hipStream_t st,
                           int wgs) {
    const int64_t end = std::min<int64_t>(x + kRegion, d);
    hipLaunchKernelGGL(invert_blocks_kernel, dim3((unsigned)ceil_div(end - x, NB)), dim3(kWave), 0, st, Tf, U, d, lda, x);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int64_t sz = NB; sz < end - x; sz *= 2) {
        const int64_t full = (end - x) / (2 * sz);
        if (full > 0) {
            if ((e = merge_right(Tf, U, Tw, d, lda, x, sz, sz, full, 2 * sz, st, wgs)) != hipSuccess) return e;
            if ((e = merge_left(U, Tw, d, lda, x, sz, sz, full, 2 * sz, st, wgs)) != hipSuccess) return e;
        }
        const int64_t i0 = x + 2 * full * sz;
        const int64_t ni = std::min<int64_t>(sz, end - i0), nj = end - i0 - ni;
        if (nj > 0) {
            if ((e = merge_right(Tf, U, Tw, d, lda, i0, ni, nj, 1, 0, st, wgs)) != hipSuccess) return e;
            if ((e = merge_left(U, Tw, d, lda, i0, ni, nj, 1, 0, st, wgs)) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// The upper-right block X = U[0:h, h:h+w] of a node [0, 2h) (left half
// L = [0, h), right half R = [h, h+w)) solves T_LL X = -T_LR U_RR = -Tw.  Its
// left half's inverse U_LL is complete only when the factorization ends, so
// instead of X = -U_LL Tw at the end, X is found by back substitution in row
// blocks of kRegion from the bottom, one block per region the factorization
// passes: X_J = -U_JJ Tw_J for the block J = [x, x + kRegion) (its diagonal
// inverse is the region's), then Tw_I += T_IJ X_J for the rows I = [0, x)
// above it, so the end is left with the first block only.
hipError_t solve_left_block(const float *Tf, float *U, float *Tw, int64_t d, int64_t lda, int64_t x, int64_t h,
                            int64_t w, hipStream_t st, int wgs) {
    const int64_t r = std::min<int64_t>(kRegion, h - x);
    GemmDesc a;  // U[x:x+r, h:h+w] = -U[x:x+r, x:x+r] Tw[x:x+r, h:h+w]
    a.max_wgs = wgs;
    a.M = r;
    a.N = w;
    a.K = r;
    a.A = U + x * d + x;
    a.lda = d;
    a.a_upper = 1;
    a.B = Tw + x * lda + h;
    a.ldb = lda;
    a.C = U + x * d + h;
    a.ldc = d;
    a.alpha = -1.0f;
    a.beta = 0.0f;
    hipError_t e = launch_wide_product(a, st);
    if (e != hipSuccess || x == 0) return e;
    GemmDesc b;  // Tw[0:x, h:h+w] += T[0:x, x:x+r] U[x:x+r, h:h+w]
    b.max_wgs = wgs;
    b.M = x;
    b.N = w;
    b.K = r;
    b.A = Tf + x;
    b.lda = lda;
    b.B = U + x * d + h;
    b.ldb = d;
    b.C = Tw + h;
    b.ldc = lda;
    b.alpha = 1.0f;
    b.beta = 1.0f;
    return launch_wide_product(b, st);
}

// Nodes [0, 2h) whose upper-right block is solved region by region (the
// others, with h = kRegion, are one product at the end).
inline bool solved_by_rows(int64_t h) { return h >= 2 * kRegion; }

// The inverse's work that becomes ready once the factorization has passed
// column x (a multiple of kRegion; x = 0 at the end): the region at x, then,
// for the nodes of 2, 4, ... regions, the left product of the node starting
// at x while x is aligned to it, and the right product of the node whose
// middle is x (its right half, starting at x, is complete by then); then the
// row block at x of every node [0, 2h) with h > x.
hipError_t assemble_at(const float *Tf, float *U, float *Tw, int64_t d, int64_t lda, int64_t x, hipStream_t st,
                       int wgs) {
    hipError_t e = assemble_region(Tf, U, Tw, d, lda, x, st, wgs);
    if (e != hipSuccess) return e;
    for (int64_t n = 2 * kRegion; n / 2 < d; n *= 2) {
        const int64_t half = n / 2;
        if (x % n == 0) {
            if (x + half < d && !(x == 0 && solved_by_rows(half)))
                if ((e = merge_left(U, Tw, d, lda, x, half, std::min<int64_t>(half, d - x - half), 1, 0, st, wgs)) != hipSuccess)
                    return e;
        } else if (x % n == half) {
            if ((e = merge_right(Tf, U, Tw, d, lda, x - half, half, std::min<int64_t>(half, d - x), 1, 0, st, wgs)) !=
                hipSuccess)
                return e;
            break;
        } else {
            break;
        }
    }
    for (int64_t h = 2 * kRegion; h < d; h *= 2)
        if (solved_by_rows(h) && x < h)
            if ((e = solve_left_block(Tf, U, Tw, d, lda, x, h, std::min<int64_t>(h, d - h), st, wgs)) != hipSuccess)
                return e;
    return hipSuccess;
}

// The inverse's assembly runs on the library's second stream for this step
// (default priority), forked from and joined to the caller's stream with its
// events: ev[0] forks, ev[1] joins.
hipError_t fork_to(SideStream &ss, hipStream_t s) { return signal_wait(ss.ev[0], s, ss.st); }

int64_t pad4(int64_t d) { return (d + 3) / 4 * 4; }

// Outer level of the factorization: the leading block gets each panel's
// product at once.
// Columns per panel of the outer level: wider panels mean fewer, longer
// products of the leading block and longer steps (512 measured best of 128-1024).
constexpr int64_t kPanel = 512;

}  // namespace

// Workspace: the working matrix A (Schur complements), the factor Tf and the
// merge staging Tw, each [d][pad4(d)] fp32.
size_t prepare_ws_bytes(int64_t d) { return 3 * align_up((size_t)d * (size_t)pad4(d) * sizeof(float), 256); }

hipError_t run_prepare(const float *H, const double *hdiag, int64_t d, float damp_rel, int act_order, float *U,
                       int32_t *perm, int32_t *info, void *ws, hipStream_t s) {
    const int64_t lda = pad4(d);
    const size_t mat = align_up((size_t)d * (size_t)lda * sizeof(float), 256);
    float *A = static_cast<float *>(ws);
    float *Tf = reinterpret_cast<float *>(static_cast<char *>(ws) + mat);
    float *Tw = reinterpret_cast<float *>(static_cast<char *>(ws) + 2 * mat);
    hipError_t e;
    hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, s, info);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (act_order) {
        // the ranks are counted in the working matrix's first d entries (free until the gather below)
        int32_t *rank = reinterpret_cast<int32_t *>(A);
        hipLaunchKernelGGL(fill_kernel, dim3((unsigned)ceil_div(d, kThreads)), dim3(kThreads), 0, s, A, d, 0.0f);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(rank_kernel, dim3((unsigned)ceil_div(d, kThreads), (unsigned)ceil_div(d, kKeySlice)), dim3(kThreads),
                           0, s, hdiag, H, d, rank);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(scatter_rank_kernel, dim3((unsigned)ceil_div(d, kThreads)), dim3(kThreads), 0, s, rank, d, perm);
    } else if (perm) {
        hipLaunchKernelGGL(iota_kernel, dim3((unsigned)ceil_div(d, kThreads)), dim3(kThreads), 0, s, perm, d);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // The working matrix: H's upper triangle as it is, or under a column order
    // the upper triangle of P H P^T, gathered by rows from H's symmetric
    // completion (staged in Tw, which is free until the factorization).
    const unsigned grow = (unsigned)std::min<int64_t>(d, 4096);
    if (act_order) {
        const unsigned nt = (unsigned)ceil_div(d, kSymTile);
        hipLaunchKernelGGL(symmetrize_kernel, dim3(nt, nt), dim3(kThreads), 0, s, H, d, lda, Tw);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (d <= kStagedRowMax)
            hipLaunchKernelGGL(gather_perm_rows_kernel, dim3(grow), dim3(kThreads), (size_t)ceil_div(d, 4) * 16, s, Tw, lda,
                               perm, d, lda, A);
        else
            hipLaunchKernelGGL(gather_rows_kernel, dim3(grow), dim3(kThreads), 0, s, Tw, lda, perm, d, lda, A);
    } else {
        hipLaunchKernelGGL(gather_rows_kernel, dim3(grow), dim3(kThreads), 0, s, H, d, nullptr, d, lda, A);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(kThreads), 0, s, A, d, lda, damp_rel);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nU = d * d;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(nU, kThreads), 65536)), dim3(kThreads), 0, s,
                       U, nU, 0.0f);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // UL-Cholesky from the bottom-right corner, panel by panel (kPanel columns,
    // aligned from column 0).  Inside a panel, steps of NB columns: the first
    // diagonal block is factored by panel_kernel; for block k0, step_kernel
    // forms its column of T for every row above it (back substitution against
    // T_kk, once per tile and row block; the tiles of the last column store it),
    // subtracts the rank-NB product from the panel's remaining columns (all
    // rows above them) and factors the next diagonal block; the panel's last
    // block has no remaining columns, and p_kernel forms its column of T.  Then
    // the panel's whole column of T updates the leading block on matrix cores
    // (K = kPanel): the leading block is read and written once per panel
    // instead of once per NB columns.
    SideStream *ss = nullptr;
    if ((e = side_stream(kSidePrepare, ss)) != hipSuccess) return e;
    std::lock_guard<std::mutex> side_lock(ss->mu);  // every fork, record and wait below, up to the join
    // ev[2]: a panel's column of T is complete; ev[3]: the far part of the last
    // panel update (second side stream) has ended.
    hipEvent_t ev_panel = ss->ev[2], ev_rest = ss->ev[3];
    if ((e = hipEventRecord(ev_rest, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->st2, ev_rest, 0)) != hipSuccess) return e;  // after the damping
    const int64_t npan = ceil_div(d, kPanel);
    for (int64_t q = npan - 1; q >= 0; --q) {
        const int64_t p0 = q * kPanel, p1 = std::min<int64_t>(p0 + kPanel, d);
        const int64_t kb_top = ceil_div(p1, NB) - 1, kb_lo = p0 / NB;
        {
            const int64_t k0 = kb_top * NB;
            hipLaunchKernelGGL(panel_kernel, dim3(1), dim3(kThreads), 0, s, A, Tf, lda, k0, (int)std::min<int64_t>(NB, d - k0),
                               info);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        for (int64_t kb = kb_top; kb >= kb_lo; --kb) {
            const int64_t k0 = kb * NB;
            const int nb = (int)std::min<int64_t>(NB, d - k0);
            if (kb > kb_lo) {
                // one launch: every tile solves its two row blocks of P, the
                // tiles of the last column write them into T, the last diagonal
                // tile factors the next block
                const int nt = (int)kb, tj_lo = (int)kb_lo;
                hipLaunchKernelGGL(step_kernel<false>, dim3((unsigned)step_tiles(tj_lo, nt)), dim3(kFThreads), 0, s, A, Tf,
                                   Tw, lda, k0, nb, nt, tj_lo, info);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            } else if (kb >= 1) {
                // the panel's last block: its column of T for every row above
                hipLaunchKernelGGL(p_kernel, dim3((unsigned)kb), dim3(kFThreads), 0, s, A, Tf, Tw, lda, k0, nb);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
            // T is complete in every column from k0 on: the inverse's work at
            // k0 can start beside the next steps.  (The right products write Tw
            // only in rows >= k0; p_kernel stages P^T in Tw's first NB rows.)
            if (k0 > 0 && k0 % kRegion == 0) {
                if ((e = fork_to(*ss, s)) != hipSuccess) return e;
                if ((e = assemble_at(Tf, U, Tw, d, lda, k0, ss->st, kSideWgs)) != hipSuccess) return e;
            }
        }
        if (p0 > 0) {
            // A[0:p0, 0:p0] -= T[0:p0, p0:p1] T[0:p0, p0:p1]^T (upper part), in two
            // parts: the next panel's columns [n0, p0) on this stream (the next
            // steps need them; the previous panel's far part wrote them too, so
            // it must have ended), and the rest, columns [0, n0), on the
            // second side stream beside the next panel's steps.
            const int64_t n0 = std::max<int64_t>(p0 - kPanel, 0);
            if ((e = hipEventRecord(ev_panel, s)) != hipSuccess) return e;
            if ((e = hipStreamWaitEvent(s, ev_rest, 0)) != hipSuccess) return e;
            GemmDesc g;
            g.M = p0;
            g.N = p0 - n0;
            g.K = p1 - p0;
            g.A = Tf + p0;
            g.lda = lda;
            g.B = Tf + n0 * lda + p0;
            g.ldb = lda;
            g.b_trans = 1;
            g.C = A + n0;
            g.ldc = lda;
            g.alpha = -1.0f;
            g.beta = 1.0f;  // the strictly lower part of A is never read
            if ((e = launch_wide_product(g, s)) != hipSuccess) return e;
            if (n0 > 0) {
                if ((e = hipStreamWaitEvent(ss->st2, ev_panel, 0)) != hipSuccess) return e;
                GemmDesc r;
                r.M = n0;
                r.N = n0;
                r.K = p1 - p0;
                r.A = Tf + p0;
                r.lda = lda;
                r.B = Tf + p0;
                r.ldb = lda;
                r.b_trans = 1;
                r.C = A;
                r.ldc = lda;
                r.alpha = -1.0f;
                r.beta = 1.0f;
                r.upper_only = 1;
                r.max_wgs = kSideWgs;
                if ((e = launch_wide_product(r, ss->st2)) != hipSuccess) return e;
                if ((e = hipEventRecord(ev_rest, ss->st2)) != hipSuccess) return e;
            }
        }
    }
    // The rest of U = T^-1 once T is complete, then the caller's stream waits
    // for all of it.
    if ((e = fork_to(*ss, s)) != hipSuccess) return e;
    if ((e = assemble_at(Tf, U, Tw, d, lda, 0, ss->st, 0)) != hipSuccess) return e;
    if ((e = signal_wait(ss->ev[1], ss->st, s)) != hipSuccess) return e;
    return hipStreamWaitEvent(s, ev_rest, 0);
}

}  // namespace gptq
