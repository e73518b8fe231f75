// Step 4 of GPTQ: the greedy column pass with error feedback, in lazy batches
// (page "PTQ 权重量化：从 GPTQ 到 AWQ", GPTQ section: update formula and
// batched updates every 128 columns; page "量化经典：LLM.int8 / GPTQ / AWQ",
// §二 "方法核心" steps 3-4), and the round-to-nearest baseline.
//
// Per batch of B columns [c0, c0+B):
//   block kernel   four lanes per output row: the row's B weights live in
//                  registers, the B x B block of U in LDS.  Column by column:
//                  fit the group grid at a group start (from the current
//                  weights), quantize, e = (w - w_hat) / U[j][j], push
//                  -e U[j][k] onto the later columns of the batch, store -e
//                  into E^T.
//   batch update   W[:, c0+B:s1] += (-E) U[c0:c0+B, c0+B:s1]  (fp32 matrix cores)
// The lazy update runs on two levels: the batches of one superblock of
// kSuperCols columns [s0, s1) update only the rest of that superblock, and
// when the superblock is done its stacked E updates every later column at
// once, W[:, s1:] += (-E_s) U[s0:s1, s1:].  Every column still receives the
// error of every earlier column before it is quantized (the same sums, in a
// different fp32 order), while the trailing W is read and written once per
// superblock instead of once per batch.
#include "block_args.h"
#include "quant_grid.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;

// One wave per (row, group): fit the group's grid from W (current values),
// or (fit == 0) take the grid stored in scales/zeros; optionally write the
// codes (round-to-nearest).  Groups g_first .. g_first+g_count-1.
__global__ __launch_bounds__(kThreads) void rtn_kernel(const float *__restrict__ W, int64_t ldw, int64_t d_out,
                                                       int64_t g, int64_t ng, int64_t g_first, int64_t g_count,
                                                       int bits, int sym, int fit, uint8_t *__restrict__ codes,
                                                       int64_t ldc, float *__restrict__ scales, float *__restrict__ zeros) {
    const int64_t wid = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    if (wid >= d_out * g_count) return;
    const int64_t r = wid / g_count, gi = g_first + wid % g_count;
    const float *src = W + r * ldw + gi * g;
    Grid gr;
    if (fit) {
        float lo = 0.0f, hi = 0.0f, amax = 0.0f;
        for (int64_t k = lane; k < g; k += kWave) {
            const float v = src[k];
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
            amax = fmaxf(amax, fabsf(v));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, off));
            hi = fmaxf(hi, __shfl_xor(hi, off));
            amax = fmaxf(amax, __shfl_xor(amax, off));
        }
        gr = grid_make(amax, lo, hi, bits, sym);
        if (lane == 0) {
            scales[r * ng + gi] = gr.s;
            zeros[r * ng + gi] = gr.zero;
        }
    } else {
        gr = grid_from_stored(scales[r * ng + gi], zeros[r * ng + gi], bits, sym);
    }
    if (codes) {
        uint8_t *dst = codes + r * ldc + gi * g;
        for (int64_t k = lane; k < g; k += kWave) dst[k] = (uint8_t)grid_code(src[k], gr);
    }
}

// Static groups: every group's grid from the original W, before the pass.  One
// wave per row.  For g dividing 256 the row is read in coalesced 16-byte pieces
// (g / 4 lanes per group, reduced by shuffles); otherwise one group at a time
// over the whole wave.  Writes scales and zeros ([d_out][ng], original group
// order) and, when tab is given, the packed grids for lookups per column.
__global__ __launch_bounds__(kThreads) void fit_static_kernel(const float *__restrict__ W, int64_t d_out, int64_t d_in,
                                                              int64_t g, int64_t ng, int bits, int sym,
                                                              float *__restrict__ scales, float *__restrict__ zeros,
                                                              float4 *__restrict__ tab) {
    const int64_t r = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kWave;  // uniform per wave
    const int lane = threadIdx.x % kWave;
    if (r >= d_out) return;
    const float *row = W + r * d_in;
    auto put = [&](int64_t gi, float amax, float lo, float hi) {
        const Grid gr = grid_make(amax, lo, hi, bits, sym);
        scales[r * ng + gi] = gr.s;
        zeros[r * ng + gi] = gr.zero;
        if (tab) tab[r * ng + gi] = grid_pack(gr);
    };
    if (g % 4 == 0 && (4 * kWave) % g == 0) {  // rows are 16-byte aligned (W is, and 4 | g | d_in)
        const int lpg = (int)(g / 4);  // lanes per group
        for (int64_t k0 = 0; k0 < d_in; k0 += 4 * kWave) {
            const int64_t k = k0 + 4 * lane;
            const float4 v = k < d_in ? *reinterpret_cast<const float4 *>(row + k) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            float hi = fmaxf(fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)), 0.0f);
            float lo = fminf(fminf(fminf(v.x, v.y), fminf(v.z, v.w)), 0.0f);
            float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
            for (int off = 1; off < lpg; off <<= 1) {
                hi = fmaxf(hi, __shfl_xor(hi, off));
                lo = fminf(lo, __shfl_xor(lo, off));
                amax = fmaxf(amax, __shfl_xor(amax, off));
            }
            if (lane % lpg == 0 && k < d_in) put(k / g, amax, lo, hi);
        }
    } else {
        for (int64_t gi = 0; gi < ng; ++gi) {
            const float *src = row + gi * g;
            float lo = 0.0f, hi = 0.0f, amax = 0.0f;
            for (int64_t k = lane; k < g; k += kWave) {
                const float v = src[k];
                lo = fminf(lo, v);
                hi = fmaxf(hi, v);
                amax = fmaxf(amax, fabsf(v));
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                lo = fminf(lo, __shfl_xor(lo, off));
                hi = fmaxf(hi, __shfl_xor(hi, off));
                amax = fmaxf(amax, __shfl_xor(amax, off));
            }
            if (lane == 0) put(gi, amax, lo, hi);
        }
    }
}

// The one grid of a whole matrix (page "LLM 量化方法原理与实现详解", §2.3:
// one scale per tensor), in two kernels that need no scratch: the outputs
// scales and zeros ([d_out][1]) first hold partial ranges.  Block b reduces its
// grid-stride share of W to hi = max(max x, 0) and nlo = max(-min x, 0)
// (exact, so the order does not matter) into scales[b] and zeros[b].
__global__ __launch_bounds__(kThreads) void tensor_range_kernel(const float *__restrict__ W, int64_t n, int vec,
                                                                float *__restrict__ hi_out, float *__restrict__ nlo_out) {
    __shared__ float red[2][kThreads / kWave];
    float hi = 0.0f, nlo = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i0 = 0;
    if (vec) {
        const int64_t n4 = n / 4;
        for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
            const float4 v = reinterpret_cast<const float4 *>(W)[i];
            hi = fmaxf(hi, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
            nlo = fmaxf(nlo, fmaxf(fmaxf(-v.x, -v.y), fmaxf(-v.z, -v.w)));
        }
        i0 = n4 * 4;
    }
    for (int64_t i = i0 + (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        hi = fmaxf(hi, W[i]);
        nlo = fmaxf(nlo, -W[i]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        hi = fmaxf(hi, __shfl_xor(hi, off));
        nlo = fmaxf(nlo, __shfl_xor(nlo, off));
    }
    const int wave = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        red[0][wave] = hi;
        red[1][wave] = nlo;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / kWave; ++w) {
            hi = fmaxf(hi, red[0][w]);
            nlo = fmaxf(nlo, red[1][w]);
        }
        hi_out[blockIdx.x] = hi;
        nlo_out[blockIdx.x] = nlo;
    }
}

// One block: the tensor's grid from the nparts partial ranges, then written
// to every row of scales and zeros (after all partials have been read).
__global__ __launch_bounds__(kThreads) void tensor_grid_kernel(float *__restrict__ scales, float *__restrict__ zeros,
                                                               int64_t d_out, int nparts, int bits, int sym) {
    __shared__ float red[2][kThreads / kWave];
    float hi = 0.0f, nlo = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += kThreads) {
        hi = fmaxf(hi, scales[i]);
        nlo = fmaxf(nlo, zeros[i]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        hi = fmaxf(hi, __shfl_xor(hi, off));
        nlo = fmaxf(nlo, __shfl_xor(nlo, off));
    }
    const int wave = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        red[0][wave] = hi;
        red[1][wave] = nlo;
    }
    __syncthreads();
    hi = red[0][0];
    nlo = red[1][0];
    for (int w = 1; w < kThreads / kWave; ++w) {
        hi = fmaxf(hi, red[0][w]);
        nlo = fmaxf(nlo, red[1][w]);
    }
    // max|x| = max(hi, nlo); lo = min(min x, 0) = -nlo
    const Grid gr = grid_make(fmaxf(hi, nlo), -nlo, hi, bits, sym);
    for (int64_t r = threadIdx.x; r < d_out; r += kThreads) {
        scales[r] = gr.s;
        zeros[r] = gr.zero;
    }
}

hipError_t tensor_grid(const float *W, int64_t d_out, int64_t d_in, const gptq_config &c, float *scales, float *zeros,
                       hipStream_t s) {
    const int nparts = (int)std::min<int64_t>(d_out, 1024);
    const int vec = (reinterpret_cast<uintptr_t>(W) & 15) == 0;
    hipLaunchKernelGGL(tensor_range_kernel, dim3((unsigned)nparts), dim3(kThreads), 0, s, W, d_out * d_in, vec, scales, zeros);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tensor_grid_kernel, dim3(1), dim3(kThreads), 0, s, scales, zeros, d_out, nparts, c.bits,
                       c.symmetric ? 1 : 0);
    return hipGetLastError();
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const float4 *__restrict__ src, float4 *__restrict__ dst, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads)
        dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void copy_tail_kernel(const float *__restrict__ src, float *__restrict__ dst,
                                                             int64_t from, int64_t n) {
    const int64_t i = from + (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// W[r][k] = Wsrc[r][perm[k]]
__global__ __launch_bounds__(kThreads) void permute_cols_kernel(const float *__restrict__ src, const int32_t *__restrict__ perm,
                                                                int64_t d_out, int64_t d_in, float *__restrict__ W) {
    for (int64_t r = blockIdx.y; r < d_out; r += gridDim.y)  // rows grid-stride (grid y is capped)
        for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < d_in; k += (int64_t)gridDim.x * kThreads)
            W[r * d_in + k] = src[r * d_in + clamp_col(perm[k], d_in)];
}

// W[r][k] = W[r][perm[k]] in place, one row at a time through LDS (d_in floats,
// d_in a multiple of 4, W 16-byte aligned).  Rows are read once and written
// once, coalesced; the gather reads LDS.
constexpr int64_t kRowPermMax = 16384;  // d_in limit of the in-place path (64 KB of LDS)
__global__ __launch_bounds__(kThreads) void permute_rows_inplace_kernel(float *__restrict__ W,
                                                                        const int32_t *__restrict__ perm, int64_t d_out,
                                                                        int64_t d_in) {
    extern __shared__ float row[];
    const int tid = threadIdx.x;
    for (int64_t r = blockIdx.x; r < d_out; r += gridDim.x) {
        float *w = W + r * d_in;
        for (int64_t k = 4 * tid; k < d_in; k += 4 * kThreads)
            *reinterpret_cast<float4 *>(&row[k]) = *reinterpret_cast<const float4 *>(w + k);
        __syncthreads();
        for (int64_t k = 4 * tid; k < d_in; k += 4 * kThreads) {
            float4 v;
            v.x = row[clamp_col(perm[k + 0], d_in)];
            v.y = row[clamp_col(perm[k + 1], d_in)];
            v.z = row[clamp_col(perm[k + 2], d_in)];
            v.w = row[clamp_col(perm[k + 3], d_in)];
            *reinterpret_cast<float4 *>(w + k) = v;
        }
        __syncthreads();  // row[] is reused by the next row
    }
}

// inv[perm[k]] = k.
__global__ __launch_bounds__(kThreads) void invert_perm_kernel(const int32_t *__restrict__ perm, int64_t d_in,
                                                               int32_t *__restrict__ inv) {
    const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (k < d_in) inv[clamp_col(perm[k], d_in)] = (int32_t)k;
}

// codes[r][c] = cp[r][inv[c]]: codes written in processing order (coalesced
// during the pass) go back to the original column order, one row at a time
// through LDS (d_in a multiple of 4); reads and writes of HBM are coalesced.
constexpr int64_t kCodePermMax = 65536;  // d_in limit (64 KB of LDS)
__global__ __launch_bounds__(kThreads) void unpermute_codes_kernel(const uint8_t *__restrict__ cp,
                                                                   const int32_t *__restrict__ inv, int64_t d_out,
                                                                   int64_t d_in, uint8_t *__restrict__ codes) {
    extern __shared__ uint32_t rowc[];
    const uint8_t *rb = reinterpret_cast<const uint8_t *>(rowc);
    const int tid = threadIdx.x;
    for (int64_t r = blockIdx.x; r < d_out; r += gridDim.x) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(cp + r * d_in);
        for (int64_t k = tid; k < d_in / 4; k += kThreads) rowc[k] = src[k];
        __syncthreads();
        uint32_t *dst = reinterpret_cast<uint32_t *>(codes + r * d_in);
        for (int64_t k = tid; k < d_in / 4; k += kThreads) {
            const int64_t c = 4 * k;
            dst[k] = (uint32_t)rb[clamp_col(inv[c + 0], d_in)] | ((uint32_t)rb[clamp_col(inv[c + 1], d_in)] << 8) |
                     ((uint32_t)rb[clamp_col(inv[c + 2], d_in)] << 16) | ((uint32_t)rb[clamp_col(inv[c + 3], d_in)] << 24);
        }
        __syncthreads();  // rowc is reused by the next row
    }
}

// The same for rows of at most kCodeRegMax codes: thread t owns the 4-byte
// words t + 256 i of every row, their columns' source positions are read once
// per workgroup and kept in registers (two 16-bit positions per word), and all
// of a row's loads are issued before the first wait.
constexpr int kCodeIters = 16;
constexpr int64_t kCodeRegMax = 4 * (int64_t)kThreads * kCodeIters;  // 16384 codes per row
__global__ __launch_bounds__(kThreads) void unpermute_codes_reg_kernel(const uint8_t *__restrict__ cp,
                                                                       const int32_t *__restrict__ inv, int64_t d_out,
                                                                       int64_t d_in, uint8_t *__restrict__ codes) {
    extern __shared__ uint32_t rowc[];
    const uint8_t *rb = reinterpret_cast<const uint8_t *>(rowc);
    const int tid = threadIdx.x;
    const int64_t nw = d_in / 4;
    uint32_t ip[kCodeIters][2];
#pragma unroll
    for (int i = 0; i < kCodeIters; ++i) {
        const int64_t k = tid + (int64_t)kThreads * i;
        if (k < nw) {
            const int64_t c = 4 * k;
            ip[i][0] = (uint32_t)clamp_col(inv[c + 0], d_in) | ((uint32_t)clamp_col(inv[c + 1], d_in) << 16);
            ip[i][1] = (uint32_t)clamp_col(inv[c + 2], d_in) | ((uint32_t)clamp_col(inv[c + 3], d_in) << 16);
        } else {
            ip[i][0] = ip[i][1] = 0u;
        }
    }
    for (int64_t r = blockIdx.x; r < d_out; r += gridDim.x) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(cp + r * d_in);
        uint32_t v[kCodeIters];
#pragma unroll
        for (int i = 0; i < kCodeIters; ++i) {
            const int64_t k = tid + (int64_t)kThreads * i;
            if (k < nw) v[i] = src[k];
        }
#pragma unroll
        for (int i = 0; i < kCodeIters; ++i) {
            const int64_t k = tid + (int64_t)kThreads * i;
            if (k < nw) rowc[k] = v[i];
        }
        __syncthreads();
        uint32_t *dst = reinterpret_cast<uint32_t *>(codes + r * d_in);
#pragma unroll
        for (int i = 0; i < kCodeIters; ++i) {
            const int64_t k = tid + (int64_t)kThreads * i;
            if (k < nw)
                dst[k] = (uint32_t)rb[ip[i][0] & 0xffffu] | ((uint32_t)rb[ip[i][0] >> 16] << 8) |
                         ((uint32_t)rb[ip[i][1] & 0xffffu] << 16) | ((uint32_t)rb[ip[i][1] >> 16] << 24);
        }
        __syncthreads();  // rowc is reused by the next row
    }
}

// Whether the act-order permutation of W runs in place (else: copy, then gather).
bool row_perm_inplace(const float *W, int64_t d_in) {
    return d_in <= kRowPermMax && d_in % 4 == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0;
}

__global__ __launch_bounds__(kThreads) void gidx_kernel(const int32_t *__restrict__ perm, int64_t d_in, int64_t g,
                                                        int32_t *__restrict__ g_idx) {
    const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (k < d_in) g_idx[perm ? clamp_col(perm[k], d_in) : k] = (int32_t)(k / g);
}

// Columns per batch kernel launch for a lazy batch width B.  Every B gives
// the same sums (in another fp32 order): the batches only decide when the
// accumulated errors reach the later columns.  B = 1 (the unblocked update)
// runs as batches of 128; a multiple of 32 as batches of the largest of 128,
// 96, 64, 32 that divides it (B > 128: blocks of B made of such batches).
int64_t batch_cols(const gptq_config &c) {
    const int64_t B = c.block_size;
    if (B == 1) return 128;
    for (int64_t w : {128, 96, 64, 32})
        if (B % w == 0) return w;
    return 0;
}

// The batch kernel's compiled width for batches of bw columns (a batch may be
// partial: the columns past it are masked).
int batch_template(int64_t bw) { return bw <= 32 ? 32 : bw <= 64 ? 64 : 128; }

int group_tile(const gptq_config &c, int64_t d_in) {
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    const int64_t bw = batch_cols(c);
    return (g <= bw && bw % g == 0) ? (int)g : 0;
}

// E^T rows are padded to whole workgroups so the batch kernel stores without a row test.
int64_t et_ld(int64_t d_out) { return ceil_div(d_out, kBlockThreads) * kBlockThreads; }

constexpr int64_t kSuperCols = 1024;  // default columns per superblock of the two-level lazy update

// Superblock width: a multiple of the batch and, when a grid fitted during
// the pass spans several batches, of its group (the grid is fitted from
// columns that must all be up to date).  Grids fitted before the pass, and the
// one grid of a row (fitted at column 0, before any update), set no such
// bound.  At least d_in means one superblock: no deferred update.
int64_t super_cols(const gptq_config &c, int64_t d_in, int gt) {
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    const bool refit = c.grid == GPTQ_GRID_DYNAMIC && gt == 0 && g < d_in;  // g is a multiple of B here
    const int64_t bw = batch_cols(c);
    const int64_t blk = c.block_size > bw ? c.block_size : bw;  // a lazy block of B > 128 columns
    const int64_t unit = refit ? g : blk;
    const int64_t want = c.super_cols > 0 ? c.super_cols : kSuperCols;
    const int64_t sc = unit >= want ? unit : (want / unit) * unit;
    return sc;
}

// Workspace of the column pass: E^T of a whole superblock [S][ldet] (one batch
// when there is a single superblock); with act-order, a copy of W for the
// column gather (rows too long for the in-place permutation only), the codes
// in processing order with the inverse permutation, and, for static groups,
// the packed grids [d_out][ng] of the lookup per column.
struct QuantLayout {
    size_t et_off, wc_off, cp_off, inv_off, tab_off, total;
    int64_t sc;       // superblock width
    int64_t et_rows;  // rows of E^T kept
};

QuantLayout quant_layout(int64_t d_out, int64_t d_in, const gptq_config &c) {
    QuantLayout l;
    l.sc = super_cols(c, d_in, group_tile(c, d_in));
    // the batch kernel writes rows for every column of its compiled width, so the
    // last batch of a stack may write past it by the width minus the batch
    const int64_t bw = batch_cols(c);
    l.et_rows = (l.sc < d_in ? l.sc : bw) + (batch_template(bw) - bw);
    l.et_off = 0;
    l.wc_off = align_up((size_t)l.et_rows * (size_t)et_ld(d_out) * sizeof(float), 256);
    const bool copy = c.act_order && d_in > kRowPermMax;  // aligned W assumed (checked at the boundary)
    l.cp_off = l.wc_off + (copy ? align_up((size_t)d_out * (size_t)d_in * sizeof(float), 256) : 0);
    // act-order: codes in processing order and the inverse permutation
    const bool cperm = c.act_order && d_in <= kCodePermMax;
    l.inv_off = l.cp_off + (cperm ? align_up((size_t)d_out * (size_t)d_in, 256) : 0);
    l.tab_off = l.inv_off + (cperm ? align_up((size_t)d_in * sizeof(int32_t), 256) : 0);
    // static groups under act-order: packed grids for the lookup per column
    const bool tab = c.act_order && c.grid == GPTQ_GRID_STATIC;
    const int64_t ng = d_in / (c.group_size > 0 ? c.group_size : d_in);
    l.total = l.tab_off + (tab ? align_up((size_t)d_out * (size_t)ng * 16, 256) : 0);
    return l;
}

// K from which a trailing update runs through the split-bf16 GEMM.
constexpr int64_t kSplitMinK = 512;

// Rows from which the superblock's inner updates are left-looking.
constexpr int64_t kLeftLookRows = 16384;

// Left-looking: once the superblock's batches not yet applied to the rest of
// it reach this many columns, one product applies them to all of it (K = 512
// on the split GEMM) instead of growing every later batch's product.
constexpr int64_t kCatchUpCols = 512;

// W[:, c1:c1+n] += (-E) U[k0:k0+k, c1:c1+n] with -E^T stored as Et [k][ldet].
hipError_t lazy_update(float *W, int64_t d_out, int64_t d_in, const float *Et, int64_t ldet, const float *U, int64_t k0,
                       int64_t k, int64_t c1, int64_t n, hipStream_t s) {
    if (n <= 0 || k <= 0) return hipSuccess;
    GemmDesc g;
    g.M = d_out;
    g.N = n;
    g.K = k;
    g.A = Et;  // A[m][kk] = Et[kk][m]
    g.lda = ldet;
    g.a_trans = 1;
    g.B = U + k0 * d_in + c1;
    g.ldb = d_in;
    g.C = W + c1;
    g.ldc = d_in;
    g.alpha = 1.0f;
    g.beta = 1.0f;
    // Long, wide updates (the superblocks') on the bf16 matrix cores through
    // the exact three-term split, whose 256 x 256 tiles need N >= 512 and
    // enough of them to fill the chip; the in-superblock ones on fp32 ones.
    const int64_t split_tiles = ceil_div(d_out, 256) * ceil_div(n, 256);
    const bool split = k >= kSplitMinK && n >= 512 && split_tiles >= 64 && gemm_split_supported(g);
    TimedScope ts(split ? kTimedLazySplit : kTimedLazy, s, 2.0 * (double)d_out * (double)n * (double)k);
    return split ? launch_gemm_split(g, s) : launch_gemm_f32(g, s);
}

}  // namespace

int quantize_supported(const gptq_config &c, int64_t d_in) {
    const int64_t bw = batch_cols(c);
    if (bw == 0 || c.block_size > (1 << 20)) return 0;
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    if (g <= bw) return bw % g == 0 && (g == 32 || g == 64 || g == 128);
    // one group per row: fitted once, at column 0, for any row length
    return g % bw == 0 || g == d_in;
}

size_t quantize_ws_bytes(int64_t d_out, int64_t d_in, const gptq_config &c) { return quant_layout(d_out, d_in, c).total; }

hipError_t run_quantize(float *W, int64_t d_out, int64_t d_in, const float *U, const int32_t *perm,
                        const gptq_config &c, uint8_t *codes, float *scales, float *zeros, int32_t *g_idx,
                        void *ws, hipStream_t s) {
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    const int64_t ng = d_in / g;
    const int64_t B = batch_cols(c);  // columns per batch kernel launch
    const int BT = batch_template(B);
    const int gt = group_tile(c, d_in);
    const QuantLayout lay = quant_layout(d_out, d_in, c);
    char *wsb = static_cast<char *>(ws);
    float *Et = reinterpret_cast<float *>(wsb + lay.et_off);
    hipError_t e;
    const int32_t *pp = c.act_order ? perm : nullptr;
    if (pp && d_in <= kRowPermMax && !row_perm_inplace(W, d_in)) return hipErrorInvalidValue;  // no copy space
    // Grids fitted on the original W, before any column moves.
    const bool fixed = c.grid != GPTQ_GRID_DYNAMIC;
    float4 *gtab = (pp && c.grid == GPTQ_GRID_STATIC) ? reinterpret_cast<float4 *>(wsb + lay.tab_off) : nullptr;
    if (c.grid == GPTQ_GRID_STATIC) {
        hipLaunchKernelGGL(fit_static_kernel, dim3((unsigned)ceil_div(d_out * kWave, kThreads)), dim3(kThreads), 0, s, W,
                           d_out, d_in, g, ng, c.bits, c.symmetric, scales, zeros, gtab);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (c.grid == GPTQ_GRID_TENSOR) {
        if ((e = tensor_grid(W, d_out, d_in, c, scales, zeros, s)) != hipSuccess) return e;
    }
    // Static groups under a column order: every column looks up its own group's grid.
    const int src = !fixed ? kFitGrids : (pp && c.grid == GPTQ_GRID_STATIC) ? kColumnGrids : kStoredGrids;
    if (pp && row_perm_inplace(W, d_in)) {
        const unsigned grid = (unsigned)std::min<int64_t>(d_out, 2048);
        hipLaunchKernelGGL(permute_rows_inplace_kernel, dim3(grid), dim3(kThreads), (size_t)d_in * sizeof(float), s, W, pp,
                           d_out, d_in);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if (pp) {
        float *Wc = reinterpret_cast<float *>(wsb + lay.wc_off);
        const int64_t n = d_out * d_in, n4 = n / 4;
        hipLaunchKernelGGL(copy_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(n4, kThreads), 65536)), dim3(kThreads), 0,
                           s, reinterpret_cast<const float4 *>(W), reinterpret_cast<float4 *>(Wc), n4);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (n4 * 4 < n) {
            hipLaunchKernelGGL(copy_tail_kernel, dim3(1), dim3(kThreads), 0, s, W, Wc, n4 * 4, n);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const unsigned gx = (unsigned)std::min<int64_t>(ceil_div(d_in, kThreads), 64);
        hipLaunchKernelGGL(permute_cols_kernel, dim3(gx, (unsigned)std::min<int64_t>(d_out, 65535)), dim3(kThreads), 0, s, Wc, pp, d_out, d_in, W);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (g_idx) {
        hipLaunchKernelGGL(gidx_kernel, dim3((unsigned)ceil_div(d_in, kThreads)), dim3(kThreads), 0, s,
                           fixed ? nullptr : pp, d_in, g, g_idx);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // With a column order the pass writes the codes in processing order
    // (coalesced) and one row-wise pass puts them in the original order.
    const bool cperm = pp && d_in <= kCodePermMax;
    uint8_t *cdst = cperm ? reinterpret_cast<uint8_t *>(wsb + lay.cp_off) : codes;
    int32_t *inv = cperm ? reinterpret_cast<int32_t *>(wsb + lay.inv_off) : nullptr;
    if (cperm) {
        hipLaunchKernelGGL(invert_perm_kernel, dim3((unsigned)ceil_div(d_in, kThreads)), dim3(kThreads), 0, s, pp, d_in, inv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t ldet = et_ld(d_out);
    const int vec = (d_in % 4 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0) && ((reinterpret_cast<uintptr_t>(cdst) & 15) == 0);
    const int64_t sc = lay.sc;
    const bool deferred = sc < d_in;  // superblocks leave an update for the columns beyond them
    // Inside a superblock, tall layers bring each batch up to date just before
    // it (one product over the superblock's earlier batches, K = their
    // columns); short ones, whose single batch column of tiles would leave most
    // of the chip idle, update the rest of the superblock after each batch.
    const bool left = deferred && d_out >= kLeftLookRows;
    const bool refit = !fixed && gt == 0;  // a grid fitted at each group start from the group's current weights
    for (int64_t s0 = 0; s0 < d_in; s0 += sc) {
        const int64_t s1 = std::min<int64_t>(s0 + sc, d_in);
        // Left-looking: every column in [c0, s1) already has the errors of the
        // columns before lb; each batch takes those of [lb, c0) just before it.
        int64_t lb = s0;
        for (int64_t c0 = s0; c0 < s1; c0 += B) {
            const int nc = (int)std::min<int64_t>(B, s1 - c0);
            if (left) {
                // Catch up the rest of the superblock: where a grid is about to be
                // fitted from a whole group (every column of the group must hold every
                // earlier column's error), and where [lb, c0) has grown to
                // kCatchUpCols columns.
                if (c0 > lb && ((refit && c0 % g == 0) || c0 - lb >= kCatchUpCols)) {
                    if ((e = lazy_update(W, d_out, d_in, Et + (lb - s0) * ldet, ldet, U, lb, c0 - lb, c0, s1 - c0, s)) !=
                        hipSuccess)
                        return e;
                    lb = c0;
                }
                if ((e = lazy_update(W, d_out, d_in, Et + (lb - s0) * ldet, ldet, U, lb, c0 - lb, c0, nc, s)) != hipSuccess)
                    return e;
            }
            if (refit && c0 % g == 0) {
                const int64_t waves = d_out;
                hipLaunchKernelGGL(rtn_kernel, dim3((unsigned)ceil_div(waves * kWave, kThreads)), dim3(kThreads), 0, s, W,
                                   d_in, d_out, g, ng, c0 / g, (int64_t)1, c.bits, c.symmetric, 1, (uint8_t *)nullptr,
                                   d_in, scales, zeros);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
            float *Eb = Et + (deferred ? (c0 - s0) * ldet : 0);  // this batch's rows of E^T
            BlockArgs a{};
            a.W = W;
            a.ldw = d_in;
            a.d_out = d_out;
            a.c0 = c0;
            a.ncols = nc;
            a.U = U;
            a.ldu = d_in;
            a.Et = Eb;
            a.ldet = ldet;
            a.codes = cdst;
            a.ldc = d_in;
            a.perm = cperm ? nullptr : pp;
            a.gperm = pp;
            a.gtab = gtab;
            a.scales = scales;
            a.zeros = zeros;
            a.ng = ng;
            a.g = g;
            a.bits = c.bits;
            a.sym = c.symmetric ? 1 : 0;
            a.vec = vec;
            const int bgt = src == kColumnGrids ? 0 : gt;
            {
                TimedScope ts(kTimedBatch, s);
                if (BT == 32)
                    e = launch_block_32(a, bgt, src, s);
                else if (BT == 64)
                    e = launch_block_64(a, bgt, src, s);
                else
                    e = launch_block_128(a, bgt, src, s);
            }
            if (e != hipSuccess) return e;
            // the rest of the superblock
            const int64_t c1 = c0 + nc;
            if (!left && (e = lazy_update(W, d_out, d_in, Eb, ldet, U, c0, nc, c1, s1 - c1, s)) != hipSuccess) return e;
        }
        // every column beyond the superblock, with the superblock's whole E
        if (deferred && (e = lazy_update(W, d_out, d_in, Et, ldet, U, s0, s1 - s0, s1, d_in - s1, s)) != hipSuccess)
            return e;
    }
    if (cperm) {
        const unsigned grid = (unsigned)std::min<int64_t>(d_out, 2048);
        if (d_in <= kCodeRegMax)
            hipLaunchKernelGGL(unpermute_codes_reg_kernel, dim3(grid), dim3(kThreads), (size_t)d_in, s, cdst, inv, d_out, d_in,
                               codes);
        else
            hipLaunchKernelGGL(unpermute_codes_kernel, dim3(grid), dim3(kThreads), (size_t)d_in, s, cdst, inv, d_out, d_in, codes);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t run_rtn(const float *W, int64_t d_out, int64_t d_in, const gptq_config &c, uint8_t *codes, float *scales,
                   float *zeros, hipStream_t s) {
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    const int64_t ng = d_in / g;
    const int64_t waves = d_out * ng;
    const int fit = c.grid != GPTQ_GRID_TENSOR;
    if (!fit) {
        const hipError_t e = tensor_grid(W, d_out, d_in, c, scales, zeros, s);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(rtn_kernel, dim3((unsigned)ceil_div(waves * kWave, kThreads)), dim3(kThreads), 0, s, W, d_in, d_out, g,
                       ng, (int64_t)0, ng, c.bits, c.symmetric, fit, codes, d_in, scales, zeros);
    return hipGetLastError();
}

}  // namespace gptq
