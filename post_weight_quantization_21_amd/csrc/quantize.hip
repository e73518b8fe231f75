// Step 4 of GPTQ: the greedy column pass with error feedback, in lazy batches
// (page "PTQ 权重量化：从 GPTQ 到 AWQ", GPTQ section: update formula and
// batched updates every 128 columns; page "量化经典：LLM.int8 / GPTQ / AWQ",
// §二 "方法核心" steps 3-4), and the round-to-nearest baseline.
//
// Per batch of B columns [c0, c0+B):
//   block kernel   one lane per output row: the row's B weights live in
//                  registers, the B x B block of U in LDS (read as wave-wide
//                  broadcasts).  Column by column: fit the group grid at a
//                  group start (from the current weights), quantize,
//                  e = (w - w_hat) / U[j][j], push -e U[j][k] onto the later
//                  columns of the batch, store -e into E^T.
//   trailing GEMM  W[:, c0+B:] += (-E) U[c0:c0+B, c0+B:]  on fp32 matrix cores.
// Rows are independent, so no lane ever talks to another.
#include "common.h"
#include "quant_grid.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;

// Column indices read from a permutation are clamped into [0, n) so that a
// malformed permutation can only give wrong results, never a wild access.
__device__ __forceinline__ int32_t clamp_col(int32_t c, int64_t n) {
    return c < 0 ? 0 : (c >= n ? (int32_t)(n - 1) : c);
}

struct BlockArgs {
    float *W;
    int64_t ldw, d_out, c0;
    int ncols;
    const float *U;
    int64_t ldu;
    float *Et;  // [B][d_out], holds -e
    uint8_t *codes;
    int64_t ldc;
    const int32_t *perm;
    float *scales, *zeros;
    int64_t ng, g;
    int bits, sym, vec;
};

template <int BT, int GT>
__global__ __launch_bounds__(kThreads) void gptq_block_kernel(BlockArgs a) {
    __shared__ float us[BT][BT];
    __shared__ float inv_d[BT];
    __shared__ int32_t pcol[BT];
    const int tid = threadIdx.x;
    const int nc = a.ncols;
    for (int e = tid; e < BT * BT; e += kThreads) {
        const int i = e / BT, k = e % BT;
        us[i][k] = (i < nc && k < nc && i <= k) ? a.U[(a.c0 + i) * a.ldu + a.c0 + k] : 0.0f;
    }
    if (tid < BT) {
        const int64_t k = a.c0 + (tid < nc ? tid : 0);
        pcol[tid] = a.perm ? clamp_col(a.perm[k], a.ldc) : (int32_t)(a.c0 + tid);
    }
    __syncthreads();
    if (tid < BT) inv_d[tid] = tid < nc ? 1.0f / us[tid][tid] : 0.0f;
    __syncthreads();

    const int64_t r = (int64_t)blockIdx.x * kThreads + tid;
    const bool active = r < a.d_out;
    float w[BT];
    float *wrow = a.W + r * a.ldw + a.c0;
#pragma unroll
    for (int j = 0; j < BT; j += 4) {
        if (active && a.vec && j + 4 <= nc) {
            const float4 v = *reinterpret_cast<const float4 *>(wrow + j);
            w[j] = v.x;
            w[j + 1] = v.y;
            w[j + 2] = v.z;
            w[j + 3] = v.w;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) w[j + t] = (active && j + t < nc) ? wrow[j + t] : 0.0f;
        }
    }

    float s = 1.0f, z = 0.0f;
    if constexpr (GT == 0) {
        if (active) {
            const int64_t gi = a.c0 / a.g;
            s = a.scales[r * a.ng + gi];
            z = a.zeros[r * a.ng + gi];
        }
    }
    uint32_t cw[BT / 4];
#pragma unroll
    for (int j = 0; j < BT / 4; ++j) cw[j] = 0u;

#pragma unroll
    for (int j = 0; j < BT; ++j) {
        if (j < nc) {
            if constexpr (GT > 0) {
                if (j % GT == 0) {
                    if (a.sym) {
                        float amax = 0.0f;
#pragma unroll
                        for (int k = j; k < j + GT; ++k) amax = fmaxf(amax, fabsf(w[k]));
                        grid_sym(amax, a.bits, s, z);
                    } else {
                        float lo = 0.0f, hi = 0.0f;
#pragma unroll
                        for (int k = j; k < j + GT; ++k) {
                            lo = fminf(lo, w[k]);
                            hi = fmaxf(hi, w[k]);
                        }
                        grid_asym(lo, hi, a.bits, s, z);
                    }
                    if (active) {
                        const int64_t gi = (a.c0 + j) / a.g;
                        a.scales[r * a.ng + gi] = s;
                        a.zeros[r * a.ng + gi] = z;
                    }
                }
            }
            const float code = grid_code(w[j], s, z, a.bits, a.sym);
            const float wh = grid_dequant(code, s, z);
            const float e = (w[j] - wh) * inv_d[j];
            cw[j >> 2] |= ((uint32_t)code) << (8 * (j & 3));
            if (active) a.Et[(int64_t)j * a.d_out + r] = -e;
#pragma unroll
            for (int k = j + 1; k < BT; ++k) w[k] = fmaf(-e, us[j][k], w[k]);
        }
    }

    if (!active) return;
    // w[j] is never touched after column j is quantized: it is the value at quantization time.
#pragma unroll
    for (int j = 0; j < BT; j += 4) {
        if (a.vec && j + 4 <= nc) {
            *reinterpret_cast<float4 *>(wrow + j) = make_float4(w[j], w[j + 1], w[j + 2], w[j + 3]);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (j + t < nc) wrow[j + t] = w[j + t];
        }
    }
    uint8_t *crow = a.codes + r * a.ldc;
    if (!a.perm && a.vec && (a.ldc % 16 == 0) && (a.c0 % 16 == 0)) {
#pragma unroll
        for (int j = 0; j < BT; j += 16) {
            if (j + 16 <= nc) {
                *reinterpret_cast<uint4 *>(crow + a.c0 + j) = make_uint4(cw[j / 4], cw[j / 4 + 1], cw[j / 4 + 2], cw[j / 4 + 3]);
            } else {
                for (int t = j; t < nc && t < j + 16; ++t) crow[a.c0 + t] = (uint8_t)(cw[t >> 2] >> (8 * (t & 3)));
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < BT; ++j)
            if (j < nc) crow[pcol[j]] = (uint8_t)(cw[j >> 2] >> (8 * (j & 3)));
    }
}

// One wave per (row, group): fit the group's grid from W (current values);
// optionally write the codes (round-to-nearest).  Groups g_first .. g_first+g_count-1.
__global__ __launch_bounds__(kThreads) void rtn_kernel(const float *__restrict__ W, int64_t ldw, int64_t d_out,
                                                       int64_t g, int64_t ng, int64_t g_first, int64_t g_count,
                                                       int bits, int sym, uint8_t *__restrict__ codes, int64_t ldc,
                                                       float *__restrict__ scales, float *__restrict__ zeros) {
    const int64_t wid = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kWave;
    const int lane = threadIdx.x % kWave;
    if (wid >= d_out * g_count) return;
    const int64_t r = wid / g_count, gi = g_first + wid % g_count;
    const float *src = W + r * ldw + gi * g;
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
    float s, z;
    if (sym)
        grid_sym(amax, bits, s, z);
    else
        grid_asym(lo, hi, bits, s, z);
    if (lane == 0) {
        scales[r * ng + gi] = s;
        zeros[r * ng + gi] = z;
    }
    if (codes) {
        uint8_t *dst = codes + r * ldc + gi * g;
        for (int64_t k = lane; k < g; k += kWave) dst[k] = (uint8_t)grid_code(src[k], s, z, bits, sym);
    }
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
    const int64_t r = blockIdx.y;
    for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < d_in; k += (int64_t)gridDim.x * kThreads)
        W[r * d_in + k] = src[r * d_in + clamp_col(perm[k], d_in)];
}

__global__ __launch_bounds__(kThreads) void gidx_kernel(const int32_t *__restrict__ perm, int64_t d_in, int64_t g,
                                                        int32_t *__restrict__ g_idx) {
    const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (k < d_in) g_idx[perm ? clamp_col(perm[k], d_in) : k] = (int32_t)(k / g);
}

int group_tile(const gptq_config &c, int64_t d_in) {
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    return (g <= c.block_size && c.block_size % g == 0) ? (int)g : 0;
}

template <int BT>
hipError_t launch_block(const BlockArgs &a, int gt, unsigned grid, hipStream_t s) {
    switch (gt) {
    case 0:
        hipLaunchKernelGGL((gptq_block_kernel<BT, 0>), dim3(grid), dim3(kThreads), 0, s, a);
        break;
    case 32:
        if constexpr (BT >= 32) hipLaunchKernelGGL((gptq_block_kernel<BT, 32>), dim3(grid), dim3(kThreads), 0, s, a);
        break;
    case 64:
        if constexpr (BT >= 64) hipLaunchKernelGGL((gptq_block_kernel<BT, 64>), dim3(grid), dim3(kThreads), 0, s, a);
        break;
    case 128:
        if constexpr (BT >= 128) hipLaunchKernelGGL((gptq_block_kernel<BT, 128>), dim3(grid), dim3(kThreads), 0, s, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int quantize_supported(const gptq_config &c, int64_t d_in) {
    if (c.block_size != 32 && c.block_size != 64 && c.block_size != 128) return 0;
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    if (g <= c.block_size) return c.block_size % g == 0 && (g == 32 || g == 64 || g == 128);
    return g % c.block_size == 0;
}

size_t quantize_ws_bytes(int64_t d_out, int64_t d_in, const gptq_config &c) {
    size_t b = align_up((size_t)c.block_size * (size_t)d_out * sizeof(float), 256);
    if (c.act_order) b += align_up((size_t)d_out * (size_t)d_in * sizeof(float), 256);
    return b;
}

hipError_t run_quantize(float *W, int64_t d_out, int64_t d_in, const float *U, const int32_t *perm,
                        const gptq_config &c, uint8_t *codes, float *scales, float *zeros, int32_t *g_idx,
                        void *ws, hipStream_t s) {
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    const int64_t ng = d_in / g;
    const int B = c.block_size;
    const int gt = group_tile(c, d_in);
    float *Et = static_cast<float *>(ws);
    hipError_t e;
    const int32_t *pp = c.act_order ? perm : nullptr;
    if (pp) {
        float *Wc = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                              align_up((size_t)B * (size_t)d_out * sizeof(float), 256));
        const int64_t n = d_out * d_in, n4 = n / 4;
        hipLaunchKernelGGL(copy_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(n4, kThreads), 65536)), dim3(kThreads), 0,
                           s, reinterpret_cast<const float4 *>(W), reinterpret_cast<float4 *>(Wc), n4);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (n4 * 4 < n) {
            hipLaunchKernelGGL(copy_tail_kernel, dim3(1), dim3(kThreads), 0, s, W, Wc, n4 * 4, n);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const unsigned gx = (unsigned)std::min<int64_t>(ceil_div(d_in, kThreads), 64);
        hipLaunchKernelGGL(permute_cols_kernel, dim3(gx, (unsigned)d_out), dim3(kThreads), 0, s, Wc, pp, d_out, d_in, W);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (g_idx) {
        hipLaunchKernelGGL(gidx_kernel, dim3((unsigned)ceil_div(d_in, kThreads)), dim3(kThreads), 0, s, pp, d_in, g, g_idx);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const unsigned grid = (unsigned)ceil_div(d_out, kThreads);
    const int vec = (d_in % 4 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0) && ((reinterpret_cast<uintptr_t>(codes) & 15) == 0);
    for (int64_t c0 = 0; c0 < d_in; c0 += B) {
        const int nc = (int)std::min<int64_t>(B, d_in - c0);
        if (gt == 0 && c0 % g == 0) {
            const int64_t waves = d_out;
            hipLaunchKernelGGL(rtn_kernel, dim3((unsigned)ceil_div(waves * kWave, kThreads)), dim3(kThreads), 0, s, W, d_in,
                               d_out, g, ng, c0 / g, (int64_t)1, c.bits, c.symmetric, (uint8_t *)nullptr, d_in, scales,
                               zeros);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        BlockArgs a;
        a.W = W;
        a.ldw = d_in;
        a.d_out = d_out;
        a.c0 = c0;
        a.ncols = nc;
        a.U = U;
        a.ldu = d_in;
        a.Et = Et;
        a.codes = codes;
        a.ldc = d_in;
        a.perm = pp;
        a.scales = scales;
        a.zeros = zeros;
        a.ng = ng;
        a.g = g;
        a.bits = c.bits;
        a.sym = c.symmetric ? 1 : 0;
        a.vec = vec;
        if (B == 32)
            e = launch_block<32>(a, gt, grid, s);
        else if (B == 64)
            e = launch_block<64>(a, gt, grid, s);
        else
            e = launch_block<128>(a, gt, grid, s);
        if (e != hipSuccess) return e;
        const int64_t c1 = c0 + nc;
        if (c1 < d_in) {
            GemmDesc t;
            t.M = d_out;
            t.N = d_in - c1;
            t.K = nc;
            t.A = Et;
            t.lda = d_out;
            t.a_trans = 1;
            t.B = U + c0 * d_in + c1;
            t.ldb = d_in;
            t.C = W + c1;
            t.ldc = d_in;
            t.alpha = 1.0f;
            t.beta = 1.0f;
            if ((e = launch_gemm_f32(t, s)) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t run_rtn(const float *W, int64_t d_out, int64_t d_in, const gptq_config &c, uint8_t *codes, float *scales,
                   float *zeros, hipStream_t s) {
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    const int64_t ng = d_in / g;
    const int64_t waves = d_out * ng;
    hipLaunchKernelGGL(rtn_kernel, dim3((unsigned)ceil_div(waves * kWave, kThreads)), dim3(kThreads), 0, s, W, d_in, d_out, g,
                       ng, (int64_t)0, ng, c.bits, c.symmetric, codes, d_in, scales, zeros);
    return hipGetLastError();
}

}  // namespace gptq
