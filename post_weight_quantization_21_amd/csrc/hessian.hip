// Step 1 of GPTQ: H += 2 X X^T from calibration activations (page "LLM 量化方法
// 原理与实现详解", §4.1: the layer objective's Hessian is 2 X X^T).
//
// bf16 activations: a symmetric rank-k update on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate), 256 x 256 tiles per 4-wave
// workgroup with 128 x 128 per wave (accumulators in AGPRs), so each 16-byte
// LDS read feeds four MFMAs.  X is [d_in][ldx], one row per channel, tokens
// contiguous, so both MFMA operands of a tile are row panels of X read along K.  Only tiles on or above the diagonal are computed (the
// algorithmic d(d+1)/2 * N multiply-adds).  When a layer has too few tiles to
// fill the chip, tokens are split across workgroups and the partial tiles are
// summed in a fixed order by a second kernel, so H is bit-reproducible.
//
// fp32 activations go through the fp32 matrix-core GEMM (upper tiles only).
#include "common.h"

namespace gptq {
namespace {

constexpr int TS = 256;        // output tile edge (4 waves, each 128 x 128)
constexpr int KT = 64;         // bf16 elements of K per LDS stage (8 chunks of 16 B per row)
constexpr int kThreads = 256;
constexpr int kCUs = 256;

// LDS panel: 256 rows x 128 B, unpadded.  Logical 16-byte chunk c of row r sits
// at position c ^ (r & 7), so eight consecutive rows read at one logical chunk
// hit eight different bank groups.
struct SyrkSmem {
    uint4 a[2][TS][KT / 8];
    uint4 b[2][TS][KT / 8];
};

__device__ __forceinline__ void tile_of(int64_t t, int nt, int &ti, int &tj) {
    // Upper-triangle tiles in row-major order: row i holds nt - i tiles.
    int i = 0;
    int64_t before = 0;
    while (before + (nt - i) <= t) {
        before += nt - i;
        ++i;
    }
    ti = i;
    tj = i + (int)(t - before);
}

// One stage of a 256-row panel straight from global memory into LDS
// (global_load_lds_dwordx4: lane l of a wave writes LDS bytes [16 l, 16 l + 16)
// of the wave's 1 KB window).  Wave w fills rows 64 w .. 64 w + 63, eight rows
// per instruction; each lane fetches the global chunk that belongs at its LDS
// position.  Rows past d are clamped to row d-1 (valid memory; those outputs
// are discarded).
__device__ __forceinline__ void panel_dma(uint4 (*dst)[KT / 8], const uint16_t *X, int64_t ldx, int64_t d,
                                          int64_t row0, int64_t k0, int wave, int lane) {
    const int rr = lane >> 3, pos = lane & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = wave * 64 + i * 8 + rr;
        const int c = pos ^ (row & 7);
        int64_t gr = row0 + row;
        gr = gr < d ? gr : d - 1;
        const uint16_t *src = X + gr * ldx + k0 + c * 8;
        __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                         (__attribute__((address_space(3))) void *)(&dst[wave * 64 + i * 8][0]),
                                         16, 0, 0);
    }
}

// The same LDS image from masked register loads (last, partial stage of K).
__device__ __forceinline__ void panel_tail(uint4 (*dst)[KT / 8], const uint16_t *X, int64_t ldx, int64_t d,
                                           int64_t row0, int64_t k0, int64_t kend, int wave, int lane) {
    const int rr = lane >> 3, pos = lane & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = wave * 64 + i * 8 + rr;
        const int c = pos ^ (row & 7);
        const int64_t gr = row0 + row, gk = k0 + c * 8;
        uint16_t tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = (gr < d && gk + e < kend) ? X[gr * ldx + gk + e] : (uint16_t)0;
        dst[row][pos] = make_uint4(tmp[0] | ((uint32_t)tmp[1] << 16), tmp[2] | ((uint32_t)tmp[3] << 16),
                                   tmp[4] | ((uint32_t)tmp[5] << 16), tmp[6] | ((uint32_t)tmp[7] << 16));
    }
}

// grid.x = splits * tiles (split-major).  Each wave owns a 128 x 128 quarter
// of the 256 x 256 tile as 4 x 4 v_mfma_f32_32x32x16_bf16 accumulators.
// out_partial == nullptr: H += 2 acc (upper triangle); else raw partial tile.
__global__ __launch_bounds__(kThreads) void syrk_bf16_kernel(const uint16_t *__restrict__ X, int64_t ldx, int64_t d,
                                                             int64_t n_tok, int64_t kchunk, int nt, int64_t ntiles,
                                                             float *__restrict__ H, float *__restrict__ out_partial) {
    const int64_t t_lin = blockIdx.x % ntiles, split = blockIdx.x / ntiles;
    int ti, tj;
    tile_of(t_lin, nt, ti, tj);
    const bool diag = ti == tj;
    const int64_t r0 = (int64_t)ti * TS, c0 = (int64_t)tj * TS;
    const int64_t kbeg = split * kchunk;
    const int64_t kend = (kbeg + kchunk) < n_tok ? (kbeg + kchunk) : n_tok;

    __shared__ SyrkSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // In a diagonal tile the lower-left quarter lies below the diagonal: it is
    // computed with the others (uniform control flow) and never stored.
    const bool idle = diag && wm > wn;

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto fill = [&](int buf, int64_t k0) {
        if (k0 + KT <= kend) {
            panel_dma(sm.a[buf], X, ldx, d, r0, k0, wave, lane);
            if (!diag) panel_dma(sm.b[buf], X, ldx, d, c0, k0, wave, lane);
        } else {
            panel_tail(sm.a[buf], X, ldx, d, r0, k0, kend, wave, lane);
            if (!diag) panel_tail(sm.b[buf], X, ldx, d, c0, k0, kend, wave, lane);
        }
    };

    if (kbeg < kend) {
        fill(0, kbeg);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int buf = 0;
        const int row = lane & 31, half = lane >> 5;
        for (int64_t k0 = kbeg; k0 < kend; k0 += KT) {
            if (k0 + KT < kend) fill(buf ^ 1, k0 + KT);
            {
                uint4(*sa)[KT / 8] = sm.a[buf];
                uint4(*sb)[KT / 8] = diag ? sm.a[buf] : sm.b[buf];
#pragma unroll
                for (int ks = 0; ks < KT / 16; ++ks) {
                    const int c = 2 * ks + half;
                    bf16x8 fa[4], fb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ra = wm * 128 + i * 32 + row;
                        fa[i] = __builtin_bit_cast(bf16x8, sa[ra][c ^ (ra & 7)]);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int rb = wn * 128 + j * 32 + row;
                        fb[j] = __builtin_bit_cast(bf16x8, sb[rb][c ^ (rb & 7)]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            buf ^= 1;
        }
    }

    if (out_partial) {
        float *dst = out_partial + (int64_t)blockIdx.x * (TS * TS);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int li = wm * 128 + i * 32 + mfma32_row(r, lane);
                    const int lj = wn * 128 + j * 32 + mfma32_col(lane);
                    dst[li * TS + lj] = acc[i][j][r];
                }
        return;
    }
    if (idle) return;
    // H += 2 acc, one 32 x 32 sub-tile at a time: its reads before its writes.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float hold[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gi = r0 + wm * 128 + i * 32 + mfma32_row(r, lane);
                const int64_t gj = c0 + wn * 128 + j * 32 + mfma32_col(lane);
                hold[r] = (gi < d && gj < d && gi <= gj) ? H[gi * d + gj] : 0.0f;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gi = r0 + wm * 128 + i * 32 + mfma32_row(r, lane);
                const int64_t gj = c0 + wn * 128 + j * 32 + mfma32_col(lane);
                if (gi < d && gj < d && gi <= gj) H[gi * d + gj] = hold[r] + 2.0f * acc[i][j][r];
            }
        }
}

// H[upper] += 2 * sum_s partial[s][tile]  (fixed summation order).
__global__ __launch_bounds__(kThreads) void syrk_reduce_kernel(const float *__restrict__ part, int splits,
                                                               int64_t ntiles, int nt, int64_t d,
                                                               float *__restrict__ H) {
    const int64_t t = blockIdx.x / (TS * TS / (kThreads * 4));
    const int64_t chunk = blockIdx.x % (TS * TS / (kThreads * 4));
    int ti, tj;
    tile_of(t, nt, ti, tj);
    const int e0 = (int)(chunk * kThreads * 4 + threadIdx.x * 4);
    const int li = e0 / TS, lj = e0 % TS;
    const int64_t gi = (int64_t)ti * TS + li, gj0 = (int64_t)tj * TS + lj;
    if (gi >= d) return;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < splits; ++k) {
        const float4 v = *reinterpret_cast<const float4 *>(part + ((int64_t)k * ntiles + t) * (TS * TS) + e0);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int64_t gj = gj0 + c;
        if (gj < d && gi <= gj) H[gi * d + gj] += 2.0f * sv[c];
    }
}

// hdiag[i] += 2 * sum_t X[i][t]^2 in fp64.  One workgroup per channel.
template <typename T>
__global__ __launch_bounds__(kThreads) void diag_f64_kernel(const T *__restrict__ X, int64_t ldx, int64_t n_tok,
                                                            double *__restrict__ hdiag) {
    const int64_t i = blockIdx.x;
    const T *row = X + i * ldx;
    double s = 0.0;
    for (int64_t t = threadIdx.x; t < n_tok; t += kThreads) {
        float v;
        if constexpr (sizeof(T) == 2) {
            v = __uint_as_float((uint32_t)row[t] << 16);
        } else {
            v = row[t];
        }
        s += (double)v * (double)v;
    }
    __shared__ double red[kThreads];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) hdiag[i] += 2.0 * red[0];
}

struct SyrkPlan {
    int nt;
    int64_t ntiles;
    int splits;
    int64_t kchunk;
};

// Token splits: pick the count that minimizes an estimate of
//   rounds of workgroups over the CUs x stages per split  +  partial-tile traffic.
SyrkPlan plan_syrk(int64_t d, int64_t n_tok) {
    SyrkPlan p;
    p.nt = (int)ceil_div(d, TS);
    p.ntiles = (int64_t)p.nt * (p.nt + 1) / 2;
    const double stage_us = 2.0;                        // one 256x256x64 stage per CU (measured order)
    const double part_us = 2.0 * TS * TS * 4 / 4.0e6;  // write + read of one partial tile at ~4 TB/s (whole chip)
    double best = 1e300;
    int best_s = 1;
    for (int s = 1; s <= 64; ++s) {
        const int64_t kc = ceil_div(ceil_div(n_tok, s), KT) * KT;
        if (s > 1 && kc < 8 * KT) break;
        const int64_t wgs = p.ntiles * s;
        const double rounds = (double)ceil_div(wgs, kCUs);
        const double t = rounds * (double)(kc / KT) * stage_us + (s > 1 ? (double)wgs * part_us : 0.0);
        if (t < best) {
            best = t;
            best_s = s;
        }
    }
    p.kchunk = ceil_div(ceil_div(n_tok, best_s), KT) * KT;
    p.splits = (int)ceil_div(n_tok, p.kchunk);
    if (p.splits < 1) p.splits = 1;
    return p;
}

}  // namespace

size_t hessian_ws_bytes(int64_t d_in, int64_t n_tok, gptq_dtype dt) {
    if (dt != GPTQ_DT_BF16 || n_tok <= 0) return 0;
    SyrkPlan p = plan_syrk(d_in, n_tok);
    if (p.splits <= 1) return 0;
    return (size_t)p.splits * (size_t)p.ntiles * TS * TS * sizeof(float);
}

hipError_t run_hessian(float *H, double *hdiag, const void *X, gptq_dtype dt, int64_t d, int64_t n_tok, int64_t ldx,
                       void *ws, hipStream_t s) {
    if (n_tok <= 0) return hipSuccess;
    if (dt == GPTQ_DT_BF16) {
        SyrkPlan p = plan_syrk(d, n_tok);
        float *part = p.splits > 1 ? static_cast<float *>(ws) : nullptr;
        hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)(p.ntiles * p.splits)), dim3(kThreads), 0, s,
                           static_cast<const uint16_t *>(X), ldx, d, n_tok, p.kchunk, p.nt, p.ntiles, H, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (part) {
            hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)(p.ntiles * (TS * TS / (kThreads * 4)))), dim3(kThreads),
                               0, s, part, p.splits, p.ntiles, p.nt, d, H);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (hdiag) {
            hipLaunchKernelGGL(diag_f64_kernel<uint16_t>, dim3((unsigned)d), dim3(kThreads), 0, s,
                               static_cast<const uint16_t *>(X), ldx, n_tok, hdiag);
            e = hipGetLastError();
        }
        return e;
    }
    GemmDesc g;
    g.M = d;
    g.N = d;
    g.K = n_tok;
    g.A = static_cast<const float *>(X);
    g.lda = ldx;
    g.a_trans = 0;
    g.B = static_cast<const float *>(X);
    g.ldb = ldx;
    g.b_trans = 1;
    g.C = H;
    g.ldc = d;
    g.alpha = 2.0f;
    g.beta = 1.0f;
    g.upper_only = 1;
    hipError_t e = launch_gemm_f32(g, s);
    if (e != hipSuccess) return e;
    if (hdiag) {
        hipLaunchKernelGGL(diag_f64_kernel<float>, dim3((unsigned)d), dim3(kThreads), 0, s,
                           static_cast<const float *>(X), ldx, n_tok, hdiag);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gptq
