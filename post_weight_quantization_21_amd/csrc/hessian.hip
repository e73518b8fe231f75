// Step 1 of GPTQ: H += 2 X X^T from calibration activations (page "LLM 量化方法
// 原理与实现详解", §4.1: the layer objective's Hessian is 2 X X^T).
//
// bf16 activations: a symmetric rank-k update on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).  X is [d_in][ldx], one row per
// channel, tokens contiguous, so both MFMA operands of a tile are row panels of
// X read along K.  Only tiles on or above the diagonal are computed (the
// algorithmic d(d+1)/2 * N multiply-adds).  When a layer has too few tiles to
// fill the chip, tokens are split across workgroups and the partial tiles are
// summed in a fixed order by a second kernel, so H is bit-reproducible.
//
// fp32 activations go through the fp32 matrix-core GEMM (upper tiles only).
#include "common.h"

namespace gptq {
namespace {

constexpr int TS = 128;        // output tile edge
constexpr int KT = 64;         // bf16 elements of K per LDS stage
constexpr int KPAD = KT + 8;   // LDS row length in bf16 (144 B: conflict-free 16 B reads)
constexpr int kThreads = 256;
constexpr int kTargetBlocks = 1024;

struct SyrkSmem {
    uint16_t a[2][TS][KPAD];
    uint16_t b[2][TS][KPAD];
};

__device__ __forceinline__ void tile_of(int64_t t, int nt, int &ti, int &tj) {
    // Upper-triangle tiles in row-major order: row i holds nt - i tiles.
    int i = 0;
    int64_t before = 0;
    // nt <= 1024 here; a short scan is cheaper than the float root for small nt.
    while (before + (nt - i) <= t) {
        before += nt - i;
        ++i;
    }
    ti = i;
    tj = i + (int)(t - before);
}

struct PanelLoader {
    const uint16_t *X;
    int64_t ldx, d;

    // 128 rows x 64 bf16: 1024 chunks of 8 elements, 4 per thread.
    __device__ __forceinline__ void load(int64_t row0, int64_t k0, int64_t kend, int tid, uint4 (&r)[4]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx >> 3, c = (idx & 7) * 8;
            const int64_t gr = row0 + row, gk = k0 + c;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (gr < d) {
                const uint16_t *src = X + gr * ldx + gk;
                if (gk + 8 <= kend) {
                    v = *reinterpret_cast<const uint4 *>(src);
                } else if (gk < kend) {
                    uint16_t tmp[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) tmp[e] = (gk + e < kend) ? src[e] : (uint16_t)0;
                    v.x = tmp[0] | ((uint32_t)tmp[1] << 16);
                    v.y = tmp[2] | ((uint32_t)tmp[3] << 16);
                    v.z = tmp[4] | ((uint32_t)tmp[5] << 16);
                    v.w = tmp[6] | ((uint32_t)tmp[7] << 16);
                }
            }
            r[i] = v;
        }
    }
    __device__ __forceinline__ static void store(uint16_t (*s)[KPAD], int tid, const uint4 (&r)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + kThreads * i;
            const int row = idx >> 3, c = (idx & 7) * 8;
            *reinterpret_cast<uint4 *>(&s[row][c]) = r[i];
        }
    }
};

// grid.x = upper tiles, grid.y = token splits.  out_partial == nullptr: H += 2 acc.
__global__ __launch_bounds__(kThreads) void syrk_bf16_kernel(const uint16_t *__restrict__ X, int64_t ldx, int64_t d,
                                                             int64_t n_tok, int64_t kchunk, int nt,
                                                             float *__restrict__ H, float *__restrict__ out_partial) {
    int ti, tj;
    tile_of(blockIdx.x, nt, ti, tj);
    const bool diag = ti == tj;
    const int64_t r0 = (int64_t)ti * TS, c0 = (int64_t)tj * TS;
    const int64_t kbeg = (int64_t)blockIdx.y * kchunk;
    const int64_t kend = (kbeg + kchunk) < n_tok ? (kbeg + kchunk) : n_tok;

    __shared__ SyrkSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    PanelLoader ld{X, ldx, d};

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (kbeg < kend) {
        uint4 ra[4], rb[4];
        ld.load(r0, kbeg, kend, tid, ra);
        if (!diag) ld.load(c0, kbeg, kend, tid, rb);
        PanelLoader::store(sm.a[0], tid, ra);
        if (!diag) PanelLoader::store(sm.b[0], tid, rb);
        __syncthreads();
        int buf = 0;
        for (int64_t k0 = kbeg; k0 < kend; k0 += KT) {
            const bool more = k0 + KT < kend;
            if (more) {
                ld.load(r0, k0 + KT, kend, tid, ra);
                if (!diag) ld.load(c0, k0 + KT, kend, tid, rb);
            }
            uint16_t(*sa)[KPAD] = sm.a[buf];
            uint16_t(*sb)[KPAD] = diag ? sm.a[buf] : sm.b[buf];
            const int row = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
            for (int kk = 0; kk < KT; kk += 16) {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(&sa[wm * 64 + row][kk + kh]);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(&sa[wm * 64 + 32 + row][kk + kh]);
                const bf16x8 b0 = *reinterpret_cast<const bf16x8 *>(&sb[wn * 64 + row][kk + kh]);
                const bf16x8 b1 = *reinterpret_cast<const bf16x8 *>(&sb[wn * 64 + 32 + row][kk + kh]);
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
            }
            if (more) {
                PanelLoader::store(sm.a[buf ^ 1], tid, ra);
                if (!diag) PanelLoader::store(sm.b[buf ^ 1], tid, rb);
            }
            __syncthreads();
            buf ^= 1;
        }
    }

    if (out_partial) {
        const int64_t t = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        float *dst = out_partial + t * (TS * TS);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int li = wm * 64 + i * 32 + mfma32_row(r, lane);
                    const int lj = wn * 64 + j * 32 + mfma32_col(lane);
                    dst[li * TS + lj] = acc[i][j][r];
                }
        return;
    }
    // H += 2 acc: all reads first, then all writes (no load waits behind a store).
    float hold[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gi = r0 + wm * 64 + i * 32 + mfma32_row(r, lane);
                const int64_t gj = c0 + wn * 64 + j * 32 + mfma32_col(lane);
                hold[i][j][r] = (gi < d && gj < d && gi <= gj) ? H[gi * d + gj] : 0.0f;
            }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t gi = r0 + wm * 64 + i * 32 + mfma32_row(r, lane);
                const int64_t gj = c0 + wn * 64 + j * 32 + mfma32_col(lane);
                if (gi < d && gj < d && gi <= gj) H[gi * d + gj] = hold[i][j][r] + 2.0f * acc[i][j][r];
            }
}

// H[upper] += 2 * sum_s partial[s][tile]  (fixed summation order).
__global__ __launch_bounds__(kThreads) void syrk_reduce_kernel(const float *__restrict__ part, int splits,
                                                               int64_t ntiles, int nt, int64_t d,
                                                               float *__restrict__ H) {
    int ti, tj;
    tile_of(blockIdx.x, nt, ti, tj);
    for (int e = threadIdx.x; e < TS * TS; e += kThreads) {
        const int li = e / TS, lj = e % TS;
        const int64_t gi = (int64_t)ti * TS + li, gj = (int64_t)tj * TS + lj;
        if (gi >= d || gj >= d || gi > gj) continue;
        float s = 0.0f;
        for (int k = 0; k < splits; ++k) s += part[((int64_t)k * ntiles + blockIdx.x) * (TS * TS) + e];
        H[gi * d + gj] += 2.0f * s;
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

SyrkPlan plan_syrk(int64_t d, int64_t n_tok) {
    SyrkPlan p;
    p.nt = (int)ceil_div(d, TS);
    p.ntiles = (int64_t)p.nt * (p.nt + 1) / 2;
    int64_t want = ceil_div(kTargetBlocks, p.ntiles);
    int64_t maxs = n_tok / (8 * KT);  // keep at least 8 stages per split
    if (want > maxs) want = maxs;
    if (want < 1) want = 1;
    p.kchunk = ceil_div(ceil_div(n_tok, want), KT) * KT;
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
        hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)p.ntiles, (unsigned)p.splits), dim3(kThreads), 0, s,
                           static_cast<const uint16_t *>(X), ldx, d, n_tok, p.kchunk, p.nt, H, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (part) {
            hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)p.ntiles), dim3(kThreads), 0, s, part, p.splits,
                               p.ntiles, p.nt, d, H);
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
