// Per-channel scaling before the pass (page "LLM 量化方法原理与实现详解", §4.2
// AWQ: s = (mean|X| / mean|W|)^alpha with alpha found by a grid search on
// ||Q(W s)(X / s) - W X||; §4.3 SmoothQuant: s = max|X|^alpha / max|W|^(1 -
// alpha)).  Either way GPTQ then solves the equivalent problem W' = W diag(s),
// H' = diag(s)^-1 H diag(s)^-1 (X' = X diag(s)^-1 at inference).
//
//   chan_stats_kernel    per input channel of X: max |x| and sum |x| (fp64),
//                        accumulated into the caller's arrays (chunks add up)
//   wcol_*_kernel        per input column of W: max |w| and sum |w| over the
//                        rows, in 256-row partials summed in a fixed order
//   awq / smooth scales  the formulas above, fp32, at least 1e-5
//   scale_*_kernel       W' and H' (upper triangle), hdiag / s^2
// The AWQ search runs on the device end to end: for each alpha the scales,
// W', H', the RTN grids and codes of W', and the loss through H' (the layer
// loss kernels); then the first smallest loss picks alpha and s.
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kRowChunk = 256;  // rows per partial of the weight statistics

__device__ __forceinline__ float widen_x(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ float widen_x(float v) { return v; }

// One block per channel c: absmax[c] = max(absmax[c], max_t |X[c][t]|), abssum[c] += sum_t |X[c][t]|.
template <typename T>
__global__ __launch_bounds__(kThreads) void chan_stats_kernel(const T *__restrict__ X, int64_t ldx, int64_t n_tok,
                                                              float *__restrict__ absmax, double *__restrict__ abssum) {
    __shared__ float smx[kThreads / kWave];
    __shared__ double ssm[kThreads / kWave];
    const int64_t c = blockIdx.x;
    const T *row = X + c * ldx;
    float mx = 0.0f;
    double sm = 0.0;
    for (int64_t t = threadIdx.x; t < n_tok; t += kThreads) {
        const float a = fabsf(widen_x(row[t]));
        mx = fmaxf(mx, a);
        sm += (double)a;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, off));
        sm += __shfl_xor(sm, off);
    }
    const int w = threadIdx.x / kWave;
    if (threadIdx.x % kWave == 0) {
        smx[w] = mx;
        ssm[w] = sm;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / kWave; ++i) {
            mx = fmaxf(mx, smx[i]);
            sm += ssm[i];
        }
        absmax[c] = fmaxf(absmax[c], mx);
        abssum[c] += sm;
    }
}

// Partials over 256-row chunks: pmax[chunk][j], psum[chunk][j] (coalesced along j).
__global__ __launch_bounds__(kThreads) void wcol_partial_kernel(const float *__restrict__ W, int64_t d_out, int64_t d_in,
                                                                float *__restrict__ pmax, double *__restrict__ psum) {
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= d_in) return;
    const int64_t r0 = (int64_t)blockIdx.y * kRowChunk, r1 = std::min<int64_t>(d_out, r0 + kRowChunk);
    float mx = 0.0f;
    double sm = 0.0;
    for (int64_t r = r0; r < r1; ++r) {
        const float a = fabsf(W[r * d_in + j]);
        mx = fmaxf(mx, a);
        sm += (double)a;
    }
    pmax[blockIdx.y * d_in + j] = mx;
    psum[blockIdx.y * d_in + j] = sm;
}

// wmax[j], wmean[j] from the partials, chunks in order.
__global__ __launch_bounds__(kThreads) void wcol_reduce_kernel(const float *__restrict__ pmax,
                                                               const double *__restrict__ psum, int64_t nchunks,
                                                               int64_t d_out, int64_t d_in, float *__restrict__ wmax,
                                                               float *__restrict__ wmean) {
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= d_in) return;
    float mx = 0.0f;
    double sm = 0.0;
    for (int64_t c = 0; c < nchunks; ++c) {
        mx = fmaxf(mx, pmax[c * d_in + j]);
        sm += psum[c * d_in + j];
    }
    if (wmax) wmax[j] = mx;
    if (wmean) wmean[j] = (float)(sm / (double)d_out);
}

// AWQ: s_j = max((a_j / w_j)^alpha, 1e-5), a_j = abssum_j / n_tok, s_j = 1 when w_j = 0.
// alpha = alpha_idx / n_grid, or (alpha_idx < 0) the index the search picked, read from *best.
__global__ __launch_bounds__(kThreads) void awq_scale_kernel(const double *__restrict__ act_abssum, int64_t n_tok,
                                                             const float *__restrict__ wmean, int64_t d_in,
                                                             int alpha_idx, int n_grid, const int32_t *__restrict__ best,
                                                             float *__restrict__ s) {
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= d_in) return;
    const int ai = alpha_idx >= 0 ? alpha_idx : *best;
    const float alpha = (float)ai / (float)n_grid;
    const float a = (float)(act_abssum[j] / (double)n_tok);
    const float w = wmean[j];
    const float r = w > 0.0f ? a / w : 1.0f;
    s[j] = fmaxf(powf(r, alpha), 1e-5f);
}

// SmoothQuant: s_j = max(amax_j^alpha / wmax_j^(1 - alpha), 1e-5), s_j = 1 when the denominator is 0.
__global__ __launch_bounds__(kThreads) void smooth_scale_kernel(const float *__restrict__ amax,
                                                                const float *__restrict__ wmax, int64_t d_in,
                                                                float alpha, float *__restrict__ s) {
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j >= d_in) return;
    const float num = powf(amax[j], alpha), den = powf(wmax[j], 1.0f - alpha);
    s[j] = fmaxf(den > 0.0f ? num / den : 1.0f, 1e-5f);
}

// Wd[r][j] = W[r][j] s_j (Wd may be W).
__global__ __launch_bounds__(kThreads) void scale_w_kernel(const float *__restrict__ W, int64_t d_out, int64_t d_in,
                                                           const float *__restrict__ s, float *__restrict__ Wd) {
    const int64_t n = d_out * d_in;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
        Wd[i] = W[i] * s[i % d_in];
}

// Hd[i][j] = H[i][j] / (s_i s_j) on the upper triangle (Hd may be H); hdiag[j] /= s_j^2.
__global__ __launch_bounds__(kThreads) void scale_h_kernel(const float *__restrict__ H, int64_t d,
                                                           const float *__restrict__ s, float *__restrict__ Hd) {
    for (int64_t i = blockIdx.y; i < d; i += gridDim.y) {  // rows, grid-stride (grid y is capped)
        const float si = 1.0f / s[i];
        for (int64_t j = i + (int64_t)blockIdx.x * kThreads + threadIdx.x; j < d; j += (int64_t)gridDim.x * kThreads)
            Hd[i * d + j] = (H[i * d + j] * si) / s[j];
    }
}

__global__ __launch_bounds__(kThreads) void scale_hdiag_kernel(double *__restrict__ hdiag, int64_t d,
                                                               const float *__restrict__ s) {
    const int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (j < d) hdiag[j] /= (double)s[j] * (double)s[j];
}

// best = the first index of the smallest loss.
__global__ void argmin_kernel(const double *__restrict__ loss, int n, int32_t *__restrict__ best) {
    if (threadIdx.x != 0) return;
    int b = 0;
    for (int i = 1; i < n; ++i)
        if (loss[i] < loss[b]) b = i;
    *best = b;
}

struct WcolLayout {
    size_t pmax, psum, wmax, wmean, total;
};
WcolLayout wcol_layout(int64_t d_out, int64_t d_in) {
    const int64_t nch = ceil_div(d_out, kRowChunk);
    WcolLayout l;
    l.pmax = 0;
    l.psum = align_up((size_t)nch * (size_t)d_in * 4, 256);
    l.wmax = l.psum + align_up((size_t)nch * (size_t)d_in * 8, 256);
    l.wmean = l.wmax + align_up((size_t)d_in * 4, 256);
    l.total = l.wmean + align_up((size_t)d_in * 4, 256);
    return l;
}

hipError_t wcol_stats(const float *W, int64_t d_out, int64_t d_in, char *ws, float **wmax, float **wmean, hipStream_t s) {
    const WcolLayout l = wcol_layout(d_out, d_in);
    const int64_t nch = ceil_div(d_out, kRowChunk);
    float *pmax = reinterpret_cast<float *>(ws + l.pmax);
    double *psum = reinterpret_cast<double *>(ws + l.psum);
    *wmax = reinterpret_cast<float *>(ws + l.wmax);
    *wmean = reinterpret_cast<float *>(ws + l.wmean);
    hipLaunchKernelGGL(wcol_partial_kernel, dim3((unsigned)ceil_div(d_in, kThreads), (unsigned)nch), dim3(kThreads), 0, s, W,
                       d_out, d_in, pmax, psum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wcol_reduce_kernel, dim3((unsigned)ceil_div(d_in, kThreads)), dim3(kThreads), 0, s, pmax, psum, nch,
                       d_out, d_in, *wmax, *wmean);
    return hipGetLastError();
}

unsigned grid_of(int64_t n) { return (unsigned)std::min<int64_t>(ceil_div(n, kThreads), 65536); }

struct AwqLayout {
    size_t wcol, s, wq, hq, codes, sc, ze, loss_ws, total;
};
AwqLayout awq_layout(int64_t d_out, int64_t d_in, const gptq_config &c) {
    const int64_t g = c.group_size > 0 ? c.group_size : d_in;
    const int64_t ng = d_in / g;
    AwqLayout l;
    l.wcol = 0;
    l.s = l.wcol + wcol_layout(d_out, d_in).total;
    l.wq = l.s + align_up((size_t)d_in * 4, 256);
    l.hq = l.wq + align_up((size_t)d_out * (size_t)d_in * 4, 256);
    l.codes = l.hq + align_up((size_t)d_in * (size_t)d_in * 4, 256);
    l.sc = l.codes + align_up((size_t)d_out * (size_t)d_in, 256);
    l.ze = l.sc + align_up((size_t)d_out * (size_t)ng * 4, 256);
    l.loss_ws = l.ze + align_up((size_t)d_out * (size_t)ng * 4, 256);
    l.total = l.loss_ws + loss_ws_bytes(d_out, d_in);
    return l;
}

}  // namespace

hipError_t run_channel_stats(const void *X, gptq_dtype dt, int64_t d_in, int64_t n_tok, int64_t ldx, float *absmax,
                             double *abssum, hipStream_t s) {
    if (n_tok <= 0) return hipSuccess;
    if (dt == GPTQ_DT_BF16)
        hipLaunchKernelGGL(chan_stats_kernel<uint16_t>, dim3((unsigned)d_in), dim3(kThreads), 0, s,
                           static_cast<const uint16_t *>(X), ldx, n_tok, absmax, abssum);
    else
        hipLaunchKernelGGL(chan_stats_kernel<float>, dim3((unsigned)d_in), dim3(kThreads), 0, s, static_cast<const float *>(X),
                           ldx, n_tok, absmax, abssum);
    return hipGetLastError();
}

size_t smooth_ws_bytes(int64_t d_out, int64_t d_in) { return wcol_layout(d_out, d_in).total; }

hipError_t run_smooth_scales(const float *act_absmax, const float *W, int64_t d_out, int64_t d_in, float alpha,
                             float *s_out, void *ws, hipStream_t s) {
    float *wmax, *wmean;
    hipError_t e = wcol_stats(W, d_out, d_in, static_cast<char *>(ws), &wmax, &wmean, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(smooth_scale_kernel, dim3((unsigned)ceil_div(d_in, kThreads)), dim3(kThreads), 0, s, act_absmax, wmax,
                       d_in, alpha, s_out);
    return hipGetLastError();
}

hipError_t run_scale_layer(float *W, int64_t d_out, int64_t d_in, float *H, double *hdiag, const float *sv,
                           hipStream_t s) {
    hipError_t e;
    if (W) {
        hipLaunchKernelGGL(scale_w_kernel, dim3(grid_of(d_out * d_in)), dim3(kThreads), 0, s, W, d_out, d_in, sv, W);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (H) {
        hipLaunchKernelGGL(scale_h_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(d_in, kThreads), 64), (unsigned)std::min<int64_t>(d_in, 65535)),
                           dim3(kThreads), 0, s, H, d_in, sv, H);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (hdiag) {
        hipLaunchKernelGGL(scale_hdiag_kernel, dim3((unsigned)ceil_div(d_in, kThreads)), dim3(kThreads), 0, s, hdiag, d_in, sv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

size_t awq_ws_bytes(int64_t d_out, int64_t d_in, const gptq_config &c) { return awq_layout(d_out, d_in, c).total; }

hipError_t run_awq_search(const float *W, int64_t d_out, int64_t d_in, const float *H, const double *act_abssum,
                          int64_t n_tok, const gptq_config &c, int n_grid, float *s_out, double *loss_out,
                          int32_t *best_out, void *ws, hipStream_t s) {
    const AwqLayout l = awq_layout(d_out, d_in, c);
    char *wsb = static_cast<char *>(ws);
    float *wmax, *wmean;
    hipError_t e = wcol_stats(W, d_out, d_in, wsb + l.wcol, &wmax, &wmean, s);
    if (e != hipSuccess) return e;
    float *sv = reinterpret_cast<float *>(wsb + l.s);
    float *Wq = reinterpret_cast<float *>(wsb + l.wq);
    float *Hq = reinterpret_cast<float *>(wsb + l.hq);
    uint8_t *codes = reinterpret_cast<uint8_t *>(wsb + l.codes);
    float *sc = reinterpret_cast<float *>(wsb + l.sc);
    float *ze = reinterpret_cast<float *>(wsb + l.ze);
    gptq_config rc = c;
    rc.grid = GPTQ_GRID_DYNAMIC;  // RTN fits every grid on the (scaled) weights it is given
    for (int a = 0; a < n_grid; ++a) {
        hipLaunchKernelGGL(awq_scale_kernel, dim3((unsigned)ceil_div(d_in, kThreads)), dim3(kThreads), 0, s, act_abssum, n_tok,
                           wmean, d_in, a, n_grid, (const int32_t *)nullptr, sv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(scale_w_kernel, dim3(grid_of(d_out * d_in)), dim3(kThreads), 0, s, W, d_out, d_in, sv, Wq);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(scale_h_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(d_in, kThreads), 64), (unsigned)std::min<int64_t>(d_in, 65535)),
                           dim3(kThreads), 0, s, H, d_in, sv, Hq);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = run_rtn(Wq, d_out, d_in, rc, codes, sc, ze, s)) != hipSuccess) return e;
        if ((e = run_loss(Wq, codes, sc, ze, nullptr, Hq, d_out, d_in, c.group_size, loss_out + a, wsb + l.loss_ws, s)) !=
            hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(argmin_kernel, dim3(1), dim3(64), 0, s, loss_out, n_grid, best_out);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(awq_scale_kernel, dim3((unsigned)ceil_div(d_in, kThreads)), dim3(kThreads), 0, s, act_abssum, n_tok,
                       wmean, d_in, -1, n_grid, (const int32_t *)best_out, s_out);
    return hipGetLastError();
}

}  // namespace gptq
