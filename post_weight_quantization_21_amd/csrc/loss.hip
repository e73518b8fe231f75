// Layer loss ||W X - W_hat X||_F^2 = 1/2 sum_r D_r H D_r^T, D = W_hat - W
// (page "LLM 量化方法原理与实现详解", §4.1: GPTQ minimizes ||WX - W_hat X||_F^2,
// and H = 2 X X^T).  D and the full symmetric H are materialized, D H runs on
// fp32 matrix cores with a fused epilogue that multiplies by D and sums each
// tile in fp64; a one-workgroup kernel adds the tile sums in a fixed order.
#include "common.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void deq_diff_kernel(const float *__restrict__ W, const uint8_t *__restrict__ codes,
                                                            const float *__restrict__ scales, const float *__restrict__ zeros,
                                                            const int32_t *__restrict__ g_idx, int64_t d_out, int64_t d_in, int64_t g,
                                                            int64_t ng, float *__restrict__ D) {
#pragma clang fp contract(off)
    for (int64_t r = blockIdx.y; r < d_out; r += gridDim.y)  // rows grid-stride (grid y is capped)
        for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < d_in; c += (int64_t)gridDim.x * kThreads) {
            int64_t gi = g_idx ? (int64_t)g_idx[c] : c / g;
            gi = gi < 0 ? 0 : (gi >= ng ? ng - 1 : gi);  // malformed g_idx: wrong values, no wild access
            const float s = scales[r * ng + gi], z = zeros[r * ng + gi];
            const float wh = ((float)codes[r * d_in + c] - z) * s;
            D[r * d_in + c] = wh - W[r * d_in + c];
        }
}

__global__ __launch_bounds__(kThreads) void symmetrize_kernel(const float *__restrict__ H, int64_t d, float *__restrict__ Hs) {
    for (int64_t i = blockIdx.y; i < d; i += gridDim.y)  // rows grid-stride (grid y is capped)
        for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < d; j += (int64_t)gridDim.x * kThreads)
            Hs[i * d + j] = i <= j ? H[i * d + j] : H[j * d + i];
}

__global__ __launch_bounds__(kThreads) void sum_partials_kernel(const double *__restrict__ p, int64_t n, double *__restrict__ out) {
    __shared__ double red[kThreads];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += kThreads) s += p[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = 0.5 * red[0];
}

struct LossLayout {
    size_t d_off, h_off, p_off, total;
};

LossLayout layout(int64_t d_out, int64_t d_in) {
    LossLayout l;
    l.d_off = 0;
    l.h_off = align_up((size_t)d_out * d_in * sizeof(float), 256);
    l.p_off = l.h_off + align_up((size_t)d_in * d_in * sizeof(float), 256);
    l.total = l.p_off + align_up((size_t)(ceil_div(d_out, kGemmTile) * ceil_div(d_in, kGemmTile)) * sizeof(double), 256);
    return l;
}

}  // namespace

size_t loss_ws_bytes(int64_t d_out, int64_t d_in) { return layout(d_out, d_in).total; }

hipError_t run_loss(const float *W, const uint8_t *codes, const float *scales, const float *zeros, const int32_t *g_idx,
                    const float *H, int64_t d_out, int64_t d_in, int32_t group_size, double *loss, void *ws,
                    hipStream_t s) {
    const LossLayout l = layout(d_out, d_in);
    char *base = static_cast<char *>(ws);
    float *D = reinterpret_cast<float *>(base + l.d_off);
    float *Hs = reinterpret_cast<float *>(base + l.h_off);
    double *part = reinterpret_cast<double *>(base + l.p_off);
    const int64_t g = group_size > 0 ? group_size : d_in;
    const unsigned gx = (unsigned)std::min<int64_t>(ceil_div(d_in, kThreads), 64);
    hipLaunchKernelGGL(deq_diff_kernel, dim3(gx, (unsigned)std::min<int64_t>(d_out, 65535)), dim3(kThreads), 0, s, W, codes,
                       scales, zeros, g_idx, d_out, d_in, g, d_in / g, D);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(symmetrize_kernel, dim3(gx, (unsigned)std::min<int64_t>(d_in, 65535)), dim3(kThreads), 0, s, H, d_in,
                       Hs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GemmDesc gd;
    gd.M = d_out;
    gd.N = d_in;
    gd.K = d_in;
    gd.A = D;
    gd.lda = d_in;
    gd.B = Hs;
    gd.ldb = d_in;
    gd.C = nullptr;
    gd.ldc = d_in;
    gd.epilogue = EPI_DOT;
    gd.Dm = D;
    gd.ldd = d_in;
    gd.partial = part;
    if ((e = launch_gemm_f32(gd, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(sum_partials_kernel, dim3(1), dim3(kThreads), 0, s, part, gemm_num_tiles(gd), loss);
    return hipGetLastError();
}

}  // namespace gptq
