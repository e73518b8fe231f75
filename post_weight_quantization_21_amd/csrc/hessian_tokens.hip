// Hessian accumulation from activations as they arrive: one row per token
// (page "LLM 量化方法原理与实现详解", §4.1: H = 2 X X^T summed over the
// calibration tokens; page "量化经典：LLM.int8 / GPTQ / AWQ", §二 step 1:
// the calibration set is run through the layer and its inputs collected).
//
// A token-major block X[t0 : t0 + T][0 : d] is transposed through LDS into a
// channel-major panel in the workspace (64 x 64 tiles: reads along channels,
// writes along tokens, both coalesced), and the panel goes through the same
// matrix-core SYRK as channel-major activations.  Blocks of at most
// kTokenBlock tokens bound the workspace; repeated calls keep accumulating.
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;
constexpr int64_t kTokenBlock = 65536;  // tokens per transposed panel

// panel[c][t] = X[t0 + t][c] for t < T, c < d, element by element (fp32).
template <typename T_>
__global__ __launch_bounds__(kThreads) void transpose_block_kernel(const T_ *__restrict__ X, int64_t ldx, int64_t d,
                                                                   int64_t t0, int64_t T, T_ *__restrict__ panel,
                                                                   int64_t ldt) {
    __shared__ T_ tile[kTile][kTile + 1];  // +1: the column reads hit distinct banks
    const int64_t c0 = (int64_t)blockIdx.x * kTile, tb = (int64_t)blockIdx.y * kTile;
    const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;  // 64 x 4
    constexpr int kRows = kThreads / kTile;  // rows per pass
#pragma unroll
    for (int i = 0; i < kTile / kRows; ++i) {
        const int r = ty + kRows * i;
        const int64_t t = tb + r, c = c0 + tx;
        tile[r][tx] = (t < T && c < d) ? X[(t0 + t) * ldx + c] : T_(0);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTile / kRows; ++i) {
        const int r = ty + kRows * i;
        const int64_t c = c0 + r, t = tb + tx;
        if (c < d && t < T) panel[c * ldt + t] = tile[tx][r];
    }
}

// bf16: 64 tokens x 128 channels per tile, moved in 16-byte pieces both ways.
// Reads: 16 threads cover one token's 128 channels (256 contiguous bytes);
// writes: 8 threads cover one channel's 64 tokens (128 contiguous bytes), each
// piece gathered from LDS as 8 halves.  Pieces past the channel edge go element
// by element; tokens past T are zero in the tile and never read by the SYRK
// (the panel rows are padded to whole pieces).
constexpr int kTT = 64, kTC = 128, kTP = kTC + 8;  // tile tokens, channels, LDS pitch (halves, 16-byte rows)
__global__ __launch_bounds__(kThreads) void transpose_bf16_kernel(const uint16_t *__restrict__ X, int64_t ldx,
                                                                  int64_t d, int64_t t0, int64_t T,
                                                                  uint16_t *__restrict__ panel, int64_t ldt) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[kTT][kTP];
    const int64_t c0 = (int64_t)blockIdx.x * kTC, tb = (int64_t)blockIdx.y * kTT;
    const int tid = threadIdx.x;
    {
        const int p = tid % 16, r0 = tid / 16;  // piece of 8 channels, first row
#pragma unroll
        for (int i = 0; i < kTT / 16; ++i) {
            const int r = r0 + 16 * i;
            const int64_t t = tb + r, c = c0 + 8 * p;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (t < T) {
                const uint16_t *src = X + (t0 + t) * ldx + c;
                if (c + 8 <= d && ((reinterpret_cast<uintptr_t>(src) & 15) == 0)) {
                    v = *reinterpret_cast<const uint4 *>(src);
                } else {
                    uint16_t h[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) h[j] = c + j < d ? src[j] : (uint16_t)0;
                    v = make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16, h[4] | (uint32_t)h[5] << 16,
                                   h[6] | (uint32_t)h[7] << 16);
                }
            }
            *reinterpret_cast<uint4 *>(&tile[r][8 * p]) = v;
        }
    }
    __syncthreads();
    {
        const int q = tid % 8, cl0 = tid / 8;  // token piece, first channel
#pragma unroll
        for (int i = 0; i < kTC / 32; ++i) {
            const int cl = cl0 + 32 * i;
            const int64_t c = c0 + cl, t = tb + 8 * q;
            if (c < d && t < T) {
                uint16_t h[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) h[j] = tile[8 * q + j][cl];
                *reinterpret_cast<uint4 *>(panel + c * ldt + t) =
                    make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16, h[4] | (uint32_t)h[5] << 16,
                               h[6] | (uint32_t)h[7] << 16);
            }
        }
    }
}

int64_t esz_of(gptq_dtype dt) { return dt == GPTQ_DT_BF16 ? 2 : 4; }
int64_t panel_ld(int64_t T) { return (T + 7) / 8 * 8; }  // 16-byte rows for both element sizes

}  // namespace

size_t hessian_tokens_ws_bytes(int64_t d_in, int64_t n_tok, gptq_dtype dt) {
    if (n_tok <= 0) return 0;
    const int64_t T = std::min<int64_t>(n_tok, kTokenBlock);
    const size_t panel = align_up((size_t)d_in * (size_t)panel_ld(T) * (size_t)esz_of(dt), 256);
    // the SYRK's own scratch for a full block and for the last, shorter one
    const int64_t tail = n_tok % kTokenBlock;
    size_t syrk = hessian_ws_bytes(d_in, T, dt);
    if (tail > 0) syrk = std::max(syrk, hessian_ws_bytes(d_in, tail, dt));
    return panel + syrk;
}

hipError_t run_hessian_tokens(float *H, double *hdiag, const void *X, gptq_dtype dt, int64_t d, int64_t n_tok,
                              int64_t ldx, void *ws, hipStream_t s) {
    if (n_tok <= 0) return hipSuccess;
    const int64_t T = std::min<int64_t>(n_tok, kTokenBlock);
    const int64_t ldt = panel_ld(T);
    char *wsb = static_cast<char *>(ws);
    void *panel = wsb;
    void *syrk_ws = wsb + align_up((size_t)d * (size_t)ldt * (size_t)esz_of(dt), 256);
    for (int64_t t0 = 0; t0 < n_tok; t0 += kTokenBlock) {
        const int64_t Tb = std::min<int64_t>(kTokenBlock, n_tok - t0);
        if (dt == GPTQ_DT_BF16)
            hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)ceil_div(d, kTC), (unsigned)ceil_div(Tb, kTT)),
                               dim3(kThreads), 0, s, static_cast<const uint16_t *>(X), ldx, d, t0, Tb,
                               static_cast<uint16_t *>(panel), ldt);
        else
            hipLaunchKernelGGL(transpose_block_kernel<float>, dim3((unsigned)ceil_div(d, kTile), (unsigned)ceil_div(Tb, kTile)),
                               dim3(kThreads), 0, s, static_cast<const float *>(X), ldx, d, t0, Tb,
                               static_cast<float *>(panel), ldt);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if ((e = run_hessian(H, hdiag, panel, dt, d, Tb, ldt, syrk_ws, s)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gptq
