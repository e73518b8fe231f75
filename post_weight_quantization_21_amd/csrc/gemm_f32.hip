// fp32 matrix-core GEMM for gfx950:  C = alpha * op(A) op(B) + beta * C.
//
// One kernel serves every dense fp32 contraction of the library: the lazy
// batch update of GPTQ (W[:, trail] -= E U[block, trail]), the panel solve and
// symmetric rank-k update of the blocked Cholesky factorization, the
// triangular products of the triangular inverse, and the layer-loss product
// D H.  Tiles are 128 x 128 per 256-thread workgroup (4 wave64s, each 64 x 64
// as 2 x 2 v_mfma_f32_32x32x2f32 tiles), K staged through LDS in slabs of
// 32, double buffered, one barrier per slab.  Operands are stored K-major in
// LDS so both matrix-core operands are read as consecutive 4-byte words.
#include "common.h"

namespace gptq {
namespace {

constexpr int BM = kGemmTile, BN = kGemmTile, BK = 32;
constexpr int LDS_LD = BM + 4;  // floats per LDS row (keeps float4 alignment)
constexpr int kThreads = 256;

struct GemmSmem {
    float a[2][BK][LDS_LD];
    float b[2][BK][LDS_LD];
};

// Loads one 128 x 32 (A) or 32 x 128 (B) slab into registers: 4 float4 per thread.
// `kmajor_src` == 1: the source is contiguous along the 128-wide dimension
// (A with a_trans, B without b_trans); 0: contiguous along K.
struct SlabLoader {
    const float *p;
    int64_t ld;
    int64_t wide0, wide_lim;  // first row/col of the tile along the 128-wide dim, bound
    int kmajor_src;
    int vec;  // float4 loads allowed (alignment)

    __device__ __forceinline__ void load(int64_t k0, int64_t klim, int tid, float4 (&r)[4]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + kThreads * i;
            int64_t w, k;
            if (kmajor_src) {
                k = idx >> 5;
                w = (idx & 31) * 4;
            } else {
                w = idx >> 3;
                k = (idx & 7) * 4;
            }
            const int64_t gw = wide0 + w, gk = k0 + k;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (kmajor_src) {
                const float *src = p + gk * ld + gw;
                if (gk < klim) {
                    if (vec && gw + 3 < wide_lim) {
                        v = *reinterpret_cast<const float4 *>(src);
                    } else {
                        if (gw + 0 < wide_lim) v.x = src[0];
                        if (gw + 1 < wide_lim) v.y = src[1];
                        if (gw + 2 < wide_lim) v.z = src[2];
                        if (gw + 3 < wide_lim) v.w = src[3];
                    }
                }
            } else {
                const float *src = p + gw * ld + gk;
                if (gw < wide_lim) {
                    if (vec && gk + 3 < klim) {
                        v = *reinterpret_cast<const float4 *>(src);
                    } else {
                        if (gk + 0 < klim) v.x = src[0];
                        if (gk + 1 < klim) v.y = src[1];
                        if (gk + 2 < klim) v.z = src[2];
                        if (gk + 3 < klim) v.w = src[3];
                    }
                }
            }
            r[i] = v;
        }
    }

    // Writes the registers into an LDS slab laid out [k][wide].
    __device__ __forceinline__ void store(float (*s)[LDS_LD], int tid, const float4 (&r)[4]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + kThreads * i;
            if (kmajor_src) {
                const int k = idx >> 5, w = (idx & 31) * 4;
                *reinterpret_cast<float4 *>(&s[k][w]) = r[i];
            } else {
                const int w = idx >> 3, k = (idx & 7) * 4;
                s[k + 0][w] = r[i].x;
                s[k + 1][w] = r[i].y;
                s[k + 2][w] = r[i].z;
                s[k + 3][w] = r[i].w;
            }
        }
    }
};

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmDesc g, int vec_a, int vec_b) {
    const int tn = blockIdx.x, tm = blockIdx.y, bz = blockIdx.z;
    if (g.upper_only && tm > tn) return;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const float *A = g.A + bz * g.strideA;
    const float *B = g.B + bz * g.strideB;
    float *C = g.C + bz * g.strideC;

    int64_t kbeg = 0, kend = g.K;
    if (g.a_upper) kbeg = m0 < kbeg ? kbeg : m0;
    if (g.b_upper) kend = (n0 + BN) < kend ? (n0 + BN) : kend;
    kbeg = (kbeg / BK) * BK;

    __shared__ GemmSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    SlabLoader la{A, g.lda, m0, g.M, g.a_trans, vec_a};
    SlabLoader lb{B, g.ldb, n0, g.N, g.b_trans ? 0 : 1, vec_b};

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // C values are fetched before the K loop so their latency hides behind the
    // matrix-core work; every store comes after every load of the tile.
    float cold[2][2][16];
    if (EPI == EPI_STORE && g.beta != 0.0f) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * 64 + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * 64 + j * 32 + mfma32_col(lane);
                    cold[i][j][r] = (m < g.M && n < g.N) ? C[m * g.ldc + n] : 0.0f;
                }
    }

    if (kbeg < kend) {
        float4 ra[4], rb[4];
        la.load(kbeg, kend, tid, ra);
        lb.load(kbeg, kend, tid, rb);
        la.store(sm.a[0], tid, ra);
        lb.store(sm.b[0], tid, rb);
        __syncthreads();
        int buf = 0;
        for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
            const bool more = k0 + BK < kend;
            if (more) {
                la.load(k0 + BK, kend, tid, ra);
                lb.load(k0 + BK, kend, tid, rb);
            }
            const int kr = lane >> 5, c = lane & 31;
#pragma unroll
            for (int kk = 0; kk < BK; kk += 2) {
                const float a0 = sm.a[buf][kk + kr][wm * 64 + c];
                const float a1 = sm.a[buf][kk + kr][wm * 64 + 32 + c];
                const float b0 = sm.b[buf][kk + kr][wn * 64 + c];
                const float b1 = sm.b[buf][kk + kr][wn * 64 + 32 + c];
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
            }
            if (more) {
                la.store(sm.a[buf ^ 1], tid, ra);
                lb.store(sm.b[buf ^ 1], tid, rb);
            }
            __syncthreads();
            buf ^= 1;
        }
    }

    if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * 64 + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * 64 + j * 32 + mfma32_col(lane);
                    if (m < g.M && n < g.N && (!g.upper_only || m <= n)) {
                        float v = g.alpha * acc[i][j][r];
                        if (g.beta != 0.0f) v += g.beta * cold[i][j][r];
                        C[m * g.ldc + n] = v;
                    }
                }
    } else {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * 64 + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * 64 + j * 32 + mfma32_col(lane);
                    if (m < g.M && n < g.N) s += (double)acc[i][j][r] * (double)g.Dm[m * g.ldd + n];
                }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        __shared__ double red[kThreads / kWave];
        if (lane == 0) red[wave] = s;
        __syncthreads();
        if (tid == 0) {
            double t = 0.0;
            for (int w = 0; w < kThreads / kWave; ++w) t += red[w];
            g.partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = t;
        }
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

int64_t gemm_num_tiles(const GemmDesc &g) { return ceil_div(g.M, BM) * ceil_div(g.N, BN); }

hipError_t launch_gemm_f32(const GemmDesc &g, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
    const bool bz = g.batch > 1;
    const int vec_a = aligned16(g.A) && g.lda % 4 == 0 && (!bz || g.strideA % 4 == 0);
    const int vec_b = aligned16(g.B) && g.ldb % 4 == 0 && (!bz || g.strideB % 4 == 0);
    dim3 grid((unsigned)ceil_div(g.N, BN), (unsigned)ceil_div(g.M, BM), (unsigned)g.batch);
    if (g.epilogue == EPI_DOT)
        hipLaunchKernelGGL(gemm_f32_kernel<EPI_DOT>, grid, dim3(kThreads), 0, s, g, vec_a, vec_b);
    else
        hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, dim3(kThreads), 0, s, g, vec_a, vec_b);
    return hipGetLastError();
}

}  // namespace gptq
