// Lazy batch update of GPTQ on fp32 matrix cores (page "PTQ 权重量化：从 GPTQ
// 到 AWQ", GPTQ section: the batch's errors are applied to the later columns
// once per batch of 128 columns; page "量化经典：LLM.int8 / GPTQ / AWQ", §二
// step 4):
//
//     W[:, c1:] += (-E) U[c0:c1, c1:]        (K = c1 - c0 <= 128)
//
// Each workgroup owns 128 rows of W and walks a run of 128-column tiles.  The
// -E block of its rows (K x 128) is loaded into LDS once; U is streamed in
// slabs of 32 rows, double buffered through registers, and the pipeline runs
// on across tile boundaries.  The matrix-core products are formed transposed
// (D[n][m] = sum_k U[k][n] (-E)[k][m]) so that each lane's accumulators hold
// four consecutive columns of one row: W is read and written as float4, and
// a tile's W values are fetched when the tile starts, a whole K loop before
// they are needed.
#include "common.h"

namespace gptq {
namespace {

constexpr int TM = 128, TN = 128, BK = 32, KMAX = 128, LDP = 132;
constexpr int kThreads = 256;

struct TrailSmem {
    float es[KMAX][LDP];    // (-E)^T block: es[k][i] = Et[k][m0 + i]
    float bs[2][BK][LDP];   // U slab: bs[k][j] = U[k0 + k][n0 + j]
};

struct TrailArgs {
    float *W;         // W + c1: the first trailing column
    int64_t ldw, M, N;
    const float *Et;  // [K][ldet]
    int64_t ldet;
    int K;
    const float *Ub;  // U + c0 * ldu + c1
    int64_t ldu;
    int ncg;          // column groups per row block
    int vec;          // float4 access to W and U allowed
};

__device__ __forceinline__ void load_u(const TrailArgs &a, int64_t n0, int k0, int tid, float4 (&r)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + kThreads * i;
        const int k = idx >> 5, j = (idx & 31) * 4;
        const int64_t gk = k0 + k, gn = n0 + j;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gk < a.K) {
            const float *src = a.Ub + gk * a.ldu + gn;
            if (a.vec && gn + 3 < a.N) {
                v = *reinterpret_cast<const float4 *>(src);
            } else {
                if (gn + 0 < a.N) v.x = src[0];
                if (gn + 1 < a.N) v.y = src[1];
                if (gn + 2 < a.N) v.z = src[2];
                if (gn + 3 < a.N) v.w = src[3];
            }
        }
        r[i] = v;
    }
}

__device__ __forceinline__ void store_u(float (*s)[LDP], int tid, const float4 (&r)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + kThreads * i;
        const int k = idx >> 5, j = (idx & 31) * 4;
        *reinterpret_cast<float4 *>(&s[k][j]) = r[i];
    }
}

__global__ __launch_bounds__(kThreads) void trailing_kernel(TrailArgs a) {
    const int64_t rb = blockIdx.x / a.ncg;
    const int cg = blockIdx.x % a.ncg;
    const int64_t m0 = rb * TM;
    const int64_t ntn = ceil_div(a.N, TN);
    const int64_t per = ceil_div(ntn, a.ncg);
    const int64_t t_beg = cg * per;
    const int64_t t_end = (t_beg + per) < ntn ? (t_beg + per) : ntn;
    if (t_beg >= t_end) return;

    __shared__ TrailSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int nst = (a.K + BK - 1) / BK;

    // (-E)^T block of this row block, rows past K zeroed.  Et is padded to
    // whole workgroups of rows, so m0 + 127 < ldet.  All sixteen loads of a
    // thread are issued before the first LDS store.
    {
        constexpr int kPer = KMAX * TM / 4 / kThreads;
        float4 ev[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e4 = tid + q * kThreads;
            const int k = e4 / (TM / 4), i = (e4 % (TM / 4)) * 4;
            ev[q] = k < a.K ? *reinterpret_cast<const float4 *>(a.Et + (int64_t)k * a.ldet + m0 + i)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
            const int e4 = tid + q * kThreads;
            const int k = e4 / (TM / 4), i = (e4 % (TM / 4)) * 4;
            *reinterpret_cast<float4 *>(&sm.es[k][i]) = ev[q];
        }
    }

    float4 ru[4];
    load_u(a, t_beg * TN, 0, tid, ru);
    store_u(sm.bs[0], tid, ru);
    __syncthreads();
    int buf = 0;
    const int kr = lane >> 5, c = lane & 31;

    for (int64_t t = t_beg; t < t_end; ++t) {
        const int64_t n0 = t * TN;
        // W values of this tile, in the accumulator layout: lane holds, for each
        // 32x32 block (ni, mi) and g = 0..3, W[m][n .. n+3] with
        // m = m0 + wm*64 + mi*32 + (lane % 32), n = n0 + wn*64 + ni*32 + 8g + 4*(lane/32).
        // They are requested right after the first U slab load of the tile, so
        // waiting for that slab never waits for them (memory counters retire in order).
        float4 cw[2][2][4];
        auto load_c = [&]() {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int64_t m = m0 + wm * 64 + mi * 32 + c;
                        const int64_t n = n0 + wn * 64 + ni * 32 + 8 * g + 4 * kr;
                        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                        if (m < a.M) {
                            const float *src = a.W + m * a.ldw + n;
                            if (a.vec && n + 3 < a.N) {
                                v = *reinterpret_cast<const float4 *>(src);
                            } else {
                                if (n + 0 < a.N) v.x = src[0];
                                if (n + 1 < a.N) v.y = src[1];
                                if (n + 2 < a.N) v.z = src[2];
                                if (n + 3 < a.N) v.w = src[3];
                            }
                        }
                        cw[ni][mi][g] = v;
                    }
        };
        floatx16 acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        for (int s = 0; s < nst; ++s) {
            // next slab: the following K slab of this tile, or the first of the next tile
            const bool more = (s + 1 < nst) || (t + 1 < t_end);
            if (more) {
                if (s + 1 < nst)
                    load_u(a, n0, (s + 1) * BK, tid, ru);
                else
                    load_u(a, n0 + TN, 0, tid, ru);
            }
            if (s == 0) load_c();
#pragma unroll
            for (int kk = 0; kk < BK; kk += 2) {
                const float u0 = sm.bs[buf][kk + kr][wn * 64 + c];
                const float u1 = sm.bs[buf][kk + kr][wn * 64 + 32 + c];
                const float e0 = sm.es[s * BK + kk + kr][wm * 64 + c];
                const float e1 = sm.es[s * BK + kk + kr][wm * 64 + 32 + c];
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(u0, e0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(u0, e1, acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(u1, e0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(u1, e1, acc[1][1], 0, 0, 0);
            }
            if (more) store_u(sm.bs[buf ^ 1], tid, ru);
            __syncthreads();
            buf ^= 1;
        }

#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t m = m0 + wm * 64 + mi * 32 + c;
                    const int64_t n = n0 + wn * 64 + ni * 32 + 8 * g + 4 * kr;
                    if (m >= a.M) continue;
                    float4 v = cw[ni][mi][g];
                    v.x += acc[ni][mi][4 * g + 0];
                    v.y += acc[ni][mi][4 * g + 1];
                    v.z += acc[ni][mi][4 * g + 2];
                    v.w += acc[ni][mi][4 * g + 3];
                    float *dst = a.W + m * a.ldw + n;
                    if (a.vec && n + 3 < a.N) {
                        *reinterpret_cast<float4 *>(dst) = v;
                    } else {
                        if (n + 0 < a.N) dst[0] = v.x;
                        if (n + 1 < a.N) dst[1] = v.y;
                        if (n + 2 < a.N) dst[2] = v.z;
                        if (n + 3 < a.N) dst[3] = v.w;
                    }
                }
    }
}

}  // namespace

hipError_t launch_trailing_update(float *W, int64_t ldw, int64_t M, int64_t N, const float *Et, int64_t ldet, int K,
                                  const float *Ub, int64_t ldu, hipStream_t s) {
    if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
    if (K > KMAX || ldet < ceil_div(M, TM) * TM) return hipErrorInvalidValue;
    TrailArgs a;
    a.W = W;
    a.ldw = ldw;
    a.M = M;
    a.N = N;
    a.Et = Et;
    a.ldet = ldet;
    a.K = K;
    a.Ub = Ub;
    a.ldu = ldu;
    const int64_t nrb = ceil_div(M, TM), ntn = ceil_div(N, TN);
    int64_t ncg = 256 / nrb;
    if (ncg < 1) ncg = 1;
    if (ncg > ntn) ncg = ntn;
    a.ncg = (int)ncg;
    const auto al = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    a.vec = al(W) && al(Ub) && ldw % 4 == 0 && ldu % 4 == 0;
    if (!al(Et) || ldet % 4 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(trailing_kernel, dim3((unsigned)(nrb * ncg)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gptq
