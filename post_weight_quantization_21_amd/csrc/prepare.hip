// Steps 2-3 of GPTQ: column order, damping and U = upper Cholesky factor of
// H_d^-1 (U^T U = H_d^-1).
//
// The column pass needs, for every column j, row j of the inverse Hessian of
// the columns not yet quantized (page "PTQ 权重量化：从 GPTQ 到 AWQ", GPTQ
// section).  Those rows, scaled by their diagonal's square root, are the rows
// of U.  Route (2/3 d^3 flops, fp32):
//   1. H_d = P H P^T + lambda I           (gather + one-workgroup damping)
//   2. UL-Cholesky H_d = T T^T, T upper   (blocked, from the bottom-right
//      corner: panel factor on one workgroup, panel solve and symmetric
//      rank-k update of the rest on matrix cores)
//   3. U = T^-1                           (the panel kernel also inverts each
//      diagonal block; off-diagonal blocks are merged pairwise by the block
//      formula inv([[A, B], [0, C]]) = [[A^-1, -A^-1 B C^-1], [0, C^-1]],
//      one batched matrix-core product pair per level.)
// Indeed T T^T = H_d gives H_d^-1 = T^-T T^-1 = U^T U with U = T^-1 upper.
#include "common.h"

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

__global__ __launch_bounds__(kThreads) void order_kernel(const double *__restrict__ hdiag, const float *__restrict__ H,
                                                         int64_t d, int32_t *__restrict__ perm) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= d) return;
    const double ki = order_key(hdiag, H, d, i);
    int64_t rank = 0;
    for (int64_t j = 0; j < d; ++j) {
        const double kj = order_key(hdiag, H, d, j);
        rank += (kj > ki) || (kj == ki && j < i);
    }
    perm[rank] = (int32_t)i;
}

// A[a][b] = H[pa][pb] for a <= b (upper triangle of P H P^T), from H's upper triangle.
__global__ __launch_bounds__(kThreads) void gather_sym_kernel(const float *__restrict__ H, const int32_t *__restrict__ perm,
                                                              int64_t d, float *__restrict__ A) {
    const int64_t a = blockIdx.y;
    for (int64_t b = a + (int64_t)blockIdx.x * kThreads + threadIdx.x; b < d; b += (int64_t)gridDim.x * kThreads) {
        int64_t pa = perm ? min(max((int64_t)perm[a], (int64_t)0), d - 1) : a;
        int64_t pb = perm ? min(max((int64_t)perm[b], (int64_t)0), d - 1) : b;
        if (pa > pb) {
            int64_t t = pa;
            pa = pb;
            pb = t;
        }
        A[a * d + b] = H[pa * d + pb];
    }
}

// lambda = damp_rel * mean(diag A) (fp64, fixed tree); A[i][i] += lambda.  One workgroup.
__global__ __launch_bounds__(kThreads) void damp_kernel(float *__restrict__ A, int64_t d, float damp_rel) {
    __shared__ double red[kThreads];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < d; i += kThreads) s += (double)A[i * d + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    const float lam = (float)((double)damp_rel * red[0] / (double)d);
    for (int64_t i = threadIdx.x; i < d; i += kThreads) A[i * d + i] += lam;
}

__global__ __launch_bounds__(kThreads) void fill_kernel(float *__restrict__ p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) p[i] = v;
}

__global__ void zero_int_kernel(int32_t *p) { *p = 0; }

__global__ __launch_bounds__(kThreads) void iota_kernel(int32_t *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) p[i] = (int32_t)i;
}

// UL-Cholesky of the diagonal block A[k0:k0+nb, k0:k0+nb] (upper storage) and
// the inverse of its factor, on one wave64 with no block barriers.
//   factor:  lane i holds row i of the block in registers.  For j = NB-1..0:
//            t_jj = sqrt(c_jj);  t_ij = c_ij / t_jj (i < j);
//            c_ii' -= t_ij t_i'j (i' < j)  -- column j is shared through LDS.
//   inverse: lane c holds column c of V = T^-1.  For i = NB-1..0:
//            V_ic = -(1/t_ii) sum_{m>i} t_im V_mc (c > i), V_ii = 1/t_ii,
//            reading row i of T from LDS with wave-uniform addresses.
// Rows and columns past nb are padded with the identity.  Writes T into A's block and V into U's block (strictly
// lower parts = 0).
__global__ __launch_bounds__(kWave) void panel_kernel(float *__restrict__ A, float *__restrict__ U, int64_t d,
                                                      int64_t k0, int nb, int32_t *__restrict__ info) {
    __shared__ float col[NB];
    __shared__ float tr[NB][NB + 4];
    const int lane = threadIdx.x;
    // Block into LDS: all loads in flight at once, identity padding past nb.
    {
        float ld[NB];
#pragma unroll
        for (int it = 0; it < NB; ++it) {
            const bool in = it < nb && lane < nb;
            ld[it] = in ? (it <= lane ? A[(k0 + it) * d + k0 + lane] : 0.0f) : (it == lane ? 1.0f : 0.0f);
        }
#pragma unroll
        for (int it = 0; it < NB; ++it) tr[it][lane] = ld[it];
    }
    __syncthreads();
    float c[NB];
#pragma unroll
    for (int m = 0; m < NB; ++m) c[m] = tr[lane][m];
    int32_t first_bad = 0;
#pragma unroll
    for (int j = NB - 1; j >= 0; --j) {
        const float p0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c[j]), j));  // pivot, from lane j
        const bool bad = !(p0 > 0.0f);
        first_bad = (bad && first_bad == 0 && j < nb) ? (int32_t)(k0 + j + 1) : first_bad;
        // hardware sqrt / reciprocal (about 1 ulp): the factor only has to be
        // accurate; branch-free selects keep the wave on one path.
        const float tjj = __builtin_amdgcn_sqrtf(bad ? 1.0f : p0);
        const float inv = __builtin_amdgcn_rcpf(tjj);
        float t = c[j] * inv;
        t = lane == j ? tjj : t;
        t = lane > j ? 0.0f : t;
        c[j] = t;
        if (j == 0) break;
        col[lane] = t;  // column j of the factor, shared through LDS
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i2 = 0; i2 < j; ++i2) c[i2] = fmaf(-t, col[i2], c[i2]);
        __builtin_amdgcn_wave_barrier();
    }
    if (first_bad != 0 && lane == 0) atomicCAS(info, 0, first_bad);
    // T rows (upper part) to LDS for the inverse and the coalesced store into A.
#pragma unroll
    for (int m = 0; m < NB; ++m) tr[lane][m] = m >= lane ? c[m] : 0.0f;
    __syncthreads();
    for (int e = lane; e < nb * NB; e += kWave) {
        const int i = e / NB, m = e % NB;
        if (m < nb && m >= i) A[(k0 + i) * d + k0 + m] = tr[i][m];
    }
    float v[NB];
#pragma unroll
    for (int i = NB - 1; i >= 0; --i) {
        const float rii = __builtin_amdgcn_rcpf(tr[i][i]);
        float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
        for (int m = i + 1; m < NB; ++m) {
            const float prod = tr[i][m] * v[m];
            if ((m & 3) == 0) s0 += prod;
            else if ((m & 3) == 1) s1 += prod;
            else if ((m & 3) == 2) s2 += prod;
            else s3 += prod;
        }
        float x = -rii * ((s0 + s1) + (s2 + s3));
        x = lane == i ? rii : x;
        v[i] = lane < i ? 0.0f : x;
    }
    __syncthreads();
    // Column `lane` of V into LDS, then coalesced rows into U (zero below the diagonal).
#pragma unroll
    for (int m = 0; m < NB; ++m) tr[m][lane] = v[m];
    __syncthreads();
    for (int e = lane; e < nb * NB; e += kWave) {
        const int i = e / NB, m = e % NB;
        if (m < nb) U[(k0 + i) * d + k0 + m] = tr[i][m];
    }
}

hipError_t merge_level(float *A, float *U, float *T, int64_t d, int64_t s, int64_t p_first, int64_t npairs,
                       int64_t ni, int64_t nj, hipStream_t st) {
    // pairs p_first .. p_first+npairs-1 of size (ni rows, nj cols): i0 = 2ps, j0 = i0 + ni.
    const int64_t i0 = 2 * p_first * s, j0 = i0 + ni;
    const int64_t stride = 2 * s * (d + 1);
    GemmDesc g;
    g.batch = (int)npairs;
    g.M = ni;
    g.N = nj;
    g.K = ni;
    g.A = U + i0 * d + i0;  // U11 (upper triangular, lower part zero)
    g.lda = d;
    g.a_upper = 1;
    g.B = A + i0 * d + j0;  // T12
    g.ldb = d;
    g.C = T + i0 * d + j0;
    g.ldc = d;
    g.strideA = g.strideB = g.strideC = stride;
    hipError_t e = launch_gemm_f32(g, st);
    if (e != hipSuccess) return e;
    GemmDesc h;
    h.batch = (int)npairs;
    h.M = ni;
    h.N = nj;
    h.K = nj;
    h.A = T + i0 * d + j0;
    h.lda = d;
    h.B = U + j0 * d + j0;  // U22 (upper triangular)
    h.ldb = d;
    h.b_upper = 1;
    h.C = U + i0 * d + j0;
    h.ldc = d;
    h.alpha = -1.0f;
    h.beta = 0.0f;
    h.strideA = h.strideB = h.strideC = stride;
    return launch_gemm_f32(h, st);
}

}  // namespace

size_t prepare_ws_bytes(int64_t d) { return 2 * align_up((size_t)d * (size_t)d * sizeof(float), 256); }

hipError_t run_prepare(const float *H, const double *hdiag, int64_t d, float damp_rel, int act_order, float *U,
                       int32_t *perm, int32_t *info, void *ws, hipStream_t s) {
    float *A = static_cast<float *>(ws);
    float *T = reinterpret_cast<float *>(static_cast<char *>(ws) + align_up((size_t)d * d * sizeof(float), 256));
    hipError_t e;
    hipLaunchKernelGGL(zero_int_kernel, dim3(1), dim3(1), 0, s, info);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (act_order) {
        hipLaunchKernelGGL(order_kernel, dim3((unsigned)ceil_div(d, kThreads)), dim3(kThreads), 0, s, hdiag, H, d, perm);
    } else if (perm) {
        hipLaunchKernelGGL(iota_kernel, dim3((unsigned)ceil_div(d, kThreads)), dim3(kThreads), 0, s, perm, d);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned gx = (unsigned)((d + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(gather_sym_kernel, dim3(gx, (unsigned)d), dim3(kThreads), 0, s, H, act_order ? perm : nullptr,
                       d, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(kThreads), 0, s, A, d, damp_rel);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nU = d * d;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(nU, kThreads), 65536)), dim3(kThreads), 0, s,
                       U, nU, 0.0f);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const int64_t nblk = ceil_div(d, NB);
    for (int64_t kb = nblk - 1; kb >= 0; --kb) {
        const int64_t k0 = kb * NB;
        const int nb = (int)std::min<int64_t>(NB, d - k0);
        hipLaunchKernelGGL(panel_kernel, dim3(1), dim3(kWave), 0, s, A, U, d, k0, nb, info);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (k0 == 0) break;
        // Panel solve: A[0:k0, k0:k0+nb] <- A[0:k0, k0:k0+nb] V^T  (V = T_kk^-1 in U's block)
        GemmDesc g;
        g.M = k0;
        g.N = nb;
        g.K = nb;
        g.A = A + k0;
        g.lda = d;
        g.B = U + k0 * d + k0;
        g.ldb = d;
        g.b_trans = 1;
        g.C = A + k0;
        g.ldc = d;
        g.alpha = 1.0f;
        g.beta = 0.0f;
        if ((e = launch_gemm_f32(g, s)) != hipSuccess) return e;
        // Rank-nb update of the leading block: A[0:k0, 0:k0] -= P P^T (upper).
        GemmDesc h;
        h.M = k0;
        h.N = k0;
        h.K = nb;
        h.A = A + k0;
        h.lda = d;
        h.B = A + k0;
        h.ldb = d;
        h.b_trans = 1;
        h.C = A;
        h.ldc = d;
        h.alpha = -1.0f;
        h.beta = 1.0f;
        h.upper_only = 1;
        if ((e = launch_gemm_f32(h, s)) != hipSuccess) return e;
    }
    // Pairwise merges of the inverted diagonal blocks.
    for (int64_t sz = NB; sz < d; sz *= 2) {
        const int64_t npairs_total = ceil_div(d, 2 * sz);
        int64_t full = d / (2 * sz);
        if (full > 0) {
            if ((e = merge_level(A, U, T, d, sz, 0, full, sz, sz, s)) != hipSuccess) return e;
        }
        if (npairs_total > full) {
            const int64_t i0 = 2 * full * sz;
            const int64_t ni = std::min<int64_t>(sz, d - i0);
            const int64_t nj = d - i0 - ni;
            if (nj > 0)
                if ((e = merge_level(A, U, T, d, sz, full, 1, ni, nj, s)) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace gptq
