// fp32 matrix-core GEMM for gfx950:  C = alpha * op(A) op(B) + beta * C.
//
// One kernel serves every dense fp32 contraction of the library: the lazy
// batch update of GPTQ (W[:, trail] -= E U[block, trail]), the triangular
// products of the triangular inverse, and the layer-loss product D H.
// Tiles are T x T per 256-thread workgroup (4 wave64s in 2 x 2, each
// T/2 x T/2 as v_mfma_f32_32x32x2f32 blocks), T = 128, or T = 64 when a
// launch has too few 128-wide tiles to fill the chip (a quarter of the
// dependent matrix-core chain per wave).  K is staged through LDS in slabs of
// 32, double buffered through registers, one barrier per slab.  Operands are
// stored K-major in LDS so both matrix-core operands are read as consecutive
// 4-byte words; each k-step's operands are read one step ahead of its MFMAs.
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int BK = 32;
constexpr int kThreads = 256;

template <int T>
struct GemmSmem {
    float a[2][BK][T + 4];  // rows of T + 4 floats keep float4 alignment
    float b[2][BK][T + 4];
};

// Loads one T x 32 (A) or 32 x T (B) slab into registers: T/32 float4 per thread.
// `kmajor_src` == 1: the source is contiguous along the T-wide dimension
// (A with a_trans, B without b_trans); 0: contiguous along K.
// VEC: every 16-byte chunk is aligned and lies either wholly inside or
// wholly outside the matrix (the contiguous extent and the leading dimension
// are multiples of 4), so the loads are unconditional 16-byte loads from
// clamped addresses, zeroed afterwards when out of range: no branches, so all
// of them stay in flight together.  Otherwise element-wise guarded loads.
template <int T, int VEC>
struct SlabLoader {
    static constexpr int kPer = T * BK / 4 / kThreads;  // float4 per thread
    static constexpr int kWideChunks = T / 4;           // float4 per K row (k-major source)
    const float *p;
    int64_t ld;
    int64_t wide0, wide_lim;  // first row/col of the tile along the T-wide dim, bound
    int kmajor_src;

    __device__ __forceinline__ void load(int64_t k0, int64_t klim, int tid, float4 (&r)[kPer]) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int idx = tid + kThreads * i;
            int64_t w, k;
            if (kmajor_src) {
                k = idx / kWideChunks;
                w = (idx % kWideChunks) * 4;
            } else {
                w = idx >> 3;
                k = (idx & 7) * 4;
            }
            const int64_t gw = wide0 + w, gk = k0 + k;
            if constexpr (VEC) {
                const bool in = gk < klim && gw < wide_lim;
                const int64_t ck = in ? gk : 0, cw = in ? gw : 0;
                const float4 v = *reinterpret_cast<const float4 *>(kmajor_src ? p + ck * ld + cw : p + cw * ld + ck);
                r[i] = in ? v : make_float4(0.f, 0.f, 0.f, 0.f);
            } else {
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (kmajor_src) {
                    const float *src = p + gk * ld + gw;
                    if (gk < klim) {
                        if (gw + 0 < wide_lim) v.x = src[0];
                        if (gw + 1 < wide_lim) v.y = src[1];
                        if (gw + 2 < wide_lim) v.z = src[2];
                        if (gw + 3 < wide_lim) v.w = src[3];
                    }
                } else {
                    const float *src = p + gw * ld + gk;
                    if (gw < wide_lim) {
                        if (gk + 0 < klim) v.x = src[0];
                        if (gk + 1 < klim) v.y = src[1];
                        if (gk + 2 < klim) v.z = src[2];
                        if (gk + 3 < klim) v.w = src[3];
                    }
                }
                r[i] = v;
            }
        }
    }

    // Writes the registers into an LDS slab laid out [k][wide].
    __device__ __forceinline__ void store(float (*s)[T + 4], int tid, const float4 (&r)[kPer]) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int idx = tid + kThreads * i;
            if (kmajor_src) {
                const int k = idx / kWideChunks, w = (idx % kWideChunks) * 4;
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

// One T x T tile of C (tile row tm, column tn, batch bz); `pidx` indexes the
// partial sum of EPI_DOT.
template <int EPI, int VA, int VB, int T>
__device__ __forceinline__ void gemm_f32_tile(const GemmDesc &g, int tm, int tn, int bz, int64_t pidx) {
    constexpr int QB = T / 64;  // 32x32 MFMA blocks per wave along each dimension
    constexpr int HW = T / 2;   // wave tile edge
    if (g.upper_only && tm > tn) return;  // strictly below the diagonal: nothing to store
    const int64_t m0 = (int64_t)tm * T, n0 = (int64_t)tn * T;

    const float *A = g.A + bz * g.strideA;
    const float *B = g.B + bz * g.strideB;
    float *C = g.C + bz * g.strideC;

    int64_t kbeg = 0, kend = g.K;
    if (g.a_upper) kbeg = m0 < kbeg ? kbeg : m0;
    if (g.b_upper) kend = (n0 + T) < kend ? (n0 + T) : kend;
    kbeg = (kbeg / BK) * BK;

    __shared__ GemmSmem<T> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    SlabLoader<T, VA> la{A, g.lda, m0, g.M, g.a_trans};
    SlabLoader<T, VB> lb{B, g.ldb, n0, g.N, g.b_trans ? 0 : 1};
    constexpr int kPer = SlabLoader<T, VA>::kPer;

    floatx16 acc[QB][QB];
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int j = 0; j < QB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // C values are fetched before the K loop so their latency hides behind the
    // matrix-core work; every store comes after every load of the tile.
    float cold[QB][QB][16];
    if (EPI == EPI_STORE && g.beta != 0.0f) {
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < QB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * HW + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * HW + j * 32 + mfma32_col(lane);
                    cold[i][j][r] = (m < g.M && n < g.N) ? C[m * g.ldc + n] : 0.0f;
                }
    }

    if (kbeg < kend) {
        float4 ra[kPer], rb[kPer];
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
            // Operands of k-step kk (A blocks, then B blocks); the next step's
            // are read from LDS while this step's MFMAs run (the scheduling
            // fences keep that order).
            float op[2][2 * QB];
            auto rd = [&](int kk, float(&o)[2 * QB]) {
#pragma unroll
                for (int i = 0; i < QB; ++i) o[i] = sm.a[buf][kk + kr][wm * HW + i * 32 + c];
#pragma unroll
                for (int j = 0; j < QB; ++j) o[QB + j] = sm.b[buf][kk + kr][wn * HW + j * 32 + c];
            };
            rd(0, op[0]);
#pragma unroll
            for (int kk = 0; kk < BK; kk += 2) {
                const int cur = (kk >> 1) & 1;
                if (kk + 2 < BK) rd(kk + 2, op[cur ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < QB; ++i)
#pragma unroll
                    for (int j = 0; j < QB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(op[cur][i], op[cur][QB + j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
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
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < QB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * HW + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * HW + j * 32 + mfma32_col(lane);
                    if (m < g.M && n < g.N && (!g.upper_only || m <= n)) {
                        float v = g.alpha * acc[i][j][r];
                        if (g.beta != 0.0f) v += g.beta * cold[i][j][r];
                        C[m * g.ldc + n] = v;
                    }
                }
    } else {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < QB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * HW + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * HW + j * 32 + mfma32_col(lane);
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
            g.partial[pidx] = t;
        }
    }
}

// Tile order of a launch: row-major over the tiles; with B upper triangular the
// tiles of the last columns have the longest K, so they are dispatched first,
// column by column over every row of tiles, and the launch does not end on long
// tiles (with A upper, the first rows are the longest, and they already come first).
__device__ __forceinline__ void tile_of(const GemmDesc &g, int64_t id, int gx, int gy, int &tm, int &tn, int &bz) {
    const int64_t per = (int64_t)gx * gy;
    bz = (int)(id / per);
    const int r = (int)(id - (int64_t)bz * per);
    if (g.b_upper) {
        tn = gx - 1 - r / gy;
        tm = r % gy;
    } else {
        tm = r / gx;
        tn = r % gx;
    }
}

// One tile per workgroup (grid gx x gy x batch), or with max_wgs a persistent
// grid of max_wgs workgroups that takes the tiles in the same order.
template <int EPI, int VA, int VB, int T>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmDesc g) {
    const int gx = (int)ceil_div(g.N, T), gy = (int)ceil_div(g.M, T);
    int tm, tn, bz;
    if (g.max_wgs <= 0) {
        const int64_t id = (int64_t)blockIdx.z * gx * gy + (int64_t)blockIdx.y * gx + blockIdx.x;
        tile_of(g, id, gx, gy, tm, tn, bz);
        gemm_f32_tile<EPI, VA, VB, T>(g, tm, tn, bz, (int64_t)blockIdx.y * gridDim.x + blockIdx.x);
        return;
    }
    const int64_t total = (int64_t)gx * gy * g.batch;
    for (int64_t id = blockIdx.x; id < total; id += gridDim.x) {
        if (id != blockIdx.x) __syncthreads();  // the previous tile's LDS reads are done
        tile_of(g, id, gx, gy, tm, tn, bz);
        gemm_f32_tile<EPI, VA, VB, T>(g, tm, tn, bz, id);
    }
}

// The same product with K streamed straight from global memory into a ring of
// LDS stages (global_load_lds_dwordx4), three 16-deep stages ahead of the
// matrix cores: no staging registers, one barrier per stage; 128 x 128 tiles.
// Each operand is either K-major (stored [k][wide]: A with a_trans, B without
// b_trans) or K-contiguous (stored [wide][k]).  Needs 16-byte aligned
// operands, leading dimensions that are multiples of 4, K-major wide extents
// that are multiples of 4, and K (after the triangular trims, which start and
// end at multiples of the tile) a multiple of 16.
//
// Stage layouts (8 KB per operand):
//   K-major      [16 k][128 wide]; the 16-byte chunk of wide columns 4c .. 4c+3
//                of row k sits at position c ^ (8 (k & 1)), so the two k rows
//                one operand read touches (lanes 0-31 and 32-63) fall in
//                complementary halves of the 64 LDS banks;
//   K-contiguous [128 wide][16 k]; the chunk of k values 4c .. 4c+3 of row r
//                sits at position c ^ ((r / 4) % 4), so one operand read (32
//                rows at two k) takes two LDS cycles.
constexpr int LKS = 16;  // K per stage
constexpr int LNS = 4;   // stages in the ring
constexpr int LT = 128;  // tile edge

struct LdsGemmSmem {
    float a[LNS][LKS * LT];
    float b[LNS][LKS * LT];
};

// LDS index of (k, w) in a stage (w: wide index in the tile).
template <int KM>
__device__ __forceinline__ int lds_index(int k, int w) {
    if constexpr (KM)
        return k * LT + ((((w >> 2) ^ ((k & 1) << 3)) << 2) | (w & 3));
    else
        return w * LKS + ((((k >> 2) ^ ((w >> 2) & 3)) << 2) | (k & 3));
}

// Wave `wave` loads its quarter of one operand's stage in two instructions of
// 1 KB.  Wide rows/columns past `wide_lim` read the tile's first one instead
// (valid memory; the products land in outputs that are never stored).
template <int KM>
__device__ __forceinline__ void lds_stage_load(float *dst, const float *src, int64_t ld, int64_t k0, int64_t wide0,
                                               int64_t wide_lim, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float *gp;
        int base;  // first float of this instruction's 1 KB window
        if constexpr (KM) {
            const int kk = 4 * wave + 2 * i + (lane >> 5);
            const int c = (lane & 31) ^ ((kk & 1) << 3);  // logical chunk at this lane's position
            int64_t w = wide0 + 4 * c;
            w = w < wide_lim ? w : wide0;
            gp = src + (k0 + kk) * ld + w;
            base = (4 * wave + 2 * i) * LT;
        } else {
            const int r = 32 * wave + 16 * i + (lane >> 2);
            const int c = (lane & 3) ^ ((r >> 2) & 3);
            int64_t w = wide0 + r;
            w = w < wide_lim ? w : wide0;
            gp = src + w * ld + k0 + 4 * c;
            base = (32 * wave + 16 * i) * LKS;
        }
        __builtin_amdgcn_global_load_lds(static_cast<const void *>(gp),
                                         (__attribute__((address_space(3))) void *)(dst + base), 16, 0, 0);
    }
}

// s_waitcnt: at most n vector-memory operations outstanding, and lgkmcnt(0).
template <int n>
__device__ __forceinline__ void lds_wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | ((n >> 4) << 14));
}

__device__ __forceinline__ void lds_bar() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int EPI, int AKM, int BKM>
__device__ __forceinline__ void gemm_f32_lds_tile(const GemmDesc &g, int tm, int tn, int bz, int64_t pidx) {
    constexpr int QB = 2, HW = 64;
    if (g.upper_only && tm > tn) return;
    const int64_t m0 = (int64_t)tm * LT, n0 = (int64_t)tn * LT;
    const float *A = g.A + bz * g.strideA;
    const float *B = g.B + bz * g.strideB;
    float *C = g.C + bz * g.strideC;
    int64_t kbeg = 0, kend = g.K;
    if (g.a_upper) kbeg = m0 < kbeg ? kbeg : m0;
    if (g.b_upper) kend = (n0 + LT) < kend ? (n0 + LT) : kend;
    kbeg = (kbeg / LKS) * LKS;
    const int nst = kend > kbeg ? (int)((kend - kbeg) / LKS) : 0;

    __shared__ LdsGemmSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    floatx16 acc[QB][QB];
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int j = 0; j < QB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    float cold[QB][QB][16];
    if (EPI == EPI_STORE && g.beta != 0.0f) {
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < QB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * HW + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * HW + j * 32 + mfma32_col(lane);
                    cold[i][j][r] = (m < g.M && n < g.N) ? C[m * g.ldc + n] : 0.0f;
                }
    }

    if (nst > 0) {
        // One stage (four loads per wave) is issued per iteration; past the
        // end the last stage again, into a slot nobody reads, so the number of
        // loads in flight at each wait is fixed.
        auto issue = [&](int st, int slot) {
            const int64_t k0 = kbeg + (int64_t)(st < nst ? st : nst - 1) * LKS;
            lds_stage_load<AKM>(sm.a[slot], A, g.lda, k0, m0, g.M, wave, lane);
            lds_stage_load<BKM>(sm.b[slot], B, g.ldb, k0, n0, g.N, wave, lane);
        };
#pragma unroll
        for (int st = 0; st < LNS - 1; ++st) issue(st, st);
        const int kr = lane >> 5, c = lane & 31;
        for (int st = 0; st < nst; ++st) {
            const int slot = st % LNS;
            lds_wait_vm<8>();  // this wave's loads of stage st landed (two later stages may be in flight),
                               // its operand reads of the previous stage are done
            lds_bar();         // ... and every wave's; slot (st - 1) % LNS is free
            issue(st + LNS - 1, (st + LNS - 1) % LNS);
            float op[2][2 * QB];
            auto rd = [&](int kk, float(&o)[2 * QB]) {
                const int k = kk + kr;
#pragma unroll
                for (int i = 0; i < QB; ++i) o[i] = sm.a[slot][lds_index<AKM>(k, wm * HW + i * 32 + c)];
#pragma unroll
                for (int j = 0; j < QB; ++j) o[QB + j] = sm.b[slot][lds_index<BKM>(k, wn * HW + j * 32 + c)];
            };
            rd(0, op[0]);
#pragma unroll
            for (int kk = 0; kk < LKS; kk += 2) {
                const int cur = (kk >> 1) & 1;
                if (kk + 2 < LKS) rd(kk + 2, op[cur ^ 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < QB; ++i)
#pragma unroll
                    for (int j = 0; j < QB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(op[cur][i], op[cur][QB + j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lds_wait_vm<0>();
    }

    if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < QB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * HW + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * HW + j * 32 + mfma32_col(lane);
                    if (m < g.M && n < g.N && (!g.upper_only || m <= n)) {
                        float v = g.alpha * acc[i][j][r];
                        if (g.beta != 0.0f) v += g.beta * cold[i][j][r];
                        C[m * g.ldc + n] = v;
                    }
                }
    } else {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
            for (int j = 0; j < QB; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + wm * HW + i * 32 + mfma32_row(r, lane);
                    const int64_t n = n0 + wn * HW + j * 32 + mfma32_col(lane);
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
            g.partial[pidx] = t;
        }
    }
}

template <int EPI, int AKM, int BKM>
__global__ __launch_bounds__(kThreads) void gemm_f32_lds_kernel(GemmDesc g) {
    const int gx = (int)ceil_div(g.N, LT), gy = (int)ceil_div(g.M, LT);
    int tm, tn, bz;
    if (g.max_wgs <= 0) {
        const int64_t id = (int64_t)blockIdx.z * gx * gy + (int64_t)blockIdx.y * gx + blockIdx.x;
        tile_of(g, id, gx, gy, tm, tn, bz);
        gemm_f32_lds_tile<EPI, AKM, BKM>(g, tm, tn, bz, (int64_t)blockIdx.y * gridDim.x + blockIdx.x);
        return;
    }
    const int64_t total = (int64_t)gx * gy * g.batch;
    for (int64_t id = blockIdx.x; id < total; id += gridDim.x) {
        if (id != blockIdx.x) __syncthreads();  // the previous tile's LDS reads are done
        tile_of(g, id, gx, gy, tm, tn, bz);
        gemm_f32_lds_tile<EPI, AKM, BKM>(g, tm, tn, bz, id);
    }
}

// One workgroup per tile, or a persistent grid of max_wgs workgroups.
template <int T>
dim3 launch_grid(const GemmDesc &g) {
    const int64_t gx = ceil_div(g.N, T), gy = ceil_div(g.M, T);
    if (g.max_wgs > 0) return dim3((unsigned)std::min<int64_t>(gx * gy * g.batch, g.max_wgs));
    return dim3((unsigned)gx, (unsigned)gy, (unsigned)g.batch);
}

template <int EPI>
void launch_lds(const GemmDesc &g, hipStream_t s) {
    const dim3 grid = launch_grid<LT>(g);
    const int akm = g.a_trans ? 1 : 0, bkm = g.b_trans ? 0 : 1;
    if (akm && bkm)
        hipLaunchKernelGGL((gemm_f32_lds_kernel<EPI, 1, 1>), grid, dim3(kThreads), 0, s, g);
    else if (akm)
        hipLaunchKernelGGL((gemm_f32_lds_kernel<EPI, 1, 0>), grid, dim3(kThreads), 0, s, g);
    else if (bkm)
        hipLaunchKernelGGL((gemm_f32_lds_kernel<EPI, 0, 1>), grid, dim3(kThreads), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_f32_lds_kernel<EPI, 0, 0>), grid, dim3(kThreads), 0, s, g);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

template <int EPI, int T>
void launch_tile(const GemmDesc &g, int va, int vb, hipStream_t s) {
    const dim3 grid = launch_grid<T>(g);
    if (va && vb)
        hipLaunchKernelGGL((gemm_f32_kernel<EPI, 1, 1, T>), grid, dim3(kThreads), 0, s, g);
    else if (va)
        hipLaunchKernelGGL((gemm_f32_kernel<EPI, 1, 0, T>), grid, dim3(kThreads), 0, s, g);
    else if (vb)
        hipLaunchKernelGGL((gemm_f32_kernel<EPI, 0, 1, T>), grid, dim3(kThreads), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<EPI, 0, 0, T>), grid, dim3(kThreads), 0, s, g);
}

constexpr int kCUs = 256;

}  // namespace

// The loss reduction indexes its partial sums by 128-wide tiles: EPI_DOT always uses them.
int64_t gemm_num_tiles(const GemmDesc &g) { return ceil_div(g.M, kGemmTile) * ceil_div(g.N, kGemmTile); }

hipError_t launch_gemm_f32(const GemmDesc &gd, hipStream_t s) {
    if (gd.M <= 0 || gd.N <= 0 || gd.batch <= 0) return hipSuccess;
    GemmDesc g = gd;
    if (g.epilogue == EPI_DOT) g.max_wgs = 0;  // its partial sums are indexed by workgroup
    const bool bz = g.batch > 1;
    // 16-byte chunks wholly inside or outside: aligned base and stride, and
    // the contiguous extent (the tile-wide dim, or K) a multiple of 4.
    const bool k4 = g.K % 4 == 0;
    const int va = aligned16(g.A) && g.lda % 4 == 0 && (!bz || g.strideA % 4 == 0) && (g.a_trans ? g.M % 4 == 0 : k4);
    const int vb = aligned16(g.B) && g.ldb % 4 == 0 && (!bz || g.strideB % 4 == 0) && (g.b_trans ? k4 : g.N % 4 == 0);
    // Aligned operands and K a multiple of the stage depth: the direct-to-LDS
    // kernel (128 x 128 tiles); the register-staged one otherwise, and with
    // 64 x 64 tiles when 128-wide ones would give fewer than two per CU.
    const bool lds_ok = va && vb && g.K % LKS == 0;
    const int64_t tiles128 = ceil_div(g.M, 128) * ceil_div(g.N, 128) * g.batch;
    if (g.epilogue == EPI_DOT) {
        if (lds_ok)
            launch_lds<EPI_DOT>(g, s);
        else
            launch_tile<EPI_DOT, kGemmTile>(g, va, vb, s);
    } else if (tiles128 < 2 * kCUs) {
        launch_tile<EPI_STORE, 64>(g, va, vb, s);
    } else if (lds_ok) {
        launch_lds<EPI_STORE>(g, s);
    } else {
        launch_tile<EPI_STORE, 128>(g, va, vb, s);
    }
    return hipGetLastError();
}

}  // namespace gptq
