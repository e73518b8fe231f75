// Step 1 of GPTQ: H += 2 X X^T from calibration activations (page "LLM 量化方法
// 原理与实现详解", §4.1: the layer objective's Hessian is 2 X X^T).
//
// bf16 activations: a symmetric rank-k update on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate), 256 x 256 tiles per 4-wave
// workgroup with 128 x 128 per wave (accumulators in AGPRs), so each 16-byte
// LDS read feeds four MFMAs.  X is [d_in][ldx], one row per channel, tokens
// contiguous, so both MFMA operands of a tile are row panels of X read along
// K.  Only tiles on or above the diagonal are computed (the algorithmic
// d(d+1)/2 * N multiply-adds).  When a layer has too few tiles to fill the
// chip, tokens are split across workgroups and the partial tiles are summed in
// a fixed order by a second kernel, so H is bit-reproducible.
//
// Pipeline: the panels stream through a ring of four 32-token LDS stages
// filled by direct global->LDS loads, three stages ahead of the matrix cores;
// the MFMA operands of the next 16-token step are read from LDS while the
// current step's MFMAs run; the LDS reads and global->LDS loads are issued one
// per MFMA.  Work order: workgroup b runs on XCD b % 8.  The upper tiles, in
// bands of four tile rows taken column by column, are cut into eight
// contiguous groups, one per XCD, and every XCD walks its group split after
// split: the tiles an XCD holds at once share a few row panels in its L2, and
// all XCDs read the same token range at the same time, so L2 misses are
// mostly served by the shared last-level cache rather than HBM.
//
// fp32 activations go through the fp32 matrix-core GEMM (upper tiles only).
#include "common.h"

namespace gptq {
namespace {

constexpr int TS = 256;        // output tile edge (4 waves, each 128 x 128)
constexpr int KT = 32;         // tokens per LDS stage: 64 bytes of bf16 per row
constexpr int CH = KT / 8;     // 16-byte chunks per row and stage
constexpr int NS = 4;          // LDS ring depth (stages)
constexpr int BAND = 4;        // tile rows per band of the work order
constexpr int kThreads = 256;
constexpr int kCUs = 256;
constexpr int kXCDs = 8;

// LDS panels: NS stages x 256 rows x 64 B, unpadded.  Logical chunk c of row r
// sits at position c ^ swz(r).  Row r starts in 16-byte bank group 4 (r % 4)
// of the 64 four-byte banks, so the position has to separate rows that agree
// mod 4: with swz(r) = (r / 4) % 4 the 32 rows one b128 read touches at a
// common chunk spread over all 16 groups, and the read takes its minimum of
// four LDS cycles (measured with a bank-conflict counter; a swizzle on bits 1
// and 3 of the row took eight).
struct SyrkSmem {
    uint4 a[NS][TS][CH];
    uint4 b[NS][TS][CH];
};

__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ int64_t tile_linear(int ti, int tj, int nt) {
    return (int64_t)ti * nt - (int64_t)ti * (ti - 1) / 2 + (tj - ti);
}

// Row-major upper-triangle index -> (ti, tj); row i holds nt - i tiles.
__device__ __forceinline__ void tile_of(int64_t t, int nt, int &ti, int &tj) {
    int i = 0;
    int64_t before = 0;
    while (before + (nt - i) <= t) {
        before += nt - i;
        ++i;
    }
    ti = i;
    tj = i + (int)(t - before);
}

// Band order: bands of BAND tile rows; inside a band, column by column, rows
// top to bottom (only i <= j).
__device__ __forceinline__ void tile_of_band(int64_t t, int nt, int &ti, int &tj) {
    int r0 = 0;
    for (;;) {
        const int r1 = min(r0 + BAND, nt) - 1;
        const int h = r1 - r0 + 1;
        // columns r0 .. r1 hold 1 .. h tiles, later columns h each
        const int64_t ramp = (int64_t)h * (h + 1) / 2;
        const int64_t cnt = ramp + (int64_t)(nt - 1 - r1) * h;
        if (t < cnt) {
            if (t < ramp) {
                int j = 0;
                while ((int64_t)(j + 1) * (j + 2) / 2 <= t) ++j;
                ti = r0 + (int)(t - (int64_t)j * (j + 1) / 2);
                tj = r0 + j;
            } else {
                const int64_t u = t - ramp;
                tj = r1 + 1 + (int)(u / h);
                ti = r0 + (int)(u % h);
            }
            return;
        }
        t -= cnt;
        r0 += BAND;
    }
}

// One 1 KB piece of a stage of a 256-row panel, straight from global memory
// into LDS (global_load_lds_dwordx4: lane l of a wave writes LDS bytes
// [16 l, 16 l + 16) of the wave's window, i.e. 16 rows of 64 B).  Wave w fills
// rows 64 w .. 64 w + 63 in four pieces i = 0..3; each lane fetches the global
// chunk that belongs at its LDS position.  Rows past d are clamped to row d-1
// (valid memory; those outputs are discarded).
__device__ __forceinline__ void panel_piece(uint4 (*dst)[CH], const uint16_t *X, int64_t ldx, int64_t d,
                                            int64_t row0, int64_t k0, int wave, int lane, int i) {
    const int row = wave * 64 + i * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    int64_t gr = row0 + row;
    gr = gr < d ? gr : d - 1;
    const uint16_t *src = X + gr * ldx + k0 + c * 8;
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                     (__attribute__((address_space(3))) void *)(&dst[wave * 64 + i * 16][0]), 16, 0, 0);
}

// The same LDS image of a partial stage (tokens k0 .. kend-1, the rest zero)
// from masked register loads.
__device__ __forceinline__ void panel_tail(uint4 (*dst)[CH], const uint16_t *X, int64_t ldx, int64_t d, int64_t row0,
                                           int64_t k0, int64_t kend, int tid) {
    for (int e = tid; e < TS * CH; e += kThreads) {
        const int row = e / CH, pos = e % CH;
        const int c = pos ^ swz(row);
        const int64_t gr = row0 + row, gk = k0 + c * 8;
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t lo = (gr < d && gk + 2 * h < kend) ? X[gr * ldx + gk + 2 * h] : 0u;
            const uint32_t hi = (gr < d && gk + 2 * h + 1 < kend) ? X[gr * ldx + gk + 2 * h + 1] : 0u;
            w[h] = lo | (hi << 16);
        }
        dst[row][pos] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// s_waitcnt with lgkmcnt(0) and at most n vector-memory operations outstanding.
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | ((n >> 4) << 14));
}

// Workgroup barrier without a memory fence: the waits before it are explicit.
// The empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void bar() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct Frags {
    bf16x8 a[4], b[4];
};

// grid.x = 8 * ceil(tiles / 8) * splits.  Each wave owns a
// 128 x 128 quarter of the 256 x 256 tile as 4 x 4 v_mfma_f32_32x32x16_bf16
// accumulators.  out_partial == nullptr: H += 2 acc (upper triangle); else the
// raw partial tile goes to out_partial[split * ntiles + row-major tile index].
__global__ __launch_bounds__(kThreads) void syrk_bf16_kernel(const uint16_t *__restrict__ X, int64_t ldx, int64_t d,
                                                             int64_t n_tok, int64_t kchunk, int nt, int64_t ntiles,
                                                             int splits, float *__restrict__ H,
                                                             float *__restrict__ out_partial) {
    // XCD x owns band-order positions [g0, g1) and runs them split after split.
    const int64_t xcd = blockIdx.x % kXCDs, slot = blockIdx.x / kXCDs;
    const int64_t g0 = xcd * ntiles / kXCDs, g1 = (xcd + 1) * ntiles / kXCDs, gsz = g1 - g0;
    if (gsz <= 0 || slot >= gsz * splits) return;
    const int64_t split = slot / gsz;
    int ti, tj;
    tile_of_band(g0 + slot % gsz, nt, ti, tj);
    const bool diag = ti == tj;
    const int64_t r0 = (int64_t)ti * TS, c0 = (int64_t)tj * TS;
    const int64_t kbeg = split * kchunk;
    const int64_t kend = (kbeg + kchunk) < n_tok ? (kbeg + kchunk) : n_tok;
    const int nfull = kend > kbeg ? (int)((kend - kbeg) / KT) : 0;
    const bool has_tail = kend > kbeg + (int64_t)nfull * KT;

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

    // This lane's operand rows are base + (lane % 32) with bases that are
    // multiples of 32, so they share one swizzle; logical chunk 2 ks + lane / 32.
    const int lrow = lane & 31, half = lane >> 5;
    const int sw = swz(lrow);
    // Stage st of both panels into ring slot `slot` (diagonal tiles load their
    // one panel twice, which keeps the load count per stage uniform: 8 per wave).
    auto issue_piece = [&](int st, int slot, int p) {
        const int64_t k0 = kbeg + (int64_t)st * KT;
        if (p < 4)
            panel_piece(sm.a[slot], X, ldx, d, r0, k0, wave, lane, p);
        else
            panel_piece(sm.b[slot], X, ldx, d, c0, k0, wave, lane, p - 4);
    };
    // Operand p of a 16-token step: p < 4 is A row block p, else B row block p-4.
    auto read_frag = [&](int slot, int ks, int p, Frags &f) {
        const int pos = (2 * ks + half) ^ sw;
        if (p < 4)
            f.a[p] = __builtin_bit_cast(bf16x8, sm.a[slot][wm * 128 + p * 32 + lrow][pos]);
        else
            f.b[p - 4] = __builtin_bit_cast(bf16x8, sm.b[slot][wn * 128 + (p - 4) * 32 + lrow][pos]);
    };
    auto mfma = [&](const Frags &f, int q) {
        acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[q >> 2], f.b[q & 3], acc[q >> 2][q & 3], 0, 0, 0);
    };

    if (nfull > 0) {
        // Exactly one stage is issued per step (past the end: the last stage
        // again, into a slot nobody reads), so the in-flight count is fixed:
        // at each wait, the stage being waited for is followed by one more.
#pragma unroll
        for (int st = 0; st < NS - 1; ++st)
#pragma unroll
            for (int p = 0; p < 8; ++p) issue_piece(min(st, nfull - 1), st, p);
        wait_vm_lgkm0<16>();  // stage 0 landed
        bar();
        Frags f0, f1;
#pragma unroll
        for (int p = 0; p < 8; ++p) read_frag(0, 0, p, f0);
        // Each step is two half-steps of 16 MFMAs; the LDS reads of the other
        // half's operands and the global->LDS loads of the stage NS-1 ahead
        // are issued one per MFMA (the scheduling fences hold that order), so
        // the matrix core never waits on instruction issue.
        for (int k = 0; k < nfull; ++k) {
            const int cur = k % NS, nxt = (k + 1) % NS;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                mfma(f0, q);
                if (q >= 1 && q <= 8) read_frag(cur, 1, q - 1, f1);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_vm_lgkm0<8>();  // stage k+1 landed (and this wave's operand reads are done)
            bar();               // ... for every wave; slot (k-1) % NS is free
            const int st = min(k + NS - 1, nfull - 1), slot = (k + NS - 1) % NS;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                mfma(f1, q);
                if (q >= 1 && q <= 8) issue_piece(st, slot, q - 1);
                if (q >= 7 && q <= 14) read_frag(nxt, 0, q - 7, f0);  // unused after the last step
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vm_lgkm0<0>();
    }
    if (has_tail) {
        const int64_t k0 = kbeg + (int64_t)nfull * KT;
        __syncthreads();  // every wave is done with the ring
        panel_tail(sm.a[0], X, ldx, d, r0, k0, kend, tid);
        panel_tail(sm.b[0], X, ldx, d, c0, k0, kend, tid);
        __syncthreads();
        Frags f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int p = 0; p < 8; ++p) read_frag(0, ks, p, f);
#pragma unroll
            for (int q = 0; q < 16; ++q) mfma(f, q);
        }
    }

    if (out_partial) {
        float *dst = out_partial + (split * ntiles + tile_linear(ti, tj, nt)) * (TS * TS);
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

// hdiag[i] += 2 * sum_t X[i][t]^2 in fp64.  One workgroup per channel; rows
// are read in 16-byte pieces (X and ldx*sizeof(T) are 16-byte aligned at the
// boundary), four pieces in flight per thread, the ragged end element-wise.
template <typename T>
__device__ __forceinline__ float widen_elem(T v) {
    if constexpr (sizeof(T) == 2) {
        return __uint_as_float((uint32_t)v << 16);
    } else {
        return v;
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void diag_f64_kernel(const T *__restrict__ X, int64_t ldx, int64_t n_tok,
                                                            double *__restrict__ hdiag) {
    constexpr int kPer = 16 / sizeof(T);  // elements per 16-byte piece
    constexpr int kUnroll = 4;
    const int64_t i = blockIdx.x;
    const T *row = X + i * ldx;
    const int64_t npieces = n_tok / kPer;
    double s = 0.0;
    int64_t p = threadIdx.x;
    for (; p + (kUnroll - 1) * kThreads < npieces; p += kUnroll * kThreads) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = *reinterpret_cast<const uint4 *>(row + (p + u * kThreads) * kPer);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const T *e = reinterpret_cast<const T *>(&v[u]);
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const double x = (double)widen_elem<T>(e[k]);
                s = fma(x, x, s);
            }
        }
    }
    for (; p < npieces; p += kThreads) {
        const uint4 v = *reinterpret_cast<const uint4 *>(row + p * kPer);
        const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const double x = (double)widen_elem<T>(e[k]);
            s = fma(x, x, s);
        }
    }
    for (int64_t t = npieces * kPer + threadIdx.x; t < n_tok; t += kThreads) {
        const double x = (double)widen_elem<T>(row[t]);
        s = fma(x, x, s);
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
//   rounds of workgroups over one XCD's CUs x stages per split  +  partial-tile traffic.
SyrkPlan plan_syrk(int64_t d, int64_t n_tok) {
    SyrkPlan p;
    p.nt = (int)ceil_div(d, TS);
    p.ntiles = (int64_t)p.nt * (p.nt + 1) / 2;
    const double stage_us = 1.0;                        // one 256x256x32 stage per CU (order of magnitude)
    const double part_us = 2.0 * TS * TS * 4 / 4.0e6;  // write + read of one partial tile at ~4 TB/s (whole chip)
    double best = 1e300;
    int best_s = 1;
    for (int s = 1; s <= 64; ++s) {
        const int64_t kc = ceil_div(ceil_div(n_tok, s), KT) * KT;
        if (s > 1 && kc < 16 * KT) break;
        const int64_t wgs = p.ntiles * s;
        const double rounds = (double)ceil_div(ceil_div(p.ntiles, kXCDs) * s, kCUs / kXCDs);  // largest group
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
        hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)(kXCDs * ceil_div(p.ntiles, kXCDs) * p.splits)),
                           dim3(kThreads), 0, s,
                           static_cast<const uint16_t *>(X), ldx, d, n_tok, p.kchunk, p.nt, p.ntiles, p.splits, H,
                           part);
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
