// Column-pass batch kernel of GPTQ (page "PTQ 权重量化：从 GPTQ 到 AWQ", GPTQ
// section: each quantized column's error goes onto the not-yet-quantized
// columns through the matching row of the inverse Hessian factor).
//
// L lanes per output row (4, or 16 for layers with few rows).  The row's BT
// weights of the batch stay in registers (BT/L per lane) for the whole batch;
// the BT x BT block of U sits in LDS.  For each column j:
// take the column's grid (SRC, see GridSource: fitted from the current
// weights at a group start, or read from the grids fitted before), quantize, form
// e = (w_j - w_hat_j) / U[j][j], update w_k -= e U[j][k] for the batch's later
// columns, and store -e into E^T for the trailing matrix-core update.  The
// unrolled column loop is branch-free: the LDS copy of U is zero on and below
// the diagonal, so every lane can run the same update; columns past the batch
// end see zero weights and a zero U block, so they change nothing and are
// never stored.
#pragma once

#include "block_args.h"
#include "quad.h"
#include "quant_grid.h"

namespace gptq {

// Each output row is owned by L consecutive lanes; lane q of the group keeps
// columns q, q+L, q+2L, ... of the batch in registers.  Column j's owner
// broadcasts the weight to its group (DPP), all L lanes quantize it (same
// result), and each lane pushes the error onto its own later columns.  With
// L = 16 each lane carries a quarter of the FMAs of L = 4 on the column chain,
// which sets the time when the layer has too few rows to fill the chip.
// NT threads per workgroup (NT / L rows).
template <int BT, int GT, int NT, int SRC, int L>
__global__ __launch_bounds__(NT) void gptq_block_kernel(BlockArgs a) {
    static_assert(SRC != kColumnGrids || GT == 0, "per-column grids take no group tile");
    static_assert(L == 4 || L == 16, "four or sixteen lanes per row");
    static_assert(BT % (4 * L) == 0 && (GT == 0 || GT % L == 0), "whole 16-byte words of U per lane; groups of whole steps");
    constexpr int CPL = BT / L;
    constexpr int kRows = NT / L;
    // The B x B block of U, strictly upper part (zero on and below the
    // diagonal), laid out per group lane: ut[j][p][q][i] = U[j][q + L (4p + i)],
    // so lane q reads its columns of row j as contiguous 16-byte words and the
    // lanes of a group hit different bank groups.
    constexpr int NP = CPL / 4;
    __shared__ __attribute__((aligned(16))) float ut[BT][NP][L][4];
    __shared__ float inv_d[BT];
    __shared__ int32_t pcol[BT];
    __shared__ int32_t gcol[SRC == kColumnGrids ? BT : 1];  // group of each column (per-column grids)
    const int tid = threadIdx.x;
    const int nc = a.ncols;
    const int q = tid & (L - 1);
    const int64_t r = (int64_t)blockIdx.x * kRows + tid / L;
    const bool active = r < a.d_out;
    float *wrow = a.W + r * a.ldw + a.c0;
    // Global loads of the prologue are all issued before the first wait: the
    // permutation entries, the row's weights, then the U block in passes of at
    // most 16 16-byte chunks per thread.  The first two read clamped addresses
    // and mask the values afterwards; the masks are opaque to the compiler, so
    // it cannot move a load under a branch and wait for it there.
    constexpr int kPc = (BT + NT - 1) / NT;  // permutation entries per thread
    int32_t pc[kPc];
    {
        // with no permutation, U stands in as a readable address; the value is masked off
        const int32_t *pp = a.perm ? a.perm : reinterpret_cast<const int32_t *>(a.U);
        uint32_t mp = a.perm ? ~0u : 0u;
        asm volatile("" : "+v"(mp));
#pragma unroll
        for (int u = 0; u < kPc; ++u) {
            const int c = tid + u * NT;
            const int64_t k = a.c0 + (c < nc ? c : 0);
            const uint32_t v = (uint32_t)clamp_col(pp[k], a.ldc);
            pc[u] = (int32_t)((v & mp) | ((uint32_t)(a.c0 + c) & ~mp));
        }
    }
    int32_t gc[SRC == kColumnGrids ? kPc : 1];
    if constexpr (SRC == kColumnGrids) {
#pragma unroll
        for (int u = 0; u < kPc; ++u) {
            const int c = tid + u * NT;
            gc[u] = (int32_t)(clamp_col(a.gperm[a.c0 + (c < nc ? c : nc - 1)], a.ldc) / a.g);
        }
    }
    const int64_t rr = active ? r : a.d_out - 1;  // a row whose grids exist
    constexpr int NG = GT > 0 ? BT / GT : 1;
    float fs[NG], fz[NG];  // grids of the batch's groups, fitted before the pass
    if constexpr (SRC == kStoredGrids && GT > 0) {
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            const int64_t gi = (a.c0 + (gg * GT < nc ? gg * GT : 0)) / a.g;
            fs[gg] = a.scales[rr * a.ng + gi];
            fz[gg] = a.zeros[rr * a.ng + gi];
        }
    }
    float w[CPL];
    {
        const float *wsrc = a.W + (active ? r : a.d_out - 1) * a.ldw + a.c0;
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
            const int k = q + L * t;
            uint32_t m = (active && k < nc) ? ~0u : 0u;
            asm volatile("" : "+v"(m));
            w[t] = __uint_as_float(__float_as_uint(wsrc[k < nc ? k : nc - 1]) & m);
        }
    }
    // 1 / U_jj of the batch's columns (zero past the batch end)
    constexpr int kDg = (BT + NT - 1) / NT;
    float dg[kDg];
#pragma unroll
    for (int u = 0; u < kDg; ++u) {
        const int c = tid + u * NT;
        const int64_t cc = a.c0 + (c < nc ? c : nc - 1);
        dg[u] = a.U[cc * a.ldu + cc];
    }
    {
        constexpr int kChunks = BT * BT / 4;  // 16-byte chunks of the U block
        static_assert(kChunks % NT == 0, "U block chunks must split evenly over the threads");
        constexpr int kUPer = kChunks / NT;                  // per thread
        constexpr int kPass = kUPer < 16 ? kUPer : 16;       // per thread and pass
        const float *src = a.U + a.c0 * a.ldu + a.c0;
        const bool vec = a.vec && (a.ldu % 4 == 0) && (a.c0 % 4 == 0) && nc == BT;
#pragma unroll
        for (int p0 = 0; p0 < kUPer; p0 += kPass) {
            float4 uv[kPass];
            if (vec) {  // full, aligned batch: 16-byte loads
#pragma unroll
                for (int u = 0; u < kPass; ++u) {
                    const int e4 = tid + (p0 + u) * NT;
                    const int i = (e4 * 4) / BT, k = (e4 * 4) % BT;
                    uv[u] = *reinterpret_cast<const float4 *>(src + i * a.ldu + k);
                }
            } else {  // partial or unaligned batch: clamped scalar loads, masked
#pragma unroll
                for (int u = 0; u < kPass; ++u) {
                    const int e4 = tid + (p0 + u) * NT;
                    const int i = (e4 * 4) / BT, k = (e4 * 4) % BT;
                    const float *p = src + (int64_t)(i < nc ? i : nc - 1) * a.ldu;
                    float v4[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        uint32_t m = (i < nc && k + x < nc) ? ~0u : 0u;
                        asm volatile("" : "+v"(m));
                        v4[x] = __uint_as_float(__float_as_uint(p[k + x < nc ? k + x : nc - 1]) & m);
                    }
                    uv[u] = make_float4(v4[0], v4[1], v4[2], v4[3]);
                }
            }
#pragma unroll
            for (int u = 0; u < kPass; ++u) {
                const int e4 = tid + (p0 + u) * NT;
                const int i = (e4 * 4) / BT, k = (e4 * 4) % BT;
                const float4 v = uv[u];
                // columns k .. k+3 belong to group lanes k % L .. k % L + 3, at t = k / L
                const int t = k / L, l0 = k % L;
                ut[i][t / 4][l0 + 0][t % 4] = (k + 0 > i) ? v.x : 0.0f;
                ut[i][t / 4][l0 + 1][t % 4] = (k + 1 > i) ? v.y : 0.0f;
                ut[i][t / 4][l0 + 2][t % 4] = (k + 2 > i) ? v.z : 0.0f;
                ut[i][t / 4][l0 + 3][t % 4] = (k + 3 > i) ? v.w : 0.0f;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kDg; ++u) {
        const int c = tid + u * NT;
        if (c < BT) inv_d[c] = c < nc ? 1.0f / dg[u] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kPc; ++u) {
        const int c = tid + u * NT;
        if (c < BT) pcol[c] = pc[u];  // every entry 0..BT-1 is written
        if constexpr (SRC == kColumnGrids)
            if (c < BT) gcol[c] = gc[u];
    }
    __syncthreads();

    Grid gr = grid_make(0.0f, 0.0f, 0.0f, a.bits, a.sym);
    if constexpr (GT == 0 && SRC != kColumnGrids) {
        if (active) {
            const int64_t gi = a.c0 / a.g;
            gr = grid_from_stored(a.scales[r * a.ng + gi], a.zeros[r * a.ng + gi], a.bits, a.sym);
        }
    }
    // Per-column grids: the packed grid of column j's group is read kPf
    // columns ahead into a ring of kPf + 1 slots (unpacking costs one ldexp).
    constexpr int kPf = 2;
    float4 ct[kPf + 1];
    const float4 *trow = a.gtab + rr * a.ng;
    auto load_grid = [&](int j, int slot) { ct[slot] = trow[gcol[j]]; };
    if constexpr (SRC == kColumnGrids) {
#pragma unroll
        for (int j = 0; j < kPf; ++j) load_grid(j, j);
    }
    // grids fitted in this batch, kept in LDS (not registers) until the end
    __shared__ float fit_sz[SRC == kFitGrids && GT > 0 ? kRows : 1][NG][2];
    uint32_t cw[(CPL + 3) / 4];
#pragma unroll
    for (int t = 0; t < (CPL + 3) / 4; ++t) cw[t] = 0u;
    float *et = a.Et + r;  // rows past d_out land in the padding of E^T

    // This lane's part of row j of U (and 1/U_jj) is read one column ahead, so
    // the LDS reads overlap the previous column's quantization chain.
    float4 urow[2][NP];
    float idn[2];
    auto load_row = [&](int j, float4(&dst)[NP], float &id) {
#pragma unroll
        for (int p = (j / L) / 4; p < NP; ++p) dst[p] = *reinterpret_cast<const float4 *>(&ut[j][p][q][0]);
        id = inv_d[j];
    };
    load_row(0, urow[0], idn[0]);

#pragma unroll
    for (int j = 0; j < BT; ++j) {
        const int oq = j & (L - 1), ot = j / L;
        const int cur = j & 1;
        if (j + 1 < BT) load_row(j + 1, urow[cur ^ 1], idn[cur ^ 1]);
        if constexpr (SRC == kColumnGrids)
            if (j + kPf < BT) load_grid(j + kPf, (j + kPf) % (kPf + 1));
        // the reads stay here, ahead of their use
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SRC == kColumnGrids) {
            gr = grid_unpack(ct[j % (kPf + 1)], a.bits, a.sym);
        } else if constexpr (SRC == kStoredGrids && GT > 0) {
            if (j % GT == 0) gr = grid_from_stored(fs[j / GT], fz[j / GT], a.bits, a.sym);
        } else if constexpr (GT > 0) {
            if (j % GT == 0) {
                float amax = 0.0f, lo = 0.0f, hi = 0.0f;
#pragma unroll
                for (int t = j / L; t < (j + GT) / L; ++t) {
                    amax = fmaxf(amax, fabsf(w[t]));
                    lo = fminf(lo, w[t]);
                    hi = fmaxf(hi, w[t]);
                }
#pragma unroll
                for (int st = 0; st < lanes_steps<L>(); ++st) {
                    amax = fmaxf(amax, lanes_step<L>(amax, st));
                    lo = fminf(lo, lanes_step<L>(lo, st));
                    hi = fmaxf(hi, lanes_step<L>(hi, st));
                }
                gr = grid_make(amax, lo, hi, a.bits, a.sym);
                fit_sz[tid / L][j / GT][0] = gr.s;
                fit_sz[tid / L][j / GT][1] = gr.zero;
            }
        }
        const float wj = lanes_bcast<L>(w[ot], oq);
        const float ql = grid_level(wj, gr);
        const float code = ql + gr.zadd;
        // e = (w_j - (code - zero) s) / U_jj, with code - zero = ql - zd exact;
        // w_j / U_jj and s / U_jj are formed beside the quantization
        const float e = fmaf(-(ql - gr.zd), gr.s * idn[cur], wj * idn[cur]);
        cw[ot / 4] |= (q == oq ? (uint32_t)code : 0u) << (8 * (ot & 3));
        et[(int64_t)j * a.ldet] = -e;
#pragma unroll
        for (int p = ot / 4; p < NP; ++p) {
            const float4 u = urow[cur][p];
            const float uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * p + i >= ot) w[4 * p + i] = fmaf(-e, uu[i], w[4 * p + i]);
        }
    }

    if (!active) return;
    if constexpr (SRC == kFitGrids && GT > 0) {
        if (q == 0) {
#pragma unroll
            for (int g = 0; g < NG; ++g)
                if (g * GT < nc) {
                    const int64_t gi = (a.c0 + g * GT) / a.g;
                    a.scales[r * a.ng + gi] = fit_sz[tid / L][g][0];
                    a.zeros[r * a.ng + gi] = fit_sz[tid / L][g][1];
                }
        }
    }
    // w[t] is never touched after its column is quantized: it is the value at quantization time.
    uint8_t *crow = a.codes + r * a.ldc;
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
        const int k = q + L * t;
        if (k < nc) {
            wrow[k] = w[t];
            crow[pcol[k]] = (uint8_t)(cw[t / 4] >> (8 * (t & 3)));
        }
    }
}

template <int BT, int GT, int NT, int L>
hipError_t launch_block_gt(const BlockArgs &a, int src, unsigned grid, hipStream_t s) {
    if (src == kStoredGrids)
        hipLaunchKernelGGL((gptq_block_kernel<BT, GT, NT, kStoredGrids, L>), dim3(grid), dim3(NT), 0, s, a);
    else
        hipLaunchKernelGGL((gptq_block_kernel<BT, GT, NT, kFitGrids, L>), dim3(grid), dim3(NT), 0, s, a);
    return hipGetLastError();
}

template <int BT, int NT, int L>
hipError_t launch_block_nt(const BlockArgs &a, int gt, int src, hipStream_t s) {
    const unsigned grid = (unsigned)ceil_div(a.d_out, NT / L);
    if (src == kColumnGrids) {
        if (!a.gperm || !a.gtab || gt != 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gptq_block_kernel<BT, 0, NT, kColumnGrids, L>), dim3(grid), dim3(NT), 0, s, a);
        return hipGetLastError();
    }
    switch (gt) {
    case 0:  // the grid is read at the batch start either way
        hipLaunchKernelGGL((gptq_block_kernel<BT, 0, NT, kFitGrids, L>), dim3(grid), dim3(NT), 0, s, a);
        return hipGetLastError();
    case 32:
        return launch_block_gt<BT, 32, NT, L>(a, src, grid, s);
    case 64:
        if constexpr (BT >= 64) return launch_block_gt<BT, 64, NT, L>(a, src, grid, s);
        return hipErrorInvalidValue;
    case 128:
        if constexpr (BT >= 128) return launch_block_gt<BT, 128, NT, L>(a, src, grid, s);
        return hipErrorInvalidValue;
    default:
        return hipErrorInvalidValue;
    }
}

// Four-wave workgroups.  Four lanes per row (64 rows per workgroup) when the
// layer has rows enough for about two waves per SIMD, else sixteen (16 rows per
// workgroup, batches of 64 and 128 columns).  One-wave workgroups at four lanes
// per row, which spread a small layer over more CUs, measured slower: each
// row's column chain, not the CU count, sets the time.
constexpr int64_t kWideRowsMax = 8192;  // rows up to which a row takes 16 lanes
template <int BT>
hipError_t launch_block_bt(const BlockArgs &a, int gt, int src, hipStream_t s) {
    if (!a.Et || !a.W || !a.U || !a.codes) return hipErrorInvalidValue;
    if constexpr (BT >= 64)
        if (a.d_out <= kWideRowsMax) return launch_block_nt<BT, kBlockThreads, 16>(a, gt, src, s);
    return launch_block_nt<BT, kBlockThreads, 4>(a, gt, src, s);
}

}  // namespace gptq
