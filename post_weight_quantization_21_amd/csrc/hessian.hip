// Step 1 of GPTQ: H += 2 X X^T from calibration activations (page "LLM 量化方法
// 原理与实现详解", §4.1: the layer objective's Hessian is 2 X X^T; page "量化经典：
// LLM.int8 / GPTQ / AWQ", §二 step 1: the calibration set is run through the layer
// and its inputs collected, token by token).
//
// bf16 activations: a symmetric rank-k update on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate), 256 x 256 tiles per 4-wave
// workgroup with 128 x 128 per wave (accumulators in AGPRs), so each 16-byte
// LDS read feeds four MFMAs.  Only tiles on or above the diagonal are computed
// (the algorithmic d(d+1)/2 * N multiply-adds).  When a layer has too few tiles
// to fill the chip, tokens are split across workgroups and the partial tiles
// are summed in a fixed order by a second kernel, so H is bit-reproducible.
//
// Two input layouts share one kernel and one order of matrix-core products
// (16-token steps in token order), so both give the same H bit for bit:
//   channel-major X[d][ldx] (tokens contiguous): stages of 64 tokens, so each
//     row's piece is one whole 128-byte line, go straight from global memory
//     into LDS (global_load_lds_dwordx4) through two slots, the next stage's
//     loads one stage ahead; a split's last tokens (fewer than 64) go through
//     the 32-token stages below;
//   token-major X[n][ldx] (channels contiguous, as a layer's inputs arrive):
//     each lane loads 8 tokens x 4 channels (8-byte loads, 512 contiguous
//     bytes per token and wave), transposes them in registers with byte
//     permutes and writes four 16-byte chunks, one per channel, into an image
//     of 256 rows = channels of 32 tokens; a ring of four such stages, three
//     stages of loads in flight in registers.  No transposed copy of X is ever
//     made.
//
// Pipeline: the MFMA operands of the next 16-token step are read from LDS
// while the current step's MFMAs run; loads, LDS reads and writes are issued
// between the MFMAs.  Work order: workgroup b runs on XCD b % 8.  The upper
// tiles, in bands of eight tile rows taken column by column (measured 0.4-1.5 %
// faster than bands of four with the 64-token stages, as fast as sixteen), are
// cut into eight contiguous groups, one per XCD, and every XCD
// walks its group split after split: the tiles an XCD holds at once share a
// few row panels in its L2, and all XCDs read the same token range at the same
// time, so L2 misses are mostly served by the shared last-level cache.
//
// With act-order the fp64 diagonal (the ordering key) is a separate pass over
// X: summed inside the diagonal tiles, the fp64 work (conversions and fused
// multiply-adds) did not hide under the MFMAs and made those tiles twice as
// long, which cost more than reading X once more.
//
// fp32 activations go through the fp32 matrix-core GEMM (upper tiles only).
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace gptq {
namespace {

constexpr int TS = 256;        // output tile edge (4 waves, each 128 x 128)
constexpr int KT = 32;         // tokens per LDS stage: 64 bytes of bf16 per row
constexpr int BAND = 8;        // tile rows per band of the work order
constexpr int kThreads = 256;
constexpr int kCUs = 256;
constexpr int kXCDs = 8;

// LDS panels: NS stages of 16 KB per panel.
// Channel-major image: 256 rows (channels) x 64 B (32 tokens).  Logical chunk
// c (tokens 8c .. 8c+7) of row r sits at position c ^ swz(r).  Row r starts in
// 16-byte bank group 4 (r % 4) of the 64 four-byte banks, so the position has
// to separate rows that agree mod 4: with swz(r) = (r / 4) % 4 the 32 rows one
// b128 read touches at a common chunk spread over all 16 groups, and the read
// takes its minimum of four LDS cycles (measured with a bank-conflict counter;
// a swizzle on bits 1 and 3 of the row took eight).
// The token-major writes (lane l writes rows 4 l .. 4 l + 3 at one chunk, in an
// order that depends on (l / 4) % 4) hit groups 4 j' + (t ^ l % 4), distinct
// over every 16 lanes.
constexpr int NS = 4;
struct SyrkSmem {
    uint4 a[NS][TS][4];
    uint4 b[NS][TS][4];
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

// Channel-major: one 1 KB piece of a stage of a 256-row panel, straight from
// global memory into LDS (global_load_lds_dwordx4: lane l of a wave writes LDS
// bytes [16 l, 16 l + 16) of the wave's window, i.e. 16 rows of 64 B).  Wave w
// fills rows 64 w .. 64 w + 63 in four pieces i = 0..3; each lane fetches the
// global chunk that belongs at its LDS position.  Rows past d are clamped to
// row d-1 (valid memory; those outputs are discarded).
__device__ __forceinline__ void panel_piece(uint4 (*dst)[4], const uint16_t *X, int64_t ldx, int64_t d,
                                            int64_t row0, int64_t k0, int wave, int lane, int i) {
    const int row = wave * 64 + i * 16 + (lane >> 2);
    const int c = (lane & 3) ^ swz(row);
    int64_t gr = row0 + row;
    gr = gr < d ? gr : d - 1;
    const uint16_t *src = X + gr * ldx + k0 + c * 8;
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                     (__attribute__((address_space(3))) void *)(&dst[wave * 64 + i * 16][0]), 16, 0, 0);
}

// Channel-major pair stages: 64 tokens, so each row's piece is one whole
// 128-byte line.  Loads of 64-byte pieces (half a line per row per 32-token
// stage) streamed X into LDS at about 7.7 TB/s; whole lines at about 12 TB/s
// (same tiles, splits and work order, loads only).  Image: two slots of
// 256 rows x 128 B per panel; logical chunk c (tokens 8c .. 8c+7) of row r at
// position c ^ swz8(r).  Rows alternate between the two halves of the 64
// banks (128-byte pitch), so the 16 rows one b128 read pass touches at a
// common chunk spread over all 16 bank groups when swz8(r) = (r / 2) % 8.
constexpr int KP = 2 * KT;  // tokens per pair stage
struct PairSmem {
    uint4 a[2][TS][8];
    uint4 b[2][TS][8];
};

__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// One 1 KB piece of a pair stage: 8 rows x 128 B; wave w fills rows
// 64 w .. 64 w + 63 in eight pieces i = 0..7.  Rows past d are clamped to row
// d-1 (valid memory; those outputs are discarded).
__device__ __forceinline__ void pair_piece(uint4 (*dst)[8], const uint16_t *X, int64_t ldx, int64_t d, int64_t row0,
                                           int64_t k0, int wave, int lane, int i) {
    const int row = wave * 64 + i * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz8(row);
    int64_t gr = row0 + row;
    gr = gr < d ? gr : d - 1;
    const uint16_t *src = X + gr * ldx + k0 + c * 8;
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                     (__attribute__((address_space(3))) void *)(&dst[wave * 64 + i * 8][0]), 16, 0, 0);
}

// Channel-major: the same LDS image of a partial stage (tokens k0 .. kend-1,
// the rest zero) from masked register loads.
__device__ __forceinline__ void panel_tail(uint4 (*dst)[4], const uint16_t *X, int64_t ldx, int64_t d, int64_t row0,
                                           int64_t k0, int64_t kend, int tid) {
    for (int e = tid; e < TS * 4; e += kThreads) {
        const int row = e / 4, pos = e % 4;
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

// Token-major: tokens t0 .. t0+7 of four channels, one 8-byte word per token.
struct TokUnit {
    uint2 x[8];
};

// Chunk j of a unit (channel jr = j ^ r of the lane's four, r = (l / 4) % 4,
// token 2m in the low half of dword m as in memory order along tokens) into
// row 4 l + jr of a stage at logical chunk tg.  The lanes of a store write the
// four channels of their quad in different orders, which keeps every store
// free of bank conflicts.  The unit's dwords are pre-swapped when r / 2 = 1
// (tok_swap), so the dword choice is fixed per j and only the half-word
// choice (the byte-permute selector `sel`) depends on the lane.
__device__ __forceinline__ void tok_swap(TokUnit &u, bool swap) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t a = u.x[i].x, b = u.x[i].y;
        u.x[i].x = swap ? b : a;
        u.x[i].y = swap ? a : b;
    }
}

__device__ __forceinline__ void tok_store_chunk(uint4 (*dst)[4], const TokUnit &u, int l, int tg, int j,
                                                uint32_t sel) {
    const int jr = j ^ ((l >> 2) & 3);
    uint32_t w[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t lo = (j >> 1) ? u.x[2 * m].y : u.x[2 * m].x;
        const uint32_t hi = (j >> 1) ? u.x[2 * m + 1].y : u.x[2 * m + 1].x;
        w[m] = __builtin_amdgcn_perm(hi, lo, sel);
    }
    dst[4 * l + jr][tg ^ (l & 3)] = make_uint4(w[0], w[1], w[2], w[3]);  // position: tg ^ swz(4 l + jr)
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

template <int V>
using IC = std::integral_constant<int, V>;

// Operands of the matrix-core kernel below.
//   SYRK (MODE 0 channel-major, 1 token-major): A = B = X with d channels and
//     n_tok tokens; the upper tiles in band order, split over tokens.
//   GEMM (MODE 2): C[m][n] = bf16(sum_k A[m][k] B[n][k]), A [M][lda] and
//     B [N][ldb] both contiguous along k, C [M][ldc]; every tile, each XCD
//     taking a contiguous range of the row-major tile order.
struct MmaArgs {
    const uint16_t *A, *B;
    int64_t lda, ldb;
    int64_t ma, mb;  // rows of A and B
    int64_t K;       // the summed axis (tokens for the SYRK)
    // SYRK plan and outputs
    int64_t kchunk, ntiles;
    int nt, splits;
    float *H, *part;
    // GEMM output
    uint16_t *C;
    int64_t ldc;
};

// fp32 -> bf16 bit pattern, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// grid.x = 8 * ceil(tiles / 8) * splits (GEMM: 8 * ceil(tiles / 8)).  Each wave
// owns a 128 x 128 quarter of the 256 x 256 tile as 4 x 4
// v_mfma_f32_32x32x16_bf16 accumulators.  SYRK: part == nullptr: H += 2 acc
// (upper triangle); else the raw partial tile goes to
// part[split * ntiles + row-major tile index].
template <int MODE>
__global__ __launch_bounds__(kThreads) void mma_bf16_kernel(MmaArgs g) {
    constexpr bool TOK = MODE == 1, GEMM = MODE == 2;
    const uint16_t *__restrict__ X = g.A;
    const int64_t ldx = g.lda, d = g.ma;
    const int64_t xcd = blockIdx.x % kXCDs, slot = blockIdx.x / kXCDs;
    int ti, tj;
    int64_t split = 0;
    if constexpr (GEMM) {
        const int gx = (int)ceil_div(g.mb, TS);
        const int64_t tiles = (int64_t)gx * ceil_div(g.ma, TS);
        const int64_t t0 = xcd * tiles / kXCDs, t1 = (xcd + 1) * tiles / kXCDs;
        if (slot >= t1 - t0) return;
        ti = (int)((t0 + slot) / gx);
        tj = (int)((t0 + slot) % gx);
    } else {
        // XCD x owns band-order positions [g0, g1) and runs them split after split.
        const int64_t g0 = xcd * g.ntiles / kXCDs, g1 = (xcd + 1) * g.ntiles / kXCDs, gsz = g1 - g0;
        if (gsz <= 0 || slot >= gsz * g.splits) return;
        split = slot / gsz;
        tile_of_band(g0 + slot % gsz, g.nt, ti, tj);
    }
    const bool diag = !GEMM && ti == tj;
    const int64_t r0 = (int64_t)ti * TS, c0 = (int64_t)tj * TS;
    const int64_t kbeg = GEMM ? 0 : split * g.kchunk;
    const int64_t kend = GEMM ? g.K : ((kbeg + g.kchunk) < g.K ? (kbeg + g.kchunk) : g.K);

    __shared__ SyrkSmem sm;
    static_assert(sizeof(PairSmem) == sizeof(SyrkSmem), "the pair stages use the ring's memory");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
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
    // Operand p of a 16-token step: p < 4 is A row block p, else B row block p-4.
    auto read_frag = [&](int slot_, int ks, int p, Frags &f) {
        const int pos = (2 * ks + half) ^ sw;
        if (p < 4)
            f.a[p] = __builtin_bit_cast(bf16x8, sm.a[slot_][wm * 128 + p * 32 + lrow][pos]);
        else
            f.b[p - 4] = __builtin_bit_cast(bf16x8, sm.b[slot_][wn * 128 + (p - 4) * 32 + lrow][pos]);
    };
    auto mfma = [&](const Frags &f, int q) {
        acc[q >> 2][q & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[q >> 2], f.b[q & 3], acc[q >> 2][q & 3], 0, 0, 0);
    };

    // Channel-major: whole 64-token pair stages first, through two slots, the
    // next pair's loads one pair ahead; each pair is four 16-token steps of
    // the same MFMAs in the same token order as the 32-token stages below, so
    // H does not depend on how the tokens are staged.  Then at most one 32-token
    // stage and the tail.
    int64_t kb2 = kbeg;
    if constexpr (!TOK) {
        const int npair = kend > kbeg ? (int)((kend - kbeg) / KP) : 0;
        if (npair > 0) {
            PairSmem &ps = *reinterpret_cast<PairSmem *>(&sm);
            const int sw8 = swz8(lrow);
            auto read_pfrag = [&](int slot_, int hs, int p, Frags &f) {
                const int pos = (2 * hs + half) ^ sw8;
                if (p < 4)
                    f.a[p] = __builtin_bit_cast(bf16x8, ps.a[slot_][wm * 128 + p * 32 + lrow][pos]);
                else
                    f.b[p - 4] = __builtin_bit_cast(bf16x8, ps.b[slot_][wn * 128 + (p - 4) * 32 + lrow][pos]);
            };
            // Piece p (0..7: panel A, 8..15: panel B) of pair pr; past the end the
            // last pair again, into a slot nobody reads.
            auto issue_pair = [&](int pr, int slot_, int p) {
                const int64_t k0 = kbeg + (int64_t)min(pr, npair - 1) * KP;
                if (p < 8)
                    pair_piece(ps.a[slot_], g.A, g.lda, g.ma, r0, k0, wave, lane, p);
                else
                    pair_piece(ps.b[slot_], g.B, g.ldb, g.mb, c0, k0, wave, lane, p - 8);
            };
#pragma unroll
            for (int p = 0; p < 16; ++p) issue_pair(0, 0, p);
#pragma unroll
            for (int p = 0; p < 16; ++p) issue_pair(1, 1, p);
            wait_vm_lgkm0<16>();  // pair 0 landed
            bar();
            Frags f0, f1;
#pragma unroll
            for (int p = 0; p < 8; ++p) read_pfrag(0, 0, p, f0);
            for (int k = 0; k < npair; ++k) {
                const int cur = k & 1;
                // steps 0-2: the MFMAs of one step while the next step's operands are read
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    mfma(f0, q);
                    if (q >= 1 && q <= 8) read_pfrag(cur, 1, q - 1, f1);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    mfma(f1, q);
                    if (q >= 1 && q <= 8) read_pfrag(cur, 2, q - 1, f0);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    mfma(f0, q);
                    if (q >= 1 && q <= 8) read_pfrag(cur, 3, q - 1, f1);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // Step 3 holds its operands: this slot is free once every wave
                // has read them, and pair k + 1 (this wave's only loads in
                // flight) must have landed for every wave.
                wait_vm_lgkm0<0>();
                bar();
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    mfma(f1, q);
                    issue_pair(k + 2, cur, q);
                    if (q >= 7 && q <= 14) read_pfrag(cur ^ 1, 0, q - 7, f0);  // unused after the last pair
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            wait_vm_lgkm0<0>();
            kb2 = kbeg + (int64_t)npair * KP;
            __syncthreads();  // the 32-token ring below reuses the slots
        }
    }
    const int nfull = kend > kb2 ? (int)((kend - kb2) / KT) : 0;
    const bool has_tail = kend > kb2 + (int64_t)nfull * KT;

    // Token-major staging: wave w loads and stores units u = 0, 1 of a stage:
    // panel A (waves 0, 1) or B (waves 2, 3), 8-token chunk tg = 2 (w % 2) + u,
    // this lane's 4 channels.  Each token's row is addressed from a wave-uniform
    // base plus the lane's offset, past d clamped in bounds (discarded).
    const bool tok_b = wave >= 2;
    const int64_t tok_base = tok_b ? c0 : r0;
    const int tok_off = (int)min<int64_t>(4 * lane, ldx - 4 - tok_base);
    const uint32_t sel0 = (lane >> 2) & 1 ? 0x07060302u : 0x05040100u;  // chunk j: j & 1 ? sel1 : sel0
    const uint32_t sel1 = (lane >> 2) & 1 ? 0x05040100u : 0x07060302u;
    const bool tok_swapped = (lane >> 3) & 1;
    auto tok_load_one = [&](int st, TokUnit &r, int u, int i) {
        const int64_t t = kbeg + (int64_t)min(st, nfull - 1) * KT + 8 * (2 * (wave & 1) + u) + i;
        const uint16_t *rowp = X + t * ldx + tok_base;
        r.x[i] = *reinterpret_cast<const uint2 *>(rowp + tok_off);
    };
    auto tok_put_chunk = [&](int slot_, const TokUnit &r, int u, int j) {
        tok_store_chunk(tok_b ? sm.b[slot_] : sm.a[slot_], r, lane, 2 * (wave & 1) + u, j, (j & 1) ? sel1 : sel0);
    };

    if (nfull > 0) {
        if constexpr (!TOK) {
            // Exactly one stage is issued per step (past the end: the last
            // stage again, into a slot nobody reads), so the in-flight count is
            // fixed: at each wait, the stage being waited for is followed by one
            // more.
            auto issue_piece = [&](int st, int slot_, int p) {
                const int64_t k0 = kb2 + (int64_t)st * KT;
                if (p < 4)
                    panel_piece(sm.a[slot_], g.A, g.lda, g.ma, r0, k0, wave, lane, p);
                else
                    panel_piece(sm.b[slot_], g.B, g.ldb, g.mb, c0, k0, wave, lane, p - 4);
            };
#pragma unroll
            for (int st = 0; st < NS - 1; ++st)
#pragma unroll
                for (int p = 0; p < 8; ++p) issue_piece(min(st, nfull - 1), st, p);
            wait_vm_lgkm0<16>();  // stage 0 landed
            bar();
            Frags f0, f1;
#pragma unroll
            for (int p = 0; p < 8; ++p) read_frag(0, 0, p, f0);
            // Each step is two half-steps of 16 MFMAs; the LDS reads of the
            // other half's operands and the global->LDS loads of the stage NS-1
            // ahead are issued one per MFMA (the scheduling fences hold that
            // order), so the matrix core never waits on instruction issue.
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
                const int st = min(k + NS - 1, nfull - 1), slot_ = (k + NS - 1) % NS;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    mfma(f1, q);
                    if (q >= 1 && q <= 8) issue_piece(st, slot_, q - 1);
                    if (q >= 7 && q <= 14) read_frag(nxt, 0, q - 7, f0);  // unused after the last step
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            wait_vm_lgkm0<0>();
        } else {
            // Stage s: loaded into registers R[s % 3] during the second half of
            // step s - 5 (the prologue for s < 5), one token row per MFMA;
            // transposed into LDS slot s % 4 during the first half of step
            // s - 2, one chunk per MFMA; read from the second half of step s - 1
            // on.  Slot s % 4 last held stage s - 4, whose reads ended in step
            // s - 4, before the barrier of step s - 3 that every wave writing in
            // step s - 2 has passed.
            TokUnit R[3][2];
            auto load_stage = [&](int st, TokUnit(&r)[2]) {
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int i = 0; i < 8; ++i) tok_load_one(st, r[u], u, i);
            };
            auto put_stage = [&](int slot_, TokUnit(&r)[2]) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    tok_swap(r[u], tok_swapped);
#pragma unroll
                    for (int j = 0; j < 4; ++j) tok_put_chunk(slot_, r[u], u, j);
                }
            };
            load_stage(0, R[0]);
            load_stage(1, R[1]);
            load_stage(2, R[2]);
            put_stage(0, R[0]);
            load_stage(3, R[0]);
            put_stage(1, R[1]);
            load_stage(4, R[1]);
            wait_vm_lgkm0<63>();
            bar();
            Frags f0, f1;
#pragma unroll
            for (int p = 0; p < 8; ++p) read_frag(0, 0, p, f0);
            auto step = [&](int k, auto rbc) {
                constexpr int RB = decltype(rbc)::value;  // (k + 2) % 3
                TokUnit(&r)[2] = R[RB];
                const int cur = k % NS, nxt = (k + 1) % NS, put = (k + 2) % NS;
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    mfma(f0, q);
                    if (q >= 1 && q <= 8) read_frag(cur, 1, q - 1, f1);
                    if (q == 5) tok_swap(r[0], tok_swapped);  // stage k + 2
                    if (q == 7) tok_swap(r[1], tok_swapped);
                    if (q >= 8) tok_put_chunk(put, r[(q - 8) >> 2], (q - 8) >> 2, (q - 8) & 3);
                    __builtin_amdgcn_sched_barrier(0);
                }
                wait_vm_lgkm0<63>();  // this wave's LDS reads and writes are done
                bar();                // ... every wave's: stage k + 1 is complete in LDS
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    mfma(f1, q);
                    tok_load_one(k + 5, r[q >> 3], q >> 3, q & 7);
                    if (q >= 7 && q <= 14) read_frag(nxt, 0, q - 7, f0);  // unused after the last step
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            int k = 0;
            for (; k + 2 < nfull; k += 3) {
                step(k, IC<2>());
                step(k + 1, IC<0>());
                step(k + 2, IC<1>());
            }
            if (k < nfull) step(k, IC<2>());
            if (k + 1 < nfull) step(k + 1, IC<0>());
            wait_vm_lgkm0<0>();
        }
    }
    if (has_tail) {
        const int64_t k0 = kb2 + (int64_t)nfull * KT;
        __syncthreads();  // every wave is done with the ring
        if constexpr (!TOK) {
            panel_tail(sm.a[0], g.A, g.lda, g.ma, r0, k0, kend, tid);
            panel_tail(sm.b[0], g.B, g.ldb, g.mb, c0, k0, kend, tid);
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                TokUnit t;
                const int64_t t0 = k0 + 8 * (2 * (wave & 1) + u);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    t.x[i] = t0 + i < kend ? *reinterpret_cast<const uint2 *>(X + (t0 + i) * ldx + tok_base + tok_off)
                                           : make_uint2(0u, 0u);
                tok_swap(t, tok_swapped);
#pragma unroll
                for (int j = 0; j < 4; ++j) tok_put_chunk(0, t, u, j);
            }
        }
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

    if constexpr (GEMM) {
        // bf16 C, one 32 x 32 sub-tile at a time (32 lanes write 64 contiguous bytes)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = r0 + wm * 128 + i * 32 + mfma32_row(r, lane);
                    const int64_t n = c0 + wn * 128 + j * 32 + mfma32_col(lane);
                    if (m < g.ma && n < g.mb) g.C[m * g.ldc + n] = bf16_rne(acc[i][j][r]);
                }
        return;
    }
    if (g.part) {
        float *dst = g.part + (split * g.ntiles + tile_linear(ti, tj, g.nt)) * (TS * TS);
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
    float *H = g.H;
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

// hdiag[i] += 2 * sum_s part[s][i]  (fixed summation order).
__global__ __launch_bounds__(kThreads) void diag_reduce_kernel(const double *__restrict__ part, int splits, int64_t d,
                                                               double *__restrict__ hdiag) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= d) return;
    double s = 0.0;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * d + i];
    hdiag[i] += 2.0 * s;
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

// hdiag[i] += 2 * sum_t x_it^2 in fp64 (the act-order key), a pass of its own.
template <typename T>
__device__ __forceinline__ double widen(T v) {
    if constexpr (sizeof(T) == 2)
        return (double)__uint_as_float((uint32_t)v << 16);
    else
        return (double)v;
}

// Channel-major X[d][ldx]: one workgroup per channel; the row is read in
// 16-byte pieces (X and ldx * element size are 16-byte aligned), four pieces in
// flight per thread, the ragged end element-wise, then a tree sum.
template <typename T>
__global__ __launch_bounds__(kThreads) void diag_rows_kernel(const T *__restrict__ X, int64_t ldx, int64_t n_tok,
                                                             double *__restrict__ hdiag) {
    constexpr int kPer = 16 / sizeof(T);  // elements per 16-byte piece
    constexpr int kUnroll = 4;
    const int64_t i = blockIdx.x;
    const T *row = X + i * ldx;
    const int64_t npieces = n_tok / kPer;
    double s = 0.0;
    auto add_piece = [&](const uint4 &v) {
        const T *e = reinterpret_cast<const T *>(&v);
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const double x = widen<T>(e[k]);
            s = fma(x, x, s);
        }
    };
    int64_t p = threadIdx.x;
    for (; p + (kUnroll - 1) * kThreads < npieces; p += kUnroll * kThreads) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = *reinterpret_cast<const uint4 *>(row + (p + u * kThreads) * kPer);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) add_piece(v[u]);
    }
    for (; p < npieces; p += kThreads) add_piece(*reinterpret_cast<const uint4 *>(row + p * kPer));
    for (int64_t t = npieces * kPer + threadIdx.x; t < n_tok; t += kThreads) {
        const double x = widen<T>(row[t]);
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

// Token-major X[n][ldx]: a workgroup takes 64 EPL channels (EPL per lane: bf16
// four, one 8-byte load per token; fp32 one) over tokens [y tchunk, (y+1) tchunk)
// in four token phases, one per wave, summed in a fixed order.  part == nullptr:
// hdiag += 2 s; else part[y][c] = s for a fixed-order reduce.
template <typename T, int EPL>
__global__ __launch_bounds__(kThreads) void diag_cols_kernel(const T *__restrict__ X, int64_t ldx, int64_t d,
                                                             int64_t n_tok, int64_t tchunk,
                                                             double *__restrict__ hdiag, double *__restrict__ part) {
    const int lane = threadIdx.x & 63, ph = threadIdx.x >> 6;
    const int64_t c = ((int64_t)blockIdx.x * 64 + lane) * EPL;
    const int64_t t0 = (int64_t)blockIdx.y * tchunk;
    const int64_t t1 = min(n_tok, t0 + tchunk);
    double s[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) s[e] = 0.0;
    if (c < d) {
#pragma unroll 4
        for (int64_t t = t0 + ph; t < t1; t += 4) {
            if constexpr (EPL == 4) {  // bf16, c + 4 <= ldx (ldx a multiple of 4)
                const uint2 v = *reinterpret_cast<const uint2 *>(X + t * ldx + c);
                const uint32_t w[2] = {v.x, v.y};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double x = (double)__uint_as_float(e & 1 ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16));
                    s[e] = fma(x, x, s[e]);
                }
            } else {
                const double x = widen<T>(X[t * ldx + c]);
                s[0] = fma(x, x, s[0]);
            }
        }
    }
    __shared__ double red[4][64 * EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) red[ph][lane * EPL + e] = s[e];
    __syncthreads();
    for (int k = threadIdx.x; k < 64 * EPL; k += kThreads) {
        const int64_t ch = (int64_t)blockIdx.x * 64 * EPL + k;
        if (ch >= d) continue;
        const double v = ((red[0][k] + red[1][k]) + red[2][k]) + red[3][k];
        if (part)
            part[(int64_t)blockIdx.y * d + ch] = v;
        else
            hdiag[ch] += 2.0 * v;
    }
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
    p.kchunk = ceil_div(ceil_div(n_tok, best_s), KP) * KP;  // whole pair stages: 128-byte aligned rows
    p.splits = (int)ceil_div(n_tok, p.kchunk);
    if (p.splits < 1) p.splits = 1;
    return p;
}

// Token splits of the token-major diagonal pass: about 2048 workgroups, at
// least 1024 tokens each, at most 64 splits.
struct DiagPlan {
    int splits;
    int64_t tchunk;
};

DiagPlan plan_diag_cols(int64_t d, int64_t n_tok, int epl) {
    const int64_t blocks = ceil_div(d, 64 * epl);
    int64_t s = std::min<int64_t>({(int64_t)64, ceil_div(n_tok, 1024), ceil_div(2048, blocks)});
    if (s < 1) s = 1;
    DiagPlan p;
    p.tchunk = ceil_div(n_tok, s);
    p.splits = (int)ceil_div(n_tok, p.tchunk);
    return p;
}

size_t syrk_part_bytes(const SyrkPlan &p) {
    return p.splits > 1 ? align_up((size_t)p.splits * (size_t)p.ntiles * TS * TS * sizeof(float), 256) : 0;
}

size_t diag_part_bytes(int64_t d, int64_t n_tok, gptq_dtype dt) {
    const DiagPlan q = plan_diag_cols(d, n_tok, dt == GPTQ_DT_BF16 ? 4 : 1);
    return q.splits > 1 ? (size_t)q.splits * (size_t)d * sizeof(double) : 0;
}

}  // namespace

hipError_t run_linear_forward(uint16_t *Y, int64_t ldy, const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                              int64_t n_tok, int64_t d_prev, int64_t d_out, hipStream_t s) {
    if (n_tok <= 0 || d_out <= 0) return hipSuccess;
    MmaArgs a{};
    a.A = X;
    a.lda = ldx;
    a.ma = n_tok;
    a.B = W;
    a.ldb = ldw;
    a.mb = d_out;
    a.K = d_prev;
    a.C = Y;
    a.ldc = ldy;
    const int64_t tiles = ceil_div(n_tok, TS) * ceil_div(d_out, TS);
    hipLaunchKernelGGL(mma_bf16_kernel<2>, dim3((unsigned)(kXCDs * ceil_div(tiles, kXCDs))), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

// Tokens per chunk of the calibration pass: the chunk of layer inputs is about
// 128 MiB (it stays in the last-level cache between its write and the SYRK's
// reads), a multiple of 1024 tokens in [1024, 65536].
int64_t calibrate_chunk_tokens(int64_t d_in) {
    const int64_t ldy = (d_in + 3) / 4 * 4;
    int64_t c = ((int64_t)128 << 20) / (2 * ldy) / 1024 * 1024;
    return c < 1024 ? 1024 : (c > 65536 ? 65536 : c);
}

size_t calibrate_ws_bytes(int64_t d_in, int64_t n_tok) {
    if (n_tok <= 0) return 0;
    const int64_t chunk = std::min<int64_t>(calibrate_chunk_tokens(d_in), n_tok);
    const int64_t ldy = (d_in + 3) / 4 * 4;
    size_t h = hessian_ws_bytes(d_in, chunk, GPTQ_DT_BF16);
    if (n_tok % chunk) h = std::max(h, hessian_ws_bytes(d_in, n_tok % chunk, GPTQ_DT_BF16));
    return align_up((size_t)chunk * (size_t)ldy * 2, 256) + h;
}

hipError_t run_calibrate(float *H, double *hdiag, const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                         int64_t n_tok, int64_t d_prev, int64_t d_in, void *ws, hipStream_t s) {
    const int64_t chunk = std::min<int64_t>(calibrate_chunk_tokens(d_in), n_tok);
    const int64_t ldy = (d_in + 3) / 4 * 4;
    uint16_t *Y = static_cast<uint16_t *>(ws);
    void *hws = static_cast<char *>(ws) + align_up((size_t)chunk * (size_t)ldy * 2, 256);
    for (int64_t t0 = 0; t0 < n_tok; t0 += chunk) {
        const int64_t c = std::min<int64_t>(chunk, n_tok - t0);
        hipError_t e = run_linear_forward(Y, ldy, X + t0 * ldx, ldx, W, ldw, c, d_prev, d_in, s);
        if (e != hipSuccess) return e;
        if ((e = run_hessian(H, hdiag, Y, GPTQ_DT_BF16, d_in, c, ldy, true, hws, s)) != hipSuccess) return e;
    }
    return hipSuccess;
}

// The same for both layouts: the SYRK's partial tiles, then the token-major
// diagonal pass's partial sums.
size_t hessian_ws_bytes(int64_t d_in, int64_t n_tok, gptq_dtype dt) {
    if (n_tok <= 0) return 0;
    const size_t syrk = dt == GPTQ_DT_BF16 ? syrk_part_bytes(plan_syrk(d_in, n_tok)) : 0;
    return syrk + diag_part_bytes(d_in, n_tok, dt);
}

hipError_t run_hessian(float *H, double *hdiag, const void *X, gptq_dtype dt, int64_t d, int64_t n_tok, int64_t ldx,
                       bool token_major, void *ws, hipStream_t s) {
    if (n_tok <= 0) return hipSuccess;
    hipError_t e;
    size_t syrk_bytes = 0;
    if (dt == GPTQ_DT_BF16) {
        SyrkPlan p = plan_syrk(d, n_tok);
        syrk_bytes = syrk_part_bytes(p);
        float *part = p.splits > 1 ? static_cast<float *>(ws) : nullptr;
        const dim3 grid((unsigned)(kXCDs * ceil_div(p.ntiles, kXCDs) * p.splits));
        MmaArgs a{};
        a.A = a.B = static_cast<const uint16_t *>(X);
        a.lda = a.ldb = ldx;
        a.ma = a.mb = d;
        a.K = n_tok;
        a.kchunk = p.kchunk;
        a.ntiles = p.ntiles;
        a.nt = p.nt;
        a.splits = p.splits;
        a.H = H;
        a.part = part;
        if (token_major)
            hipLaunchKernelGGL(mma_bf16_kernel<1>, grid, dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL(mma_bf16_kernel<0>, grid, dim3(kThreads), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (part) {
            hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)(p.ntiles * (TS * TS / (kThreads * 4)))), dim3(kThreads),
                               0, s, part, p.splits, p.ntiles, p.nt, d, H);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else {
        // fp32: H += 2 X X^T (channel-major) or 2 X^T X (token-major) on the
        // fp32 matrix-core GEMM, upper tiles only.
        const float *Xf = static_cast<const float *>(X);
        GemmDesc g;
        g.M = d;
        g.N = d;
        g.K = n_tok;
        g.A = Xf;
        g.lda = ldx;
        g.a_trans = token_major ? 1 : 0;
        g.B = Xf;
        g.ldb = ldx;
        g.b_trans = token_major ? 0 : 1;
        g.C = H;
        g.ldc = d;
        g.alpha = 2.0f;
        g.beta = 1.0f;
        g.upper_only = 1;
        if ((e = launch_gemm_f32(g, s)) != hipSuccess) return e;
    }
    if (!hdiag) return hipSuccess;
    const bool bf = dt == GPTQ_DT_BF16;
    if (!token_major) {
        if (bf)
            hipLaunchKernelGGL(diag_rows_kernel<uint16_t>, dim3((unsigned)d), dim3(kThreads), 0, s,
                               static_cast<const uint16_t *>(X), ldx, n_tok, hdiag);
        else
            hipLaunchKernelGGL(diag_rows_kernel<float>, dim3((unsigned)d), dim3(kThreads), 0, s,
                               static_cast<const float *>(X), ldx, n_tok, hdiag);
        return hipGetLastError();
    }
    const int epl = bf ? 4 : 1;
    const DiagPlan q = plan_diag_cols(d, n_tok, epl);
    double *dpart = q.splits > 1 ? reinterpret_cast<double *>(static_cast<char *>(ws) + syrk_bytes) : nullptr;
    const dim3 grid((unsigned)ceil_div(d, 64 * epl), (unsigned)q.splits);
    if (bf)
        hipLaunchKernelGGL((diag_cols_kernel<uint16_t, 4>), grid, dim3(kThreads), 0, s,
                           static_cast<const uint16_t *>(X), ldx, d, n_tok, q.tchunk, hdiag, dpart);
    else
        hipLaunchKernelGGL((diag_cols_kernel<float, 1>), grid, dim3(kThreads), 0, s, static_cast<const float *>(X),
                           ldx, d, n_tok, q.tchunk, hdiag, dpart);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (dpart) {
        hipLaunchKernelGGL(diag_reduce_kernel, dim3((unsigned)ceil_div(d, kThreads)), dim3(kThreads), 0, s, dpart,
                           q.splits, d, hdiag);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gptq
