// fp32 products on the bf16 matrix cores, for the long trailing updates of the
// column pass:  C = alpha * op(A) op(B) + beta * C, each operand stored either
// K-major (A[m][k] at A[k * lda + m], B[k][n] at B[k * ldb + n]) or
// K-contiguous (A[m][k] at A[m * lda + k], B[k][n] at B[n * ldb + k]).
//
// Every fp32 operand value x is split exactly into three bf16 terms, each
// rounded to nearest even:
//   h = bf16(x),  m = bf16(x - h),  l = bf16(x - h - m) = x - h - m,
// so |m| <= 2^-8 |x| and |l| <= 2^-16 |x| (x - h has at most 16 significant
// bits, x - h - m at most 8).  A product a b is taken as its six terms of size
// 2^-16 |a b| and up,
//   l_a h_b + m_a m_b + h_a l_b + m_a h_b + h_a m_b + h_a h_b,
// each exact in fp32 and summed in fp32 by v_mfma_f32_32x32x16_bf16; the
// dropped terms m_a l_b + l_a m_b + l_a l_b stay below 2^-23 |a b|, the size of
// one fp32 rounding.  Six bf16 matrix-core products cost 6/16 of one fp32
// product (v_mfma_f32_32x32x2f32 runs at 1/16 of the bf16 rate).  Values
// beyond 2^127 (2 - 2^-8) would round h to infinity; the updates this serves
// stay far below that.
//
// 256 x 256 tiles per 4-wave workgroup, each wave 128 x 128 as 4 x 4 32x32
// accumulators.  K streams straight from global memory into a ring of four
// 16-deep fp32 LDS stages [16 k][256 wide] (global_load_lds_dwordx4), two
// stages ahead of the operand reads.  A lane's operand fragment is 8
// consecutive k of one row (A) or column (B), read as 4-byte words; the reads
// and splits of the next pieces run between the current pieces' products:
// B block j + 1 of this stage and A block j of the next one while the 24
// products of B block j run.
#include "common.h"

namespace gptq {
namespace {

constexpr int ST = 256;      // tile edge
constexpr int SK = 16;       // K per stage: one matrix-core step
constexpr int SNS = 4;       // stages in the ring
constexpr int kThr = 256;    // 4 waves
constexpr int kXcds = 8;     // L2 domains: workgroup i runs on domain i % 8

struct SplitSmem {
    float a[SNS][SK * ST];
    float b[SNS][SK * ST];
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values rounded to nearest even bf16, the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
    const floatx2 f = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

struct Split {
    u32x4 h, m, l;  // bf16 pairs
};

// The split of values v[2p], v[2p + 1] into pair p of the three terms, in
// three pieces (5, 5 and 1 VALU) that sit between matrix-core products.
struct PairSplit {
    uint32_t hp, mp;
    float r0, r1;  // what the terms so far leave of the two values
};

__device__ __forceinline__ void split_a(const float (&v)[8], int p, PairSplit &t) {
    const float x0 = v[2 * p], x1 = v[2 * p + 1];
    t.hp = pack_bf16(x0, x1);
    t.r0 = x0 - __uint_as_float(t.hp << 16);
    t.r1 = x1 - __uint_as_float(t.hp & 0xffff0000u);
}

__device__ __forceinline__ void split_b(PairSplit &t) {
    t.mp = pack_bf16(t.r0, t.r1);
    t.r0 -= __uint_as_float(t.mp << 16);
    t.r1 -= __uint_as_float(t.mp & 0xffff0000u);
}

__device__ __forceinline__ void split_c(const PairSplit &t, int p, Split &s) {
    s.h[p] = t.hp;
    s.m[p] = t.mp;
    s.l[p] = pack_bf16(t.r0, t.r1);
}

__device__ __forceinline__ void split3(const float (&v)[8], Split &s) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        PairSplit t;
        split_a(v, p, t);
        split_b(t);
        split_c(t, p, s);
    }
}

// Stage layouts (16 KB per operand), each written by four 1 KB
// global_load_lds_dwordx4 per wave (instruction i of wave w: rows 4 w + i,
// or rows 16 (4 w + i) .. + 15):
//   K-major [16 k][256 wide] (A stored [k][m], B stored [k][n]): the 16-byte
//     chunk of wide columns 4c .. 4c+3 of row k sits at position
//     c ^ (8 ((k / 8) % 2)); a fragment read touches rows t and 8 + t (lanes
//     0-31 and 32-63), which then fall in complementary halves of the 64 banks.
//   K-contiguous [256 wide][16 k] (A stored [m][k], B stored [n][k]): the chunk
//     of k values 4c .. 4c+3 of row w sits at position c ^ ((w / 4) % 4), so
//     the 16 lanes of one b128 read pass (16 consecutive rows) use 16 distinct
//     16-byte bank groups.
// Wide rows at or past `lim` read the tile's first one instead (valid memory;
// their products land in outputs that are never stored).
template <int KM>
__device__ __forceinline__ void stage_load(float *dst, const float *src, int64_t ld, int64_t k0, int64_t w0,
                                           int64_t lim, int wave, int lane, int i) {
    const float *gp;
    if constexpr (KM) {
        const int kk = 4 * wave + i;
        const int c = lane ^ (((kk >> 3) & 1) << 3);
        int64_t w = w0 + 4 * c;
        w = w < lim ? w : w0;
        gp = src + (k0 + kk) * ld + w;
    } else {
        const int r = 64 * wave + 16 * i + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 2) & 3);
        int64_t w = w0 + r;
        w = w < lim ? w : w0;
        gp = src + w * ld + k0 + 4 * c;
    }
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(gp),
                                     (__attribute__((address_space(3))) void *)(dst + (4 * wave + i) * ST), 16, 0, 0);
}

// This lane's fragment of the 32 rows (or columns) from `base` (a multiple of
// 32): k = 8 half .. 8 half + 7 of wide index base + lrow.  K-major: wide index
// w of row k = 8 half + t sits at t * ST + (w ^ 32 half); K-contiguous: two
// 16-byte chunks of row w.
template <int KM>
__device__ __forceinline__ void frag_read(const float *stage, int base, int half, int lrow, float (&v)[8]) {
    if constexpr (KM) {
        const float *p = stage + 8 * half * ST + (base ^ (half << 5)) + lrow;
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = p[t * ST];
    } else {
        const int w = base + lrow, sw = (w >> 2) & 3;
        const float *row = stage + w * SK;
        const float4 x = *reinterpret_cast<const float4 *>(row + 4 * ((2 * half) ^ sw));
        const float4 y = *reinterpret_cast<const float4 *>(row + 4 * ((2 * half + 1) ^ sw));
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    }
}

template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | ((n >> 4) << 14));
}

__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int V>
struct IC {
    static constexpr int value = V;
};

template <int AKM, int BKM>
__global__ __launch_bounds__(kThr) void gemm_split_kernel(GemmDesc g) {
    const int gx = (int)ceil_div(g.N, ST);
    // upper_only (M = N): only the tiles on and above the diagonal, row-major
    const int64_t tiles = g.upper_only ? (int64_t)gx * (gx + 1) / 2 : (int64_t)gx * ceil_div(g.M, ST);
    // L2 domain x runs tiles [t0, t1) in row-major order: its resident
    // workgroups share rows of A.
    const int64_t xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int64_t t0 = xcd * tiles / kXcds, t1 = (xcd + 1) * tiles / kXcds;
    if (slot >= t1 - t0) return;
    int64_t tm = (t0 + slot) / gx, tn = (t0 + slot) % gx;
    if (g.upper_only) {
        int64_t t = t0 + slot, i = 0;
        while (t >= gx - i) t -= gx - i++;  // row i holds gx - i tiles
        tm = i;
        tn = i + t;
    }
    const int64_t m0 = tm * ST, n0 = tn * ST;
    // Triangular operands are zero outside their triangle: A upper (A[m][k] = 0
    // for k < m) starts K at the tile's first row, B upper (B[k][n] = 0 for
    // k > n) ends it after the tile's last column.  Both ends are multiples of
    // 256 or K, so the stage count stays even.
    int64_t kbeg = 0, kend = g.K;
    if (g.a_upper) kbeg = m0 < g.K ? m0 : g.K;
    if (g.b_upper) kend = n0 + ST < g.K ? n0 + ST : g.K;
    const int nst = kend > kbeg ? (int)((kend - kbeg) / SK) : 0;

    __shared__ SplitSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, half = lane >> 5, lrow = lane & 31;

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Load `part` (0 .. 7: A's four rows, then B's) of stage st; past the end
    // the last stage again, into a slot nobody reads, so the loads in flight
    // at each wait are fixed.
    auto issue = [&](int st, int part) {
        const int64_t k0 = kbeg + (int64_t)(st < nst ? st : nst - 1) * SK;
        if (part < 4)
            stage_load<AKM>(sm.a[st % SNS], g.A, g.lda, k0, m0, g.M, wave, lane, part);
        else
            stage_load<BKM>(sm.b[st % SNS], g.B, g.ldb, k0, n0, g.N, wave, lane, part - 4);
    };

    Split ap[2][4], bp[2];
    float ra[2][8], rb[8];
    // Product q (0 .. 11) of one half of B block j's 24: A block 2 hf + q % 2,
    // term q / 2 (l h, m m, h l, m h, h m, h h); two accumulators alternate.
    auto product = [&](const Split(&a)[4], const Split &b, int j, int hf, int q) {
        const int i = 2 * hf + (q & 1), t = q >> 1;
        const u32x4 x = t == 0 ? a[i].l : t == 1 || t == 3 ? a[i].m : a[i].h;
        const u32x4 y = t == 0 || t == 3 || t == 5 ? b.h : t == 1 || t == 4 ? b.m : b.l;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y),
                                                            acc[i][j], 0, 0, 0);
    };
    // Twelve products with the split of fragment v (read a step or half a step
    // earlier) into dst between them, one piece per product.
    auto half_step = [&](const Split(&a)[4], const Split &b, int j, int hf, const float(&v)[8], Split &dst) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            PairSplit t;
            __builtin_amdgcn_sched_barrier(0);
            split_a(v, p, t);
            __builtin_amdgcn_sched_barrier(0);
            product(a, b, j, hf, 3 * p);
            __builtin_amdgcn_sched_barrier(0);
            split_b(t);
            __builtin_amdgcn_sched_barrier(0);
            product(a, b, j, hf, 3 * p + 1);
            __builtin_amdgcn_sched_barrier(0);
            split_c(t, p, dst);
            __builtin_amdgcn_sched_barrier(0);
            product(a, b, j, hf, 3 * p + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Stage st from registers: step j takes B block j against A blocks 0, 1
    // (while the A fragment read a step earlier is split: this stage's block 3
    // at j = 0, else the next stage's block j - 1) and A blocks 2, 3 (while B
    // block j + 1, read at the step's start, is split).  Each step reads the
    // next B fragment and the next stage's A block j, and issues two of the
    // eight loads of stage st + 3.
    auto stage = [&](int st, auto cur_c) {
        constexpr int CUR = decltype(cur_c)::value;
        wait_vm<8>();  // this wave's loads of stage st + 1 landed (stage st + 2's may be in flight)
        barrier();     // ... and every wave's; every wave is done with stage st - 1's slot
        const float *a_next = sm.a[(st + 1) % SNS];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float *b_src = j < 3 ? sm.b[st % SNS] : sm.b[(st + 1) % SNS];
            frag_read<BKM>(b_src, wn * 128 + 32 * ((j + 1) & 3), half, lrow, rb);
            frag_read<AKM>(a_next, wm * 128 + 32 * j, half, lrow, ra[j & 1]);
            issue(st + 3, 2 * j);
            issue(st + 3, 2 * j + 1);
            half_step(ap[CUR], bp[j & 1], j, 0, ra[(j + 1) & 1], j == 0 ? ap[CUR][3] : ap[CUR ^ 1][(j + 3) & 3]);
            half_step(ap[CUR], bp[j & 1], j, 1, rb, bp[(j + 1) & 1]);
        }
    };

    if (nst > 0) {
#pragma unroll
        for (int st = 0; st < 3; ++st)
#pragma unroll
            for (int part = 0; part < 8; ++part) issue(st, part);
        wait_vm<16>();  // stage 0 landed
        barrier();
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            frag_read<AKM>(sm.a[0], wm * 128 + 32 * i, half, lrow, ra[0]);
            split3(ra[0], ap[0][i]);
        }
        frag_read<AKM>(sm.a[0], wm * 128 + 96, half, lrow, ra[1]);  // split during the first step
        frag_read<BKM>(sm.b[0], wn * 128, half, lrow, rb);
        split3(rb, bp[0]);
        for (int st = 0; st < nst; st += 2) {  // nst is even
            stage(st, IC<0>{});
            stage(st + 1, IC<1>{});
        }
        wait_vm<0>();
    }

    // C = alpha acc + beta C; interior tiles without bounds checks.
    // with upper_only, a diagonal tile stores only m <= n
    const bool full = m0 + ST <= g.M && n0 + ST <= g.N && !(g.upper_only && m0 == n0);
    // Accumulator block (i, j) of this lane: element r at row dr(r), column 0.
    auto cptr = [&](int i, int j) {
        const int64_t mb = m0 + wm * 128 + i * 32 + 4 * half, n = n0 + wn * 128 + j * 32 + lrow;
        return g.C + mb * g.ldc + n;
    };
    auto dr = [](int r) { return 8 * (r >> 2) + (r & 3); };
    if (full && g.beta != 0.0f) {
        // The operand registers are free now: C is read two accumulator
        // blocks at a time (32 loads per lane), the next pair's loads issued
        // before this pair's stores.
        float cold[2][2][16];
        auto load_pair = [&](int p, float(&c)[2][16]) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const float *cp = cptr(p >> 1, 2 * (p & 1) + jj);
#pragma unroll
                for (int r = 0; r < 16; ++r) c[jj][r] = cp[dr(r) * g.ldc];
            }
        };
        load_pair(0, cold[0]);
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            if (p + 1 < 8) load_pair(p + 1, cold[(p + 1) & 1]);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int i = p >> 1, j = 2 * (p & 1) + jj;
                float *cp = cptr(i, j);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float v = g.alpha * acc[i][j][r];
                    v += g.beta * cold[p & 1][jj][r];
                    cp[dr(r) * g.ldc] = v;
                }
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t mb = m0 + wm * 128 + i * 32 + 4 * half, n = n0 + wn * 128 + j * 32 + lrow;
            float *cp = g.C + mb * g.ldc + n;
            if (full) {
#pragma unroll
                for (int r = 0; r < 16; ++r) cp[(8 * (r >> 2) + (r & 3)) * g.ldc] = g.alpha * acc[i][j][r];
            } else if (n < g.N) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int dr = 8 * (r >> 2) + (r & 3);
                    if (mb + dr < g.M && (!g.upper_only || mb + dr <= n)) {
                        float v = g.alpha * acc[i][j][r];
                        if (g.beta != 0.0f) v += g.beta * cp[dr * g.ldc];
                        cp[dr * g.ldc] = v;
                    }
                }
            }
        }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

bool gemm_split_supported(const GemmDesc &g) {
    // 16-byte chunks wholly inside or outside: aligned bases and leading
    // dimensions, the contiguous extents (M or N when K-major, else K) multiples of 4.
    return (!g.upper_only || g.M == g.N) && g.batch == 1 && g.epilogue == EPI_STORE && g.K > 0 &&
           g.K % (2 * SK) == 0 && aligned16(g.A) && aligned16(g.B) && g.lda % 4 == 0 && g.ldb % 4 == 0 &&
           (!g.a_trans || g.M % 4 == 0) && (g.b_trans || g.N % 4 == 0);
}

hipError_t launch_gemm_split(const GemmDesc &g, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0) return hipSuccess;
    if (!gemm_split_supported(g)) return hipErrorInvalidValue;
    const int64_t gx = ceil_div(g.N, ST);
    const int64_t tiles = g.upper_only ? gx * (gx + 1) / 2 : ceil_div(g.M, ST) * gx;
    const dim3 grid((unsigned)(kXcds * ceil_div(tiles, kXcds)));
    const int akm = g.a_trans ? 1 : 0, bkm = g.b_trans ? 0 : 1;
    if (akm && bkm)
        hipLaunchKernelGGL((gemm_split_kernel<1, 1>), grid, dim3(kThr), 0, s, g);
    else if (akm)
        hipLaunchKernelGGL((gemm_split_kernel<1, 0>), grid, dim3(kThr), 0, s, g);
    else if (bkm)
        hipLaunchKernelGGL((gemm_split_kernel<0, 1>), grid, dim3(kThr), 0, s, g);
    else
        hipLaunchKernelGGL((gemm_split_kernel<0, 0>), grid, dim3(kThr), 0, s, g);
    return hipGetLastError();
}

}  // namespace gptq
