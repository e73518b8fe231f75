// After the pass: the codes packed into words, and the W4A16 product that
// consumes them (page "量化经典：LLM.int8 / GPTQ / AWQ", GPTQ section: 3/4-bit
// weights plus scales, activations stay 16-bit; page "LLM 量化方法原理与实现
// 详解", §6.2 W4A16 and §2.2 dequantization x = (q - z) s).
//
// Packed format: the codes of a row as one little-endian bit stream, code k
// at bits [b k, b k + b), in 32-bit words, the tail padded with zero bits.
//
// Product Y = X' W^T with W[o][k] = (q[o][k] - z[o][k/g]) s[o][k/g]:
//   * each lane turns one packed word (8 codes) into 8 fp16 values q - z,
//     exactly: 0x6400 | q is the fp16 number 1024 + q, and subtracting 1024 + z
//     in packed fp16 is exact;
//   * v_mfma_f32_32x32x16_f16 multiplies them with the fp16 activations, so
//     every product is exact and only the fp32 sums round;
//   * the scale is applied per group on the accumulators in fp32
//     (acc += s * acc_group), never rounded into the weights.
// Work is split over K when the output tiles alone would leave the chip idle
// (decode: M of a few tokens); the partial sums are added in a fixed order.
#include <algorithm>

#include "common.h"

namespace gptq {
namespace {

constexpr int kThreads = 256;
constexpr int kTileN = 128;  // output features per workgroup (4 waves x 32)

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Word w of row o covers stream bits [32 w, 32 w + 32).  Codes are masked to
// the bit width, so a bad code cannot spill into its neighbours.
__global__ __launch_bounds__(kThreads) void pack_codes_kernel(const uint8_t *__restrict__ codes, int64_t d_out,
                                                              int64_t d_in, int bits, const int32_t *__restrict__ perm,
                                                              uint32_t *__restrict__ packed, int64_t ldp) {
    const int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (w >= ldp) return;
    const uint32_t mask = (1u << bits) - 1u;
    const int64_t b0 = 32 * w;
    const int64_t k_lo = b0 / bits;
    const int64_t k_hi = std::min<int64_t>(d_in, (b0 + 32 + bits - 1) / bits);  // codes starting below b0 + 32
    for (int64_t o = blockIdx.y; o < d_out; o += gridDim.y) {
        const uint8_t *row = codes + o * d_in;
        uint32_t v = 0;
        for (int64_t k = k_lo; k < k_hi; ++k) {
            int64_t c = perm ? perm[k] : k;
            c = c < 0 ? 0 : (c >= d_in ? d_in - 1 : c);
            const uint32_t q = row[c] & mask;
            const int64_t sh = bits * k - b0;  // in (-bits, 32)
            v |= sh >= 0 ? q << sh : q >> (-sh);
        }
        packed[o * ldp + w] = v;
    }
}

// The activations in the operand order: Xp[m][8 c + j] = X[m][kp(8 c + il(j))]
// with il = (0, 4, 1, 5, 2, 6, 3, 7) (the order dequant8 yields the codes of a
// word in) and kp = kperm, or the identity.  d_in is a multiple of 8.
__global__ __launch_bounds__(kThreads) void gather_cols_kernel(const uint16_t *__restrict__ X, int64_t ldx, int64_t M,
                                                               int64_t d_in, const int32_t *__restrict__ kperm,
                                                               uint16_t *__restrict__ Xp, int64_t ldxp) {
    const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (k >= d_in) return;
    const int j = (int)(k & 7);
    const int64_t src = (k & ~(int64_t)7) + ((j & 1) ? 4 + (j >> 1) : (j >> 1));
    int64_t c = kperm ? kperm[src] : src;
    c = c < 0 ? 0 : (c >= d_in ? d_in - 1 : c);
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) Xp[m * ldxp + k] = X[m * ldx + c];
}

// Eight 4-bit codes (code i at bits 4i) as fp16 (code - z), exactly, in the
// order 0, 4, 1, 5, 2, 6, 3, 7 (the activations are stored in the same order
// within each 8-column chunk).  Masking a code into mantissa bits 0-3 or 4-7
// of an fp16 with exponent 10 gives 1024 + q or 1024 + 16 q:
//   codes 0, 4:  (w      & 0x000F000F) | 0x6400 6400 -> 1024 + q, minus (1024 + z)
//   codes 1, 5:  (w      & 0x00F000F0) | 0x6400 6400 -> 1024 + 16 q, times 1/16 minus (64 + z)
//   codes 2, 6 and 3, 7: the same on w >> 8.
// Each result is a small integer, so the packed fp16 add and fma are exact.
struct Bias {
    f16x2 b1;   // 1024 + z
    f16x2 b16;  // 64 + z
};
__device__ __forceinline__ Bias bias_of(float z) {
    Bias b;
    b.b1[0] = b.b1[1] = (_Float16)(1024.0f + z);
    b.b16[0] = b.b16[1] = (_Float16)(64.0f + z);
    return b;
}
// The exponent pattern is passed in a register (`magic`): a VOP3 instruction on
// this architecture takes no literal, so a register operand is what lets each
// mask-and-insert be one v_and_or_b32.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, const Bias &b, uint32_t magic) {
    const uint32_t w8 = w >> 8;
    f16x2 sixteenth;
    sixteenth[0] = sixteenth[1] = (_Float16)0.0625f;
    const f16x2 h0 = __builtin_bit_cast(f16x2, (w & 0x000F000Fu) | magic) - b.b1;
    const f16x2 h1 = __builtin_bit_cast(f16x2, (w & 0x00F000F0u) | magic) * sixteenth - b.b16;
    const f16x2 h2 = __builtin_bit_cast(f16x2, (w8 & 0x000F000Fu) | magic) - b.b1;
    const f16x2 h3 = __builtin_bit_cast(f16x2, (w8 & 0x00F000F0u) | magic) * sixteenth - b.b16;
    f16x8 r;
    r[0] = h0[0];  // code 0
    r[1] = h0[1];  // code 4
    r[2] = h1[0];  // code 1
    r[3] = h1[1];  // code 5
    r[4] = h2[0];  // code 2
    r[5] = h2[1];  // code 6
    r[6] = h3[0];  // code 3
    r[7] = h3[1];  // code 7
    return r;
}

// One workgroup: 128 output features x 32 TM tokens over K range
// [kb, kb + kspan).  Wave w owns features 32 w .. 32 w + 31; lane l supplies
// feature l % 32 of the weight operand and token l % 32 of each activation
// block.  K advances in steps of 16 U columns (U MFMAs): lane half h takes
// packed words U h .. U h + U - 1 of the step (one 4U-byte load) and the
// matching 8 U activations (one contiguous 16U-byte load), and MFMA u uses
// word U h + u -- A and B agree on every K index, which is all the product
// needs.  Two steps form a body, which never crosses a group (32 U divides
// g); each body's sum is scaled into the accumulators at its end (the same
// as once per group, up to fp32 rounding).  The main loop is branch-free:
// operands are read three steps ahead into a ring of four slots (two bodies
// per iteration), and each body's scale and zero a body ahead.
// (Used for more than 32 tokens; fewer take the few-token kernels below.)
template <int U>
struct WordsT;
template <>
struct WordsT<1> {
    typedef uint32_t T;
};
template <>
struct WordsT<2> {
    typedef uint2 T;
};
template <>
struct WordsT<4> {
    typedef uint4 T;
};
__device__ __forceinline__ uint32_t word_at(const uint32_t &w, int) { return w; }
__device__ __forceinline__ uint32_t word_at(const uint2 &w, int u) { return u == 0 ? w.x : w.y; }
__device__ __forceinline__ uint32_t word_at(const uint4 &w, int u) { return u == 0 ? w.x : (u == 1 ? w.y : (u == 2 ? w.z : w.w)); }

template <int TM, int U>
__global__ __launch_bounds__(kThreads) void w4a16_kernel(const _Float16 *__restrict__ X, int64_t ldx, int64_t M,
                                                         int64_t d_in, const uint32_t *__restrict__ packed, int64_t ldp,
                                                         const float *__restrict__ scales,
                                                         const float *__restrict__ zeros, int64_t g, int64_t ng,
                                                         int64_t d_out, int64_t kspan, float *__restrict__ out,
                                                         int64_t ldo, int64_t split_stride) {
    constexpr int KS = 16 * U;  // K columns per step
    constexpr int BL = 2 * KS;  // K columns per body
    constexpr int NS = 4;       // ring slots: operands are read NS - 1 steps ahead
    typedef typename WordsT<U>::T Words;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int64_t o = (int64_t)blockIdx.x * kTileN + wave * 32 + (lane & 31);
    const int64_t oc = o < d_out ? o : d_out - 1;
    const int64_t m0 = (int64_t)blockIdx.y * 32 * TM;
    const int64_t kb = (int64_t)blockIdx.z * kspan;
    const int64_t ke = std::min<int64_t>(d_in, kb + kspan);
    if (kb >= ke) return;  // uniform over the workgroup
    const int64_t nsteps = (ke - kb) / KS, nbody = nsteps / 2;
    const uint32_t *brow = packed + oc * ldp + U * half;  // + k / 8
    const _Float16 *arow[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int64_t m = m0 + 32 * t + (lane & 31);
        const int64_t mc = m < M ? m : M - 1;
        arow[t] = X + mc * ldx + 8 * U * half;  // + k
    }
    floatx16 acc[TM], accg[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = accg[t][r] = 0.0f;

    const float *srow = scales + oc * ng, *zrow = zeros + oc * ng;
    auto body_group = [&](int64_t b) {  // clamped: reads past the end are harmless
        const int64_t bb = b < nbody ? b : nbody - 1;
        return (kb + bb * BL) / g;
    };
    // scale and zero of the even and the odd body of an iteration
    float se = srow[body_group(0)], ze = zrow[body_group(0)];
    float so = srow[body_group(1)], zo = zrow[body_group(1)];

    Words bw[NS];
    f16x8 a[NS][TM][U];
    auto load = [&](int slot, int64_t step) {
        const int64_t k = kb + (step < nsteps ? step : nsteps - 1) * KS;
        bw[slot] = *reinterpret_cast<const Words *>(brow + k / 8);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < U; ++u) a[slot][t][u] = *reinterpret_cast<const f16x8 *>(arow[t] + k + 8 * u);
    };
    uint32_t magic = 0x64006400u;  // fp16 exponent of 1024 in both halves, kept in a register
    asm volatile("" : "+v"(magic));
    auto mma = [&](int slot, const Bias &bias) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const f16x8 b = dequant8(word_at(bw[slot], u), bias, magic);
#pragma unroll
            for (int t = 0; t < TM; ++t) accg[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[slot][t][u], b, accg[t], 0, 0, 0);
        }
    };
    auto fold = [&](float sc) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[t][r] = fmaf(sc, accg[t][r], acc[t][r]);
                accg[t][r] = 0.0f;
            }
    };
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) load(p, p);

    int64_t step = 0;
    for (int64_t b = 0; b + 2 <= nbody; b += 2, step += 4) {
        {  // even body: steps 0, 1
            const Bias bias = bias_of(ze);
            load(3, step + 3);
            mma(0, bias);
            load(0, step + 4);
            mma(1, bias);
            fold(se);
            se = srow[body_group(b + 2)];
            ze = zrow[body_group(b + 2)];
        }
        {  // odd body: steps 2, 3
            const Bias bias = bias_of(zo);
            load(1, step + 5);
            mma(2, bias);
            load(2, step + 6);
            mma(3, bias);
            fold(so);
            so = srow[body_group(b + 3)];
            zo = zrow[body_group(b + 3)];
        }
    }
    if (nbody & 1) {  // the last body (slots 0 and 1 hold its operands)
        const Bias bias = bias_of(ze);
        mma(0, bias);
        mma(1, bias);
        fold(se);
    }
    if (o >= d_out) return;
    float *dst = out + (int64_t)blockIdx.z * split_stride + o;
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + 32 * t + mfma32_row(r, lane);
            if (m < M) dst[m * ldo] = acc[t][r];
        }
}

// Staging of the few-token kernels: the workgroup's rows of X over [kb, ke)
// into xs (rows ldxs halves apart), and the scales and zeros of its 128
// features over groups g0 .. g0 + ngs - 1 into sz ([group][feature][scale,
// zero]).  Every load is issued before the first store (batches of 8 pieces of
// X; one feature's contiguous run of scales or of zeros per thread), so the
// staging costs about one memory latency.  ngs <= kMaxGroups.
constexpr int kMaxGroups = 32;
__device__ __forceinline__ void stage_few(const _Float16 *__restrict__ X, int64_t ldx, int64_t M, int64_t kb,
                                          int64_t ke, _Float16 *xs, int64_t ldxs, const float *__restrict__ scales,
                                          const float *__restrict__ zeros, int64_t ng, int64_t n0, int64_t d_out,
                                          int64_t g0, int64_t ngs, float *sz) {
    const int tid = threadIdx.x;
    {
        const int f = tid >> 1;  // feature of the tile; tid & 1: scales or zeros
        const int64_t of = n0 + f < d_out ? n0 + f : d_out - 1;
        const float *src = ((tid & 1) ? zeros : scales) + of * ng + g0;
        float v[kMaxGroups];
#pragma unroll
        for (int j = 0; j < kMaxGroups; ++j)
            if (j < ngs) v[j] = src[j];
#pragma unroll
        for (int j = 0; j < kMaxGroups; ++j)
            if (j < ngs) sz[(j * kTileN + f) * 2 + (tid & 1)] = v[j];
    }
    const int64_t chunks = (ke - kb) / 8;  // 16-byte pieces per row
    const int64_t n = M * chunks;
    for (int64_t i0 = 0; i0 < n; i0 += 8 * kThreads) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = i0 + u * kThreads + tid;
            const int64_t ic = i < n ? i : n - 1;
            v[u] = *reinterpret_cast<const uint4 *>(X + (ic / chunks) * ldx + kb + 8 * (ic % chunks));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = i0 + u * kThreads + tid;
            if (i < n) *reinterpret_cast<uint4 *>(xs + (i / chunks) * ldxs + 8 * (i % chunks)) = v[u];
        }
    }
}

// Few tokens (M <= 32): the product is a stream of packed weights.  The
// workgroup first stages in LDS its rows of X over [kb, ke) and the scales and
// zeros of its 128 features over the groups the range touches; the loop then
// issues one global load per step (the lane's packed words), kNB - 1 steps
// ahead through a ring of kNB slots, reads the activation operand from LDS
// one step ahead, and folds each two-step body with its group's scale.
// Bodies past the end of the range (the last chunk of kNB steps may overrun
// it) read clamped addresses and fold with scale 0, so the loop has no
// branches.  Lane layout and K order are those of w4a16_kernel.
constexpr int kNB = 8;  // packed-word ring slots (steps of look-ahead + 1)

template <int U>
__global__ __launch_bounds__(kThreads) void w4a16_few_kernel(const _Float16 *__restrict__ X, int64_t ldx, int64_t M,
                                                             int64_t d_in, const uint32_t *__restrict__ packed,
                                                             int64_t ldp, const float *__restrict__ scales,
                                                             const float *__restrict__ zeros, int64_t g, int64_t ng,
                                                             int64_t d_out, int64_t kspan, float *__restrict__ out,
                                                             int64_t ldo, int64_t split_stride) {
    constexpr int KS = 16 * U;  // K columns per step
    constexpr int BL = 2 * KS;  // K columns per body
    typedef typename WordsT<U>::T Words;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int64_t n0 = (int64_t)blockIdx.x * kTileN;
    const int fl = wave * 32 + (lane & 31);  // feature within the tile
    const int64_t o = n0 + fl;
    const int64_t oc = o < d_out ? o : d_out - 1;
    const int64_t kb = (int64_t)blockIdx.z * kspan;
    const int64_t ke = std::min<int64_t>(d_in, kb + kspan);
    if (kb >= ke) return;  // uniform over the workgroup
    const int64_t nsteps = (ke - kb) / KS, nbody = nsteps / 2;
    const int64_t g0 = kb / g, ngs = (ke - 1) / g - g0 + 1;  // groups the range touches

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int64_t ldxs = kspan + 8;  // halves; the pad staggers the banks
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem);
    float2 *szs = reinterpret_cast<float2 *>(smem + align_up((size_t)M * (size_t)ldxs * 2, 16));  // [group][feature]
    stage_few(X, ldx, M, kb, ke, xs, ldxs, scales, zeros, ng, n0, d_out, g0, ngs, reinterpret_cast<float *>(szs));
    __syncthreads();

    const uint32_t *brow = packed + oc * ldp + U * half + kb / 8;  // + 2 U step
    const int64_t mc = (lane & 31) < M ? (lane & 31) : M - 1;
    const _Float16 *arow = xs + mc * ldxs + 8 * U * half;  // + KS step
    floatx16 acc, accg;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = accg[r] = 0.0f;
    uint32_t magic = 0x64006400u;  // fp16 exponent of 1024 in both halves, kept in a register
    asm volatile("" : "+v"(magic));

    Words bw[kNB];
    f16x8 a[2][U];
    auto load_b = [&](int slot, int64_t st) { bw[slot] = *reinterpret_cast<const Words *>(brow + 2 * U * (st < nsteps ? st : nsteps - 1)); };
    auto load_a = [&](int slot, int64_t st) {
        const int64_t sc = st < nsteps ? st : nsteps - 1;
#pragma unroll
        for (int u = 0; u < U; ++u) a[slot][u] = *reinterpret_cast<const f16x8 *>(arow + KS * sc + 8 * u);
    };
    auto body_sz = [&](int64_t b) {  // scale (0 past the end) and zero of body b
        const int64_t bc = b < nbody ? b : nbody - 1;
        float2 v = szs[((kb + bc * BL) / g - g0) * kTileN + fl];
        if (b >= nbody) v.x = 0.0f;
        return v;
    };
#pragma unroll
    for (int p = 0; p < kNB - 1; ++p) load_b(p, p);
    load_a(0, 0);

    for (int64_t base = 0; base < nsteps; base += kNB) {
#pragma unroll
        for (int st = 0; st < kNB; st += 2) {  // one body: steps base + st, base + st + 1
            const float2 sz = body_sz((base + st) / 2);
            const Bias bias = bias_of(sz.y);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int s = st + h;
                load_b((s + kNB - 1) % kNB, base + s + kNB - 1);
                load_a((s + 1) & 1, base + s + 1);
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const f16x8 b = dequant8(word_at(bw[s], u), bias, magic);
                    accg = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s & 1][u], b, accg, 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc[r] = fmaf(sz.x, accg[r], acc[r]);
                accg[r] = 0.0f;
            }
        }
    }
    if (o >= d_out) return;
    float *dst = out + (int64_t)blockIdx.z * split_stride + o;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = mfma32_row(r, lane);
        if (m < M) dst[m * ldo] = acc[r];
    }
}

// Few tokens with groups of a multiple of 128: the weight stream in 64-byte
// pieces.  K advances in chunks of 256 columns (32 packed words of a row).
// Lane half h loads words 16 h .. 16 h + 15 of the chunk (64 contiguous bytes;
// rows read this way stream near full bandwidth, where 16-byte pieces of many
// rows do not), i.e. half 0 holds the chunk's first group-aligned 128 columns
// (A) and half 1 its second (B).  v_permlane32_swap then trades the upper
// halves of A for the lower halves of B between the two lane halves, so that
// each half holds 8 words of A and 8 of B: half h takes words 8 h .. 8 h + 7
// of each, and MFMA i of a 128-column body uses word 8 h + i (columns
// 64 h + 8 i .. + 7), both halves in one group.  The next chunk's words and its
// two bodies' scales and zeros are read while the current chunk is used; the
// activation operand comes from LDS, staged once (IL: straight from X, put in
// the operand order on the way).  Bodies past the end fold with scale 0.
// GB: columns per group fold, 128 for groups of a multiple of 128; 64 or 32
// for smaller groups.  Then MFMA step i of a body takes columns 16 i + 8 h ..
// + 7 in lane half h (word 2 i + h), so a step lies inside one group: four more
// swaps per body (word pairs (j, j + 1), j even) put the even words in half 0
// and the odd words in half 1, and the body's sum is folded at every group end.
template <bool IL, int GB>
__global__ __launch_bounds__(kThreads, 2) void w4a16_chunk_kernel(const _Float16 *__restrict__ X, int64_t ldx, int64_t M,
                                                               int64_t d_in, const uint32_t *__restrict__ packed,
                                                               int64_t ldp, const float *__restrict__ scales,
                                                               const float *__restrict__ zeros, int64_t g, int64_t ng,
                                                               int64_t d_out, int64_t kspan, float *__restrict__ out,
                                                               int64_t ldo, int64_t split_stride) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int64_t o = (int64_t)blockIdx.x * kTileN + wave * 32 + (lane & 31);
    const int64_t oc = o < d_out ? o : d_out - 1;
    const int64_t kb = (int64_t)blockIdx.z * kspan;
    const int64_t ke = std::min<int64_t>(d_in, kb + kspan);
    if (kb >= ke) return;  // uniform over the workgroup
    const int64_t nbody = (ke - kb) / 128, nchunks = (nbody + 1) / 2;

    // this lane's 64 bytes of chunk c: words 32 c + 16 h .. + 15 past kb, clamped into [kb, ke)
    const uint32_t *brow = packed + oc * ldp + kb / 8;
    const int64_t wlast = (ke - kb) / 8 - 16;  // last 16-word piece that stays inside the range
    const float *srow = scales + oc * ng, *zrow = zeros + oc * ng;
    constexpr int NG = 128 / GB;  // groups per body
    uint4 q[2][4];
    float2 sz[2][2][NG];  // [slot][body of the chunk][group of the body]: scale (0 past the end), zero
    auto load = [&](int slot, int64_t c) {
        const int64_t cc = c < nchunks ? c : nchunks - 1;
        const int64_t w = std::min<int64_t>(32 * cc + 16 * half, wlast);
        const uint4 *p = reinterpret_cast<const uint4 *>(brow + w);
#pragma unroll
        for (int j = 0; j < 4; ++j) q[slot][j] = p[j];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t b = 2 * c + h, bc = b < nbody ? b : nbody - 1;
#pragma unroll
            for (int k = 0; k < NG; ++k) {
                const int64_t gi = (kb + 128 * bc + GB * k) / g;
                sz[slot][h][k] = make_float2(srow[gi], zrow[gi]);
            }
        }
    };
    load(0, 0);  // the first chunk is in flight during the staging

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int64_t ldxs = kspan + 8;  // halves; the pad staggers the banks
    _Float16 *xs = reinterpret_cast<_Float16 *>(smem);
    {  // rows of X over [kb, ke) into LDS, every load issued before the first store
        const int64_t chunks = (ke - kb) / 8;  // 16-byte pieces per row
        const int64_t n = M * chunks;
        for (int64_t i0 = 0; i0 < n; i0 += 8 * kThreads) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t i = i0 + u * kThreads + threadIdx.x;
                const int64_t ic = i < n ? i : n - 1;
                v[u] = *reinterpret_cast<const uint4 *>(X + (ic / chunks) * ldx + kb + 8 * (ic % chunks));
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t i = i0 + u * kThreads + threadIdx.x;
                uint4 w = v[u];
                if constexpr (IL) {  // halves 0..7 -> 0, 4, 1, 5, 2, 6, 3, 7
                    w = make_uint4(__builtin_amdgcn_perm(v[u].z, v[u].x, 0x05040100u), __builtin_amdgcn_perm(v[u].z, v[u].x, 0x07060302u),
                                   __builtin_amdgcn_perm(v[u].w, v[u].y, 0x05040100u), __builtin_amdgcn_perm(v[u].w, v[u].y, 0x07060302u));
                }
                if (i < n) *reinterpret_cast<uint4 *>(xs + (i / chunks) * ldxs + 8 * (i % chunks)) = w;
            }
        }
    }
    __syncthreads();

    const int64_t mc = (lane & 31) < M ? (lane & 31) : M - 1;
    // + 128 body + 8 i (GB = 128: columns 64 h + 8 i), else + 128 body + 16 i (columns 16 i + 8 h)
    const _Float16 *arow = xs + mc * ldxs + (GB == 128 ? 64 : 8) * half;
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const floatx16 zero16 = {};
    uint32_t magic = 0x64006400u;  // fp16 exponent of 1024 in both halves, kept in a register
    asm volatile("" : "+v"(magic));

    auto swap = [&](uint4 &x, uint4 &y) {  // x's upper lane half <-> y's lower lane half
        uint32_t xv[4] = {x.x, x.y, x.z, x.w}, yv[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const auto r = __builtin_amdgcn_permlane32_swap(xv[j], yv[j], false, false);
            xv[j] = r[0];
            yv[j] = r[1];
        }
        x = make_uint4(xv[0], xv[1], xv[2], xv[3]);
        y = make_uint4(yv[0], yv[1], yv[2], yv[3]);
    };
    // The chunk's two bodies, their MFMAs interleaved: two independent sums, so
    // each MFMA issues without waiting for the previous one's result.  Each
    // body's sum and the folds keep their order (body b, then b + 1).
    auto bodies = [&](const uint4 (&w)[4], int64_t b, const float2 (&v)[2][NG]) {
        constexpr int kSteps = 8 / NG;  // MFMA steps per group
        const _Float16 *ap[2];
        bool live[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            live[h] = b + h < nbody;
            ap[h] = arow + 128 * (live[h] ? b + h : nbody - 1);
        }
        floatx16 g[2];
#pragma unroll
        for (int k = 0; k < NG; ++k) {
            Bias bias[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) bias[h] = bias_of(v[h][k].y);
#pragma unroll
            for (int i = k * kSteps; i < (k + 1) * kSteps; ++i)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f16x8 a = *reinterpret_cast<const f16x8 *>(ap[h] + (GB == 128 ? 8 : 16) * i);
                    // GB = 128: word 8 h + i; else word 2 i + h, in register (i < 4 ? 2 i : 2 (i - 4) + 1)
                    const int rj = GB == 128 ? i : (i < 4 ? 2 * i : 2 * (i - 4) + 1);
                    const uint4 &wv = w[2 * h + (rj < 4 ? 0 : 1)];
                    const f16x8 bq = dequant8(word_at(wv, rj & 3), bias[h], magic);
                    g[h] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bq, i == k * kSteps ? zero16 : g[h], 0, 0, 0);
                }
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // group k of both bodies ends: fold with its scale
                const float sc = live[h] ? v[h][k].x : 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = fmaf(sc, g[h][r], acc[r]);
            }
        }
    };
    for (int64_t c = 0; c < nchunks; c += 2) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            load(sl ^ 1, c + sl + 1);
            uint4(&w)[4] = q[sl];
            swap(w[0], w[2]);
            swap(w[1], w[3]);
            if constexpr (GB < 128) {  // word pairs (j, j + 1), j even: even words to half 0, odd to half 1
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    uint4 &x = w[t];
                    const auto r01 = __builtin_amdgcn_permlane32_swap(x.x, x.y, false, false);
                    const auto r23 = __builtin_amdgcn_permlane32_swap(x.z, x.w, false, false);
                    x = make_uint4(r01[0], r01[1], r23[0], r23[1]);
                }
            }
            bodies(w, 2 * (c + sl), sz[sl]);
        }
    }
    if (o >= d_out) return;
    float *dst = out + (int64_t)blockIdx.z * split_stride + o;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = mfma32_row(r, lane);
        if (m < M) dst[m * ldo] = acc[r];
    }
}

// More tokens (M > 32), groups of a multiple of 64: a tiled product.  A
// workgroup computes 128 tokens x 128 features; wave (wm, wn) owns tokens
// 64 wm .. + 63 and features 64 wn .. + 63 (two 32-row by two 32-column
// blocks).  K advances in chunks of 64 columns: the activation tile
// (128 x 64 fp16, rows padded by 16 bytes) is double-buffered in LDS, staged
// through registers one chunk ahead; each lane reads its two features' packed
// words of the chunk (16 bytes each: half h takes words 4 h .. 4 h + 3, and
// MFMA step u uses word 4 h + u, columns 32 h + 8 u .. + 7, the activation
// operand read to match) one chunk ahead.  A body (two chunks for groups of a
// multiple of 128, one for a multiple of 64) lies inside one group: its sums
// start from zero and are folded into the running ones with its scale.
constexpr int kWM = 128, kWN = 128, kWK = 64;  // tile tokens, features, K per chunk
constexpr int kWP = kWK + 8;                   // LDS row pitch in halves (144 bytes)
// CPB: chunks per body (the columns one scale covers), 2 for groups of a
// multiple of 128 columns, 1 for a multiple of 64, 0 for 32-column bodies (two
// per chunk).  With CPB = 0 the MFMA steps change: step s takes columns
// 16 s + 8 h .. + 7 in lane half h, so its 16 K values lie in one 32-column
// group; two v_permlane32_swap per 16-byte load move the words there (half 0
// loaded words 0..3, half 1 words 4..7; step s needs word 2 s + h).
template <bool IL, int CPB>  // IL: X in its own column order, put in the operand order on the way into LDS
__global__ __launch_bounds__(kThreads, 2) void w4a16_wide_kernel(const _Float16 *__restrict__ X, int64_t ldx, int64_t M,
                                                              int64_t d_in, const uint32_t *__restrict__ packed,
                                                              int64_t ldp, const float *__restrict__ scales,
                                                              const float *__restrict__ zeros, int64_t g, int64_t ng,
                                                              int64_t d_out, int64_t kspan, float *__restrict__ out,
                                                              int64_t ldo, int64_t split_stride) {
    __shared__ __attribute__((aligned(16))) _Float16 xs[2][kWM][kWP];
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
    const int half = lane >> 5, l32 = lane & 31;
    const int wm = wave & 1, wn = wave >> 1;
    // token tiles first: the workgroups that share a weight tile run together
    const int64_t m0 = (int64_t)blockIdx.x * kWM, n0 = (int64_t)blockIdx.y * kWN;
    const int64_t kb = (int64_t)blockIdx.z * kspan;
    const int64_t ke = std::min<int64_t>(d_in, kb + kspan);
    if (kb >= ke) return;  // uniform over the workgroup
    const int64_t nchunk = (ke - kb) / kWK;  // the range holds whole bodies (an even count when CPB = 2)

    // the lane's two features and their packed rows (+ word of the chunk)
    const uint32_t *brow[2];
    const float *srow[2], *zrow[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t o = n0 + 64 * wn + 32 * nb + l32;
        const int64_t oc = o < d_out ? o : d_out - 1;
        brow[nb] = packed + oc * ldp + kb / 8 + 4 * half;
        srow[nb] = scales + oc * ng;
        zrow[nb] = zeros + oc * ng;
    }
    // staging of the activation tile: thread t moves 16-byte pieces (row t / 8, piece t % 8) of 4 row groups
    const int sr = tid / 8, sp = tid % 8;
    // (four named registers rather than an array, which the compiler would keep on the stack)
    uint4 sv0, sv1, sv2, sv3;
    auto stage_piece = [&](int i, int64_t k) {
        const int64_t m = m0 + sr + 32 * i;
        return *reinterpret_cast<const uint4 *>(X + (m < M ? m : M - 1) * ldx + k + 8 * sp);
    };
    auto stage_load = [&](int64_t c) {
        const int64_t k = kb + kWK * (c < nchunk ? c : nchunk - 1);
        sv0 = stage_piece(0, k);
        sv1 = stage_piece(1, k);
        sv2 = stage_piece(2, k);
        sv3 = stage_piece(3, k);
    };
    auto order = [](uint4 v) {  // halves 0..7 -> 0, 4, 1, 5, 2, 6, 3, 7 (or as they are)
        if constexpr (!IL) return v;
        return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                          __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
    };
    auto stage_store = [&](int buf) {
        *reinterpret_cast<uint4 *>(&xs[buf][sr][8 * sp]) = order(sv0);
        *reinterpret_cast<uint4 *>(&xs[buf][sr + 32][8 * sp]) = order(sv1);
        *reinterpret_cast<uint4 *>(&xs[buf][sr + 64][8 * sp]) = order(sv2);
        *reinterpret_cast<uint4 *>(&xs[buf][sr + 96][8 * sp]) = order(sv3);
    };
    uint4 bw[2][2];
    auto load_b = [&](int slot, int64_t c) {
        const int64_t cc = c < nchunk ? c : nchunk - 1;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bw[slot][nb] = *reinterpret_cast<const uint4 *>(brow[nb] + 8 * cc);
    };
    float2 sz[2], szn[2];  // scale, zero per feature block: this body's, the next body's
    float2 szh[2][2], szhn[2][2];  // CPB = 0: [body of the chunk][feature block], this chunk's and the next
    constexpr int kBody = CPB == 0 ? kWK / 2 : kWK * CPB;  // columns per body
    const uint32_t body0 = (uint32_t)(kb / kBody), bodies_per_group = (uint32_t)(g / kBody);
    auto group_of = [&](int64_t c, int j) {  // group of body j of chunk c (j = 0 unless CPB = 0)
        const int64_t cc = c < nchunk ? c : nchunk - 1;
        const uint32_t b = CPB == 0 ? (uint32_t)(2 * cc + j) : (uint32_t)(cc / (CPB == 0 ? 1 : CPB));
        return (body0 + b) / bodies_per_group;  // 32-bit: a scalar division
    };
    auto load_sz = [&](float2(&dst)[2], int64_t c) {
        const uint32_t gi = group_of(c, 0);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) dst[nb] = make_float2(srow[nb][gi], zrow[nb][gi]);
    };
    auto load_szh = [&](float2(&dst)[2][2], int64_t c) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t gi = group_of(c, j);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) dst[j][nb] = make_float2(srow[nb][gi], zrow[nb][gi]);
        }
    };

    floatx16 acc[2][2], accg[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    const floatx16 zero16 = {};
    uint32_t magic = 0x64006400u;  // fp16 exponent of 1024 in both halves, kept in a register
    asm volatile("" : "+v"(magic));

    stage_load(0);
    load_b(0, 0);
    if constexpr (CPB == 0)
        load_szh(szh, 0);
    else
        load_sz(sz, 0);
    stage_store(0);
    __syncthreads();
    for (int64_t c0 = 0; c0 < nchunk; c0 += 2) {
#pragma unroll
      for (int buf = 0; buf < 2; ++buf) {  // unrolled: the register slot index is a constant
        const int64_t c = c0 + buf;
        if constexpr (CPB <= 1)
            if (buf == 1 && c >= nchunk) break;  // an odd chunk count; uniform
        // next chunk: activations into registers, weights into the other slot
        stage_load(c + 1);
        load_b(buf ^ 1, c + 1);
        if constexpr (CPB == 0) {
            load_szh(szhn, c + 1);  // the next chunk's two bodies
            Bias bias[2][2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) bias[j][nb] = bias_of(szh[j][nb].y);
            uint4 wq[2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {  // lane half h: words h, 2 + h, 4 + h, 6 + h for steps 0, 1, 2, 3
                wq[nb] = bw[buf][nb];
                const auto r01 = __builtin_amdgcn_permlane32_swap(wq[nb].x, wq[nb].y, false, false);
                const auto r23 = __builtin_amdgcn_permlane32_swap(wq[nb].z, wq[nb].w, false, false);
                wq[nb] = make_uint4(r01[0], r23[0], r01[1], r23[1]);
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const int j = st >> 1;  // the body (32-column group) of this step
                f16x8 a[2];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    a[mb] = *reinterpret_cast<const f16x8 *>(&xs[buf][64 * wm + 32 * mb + l32][16 * st + 8 * half]);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const f16x8 bq = dequant8(word_at(wq[nb], st), bias[j][nb], magic);
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)  // a body's first product starts its sums from zero
                        accg[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            a[mb], bq, (st % 2 == 0) ? zero16 : accg[mb][nb], 0, 0, 0);
                }
                if (st % 2 == 1) {  // body j ends: fold it in with its scales
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                acc[mb][nb][r] = fmaf(szh[j][nb].x, accg[mb][nb][r], acc[mb][nb][r]);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) szh[j][nb] = szhn[j][nb];
            stage_store(buf ^ 1);  // the other buffer was last read before the previous barrier
            __syncthreads();
            continue;
        }
        constexpr int kCpb = CPB == 0 ? 1 : CPB;
        const bool body_start = buf % kCpb == 0, body_end = buf % kCpb == kCpb - 1;
        if (body_start) load_sz(szn, c + kCpb);  // the next body's scales, a body ahead
        Bias bias[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) bias[nb] = bias_of(sz[nb].y);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f16x8 a[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                a[mb] = *reinterpret_cast<const f16x8 *>(&xs[buf][64 * wm + 32 * mb + l32][32 * half + 8 * u]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const f16x8 bq = dequant8(word_at(bw[buf][nb], u), bias[nb], magic);
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)  // a body's first product starts its sums from zero
                    accg[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        a[mb], bq, (body_start && u == 0) ? zero16 : accg[mb][nb], 0, 0, 0);
            }
        }
        if (body_end) {  // a body ends: fold in its scales, then the next body's
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[mb][nb][r] = fmaf(sz[nb].x, accg[mb][nb][r], acc[mb][nb][r]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) sz[nb] = szn[nb];
        }
        stage_store(buf ^ 1);  // the other buffer was last read before the previous barrier
        __syncthreads();
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t o = n0 + 64 * wn + 32 * nb + l32;
        if (o >= d_out) continue;
        float *dst = out + (int64_t)blockIdx.z * split_stride + o;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + 64 * wm + 32 * mb + mfma32_row(r, lane);
                if (m < M) dst[m * ldo] = acc[mb][nb][r];
            }
    }
}

// Y[m][o] = sum over splits of P[split][m][o], splits in order.
__global__ __launch_bounds__(kThreads) void split_sum_kernel(const float *__restrict__ P, int splits, int64_t M,
                                                             int64_t d_out, float *__restrict__ Y, int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= M * d_out) return;
    const int64_t m = i / d_out, o = i % d_out;
    float v = 0.0f;
    for (int sp = 0; sp < splits; ++sp) v += P[(int64_t)sp * M * d_out + i];
    Y[m * ldy + o] = v;
}

int64_t xp_ld(int64_t d_in) { return (d_in + 7) / 8 * 8; }

constexpr size_t kXlBytes = 32768;  // LDS budget for the activations of one workgroup

struct GemmPlan {
    int tm, u;
    bool xl;           // few tokens (M <= 32): activations through LDS
    bool chunk;        // few tokens, groups of a multiple of 128: w4a16_chunk_kernel
    bool wide;         // more tokens, groups of a multiple of 128: w4a16_wide_kernel
    size_t lds_bytes;  // dynamic LDS per workgroup (few-token kernels)
    int64_t n_tiles, m_tiles, splits, kspan;
    size_t xp_bytes, part_bytes;
};

GemmPlan plan_gemm(int64_t M, int64_t d_in, int64_t d_out, int64_t g) {
    GemmPlan p;
    p.tm = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
    p.u = g % 128 == 0 ? 4 : (g % 64 == 0 ? 2 : 1);  // a body (32 U columns) stays inside one group
    p.n_tiles = ceil_div(d_out, kTileN);
    p.m_tiles = ceil_div(M, 32 * p.tm);
    // about four workgroups per CU; a split keeps at least 256 K values
    const int64_t tiles = p.n_tiles * p.m_tiles;
    int64_t sp = tiles >= 1024 ? 1 : ceil_div(1024, tiles);
    sp = std::min<int64_t>(sp, std::max<int64_t>(1, d_in / 256));
    p.xl = M <= 32;
    // whole 128-column bodies (folded per group inside them); with groups under 128
    // columns only up to 4 tokens, where the streamed words win over scales in LDS
    p.chunk = p.xl && d_in % 128 == 0 && (p.u == 4 || M <= 4);
    // weight tiles along grid y; whole 64-column chunks
    p.wide = !p.xl && d_in % kWK == 0 && ceil_div(d_out, kWN) <= 65535;
    if (p.wide) {  // 128 x 128 tiles; split K (whole bodies and chunks) while there are few tiles
        p.n_tiles = ceil_div(d_out, kWN);
        p.m_tiles = ceil_div(M, kWM);
        const int64_t t = p.n_tiles * p.m_tiles;
        sp = t >= 512 ? 1 : std::min<int64_t>(ceil_div(512, t), std::max<int64_t>(1, d_in / 512));
    }
    if (p.chunk) {  // the activations of a whole split in 32 KB of LDS; no more splits than that needs
        const int64_t kmax = std::max<int64_t>(128, (int64_t)(kXlBytes / (2 * M)) - 8);
        sp = ceil_div(d_in, kmax);
    } else if (p.xl) {  // at most 32 KB of activations and 32 groups of scales per workgroup: more splits if needed
        const int64_t kmax = std::max<int64_t>(32 * p.u, std::min<int64_t>((int64_t)(kXlBytes / (2 * M)) - 8, 30 * g));
        sp = std::max<int64_t>(sp, ceil_div(d_in, kmax));
    }
    const int64_t unit = p.wide ? std::max<int64_t>(32 * p.u, kWK) : p.chunk ? 128 : 32 * p.u;  // whole bodies (and chunks)
    p.kspan = ceil_div(ceil_div(d_in, sp), unit) * unit;
    if (p.chunk)
        while ((size_t)M * (size_t)(p.kspan + 8) * 2 > kXlBytes && p.kspan > 128) p.kspan -= 128;
    else if (p.xl)
        while (((size_t)M * (size_t)(p.kspan + 8) * 2 > kXlBytes || p.kspan > 30 * g) && p.kspan > 32 * p.u)
            p.kspan -= 32 * p.u;
    p.splits = ceil_div(d_in, p.kspan);
    // activations, then float2 (scale, zero) for 128 features x the groups a range touches
    // (a range touches at most kspan / g + 2 <= kMaxGroups groups)
    p.lds_bytes = p.chunk ? (size_t)M * (size_t)(p.kspan + 8) * 2
                : p.xl  ? align_up((size_t)M * (size_t)(p.kspan + 8) * 2, 16) + (size_t)(p.kspan / g + 2) * kTileN * 8
                        : 0;
    p.xp_bytes = align_up((size_t)M * (size_t)xp_ld(d_in) * 2, 256);
    p.part_bytes = p.splits > 1 ? align_up((size_t)p.splits * (size_t)M * (size_t)d_out * 4, 256) : 0;
    return p;
}

}  // namespace

hipError_t run_pack(const uint8_t *codes, int64_t d_out, int64_t d_in, int bits, const int32_t *perm,
                    uint32_t *packed, hipStream_t s) {
    const int64_t ldp = ceil_div(d_in * bits, 32);
    const dim3 grid((unsigned)ceil_div(ldp, kThreads), (unsigned)std::min<int64_t>(d_out, 65535));
    hipLaunchKernelGGL(pack_codes_kernel, grid, dim3(kThreads), 0, s, codes, d_out, d_in, bits, perm, packed, ldp);
    return hipGetLastError();
}

size_t w4a16_ws_bytes(int64_t M, int64_t d_in, int64_t d_out, int64_t g) {
    const GemmPlan p = plan_gemm(M, d_in, d_out, g);
    return p.xp_bytes + p.part_bytes;
}

hipError_t run_w4a16(const void *X, int64_t M, int64_t d_in, int64_t ldx, const int32_t *kperm,
                     const uint32_t *packed, const float *scales, const float *zeros, int64_t g, int64_t d_out,
                     float *Y, int64_t ldy, void *ws, hipStream_t s) {
    const GemmPlan p = plan_gemm(M, d_in, d_out, g);
    char *wsb = static_cast<char *>(ws);
    const _Float16 *Xk = static_cast<const _Float16 *>(X);
    int64_t ldk = ldx;
    hipError_t e;
    if (kperm || !(p.chunk || p.wide)) {  // columns of X into the operand order (and the packed order), once
        uint16_t *Xp = reinterpret_cast<uint16_t *>(wsb);
        const dim3 grid((unsigned)ceil_div(d_in, kThreads), (unsigned)std::min<int64_t>(M, 65535));
        hipLaunchKernelGGL(gather_cols_kernel, grid, dim3(kThreads), 0, s, static_cast<const uint16_t *>(X), ldx, M, d_in,
                           kperm, Xp, xp_ld(d_in));
        if ((e = hipGetLastError()) != hipSuccess) return e;
        Xk = reinterpret_cast<const _Float16 *>(Xp);
        ldk = xp_ld(d_in);
    }
    const int64_t ng = d_in / g;
    const int64_t ldp = d_in / 8;
    float *out = p.splits > 1 ? reinterpret_cast<float *>(wsb + p.xp_bytes) : Y;
    const int64_t ldo = p.splits > 1 ? d_out : ldy;
    const int64_t stride = p.splits > 1 ? M * d_out : 0;
    const dim3 grid((unsigned)p.n_tiles, (unsigned)p.m_tiles, (unsigned)p.splits);
#define W4A16_LAUNCH(TM, U)                                                                                     \
    hipLaunchKernelGGL((w4a16_kernel<TM, U>), grid, dim3(kThreads), 0, s, Xk, ldk, M, d_in, packed, ldp, scales, \
                       zeros, g, ng, d_out, p.kspan, out, ldo, stride)
#define W4A16_TM(U)                                                                                              \
    if (p.wide && !kperm)                                                                                        \
        hipLaunchKernelGGL((w4a16_wide_kernel<true, ((U) >= 4 ? 2 : (U) == 2 ? 1 : 0)>), dim3(grid.y, grid.x, grid.z), dim3(kThreads), 0, s, Xk, ldk, M,\
                           d_in, packed, ldp, scales, zeros, g, ng, d_out, p.kspan, out, ldo, stride);           \
    else if (p.wide)                                                                                             \
        hipLaunchKernelGGL((w4a16_wide_kernel<false, ((U) >= 4 ? 2 : (U) == 2 ? 1 : 0)>), dim3(grid.y, grid.x, grid.z), dim3(kThreads), 0, s, Xk, ldk, M,\
                           d_in, packed, ldp, scales, zeros, g, ng, d_out, p.kspan, out, ldo, stride);           \
    else if (p.chunk && !kperm)                                                                                       \
        hipLaunchKernelGGL((w4a16_chunk_kernel<true, ((U) >= 4 ? 128 : (U) == 2 ? 64 : 32)>), grid, dim3(kThreads), p.lds_bytes, s, Xk, ldk, M, d_in, packed, \
                           ldp, scales, zeros, g, ng, d_out, p.kspan, out, ldo, stride);                       \
    else if (p.chunk)                                                                                            \
        hipLaunchKernelGGL((w4a16_chunk_kernel<false, ((U) >= 4 ? 128 : (U) == 2 ? 64 : 32)>), grid, dim3(kThreads), p.lds_bytes, s, Xk, ldk, M, d_in, packed, \
                           ldp, scales, zeros, g, ng, d_out, p.kspan, out, ldo, stride);                       \
    else if (p.xl)                                                                                               \
        hipLaunchKernelGGL((w4a16_few_kernel<U>), grid, dim3(kThreads), p.lds_bytes, s, Xk, ldk, M, d_in, packed, ldp, \
                           scales, zeros, g, ng, d_out, p.kspan, out, ldo, stride);                            \
    else if (p.tm == 2)                                                                                          \
        W4A16_LAUNCH(2, U);                                                                                      \
    else                                                                                                         \
        W4A16_LAUNCH(4, U);
    if (p.u == 4) {
        W4A16_TM(4)
    } else if (p.u == 2) {
        W4A16_TM(2)
    } else {
        W4A16_TM(1)
    }
#undef W4A16_TM
#undef W4A16_LAUNCH
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (p.splits > 1) {
        hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)ceil_div(M * d_out, kThreads)), dim3(kThreads), 0, s, out,
                           (int)p.splits, M, d_out, Y, ldy);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gptq
