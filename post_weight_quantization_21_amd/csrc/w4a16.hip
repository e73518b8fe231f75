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

// Xp[m][k] = X[m][kperm[k]] (fp16), rows of ldxp elements.
__global__ __launch_bounds__(kThreads) void gather_cols_kernel(const uint16_t *__restrict__ X, int64_t ldx, int64_t M,
                                                               int64_t d_in, const int32_t *__restrict__ kperm,
                                                               uint16_t *__restrict__ Xp, int64_t ldxp) {
    const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (k >= d_in) return;
    int64_t c = kperm[k];
    c = c < 0 ? 0 : (c >= d_in ? d_in - 1 : c);
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) Xp[m * ldxp + k] = X[m * ldx + c];
}

// Eight 4-bit codes (code i at bits 4i) as fp16 (code - z).  bias = 1024 + z in both halves.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 bias) {
    const uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6 in bytes 0..3
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // bytes: lo.byte i, 0, hi.byte i, 0 (selector 12 gives a zero byte)
        const uint32_t sel = 0x0C000C00u | ((uint32_t)(4 + i) << 16) | (uint32_t)i;
        const uint32_t d = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
        const f16x2 h = __builtin_bit_cast(f16x2, d) - bias;
        r[2 * i] = h[0];
        r[2 * i + 1] = h[1];
    }
    return r;
}

// One workgroup: 128 output features x 32 TM tokens over K range
// [kb, kb + kspan).  Wave w owns features 32 w .. 32 w + 31; lane l supplies
// feature l % 32 of the weight operand and token l % 32 of each activation
// block.  K advances in macro steps of 16 U columns (U MFMAs): lane half h
// takes packed words U h .. U h + U - 1 of the step (one 4U-byte load) and the
// matching 8 U activations (one contiguous 16U-byte load), and MFMA u uses
// word U h + u -- A and B agree on every K index, which is all the product
// needs.  Operands are read PD macro steps ahead into a ring of PD + 1 slots.
template <int U>
struct WordsT;
template <>
struct WordsT<2> {
    typedef uint2 T;
};
template <>
struct WordsT<4> {
    typedef uint4 T;
};
__device__ __forceinline__ uint32_t word_at(const uint2 &w, int u) { return u == 0 ? w.x : w.y; }
__device__ __forceinline__ uint32_t word_at(const uint4 &w, int u) { return u == 0 ? w.x : (u == 1 ? w.y : (u == 2 ? w.z : w.w)); }

template <int TM, int U, int PD>
__global__ __launch_bounds__(kThreads) void w4a16_kernel(const _Float16 *__restrict__ X, int64_t ldx, int64_t M,
                                                         int64_t d_in, const uint32_t *__restrict__ packed, int64_t ldp,
                                                         const float *__restrict__ scales,
                                                         const float *__restrict__ zeros, int64_t g, int64_t ng,
                                                         int64_t d_out, int64_t kspan, float *__restrict__ out,
                                                         int64_t ldo, int64_t split_stride) {
    constexpr int KS = 16 * U;  // K columns per macro step
    constexpr int NS = PD + 1;  // ring slots
    typedef typename WordsT<U>::T Words;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int half = lane >> 5;
    const int64_t o = (int64_t)blockIdx.x * kTileN + wave * 32 + (lane & 31);
    const int64_t oc = o < d_out ? o : d_out - 1;
    const int64_t m0 = (int64_t)blockIdx.y * 32 * TM;
    const int64_t kb = (int64_t)blockIdx.z * kspan;
    const int64_t ke = std::min<int64_t>(d_in, kb + kspan);
    if (kb >= ke) return;  // uniform over the workgroup
    const uint32_t *brow = packed + oc * ldp + U * half;  // + k / 8
    const _Float16 *arow[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int64_t m = m0 + 32 * t + (lane & 31);
        arow[t] = X + (m < M ? m : M - 1) * ldx + 8 * U * half;  // + k
    }
    floatx16 acc[TM], accg[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = accg[t][r] = 0.0f;

    int64_t grp = kb / g;
    int64_t gend = std::min<int64_t>((grp + 1) * g, ke);
    const float *srow = scales + oc * ng, *zrow = zeros + oc * ng;
    float s = srow[grp];
    f16x2 bias;
    bias[0] = bias[1] = (_Float16)(1024.0f + zrow[grp]);
    // the next group's scale and zero are read a group ahead
    const int64_t gn0 = grp + 1 < ng ? grp + 1 : grp;
    float s_n = srow[gn0], z_n = zrow[gn0];

    Words bw[NS];
    f16x8 a[NS][TM][U];
    auto load = [&](int slot, int64_t k) {  // k < ke
        bw[slot] = *reinterpret_cast<const Words *>(brow + k / 8);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < U; ++u) a[slot][t][u] = *reinterpret_cast<const f16x8 *>(arow[t] + k + 8 * u);
    };
#pragma unroll
    for (int p = 0; p < PD; ++p) load(p, std::min<int64_t>(kb + p * KS, ke - KS));

    for (int64_t k0 = kb; k0 < ke; k0 += NS * KS) {
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            const int64_t k = k0 + st * KS;
            if (k < ke) {  // uniform
                // read PD steps ahead (the last steps re-read the final step: always in bounds)
                load((st + PD) % NS, std::min<int64_t>(k + PD * KS, ke - KS));
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const f16x8 b = dequant8(word_at(bw[st], u), bias);
#pragma unroll
                    for (int t = 0; t < TM; ++t)
                        accg[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[st][t][u], b, accg[t], 0, 0, 0);
                }
                if (k + KS >= gend) {  // the group (or this split's part of it) ends: fold in its scale
#pragma unroll
                    for (int t = 0; t < TM; ++t)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            acc[t][r] = fmaf(s, accg[t][r], acc[t][r]);
                            accg[t][r] = 0.0f;
                        }
                    ++grp;
                    gend = std::min<int64_t>(gend + g, ke);
                    s = s_n;
                    bias[0] = bias[1] = (_Float16)(1024.0f + z_n);
                    const int64_t gn = grp + 1 < ng ? grp + 1 : ng - 1;
                    s_n = srow[gn];
                    z_n = zrow[gn];
                }
            }
        }
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

struct GemmPlan {
    int tm, u;
    int64_t n_tiles, m_tiles, splits, kspan;
    size_t xp_bytes, part_bytes;
};

GemmPlan plan_gemm(int64_t M, int64_t d_in, int64_t d_out, int64_t g) {
    GemmPlan p;
    p.tm = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
    p.u = g % 64 == 0 ? 4 : 2;  // a macro step stays inside one group
    p.n_tiles = ceil_div(d_out, kTileN);
    p.m_tiles = ceil_div(M, 32 * p.tm);
    // about four workgroups per CU; a split keeps at least 256 K values
    const int64_t tiles = p.n_tiles * p.m_tiles;
    int64_t sp = tiles >= 1024 ? 1 : ceil_div(1024, tiles);
    sp = std::min<int64_t>(sp, std::max<int64_t>(1, d_in / 256));
    p.kspan = ceil_div(ceil_div(d_in, sp), 16 * p.u) * 16 * p.u;
    p.splits = ceil_div(d_in, p.kspan);
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
    if (kperm) {  // columns of X into the packed order, once
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
#define W4A16_LAUNCH(TM, U, PD)                                                                                 \
    hipLaunchKernelGGL((w4a16_kernel<TM, U, PD>), grid, dim3(kThreads), 0, s, Xk, ldk, M, d_in, packed, ldp, scales, \
                       zeros, g, ng, d_out, p.kspan, out, ldo, stride)
    if (p.u == 4) {
        if (p.tm == 1)
            W4A16_LAUNCH(1, 4, 2);
        else if (p.tm == 2)
            W4A16_LAUNCH(2, 4, 1);
        else
            W4A16_LAUNCH(4, 4, 1);
    } else {
        if (p.tm == 1)
            W4A16_LAUNCH(1, 2, 2);
        else if (p.tm == 2)
            W4A16_LAUNCH(2, 2, 1);
        else
            W4A16_LAUNCH(4, 2, 1);
    }
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
