// Integer grids of GPTQ's quantizer, device side.
//
// Symmetric and asymmetric uniform grids as defined on page "LLM 量化方法原理
// 与实现详解", §2.2 (scale from max|x| or from the range, zero point, rounding
// of x/scale (+ zero) and clamping), applied per group of consecutive input
// columns (§2.3).  All decisions are binary32 with round-half-to-even
// (v_rndne_f32), the rounding of the pages' torch.round.  Readings of points
// the pages leave open: the asymmetric range always contains 0
// (lo = min(min x, 0), hi = max(max x, 0)); a zero-width group gets scale 1.
//
// Both grids are evaluated by one branch-free formula,
//     code = clamp(rint(x / s + zoff), qlo, qhi) + zadd,
// symmetric: zoff = 0, [qlo, qhi] = [-qmax, qmax], zadd = 2^(b-1);
// asymmetric: zoff = zero, [qlo, qhi] = [0, 2^b - 1], zadd = 0.
// (x/s + 0 equals x/s, and a -0 that would become +0 is clamped and shifted to
// the same code, so the symmetric case is exactly the printed rint(x/s).)
//
// x / s is the correctly rounded binary32 quotient, formed without a division
// per element by Markstein's correction (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990): with r = RN(1/s) and q0 = RN(x r), the remainder
// x - q0 s is exact and RN(q0 + (x - q0 s) r) = RN(x / s), provided nothing
// over- or underflows.  That is arranged per group: s = s' 2^-k with s' in
// [1, 2) (exact), x' = x 2^k (exact unless x / s is tiny or huge), and
// x' / s' = x / s.  |x'| is clamped to 2^21: beyond it |x / s| > 2^20 and the
// code saturates either way; if x' is tiny, so is x / s, and
// rint(x / s + zoff) = zoff either way.
#pragma once

#include <hip/hip_runtime.h>

namespace gptq {

struct Grid {
    float s, zoff, qlo, qhi, zadd, zero;
    float ss, rs;  // s' = s 2^k in [1, 2) and RN(1 / s')
    float zd;      // zero - zadd: code - zero = level - zd (small integers, exact)
    int k;
};

__device__ __forceinline__ void grid_scale(Grid &g) {
    int e;
    const float m = frexpf(g.s, &e);  // s = m 2^e, m in [0.5, 1)
    g.ss = 2.0f * m;
    g.k = 1 - e;
    g.rs = 1.0f / g.ss;  // IEEE division, once per group
}

// Grid of a group from its statistics: amax = max|x|, lo = min(min x, 0), hi = max(max x, 0).
__device__ __forceinline__ Grid grid_make(float amax, float lo, float hi, int bits, int sym) {
#pragma clang fp contract(off)
    Grid g;
    const float half = (float)(1 << (bits - 1));
    const float qmax_s = half - 1.0f;
    const float maxq = (float)((1 << bits) - 1);
    // symmetric
    float ss = amax / qmax_s;
    ss = (ss == 0.0f) ? 1.0f : ss;
    // asymmetric
    float sa = (hi - lo) / maxq;
    const bool za = (sa == 0.0f);
    sa = za ? 1.0f : sa;
    // The zero point is formed unconditionally and made opaque before the
    // select: otherwise the division goes under a branch, and the compiler
    // then sinks the pending weight updates of later columns past it.
    float zq = fminf(fmaxf(rintf(-lo / sa), 0.0f), maxq);
    asm volatile("" : "+v"(zq));
    const float z = za ? 0.0f : zq;
    g.s = sym ? ss : sa;
    g.zoff = sym ? 0.0f : z;
    g.qlo = sym ? -qmax_s : 0.0f;
    g.qhi = sym ? qmax_s : maxq;
    g.zadd = sym ? half : 0.0f;
    g.zero = sym ? half : z;
    g.zd = g.zero - g.zadd;
    grid_scale(g);
    return g;
}

// A grid given by its stored scale and zero point.
__device__ __forceinline__ Grid grid_from_stored(float s, float zero, int bits, int sym) {
    Grid g;
    const float half = (float)(1 << (bits - 1));
    g.s = s;
    g.zoff = sym ? 0.0f : zero;
    g.qlo = sym ? -(half - 1.0f) : 0.0f;
    g.qhi = sym ? (half - 1.0f) : (float)((1 << bits) - 1);
    g.zadd = sym ? half : 0.0f;
    g.zero = zero;
    g.zd = zero - g.zadd;
    grid_scale(g);
    return g;
}

// Compact form {s, zoff, RN(1/s'), k} of a grid, for lookups per column: s' =
// s 2^k is rebuilt exactly by ldexp, and zd equals zoff (symmetric: both 0;
// asymmetric: zadd = 0, so zd = zero = zoff).
__device__ __forceinline__ float4 grid_pack(const Grid &g) { return make_float4(g.s, g.zoff, g.rs, __int_as_float(g.k)); }

__device__ __forceinline__ Grid grid_unpack(float4 t, int bits, int sym) {
    Grid g;
    const float half = (float)(1 << (bits - 1));
    g.s = t.x;
    g.zoff = t.y;
    g.zd = t.y;
    g.rs = t.z;
    g.k = __float_as_int(t.w);
    g.ss = ldexpf(t.x, g.k);
    g.qlo = sym ? -(half - 1.0f) : 0.0f;
    g.qhi = sym ? (half - 1.0f) : (float)((1 << bits) - 1);
    g.zadd = sym ? half : 0.0f;
    g.zero = sym ? half : t.y;
    return g;
}

// Grid level clamp(rint(x / s + zoff), qlo, qhi); the stored code is level + zadd.
__device__ __forceinline__ float grid_level(float x, const Grid &g) {
#pragma clang fp contract(off)
    const float xs = __builtin_amdgcn_fmed3f(ldexpf(x, g.k), -2097152.0f, 2097152.0f);
    const float q0 = xs * g.rs;
    const float qd = fmaf(fmaf(-q0, g.ss, xs), g.rs, q0);  // RN(x / s)
    return __builtin_amdgcn_fmed3f(rintf(qd + g.zoff), g.qlo, g.qhi);
}

// Stored code (as a float holding a small integer).
__device__ __forceinline__ float grid_code(float x, const Grid &g) { return grid_level(x, g) + g.zadd; }

}  // namespace gptq
