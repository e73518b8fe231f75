// Integer grids of GPTQ's quantizer, device side.
//
// Symmetric and asymmetric uniform grids as defined on page "LLM 量化方法原理
// 与实现详解", §2.2 (scale from max|x| or from the range, zero point, rounding
// of x/scale (+ zero) and clamping), applied per group of consecutive input
// columns (§2.3).  All decisions are binary32 with round-half-to-even
// (v_rndne_f32), the rounding of the pages' torch.round.  Readings of points
// the pages leave open: the asymmetric range always contains 0
// (lo = min(min x, 0), hi = max(max x, 0)); a zero-width group gets scale 1.
#pragma once

#include <hip/hip_runtime.h>

namespace gptq {

struct GridSpec {
    int bits;
    int sym;
};

// Symmetric grid from max|x| of the group.
__device__ __forceinline__ void grid_sym(float amax, int bits, float &scale, float &zero) {
#pragma clang fp contract(off)
    const float qmax = (float)((1 << (bits - 1)) - 1);
    float s = amax / qmax;
    scale = (s == 0.0f) ? 1.0f : s;
    zero = (float)(1 << (bits - 1));
}

// Asymmetric grid from the group's min and max (both already clamped to span 0).
__device__ __forceinline__ void grid_asym(float lo, float hi, int bits, float &scale, float &zero) {
#pragma clang fp contract(off)
    const float maxq = (float)((1 << bits) - 1);
    float s = (hi - lo) / maxq;
    if (s == 0.0f) {
        scale = 1.0f;
        zero = 0.0f;
    } else {
        float z = rintf(-lo / s);
        scale = s;
        zero = fminf(fmaxf(z, 0.0f), maxq);
    }
}

// Stored code (as a float holding a small integer).
__device__ __forceinline__ float grid_code(float x, float scale, float zero, int bits, int sym) {
#pragma clang fp contract(off)
    if (sym) {
        const float qmax = (float)((1 << (bits - 1)) - 1);
        float q = rintf(x / scale);
        q = fminf(fmaxf(q, -qmax), qmax);
        return q + zero;
    }
    const float maxq = (float)((1 << bits) - 1);
    float q = rintf(x / scale + zero);
    return fminf(fmaxf(q, 0.0f), maxq);
}

// Rounded to fp32 on its own (never fused into a following add), like the stored format.
__device__ __forceinline__ float grid_dequant(float code, float scale, float zero) {
#pragma clang fp contract(off)
    return (code - zero) * scale;
}

}  // namespace gptq
