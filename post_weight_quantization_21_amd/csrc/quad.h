// Lane exchange inside quads (4 consecutive lanes of a wave64) through DPP.
#pragma once

#include <hip/hip_runtime.h>

namespace gptq {

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Value of lane `src_lane` of each quad (src_lane is a constant after unrolling).
__device__ __forceinline__ float quad_bcast(float v, int src_lane) {
    switch (src_lane) {
    case 0: return dpp_f<0x00>(v);
    case 1: return dpp_f<0x55>(v);
    case 2: return dpp_f<0xAA>(v);
    default: return dpp_f<0xFF>(v);
    }
}
__device__ __forceinline__ float quad_xor1(float v) { return dpp_f<0xB1>(v); }  // quad_perm(1,0,3,2)
__device__ __forceinline__ float quad_xor2(float v) { return dpp_f<0x4E>(v); }  // quad_perm(2,3,0,1)

}  // namespace gptq
