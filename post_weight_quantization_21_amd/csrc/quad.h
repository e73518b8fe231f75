// Lane exchange inside quads (4 consecutive lanes of a wave64) and rows (16
// consecutive lanes) through DPP.
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

// Value of lane `src_lane` of each row of 16 lanes (row_newbcast; src_lane is
// a constant after unrolling).
__device__ __forceinline__ float row_bcast(float v, int src_lane) {
    switch (src_lane) {
    case 0: return dpp_f<0x150>(v);
    case 1: return dpp_f<0x151>(v);
    case 2: return dpp_f<0x152>(v);
    case 3: return dpp_f<0x153>(v);
    case 4: return dpp_f<0x154>(v);
    case 5: return dpp_f<0x155>(v);
    case 6: return dpp_f<0x156>(v);
    case 7: return dpp_f<0x157>(v);
    case 8: return dpp_f<0x158>(v);
    case 9: return dpp_f<0x159>(v);
    case 10: return dpp_f<0x15A>(v);
    case 11: return dpp_f<0x15B>(v);
    case 12: return dpp_f<0x15C>(v);
    case 13: return dpp_f<0x15D>(v);
    case 14: return dpp_f<0x15E>(v);
    default: return dpp_f<0x15F>(v);
    }
}
__device__ __forceinline__ float row_half_mirror(float v) { return dpp_f<0x141>(v); }  // lane i <- 7 - i in each half
__device__ __forceinline__ float row_mirror(float v) { return dpp_f<0x140>(v); }       // lane i <- 15 - i

// The same over the L lanes that own one output row (L = 4: a quad, L = 16: a row).
template <int L>
__device__ __forceinline__ float lanes_bcast(float v, int src_lane) {
    static_assert(L == 4 || L == 16, "four or sixteen lanes per row");
    if constexpr (L == 4) return quad_bcast(v, src_lane);
    else return row_bcast(v, src_lane);
}
// Exchange steps of a max/min over the L lanes: after steps 0 .. log2(L)-1,
// each lane has combined every lane of its group (quad: xor 1, xor 2; a row
// adds the half and whole mirrors, which pair every lane with the other quad
// of its half and then with the other half).
template <int L>
__device__ __forceinline__ float lanes_step(float v, int step) {
    switch (step) {
    case 0: return quad_xor1(v);
    case 1: return quad_xor2(v);
    case 2: return row_half_mirror(v);
    default: return row_mirror(v);
    }
}
template <int L>
constexpr int lanes_steps() { return L == 4 ? 2 : 4; }

}  // namespace gptq
