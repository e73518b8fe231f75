// Arguments of the column-pass batch kernel (see block_kernel.h) and its launchers.
#pragma once

#include "common.h"

namespace gptq {

struct BlockArgs {
    float *W;  // [d_out][ldw], processing order
    int64_t ldw, d_out, c0;
    int ncols;  // columns in this batch (<= batch width)
    const float *U;
    int64_t ldu;
    float *Et;  // [batch width][ldet] fp32, holds -e; ldet >= rows covered by the grid
    int64_t ldet;
    uint8_t *codes;  // [d_out][ldc], original column order
    int64_t ldc;
    const int32_t *perm;  // processing position -> original column (code destination), or NULL
    // grids fitted before the pass, per column: processing position -> original
    // column, whose group's stored grid is used (the grid-per-column kernels only)
    const int32_t *gperm;
    const float4 *gtab;  // [d_out][ng] packed grids (grid_pack) for the per-column lookup
    float *scales, *zeros;
    int64_t ng, g;
    int bits, sym, vec;
};

constexpr int kBlockThreads = 256;

// How the batch kernel gets its grids:
//   kFitGrids    fitted from the current weights at each group start (GT > 0),
//                or read from scales/zeros at the batch start (GT == 0: the
//                group spans whole batches and was fitted before the batch);
//   kStoredGrids read from scales/zeros (fitted before the pass) at each
//                group start (GT > 0) or at the batch start (GT == 0);
//   kColumnGrids read from gtab for every column, group gperm[c] / g (groups
//                in original column order while columns are processed in
//                another order).
enum GridSource { kFitGrids = 0, kStoredGrids = 1, kColumnGrids = 2 };

hipError_t launch_block_32(const BlockArgs &a, int gt, int src, hipStream_t s);
hipError_t launch_block_64(const BlockArgs &a, int gt, int src, hipStream_t s);
hipError_t launch_block_128(const BlockArgs &a, int gt, int src, hipStream_t s);

// Column indices read from a permutation are clamped into [0, n) so that a
// malformed permutation can only give wrong results, never a wild access.
__device__ __forceinline__ int32_t clamp_col(int32_t c, int64_t n) {
    return c < 0 ? 0 : (c >= n ? (int32_t)(n - 1) : c);
}

}  // namespace gptq
