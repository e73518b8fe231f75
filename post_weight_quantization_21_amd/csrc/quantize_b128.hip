// Column-pass batch kernels for batches of 128 columns.
#include "block_kernel.h"

namespace gptq {
hipError_t launch_block_128(const BlockArgs &a, int gt, int src, hipStream_t s) { return launch_block_bt<128>(a, gt, src, s); }
}  // namespace gptq
