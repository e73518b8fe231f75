// Column-pass batch kernels for batches of 64 columns.
#include "block_kernel.h"

namespace gptq {
hipError_t launch_block_64(const BlockArgs &a, int gt, int src, hipStream_t s) { return launch_block_bt<64>(a, gt, src, s); }
}  // namespace gptq
