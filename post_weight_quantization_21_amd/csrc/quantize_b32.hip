// Column-pass batch kernels for batches of 32 columns.
#include "block_kernel.h"

namespace gptq {
hipError_t launch_block_32(const BlockArgs &a, int gt, int src, hipStream_t s) { return launch_block_bt<32>(a, gt, src, s); }
}  // namespace gptq
