// Launcher of the block swap between two pools (swap_blocks in the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Copies, for each pair (src, dst) of block_mapping, block src of the source
// pools to block dst of the destination pools (K and V, block_bytes each).
// Any pointer may be device memory or device-accessible pinned host memory.
hipError_t launch_swap_blocks(const void* src_key, const void* src_value, void* dst_key,
                              void* dst_value, const int64_t* block_mapping, int num_pairs,
                              int src_blocks, int dst_blocks, int64_t block_bytes,
                              hipStream_t stream);

}  // namespace pkv
