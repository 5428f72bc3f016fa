// Launch of the streaming-read kernel (a measurement aid, not part of decode).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t stream);

}  // namespace pkv
