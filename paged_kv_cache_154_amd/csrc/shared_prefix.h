// Launcher of the merge step of shared-prefix (cascade) decode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// out[r] = (w_a o_a[r] + w_b o_b[r]) / (w_a + w_b), w_x = 2^(lse_x[r] - max(lse_a[r], lse_b[r])),
// for `rows` rows of head_dim fp32 values; out is fp32 (out_dtype 0), fp16 (1) or bf16 (2).
hipError_t launch_cascade_merge(void* out, const float* o_a, const float* lse_a, const float* o_b,
                                const float* lse_b, int64_t rows, int head_dim, int out_dtype,
                                hipStream_t stream);

}  // namespace pkv
