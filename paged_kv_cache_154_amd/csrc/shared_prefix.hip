// The merge step of shared-prefix decode. A sample of a group attends over
// the group's shared prefix and then its own suffix; the two parts are
// computed apart (the prefix once for all samples of the group, the suffix
// per sample), each as a normalised output o and the log2 of its sum of
// weights, lse. The softmax over the union of the two token sets is then the
// weighted mean of the two parts, weights 2^lse: a row that saw no token
// (lse = -1e30) weighs nothing against one that did.

#include "shared_prefix.h"

namespace pkv {
namespace {

template <class OutT>
__device__ inline void store4(void* out, int64_t i, float4 x) {
  if constexpr (sizeof(OutT) == 4) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + i) = x;
  } else {
    const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<OutT>(x.x)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<OutT>(x.y)) << 16);
    const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<OutT>(x.z)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<OutT>(x.w)) << 16);
    *reinterpret_cast<uint2*>(static_cast<OutT*>(out) + i) = make_uint2(lo, hi);
  }
}

// One thread per 4 consecutive values of a row.
template <class OutT>
__global__ __launch_bounds__(256) void cascade_merge_kernel(void* __restrict__ out,
                                                            const float4* __restrict__ o_a,
                                                            const float* __restrict__ lse_a,
                                                            const float4* __restrict__ o_b,
                                                            const float* __restrict__ lse_b,
                                                            int64_t rows, int quads_per_row) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= rows * quads_per_row) return;
  const int64_t row = gid / quads_per_row;
  const float la = lse_a[row];
  const float lb = lse_b[row];
  const float m = fmaxf(la, lb);
  const float wa = exp2f(la - m);
  const float wb = exp2f(lb - m);
  const float den = wa + wb;
  const float4 a = o_a[gid];
  const float4 b = o_b[gid];
  store4<OutT>(out, gid * 4,
               make_float4((wa * a.x + wb * b.x) / den, (wa * a.y + wb * b.y) / den,
                           (wa * a.z + wb * b.z) / den, (wa * a.w + wb * b.w) / den));
}

}  // namespace

hipError_t launch_cascade_merge(void* out, const float* o_a, const float* lse_a, const float* o_b,
                                const float* lse_b, int64_t rows, int head_dim, int out_dtype,
                                hipStream_t stream) {
  const int qpr = head_dim / 4;
  const int64_t total = rows * qpr;
  const unsigned grid = (unsigned)((total + 255) / 256);
  const float4* a = reinterpret_cast<const float4*>(o_a);
  const float4* b = reinterpret_cast<const float4*>(o_b);
  switch (out_dtype) {
    case 0:
      cascade_merge_kernel<float><<<dim3(grid), dim3(256), 0, stream>>>(out, a, lse_a, b, lse_b, rows, qpr);
      break;
    case 1:
      cascade_merge_kernel<_Float16><<<dim3(grid), dim3(256), 0, stream>>>(out, a, lse_a, b, lse_b, rows, qpr);
      break;
    case 2:
      cascade_merge_kernel<__bf16><<<dim3(grid), dim3(256), 0, stream>>>(out, a, lse_a, b, lse_b, rows, qpr);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv
