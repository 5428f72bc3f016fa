// KV-pool maintenance kernels for CDNA4 (gfx950): the new-token scatter
// (reshape_and_cache), the copy-on-write block copy (copy_blocks) and the
// contract checks of decode and cache-operation inputs. All are pure data movement in 16-byte
// units: one lane moves one 16-byte chunk, so a wave moves 1 KiB per access
// and consecutive lanes touch consecutive addresses.

#include "pagedkv_internal.h"
#include "swap_blocks.h"

namespace pkv {
namespace {

// Pools are [num_blocks, block_size, num_kv_heads, head_dim]: the row of slot
// `slot` (all KV heads of one token) starts at slot * row_bytes, so the slot
// handed out by the block engine (block * block_size + offset, "LLM
// inference engine internals" section 2.3) indexes the pool directly.
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ key_cache,
    uint4* __restrict__ value_cache, const int64_t* __restrict__ slot_mapping, int num_tokens,
    int chunks_per_row, int64_t num_slots) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * chunks_per_row;
  if (gid >= total) return;
  const int64_t i = gid / chunks_per_row;
  const int64_t c = gid - i * chunks_per_row;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // no slot (padding) or outside the pool
  const int64_t src = i * chunks_per_row + c;
  const int64_t dst = slot * chunks_per_row + c;
  key_cache[dst] = key[src];
  value_cache[dst] = value[src];
}

// The e4m3 code of x (OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormals
// m * 2^-9, no infinity, 0x7F the NaN): the nearest e4m3 value with ties to
// the even code, magnitudes of 448 and more (infinity too) saturating to 448,
// NaN kept. Exact in fp32: the subnormal step is a power of two, and the
// normal range rounds the fp32 mantissa to 3 bits by integer arithmetic.
__device__ inline uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a == a)) return sign | 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {
    // below 2^-6: multiples of 2^-9, rounded half to even (8 is code 0x08 = 2^-6)
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  }
  // 2^-6 <= a < 448: drop 20 of the 23 mantissa bits, half to even; a carry
  // out of the mantissa moves the exponent up, as it should
  const uint32_t au = u & 0x7FFFFFFFu;
  const uint32_t r = au + 0x7FFFFu + ((au >> 20) & 1u);
  const uint32_t e = (r >> 23) - 120u;  // fp32 exponent bias 127 -> e4m3 bias 7
  return sign | (e << 3) | ((r >> 20) & 7u);
}

// The quantising scatter of an e4m3 cache: one lane per 16 elements of a
// token's row (within one KV head), each divided by its KV head's scale in
// fp32 and stored as 16 one-byte codes. T is the type of key and value.
template <class T>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const T* __restrict__ key, const T* __restrict__ value, uint4* __restrict__ key_cache,
    uint4* __restrict__ value_cache, const int64_t* __restrict__ slot_mapping,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int num_tokens,
    int chunks_per_row, int chunks_per_head, int64_t num_slots) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * chunks_per_row;
  if (gid >= total) return;
  const int64_t i = gid / chunks_per_row;
  const int c = (int)(gid - i * chunks_per_row);
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // no slot (padding) or outside the pool
  const int head = c / chunks_per_head;
  constexpr int NQ = (int)sizeof(T);          // 16-byte loads per 16 elements
  auto quantise = [&](const T* src, float scale) -> uint4 {
    union { uint4 v[NQ]; T e[16]; } in;
#pragma unroll
    for (int k = 0; k < NQ; ++k) in.v[k] = reinterpret_cast<const uint4*>(src)[k];
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e >> 2] |= e4m3_code(static_cast<float>(in.e[e]) / scale) << (8 * (e & 3));
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  const int64_t src = (i * chunks_per_row + c) * 16;
  const int64_t dst = slot * chunks_per_row + c;
  key_cache[dst] = quantise(key + src, k_scale[head]);
  value_cache[dst] = quantise(value + src, v_scale[head]);
}

// Whole-block copies src -> dst for K and V ("vLLM core concepts" section
// 4.2.2: a shared block is copied before it is written).
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
    const int64_t* __restrict__ block_mapping, int num_pairs, int num_blocks,
    int64_t chunks_per_block) {
  const int64_t total = (int64_t)num_pairs * chunks_per_block;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < total; gid += stride) {
    const int64_t pr = gid / chunks_per_block;
    const int64_t c = gid - pr * chunks_per_block;
    const int64_t src = block_mapping[2 * pr];
    const int64_t dst = block_mapping[2 * pr + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
    key_cache[dst * chunks_per_block + c] = key_cache[src * chunks_per_block + c];
    value_cache[dst * chunks_per_block + c] = value_cache[src * chunks_per_block + c];
  }
}

// Whole-block moves between two pools of the same layout, K and V: preemption
// by swapping out to a CPU swap space and back ("LLM inference engine
// internals" sections 3.1-3.2). Either pool may be pinned host memory, read
// or written by the kernel across the host link; one launch covers every
// pair, each lane moving 4 chunks of 16 bytes per pass (all loads issued
// before the stores) so that many host-link requests are in flight.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v, uint4* __restrict__ dst_k,
    uint4* __restrict__ dst_v, const int64_t* __restrict__ block_mapping, int num_pairs,
    int src_blocks, int dst_blocks, int64_t chunks_per_block) {
  constexpr int U = 4;
  const int64_t total = (int64_t)num_pairs * chunks_per_block;
  const int64_t stride = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < total; base += stride) {
    uint4 k[U], v[U];
    int64_t dk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      dk[u] = -1;
      const int64_t gid = base + (int64_t)u * 256;
      if (gid >= total) continue;
      const int64_t pr = gid / chunks_per_block;
      const int64_t c = gid - pr * chunks_per_block;
      const int64_t src = block_mapping[2 * pr];
      const int64_t dst = block_mapping[2 * pr + 1];
      if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) continue;
      k[u] = src_k[src * chunks_per_block + c];
      v[u] = src_v[src * chunks_per_block + c];
      dk[u] = dst * chunks_per_block + c;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (dk[u] < 0) continue;
      dst_k[dk[u]] = k[u];
      dst_v[dk[u]] = v[u];
    }
  }
}

// One workgroup counts contract violations of decode inputs: table entries of
// used logical blocks outside the pool, and lengths outside [0, max_seq_len].
__global__ __launch_bounds__(256) void check_decode_inputs_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int num_seqs,
    int block_size, int num_blocks, int max_blocks, int max_seq_len, int32_t* __restrict__ counts) {
  __shared__ int s_blk[256];
  __shared__ int s_len[256];
  int bad_blk = 0, bad_len = 0;
  for (int s = threadIdx.x; s < num_seqs; s += 256) {
    const int L = seq_lens[s];
    if (L < 0 || L > max_seq_len) ++bad_len;
  }
  const int64_t total = (int64_t)num_seqs * max_blocks;
  for (int64_t idx = threadIdx.x; idx < total; idx += 256) {
    const int s = (int)(idx / max_blocks);
    const int i = (int)(idx - (int64_t)s * max_blocks);
    int L = seq_lens[s];
    L = L < 0 ? 0 : (L > max_seq_len ? max_seq_len : L);
    if (i < (L + block_size - 1) / block_size) {
      const int b = block_table[idx];
      if (b < 0 || b >= num_blocks) ++bad_blk;
    }
  }
  s_blk[threadIdx.x] = bad_blk;
  s_len[threadIdx.x] = bad_len;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      s_blk[threadIdx.x] += s_blk[threadIdx.x + w];
      s_len[threadIdx.x] += s_len[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x < 2) counts[threadIdx.x] = threadIdx.x == 0 ? s_blk[0] : s_len[0];
}

// Clears n counters (a kernel rather than a memset, so that a captured
// graph holds no memset node).
__global__ __launch_bounds__(64) void zero_counts_kernel(int32_t* counts, int n) {
  if ((int)threadIdx.x < n) counts[threadIdx.x] = 0;
}

// Contract check of the cache operations' index arguments. Workgroups
// [0, slot_groups) take 256 tokens of slot_mapping each, the rest 256 pairs of
// block_mapping each; every workgroup compares its entries with the others
// through LDS tiles of 256 and adds what it finds to
//   counts[0]  slots >= num_slots (negative slots mean "no slot")
//   counts[1]  slots in the pool equal to the slot of an earlier token
//              (append_slot hands out each slot once: "LLM inference engine
//              internals" section 2.3)
//   counts[2]  pairs with a block id outside [0, num_blocks)
//   counts[3]  pairs (ids in range) whose destination is some pair's source
//              or an earlier pair's destination (blocks_to_copy destinations
//              are fresh blocks: the same page, section 3.1)
__global__ __launch_bounds__(256) void check_cache_ops_kernel(
    const int64_t* __restrict__ slots, int num_tokens, int64_t num_slots, const int64_t* __restrict__ pairs,
    int num_pairs, int num_blocks, int slot_groups, int32_t* __restrict__ counts) {
  __shared__ int64_t tile[2 * 256];
  const int t = threadIdx.x;
  if ((int)blockIdx.x < slot_groups) {
    const int i = blockIdx.x * 256 + t;
    const int64_t me = i < num_tokens ? slots[i] : -1;
    const bool in_pool = me >= 0 && me < num_slots;
    int dup = 0;
    const int end = min(num_tokens, (int)(blockIdx.x + 1) * 256);  // tokens before this group's last
    for (int j0 = 0; j0 < end; j0 += 256) {
      __syncthreads();
      tile[t] = j0 + t < num_tokens ? slots[j0 + t] : -1;
      __syncthreads();
      if (in_pool && !dup) {
        const int n = min(256, i - j0);  // earlier tokens only
        for (int k = 0; k < n; ++k) dup |= tile[k] == me;
      }
    }
    if (me >= num_slots) atomicAdd(counts + 0, 1);
    if (dup) atomicAdd(counts + 1, 1);
  } else {
    const int i = ((int)blockIdx.x - slot_groups) * 256 + t;
    int64_t src = -1, dst = -1;
    if (i < num_pairs) {
      src = pairs[2 * (int64_t)i];
      dst = pairs[2 * (int64_t)i + 1];
    }
    const bool in_range = i < num_pairs && src >= 0 && src < num_blocks && dst >= 0 && dst < num_blocks;
    int overlap = 0;
    for (int j0 = 0; j0 < num_pairs; j0 += 256) {
      __syncthreads();
      tile[2 * t] = j0 + t < num_pairs ? pairs[2 * (int64_t)(j0 + t)] : -1;
      tile[2 * t + 1] = j0 + t < num_pairs ? pairs[2 * (int64_t)(j0 + t) + 1] : -1;
      __syncthreads();
      if (in_range && !overlap) {
        const int n = min(256, num_pairs - j0);
        for (int k = 0; k < n; ++k)
          overlap |= tile[2 * k] == dst || (j0 + k < i && tile[2 * k + 1] == dst);
      }
    }
    if (i < num_pairs && !in_range) atomicAdd(counts + 2, 1);
    if (overlap) atomicAdd(counts + 3, 1);
  }
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int64_t* slot_mapping,
                                    int num_tokens, int row_bytes, int64_t num_slots,
                                    hipStream_t stream) {
  const int chunks = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * chunks;
  const unsigned grid = (unsigned)((total + 255) / 256);
  reshape_and_cache_kernel<<<dim3(grid), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(key), static_cast<const uint4*>(value),
      static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache), slot_mapping, num_tokens,
      chunks, num_slots);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                                        void* value_cache, const int64_t* slot_mapping,
                                        const float* k_scale, const float* v_scale, int num_tokens,
                                        int num_kv_heads, int head_dim, int src_dtype,
                                        int64_t num_slots, hipStream_t stream) {
  const int per_head = head_dim / 16;
  const int chunks = num_kv_heads * per_head;
  const int64_t total = (int64_t)num_tokens * chunks;
  const unsigned grid = (unsigned)((total + 255) / 256);
  uint4* kc = static_cast<uint4*>(key_cache);
  uint4* vc = static_cast<uint4*>(value_cache);
  switch (src_dtype) {
    case 0:
      reshape_and_cache_fp8_kernel<float><<<dim3(grid), dim3(256), 0, stream>>>(
          static_cast<const float*>(key), static_cast<const float*>(value), kc, vc, slot_mapping,
          k_scale, v_scale, num_tokens, chunks, per_head, num_slots);
      break;
    case 1:
      reshape_and_cache_fp8_kernel<_Float16><<<dim3(grid), dim3(256), 0, stream>>>(
          static_cast<const _Float16*>(key), static_cast<const _Float16*>(value), kc, vc,
          slot_mapping, k_scale, v_scale, num_tokens, chunks, per_head, num_slots);
      break;
    case 2:
      reshape_and_cache_fp8_kernel<__bf16><<<dim3(grid), dim3(256), 0, stream>>>(
          static_cast<const __bf16*>(key), static_cast<const __bf16*>(value), kc, vc,
          slot_mapping, k_scale, v_scale, num_tokens, chunks, per_head, num_slots);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping,
                              int num_pairs, int num_blocks, int64_t block_bytes,
                              hipStream_t stream) {
  const int64_t chunks = block_bytes / 16;
  const int64_t total = (int64_t)num_pairs * chunks;
  int64_t grid = (total + 255) / 256;
  if (grid > 65536) grid = 65536;
  copy_blocks_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
      static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache), block_mapping, num_pairs,
      num_blocks, chunks);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const void* src_key, const void* src_value, void* dst_key,
                              void* dst_value, const int64_t* block_mapping, int num_pairs,
                              int src_blocks, int dst_blocks, int64_t block_bytes,
                              hipStream_t stream) {
  const int64_t chunks = block_bytes / 16;
  const int64_t total = (int64_t)num_pairs * chunks;
  int64_t grid = (total + 1023) / 1024;
  if (grid > 4096) grid = 4096;
  swap_blocks_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(src_key), static_cast<const uint4*>(src_value),
      static_cast<uint4*>(dst_key), static_cast<uint4*>(dst_value), block_mapping, num_pairs,
      src_blocks, dst_blocks, chunks);
  return hipGetLastError();
}

hipError_t launch_check_decode_inputs(const int32_t* block_table, const int32_t* seq_lens,
                                      int num_seqs, int block_size, int num_blocks, int max_blocks,
                                      int max_seq_len, int32_t* counts, hipStream_t stream) {
  check_decode_inputs_kernel<<<dim3(1), dim3(256), 0, stream>>>(
      block_table, seq_lens, num_seqs, block_size, num_blocks, max_blocks, max_seq_len, counts);
  return hipGetLastError();
}

hipError_t launch_check_cache_ops(const int64_t* slot_mapping, int num_tokens, int64_t num_slots,
                                  const int64_t* block_mapping, int num_pairs, int num_blocks,
                                  int32_t* counts, hipStream_t stream) {
  zero_counts_kernel<<<dim3(1), dim3(64), 0, stream>>>(counts, 4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int slot_groups = (num_tokens + 255) / 256;
  const int pair_groups = (num_pairs + 255) / 256;
  if (slot_groups + pair_groups == 0) return hipSuccess;
  check_cache_ops_kernel<<<dim3(slot_groups + pair_groups), dim3(256), 0, stream>>>(
      slot_mapping, num_tokens, num_slots, block_mapping, num_pairs, num_blocks, slot_groups, counts);
  return hipGetLastError();
}

}  // namespace pkv
