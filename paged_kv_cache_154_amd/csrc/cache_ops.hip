// KV-pool maintenance kernels for CDNA4 (gfx950): the new-token scatter
// (reshape_and_cache), the copy-on-write block copy (copy_blocks) and the
// contract check of decode inputs. All are pure data movement in 16-byte
// units: one lane moves one 16-byte chunk, so a wave moves 1 KiB per access
// and consecutive lanes touch consecutive addresses.

#include "pagedkv_internal.h"

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

hipError_t launch_check_decode_inputs(const int32_t* block_table, const int32_t* seq_lens,
                                      int num_seqs, int block_size, int num_blocks, int max_blocks,
                                      int max_seq_len, int32_t* counts, hipStream_t stream) {
  check_decode_inputs_kernel<<<dim3(1), dim3(256), 0, stream>>>(
      block_table, seq_lens, num_seqs, block_size, num_blocks, max_blocks, max_seq_len, counts);
  return hipGetLastError();
}

}  // namespace pkv
