// Internal declarations shared by the kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Launch parameters of the decode kernels (host-validated).
struct DecodeParams {
  void* out;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  // control word of the launch: (workgroups finished << 32) | items taken
  // from the counter; zero when the launch starts, and set back to zero by
  // the last workgroup to finish
  unsigned long long* work;
  float* ws_o;    // [S, q_len, H, NP, D] weighted-V partial sums (split only); the D
                  // values of one partial: the (0, 1) pairs of its quads, then the (2, 3) pairs
  float* ws_ml;   // [S, q_len, H, NP, 2] (running max in log2 units, sum of weights)
  uint32_t* arrive;  // [S, Hkv] partitions done (split only): zero when the launch
                     // starts, set back to zero by the partition that merges
  const float* k_scale;  // [Hkv] e4m3 pools: value = code * scale (else unused)
  const float* v_scale;  // [Hkv]
  int num_seqs;
  int q_len;           // new tokens per sequence (1: decode); query and out are
                       // [S, q_len, H, D]; token j sees positions <= L - q_len + j
  int num_heads;
  int num_kv_heads;
  int group;           // num_heads / num_kv_heads
  int num_blocks;
  int max_blocks;      // block-table row length
  int max_seq_len;
  int partition;       // tokens per partition (multiple of 16 and block_size)
  int num_partitions;  // partitions per sequence at most (ceil(max_seq_len / partition)), >= 1
  float scale_log2;    // scale * log2(e)
  int out_f32;         // 1: out is fp32; 0: out has the KV dtype
  int causal;          // q_len > 1: 1 new token j sees positions <= L - q_len + j; 0 every row sees all L
  float* lse;          // optional [S, q_len, H]: M + log2(sum of weights) per row, log2 units (or -1e30)
};

// Tokens a wave handles per step (one MFMA tile of keys).
constexpr int kTile = 16;
// Waves per decode workgroup.
#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 8
#endif
constexpr int kWaves = PKV_DECODE_WAVES;
constexpr int kThreads = 64 * kWaves;
// Largest partition whose block-table slice is staged in LDS.
constexpr int kMaxPartition = 16384;
// Sequences per launch of the partition kernel (its schedule lives in LDS).
constexpr int kMaxSeqsPerLaunch = 2048;

// kv_dtype: 0 fp32, 1 fp16, 2 bf16 (the query's type too), 3 e4m3 with a
// query of type query_dtype (1 fp16 or 2 bf16).
// start / stop (optional): events updated with the start of the first launch
// and the end of the last (hipExtLaunchKernel's own timestamps).
hipError_t launch_decode(const DecodeParams& p, int kv_dtype, int query_dtype, int head_dim,
                         int block_size, hipStream_t stream, hipEvent_t start = nullptr,
                         hipEvent_t stop = nullptr);

// Two passes over the same pools (dtypes as for launch_decode) in one launch,
// the second's items taken after the first's: a.work and b.work are separate
// workspaces. hipErrorNotSupported when they do not fit one launch (then
// nothing is launched).
hipError_t launch_decode_pair(const DecodeParams& a, const DecodeParams& b, int kv_dtype, int query_dtype,
                              int head_dim, int block_size, hipStream_t stream);

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value,
                                        void* key_cache, void* value_cache,
                                        const int64_t* slot_mapping, const float* k_scale,
                                        const float* v_scale, int num_tokens,
                                        int num_kv_heads, int head_dim, int src_dtype,
                                        int64_t num_slots, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value,
                                    void* key_cache, void* value_cache,
                                    const int64_t* slot_mapping, int num_tokens,
                                    int row_bytes, int64_t num_slots,
                                    hipStream_t stream);

hipError_t launch_copy_blocks(void* key_cache, void* value_cache,
                              const int64_t* block_mapping, int num_pairs,
                              int num_blocks, int64_t block_bytes,
                              hipStream_t stream);

hipError_t launch_check_decode_inputs(const int32_t* block_table,
                                      const int32_t* seq_lens, int num_seqs,
                                      int block_size, int num_blocks,
                                      int max_blocks, int max_seq_len,
                                      int32_t* counts, hipStream_t stream);

hipError_t launch_check_cache_ops(const int64_t* slot_mapping, int num_tokens, int64_t num_slots,
                                  const int64_t* block_mapping, int num_pairs, int num_blocks,
                                  int32_t* counts, hipStream_t stream);

}  // namespace pkv
