/*
 * pagedkv.h - C ABI of the paged KV-cache decode library for AMD CDNA4
 * (MI355X, gfx950).
 *
 * The problem, as the PagedAttention pages state it: the K and V of every
 * cached token live in fixed-size physical blocks of a shared pool; a
 * sequence reaches its tokens through a block table that maps its logical
 * block i to a physical block ("PagedAttention principle", tbr8.org,
 * sections 2.1-2.2; "LLM inference engine internals", sections 2.2-2.4).
 *
 * Conventions for every entry point:
 *   - Every pointer is a DEVICE pointer (memory of the current HIP device),
 *     dense and row-major; no strides. The caller allocates and owns all of
 *     it, including the workspace. The library allocates nothing, and the
 *     only host state it keeps is a cache of how many workgroups of each
 *     kernel fit on a device (a property of the device) and, once
 *     paged_attn_decode_noalloc has run on a device, the address of that
 *     entry point's static device scratch there. Per-call state lives
 *     in the caller's workspace (see paged_attn_decode): calls with separate
 *     workspaces are independent and may run concurrently; calls in order on
 *     one stream may share one. A call may be captured into a HIP graph and
 *     the graph replayed: every launch leaves its workspace's control area
 *     as it found it (zero).
 *   - Query, output, key/value rows, pools and the workspace move in 16-byte
 *     vector accesses: those pointers must be 16-byte aligned (every torch
 *     or hipMalloc allocation is), else the call returns PKV_ERR_SHAPE.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without waiting for it.
 *   - Return value: PKV_OK (0) or a negative pkv_status. Arguments are
 *     checked on the host before anything is launched; a call that fails the
 *     check launches nothing. PKV_ERR_HIP reports a launch failure
 *     (hipGetLastError after the launch). No C++ exception crosses the ABI.
 *   - Contents of device buffers (block ids, slots, lengths) are the
 *     caller's contract and are not checked in the fast path, but the kernels
 *     never read or write outside the buffers the shape arguments describe:
 *     an out-of-range block id, slot or length is skipped or clamped, and
 *     then the result for that sequence or token is unspecified.
 *     pagedkv_check_decode_inputs() reports such entries.
 *   - dtype codes: PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 (IEEE binary32,
 *     binary16, bfloat16), PKV_E4M3 = 3 (OCP FP8 E4M3: one byte, bias 7,
 *     3 mantissa bits, largest finite 448, 0x7F/0xFF NaN, no infinity; a
 *     KV-cache format that stands for code * scale with a scale per KV head,
 *     see the *_fp8 entry points; reshape_and_cache and copy_blocks move its
 *     codes as bytes like any other type).
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef PAGEDKV_STREAM_T_DEFINED
#define PAGEDKV_STREAM_T_DEFINED
/* Same type as HIP's hipStream_t (an opaque handle). */
typedef struct ihipStream_t* hipStream_t;
#endif
#ifndef PAGEDKV_EVENT_T_DEFINED
#define PAGEDKV_EVENT_T_DEFINED
/* Same type as HIP's hipEvent_t (an opaque handle). */
typedef struct ihipEvent_t* hipEvent_t;
#endif

enum pkv_dtype { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_E4M3 = 3 };

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,       /* inconsistent or negative sizes, or a misaligned pointer */
  PKV_ERR_UNSUPPORTED = -3, /* valid but not built: dtype, head_dim, block_size, group size */
  PKV_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  PKV_ERR_HIP = -5          /* the HIP runtime reported an error at launch */
};

/*
 * paged_attn_decode - one decode step of attention for a batch of sequences,
 * each with one query token, over K/V held in a paged block pool.
 *
 * For sequence s, query head h, with G = num_heads / num_kv_heads and KV head
 * j = h / G (consecutive query heads share a KV head), L = seq_lens[s]:
 *   k_t = key_cache[block_table[s][t / block_size], t % block_size, j, :]
 *   v_t = value_cache[same]                                   (t = 0 .. L-1)
 *   out[s, h, :] = sum_t softmax_t(scale * q . k_t) * v_t
 * The gather through the block table, the stop at seq_len and the score scale
 * follow the paged-attention listing of "PagedAttention principle" section
 * 2.2 and the two-level addressing of "LLM inference engine internals"
 * section 2.4; the softmax runs over all L positions of one (sequence, head).
 * L counts every cached token the query attends to, the new token included
 * (write it with reshape_and_cache first). L = 0 gives a zero row. Slots at
 * positions >= L are never read into the arithmetic (they may hold NaN).
 * Accumulation is in fp32.
 *
 *   out          [num_seqs, num_heads, head_dim], dtype out_dtype
 *   query        [num_seqs, num_heads, head_dim], dtype kv_dtype
 *   key_cache,
 *   value_cache  [num_blocks, block_size, num_kv_heads, head_dim], kv_dtype
 *   block_table  int32 [num_seqs, max_blocks_per_seq]; entries of logical
 *                blocks 0 .. ceil(L/block_size)-1 must be in [0, num_blocks)
 *   seq_lens     int32 [num_seqs], each in [0, max_seq_len]
 *   max_seq_len  host-side upper bound of seq_lens; sizes the launch without
 *                a device->host copy; must be <= max_blocks_per_seq*block_size
 *   scale        score scale (the pages use 1/sqrt(head_dim))
 *   kv_dtype     PKV_F32, PKV_F16 or PKV_BF16
 *   out_dtype    kv_dtype or PKV_F32 (narrowing rounds to nearest even)
 *   partition_size  tokens of one sequence partition, a multiple of 16 and
 *                of block_size; 0 lets the library choose (see
 *                paged_attn_partition_tokens). A sequence longer than one
 *                partition is split; each partition's (max, sum, weighted V)
 *                is written to the workspace, and the last partition of a
 *                (sequence, KV head) to finish merges them (one kernel).
 *                When one partition covers max_seq_len it may hold at most
 *                16384 tokens; a splitting partition likewise.
 *   workspace    device scratch of at least paged_attn_workspace_size(...)
 *                bytes for the same arguments (always needed). It begins
 *                with a control area that MUST BE ZERO when the workspace is
 *                first used: the decode kernel's control word (items taken,
 *                workgroups finished) and, when sequences are split, one
 *                arrival count per (sequence, KV head). Every call sets the
 *                control area back to zero before its last kernel ends, so
 *                zeroing once (hipMemset after hipMalloc) serves every later
 *                call, and a call captured into a HIP graph can be replayed
 *                any number of times. The control area is the first C bytes,
 *                C = 256 + (split ? roundup(4 * min(num_seqs, 2048) *
 *                num_kv_heads, 256) : 0); the rest holds the split-K
 *                partials and may hold anything (it is garbage after a
 *                call). A nonzero control area is a contract violation: the
 *                kernels still stay inside the buffers, but items are skipped
 *                or merged early and the output is unspecified. Calls that
 *                may run at the same time need separate workspaces; calls in
 *                order on one stream can share one.
 * Supported: head_dim 64 or 128; block_size 8, 16 or 32; 1 <= G <= 16;
 * num_blocks * block_size < 2^31.
 */
int paged_attn_decode(void* out, const void* query, const void* key_cache,
                      const void* value_cache, const int32_t* block_table,
                      const int32_t* seq_lens, int num_seqs, int num_heads,
                      int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_seq_len,
                      float scale, int kv_dtype, int out_dtype,
                      int partition_size, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attn_multi_query - attention of q_len new tokens per sequence over
 * the paged cache: the verification pass of speculative decoding, where the
 * target model checks a draft model's q_len candidate tokens in one forward
 * pass over the cached prefix ("LLM inference optimisation in practice"
 * sections 4.1-4.2; "vLLM core concepts" section 4.4.1; "LLM inference
 * engine internals" section 5.2: the candidates' K/V share the blocks), or
 * one chunk of a chunked prefill (the same page, section 5.3).
 *
 * The new tokens are the last q_len positions of each sequence (write their
 * K and V with reshape_and_cache first); new token j attends causally:
 *   out[s, j, h, :] = sum_{t <= L - q_len + j} softmax_t(scale * q[s, j, h] . k_t) * v_t
 * with L = seq_lens[s], k_t, v_t as in paged_attn_decode. A token that sees
 * no position (L < q_len) gives a zero row. q_len = 1 is paged_attn_decode.
 *
 *   out, query   [num_seqs, q_len, num_heads, head_dim]
 *   q_len        1 .. 128 / (num_heads / num_kv_heads): the q_len * G query
 *                rows of a KV head fill 16-column MFMA tiles, one per group
 *                of waves (up to 8 groups); beyond that PKV_ERR_UNSUPPORTED
 *   workspace    at least paged_attn_multi_query_workspace_size(...) bytes
 * All other arguments, the partitioning, the status codes and the
 * workspace rules are those of paged_attn_decode.
 */
int paged_attn_multi_query(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_table,
                           const int32_t* seq_lens, int num_seqs, int q_len,
                           int num_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int max_blocks_per_seq,
                           int max_seq_len, float scale, int kv_dtype, int out_dtype,
                           int partition_size, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attn_multi_query_workspace_size - paged_attn_workspace_size for
 * q_len new tokens per sequence (the partials hold q_len * num_heads rows per
 * sequence). 0 when the arguments are invalid or num_seqs is 0.
 */
size_t paged_attn_multi_query_workspace_size(int num_seqs, int q_len, int num_heads,
                                             int num_kv_heads, int head_dim,
                                             int block_size, int max_seq_len,
                                             int partition_size);

/*
 * paged_attn_decode_fp8, paged_attn_multi_query_fp8 - paged_attn_decode and
 * paged_attn_multi_query over an e4m3 KV cache ("LLM inference optimisation
 * in practice" section 6.2: attention computed on a low-precision KV cache,
 * halving the bytes each step reads from a 16-bit cache). Element d of the
 * K row of a cached token, KV head j, stands for
 *   e4m3_value(key_cache[...][j][d]) * k_scale[j],
 * and likewise for V with v_scale: the attention is that of the two entry
 * points above on those values. In the kernels the keys are widened to the
 * query's type (exactly) for the 16-bit MFMA, the values to fp32, k_scale
 * multiplies the scores and v_scale the output.
 *
 *   key_cache, value_cache  uint8 e4m3 codes [num_blocks, block_size, num_kv_heads, head_dim]
 *   k_scale, v_scale        fp32 [num_kv_heads], device memory
 *   query                   [num_seqs, (q_len,) num_heads, head_dim] of query_dtype
 *   query_dtype             PKV_F16 or PKV_BF16
 *   out_dtype               query_dtype or PKV_F32
 * Everything else (shapes, partitions, the workspace and its size, status
 * codes) is that of the 16-bit entry points; a NULL scale is PKV_ERR_NULL.
 */
int paged_attn_decode_fp8(void* out, const void* query, const void* key_cache,
                          const void* value_cache, const float* k_scale, const float* v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                          int num_heads, int num_kv_heads, int head_dim, int block_size,
                          int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                          int query_dtype, int out_dtype, int partition_size, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

int paged_attn_multi_query_fp8(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const float* k_scale,
                               const float* v_scale, const int32_t* block_table,
                               const int32_t* seq_lens, int num_seqs, int q_len, int num_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, int max_seq_len, float scale,
                               int query_dtype, int out_dtype, int partition_size,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attn_decode_shared_prefix - decode for groups of sequences that share
 * a prefix of whole blocks (parallel sampling: the samples of one prompt
 * point at the same physical blocks, "vLLM core concepts" section 4.2.2,
 * "LLM inference engine internals" section 3.3; "PagedAttention principle"
 * section 5), reading each shared block once per group instead of once per
 * sample. Sequences g * group_size .. (g+1) * group_size - 1 form group g.
 * Sequence s of group g attends over the prefix_lens[g] tokens of
 * prefix_block_table[g] followed by the suffix_lens[s] tokens of
 * suffix_block_table[s]:
 *   out[s,h] = paged_attn_decode of s with the block table
 *              prefix_block_table[g][0 .. prefix_lens[g]/block_size) ++ suffix_block_table[s]
 *              and seq_len prefix_lens[g] + suffix_lens[s]
 * (prefix_lens[g] a multiple of block_size: a partly filled shared block is
 * copied on write before a sample writes to it). Computed as a multi-query
 * pass over each group's prefix (the group's samples are its query rows) and
 * a decode pass over each suffix, in one launch (the suffixes' items follow
 * the prefixes' as workgroups run out of them; two launches when the batch
 * exceeds one launch's work list), then a merge of the two by their
 * log-sum-exp.
 *
 *   out, query             [num_groups * group_size, num_heads, head_dim]
 *   prefix_block_table     int32 [num_groups, max_prefix_blocks]; prefix_lens int32 [num_groups]
 *   suffix_block_table     int32 [num_groups * group_size, max_suffix_blocks];
 *                          suffix_lens int32 [num_groups * group_size]
 *   max_prefix_len, max_suffix_len  host bounds of the lengths
 *   group_size * (num_heads / num_kv_heads) <= 128
 *   kv_dtype               PKV_F32, PKV_F16 or PKV_BF16 (query of the same type)
 *   workspace              paged_attn_shared_prefix_workspace_size(...) bytes
 * Status codes as for paged_attn_decode.
 */
int paged_attn_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* prefix_block_table,
                                    const int32_t* prefix_lens, int num_groups, int group_size,
                                    int max_prefix_blocks, int max_prefix_len,
                                    const int32_t* suffix_block_table, const int32_t* suffix_lens,
                                    int max_suffix_blocks, int max_suffix_len, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                    float scale, int kv_dtype, int out_dtype, int partition_size,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attn_decode_shared_prefix_fp8 - paged_attn_decode_shared_prefix over
 * e4m3 pools (reshape_and_cache_fp8's format: a code stands for code *
 * k_scale[kv head] in key_cache, code * v_scale[kv head] in value_cache;
 * "LLM inference optimisation in practice", section 6.2, and the groups'
 * sharing as above). query and out as for paged_attn_decode_fp8: query of
 * query_dtype PKV_F16 or PKV_BF16, out of the query's type or PKV_F32.
 * k_scale, v_scale: fp32 [num_kv_heads] device arrays (NULL: PKV_ERR_NULL).
 * Workspace: the size that
 * paged_attn_shared_prefix_workspace_size gives for the same arguments.
 */
int paged_attn_decode_shared_prefix_fp8(void* out, const void* query, const void* key_cache,
                                        const void* value_cache, const float* k_scale,
                                        const float* v_scale, const int32_t* prefix_block_table,
                                        const int32_t* prefix_lens, int num_groups, int group_size,
                                        int max_prefix_blocks, int max_prefix_len,
                                        const int32_t* suffix_block_table, const int32_t* suffix_lens,
                                        int max_suffix_blocks, int max_suffix_len, int num_heads,
                                        int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                        float scale, int query_dtype, int out_dtype, int partition_size,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attn_shared_prefix_workspace_size - bytes of workspace that
 * paged_attn_decode_shared_prefix needs: the control areas of its two passes
 * first, then their fp32 outputs and log-sum-exps and their split-K
 * partials. As for paged_attn_decode, the control area must be zero before
 * the workspace's first use and every call leaves it zero again: it is the
 * first C_pre + C_suf bytes, where C_pre is the control area (as
 * paged_attn_decode states it) of num_groups sequences of at most
 * max_prefix_len tokens and C_suf that of num_groups * group_size sequences
 * of at most max_suffix_len tokens, each split as paged_attn_partition_tokens
 * gives for its own arguments. 0 when the arguments are invalid.
 */
size_t paged_attn_shared_prefix_workspace_size(int num_groups, int group_size, int num_heads,
                                               int num_kv_heads, int head_dim, int block_size,
                                               int max_prefix_len, int max_suffix_len,
                                               int partition_size);

/*
 * paged_attn_partition_tokens - the partition length the attention entry
 * points use for these arguments (resolving partition_size = 0) over a pool
 * of kv_dtype with q_len new tokens per sequence (1 for decode), or a
 * negative pkv_status for invalid arguments. A value >= max_seq_len means no
 * split. The choice for 0 starts from a base B that depends on the query
 * rows per KV head, R = q_len * num_heads / num_kv_heads: for 16-bit and fp32
 * pools 1280 tokens (R <= 8) or 1024 (R <= 16); for PKV_E4M3 pools 2048
 * (R <= 16); above 16 rows 1280 for every pool. Then: no split when there
 * are at least 2048 (sequence, KV head) pairs and max_seq_len <= 4096; else
 * B while that makes at most 4096 (sequence, KV head, partition) units; else
 * 2 B. The workspace sizes are those of the shortest choice (16-bit pools),
 * which serve every dtype.
 */
int paged_attn_partition_tokens(int num_seqs, int q_len, int num_heads, int num_kv_heads,
                                int block_size, int max_seq_len, int partition_size,
                                int kv_dtype);

/*
 * paged_attn_workspace_size - bytes of workspace paged_attn_decode needs for
 * these arguments: the control area (a 256-byte header and, when sequences
 * are split, a 32-bit arrival count per (sequence, KV head), padded to 256
 * bytes) and, when split, fp32 (max, sum) pairs and head_dim weighted-V
 * partial sums per (sequence, head, partition), for min(num_seqs, 2048)
 * sequences (larger batches run as several launches of at most 2048
 * sequences that reuse them). 0 when the arguments are invalid or num_seqs
 * is 0.
 */
size_t paged_attn_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                 int head_dim, int block_size, int max_seq_len,
                                 int partition_size);

/*
 * reshape_and_cache - write the K and V of each new token into its slot of
 * the pools. slot_mapping[i] = physical_block * block_size + offset, the slot
 * the block engine hands out for the token ("LLM inference engine
 * internals" section 2.3, append_slot; growth as in "vLLM core concepts"
 * section 4.2.2). key_cache[slot / block_size, slot % block_size] = key[i],
 * and the same for value, as bit copies. slot < 0 means "no slot": the token
 * is skipped. Slots must be distinct (else which write lands is
 * unspecified); slots >= num_blocks*block_size are skipped.
 *
 *   key, value        [num_tokens, num_kv_heads, head_dim], dtype
 *   key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim]
 *   slot_mapping      int64 [num_tokens]
 */
int reshape_and_cache(const void* key, const void* value, void* key_cache,
                      void* value_cache, const int64_t* slot_mapping,
                      int num_tokens, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int dtype,
                      hipStream_t stream);

/*
 * reshape_and_cache_fp8 - reshape_and_cache into e4m3 pools, quantising:
 * element d of KV head j of token i is stored as the e4m3 code of
 * key[i][j][d] / k_scale[j] (the quotient formed in fp32, then rounded to
 * the nearest e4m3 value, ties to the even code; magnitudes of 448 and more
 * saturate to 448; NaN stays NaN), and likewise for value with v_scale.
 * Slots as for reshape_and_cache. The scales are the caller's (for example
 * calibrated per layer and KV head) and the same ones go to the attention.
 *
 *   key, value              [num_tokens, num_kv_heads, head_dim] of src_dtype
 *                           (PKV_F32, PKV_F16 or PKV_BF16)
 *   key_cache, value_cache  uint8 [num_blocks, block_size, num_kv_heads, head_dim]
 *   k_scale, v_scale        fp32 [num_kv_heads], device memory
 */
int reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                          void* value_cache, const int64_t* slot_mapping, const float* k_scale,
                          const float* v_scale, int num_tokens, int num_kv_heads, int head_dim,
                          int block_size, int num_blocks, int src_dtype, hipStream_t stream);

/*
 * swap_blocks - preemption by swapping ("LLM inference engine internals"
 * sections 3.1-3.2: the scheduler's blocks_to_swap_out and
 * blocks_to_swap_in; the CPU swap space of "vLLM core concepts" section
 * 4.2.4): for each pair (src, dst) of block_mapping, block src of the source
 * pools (K and V) is copied to block dst of the destination pools. Swapping
 * out goes from the GPU pools to pools in pinned host memory, swapping in
 * back to any free GPU blocks (the caller then points the block table at
 * them). One kernel launch moves every pair, reading or writing host memory
 * across the host link.
 *
 *   src_*, dst_*     [src_num_blocks | dst_num_blocks, block_size, num_kv_heads,
 *                    head_dim] of dtype; each either device memory or pinned
 *                    host memory (hipHostMalloc, a torch pin_memory tensor);
 *                    pageable host memory is refused with PKV_ERR_UNSUPPORTED
 *   block_mapping    int64 [num_pairs, 2] (src, dst), device or pinned memory
 * Pairs outside either pool are skipped; destination blocks must be distinct
 * and, when both pools are the same memory, disjoint from the sources.
 */
int swap_blocks(const void* src_key_cache, const void* src_value_cache, void* dst_key_cache,
                void* dst_value_cache, const int64_t* block_mapping, int num_pairs,
                int src_num_blocks, int dst_num_blocks, int block_size, int num_kv_heads,
                int head_dim, int dtype, hipStream_t stream);

/*
 * copy_blocks - copy-on-write block copies: for each pair (src, dst) of
 * block_mapping, the whole physical block src of both pools (every slot, every
 * KV head) is copied to block dst. A block shared by several sequences is
 * copied before one of them modifies it ("vLLM core concepts" section 4.2.2;
 * "LLM inference engine internals" sections 3.1 (blocks_to_copy) and 3.3;
 * "PagedAttention principle" section 5). The destinations must be distinct
 * and disjoint from every source (then the result equals reading every
 * source before writing any destination). Pairs with an id outside
 * [0, num_blocks) are skipped.
 *
 *   block_mapping  int64 [num_pairs, 2], row = (src, dst)
 */
int copy_blocks(void* key_cache, void* value_cache,
                const int64_t* block_mapping, int num_pairs, int num_blocks,
                int block_size, int num_kv_heads, int head_dim, int dtype,
                hipStream_t stream);

/*
 * pagedkv_check_decode_inputs - the contract check that the fast path does
 * not make. Counts, on the device, the block-table entries of used logical
 * blocks outside [0, num_blocks) and the seq_lens outside [0, max_seq_len];
 * writes the two counts to counts[0] and counts[1] (device int32[2], cleared
 * by the call). Asynchronous like the others; read counts after the stream
 * has finished.
 */
int pagedkv_check_decode_inputs(const int32_t* block_table,
                                const int32_t* seq_lens, int num_seqs,
                                int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_seq_len,
                                int32_t* counts, hipStream_t stream);

/*
 * pagedkv_check_cache_op_inputs - the contract check of reshape_and_cache's
 * slot_mapping and copy_blocks' block_mapping that those calls do not make.
 * Slots come from the block engine's append_slot, which hands out each slot
 * once ("LLM inference engine internals" section 2.3), and the scheduler's
 * blocks_to_copy names fresh destination blocks (the same page, section
 * 3.1). Counts on the device, into counts (device int32[4], cleared by the
 * call):
 *   counts[0]  slots >= num_blocks * block_size (negative slots are
 *              "no slot" and not counted)
 *   counts[1]  slots inside the pool that repeat an earlier token's slot
 *   counts[2]  pairs with a source or destination outside [0, num_blocks)
 *   counts[3]  pairs (ids in range) whose destination is the source of any
 *              pair (its own included) or the destination of an earlier pair
 * Either list may be empty (num_tokens or num_pairs 0, its pointer then may
 * be NULL). Cost grows with the square of each list's length (it is meant
 * for checked runs, not the fast path). Asynchronous like the others; read
 * counts after the stream has finished.
 */
int pagedkv_check_cache_op_inputs(const int64_t* slot_mapping, int num_tokens, int block_size,
                                  int num_blocks, const int64_t* block_mapping, int num_pairs,
                                  int32_t* counts, hipStream_t stream);

/*
 * pagedkv_stream_read - measurement aid, not part of the decode path: reads
 * `bytes` (a multiple of 16) from device buffer `src` once with 16-byte loads
 * per lane, 4 loads in flight per lane, `grid` workgroups of 256 threads in
 * a grid-stride loop, and writes one XOR fold per workgroup to sink[0 ..
 * grid) (device uint32, so the loads cannot be dropped). Timed on a buffer
 * much larger than the caches it gives the streaming-read rate the device
 * reaches, which the decode call's bandwidth is compared with (the pages
 * call decode memory-bound: "LLM inference optimisation in practice",
 * arithmetic-intensity section). bytes = 0 is a no-op; grid must be > 0.
 */
int pagedkv_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                        hipStream_t stream);

/*
 * paged_attn_timed - measurement aid: the attention of paged_attn_decode
 * (q_len 1, kv_dtype PKV_F32/F16/BF16, query of the KV dtype, no scales),
 * paged_attn_multi_query (q_len > 1), paged_attn_decode_fp8 or
 * paged_attn_multi_query_fp8 (kv_dtype PKV_E4M3 with k_scale, v_scale and a
 * query_dtype of PKV_F16 or PKV_BF16), with the same arguments, checks and
 * results as those calls, and two HIP events that the caller created
 * (hipEventCreate): start is set to the start of the call's first kernel
 * launch and stop to the end of its last one, by the launches themselves
 * (hipExtLaunchKernel), so that hipEventElapsedTime(start, stop) is the
 * kernels' own time, without the dispatch latency of separately recorded
 * events. k_scale / v_scale may be NULL for the 16-bit dtypes.
 * Returns PKV_ERR_NULL when an event is NULL; with num_seqs = 0 nothing is
 * launched and the events are left as they are.
 */
int paged_attn_timed(void* out, const void* query, const void* key_cache, const void* value_cache,
                     const float* k_scale, const float* v_scale, const int32_t* block_table,
                     const int32_t* seq_lens, int num_seqs, int q_len, int num_heads,
                     int num_kv_heads, int head_dim, int block_size, int num_blocks,
                     int max_blocks_per_seq, int max_seq_len, float scale, int kv_dtype,
                     int query_dtype, int out_dtype, int partition_size, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

/*
 * paged_attn_decode_noalloc - paged_attn_decode without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * caller still passes every input and output; the workspace is a static
 * device array of PKV_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one
 * per GPU, held until the process ends. Nothing is allocated by the call.
 * Its first call on a device looks up the array's address
 * (hipGetSymbolAddress) and clears it with a kernel on `stream`; every call
 * leaves its control area zero again, as for paged_attn_decode.
 * Arguments, layout, results and status codes are those of
 * paged_attn_decode, plus PKV_ERR_WORKSPACE (nothing launched) when the call
 * needs more workspace than the array holds (paged_attn_workspace_size(...) >
 * PKV_NOALLOC_SCRATCH_BYTES: e.g. 256 sequences of up to 10 000 tokens at 32
 * query heads split into 512-token partitions; the library's own partition
 * choice keeps the page-shaped batches within it) and PKV_ERR_HIP when the
 * runtime refuses the address lookup. Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (different streams, other
 * threads) race and must be serialised by the caller; calls in order on one
 * stream, and replays of a graph that captured a call, are fine.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int paged_attn_decode_noalloc(void* out, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_table,
                              const int32_t* seq_lens, int num_seqs, int num_heads,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              int max_blocks_per_seq, int max_seq_len, float scale, int kv_dtype,
                              int out_dtype, int partition_size, hipStream_t stream);

/* pagedkv_status_string - a static, NUL-terminated name for a status code. */
const char* pagedkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
