// C-ABI entry points (declared in include/pagedkv.h): host-side argument
// checks, partition and workspace sizing, dispatch to the kernels. Nothing
// here allocates, synchronises or keeps state.

#include <math.h>
#include <stdint.h>

#include "pagedkv.h"
#include "pagedkv_internal.h"
#include "stream_read.h"
#include "shared_prefix.h"
#include "swap_blocks.h"

namespace {

int elem_bytes(int dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16:
    case PKV_BF16: return 2;
    case PKV_E4M3: return 1;
    default: return 0;
  }
}

bool supported_block_size(int bs) { return bs == 8 || bs == 16 || bs == 32; }

bool supported_head_dim(int d) { return d == 64 || d == 128; }

// Rows and quads of rows move in 16-byte vector accesses.
bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

// The address a kernel uses for ptr: device (or managed) memory as it is,
// pinned host memory through its device mapping; nullptr for memory the
// device cannot reach (pageable host memory), which must never reach a
// kernel. Clears the error a failed query leaves behind.
void* device_view(const void* ptr) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  switch (a.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged: return const_cast<void*>(ptr);
    case hipMemoryTypeHost: return a.devicePointer;
    default: return nullptr;
  }
}

// Query rows (q_len x group) one KV head's workgroup takes: a tile of 16 MFMA
// columns per wave.
constexpr int kMaxQueryRows = 16 * pkv::kWaves;

// Partition length chosen when partition_size is 0. A workgroup (8 waves)
// handles one (sequence, KV head, partition); 512 fit on the GPU at once (256
// CUs, 2 each). A base of B tokens: for 16-bit and fp32 pools 1280 (1024
// with 9 to 16 query rows per KV head), for e4m3 pools (half the bytes per
// token) 2048; with more than 16 query rows per KV head (column groups
// sharing each tile through LDS) 1280 for every pool.
// Measured on MI355X: with >= 2048 (sequence, KV head) pairs and
// sequences of at most 4096 tokens, not splitting is best; otherwise B-token
// partitions while that gives at most 4096 (sequence, KV head, partition)
// units, else 2 B (fewer partials to write and merge).
int auto_partition(int num_seqs, int num_kv_heads, int block_size, int max_seq_len, int kv_elem_bytes,
                   int rows) {
  const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
  const int unit = block_size > pkv::kTile ? block_size : pkv::kTile;
  int base = kv_elem_bytes == 1 ? 2048 : (rows > 8 ? 1024 : 1280);
  if (rows > 16) base = 1280;
  if (pairs >= 2048 && max_seq_len <= 4096) {
    const int P = (max_seq_len + unit - 1) / unit * unit;
    return P > 0 ? P : unit;
  }
  if (pairs * ((max_seq_len + base - 1) / base) <= 4096) return base;
  return 2 * base;
}

// Partition length for these arguments (> 0), or a negative status.
// kv_elem_bytes and rows (query rows per KV head) only steer the choice for
// partition_size 0; the workspace sizes take 2 bytes, the shortest choice.
int resolve_partition(int num_seqs, int num_kv_heads, int block_size, int max_seq_len,
                      int partition_size, int kv_elem_bytes, int rows) {
  if (partition_size < 0) return PKV_ERR_SHAPE;
  if (!supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  const int P = partition_size == 0
                    ? auto_partition(num_seqs, num_kv_heads, block_size, max_seq_len, kv_elem_bytes, rows)
                    : partition_size;
  if (P % pkv::kTile != 0 || P % block_size != 0) return PKV_ERR_SHAPE;
  if (P >= max_seq_len) {
    // one partition per sequence: its block-table slice must fit in LDS
    if (max_seq_len > pkv::kMaxPartition) return PKV_ERR_UNSUPPORTED;
  } else if (P > pkv::kMaxPartition) {
    return PKV_ERR_UNSUPPORTED;
  }
  return P;
}

// Partitions for these arguments: `partition` tokens (when one covers
// max_seq_len, the shortest multiple of the tile and block size that does)
// and `np` partitions per sequence at most.
struct Cutting {
  int partition, np;
};

Cutting cutting_for(int max_seq_len, int block_size, int P) {
  Cutting c;
  const int unit = block_size > pkv::kTile ? block_size : pkv::kTile;
  if (P >= max_seq_len) P = max_seq_len > 0 ? (max_seq_len + unit - 1) / unit * unit : unit;
  c.partition = P;
  c.np = max_seq_len > P ? (max_seq_len + P - 1) / P : 1;
  return c;
}

// Workspace layout: the control area, then the split-K partials.
//   * control area (zero before the first use; every call leaves it zero
//     again): a 256-byte header whose first 64-bit word is the partition
//     kernel's control word (item counter and finished workgroups), then,
//     when sequences are split, one 32-bit arrival count per (sequence, KV
//     head) [S', Hkv], padded to a multiple of 256 bytes;
//   * partials (any contents; garbage after a call), when split: fp32 O
//     [S', q_len, H, NP, D] (the D values of one partial in the kernel's own
//     order) and (m, l) pairs [S', q_len, H, NP, 2];
// for S' = min(S, the sequences of one launch); launches run in order and
// reuse them.
constexpr size_t kHeaderBytes = 256;

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

int launch_seqs(int num_seqs) { return num_seqs < pkv::kMaxSeqsPerLaunch ? num_seqs : pkv::kMaxSeqsPerLaunch; }

size_t control_bytes_for(int num_seqs, int num_kv_heads, int np) {
  if (np <= 1) return kHeaderBytes;
  return kHeaderBytes + round256((size_t)launch_seqs(num_seqs) * num_kv_heads * sizeof(uint32_t));
}

size_t workspace_bytes_for(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int np) {
  const size_t ctl = control_bytes_for(num_seqs, num_kv_heads, np);
  if (np <= 1) return ctl;
  return ctl + (size_t)launch_seqs(num_seqs) * num_heads * np * (size_t)(head_dim + 2) * sizeof(float);
}

}  // namespace

extern "C" {

int paged_attn_partition_tokens(int num_seqs, int q_len, int num_heads, int num_kv_heads, int block_size,
                                int max_seq_len, int partition_size, int kv_dtype) {
  if (num_seqs < 0 || q_len < 1 || num_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0 ||
      num_heads % num_kv_heads != 0)
    return PKV_ERR_SHAPE;
  if (elem_bytes(kv_dtype) == 0) return PKV_ERR_UNSUPPORTED;
  return resolve_partition(num_seqs, num_kv_heads, block_size, max_seq_len, partition_size,
                           elem_bytes(kv_dtype), q_len * (num_heads / num_kv_heads));
}

}  // extern "C"

namespace {

// Every attention entry point: q_len new tokens per sequence (1 for decode),
// query and out [num_seqs, q_len, num_heads, head_dim]. The query has
// query_dtype: the KV dtype, or fp16/bf16 over an e4m3 pool (which takes a
// K and a V scale per KV head). With `prepared`, the checked launch
// parameters are stored there and nothing is launched.
int attention(void* out, const void* query, const void* key_cache, const void* value_cache,
              const float* k_scale, const float* v_scale, const int32_t* block_table,
              const int32_t* seq_lens, int num_seqs, int q_len, int num_heads, int num_kv_heads,
              int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
              int max_seq_len, float scale, int kv_dtype, int query_dtype, int out_dtype,
              int partition_size, void* workspace, size_t workspace_bytes, hipStream_t stream,
              float* lse = nullptr, int causal = 1, pkv::DecodeParams* prepared = nullptr,
              hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr, void* partials = nullptr) {
  if (num_seqs < 0 || q_len < 1) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !key_cache || !value_cache || !block_table || !seq_lens)
    return PKV_ERR_NULL;
  const bool f8 = kv_dtype == PKV_E4M3;
  if (f8 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  const int group = num_heads / num_kv_heads;
  // the q_len * group query rows of a KV head: at most one 16-column MFMA tile
  // per wave of a workgroup
  if (group > 16 || q_len > kMaxQueryRows || q_len * group > kMaxQueryRows) return PKV_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  if (elem_bytes(kv_dtype) == 0) return PKV_ERR_UNSUPPORTED;
  if (f8 ? (query_dtype != PKV_F16 && query_dtype != PKV_BF16) : query_dtype != kv_dtype)
    return PKV_ERR_UNSUPPORTED;
  if (out_dtype != query_dtype && out_dtype != PKV_F32) return PKV_ERR_UNSUPPORTED;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return PKV_ERR_SHAPE;
  if ((int64_t)num_blocks * block_size > (int64_t)INT32_MAX) return PKV_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  const int P = resolve_partition(num_seqs, num_kv_heads, block_size, max_seq_len, partition_size,
                                  elem_bytes(kv_dtype), q_len * group);
  if (P < 0) return P;
  const Cutting cut = cutting_for(max_seq_len, block_size, P);
  const int np = cut.np;
  // the items of one launch and its item counter (which overshoots by up to
  // the grid) stay in int32
  const int s_launch = launch_seqs(num_seqs);
  if ((int64_t)s_launch * num_kv_heads * np > (int64_t)INT32_MAX - (1 << 24)) return PKV_ERR_SHAPE;
  // with `partials` (shared-prefix decode) the workspace is the control area
  // alone and the partials are elsewhere
  const size_t ctl = control_bytes_for(num_seqs, num_kv_heads, np);
  const size_t need = partials ? ctl : workspace_bytes_for(num_seqs, q_len * num_heads, num_kv_heads, head_dim, np);
  if (workspace == nullptr || workspace_bytes < need) return PKV_ERR_WORKSPACE;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned16(workspace) || (partials && !aligned16(partials)))
    return PKV_ERR_SHAPE;

  pkv::DecodeParams p{};
  p.out = out;
  p.q = query;
  p.k = key_cache;
  p.v = value_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  p.work = reinterpret_cast<unsigned long long*>(ws);
  if (np > 1) {
    const int s = launch_seqs(num_seqs);
    p.arrive = reinterpret_cast<uint32_t*>(ws + kHeaderBytes);
    p.ws_o = reinterpret_cast<float*>(partials ? static_cast<unsigned char*>(partials) : ws + ctl);
    p.ws_ml = p.ws_o + (size_t)s * q_len * num_heads * np * head_dim;
  }
  p.num_seqs = num_seqs;
  p.q_len = q_len;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.num_blocks = num_blocks;
  p.max_blocks = max_blocks_per_seq;
  p.max_seq_len = max_seq_len;
  p.partition = cut.partition;
  p.num_partitions = np;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.out_f32 = out_dtype == PKV_F32 ? 1 : 0;
  p.causal = causal;
  p.lse = lse;
  if (prepared) {
    *prepared = p;
    return PKV_OK;
  }
  const hipError_t e = pkv::launch_decode(p, kv_dtype, query_dtype, head_dim, block_size, stream, ev_start,
                                          ev_stop);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// Bytes of the control area and of the partials of a decode / multi-query
// workspace for these arguments; both 0 when the arguments are invalid.
struct WorkspaceParts {
  size_t ctl, partials;
  size_t total() const { return ctl + partials; }
};

WorkspaceParts workspace_parts(int num_seqs, int q_len, int num_heads, int num_kv_heads, int head_dim,
                               int block_size, int max_seq_len, int partition_size) {
  WorkspaceParts w{0, 0};
  if (num_seqs <= 0 || q_len < 1 || num_heads <= 0 || num_kv_heads <= 0 || max_seq_len < 0) return w;
  if (num_heads % num_kv_heads != 0 || q_len > kMaxQueryRows ||
      q_len * (num_heads / num_kv_heads) > kMaxQueryRows)
    return w;
  if (!supported_head_dim(head_dim)) return w;
  // the shortest partition any pool dtype gets (2-byte elements): the most
  // partials, so the size serves every dtype
  const int P = resolve_partition(num_seqs, num_kv_heads, block_size, max_seq_len, partition_size, 2,
                                  q_len * (num_heads / num_kv_heads));
  if (P < 0) return w;
  const int np = cutting_for(max_seq_len, block_size, P).np;
  w.ctl = control_bytes_for(num_seqs, num_kv_heads, np);
  w.partials = workspace_bytes_for(num_seqs, q_len * num_heads, num_kv_heads, head_dim, np) - w.ctl;
  return w;
}

size_t workspace_size(int num_seqs, int q_len, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int max_seq_len, int partition_size) {
  return workspace_parts(num_seqs, q_len, num_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                         partition_size)
      .total();
}

// Shared-prefix decode workspace: the control areas of the prefix pass and of
// the suffix pass first (together the area that must be zero at first use),
// then the two passes' fp32 outputs and lse rows, then the prefix pass's
// partials and the suffix pass's (both passes run in one launch); every area
// 256-byte aligned.
struct PrefixLayout {
  size_t ctl_pre, ctl_suf, o_bytes, lse_bytes, part_pre, part_suf;
  size_t control() const { return ctl_pre + ctl_suf; }
  size_t total() const { return control() + 2 * o_bytes + 2 * lse_bytes + part_pre + part_suf; }
};
PrefixLayout prefix_layout(int num_groups, int group_size, int num_heads, int num_kv_heads,
                           int head_dim, int block_size, int max_prefix_len, int max_suffix_len,
                           int partition_size) {
  PrefixLayout l{0, 0, 0, 0, 0, 0};
  const int64_t rows = (int64_t)num_groups * group_size * num_heads;
  const WorkspaceParts a = workspace_parts(num_groups, group_size, num_heads, num_kv_heads, head_dim, block_size,
                                           max_prefix_len, partition_size);
  const WorkspaceParts b = workspace_parts(num_groups * group_size, 1, num_heads, num_kv_heads, head_dim,
                                           block_size, max_suffix_len, partition_size);
  if (a.ctl == 0 || b.ctl == 0) return l;
  l.ctl_pre = a.ctl;  // multiples of 256
  l.ctl_suf = b.ctl;
  l.o_bytes = round256((size_t)rows * head_dim * sizeof(float));
  l.lse_bytes = round256((size_t)rows * sizeof(float));
  l.part_pre = round256(a.partials);
  l.part_suf = b.partials;
  return l;
}

}  // namespace

extern "C" {

size_t paged_attn_shared_prefix_workspace_size(int num_groups, int group_size, int num_heads,
                                               int num_kv_heads, int head_dim, int block_size,
                                               int max_prefix_len, int max_suffix_len,
                                               int partition_size) {
  if (num_groups <= 0 || group_size <= 0 || (int64_t)num_groups * group_size > INT32_MAX / 2) return 0;
  return prefix_layout(num_groups, group_size, num_heads, num_kv_heads, head_dim, block_size,
                       max_prefix_len, max_suffix_len, partition_size)
      .total();
}

}  // extern "C"

namespace {

// Shared-prefix decode over a 16-bit or fp32 pool (query of the KV dtype, no
// scales) or an e4m3 pool (k_scale, v_scale; query_dtype fp16 or bf16).
int shared_prefix(void* out, const void* query, const void* key_cache, const void* value_cache,
                  const float* k_scale, const float* v_scale, const int32_t* prefix_block_table,
                  const int32_t* prefix_lens, int num_groups, int group_size, int max_prefix_blocks,
                  int max_prefix_len, const int32_t* suffix_block_table, const int32_t* suffix_lens,
                  int max_suffix_blocks, int max_suffix_len, int num_heads, int num_kv_heads,
                  int head_dim, int block_size, int num_blocks, float scale, int kv_dtype,
                  int query_dtype, int out_dtype, int partition_size, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  if (num_groups < 0 || group_size < 1) return PKV_ERR_SHAPE;
  if (num_groups == 0) return PKV_OK;
  if ((int64_t)num_groups * group_size > INT32_MAX / 2) return PKV_ERR_SHAPE;
  if (!out || !query || !key_cache || !value_cache || !prefix_block_table || !prefix_lens ||
      !suffix_block_table || !suffix_lens)
    return PKV_ERR_NULL;
  if (kv_dtype == PKV_E4M3 && (!k_scale || !v_scale)) return PKV_ERR_NULL;
  if (kv_dtype == PKV_E4M3 ? (query_dtype != PKV_F16 && query_dtype != PKV_BF16) : query_dtype != kv_dtype)
    return PKV_ERR_UNSUPPORTED;
  if (out_dtype != query_dtype && out_dtype != PKV_F32) return PKV_ERR_UNSUPPORTED;
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  const PrefixLayout l = prefix_layout(num_groups, group_size, num_heads, num_kv_heads, head_dim,
                                       block_size, max_prefix_len, max_suffix_len, partition_size);
  if (l.total() == 0) {
    // the passes' own checks name what is wrong (group too large, sizes, partition)
    const int st = attention(out, query, key_cache, value_cache, k_scale, v_scale, prefix_block_table,
                             prefix_lens, num_groups, group_size, num_heads, num_kv_heads, head_dim,
                             block_size, num_blocks, max_prefix_blocks, max_prefix_len, scale, kv_dtype,
                             query_dtype, PKV_F32, partition_size, nullptr, 0, stream, nullptr, 0);
    return st != PKV_OK && st != PKV_ERR_WORKSPACE ? st : PKV_ERR_SHAPE;
  }
  if (!workspace || workspace_bytes < l.total()) return PKV_ERR_WORKSPACE;
  if (!aligned16(out) || !aligned16(workspace)) return PKV_ERR_SHAPE;
  unsigned char* w = static_cast<unsigned char*>(workspace);
  void* ctl_pre = w;
  void* ctl_suf = w + l.ctl_pre;
  unsigned char* o0 = w + l.control();
  float* o_pre = reinterpret_cast<float*>(o0);
  float* o_suf = reinterpret_cast<float*>(o0 + l.o_bytes);
  float* lse_pre = reinterpret_cast<float*>(o0 + 2 * l.o_bytes);
  float* lse_suf = reinterpret_cast<float*>(o0 + 2 * l.o_bytes + l.lse_bytes);
  void* part_pre = o0 + 2 * l.o_bytes + 2 * l.lse_bytes;
  void* part_suf = static_cast<unsigned char*>(part_pre) + l.part_pre;
  const int num_seqs = num_groups * group_size;
  // the prefix once per group: the group's samples are its query rows
  // ([num_seqs, H, D] read as [num_groups, group_size, H, D]), all of them
  // seeing the whole prefix
  pkv::DecodeParams pre{}, suf{};
  int st = attention(o_pre, query, key_cache, value_cache, k_scale, v_scale, prefix_block_table, prefix_lens,
                     num_groups, group_size, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                     max_prefix_blocks, max_prefix_len, scale, kv_dtype, query_dtype, PKV_F32,
                     partition_size, ctl_pre, l.ctl_pre, stream, lse_pre, 0, &pre, nullptr, nullptr,
                     part_pre);
  if (st != PKV_OK) return st;
  // each sample's own suffix
  st = attention(o_suf, query, key_cache, value_cache, k_scale, v_scale, suffix_block_table, suffix_lens,
                 num_seqs, 1, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_suffix_blocks,
                 max_suffix_len, scale, kv_dtype, query_dtype, PKV_F32, partition_size, ctl_suf,
                 l.ctl_suf, stream, lse_suf, 1, &suf, nullptr, nullptr, part_suf);
  if (st != PKV_OK) return st;
  // both passes in one launch, the suffixes filling the prefix pass's
  // ramp-down; one after the other when they do not fit one launch
  hipError_t e = pkv::launch_decode_pair(pre, suf, kv_dtype, query_dtype, head_dim, block_size, stream);
  if (e == hipErrorNotSupported) {
    (void)hipGetLastError();
    e = pkv::launch_decode(pre, kv_dtype, query_dtype, head_dim, block_size, stream);
    if (e == hipSuccess) e = pkv::launch_decode(suf, kv_dtype, query_dtype, head_dim, block_size, stream);
  }
  if (e != hipSuccess) return PKV_ERR_HIP;
  e = pkv::launch_cascade_merge(out, o_pre, lse_pre, o_suf, lse_suf, (int64_t)num_seqs * num_heads, head_dim,
                                out_dtype, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

extern "C" {

int paged_attn_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                                    const void* value_cache, const int32_t* prefix_block_table,
                                    const int32_t* prefix_lens, int num_groups, int group_size,
                                    int max_prefix_blocks, int max_prefix_len,
                                    const int32_t* suffix_block_table, const int32_t* suffix_lens,
                                    int max_suffix_blocks, int max_suffix_len, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                    float scale, int kv_dtype, int out_dtype, int partition_size,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (kv_dtype == PKV_E4M3) return PKV_ERR_UNSUPPORTED;  // needs the scales: the _fp8 entry point
  return shared_prefix(out, query, key_cache, value_cache, nullptr, nullptr, prefix_block_table, prefix_lens,
                       num_groups, group_size, max_prefix_blocks, max_prefix_len, suffix_block_table,
                       suffix_lens, max_suffix_blocks, max_suffix_len, num_heads, num_kv_heads, head_dim,
                       block_size, num_blocks, scale, kv_dtype, kv_dtype, out_dtype, partition_size,
                       workspace, workspace_bytes, stream);
}

int paged_attn_decode_shared_prefix_fp8(void* out, const void* query, const void* key_cache,
                                        const void* value_cache, const float* k_scale,
                                        const float* v_scale, const int32_t* prefix_block_table,
                                        const int32_t* prefix_lens, int num_groups, int group_size,
                                        int max_prefix_blocks, int max_prefix_len,
                                        const int32_t* suffix_block_table, const int32_t* suffix_lens,
                                        int max_suffix_blocks, int max_suffix_len, int num_heads,
                                        int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                        float scale, int query_dtype, int out_dtype, int partition_size,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return shared_prefix(out, query, key_cache, value_cache, k_scale, v_scale, prefix_block_table, prefix_lens,
                       num_groups, group_size, max_prefix_blocks, max_prefix_len, suffix_block_table,
                       suffix_lens, max_suffix_blocks, max_suffix_len, num_heads, num_kv_heads, head_dim,
                       block_size, num_blocks, scale, PKV_E4M3, query_dtype, out_dtype, partition_size,
                       workspace, workspace_bytes, stream);
}

size_t paged_attn_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                 int block_size, int max_seq_len, int partition_size) {
  return workspace_size(num_seqs, 1, num_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                        partition_size);
}

size_t paged_attn_multi_query_workspace_size(int num_seqs, int q_len, int num_heads, int num_kv_heads,
                                             int head_dim, int block_size, int max_seq_len,
                                             int partition_size) {
  return workspace_size(num_seqs, q_len, num_heads, num_kv_heads, head_dim, block_size, max_seq_len,
                        partition_size);
}

int paged_attn_timed(void* out, const void* query, const void* key_cache, const void* value_cache,
                     const float* k_scale, const float* v_scale, const int32_t* block_table,
                     const int32_t* seq_lens, int num_seqs, int q_len, int num_heads,
                     int num_kv_heads, int head_dim, int block_size, int num_blocks,
                     int max_blocks_per_seq, int max_seq_len, float scale, int kv_dtype,
                     int query_dtype, int out_dtype, int partition_size, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (!start || !stop) return PKV_ERR_NULL;
  if (kv_dtype != PKV_E4M3 && (k_scale || v_scale)) return PKV_ERR_UNSUPPORTED;  // scales are e4m3's
  return attention(out, query, key_cache, value_cache, k_scale, v_scale, block_table, seq_lens, num_seqs,
                   q_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                   max_seq_len, scale, kv_dtype, query_dtype, out_dtype, partition_size, workspace,
                   workspace_bytes, stream, nullptr, 1, nullptr, start, stop);
}

int paged_attn_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                      int kv_dtype, int out_dtype, int partition_size, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  if (kv_dtype == PKV_E4M3) return PKV_ERR_UNSUPPORTED;  // needs the scales: paged_attn_decode_fp8
  return attention(out, query, key_cache, value_cache, nullptr, nullptr, block_table, seq_lens, num_seqs,
                   1, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                   max_seq_len, scale, kv_dtype, kv_dtype, out_dtype, partition_size, workspace,
                   workspace_bytes, stream);
}

int paged_attn_multi_query(void* out, const void* query, const void* key_cache, const void* value_cache,
                           const int32_t* block_table, const int32_t* seq_lens, int num_seqs, int q_len,
                           int num_heads, int num_kv_heads, int head_dim, int block_size,
                           int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                           int kv_dtype, int out_dtype, int partition_size, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (kv_dtype == PKV_E4M3) return PKV_ERR_UNSUPPORTED;  // needs the scales: paged_attn_multi_query_fp8
  return attention(out, query, key_cache, value_cache, nullptr, nullptr, block_table, seq_lens, num_seqs,
                   q_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                   max_seq_len, scale, kv_dtype, kv_dtype, out_dtype, partition_size, workspace,
                   workspace_bytes, stream);
}

int paged_attn_decode_fp8(void* out, const void* query, const void* key_cache, const void* value_cache,
                          const float* k_scale, const float* v_scale, const int32_t* block_table,
                          const int32_t* seq_lens, int num_seqs, int num_heads, int num_kv_heads,
                          int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                          int max_seq_len, float scale, int query_dtype, int out_dtype,
                          int partition_size, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return attention(out, query, key_cache, value_cache, k_scale, v_scale, block_table, seq_lens, num_seqs,
                   1, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                   max_seq_len, scale, PKV_E4M3, query_dtype, out_dtype, partition_size, workspace,
                   workspace_bytes, stream);
}

int paged_attn_multi_query_fp8(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                               int q_len, int num_heads, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, int max_blocks_per_seq, int max_seq_len, float scale,
                               int query_dtype, int out_dtype, int partition_size, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return attention(out, query, key_cache, value_cache, k_scale, v_scale, block_table, seq_lens, num_seqs,
                   q_len, num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                   max_seq_len, scale, PKV_E4M3, query_dtype, out_dtype, partition_size, workspace,
                   workspace_bytes, stream);
}

int reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int dtype, hipStream_t stream) {
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return PKV_ERR_SHAPE;
  if (num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_UNSUPPORTED;
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * eb;
  if (row_bytes > INT32_MAX / 2) return PKV_ERR_SHAPE;
  const hipError_t e = pkv::launch_reshape_and_cache(
      key, value, key_cache, value_cache, slot_mapping, num_tokens, (int)row_bytes,
      (int64_t)num_blocks * block_size, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int reshape_and_cache_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int64_t* slot_mapping, const float* k_scale, const float* v_scale,
                          int num_tokens, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                          int src_dtype, hipStream_t stream) {
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping || !k_scale || !v_scale)
    return PKV_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return PKV_ERR_SHAPE;
  if (num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16 && src_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)num_kv_heads * head_dim > INT32_MAX / 8) return PKV_ERR_SHAPE;
  const hipError_t e = pkv::launch_reshape_and_cache_fp8(
      key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale, num_tokens, num_kv_heads,
      head_dim, src_dtype, (int64_t)num_blocks * block_size, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int swap_blocks(const void* src_key_cache, const void* src_value_cache, void* dst_key_cache,
                void* dst_value_cache, const int64_t* block_mapping, int num_pairs, int src_num_blocks,
                int dst_num_blocks, int block_size, int num_kv_heads, int head_dim, int dtype,
                hipStream_t stream) {
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache || !block_mapping)
    return PKV_ERR_NULL;
  if (!aligned16(src_key_cache) || !aligned16(src_value_cache) || !aligned16(dst_key_cache) ||
      !aligned16(dst_value_cache))
    return PKV_ERR_SHAPE;
  if (num_kv_heads <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_UNSUPPORTED;
  const void* sk = device_view(src_key_cache);
  const void* sv = device_view(src_value_cache);
  void* dk = device_view(dst_key_cache);
  void* dv = device_view(dst_value_cache);
  const void* bm = device_view(block_mapping);
  if (!sk || !sv || !dk || !dv || !bm) return PKV_ERR_UNSUPPORTED;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * eb;
  const hipError_t e = pkv::launch_swap_blocks(sk, sv, dk, dv, static_cast<const int64_t*>(bm), num_pairs,
                                               src_num_blocks, dst_num_blocks, block_bytes, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping, int num_pairs,
                int num_blocks, int block_size, int num_kv_heads, int head_dim, int dtype,
                hipStream_t stream) {
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!key_cache || !value_cache || !block_mapping) return PKV_ERR_NULL;
  if (!aligned16(key_cache) || !aligned16(value_cache)) return PKV_ERR_SHAPE;
  if (num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  const int eb = elem_bytes(dtype);
  if (eb == 0) return PKV_ERR_UNSUPPORTED;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * eb;
  const hipError_t e = pkv::launch_copy_blocks(key_cache, value_cache, block_mapping, num_pairs,
                                               num_blocks, block_bytes, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pagedkv_check_decode_inputs(const int32_t* block_table, const int32_t* seq_lens, int num_seqs,
                                int block_size, int num_blocks, int max_blocks_per_seq,
                                int max_seq_len, int32_t* counts, hipStream_t stream) {
  if (num_seqs < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0)
    return PKV_ERR_SHAPE;
  if (!counts) return PKV_ERR_NULL;
  if (num_seqs > 0 && (!block_table || !seq_lens)) return PKV_ERR_NULL;
  if (!supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  const hipError_t e = pkv::launch_check_decode_inputs(block_table, seq_lens, num_seqs, block_size,
                                                       num_blocks, max_blocks_per_seq, max_seq_len,
                                                       counts, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pagedkv_check_cache_op_inputs(const int64_t* slot_mapping, int num_tokens, int block_size,
                                  int num_blocks, const int64_t* block_mapping, int num_pairs,
                                  int32_t* counts, hipStream_t stream) {
  if (num_tokens < 0 || num_pairs < 0 || num_blocks <= 0) return PKV_ERR_SHAPE;
  if (!counts) return PKV_ERR_NULL;
  if ((num_tokens > 0 && !slot_mapping) || (num_pairs > 0 && !block_mapping)) return PKV_ERR_NULL;
  if (!supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  const hipError_t e = pkv::launch_check_cache_ops(slot_mapping, num_tokens, (int64_t)num_blocks * block_size,
                                                   block_mapping, num_pairs, num_blocks, counts, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pagedkv_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid,
                        hipStream_t stream) {
  if (grid < 0) return PKV_ERR_SHAPE;
  if (bytes == 0) return PKV_OK;
  if (!src || !sink) return PKV_ERR_NULL;
  if (bytes % 16 != 0 || grid == 0 || !aligned16(src)) return PKV_ERR_SHAPE;
  const hipError_t e = pkv::launch_stream_read(src, bytes, sink, grid, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

const char* pagedkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_NULL: return "PKV_ERR_NULL: a required pointer is NULL";
    case PKV_ERR_SHAPE: return "PKV_ERR_SHAPE: inconsistent or negative sizes, or a misaligned pointer";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED: dtype, head_dim, block_size or group size not built";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE: split-K workspace missing or too small";
    case PKV_ERR_HIP: return "PKV_ERR_HIP: the HIP runtime reported a launch error";
    default: return "unknown pagedkv status";
  }
}

}  // extern "C"
