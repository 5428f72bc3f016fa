// paged_attn_decode_noalloc: decode with the library's own static device
// scratch as the workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). The scratch is a file-scope __device__ array: every GPU the
// library runs on holds its own copy (kNoallocScratchBytes) until the
// process ends. Host code never passes the array's name to a kernel (in host
// code it is a stand-in, not a device address): its device address is taken
// once per device with hipGetSymbolAddress and kept.

#include <mutex>

#include "pagedkv.h"
#include "pagedkv_internal.h"

namespace pkv {
namespace {

constexpr size_t kNoallocScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocScratchBytes % 256 == 0, "scratch size must keep 256-byte areas aligned");

// Zero-filled when the code object is loaded (it has no initial contents);
// cleared once more by a kernel at each device's set-up below.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

__global__ __launch_bounds__(256) void zero_scratch_kernel(uint4* p, size_t n16) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) p[i] = z;
}

constexpr int kMaxDevices = 64;

// The scratch's device address on the current device, set up on the first
// call there: hipGetSymbolAddress with the device current, then a fill
// kernel on `stream` (not a memset, so that a captured first call records no
// memset node) puts the control area the decode kernels need at zero.
// PKV_OK, or PKV_ERR_HIP when the runtime refuses.
int scratch_on_current_device(hipStream_t stream, void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> g(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return PKV_ERR_HIP;
    }
    zero_scratch_kernel<<<dim3(1024), dim3(256), 0, stream>>>(static_cast<uint4*>(p), kNoallocScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attn_decode_noalloc(void* out, const void* query, const void* key_cache,
                                         const void* value_cache, const int32_t* block_table,
                                         const int32_t* seq_lens, int num_seqs, int num_heads,
                                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                         int max_blocks_per_seq, int max_seq_len, float scale, int kv_dtype,
                                         int out_dtype, int partition_size, hipStream_t stream) {
  if (num_seqs < 0) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  const size_t need = paged_attn_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                                max_seq_len, partition_size);
  if (need == 0) {
    // invalid arguments: the decode entry point's checks name them (they run
    // before its workspace check, and nothing is launched)
    const int st = paged_attn_decode(out, query, key_cache, value_cache, block_table, seq_lens, num_seqs,
                                     num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                     max_blocks_per_seq, max_seq_len, scale, kv_dtype, out_dtype,
                                     partition_size, nullptr, 0, stream);
    return st == PKV_OK ? PKV_ERR_SHAPE : st;
  }
  if (need > pkv::kNoallocScratchBytes) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = pkv::scratch_on_current_device(stream, &ws);
  if (st != PKV_OK) return st;
  return paged_attn_decode(out, query, key_cache, value_cache, block_table, seq_lens, num_seqs, num_heads,
                           num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_seq_len,
                           scale, kv_dtype, out_dtype, partition_size, ws, pkv::kNoallocScratchBytes, stream);
}
