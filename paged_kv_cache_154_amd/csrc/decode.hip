// Paged decode attention for CDNA4 (gfx950).
//
// What is computed (the paged-attention listing of "PagedAttention principle",
// tbr8.org, section 2.2, with the two-level addressing of "LLM inference
// engine internals" section 2.4): for each sequence s and query head h, over
// the tokens t < seq_len reached through the block table,
//   out[s,h] = sum_t softmax_t(scale * q[s,h] . K[t, h/G]) * V[t, h/G].
//
// How (an MI355X design, not the pages' kernel):
//  * One workgroup of 4 waves per (sequence, KV head, partition of the
//    sequence). The partition's slice of the block-table row is staged in LDS
//    once ("the block table of a sequence can be loaded into shared memory at
//    once", PagedAttention principle section 2.2).
//  * Waves take 16-token key tiles round-robin. Q.K^T of a tile is one MFMA
//    chain v_mfma_f32_16x16x32_{f16,bf16} per 64 bytes of head_dim (fp32
//    pools: v_mfma_f32_16x16x4_f32): the A operand is the key tile, 16 tokens
//    x 32 head-dim elements, loaded straight from the pool as 16-byte chunks;
//    the B operand is the G query heads of this KV head (columns >= G are
//    zero). The result tile S[token][head] leaves each lane one head's scores
//    for 4 tokens, so a head's softmax state (running max, sum) lives in one
//    lane column and reductions are two cross-lane exchanges.
//  * P.V runs on v_mfma_f32_16x16x4_f32 with A = V^T (each lane holds
//    head_dim/16 contiguous elements of one token's V row, widened to fp32)
//    and B = P^T in fp32: the probabilities never drop below fp32, and the
//    output tile O^T[d][head] keeps a head in the same lane column as its
//    softmax state, so the online rescale is lane-local.
//  * Tokens past seq_len in the last tile are never read: their address is
//    clamped to the last valid token (finite data) and their score is set to
//    -inf before the exponent, so their weight is exactly 0.
//  * The 4 waves merge their (max, sum, O) through LDS. A sequence that fits
//    in one partition is written directly; otherwise each partition writes
//    (max, sum, O) to the workspace and decode_reduce_kernel merges them.

#include "pagedkv_internal.h"

#include <math.h>

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct F32Tag {};
struct F16Tag {};
struct BF16Tag {};

template <class Tag>
struct KV;

template <>
struct KV<F32Tag> {
  static constexpr int kBytes = 4;
  // One 16-byte key chunk (4 head-dim elements) against the matching query
  // chunk: four K=4 steps of the fp32 MFMA.
  __device__ static inline f32x4 qk(const uint4& k, const uint4& q, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.x), __uint_as_float(q.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.y), __uint_as_float(q.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.z), __uint_as_float(q.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k.w), __uint_as_float(q.w), acc, 0, 0, 0);
    return acc;
  }
  __device__ static inline float elem(const uint32_t* w, int j) { return __uint_as_float(w[j]); }
  __device__ static inline void store(void* out, size_t i, float x) {
    static_cast<float*>(out)[i] = x;
  }
};

template <>
struct KV<F16Tag> {
  static constexpr int kBytes = 2;
  __device__ static inline f32x4 qk(const uint4& k, const uint4& q, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), acc, 0, 0, 0);
  }
  __device__ static inline float elem(const uint32_t* w, int j) {
    const uint16_t h = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
  }
  __device__ static inline void store(void* out, size_t i, float x) {
    static_cast<_Float16*>(out)[i] = static_cast<_Float16>(x);
  }
};

template <>
struct KV<BF16Tag> {
  static constexpr int kBytes = 2;
  __device__ static inline f32x4 qk(const uint4& k, const uint4& q, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), acc, 0, 0, 0);
  }
  __device__ static inline float elem(const uint32_t* w, int j) {
    // bf16 is the upper half of an fp32: widening is a shift or a mask
    return __uint_as_float((j & 1) ? (w[j >> 1] & 0xffff0000u) : (w[j >> 1] << 16));
  }
  __device__ static inline void store(void* out, size_t i, float x) {
    static_cast<__bf16*>(out)[i] = static_cast<__bf16>(x);
  }
};

template <int NW>
__device__ inline void load_words(uint32_t (&w)[NW], const unsigned char* ptr) {
  if constexpr (NW == 2) {
    const uint2 a = *reinterpret_cast<const uint2*>(ptr);
    w[0] = a.x; w[1] = a.y;
  } else {
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const uint4 a = *reinterpret_cast<const uint4*>(ptr + 16 * c);
      w[4 * c + 0] = a.x; w[4 * c + 1] = a.y; w[4 * c + 2] = a.z; w[4 * c + 3] = a.w;
    }
  }
}

template <class Tag>
__device__ inline void store_out(const DecodeParams& p, size_t i, float x) {
  if (p.out_f32) {
    static_cast<float*>(p.out)[i] = x;
  } else {
    KV<Tag>::store(p.out, i, x);
  }
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS layout of the partition kernel (bytes): the block-table slice, later
// reused for the per-wave O tiles, then per-wave (max, sum).
__host__ __device__ inline int o_stride(int D) { return D + 4; }

template <class Tag, int D, int BS, int U>
__global__ __launch_bounds__(256) void decode_partition_kernel(DecodeParams p) {
  using Tr = KV<Tag>;
  constexpr int E = Tr::kBytes;
  constexpr int RB = D * E;        // bytes of one token row of one KV head
  constexpr int NKL = RB / 64;     // 16-byte key chunks per lane per tile
  constexpr int VPL = D / 16;      // V elements per lane per token
  constexpr int VW = VPL * E / 4;  // 32-bit words per lane per token of V
  static_assert(RB % 64 == 0, "row must split into 4 lane groups of 16-byte chunks");

  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // MFMA column: head within the group
  const int grp = lane >> 4;  // lane group 0..3

  int wg = blockIdx.x;
  const int part = wg % p.num_partitions;
  wg /= p.num_partitions;
  const int kvh = wg % p.num_kv_heads;
  const int seq = wg / p.num_kv_heads;
  const int G = p.group;
  const int head0 = kvh * G;

  int L = p.seq_lens[seq];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int t_begin = part * p.partition;

  if (L == 0) {  // nothing to attend to: a zero row
    if (part == 0) {
      for (int idx = threadIdx.x; idx < G * D; idx += 256)
        store_out<Tag>(p, ((size_t)seq * p.num_heads + head0) * D + idx, 0.0f);
    }
    return;
  }
  if (t_begin >= L) return;
  const int t_end = min(L, t_begin + p.partition);
  const int nparts = (L + p.partition - 1) / p.partition;

  // ---- stage this partition's slice of the block-table row --------------
  int* s_bt = reinterpret_cast<int*>(smem);
  const int lb0 = t_begin / BS;
  const int nlb = (t_end + BS - 1) / BS - lb0;
  {
    const int32_t* row = p.block_table + (size_t)seq * p.max_blocks + lb0;
    for (int i = threadIdx.x; i < nlb; i += 256) {
      const int b = row[i];
      s_bt[i] = ((unsigned)b < (unsigned)p.num_blocks) ? b : 0;  // never leave the pool
    }
  }

  // ---- query operand: head (head0 + col), 16-byte chunks 4*i + grp -------
  uint4 qv[NKL];
  {
    const unsigned char* qrow = static_cast<const unsigned char*>(p.q) +
                                ((size_t)seq * p.num_heads + head0 + (col < G ? col : 0)) * RB;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      qv[i] = col < G ? *reinterpret_cast<const uint4*>(qrow + 16 * (4 * i + grp))
                      : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __syncthreads();

  const size_t slot_bytes = (size_t)p.num_kv_heads * RB;  // bytes between slots
  const unsigned char* kbase = static_cast<const unsigned char*>(p.k) + (size_t)kvh * RB;
  const unsigned char* vbase = static_cast<const unsigned char*>(p.v) + (size_t)kvh * RB;

  // byte offset of token t's row (this KV head), clamped to the last valid token
  auto row_offset = [&](int t) -> size_t {
    const int tt = t < t_end ? t : t_end - 1;
    const int phys = s_bt[tt / BS - lb0];
    return ((size_t)phys * BS + (tt % BS)) * slot_bytes;
  };

  float m = -INFINITY;  // running max of this lane's head (log2 units)
  float lsum = 0.0f;    // this lane's share of the running sum of weights
  f32x4 acc[VPL];       // O^T tiles: acc[j][i] = O[head col][VPL*(4*grp+i)+j]
#pragma unroll
  for (int j = 0; j < VPL; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = t_begin + wave * (kTile * U); c0 < t_end; c0 += kWaves * kTile * U) {
    uint4 kr[U][NKL];
    uint32_t vr[U][4][VW];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cs = c0 + u * kTile;
      const unsigned char* kp = kbase + row_offset(cs + col);
#pragma unroll
      for (int i = 0; i < NKL; ++i) kr[u][i] = *reinterpret_cast<const uint4*>(kp + 16 * (4 * i + grp));
#pragma unroll
      for (int r = 0; r < 4; ++r)
        load_words<VW>(vr[u][r], vbase + row_offset(cs + 4 * grp + r) + col * (VPL * E));
    }

    // scores S[token][head]: lane holds tokens cs + 4*grp + r of head col
    float s[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NKL; ++i) a = Tr::qk(kr[u][i], qv[i], a);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = c0 + u * kTile + 4 * grp + r;
        s[u][r] = t < t_end ? a[r] * p.scale_log2 : -INFINITY;
      }
    }

    // online softmax over this step's tokens
    float cmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) cmax = fmaxf(cmax, s[u][r]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m, cmax);
    const float alpha = fast_exp2(m - m_new);
    float ps = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[u][r] = fast_exp2(s[u][r] - m_new);
        ps += s[u][r];
      }
    lsum = lsum * alpha + ps;
    m = m_new;
#pragma unroll
    for (int j = 0; j < VPL; ++j) acc[j] *= alpha;

    // O^T += V^T P^T, 4 tokens per MFMA
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < VPL; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(Tr::elem(vr[u][r], j), s[u][r], acc[j], 0, 0, 0);
  }

  // ---- merge the 4 waves -------------------------------------------------
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();  // block-table slice no longer needed: reuse its LDS
  const int OST = o_stride(D);
  float* s_o = reinterpret_cast<float*>(smem);
  const int o_bytes_all = kWaves * G * OST * 4;
  const int bt_bytes = ((p.partition < p.max_seq_len ? p.partition : p.max_seq_len) / BS + 1) * 4;
  const int base = ((o_bytes_all > bt_bytes ? o_bytes_all : bt_bytes) + 15) & ~15;
  float* s_m = reinterpret_cast<float*>(smem + base);
  float* s_l = s_m + kWaves * 16;
  if (col < G) {
    if (grp == 0) {
      s_m[wave * 16 + col] = m;
      s_l[wave * 16 + col] = lsum;
    }
    float* orow = s_o + (size_t)(wave * G + col) * OST;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < VPL; ++j) orow[VPL * (4 * grp + i) + j] = acc[j][i];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w * 16 + h]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fast_exp2(s_m[w * 16 + h] - M);
      den += sc * s_l[w * 16 + h];
      num += sc * s_o[(w * G + h) * OST + d];
    }
    const size_t row = (size_t)seq * p.num_heads + head0 + h;
    if (nparts <= 1) {
      store_out<Tag>(p, row * D + d, num / den);
    } else {
      const size_t pi = row * p.num_partitions + part;
      p.ws_o[pi * D + d] = num;
      if (d == 0) {
        p.ws_ml[2 * pi] = M;
        p.ws_ml[2 * pi + 1] = den;
      }
    }
  }
}

// Merge the partitions of each split sequence:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p.
template <class Tag, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams p) {
  const int kvh = blockIdx.x % p.num_kv_heads;
  const int seq = blockIdx.x / p.num_kv_heads;
  int L = p.seq_lens[seq];
  L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
  const int nparts = (L + p.partition - 1) / p.partition;
  if (nparts <= 1) return;  // written by the partition kernel
  const int G = p.group;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D;
    const int d = idx - h * D;
    const size_t row = (size_t)seq * p.num_heads + kvh * G + h;
    const float* ml = p.ws_ml + row * p.num_partitions * 2;
    const float* o = p.ws_o + row * p.num_partitions * D + d;
    float M = -INFINITY;
    for (int q = 0; q < nparts; ++q) M = fmaxf(M, ml[2 * q]);
    float den = 0.0f, num = 0.0f;
    for (int q = 0; q < nparts; ++q) {
      const float sc = fast_exp2(ml[2 * q] - M);
      den += sc * ml[2 * q + 1];
      num += sc * o[(size_t)q * D];
    }
    store_out<Tag>(p, row * D + d, num / den);
  }
}

template <class Tag, int D, int BS>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  constexpr int U = 2;
  const int span = p.partition < p.max_seq_len ? p.partition : p.max_seq_len;
  const int bt_bytes = (span / BS + 1) * 4;
  const int o_bytes = kWaves * p.group * o_stride(D) * 4;
  const int base = ((o_bytes > bt_bytes ? o_bytes : bt_bytes) + 15) & ~15;
  const size_t lds = (size_t)base + 2 * kWaves * 16 * 4;
  const unsigned grid = (unsigned)((size_t)p.num_seqs * p.num_kv_heads * p.num_partitions);
  decode_partition_kernel<Tag, D, BS, U><<<dim3(grid), dim3(256), lds, stream>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.num_partitions > 1) {
    decode_reduce_kernel<Tag, D><<<dim3((unsigned)(p.num_seqs * p.num_kv_heads)), dim3(256), 0, stream>>>(p);
    e = hipGetLastError();
  }
  return e;
}

template <class Tag, int D>
hipError_t launch_bs(const DecodeParams& p, int bs, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_t<Tag, D, 8>(p, stream);
    case 16: return launch_t<Tag, D, 16>(p, stream);
    case 32: return launch_t<Tag, D, 32>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class Tag>
hipError_t launch_d(const DecodeParams& p, int d, int bs, hipStream_t stream) {
  switch (d) {
    case 64: return launch_bs<Tag, 64>(p, bs, stream);
    case 128: return launch_bs<Tag, 128>(p, bs, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int kv_dtype, int head_dim, int block_size,
                         hipStream_t stream) {
  switch (kv_dtype) {
    case 0: return launch_d<F32Tag>(p, head_dim, block_size, stream);
    case 1: return launch_d<F16Tag>(p, head_dim, block_size, stream);
    case 2: return launch_d<BF16Tag>(p, head_dim, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
