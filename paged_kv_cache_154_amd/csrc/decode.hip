// Paged decode attention for CDNA4 (gfx950).
//
// What is computed (the paged-attention listing of "PagedAttention principle",
// tbr8.org, section 2.2, with the two-level addressing of "LLM inference
// engine internals" section 2.4): for each sequence s and query head h, over
// the tokens t < seq_len reached through the block table,
//   out[s,h] = sum_t softmax_t(scale * q[s,h] . K[t, h/G]) * V[t, h/G].
//
// How (an MI355X design, not the pages' kernel):
//  * The unit of work is a 16-token key tile of one (sequence, KV head). A
//    wave processes tiles one at a time: it issues all of the tile's K and V
//    loads (16-byte chunks) before computing, then
//      - Q.K^T on v_mfma_f32_16x16x32_{f16,bf16} (fp32 pools:
//        v_mfma_f32_16x16x4_f32) with the key tile as the A operand (16
//        tokens x 32 head-dim elements, straight from the pool) and the G
//        query heads of the KV head as the B operand (columns >= G are 0).
//        The result S[token][head] leaves each lane one head's scores for 4
//        tokens, so a head's softmax state lives in one lane column;
//      - P.V on v_mfma_f32_16x16x4_f32 with A = V^T (each lane holds head_dim
//        / 16 contiguous elements of one token's V row, widened to fp32) and
//        B = P^T in fp32: probabilities never drop below fp32, and the output
//        tile O^T[d][head] keeps a head in the same lane column as its
//        softmax state, so the online rescale is lane-local.
//  * Tokens past seq_len in the last tile are never read: their address is
//    clamped to the last valid token (finite data) and their score is set to
//    -inf before the exponent, so their weight is exactly 0.
//  * One workgroup of 4 waves per (sequence, KV head, partition of the
//    sequence). The partition's slice of the block table is staged in LDS
//    ("the block table of a sequence can be loaded into shared memory at
//    once", PagedAttention principle section 2.2); the 4 waves take the
//    partition's tiles round-robin and merge their (max, sum, O) through LDS.
//    A sequence that fits in one partition is written directly; otherwise
//    each partition writes (max, sum, O) to the workspace and
//    decode_reduce_kernel merges them.
//  * Workgroup i runs on XCD i mod 8. Workgroups are numbered partition-major
//    and KV-head-minor, so the 8 XCDs share every partition index evenly
//    (short sequences have only the low partition indices).

#include "pagedkv_internal.h"

#include <math.h>

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct F32Tag { static constexpr int kBytes = 4; };
struct F16Tag { static constexpr int kBytes = 2; };
struct BF16Tag { static constexpr int kBytes = 2; };

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

__device__ inline int clamp_len(int L, int max_len) {
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}

// A value known to be equal in every lane of the wave, moved to a scalar
// register so that the bookkeeping derived from it stays scalar.
__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Waves per SIMD the decode kernels are compiled for: 4 (<= 128 VGPRs) for
// every case except fp32 rows of 128 elements, whose tile buffers need 2.
template <class Tag, int D>
struct WavesPerEU {
  static constexpr int value = (Tag::kBytes == 4 && D == 128) ? 2 : 4;
};
#ifndef PKV_LPT_ORDER
#define PKV_LPT_ORDER 1
#endif
// log2 of the largest weight allowed before the running max is moved.
constexpr float kRescaleSlack = 8.0f;

// Per-lane state of one wave working through the tiles of one (sequence, KV
// head): the query operand, the softmax state of head `col` and its O^T
// accumulators.
template <class Tag, int D, int BS>
struct TileEngine {
  using Tr = KV<Tag>;
  static constexpr int E = Tr::kBytes;
  static constexpr int RB = D * E;        // bytes of one token row of one KV head
  static constexpr int NKL = RB / 64;     // 16-byte key chunks per lane per tile
  static constexpr int VPL = D / 16;      // V elements per lane per token
  static constexpr int VW = VPL * E / 4;  // 32-bit words per lane per token of V
  static_assert(RB % 64 == 0, "row must split into 4 lane groups of 16-byte chunks");

  int col;  // MFMA column: head within the group
  int grp;  // lane group 0..3
  uint4 qv[NKL];
  float m;     // running max of head `col` (log2 units)
  float lsum;  // this lane's share of the running sum of weights
  f32x4 acc[VPL];  // acc[j][i] = O[head col][VPL * (4 * grp + i) + j]

  __device__ void init(int lane) {
    col = lane & 15;
    grp = lane >> 4;
  }

  // q_group: the row of the first query head of this KV head's group.
  __device__ void load_q(const unsigned char* q_group, int G) {
    const unsigned char* qrow = q_group + (size_t)(col < G ? col : 0) * RB;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      qv[i] = col < G ? *reinterpret_cast<const uint4*>(qrow + 16 * (4 * i + grp))
                      : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  __device__ void reset() {
    m = -INFINITY;
    lsum = 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One tile of tokens cs .. cs+15 (cs a multiple of 16, cs <= t_last).
  // row_off(t) is the byte offset of token t's row for this KV head (t <= t_last).
  template <class RowOff>
  __device__ void step(const unsigned char* kbase, const unsigned char* vbase, int cs, int t_last,
                       uint32_t slot_bytes, float scale_log2, RowOff row_off) {
    uint4 kr[NKL];
    uint32_t vr[4][VW];
    const unsigned char* kp = kbase + row_off(min(cs + col, t_last)) + 16 * grp;
#pragma unroll
    for (int i = 0; i < NKL; ++i) kr[i] = *reinterpret_cast<const uint4*>(kp + 64 * i);
    // V rows of tokens t4 .. t4+3: a 4-aligned group never crosses a block
    const int t4 = min(cs + 4 * grp, t_last);
    const unsigned char* vp = vbase + row_off(t4) + col * (VPL * E);
    const uint32_t room = (uint32_t)(t_last - t4);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      load_words<VW>(vr[r], vp + (uint32_t)((uint32_t)r < room ? r : room) * slot_bytes);
    __builtin_amdgcn_sched_barrier(0);  // every load of the tile in flight first

    // scores S[token][head]: lane holds tokens cs + 4*grp + r of head col
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NKL; ++i) a = Tr::qk(kr[i], qv[i], a);
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = (cs + 4 * grp + r) <= t_last ? a[r] * scale_log2 : -INFINITY;

    // Online softmax with a lazy running max: the max (and the rescale of
    // lsum and O) moves only when some lane's tile max exceeds it by more than
    // 2^kRescaleSlack, so weights stay <= 2^kRescaleSlack and the rescale of
    // the accumulators is rare. Same algebra: every weight and the sum share
    // the reference m.
    float cmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    if (__any(cmax > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, cmax);
      const float alpha = fast_exp2(m - m_new);
      lsum *= alpha;
#pragma unroll
      for (int j = 0; j < VPL; ++j) acc[j] *= alpha;
      m = m_new;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = fast_exp2(s[r] - m);
      lsum += s[r];
    }

    // O^T += V^T P^T, 4 tokens per MFMA
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(Tr::elem(vr[r], j), s[r], acc[j], 0, 0, 0);
  }

  // Sum of weights of head col over all tokens seen (all 4 lane groups).
  __device__ float total_sum() const {
    float l = lsum;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    return l;
  }

  __device__ int d_of(int i, int j) const { return VPL * (4 * grp + i) + j; }
};

// ============================================================================
// fixed partitions
// ============================================================================

__host__ __device__ inline int o_stride(int D) { return D + 4; }

template <class Tag, int D, int BS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WavesPerEU<Tag, D>::value)))
void decode_partition_kernel(DecodeParams p) {
  using Eng = TileEngine<Tag, D, BS>;
  constexpr int RB = Eng::RB;
  constexpr int VPL = Eng::VPL;

  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);

  // Workgroup i runs on XCD i mod 8. The KV head varies fastest and the
  // partition slowest, so each XCD gets an even share of every partition
  // index (only low partition indices exist for short sequences).
  int wg = blockIdx.x;
  const int kvh = wg % p.num_kv_heads;
  wg /= p.num_kv_heads;
  const int seq = wg % p.num_seqs;
#if PKV_LPT_ORDER
  const int part = p.num_partitions - 1 - wg / p.num_seqs;
#else
  const int part = wg / p.num_seqs;
#endif
  const int G = p.group;
  const int head0 = kvh * G;

  const int L = clamp_len(p.seq_lens[seq], p.max_seq_len);
  if (L == 0) {  // nothing to attend to: a zero row
    if (part == 0) {
      for (int idx = threadIdx.x; idx < G * D; idx += kThreads)
        store_out<Tag>(p, ((size_t)seq * p.num_heads + head0) * D + idx, 0.0f);
    }
    return;
  }
  const int nparts = (L + p.partition - 1) / p.partition;
  if (part >= nparts) return;
#if PKV_LPT_ORDER
  // Partition 0 is the short one: [0, first) with first in (0, P], a multiple
  // of 16; partitions 1.. are full. Workgroups run from the highest partition
  // index down, so the long partitions start first and the short ones last.
  const int first = (L + kTile - 1) / kTile * kTile - (nparts - 1) * p.partition;
  const int t_begin = part == 0 ? 0 : first + (part - 1) * p.partition;
  const int t_end = min(L, part == 0 ? first : t_begin + p.partition);
#else
  const int t_begin = part * p.partition;
  const int t_end = min(L, t_begin + p.partition);
#endif

  // ---- stage this partition's slice of the block-table row --------------
  int* s_bt = reinterpret_cast<int*>(smem);
  const int lb0 = t_begin / BS;
  const int nlb = (t_end + BS - 1) / BS - lb0;
  {
    const int32_t* row = p.block_table + (size_t)seq * p.max_blocks + lb0;
    for (int i = threadIdx.x; i < nlb; i += kThreads) {
      const int b = row[i];
      s_bt[i] = ((unsigned)b < (unsigned)p.num_blocks) ? b : 0;  // never leave the pool
    }
  }

  TileEngine<Tag, D, BS> eng;
  eng.init(lane);
  eng.load_q(static_cast<const unsigned char*>(p.q) + ((size_t)seq * p.num_heads + head0) * RB, G);
  eng.reset();
  __syncthreads();

  const uint32_t slot_bytes = (uint32_t)p.num_kv_heads * RB;  // bytes between slots
  const unsigned char* kbase = static_cast<const unsigned char*>(p.k) + (size_t)kvh * RB;
  const unsigned char* vbase = static_cast<const unsigned char*>(p.v) + (size_t)kvh * RB;
  // The slot index phys * BS + offset fits in 32 bits (checked on the host),
  // so the byte offset is a single 32x32->64 multiply.
  auto row_off = [&](int tt) -> uint64_t {
    const uint32_t u = (uint32_t)tt;
    const uint32_t phys = (uint32_t)s_bt[u / BS - (uint32_t)lb0];
    return (uint64_t)(phys * BS + (u % BS)) * slot_bytes;
  };
  for (int cs = t_begin + wave * kTile; cs < t_end; cs += kWaves * kTile)
    eng.step(kbase, vbase, cs, t_end - 1, slot_bytes, p.scale_log2, row_off);

  // ---- merge the 4 waves -------------------------------------------------
  const float lsum = eng.total_sum();
  __syncthreads();  // block-table slice no longer needed: reuse its LDS
  const int OST = o_stride(D);
  float* s_o = reinterpret_cast<float*>(smem);
  const int o_bytes_all = kWaves * G * OST * 4;
  const int bt_bytes = ((p.partition < p.max_seq_len ? p.partition : p.max_seq_len) / BS + 1) * 4;
  const int base = ((o_bytes_all > bt_bytes ? o_bytes_all : bt_bytes) + 15) & ~15;
  float* s_m = reinterpret_cast<float*>(smem + base);
  float* s_l = s_m + kWaves * 16;
  if (eng.col < G) {
    if (eng.grp == 0) {
      s_m[wave * 16 + eng.col] = eng.m;
      s_l[wave * 16 + eng.col] = lsum;
    }
    float* orow = s_o + (size_t)(wave * G + eng.col) * OST;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < VPL; ++j) orow[eng.d_of(i, j)] = eng.acc[j][i];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
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

// One wave per (sequence, query head) of a split sequence, 4 waves per
// workgroup. Lane q loads (m_q, l_q) of partition q and the partial O loads
// do not wait for the weights, so the merge costs about one memory round
// trip; the weights 2^(m_q - M) are broadcast from their lanes.
template <class Tag, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeParams p) {
  constexpr int DPL = D / 64;  // output elements per lane
  const int lane = threadIdx.x & 63;
  const size_t rowid = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // seq * H + head
  if (rowid >= (size_t)p.num_seqs * p.num_heads) return;
  const int seq = (int)(rowid / p.num_heads);
  const int L = clamp_len(p.seq_lens[seq], p.max_seq_len);
  const int nparts = (L + p.partition - 1) / p.partition;
  if (nparts <= 1) return;  // written by the partition kernel
  const int NP = p.num_partitions;
  const float2* ml = reinterpret_cast<const float2*>(p.ws_ml) + rowid * NP;
  const float* o = p.ws_o + rowid * NP * D;

  float num[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) num[k] = 0.0f;
  float M = -INFINITY, den = 0.0f;
  // partitions in chunks of 64: lane q of the chunk holds partition base + q
  for (int base = 0; base < nparts; base += 64) {
    const int q = base + lane;
    const float2 mlq = q < nparts ? ml[q] : make_float2(-INFINITY, 0.0f);
    float cm = mlq.x;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float M_new = fmaxf(M, cm);
    const float alpha = fast_exp2(M - M_new);  // rescale of the earlier chunks
#pragma unroll
    for (int k = 0; k < DPL; ++k) num[k] *= alpha;
    den *= alpha;
    M = M_new;
    const float w = q < nparts ? fast_exp2(mlq.x - M) : 0.0f;
    float dw = w * mlq.y;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dw += __shfl_xor(dw, off);
    den += dw;
    const int n = min(64, nparts - base);
#pragma unroll 8
    for (int j = 0; j < n; ++j) {
      const float wj = __shfl(w, j);
      const float* oj = o + (size_t)(base + j) * D + lane;
#pragma unroll
      for (int k = 0; k < DPL; ++k) num[k] += wj * oj[64 * k];
    }
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) store_out<Tag>(p, rowid * D + lane + 64 * k, num[k] / den);
}

// ============================================================================
// launchers
// ============================================================================

template <class Tag, int D, int BS>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int span = p.partition < p.max_seq_len ? p.partition : p.max_seq_len;
  const int bt_bytes = (span / BS + 1) * 4;
  const int o_bytes = kWaves * p.group * o_stride(D) * 4;
  const int base = ((o_bytes > bt_bytes ? o_bytes : bt_bytes) + 15) & ~15;
  const size_t lds = (size_t)base + 2 * kWaves * 16 * 4;
  const unsigned grid = (unsigned)((size_t)p.num_seqs * p.num_kv_heads * p.num_partitions);
  decode_partition_kernel<Tag, D, BS><<<dim3(grid), dim3(kThreads), lds, stream>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.num_partitions > 1) {
    const size_t rows = (size_t)p.num_seqs * p.num_heads;
    decode_reduce_kernel<Tag, D><<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(p);
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
