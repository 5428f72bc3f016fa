// Paged decode attention for CDNA4 (gfx950).
//
// What is computed (the paged-attention listing of "PagedAttention principle",
// tbr8.org, section 2.2, with the two-level addressing of "LLM inference
// engine internals" section 2.4): for each sequence s and query head h, over
// the tokens t < seq_len reached through the block table,
//   out[s,h] = sum_t softmax_t(scale * q[s,h] . K[t, h/G]) * V[t, h/G].
// With q_len > 1 new tokens per sequence (the candidates of speculative
// decoding verified in one pass, or a chunk of a prefill: "LLM inference
// optimisation in practice" sections 4.1-4.2 and 5.3), new token j attends
// to the positions t <= seq_len - q_len + j; its q_len * G query rows fill
// the MFMA columns of a KV head, each column with its own limit.
//
// How (an MI355X design, not the pages' kernel):
//  * The unit of work is a 16-token key tile of one (sequence, KV head). A
//    wave processes tiles one at a time: it issues all of the tile's K and V
//    loads (16-byte chunks) before computing. Each load instruction reads
//    whole rows (16 lanes cover one token's 256-byte row of the KV head), the
//    shape in which HBM streams fastest, and the loads are non-temporal
//    unless the blocks look shared (see decode_item): on MI355X that reads
//    ~6.6 TB/s where 16 rows x 64 bytes per instruction, the layout the MFMA
//    operand wants, reads ~5.7 (and worse when non-temporal). K is therefore
//    reordered through a per-wave LDS tile into the operand layout (e4m3
//    rows of 128 bytes instead stream from HBM into two LDS tile buffers per
//    wave, the next tile in flight while the current one is worked on; see
//    TileEngine). Then
//      - Q.K^T on v_mfma_f32_16x16x32_{f16,bf16} (fp32 pools:
//        v_mfma_f32_16x16x4_f32) with the key tile as the A operand (16
//        tokens x 32 head-dim elements, straight from the pool) and the G
//        query heads of the KV head (q_len * G query rows with several new
//        tokens) as the B operand (the other columns are 0).
//        The result S[token][head] leaves each lane one head's scores for 4
//        tokens, so a head's softmax state lives in one lane column;
//      - P.V with A = V^T (each lane holds head_dim / 16 contiguous elements
//        of 4 tokens' V rows) and B = P^T: on v_mfma_f32_16x16x32_bf16 for
//        bf16 pools and v_mfma_f32_16x16x16_bf16 for e4m3 pools (codes
//        widened to bf16), each weight cut exactly into three bf16 parts
//        (hi + mid + lo = the fp32 weight), on v_mfma_f32_16x16x4_f32 with
//        fp32 weights otherwise: the probabilities keep fp32 precision, and
//        the output tile O^T[d][head] keeps a head in the same lane column
//        as its softmax state, so the online rescale is lane-local.
//  * Tokens past seq_len in the last tile are never read: their address is
//    clamped to the last valid token (finite data) and their score is set to
//    -inf before the exponent, so their weight is exactly 0.
//  * Work items are (sequence, partition of P tokens, KV head). A persistent
//    grid (as many 8-wave workgroups as fit on the GPU) works through them;
//    each workgroup builds the launch's schedule in LDS from seq_lens (long
//    partitions first, each sequence's short first partition last) and
//    stages an item's slice of the block table in LDS (the page suggests
//    keeping a sequence's block table in shared memory: PagedAttention
//    principle, section 2.2). Its 8 waves take the item's tiles round-robin
//    and merge their (max, sum, O) through LDS. A sequence in one partition
//    is written directly; otherwise each partition writes (max, sum, O) to
//    the workspace and the last partition of the (sequence, KV head) to
//    finish merges them all and writes the output (see decode_item).
//  * Items are dealt to workgroups in static rounds that keep each KV head on
//    one XCD, and (unless the batch is of near-uniform length) all items
//    after the first round are taken from an atomic counter, which evens out
//    XCDs of different speeds and sequences of different lengths.

#include "pagedkv_internal.h"

#include <hip/hip_ext.h>

#include <math.h>

#include <mutex>
#include <type_traits>
#include <vector>

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

struct F32Tag { static constexpr int kBytes = 4; };
struct F16Tag { static constexpr int kBytes = 2; };
struct BF16Tag { static constexpr int kBytes = 2; };
// e4m3 K/V (one byte per element, a scale per KV head) with a bf16 or fp16
// query and output ("LLM inference optimisation in practice" section 6.2:
// attention over a low-precision KV cache).
struct E4M3BF16Tag { static constexpr int kBytes = 1; };
struct E4M3F16Tag { static constexpr int kBytes = 1; };

template <class Tag>
struct KV;

template <>
struct KV<F32Tag> {
  static constexpr int kBytes = 4;
  static constexpr int kQBytes = 4;   // query element
  static constexpr bool kF8 = false;
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
  __device__ static inline void store4(void* out, size_t i, float4 x) {
    *reinterpret_cast<float4*>(static_cast<float*>(out) + i) = x;
  }
};

template <>
struct KV<F16Tag> {
  static constexpr int kBytes = 2;
  static constexpr int kQBytes = 2;
  static constexpr bool kF8 = false;
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
  __device__ static inline void store4(void* out, size_t i, float4 x) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x.x)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(x.y)) << 16);
    const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x.z)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(x.w)) << 16);
    *reinterpret_cast<uint2*>(static_cast<_Float16*>(out) + i) = make_uint2(lo, hi);
  }
};

template <>
struct KV<BF16Tag> {
  static constexpr int kBytes = 2;
  static constexpr int kQBytes = 2;
  static constexpr bool kF8 = false;
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
  __device__ static inline void store4(void* out, size_t i, float4 x) {
    const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x.x)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x.y)) << 16);
    const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x.z)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x.w)) << 16);
    *reinterpret_cast<uint2*>(static_cast<__bf16*>(out) + i) = make_uint2(lo, hi);
  }
};

typedef float f32x2v __attribute__((ext_vector_type(2)));

// The e4m3 K/V traits over a 16-bit query type Q16 (KV<BF16Tag> or
// KV<F16Tag>): the key codes are widened to Q16 in registers (exactly: e4m3
// has 3 mantissa bits and a range inside both) for the 16-bit MFMA, values
// to bf16 (exactly) for the bf16 P.V MFMA.
template <class Q16, bool kBF>
struct KVe4m3 {
  static constexpr int kBytes = 1;
  static constexpr int kQBytes = 2;
  static constexpr bool kF8 = true;
  __device__ static inline f32x4 qk(const uint4& k, const uint4& q, f32x4 acc) { return Q16::qk(k, q, acc); }
  // four codes -> two words of 16-bit values (element order kept): the
  // scaled pair conversions at scale 1, one instruction per two codes (exact
  // for every code; checked on MI355X against the format's values, NaN kept)
  __device__ static inline void widen4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    if constexpr (kBF) {
      lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
      hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    } else {
      lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
      hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
    }
  }
  // 16 codes -> the two 8-element key chunks of the 16-bit MFMA
  __device__ static inline void widen(const uint4& raw, uint4& c0, uint4& c1) {
    widen4(raw.x, c0.x, c0.y);
    widen4(raw.y, c0.z, c0.w);
    widen4(raw.z, c1.x, c1.y);
    widen4(raw.w, c1.z, c1.w);
  }
  __device__ static inline void store(void* out, size_t i, float x) { Q16::store(out, i, x); }
  __device__ static inline void store4(void* out, size_t i, float4 x) { Q16::store4(out, i, x); }
};
template <> struct KV<E4M3BF16Tag> : KVe4m3<KV<BF16Tag>, true> {};
template <> struct KV<E4M3F16Tag> : KVe4m3<KV<F16Tag>, false> {};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Loads that stream past the caches (true) or are cached as usual (false).
template <bool NT> struct NTL;
template <> struct NTL<true> {
  template <class T> __device__ static inline T ld(const T* p) { return __builtin_nontemporal_load(p); }
};
template <> struct NTL<false> {
  template <class T> __device__ static inline T ld(const T* p) { return *p; }
};
template <bool nt, int NW>
__device__ inline void load_words(uint32_t (&w)[NW], const unsigned char* ptr) {
  if constexpr (NW == 1) {
    w[0] = NTL<nt>::ld(reinterpret_cast<const uint32_t*>(ptr));
  } else if constexpr (NW == 2) {
    const u32x2* a2 = reinterpret_cast<const u32x2*>(ptr);
    const u32x2 a = NTL<nt>::ld(a2);
    w[0] = a.x; w[1] = a.y;
  } else {
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const u32x4* a4 = reinterpret_cast<const u32x4*>(ptr + 16 * c);
      const u32x4 a = NTL<nt>::ld(a4);
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

// Elements i .. i+3 of out (i a multiple of 4).
template <class Tag>
__device__ inline void store_out4(const DecodeParams& p, size_t i, float4 x) {
  if (p.out_f32) {
    KV<F32Tag>::store4(p.out, i, x);
  } else {
    KV<Tag>::store4(p.out, i, x);
  }
}

// (a, b) as one 8-byte word, a in the low half, and back.
__device__ inline unsigned long long pack2(float a, float b) {
  return (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
}
__device__ inline float lo_of(unsigned long long w) { return __uint_as_float((uint32_t)w); }
__device__ inline float hi_of(unsigned long long w) { return __uint_as_float((uint32_t)(w >> 32)); }

// MFMA column tiles of 16 query rows for R rows per KV head, one per group of
// waves: 1, 2, 4 or 8 (R <= 16 * kWaves).
__host__ __device__ inline int col_tiles(int R) { return R <= 16 ? 1 : R <= 32 ? 2 : R <= 64 ? 4 : 8; }

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
// log2 of the largest weight allowed before the running max is moved.
constexpr float kRescaleSlack = 8.0f;
// Starting running max: a finite stand-in for -inf, so that a column that
// sees no position in a tile (or a whole partition: a causal limit) keeps
// exact zero weights instead of NaN (2^(-inf - -inf)); the first attended
// score replaces it, and 2^(kNoMax - score) is 0 like 2^-inf.
constexpr float kNoMax = -1e30f;
// log2 of a row's sum of weights, in the units of the scores (log2, scale
// included): M + log2(den); kNoMax for a row that saw no position.
__device__ inline float lse_of(float M, float den) { return den > 0.0f ? M + __log2f(den) : kNoMax; }

// Per-lane state of one wave working through the tiles of one (sequence, KV
// head): the query operand, the softmax state of head `col` and its O^T
// accumulators.
template <class Tag, int D, int BS>
struct TileEngine {
  using Tr = KV<Tag>;
  static constexpr int E = Tr::kBytes;
  static constexpr bool kF8 = Tr::kF8;
  static constexpr int RB = D * E;        // bytes of one token row of one KV head
  static constexpr int QB = D * Tr::kQBytes;  // bytes of one query row
  static constexpr int NKR = RB / 64;     // 16-byte key chunks per lane per tile, as loaded
  // key operands per lane per tile (e4m3: each loaded chunk widens to two)
  static constexpr int NKL = kF8 ? 2 * NKR : NKR;
  static constexpr int VPL = D / 16;      // V elements per lane per token
  static constexpr int VW = VPL * E / 4;  // 32-bit words per lane per token of V
  static_assert(RB % 64 == 0, "row must split into 4 lane groups of 16-byte chunks");
  // Rows of >= 256 bytes load K like V (whole rows) and reorder it through
  // LDS; rows of 128 bytes (e4m3 at head_dim 128, 16-bit types at 64) are
  // read whole too, 8 rows per instruction, and reordered the same way;
  // shorter rows load it in the operand layout.
  static constexpr bool kKLds = RB >= 256;
  static constexpr bool kKLds128 = RB == 128;
  static constexpr int KCL = RB / 256;     // 16-byte chunks per lane per token (K rows whole)
  static constexpr int KTS = RB + 16;      // LDS row stride of the K tile
  // e4m3 rows of 128 bytes: each wave's tiles go from HBM straight into two
  // LDS tile buffers of its own (the shared-tile layout below), the next
  // tile streaming into one while the other is consumed
  static constexpr bool kPipe = kF8 && RB == 128;
  // one wave's K tile (and, for 128-byte rows, its V tile after it); with
  // kPipe its two tile buffers (K then V rows, 16 RB bytes each)
  static constexpr int KT_BYTES = kPipe ? 4 * 16 * RB : (kKLds ? 16 * KTS : (kKLds128 ? 2 * 16 * KTS : 0));
  static constexpr int NACC = VPL;  // O^T accumulator tiles
  // bf16 and e4m3 pools: P.V on the bf16 MFMA with the weights cut into exact
  // parts (e4m3 values are bf16 values)
  static constexpr bool kPVbf16 = std::is_same<Tag, BF16Tag>::value || kF8;

  int col;  // MFMA column: query row within the KV head's rows
  int grp;  // lane group 0..3
  int lim;  // last position column `col` attends to
  uint4 qv[NKL];
  float m;     // running max of head `col` (log2 units)
  float lsum;  // this lane's share of the running sum of weights
  f32x4 acc[NACC];  // acc[j][i] = O[head col][VPL * (4 * grp + i) + j]

  __device__ void init(int lane) {
    col = lane & 15;
    grp = lane >> 4;
  }

  // qrow: this lane's query row (column col), read when `valid`. Chunk i
  // holds the head-dim elements that key operand i of this lane holds:
  // 32 i + 8 grp .. +7 when keys are loaded in 16-byte chunks of 8 elements;
  // for e4m3 keys (16 elements per loaded chunk, widened to operands 2u and
  // 2u + 1) 64 u + 16 grp + 8 h .. +7 for i = 2u + h.
  __device__ void load_q(const unsigned char* qrow, bool valid) {
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int off = kF8 ? 128 * (i >> 1) + 32 * grp + 16 * (i & 1) : 16 * (4 * i + grp);
      qv[i] = valid ? *reinterpret_cast<const uint4*>(qrow + off) : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  __device__ void reset() {
    m = kNoMax;
    lsum = 0.0f;
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The registers of one tile's K and V, as loaded.
  struct Tile {
    uint4 kr[NKL];
    uint32_t vr[4][VW];
  };

  // Loads of the tile of tokens cs .. cs+15 (cs a multiple of 16, cs <=
  // t_last; tokens past t_last read t_last's row). row_off(t) is the byte
  // offset of token t's row for this KV head (t <= t_last); nt selects
  // non-temporal loads.
  template <bool nt, class RowOff>
  __device__ void issue(Tile& g, const unsigned char* kbase, const unsigned char* vbase, int cs, int t_last,
                        uint32_t slot_bytes, RowOff row_off) {
    uint4 (&kr)[NKL] = g.kr;
    // rows of tokens t4 .. t4+3: a 4-aligned group never crosses a block
    const int t4 = min(cs + 4 * grp, t_last);
    const uint64_t off4 = row_off(t4);
    const uint32_t room = (uint32_t)(t_last - t4);
    if constexpr (kKLds) {
      // K rows whole: 16 lanes read a token's row (256 contiguous bytes per
      // instruction and row), like V
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const unsigned char* kp = kbase + off4 + (uint32_t)((uint32_t)r < room ? r : room) * slot_bytes;
#pragma unroll
        for (int u = 0; u < KCL; ++u) {
          const u32x4* a4 = reinterpret_cast<const u32x4*>(kp + 16 * (col + 16 * u));
          const u32x4 a = NTL<nt>::ld(a4);
          kr[r * KCL + u] = make_uint4(a.x, a.y, a.z, a.w);
        }
      }
    } else if constexpr (kKLds128) {
      // 8 lanes read a token's 128-byte row: instruction a takes rows 8 a ..
      // 8 a + 7 of the tile (raw codes for e4m3)
      const int lane = col + 16 * grp;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const unsigned char* kp = kbase + row_off(min(cs + 8 * a + (lane >> 3), t_last)) + 16 * (lane & 7);
        const u32x4 v = NTL<nt>::ld(reinterpret_cast<const u32x4*>(kp));
        kr[a] = make_uint4(v.x, v.y, v.z, v.w);
      }
    } else {
      const unsigned char* kp = kbase + row_off(min(cs + col, t_last)) + 16 * grp;
      if constexpr (kF8) {
        // raw codes in the first NKR slots, widened after the loads are issued
#pragma unroll
        for (int u = 0; u < NKR; ++u) {
          const u32x4 a = NTL<nt>::ld(reinterpret_cast<const u32x4*>(kp + 64 * u));
          kr[u] = make_uint4(a.x, a.y, a.z, a.w);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NKL; ++i) kr[i] = *reinterpret_cast<const uint4*>(kp + 64 * i);
      }
    }
    if constexpr (kKLds128) {
      // V rows whole as well, 8 per instruction, into the words vr holds
      // (reordered in consume)
      const int lane = col + 16 * grp;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const unsigned char* vp = vbase + row_off(min(cs + 8 * a + (lane >> 3), t_last)) + 16 * (lane & 7);
        const u32x4 v = NTL<nt>::ld(reinterpret_cast<const u32x4*>(vp));
        g.vr[2 * a][0] = v.x;
        g.vr[2 * a][1] = v.y;
        g.vr[2 * a + 1][0] = v.z;
        g.vr[2 * a + 1][1] = v.w;
      }
    } else {
      const unsigned char* vp = vbase + off4 + col * (VPL * E);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        load_words<nt, VW>(g.vr[r], vp + (uint32_t)((uint32_t)r < room ? r : room) * slot_bytes);
    }
  }

  // The tile's scores, softmax update and P.V, on the registers `issue`
  // filled for the tile at cs (every score past t_last is masked, so a tile
  // wholly past the end changes nothing). kt is the wave's LDS tile
  // (KT_BYTES); causal applies the column's own limit `lim` as well
  // (several new tokens).
  template <bool causal, bool k_ops = false>
  __device__ void consume(Tile& g, int cs, int t_last, float scale_log2, unsigned char* kt) {
    uint4 (&kr)[NKL] = g.kr;
    if constexpr (kKLds128 && !k_ops) {
      // whole rows through the wave's LDS tile (rows padded by 16 bytes) into
      // the operand layout: lane (col, grp) takes chunk 4u + grp of token cs
      // + col (raw codes for e4m3, widened below)
      const int lane = col + 16 * grp;
#pragma unroll
      for (int a = 0; a < 2; ++a)
        *reinterpret_cast<uint4*>(kt + (8 * a + (lane >> 3)) * KTS + 16 * (lane & 7)) = kr[a];
#pragma unroll
      for (int u = 0; u < NKR; ++u)
        kr[u] = *reinterpret_cast<const uint4*>(kt + col * KTS + 16 * (4 * u + grp));
      // V the same way: lane (col, grp) takes bytes [8 col, 8 col + 8) of
      // tokens cs + 4 grp + r
      unsigned char* vt = kt + 16 * KTS;
#pragma unroll
      for (int a = 0; a < 2; ++a)
        *reinterpret_cast<uint4*>(vt + (8 * a + (lane >> 3)) * KTS + 16 * (lane & 7)) =
            make_uint4(g.vr[2 * a][0], g.vr[2 * a][1], g.vr[2 * a + 1][0], g.vr[2 * a + 1][1]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint2 w = *reinterpret_cast<const uint2*>(vt + (4 * grp + r) * KTS + 8 * col);
        g.vr[r][0] = w.x;
        g.vr[r][1] = w.y;
      }
    }
    if constexpr (kF8) {
#pragma unroll
      for (int u = NKR - 1; u >= 0; --u) {  // from the top: slot u is read before it is written
        const uint4 raw = kr[u];
        Tr::widen(raw, kr[2 * u], kr[2 * u + 1]);
      }
    }
    if constexpr (kKLds && !k_ops) {
      // through the wave's LDS tile (rows padded by 16 bytes: both the row
      // writes and the column reads below hit every bank once) into the
      // MFMA layout: lane (col, grp) takes chunk 4i + grp of token cs + col
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int u = 0; u < KCL; ++u)
          *reinterpret_cast<uint4*>(kt + (4 * grp + r) * KTS + 16 * (col + 16 * u)) = kr[r * KCL + u];
#pragma unroll
      for (int i = 0; i < NKL; ++i)
        kr[i] = *reinterpret_cast<const uint4*>(kt + col * KTS + 16 * (4 * i + grp));
    }

    // scores S[token][head]: lane holds tokens cs + 4*grp + r of head col
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NKL; ++i) a = Tr::qk(kr[i], qv[i], a);
    float s[4];
    // e4m3 pools (issue-bound): no mask when the whole tile is inside the
    // sequence
    if (kF8 && !causal && cs + kTile - 1 <= t_last) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = a[r] * scale_log2;
    } else {
      const int last = causal ? min(t_last, lim) : t_last;
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = (cs + 4 * grp + r) <= last ? a[r] * scale_log2 : -INFINITY;
    }

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
      for (int j = 0; j < NACC; ++j) acc[j] *= alpha;
      m = m_new;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = fast_exp2(s[r] - m);
      lsum += s[r];
    }

    if constexpr (kPVbf16) {
      // O^T += V^T P^T on the bf16 MFMA, exactly: each weight is cut into
      // three bf16 parts by truncation (hi = the top 16 bits of its fp32
      // pattern, mid the same of the remainder, lo the rest, which has at
      // most 8 significant bits), so hi + mid + lo is the weight itself; the
      // products with the bf16 V elements are exact and the MFMA sums them in
      // fp32. bf16 pools: a lane group's 32 k slots of the 16x16x32 MFMA
      // carry its 4 tokens twice, against (hi, mid) in one MFMA and (lo, 0)
      // in a second. e4m3 pools (issue-bound): its 16 k slots of the 16x16x16
      // MFMA are its 4 tokens, three MFMAs against hi, mid and lo, on the V
      // pairs as they are widened, without the copies that writing the
      // tokens twice takes. (The fp32 16x16x4 form took four MFMAs of twice
      // the cycles per head-dim block.)
      uint32_t hp[4], mp[4], lp[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t u = __float_as_uint(s[r]);
        hp[r] = u & 0xffff0000u;
        const float r1 = s[r] - __uint_as_float(hp[r]);
        mp[r] = __float_as_uint(r1) & 0xffff0000u;
        lp[r] = __float_as_uint(r1 - __uint_as_float(mp[r]));
      }
      // upper halves of a and b -> (a.hi | b.hi << 16)
      auto hi2 = [](uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); };
      const uint2 h01 = make_uint2(hi2(hp[0], hp[1]), hi2(hp[2], hp[3]));
      const uint2 m01 = make_uint2(hi2(mp[0], mp[1]), hi2(mp[2], mp[3]));
      const uint2 l01 = make_uint2(hi2(lp[0], lp[1]), hi2(lp[2], lp[3]));
      auto pv = [&](int j, uint32_t x01, uint32_t x23) {
        if constexpr (kF8) {
          const s16x4 av = __builtin_bit_cast(s16x4, make_uint2(x01, x23));
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, h01), acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, m01), acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, l01), acc[j], 0, 0, 0);
        } else {
          const bf16x8 av = __builtin_bit_cast(bf16x8, make_uint4(x01, x23, x01, x23));
          const uint4 bhm = make_uint4(h01.x, h01.y, m01.x, m01.y);
          const uint4 bl0 = make_uint4(l01.x, l01.y, 0u, 0u);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bhm), acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bl0), acc[j], 0, 0, 0);
        }
      };
      if constexpr (kF8) {
        // e4m3 V: bytes j and j + 1 of tokens (0, 1) gathered into one word
        // and widened to bf16 exactly (e4m3 values are bf16 values), two
        // elements per conversion
#pragma unroll
        for (int j = 0; j < VPL; j += 2) {
          const uint32_t b0 = j & 3;
          const uint32_t sel = b0 | ((4u + b0) << 8) | ((b0 + 1u) << 16) | ((5u + b0) << 24);
          const uint32_t t01 = __builtin_amdgcn_perm(g.vr[1][j >> 2], g.vr[0][j >> 2], sel);
          const uint32_t t23 = __builtin_amdgcn_perm(g.vr[3][j >> 2], g.vr[2][j >> 2], sel);
          pv(j, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t01, 1.0f, false)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t23, 1.0f, false)));
          pv(j + 1, __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t01, 1.0f, true)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(t23, 1.0f, true)));
        }
      } else {
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          // element j of tokens (0, 1) and (2, 3), as bf16 pairs
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
          pv(j, __builtin_amdgcn_perm(g.vr[1][j >> 1], g.vr[0][j >> 1], sel),
             __builtin_amdgcn_perm(g.vr[3][j >> 1], g.vr[2][j >> 1], sel));
        }
      }
    } else {
      // O^T += V^T P^T, 4 tokens per MFMA
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int j = 0; j < VPL; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(Tr::elem(g.vr[r], j), s[r], acc[j], 0, 0, 0);
      }
    }
  }

  // One tile: every load in flight, then the math.
  template <bool nt, bool causal, class RowOff>
  __device__ void step(const unsigned char* kbase, const unsigned char* vbase, int cs, int t_last,
                       uint32_t slot_bytes, float scale_log2, RowOff row_off, unsigned char* kt) {
    Tile g;
    issue<nt>(g, kbase, vbase, cs, t_last, slot_bytes, row_off);
    __builtin_amdgcn_sched_barrier(0);  // every load of the tile in flight first
    consume<causal>(g, cs, t_last, scale_log2, kt);
  }

  // ---- tiles shared by the waves of a workgroup (more than 16 query rows
  // per KV head: several column groups read every tile) ----------------------
  // A tile's K and V rows go from HBM straight into LDS (global_load_lds, no
  // registers held while in flight), once, and every column group reads its
  // operands from there. A slot holds 16 rows of RB bytes for K and as much
  // for V; the 16-byte chunks of row t sit at position chunk ^ swz(t), so that
  // the 16 lanes of a column read (16 rows, one chunk each) and of a V read
  // (one row, 16 chunks) touch 16 different bank groups.
  static constexpr int CH = RB / 16;        // 16-byte chunks per row
  static constexpr int TPI = 64 / CH;       // rows per load instruction (64 lanes x 16 bytes)
  static constexpr bool kShared = CH == 8 || CH == 16;
  static constexpr int SLOT_BYTES = 16 * RB;
  __device__ static inline int swz(int t) { return (t / (16 / CH)) & (CH - 1); }

  // Loads of the tile at cs (cs <= t_last; rows past t_last read t_last's)
  // into the slot pair (sk, sv): instruction a takes rows a TPI .. a TPI +
  // TPI - 1, lane l the chunk (l mod CH) ^ swz(row) of row a TPI + l / CH,
  // written to LDS at the lane's own 16 bytes. Completion: vmcnt.
  template <bool nt, class RowOff>
  __device__ void issue_shared(unsigned char* sk, unsigned char* sv, const unsigned char* kbase,
                               const unsigned char* vbase, int cs, int t_last, RowOff row_off) {
    static_assert(kShared, "shared tiles take rows of 128 or 256 bytes");
    const int lane = col + 16 * grp;
    const int c = lane % CH;
#pragma unroll
    for (int a = 0; a < 16 / TPI; ++a) {
      const int tt = a * TPI + lane / CH;
      const uint64_t off = row_off(min(cs + tt, t_last)) + 16 * (c ^ swz(tt));
      __builtin_amdgcn_global_load_lds(kbase + off, (__attribute__((address_space(3))) void*)(sk + a * 1024), 16,
                                       0, nt ? 2 : 0);
      __builtin_amdgcn_global_load_lds(vbase + off, (__attribute__((address_space(3))) void*)(sv + a * 1024), 16,
                                       0, nt ? 2 : 0);
    }
  }

  // The loads of one half of the tile at cs (K rows from kbase or V rows from
  // vbase, as issue_shared) into the slot s. Completion: vmcnt.
  template <bool nt, class RowOff>
  __device__ void issue_half(unsigned char* s, const unsigned char* base, int cs, int t_last, RowOff row_off) {
    static_assert(kShared, "shared tiles take rows of 128 or 256 bytes");
    const int lane = col + 16 * grp;
    const int c = lane % CH;
#pragma unroll
    for (int a = 0; a < 16 / TPI; ++a) {
      const int tt = a * TPI + lane / CH;
      const uint64_t off = row_off(min(cs + tt, t_last)) + 16 * (c ^ swz(tt));
      __builtin_amdgcn_global_load_lds(base + off, (__attribute__((address_space(3))) void*)(s + a * 1024), 16, 0,
                                       nt ? 2 : 0);
    }
  }

  // fetch_shared with the reads written as LDS instructions the compiler
  // does not see, so that it adds no wait for loads still streaming into
  // another slot (it cannot tell the slots apart); the reads are complete
  // when this returns. The caller waits for the slot's own loads first.
  __device__ void fetch_unseen(Tile& g, const unsigned char* sk, const unsigned char* sv) {
    static_assert(kShared && NKR == VW && (NKR == 2 || NKR == 4), "rows of 128 or 256 bytes");
    auto lds = [](const unsigned char* p) {
      return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
    };
    // the lane's place passes through an empty asm statement so that its
    // addressing is recomputed per tile instead of being hoisted out of the
    // tile loops and held in registers across the math
    int cl = col, gr = grp;
    asm volatile("" : "+v"(cl), "+v"(gr));
    uint32_t ka[NKR], va[4];
#pragma unroll
    for (int u = 0; u < NKR; ++u) ka[u] = lds(sk + cl * RB + 16 * ((4 * u + gr) ^ swz(cl)));
    const int b = cl * VPL * E;  // the lane's V bytes within a row
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = 4 * gr + r;
      va[r] = lds(sv + tt * RB + 16 * ((b / 16) ^ swz(tt)) + (b % 16));
    }
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    if constexpr (NKR == 2) {
      u32x4_t a0, a1;
      u32x2_t w0, w1, w2, w3;
      asm volatile(
          "ds_read_b128 %0, %6\n\t"
          "ds_read_b128 %1, %7\n\t"
          "ds_read_b64 %2, %8\n\t"
          "ds_read_b64 %3, %9\n\t"
          "ds_read_b64 %4, %10\n\t"
          "ds_read_b64 %5, %11\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a0), "=&v"(a1), "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
          : "v"(ka[0]), "v"(ka[1]), "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])
          : "memory");
      g.kr[0] = make_uint4(a0.x, a0.y, a0.z, a0.w);
      g.kr[1] = make_uint4(a1.x, a1.y, a1.z, a1.w);
      const u32x2_t w[4] = {w0, w1, w2, w3};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        g.vr[r][0] = w[r].x;
        g.vr[r][1] = w[r].y;
      }
    } else {
      // two blocks of four reads (K, then V): fewer registers tied up at once
      u32x4_t a0, a1, a2, a3;
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
          : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3])
          : "memory");
      g.kr[0] = make_uint4(a0.x, a0.y, a0.z, a0.w);
      g.kr[1] = make_uint4(a1.x, a1.y, a1.z, a1.w);
      g.kr[2] = make_uint4(a2.x, a2.y, a2.z, a2.w);
      g.kr[3] = make_uint4(a3.x, a3.y, a3.z, a3.w);
      u32x4_t w0, w1, w2, w3;
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(w0), "=&v"(w1), "=&v"(w2), "=&v"(w3)
          : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3])
          : "memory");
      const u32x4_t w[4] = {w0, w1, w2, w3};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        g.vr[r][0] = w[r].x;
        g.vr[r][1] = w[r].y;
        g.vr[r][2] = w[r].z;
        g.vr[r][3] = w[r].w;
      }
    }
  }

  // The operands of the tile in the slot pair (sk, sv), in the layout issue
  // leaves in registers: key chunk 4u + grp of row col (raw codes for e4m3),
  // and the V bytes [col VPL E, + VPL E) of rows 4 grp + r.
  __device__ void fetch_shared(Tile& g, const unsigned char* sk, const unsigned char* sv) {
#pragma unroll
    for (int u = 0; u < NKR; ++u)
      g.kr[u] = *reinterpret_cast<const uint4*>(sk + col * RB + 16 * ((4 * u + grp) ^ swz(col)));
    constexpr int VB = VPL * E;  // V bytes per lane per row
    const int b = col * VB;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = 4 * grp + r;
      load_words<false, VW>(g.vr[r], sv + tt * RB + 16 * ((b / 16) ^ swz(tt)) + (b % 16));
    }
  }

  // The wave's unnormalised O rows to LDS: head h's row at o0 + h * ost.
  // Called by every lane; writes the rows of this lane's column when `valid`.
  __device__ void write_o(float* o0, int ost, bool valid) {
    if (valid) {
      float* orow = o0 + (size_t)col * ost;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < VPL; ++j) orow[d_of(i, j)] = acc[j][i];
    }
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
// work list and partition kernel
// ============================================================================

__host__ __device__ inline int o_stride(int D) { return D + 4; }

// How a sequence of L > 0 tokens is cut into partitions of P tokens (a
// multiple of 16): n = ceil(L / P) partitions; partition 0 is the short one,
// [0, r) with r = roundup16(L) - (n-1) P in [16, P]; partitions 1 .. n-1
// follow, each [r + (j-1) P, r + j P) (the last one ends at L). A sequence in
// one partition is written out directly; the others are merged by whichever
// of their partitions finishes last. The short partitions 0 are scheduled last.
struct Cut {
  int n, r;
};

__device__ inline Cut cut_of(int L, int P) {
  Cut c;
  c.n = (L + P - 1) / P;
  c.r = (L + kTile - 1) / kTile * kTile - (c.n - 1) * P;
  return c;
}

// The work list of one launch (at most kMaxSeqsPerLaunch sequences), built
// by every workgroup in its own LDS from seq_lens. Entries are (sequence,
// partition):
//   * first the full partitions n-1 .. 1 of every split sequence, in batch
//     order: sequence s owns entries [full[s], full[s+1]) (an exclusive scan
//     of n_s - 1);
//   * then the partition 0 of every sequence, stably sorted into kClasses
//     length classes, longest first; sequences of length 0 (one empty entry
//     that writes the zero row) last.
// Item w is entry w / num_kv_heads with KV head w % num_kv_heads. Long items
// first and short ones last even out the end of the launch; the stable order
// keeps sequences that sit next to each other in the batch (such as samples
// of one prompt sharing its blocks) next to each other in time. A
// workgroup whose first item is a full partition of one of the first 64
// sequences finds it with a scan of those 64 lengths in each wave (see
// first_entry) and builds the list after that item.
constexpr int kClasses = 4;
constexpr int kClassBits = 12;  // packed per-class counts: kMaxSeqsPerLaunch < 2^12
static_assert(kMaxSeqsPerLaunch < (1 << kClassBits), "class counts must fit their field");
static_assert((kClasses + 1) * kClassBits <= 64, "class counts must pack into 64 bits");
constexpr int kSeqsPerThread = (kMaxSeqsPerLaunch + kThreads - 1) / kThreads;

__host__ __device__ inline int plan_bytes(int S) { return ((S + 1) * 4 + S * 4 + S * 2 + 15) & ~15; }

struct Plan {
  int* full;         // [S + 1]
  int* len;          // [S]: sequence lengths, clamped to max_seq_len
  uint16_t* first;   // [S]: partitions 0, sorted
  int S;
  int n_full;        // entries of full partitions
  int n_long;        // entries in the longest class (full partitions included)
};

__device__ inline Plan plan_at(unsigned char* base, int S) {
  Plan pl;
  pl.full = reinterpret_cast<int*>(base);
  pl.len = pl.full + S + 1;
  pl.first = reinterpret_cast<uint16_t*>(pl.len + S);
  pl.S = S;
  pl.n_full = pl.n_long = 0;
  return pl;
}

// Class of a partition 0 of `len` tokens (1 .. P): 0 (longest) ..
// kClasses-1; kClasses for an empty sequence (len 0).
__device__ inline int length_class(int len, int P) {
  if (len == 0) return kClasses;
  return (kClasses - 1) - (int)(((int64_t)(len - 1) * kClasses) / P);
}

__device__ inline uint64_t shfl_up_u64(uint64_t v, int o) {
  const int lo = __shfl_up((int)(uint32_t)v, o);
  const int hi = __shfl_up((int)(uint32_t)(v >> 32), o);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Builds the plan in LDS. Thread t takes the consecutive sequences
// [t K, t K + K); one block-wide exclusive scan of (full partitions, packed
// per-class counts) gives every sequence its entries. `xw` is LDS scratch
// for 2 * kWaves 64-bit values. Ends with a barrier.
__device__ void build_plan(const DecodeParams& p, Plan& pl, uint64_t* xw) {
  const int S = pl.S;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = (S + kThreads - 1) / kThreads;
  const int s0 = threadIdx.x * K;
  int a_of[kSeqsPerThread], c_of[kSeqsPerThread];
  int na = 0;
  uint64_t cls = 0;
  // every length this thread needs, loaded before any is used (in bounds:
  // sequence S-1 stands in for the ones past the end)
  int len_of[kSeqsPerThread];
#pragma unroll
  for (int k = 0; k < kSeqsPerThread; ++k) len_of[k] = p.seq_lens[min(s0 + k, S - 1)];
#pragma unroll
  for (int k = 0; k < kSeqsPerThread; ++k) {
    a_of[k] = c_of[k] = 0;
    const int s = s0 + k;
    if (k < K && s < S) {
      const int L = clamp_len(len_of[k], p.max_seq_len);
      pl.len[s] = L;
      if (L == 0) {
        c_of[k] = kClasses;
      } else {
        const Cut c = cut_of(L, p.partition);
        a_of[k] = c.n - 1;
        c_of[k] = length_class(c.r, p.partition);
      }
      na += a_of[k];
      cls += 1ull << (kClassBits * c_of[k]);
    }
  }
  uint64_t ia = (uint32_t)na, ic = cls;  // inclusive scans in the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t ta = shfl_up_u64(ia, o);
    const uint64_t tc = shfl_up_u64(ic, o);
    if (lane >= o) {
      ia += ta;
      ic += tc;
    }
  }
  if (lane == 63) {
    xw[2 * wave] = ia;
    xw[2 * wave + 1] = ic;
  }
  __syncthreads();
  uint64_t ba = 0, bc = 0, ta = 0, tc = 0;  // before this wave; totals
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint64_t xa = xw[2 * w], xc = xw[2 * w + 1];
    if (w < wave) {
      ba += xa;
      bc += xc;
    }
    ta += xa;
    tc += xc;
  }
  int pa = (int)(ba + ia) - na;
  const uint64_t pc = bc + ic - cls;
  int cbase[kClasses + 1];
  int run = 0;
#pragma unroll
  for (int c = 0; c <= kClasses; ++c) {
    cbase[c] = run + (int)((pc >> (kClassBits * c)) & ((1u << kClassBits) - 1));
    run += (int)((tc >> (kClassBits * c)) & ((1u << kClassBits) - 1));
  }
#pragma unroll
  for (int k = 0; k < kSeqsPerThread; ++k) {
    const int s = s0 + k;
    if (k < K && s < S) {
      pl.full[s] = pa;
      pa += a_of[k];
#pragma unroll
      for (int c = 0; c <= kClasses; ++c)
        if (c == c_of[k]) pl.first[cbase[c]++] = (uint16_t)s;
    }
  }
  if (threadIdx.x == 0) pl.full[S] = (int)ta;
  __syncthreads();
  pl.n_full = uniform(pl.full[S]);
  pl.n_long = pl.n_full + (int)(tc & ((1u << kClassBits) - 1));
}

// Entry e of the plan: (sequence, partition), both wave-uniform.
__device__ inline void plan_entry(const Plan& pl, int e, int& seq, int& part) {
  if (e < pl.n_full) {
    int lo = 0, hi = pl.S;  // full[lo] <= e < full[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (uniform(pl.full[mid]) <= e) lo = mid; else hi = mid;
    }
    seq = lo;
    part = uniform(pl.full[lo + 1]) - e;  // highest partition first
  } else {
    seq = uniform(pl.first[e - pl.n_full]);
    part = 0;
  }
}

// Entry e of the work list when it is a full partition of one of the first
// 64 sequences, or, in a launch that splits no sequence, one of the first 64
// sequences in the longest class (the list's order, without the list): each
// wave loads those lengths, one per lane, and an inclusive scan of their
// n_s - 1 gives full[s + 1]; the sequence is the first lane whose count
// exceeds e. False (and nothing set) when entry e lies further on. len: the
// sequence's length.
__device__ inline bool first_entry(const DecodeParams& p, int e, int& seq, int& part, int& len) {
  const int lane = threadIdx.x & 63;
  const int n = p.num_seqs < 64 ? p.num_seqs : 64;
  const int L = lane < n ? clamp_len(p.seq_lens[lane], p.max_seq_len) : 0;
  int incl = L > 0 ? cut_of(L, p.partition).n - 1 : 0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  const unsigned long long past = __ballot(incl > e);
  if (past != 0ull) {
    const int s = __ffsll((long long)past) - 1;
    seq = s;
    part = uniform(__shfl(incl, s)) - e;  // full[s + 1] - e: highest partition first
    len = uniform(__shfl(L, s));
    return true;
  }
  if (p.num_partitions != 1) return false;
  // No sequence is split: the list is the partitions 0 by class, and the
  // longest-class sequences among the first 64 are its first entries, in
  // batch order. Entry e is the one with e such sequences before it.
  const bool longest = L > 0 && length_class(cut_of(L, p.partition).r, p.partition) == 0;
  const unsigned long long m = __ballot(longest);
  const int before = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  const unsigned long long hit = __ballot(longest && before == e);
  if (hit == 0ull) return false;
  const int s = __ffsll((long long)hit) - 1;
  seq = s;
  part = 0;
  len = uniform(__shfl(L, s));
  return true;
}

// ---------------------------------------------------------------------------
// Schedule of one launch over a persistent grid of `grid` workgroups (a
// multiple of 8). Items below a split point are dealt statically in rounds of
// `grid`: workgroup b takes item b of round 0, and of each later round item b
// or, on odd rounds, item grid-1-b (alternating directions even out the
// long-first items). Workgroup b runs on XCD b mod 8, so with items numbered
// KV head fastest each XCD keeps to a fixed set of KV heads within a round,
// and the KV heads of the same tokens are worked on at the same time on
// different XCDs; on MI355X numbering the same work sequence-fastest instead
// is 8-20% slower, and a shared prompt's blocks are reused from the XCD's L2.
// The items from the split point on are taken one at a time from a counter,
// which evens out workgroups and XCDs that run at different speeds and
// items of different lengths. When nearly all entries are of the longest
// class (a batch of similar lengths) every item is dealt statically (kept on
// its XCD, which helps most when sequences share blocks); otherwise all
// items after the first round go through the counter.
// The counter is the low half of the workspace's control word (see take_ticket).

__device__ inline int static_end(int total, int grid, bool uniform_batch) {
  if (uniform_batch) return total;
  return total < grid ? total : grid;  // every workgroup's first item is static
}

// LDS budget of one workgroup when two share a CU (160 KiB each).
constexpr int kLdsPerWorkgroup = 80 * 1024;

// The launch's control word (the first 64-bit word of the workspace):
// (workgroups finished << 32) | items taken from the counter. It is zero when
// the launch starts and zero again when it ends, so the workspace needs
// zeroing once, before its first use, and every later launch on the same
// stream (a replayed graph included) finds it ready.
//
// Ticket for the next counter item: the low half of the word before this
// add.
__device__ inline int take_ticket(unsigned long long* word) {
  return (int)(uint32_t)atomicAdd(word, 1ull);
}

// Called once per workgroup by the thread that took its tickets, after its
// last take: counts the workgroup as finished, and the last of the grid sets
// the word back to zero. Every take and every finish is an atomic on this one
// word, and a thread's atomics on one location are ordered as the thread
// issued them; the last finisher has seen every other workgroup's finish, so
// every take precedes the reset.
__device__ inline void finish_launch(unsigned long long* word) {
  const unsigned long long old = atomicAdd(word, 1ull << 32);
  if ((uint32_t)(old >> 32) == gridDim.x - 1) atomicExch(word, 0ull);
}

// Control ints of a workgroup in LDS (next-item slots, merge flag, pending item).
constexpr int kCtlInts = 8;

// Partitions a merge reads per round trip.
constexpr int kMergeBatch = 8;

// LDS of the partition kernel: the partition's block-table slice and the
// waves' K tiles, reused for the waves' O rows (and at the start for the
// plan's scan); then the waves' (m, l); then the control ints; then the plan.
__host__ __device__ inline int bt_lds_bytes(int span, int BS) { return ((span / BS + 1) * 4 + 15) & ~15; }
// R: query rows per KV head (q_len * G); a wave keeps at most 16 of them.
__host__ __device__ inline int lds_main_bytes(int D, int R, int span, int BS, int kt_bytes) {
  const int o_bytes = kWaves * (R < 16 ? R : 16) * o_stride(D) * 4;
  const int tile_bytes = bt_lds_bytes(span, BS) + kWaves * kt_bytes;
  return ((o_bytes > tile_bytes ? o_bytes : tile_bytes) + 15) & ~15;
}
__host__ __device__ inline int lds_total_bytes(int D, int R, int span, int BS, int kt_bytes, int S) {
  return lds_main_bytes(D, R, span, BS, kt_bytes) + 2 * kWaves * 16 * 4 + 4 * kCtlInts + plan_bytes(S);
}

// LDS of one wave's share of the tile area for R query rows per KV head: its
// K reorder tile, or, with several column groups, a shared tile slot pair.
template <class Eng>
__host__ __device__ inline int wave_tile_bytes(int R) {
  if constexpr (Eng::kShared) {
    if (col_tiles(R) > 1) return Eng::KT_BYTES > 2 * Eng::SLOT_BYTES ? Eng::KT_BYTES : 2 * Eng::SLOT_BYTES;
  }
  return Eng::KT_BYTES;
}

// One work item: KV head kvh of partition `part` of sequence `seq`, by the
// whole workgroup. Waves take its 16-token tiles round-robin and merge
// (m, l, O) through LDS; a sequence in one partition is normalised and
// written to out. A partition of a split sequence writes its (m, l, O) to
// the workspace and arrives at the (sequence, KV head) word; the last to
// arrive merges every partition's partials and writes out. With `draw`,
// thread 0 takes a ticket from the counter for the workgroup's next item.
// Merge of the split (seq, kvh): run by the workgroup whose arrival
// completed the count. The partials are read with agent-scope atomic loads
// (sc1: from the level every XCD shares, never a stale line of this XCD's
// L2) and combined in partition order: M = max m_q, then the sums of
// 2^(m_q - M) l_q and 2^(m_q - M) O_q, the running max moved between batches
// of loads.
template <class Tag, int D>
__device__ __forceinline__ void merge_partials(const DecodeParams& p, int seq, int kvh, int nparts, int tid) {
  constexpr int DQ = D / 4;
  const int G = p.group;
  const int R = p.q_len * G;
  const int head0 = kvh * G;
  const int g_inv = (2048 + G - 1) / G;  // token of row c: (c * g_inv) >> 11, as in decode_item
  float v_scale = 1.0f;
  if constexpr (KV<Tag>::kF8) v_scale = p.v_scale[kvh];
  for (int qi = tid; qi < R * DQ; qi += kThreads) {
    const int r = qi / DQ;
    const int qd = qi - r * DQ;
    const int d = 4 * qd;
    const int j = (r * g_inv) >> 11;
    const size_t row = ((size_t)seq * p.q_len + j) * p.num_heads + head0 + (r - j * G);
    const unsigned long long* ml =
        reinterpret_cast<const unsigned long long*>(p.ws_ml + 2 * row * p.num_partitions);
    const unsigned long long* o =
        reinterpret_cast<const unsigned long long*>(p.ws_o + row * p.num_partitions * D + 2 * qd);
    // kMergeBatch partitions per round trip: every load of a batch (the
    // (m, l) pair and the quad of each partition) is issued before any is
    // used
    float M = kNoMax, den = 0.0f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = 0; q0 < nparts; q0 += kMergeBatch) {
      unsigned long long mlq[kMergeBatch], oa[kMergeBatch], ob[kMergeBatch];
      // one base per batch: the loads below take constant offsets from it
      const unsigned long long* mlb = ml + q0;
      const unsigned long long* ob0 = o + (size_t)q0 * (D / 2);
#pragma unroll
      for (int jj = 0; jj < kMergeBatch; ++jj) {
        mlq[jj] = pack2(kNoMax, 0.0f);
        oa[jj] = ob[jj] = 0ull;
        if (q0 + jj < nparts) {
          mlq[jj] = __hip_atomic_load(&mlb[jj], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          oa[jj] = __hip_atomic_load(&ob0[jj * (D / 2)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ob[jj] = __hip_atomic_load(&ob0[jj * (D / 2) + DQ], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      float cm = lo_of(mlq[0]);
#pragma unroll
      for (int jj = 1; jj < kMergeBatch; ++jj) cm = fmaxf(cm, lo_of(mlq[jj]));
      const float M_new = fmaxf(M, cm);
      const float alpha = fast_exp2(M - M_new);  // 0 for the first batch
      den *= alpha;
      num.x *= alpha;
      num.y *= alpha;
      num.z *= alpha;
      num.w *= alpha;
      M = M_new;
#pragma unroll
      for (int jj = 0; jj < kMergeBatch; ++jj) {
        const float wq = fast_exp2(lo_of(mlq[jj]) - M);
        den += wq * hi_of(mlq[jj]);
        num.x += wq * lo_of(oa[jj]);
        num.y += wq * hi_of(oa[jj]);
        num.z += wq * lo_of(ob[jj]);
        num.w += wq * hi_of(ob[jj]);
      }
    }
    // num / den per element (times the V scale of an e4m3 pool), as for an
    // unsplit row; 0 for a row that saw no position
    float4 out = make_float4(0.f, 0.f, 0.f, 0.f);
    if (den > 0.0f) {
      out = make_float4(num.x / den, num.y / den, num.z / den, num.w / den);
      if constexpr (KV<Tag>::kF8) {
        out.x *= v_scale;
        out.y *= v_scale;
        out.z *= v_scale;
        out.w *= v_scale;
      }
    }
    store_out4<Tag>(p, row * D + d, out);
    if (p.lse && d == 0) p.lse[row] = lse_of(M, den);
  }
}

template <class Tag, int D, int BS, bool SH>
__device__ __forceinline__ void decode_item(const DecodeParams& p, unsigned char* smem, int lds_main,
                                            int seq, int L, int kvh, int part, int tid, int wave,
                                            bool draw, int& ticket) {
  const int lane = tid & 63;
  using Eng = TileEngine<Tag, D, BS>;
  constexpr int RB = Eng::RB;
  constexpr int DQ = D / 4;  // quads (4 consecutive head-dim elements) per row
  const int G = p.group;
  const int R = p.q_len * G;  // query rows of this KV head: (token j, head g) -> j * G + g
  const int head0 = kvh * G;
  // new token of query row c, c / G, as a multiply and a shift (exact for
  // every c < 128 and G <= 16): no division before the query load of an item
  const int g_inv = (2048 + G - 1) / G;
  auto token_of = [&](int c) { return (c * g_inv) >> 11; };
  // global row of query row c: [S, q_len, H] flattened
  auto row_of = [&](int c) -> size_t {
    const int j = token_of(c);
    return ((size_t)seq * p.q_len + j) * p.num_heads + head0 + (c - j * G);
  };

  if (L == 0) {  // nothing to attend to: zero rows
    if (draw && tid == 0) ticket = take_ticket(p.work);
    for (int qi = tid; qi < R * DQ; qi += kThreads) {
      const int r = qi / DQ;
      store_out4<Tag>(p, row_of(r) * D + 4 * (qi - r * DQ), make_float4(0.f, 0.f, 0.f, 0.f));
      if (p.lse && qi - r * DQ == 0) p.lse[row_of(r)] = kNoMax;
    }
    return;
  }
  const Cut c = cut_of(L, p.partition);
  const int nparts = c.n;
  const int t_begin = part == 0 ? 0 : c.r + (part - 1) * p.partition;
  const int t_end = min(L, part == 0 ? c.r : t_begin + p.partition);
  if (t_begin >= t_end) {  // only for a seq_lens entry changed under the launch
    if (draw && tid == 0) ticket = take_ticket(p.work);
    return;
  }

  // Column groups: with more than 16 query rows the rows are cut into tiles
  // of 16 MFMA columns and the waves into as many groups; the waves of group
  // g keep rows 16 g .. 16 g + 15 and share out the key tiles among
  // themselves, so every group reads every key tile (once from HBM, then
  // from L2: those loads are cached).
  const int nct = col_tiles(R);
  const int wpg = kWaves / nct;  // waves per group
  const int cgroup = wave / wpg;
  const int wi = wave - cgroup * wpg;
  const int RW = R < 16 ? R : 16;  // rows per wave
  Eng eng;
  eng.init(lane);
  const int myrow = 16 * cgroup + eng.col;
  const bool valid = myrow < R;

  // ---- stage this partition's slice of the block-table row --------------
  // Every global load of the item's start (the query rows, the slice, the
  // neighbours' entries of the caching guess below) is issued, unconditional
  // and in bounds, before any of them is used: the start costs one round
  // trip to memory instead of one per dependent load.
  eng.load_q(static_cast<const unsigned char*>(p.q) + row_of(valid ? myrow : 0) * Eng::QB, valid);
  int* s_bt = reinterpret_cast<int*>(smem);
  const int lb0 = t_begin / BS;
  const int nlb = (t_end + BS - 1) / BS - lb0;  // >= 1
  const int32_t* row = p.block_table + (size_t)seq * p.max_blocks + lb0;
  const int32_t* prev = seq > 0 ? row - p.max_blocks : row;
  const int32_t* next = seq + 1 < p.num_seqs ? row + p.max_blocks : row;
  const int e0 = row[tid < nlb ? tid : nlb - 1];
  const int b0 = row[0];
  const int bprev = prev[0];
  const int bnext = next[0];
  eng.lim = valid && p.causal ? L - p.q_len + token_of(myrow) : L - 1;
  eng.reset();
  // A split item of this workgroup that has not yet arrived (the pending
  // item, recorded in ctl[4..6] at the end of that item): its partial stores
  // were issued then; waiting for them here costs nothing beyond the start's
  // own round trip, which is in flight with them.
  int* ctl = reinterpret_cast<int*>(smem + lds_main + 2 * kWaves * 16 * 4);
  const int pseq0 = uniform(ctl[4]);
  const int pkvh0 = uniform(ctl[5]);
  if (pseq0 >= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (tid < nlb) s_bt[tid] = ((unsigned)e0 < (unsigned)p.num_blocks) ? e0 : 0;  // never leave the pool
  for (int i = tid + kThreads; i < nlb; i += kThreads) {
    const int b = row[i];
    s_bt[i] = ((unsigned)b < (unsigned)p.num_blocks) ? b : 0;
  }
  // Blocks shared with the neighbouring sequences of the batch (samples
  // forked from one prompt sit next to each other) are read with caching
  // loads so that the neighbours find them in L2; everything else streams
  // with non-temporal loads. Only the speed depends on this guess.
  const bool shared = (seq > 0 && bprev == b0) || (seq + 1 < p.num_seqs && bnext == b0);
  __syncthreads();
  // every thread's stores of the pending item are acknowledged: it arrives
  // now, and the count comes back while the tiles stream
  uint32_t pdone = 0;
  if (pseq0 >= 0 && tid == 0)
    pdone = __hip_atomic_fetch_add(p.arrive + (size_t)pseq0 * p.num_kv_heads + pkvh0, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);

  unsigned char* kt = smem + bt_lds_bytes(p.partition < p.max_seq_len ? p.partition : p.max_seq_len, BS) +
                     wave * Eng::KT_BYTES;
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
  // e4m3 pools: the KV head's K scale multiplies every score, its V scale
  // the output (applied once, after the weighted sums)
  float scale_log2 = p.scale_log2;
  float v_scale = 1.0f;
  if constexpr (Eng::kF8) {
    scale_log2 *= p.k_scale[kvh];
    v_scale = p.v_scale[kvh];
  }
  // the loop is compiled four ways (load kind x causal limit), chosen per item
  auto tiles = [&](auto nt, auto causal) {
    constexpr bool NT = decltype(nt)::value;
    constexpr bool CAUSAL = decltype(causal)::value;
    if constexpr (Eng::kPipe) {
      // The wave's tiles through its two LDS buffers: tile k is read into
      // registers as soon as its rows have landed, then the loads of tile k+1
      // (issue_shared: global_load_lds, no registers held) are issued into
      // the other buffer, and tile k's math runs while they stream.
      constexpr int TB = 2 * Eng::SLOT_BYTES;  // one buffer: K rows, then V rows
      const int stride = wpg * kTile;
      int cs = t_begin + wi * kTile;
      if (cs < t_end) eng.template issue_shared<NT>(kt, kt + Eng::SLOT_BYTES, kbase, vbase, cs, t_end - 1, row_off);
      for (int b = 0; cs < t_end; cs += stride, b ^= 1) {
        unsigned char* cur = kt + b * TB;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile k's rows are in LDS
        typename Eng::Tile g;
        eng.fetch_shared(g, cur, cur + Eng::SLOT_BYTES);
        if (cs + stride < t_end) {
          unsigned char* nx = kt + (b ^ 1) * TB;
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every read of the buffers so far is done
          eng.template issue_shared<NT>(nx, nx + Eng::SLOT_BYTES, kbase, vbase, cs + stride, t_end - 1, row_off);
        }
        eng.template consume<CAUSAL, true>(g, cs, t_end - 1, scale_log2, nullptr);
      }
    } else {
      for (int cs = t_begin + wi * kTile; cs < t_end; cs += wpg * kTile)
        eng.template step<NT, CAUSAL>(kbase, vbase, cs, t_end - 1, slot_bytes, scale_log2, row_off, kt);
    }
  };
  using Yes = std::true_type;
  using No = std::false_type;
  // several column groups: every key and value tile loaded once into the
  // tile slots in LDS and read from there by one wave of every group.
  //  * 16-bit pools with two groups: rounds of kWaves / 2 tiles (the K rows
  //    of tile i of the round loaded by wave i, its V rows by wave
  //    i + kWaves / 2); the slots hold two rounds, the next streaming into
  //    one half while this one is worked on; one barrier per round.
  //  * otherwise: rounds of kWaves tiles (wave w loads tile w of the round),
  //    barriers around the loads of each round (measured faster there:
  //    e4m3 tiles are half the bytes, and four or more groups do more math
  //    per tile).
  auto shared_tiles = [&](auto nt, auto causal) {
    if constexpr (SH && Eng::kShared) {
      constexpr bool NT = decltype(nt)::value;
      constexpr bool CAUSAL = decltype(causal)::value;
      constexpr int TS = 2 * Eng::SLOT_BYTES;  // one tile: K rows, then V rows
      unsigned char* slots = smem + bt_lds_bytes(p.partition < p.max_seq_len ? p.partition : p.max_seq_len, BS);
      const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
      if (!Eng::kF8 && nct == 2) {
        constexpr int RT = kWaves / 2;  // tiles per round
        const int half = wave / RT;     // 0: K rows, 1: V rows
        const int mine = wave - half * RT;
        auto issue = [&](int r0) {  // the round of tiles r0 .. r0 + RT - 1
          if (r0 + mine < ntiles)
            eng.template issue_half<NT>(slots + (((r0 / RT) & 1) * RT + mine) * TS + half * Eng::SLOT_BYTES,
                                        half ? vbase : kbase, t_begin + (r0 + mine) * kTile, t_end - 1, row_off);
        };
        issue(0);
        for (int r0 = 0; r0 < ntiles; r0 += RT) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of the round
          __syncthreads();  // every wave's; and every wave is done with the other half
          if (r0 + RT < ntiles) issue(r0 + RT);
          const unsigned char* buf = slots + ((r0 / RT) & 1) * RT * TS;
          for (int k = wi; k < RT && r0 + k < ntiles; k += wpg) {
            typename Eng::Tile g;
            eng.fetch_unseen(g, buf + k * TS, buf + k * TS + Eng::SLOT_BYTES);
            eng.template consume<CAUSAL, true>(g, t_begin + (r0 + k) * kTile, t_end - 1, scale_log2, nullptr);
          }
        }
      } else {
        for (int r0 = 0; r0 < ntiles; r0 += kWaves) {
          __syncthreads();  // every wave is done with the previous round's slots
          if (r0 + wave < ntiles)
            eng.template issue_shared<NT>(slots + wave * TS, slots + wave * TS + Eng::SLOT_BYTES, kbase, vbase,
                                          t_begin + (r0 + wave) * kTile, t_end - 1, row_off);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          for (int k = wi; k < kWaves && r0 + k < ntiles; k += wpg) {
            typename Eng::Tile g;
            eng.fetch_shared(g, slots + k * TS, slots + k * TS + Eng::SLOT_BYTES);
            eng.template consume<CAUSAL, true>(g, t_begin + (r0 + k) * kTile, t_end - 1, scale_log2, nullptr);
          }
        }
      }
    }
  };
  const bool causal_rows = p.q_len > 1 && p.causal;
  if (SH && Eng::kShared && nct > 1) {
    if (shared) {
      if (causal_rows) shared_tiles(No{}, Yes{}); else shared_tiles(No{}, No{});
    } else {
      if (causal_rows) shared_tiles(Yes{}, Yes{}); else shared_tiles(Yes{}, No{});
    }
  } else {
    const bool cached = shared || nct > 1;
    if (!causal_rows) {
      if (cached) tiles(No{}, No{}); else tiles(Yes{}, No{});
    } else {
      if (cached) tiles(No{}, Yes{}); else tiles(Yes{}, Yes{});
    }
  }

  // ---- merge the waves ---------------------------------------------------
  const float lsum = eng.total_sum();
  __syncthreads();  // block-table slice no longer needed: reuse its LDS
  // Every wave is done with its tiles: a workgroup in the dynamic part of the
  // schedule draws the ticket for its next item now, while it merges, so that
  // items taken one after the other (the KV heads of the same tokens) start
  // close together in time.
  if (draw && tid == 0) ticket = take_ticket(p.work);
  // the pending item's count: the partition that completes it merges. The
  // record is read here, before the barrier below, so that thread 0 may
  // rewrite it at the end of this item.
  const int pseq = uniform(ctl[4]);
  const int pkvh = uniform(ctl[5]);
  const int pn = uniform(ctl[6]);
  if (pseq >= 0 && tid == 0) {
    const bool last = pdone == (uint32_t)(pn - 1);
    if (last)  // every other partition has arrived: ready for the next launch
      __hip_atomic_store(p.arrive + (size_t)pseq * p.num_kv_heads + pkvh, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    ctl[2] = last;
  }
  // num / den per element (times the V scale of an e4m3 pool); 0 for a row
  // that saw no position
  auto finish = [&](float4 num, float den) -> float4 {
    if (!(den > 0.0f)) return make_float4(0.f, 0.f, 0.f, 0.f);
    float4 o = make_float4(num.x / den, num.y / den, num.z / den, num.w / den);
    if constexpr (Eng::kF8) {
      o.x *= v_scale;
      o.y *= v_scale;
      o.z *= v_scale;
      o.w *= v_scale;
    }
    return o;
  };
  const int OST = o_stride(D);
  float* s_o = reinterpret_cast<float*>(smem);
  float* s_m = reinterpret_cast<float*>(smem + lds_main);
  float* s_l = s_m + kWaves * 16;
  if (valid && eng.grp == 0) {
    s_m[wave * 16 + eng.col] = eng.m;
    s_l[wave * 16 + eng.col] = lsum;
  }
  eng.write_o(s_o + (size_t)(wave * RW) * OST, OST, valid);
  __syncthreads();

  // One quad of one row per thread and pass: the group's waves combined with
  // one scale factor per wave. Straight-line code (a wave past the group's
  // end is read at the group's first and weighted 0), so that every LDS read
  // of the pass is issued at once.
  for (int qi = tid; qi < R * DQ; qi += kThreads) {
    const int r = qi / DQ;
    const int qd = qi - r * DQ;  // quad within the row
    const int d = 4 * qd;
    const int col = r & 15;
    const int w0 = (r >> 4) * wpg;
    float mw[kWaves], lw[kWaves];
    float4 ow[kWaves];
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int w = w0 + (i < wpg ? i : 0);
      mw[i] = s_m[w * 16 + col];
      lw[i] = s_l[w * 16 + col];
      ow[i] = *reinterpret_cast<const float4*>(s_o + (size_t)(w * RW + col) * OST + d);
    }
    float M = kNoMax;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) M = fmaxf(M, mw[i]);  // repeats change nothing
    float den = 0.0f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const float sc = i < wpg ? fast_exp2(mw[i] - M) : 0.0f;
      den += sc * lw[i];
      num.x += sc * ow[i].x;
      num.y += sc * ow[i].y;
      num.z += sc * ow[i].z;
      num.w += sc * ow[i].w;
    }
    const size_t row = row_of(r);
    if (nparts <= 1) {
      store_out4<Tag>(p, row * D + d, finish(num, den));
      if (p.lse && d == 0) p.lse[row] = lse_of(M, den);
    } else {
      // agent-scope stores: written through to where every XCD reads them.
      // A partial's D values are kept as its quads' (0, 1) pairs, then their
      // (2, 3) pairs, so that each store (and each load of the merge) of the
      // wave covers contiguous memory.
      const size_t pi = row * p.num_partitions + part;
      unsigned long long* o2 = reinterpret_cast<unsigned long long*>(p.ws_o + pi * D + 2 * qd);
      __hip_atomic_store(o2, pack2(num.x, num.y), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(o2 + DQ, pack2(num.z, num.w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0)
        __hip_atomic_store(reinterpret_cast<unsigned long long*>(p.ws_ml + 2 * pi), pack2(M, den),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the pending item's merge, when its arrival completed the count
  if (pseq >= 0 && ctl[2]) merge_partials<Tag, D>(p, pseq, pkvh, pn, tid);
  // This item's partials are in flight: it becomes the pending item and
  // arrives at the start of the workgroup's next item (or at the end of the
  // pass). Every wave read the old record before the last barrier.
  if (tid == 0) {
    ctl[4] = nparts > 1 ? seq : -1;
    ctl[5] = kvh;
    ctl[6] = nparts;
  }
}

// Arrival of the workgroup's pending item at the end of a pass (see
// decode_item), and its merge when that completes the count.
//
// Publication of the partials across XCDs (each XCD has its own L2): the
// partials are agent-scope atomic stores, which gfx950 issues with the sc1
// bit, written through to the level all XCDs share (LLVM AMDGPUUsage,
// memory model for GFX942 and later: "store atomic monotonic agent" is a
// global_store with sc1); every thread's s_waitcnt vmcnt(0) waits until its
// stores are acknowledged by that level; after a workgroup barrier, thread
// 0 arrives with an agent-scope atomic add on the (seq, kvh) word (performed
// at the same level); the partition that sees the count reach nparts - 1
// reads the partials with agent-scope atomic loads (sc1: served from the
// shared level). So every partial is complete where the merger reads it
// before the merger can see the count. (The language-level alternative, an
// agent-scope release fence before the arrival and an acquire fence in the
// merger, adds an L2-wide write-back and invalidate per partition: measured
// 151.7 vs 102.9 us on the Llama-3-8B-shaped batch, 576 vs 293 us on the
// mixed batch at 512-token partitions.) The merging partition sets the word
// back to zero for the next launch: every other partition's add precedes
// it (atomics on one location, the count seen complete).
template <class Tag, int D>
__device__ __forceinline__ void arrive_pending(const DecodeParams& p, int* ctl) {
  const int pseq = uniform(ctl[4]);
  if (pseq < 0) return;
  const int pkvh = uniform(ctl[5]);
  const int pn = uniform(ctl[6]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* word = p.arrive + (size_t)pseq * p.num_kv_heads + pkvh;
    const uint32_t done = __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = done == (uint32_t)(pn - 1);
    if (last) __hip_atomic_store(word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ctl[2] = last;
    ctl[4] = -1;
  }
  __syncthreads();
  if (ctl[2]) merge_partials<Tag, D>(p, pseq, pkvh, pn, (int)threadIdx.x);
}

// The items of one pass (a launch's work list `pl` over the parameters p),
// taken in turn by this workgroup: from item b of a static first round
// (then static rounds or counter tickets, as above), or, with `dynamic`,
// every item from the counter. `parity` alternates the two next-item slots
// across passes.
template <class Tag, int D, int BS, bool SH>
__device__ __forceinline__ void run_items(const DecodeParams& p, const Plan& pl, unsigned char* smem, int lds_main,
                                          int* s_next, int wave, bool dynamic, bool first_done, int& parity) {
  const int hkv = p.num_kv_heads;
  const int entries = pl.n_full + pl.S;
  const int total = entries * hkv;
  const int grid = (int)gridDim.x;
  const int ws = dynamic ? 0 : static_end(total, grid, 8 * pl.n_long >= 7 * entries);
  const int b = (int)blockIdx.x;
  int w = b;
  int round = 0;  // static round of the current item
  if (first_done) {  // this workgroup's item of round 0 is done: round 1 next
    round = 1;
    w = 2 * grid - 1 - b;
  }
  if (dynamic || (first_done && w >= ws)) {
    if (threadIdx.x == 0) {
      const int t = take_ticket(p.work);
      const int64_t nx = (int64_t)(dynamic ? 0 : ws) + t;
      s_next[parity] = (nx >= 0 && nx < total) ? (int)nx : total;
    }
    __syncthreads();
    w = uniform(s_next[parity]);
    parity ^= 1;
  }
  for (; (unsigned)w < (unsigned)total; parity ^= 1) {
    const int e = w / hkv;
    const int kvh = w - e * hkv;
    int seq, part;
    plan_entry(pl, e, seq, part);
    ++round;
    const int nxt_static = round * grid + ((round & 1) ? grid - 1 - b : b);
    const bool draw = w >= ws || nxt_static >= ws;  // the next item is a counter one
    int ticket = 0;
    // The thread index passes through an empty asm statement so that the
    // lane-dependent addressing is recomputed per item instead of being
    // hoisted out of this loop and held in registers across the tiles.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    decode_item<Tag, D, BS, SH>(p, smem, lds_main, seq, uniform(pl.len[seq]), kvh, part, tid, wave, draw,
                                    ticket);
    if (threadIdx.x == 0) {
      const int64_t nx = !draw ? (int64_t)nxt_static : (int64_t)ws + ticket;
      s_next[parity] = (nx >= 0 && nx < total) ? (int)nx : total;
    }
    __syncthreads();
    w = uniform(s_next[parity]);
  }
  arrive_pending<Tag, D>(p, s_next);
}

// Persistent: a grid of as many workgroups as fit on the GPU at once (a
// multiple of 8), each working through its items of the schedule above. A
// workgroup whose next item is a counter one draws a ticket while it merges
// its current item; every ticket advances the counter, so every workgroup
// ends. The last workgroup to end sets the control word back to zero. WIDE:
// compiled with the tiles shared by column groups (more than 16 query rows
// per KV head); the other instance leaves that code out.
template <class Tag, int D, int BS, bool WIDE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WavesPerEU<Tag, D>::value)))
void decode_partition_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = uniform(threadIdx.x >> 6);
  const int span = p.partition < p.max_seq_len ? p.partition : p.max_seq_len;
  const int lds_main = lds_main_bytes(D, p.q_len * p.group, span, BS,
                                      wave_tile_bytes<TileEngine<Tag, D, BS>>(p.q_len * p.group));
  // Control ints: two slots for the next item, used alternately (an item
  // may pass no barrier (a zero-length sequence), and a slot is rewritten
  // only after the barrier that follows every wave's read of it); the merge
  // flag; the pending item (sequence or -1, KV head, partitions).
  int* s_next = reinterpret_cast<int*>(smem + lds_main + 2 * kWaves * 16 * 4);
  // (written by every wave for itself: the first item reads it before any
  // barrier)
  if ((threadIdx.x & 63) == 0) s_next[4] = -1;
  // A first item that first_entry finds needs only the first 64 lengths,
  // not the work list: it starts streaming right away, and the list is
  // built after it (while the other workgroup on the CU streams).
  int seq0, part0, len0;
  const int e0 = (int)blockIdx.x / p.num_kv_heads;
  const bool first = first_entry(p, e0, seq0, part0, len0);
  if (first) {
    const int kvh = (int)blockIdx.x - e0 * p.num_kv_heads;
    int ticket = 0;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    decode_item<Tag, D, BS, WIDE>(p, smem, lds_main, seq0, len0, kvh, part0, tid, wave, false, ticket);
    __syncthreads();  // the list's scan reuses the item's LDS
  }
  Plan pl = plan_at(reinterpret_cast<unsigned char*>(s_next + kCtlInts), p.num_seqs);
  build_plan(p, pl, reinterpret_cast<uint64_t*>(smem));
  int parity = 0;
  run_items<Tag, D, BS, WIDE>(p, pl, smem, lds_main, s_next, wave, false, first, parity);
  if (threadIdx.x == 0) finish_launch(p.work);  // after the workgroup's last ticket
}

// LDS of a two-pass launch: the larger main area of the two passes, then the
// (m, l) slots and next-item slots, then both work lists.
template <class EngA, class EngB>
__host__ __device__ inline int pair_lds_main(int D, int BS, const DecodeParams& a, const DecodeParams& b) {
  const int la = lds_main_bytes(D, a.q_len * a.group, a.partition < a.max_seq_len ? a.partition : a.max_seq_len,
                                BS, EngA::KT_BYTES);
  const int lb = lds_main_bytes(D, b.q_len * b.group, b.partition < b.max_seq_len ? b.partition : b.max_seq_len,
                                BS, EngB::KT_BYTES);
  return la > lb ? la : lb;
}

// Two passes over the same pools in one launch (shared-prefix decode: the
// groups' prefixes, then the samples' own blocks). Every workgroup works
// through the first pass's items as the partition kernel does, then takes
// the second pass's items from that pass's own counter, so the first pass's
// ramp-down is filled with the second pass's (short) items instead of
// ending the launch. Each pass has its own control word, work list and
// split-K workspace.
template <class Tag, int D, int BS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WavesPerEU<Tag, D>::value)))
void decode_pair_kernel(DecodeParams p0, DecodeParams p1) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int wave = uniform(threadIdx.x >> 6);
  const int lds_main = pair_lds_main<TileEngine<Tag, D, BS>, TileEngine<Tag, D, BS>>(D, BS, p0, p1);
  int* s_next = reinterpret_cast<int*>(smem + lds_main + 2 * kWaves * 16 * 4);
  if (threadIdx.x == 0) s_next[4] = -1;  // no pending item (seen after the plans' barriers)
  unsigned char* plans = reinterpret_cast<unsigned char*>(s_next + kCtlInts);
  Plan pl0 = plan_at(plans, p0.num_seqs);
  Plan pl1 = plan_at(plans + plan_bytes(p0.num_seqs), p1.num_seqs);
  build_plan(p0, pl0, reinterpret_cast<uint64_t*>(smem));
  build_plan(p1, pl1, reinterpret_cast<uint64_t*>(smem));
  int parity = 0;
  // (the shared tile slots are left to the single-pass kernel: two passes'
  // worth of tile loops in one kernel would spill registers)
  run_items<Tag, D, BS, false>(p0, pl0, smem, lds_main, s_next, wave, false, false, parity);
  run_items<Tag, D, BS, false>(p1, pl1, smem, lds_main, s_next, wave, true, false, parity);
  if (threadIdx.x == 0) {  // after the workgroup's last ticket of each pass
    finish_launch(p0.work);
    finish_launch(p1.work);
  }
}

// ============================================================================
// launchers
// ============================================================================

// Workgroups of the partition kernel that fit on the device at once (the
// persistent grid), cached per (device, kernel, LDS bytes).
int resident_workgroups(const void* kernel, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  struct Entry { int dev; const void* k; size_t lds; int n; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  {
    std::lock_guard<std::mutex> g(mu);
    for (const Entry& c : cache)
      if (c.dev == dev && c.k == kernel && c.lds == lds) return c.n;
  }
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kThreads, lds) != hipSuccess || per <= 0)
    per = 1;
  const int n = cus * per;
  std::lock_guard<std::mutex> g(mu);
  cache.push_back(Entry{dev, kernel, lds, n});
  return n;
}

template <class Tag, int D, int BS, bool WIDE>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  using Eng = TileEngine<Tag, D, BS>;
  const int span = p.partition < p.max_seq_len ? p.partition : p.max_seq_len;
  const void* kfn = reinterpret_cast<const void*>(&decode_partition_kernel<Tag, D, BS, WIDE>);
  const size_t q_row = (size_t)p.q_len * p.num_heads * D;  // elements per sequence
  const size_t q_elem = (size_t)KV<Tag>::kQBytes;  // the output, unless fp32, has the query's type
  const size_t out_elem = p.out_f32 ? 4 : q_elem;
  // Launches of at most `chunk` sequences each, in order on the stream; they
  // share the workspace (header, partials, arrival words). The chunk keeps the LDS of a
  // workgroup (its plan grows with the sequences) within half a CU's 160 KiB,
  // so that two workgroups fit per CU, when the rest of it leaves room.
  int chunk = kMaxSeqsPerLaunch;
  {
    const int fixed = lds_total_bytes(D, p.q_len * p.group, span, BS, wave_tile_bytes<Eng>(p.q_len * p.group), 0);
    const int room = (kLdsPerWorkgroup - fixed - 32) / 10;
    if (room < chunk) chunk = room > 256 ? room : 256;
  }
  for (int s0 = 0; s0 < p.num_seqs; s0 += chunk) {
    DecodeParams c = p;
    c.num_seqs = p.num_seqs - s0 < chunk ? p.num_seqs - s0 : chunk;
    c.q = static_cast<const unsigned char*>(p.q) + (size_t)s0 * q_row * q_elem;
    c.out = static_cast<unsigned char*>(p.out) + (size_t)s0 * q_row * out_elem;
    if (p.lse) c.lse = p.lse + (size_t)s0 * p.q_len * p.num_heads;
    c.block_table = p.block_table + (size_t)s0 * p.max_blocks;
    c.seq_lens = p.seq_lens + s0;
    const size_t lds =
        (size_t)lds_total_bytes(D, c.q_len * c.group, span, BS, wave_tile_bytes<Eng>(c.q_len * c.group), c.num_seqs);
    const int64_t max_items = (int64_t)c.num_seqs * c.num_kv_heads * c.num_partitions;
    int64_t grid = resident_workgroups(kfn, lds);
    if (grid > max_items) grid = max_items;
    if (grid >= 8) grid = grid / 8 * 8;  // whole rounds over the 8 XCDs
    hipEvent_t ev0 = s0 == 0 ? start : nullptr;                 // the first launch's start
    hipEvent_t ev1 = s0 + c.num_seqs >= p.num_seqs ? stop : nullptr;  // the last one's end
    if (ev0 || ev1)
      hipExtLaunchKernelGGL(decode_partition_kernel<Tag, D, BS, WIDE>, dim3((unsigned)grid), dim3(kThreads),
                            (uint32_t)lds, stream, ev0, ev1, 0u, c);
    else
      decode_partition_kernel<Tag, D, BS, WIDE><<<dim3((unsigned)grid), dim3(kThreads), lds, stream>>>(c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Two passes in one launch when both fit one launch's work list and LDS
// budget; hipErrorNotSupported otherwise (the caller then runs them one
// after the other).
template <class Tag, int D, int BS>
hipError_t launch_pair_t(DecodeParams a, DecodeParams b, hipStream_t stream) {
  if (a.num_seqs > kMaxSeqsPerLaunch || b.num_seqs > kMaxSeqsPerLaunch) return hipErrorNotSupported;
  const size_t lds = (size_t)pair_lds_main<TileEngine<Tag, D, BS>, TileEngine<Tag, D, BS>>(D, BS, a, b) +
                     2 * kWaves * 16 * 4 + 4 * kCtlInts + plan_bytes(a.num_seqs) +
                     plan_bytes(b.num_seqs);
  if (lds > (size_t)kLdsPerWorkgroup) return hipErrorNotSupported;
  const void* kfn = reinterpret_cast<const void*>(&decode_pair_kernel<Tag, D, BS>);
  const int64_t max_items = (int64_t)a.num_seqs * a.num_kv_heads * a.num_partitions +
                            (int64_t)b.num_seqs * b.num_kv_heads * b.num_partitions;
  int64_t grid = resident_workgroups(kfn, lds);
  if (grid > max_items) grid = max_items;
  if (grid >= 8) grid = grid / 8 * 8;
  decode_pair_kernel<Tag, D, BS><<<dim3((unsigned)grid), dim3(kThreads), lds, stream>>>(a, b);
  return hipGetLastError();
}

template <class Tag, int D>
hipError_t launch_pair_bs(const DecodeParams& a, const DecodeParams& b, int bs, hipStream_t stream) {
  switch (bs) {
    case 8: return launch_pair_t<Tag, D, 8>(a, b, stream);
    case 16: return launch_pair_t<Tag, D, 16>(a, b, stream);
    case 32: return launch_pair_t<Tag, D, 32>(a, b, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class Tag>
hipError_t launch_pair_d(const DecodeParams& a, const DecodeParams& b, int d, int bs, hipStream_t stream) {
  switch (d) {
    case 64: return launch_pair_bs<Tag, 64>(a, b, bs, stream);
    case 128: return launch_pair_bs<Tag, 128>(a, b, bs, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class Tag, int D>
hipError_t launch_bs(const DecodeParams& p, int bs, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  // more than 16 query rows per KV head: the instance with the tiles shared
  // by its column groups; decode and up to 16 rows run an instance without
  // that code
  const bool wide = col_tiles(p.q_len * p.group) > 1;
  switch (bs) {
    case 8: return wide ? launch_t<Tag, D, 8, true>(p, stream, start, stop)
                        : launch_t<Tag, D, 8, false>(p, stream, start, stop);
    case 16: return wide ? launch_t<Tag, D, 16, true>(p, stream, start, stop)
                         : launch_t<Tag, D, 16, false>(p, stream, start, stop);
    case 32: return wide ? launch_t<Tag, D, 32, true>(p, stream, start, stop)
                         : launch_t<Tag, D, 32, false>(p, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}

template <class Tag>
hipError_t launch_d(const DecodeParams& p, int d, int bs, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  switch (d) {
    case 64: return launch_bs<Tag, 64>(p, bs, stream, start, stop);
    case 128: return launch_bs<Tag, 128>(p, bs, stream, start, stop);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int kv_dtype, int query_dtype, int head_dim,
                         int block_size, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  switch (kv_dtype) {
    case 0: return launch_d<F32Tag>(p, head_dim, block_size, stream, start, stop);
    case 1: return launch_d<F16Tag>(p, head_dim, block_size, stream, start, stop);
    case 2: return launch_d<BF16Tag>(p, head_dim, block_size, stream, start, stop);
    case 3:
      if (query_dtype == 1) return launch_d<E4M3F16Tag>(p, head_dim, block_size, stream, start, stop);
      if (query_dtype == 2) return launch_d<E4M3BF16Tag>(p, head_dim, block_size, stream, start, stop);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_pair(const DecodeParams& a, const DecodeParams& b, int kv_dtype, int query_dtype,
                              int head_dim, int block_size, hipStream_t stream) {
  switch (kv_dtype) {
    case 0: return launch_pair_d<F32Tag>(a, b, head_dim, block_size, stream);
    case 1: return launch_pair_d<F16Tag>(a, b, head_dim, block_size, stream);
    case 2: return launch_pair_d<BF16Tag>(a, b, head_dim, block_size, stream);
    case 3:
      if (query_dtype == 1) return launch_pair_d<E4M3F16Tag>(a, b, head_dim, block_size, stream);
      if (query_dtype == 2) return launch_pair_d<E4M3BF16Tag>(a, b, head_dim, block_size, stream);
      return hipErrorNotSupported;
    default: return hipErrorNotSupported;
  }
}

}  // namespace pkv
