"""FP8 (e4m3) KV cache: the quantising scatter and attention over the
quantised pool, plain and slow (test infrastructure; only tests, smoke() and
bench's cpu_baseline leg may use it).

"LLM inference optimisation in practice" (section 6.2) names KV-cache
quantisation: attention computed on low-precision K and V, with almost no
loss of accuracy and a matching saving of memory and bandwidth. The page
fixes neither the format nor the scaling; the readings taken here:

  * format: OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 holds the subnormals m * 2^-9; the code with
    all exponent and mantissa bits set is NaN; there is no infinity; the
    largest finite value is 448;
  * one fp32 scale per KV head for K and one for V, given by the caller; a
    stored code c stands for value(c) * scale;
  * quantising x: the quotient x / scale is formed in fp32 (as a kernel
    forms it: fp32 division, round to nearest even), then rounded to the
    nearest e4m3 value, ties to the even code, magnitudes above 448
    saturating to 448 and NaN staying NaN;
  * the query stays in its 16-bit type; attention is the decode (or
    multi-query) of the paged_attention module over the dequantised pool.

The value table is built from the format's definition; encoding searches it
for the nearest value (a different route from any bit manipulation).
"""

from __future__ import annotations

import numpy as np
import torch

from .paged_attention import decode, decode_shared_prefix, multi_query

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_value_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_value_table()
_POS = _TABLE[:0x7F]          # codes 0 .. 126: the non-negative finite values, ascending


def e4m3_decode(codes) -> np.ndarray:
    """Codes (uint8, any shape) -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x32) -> np.ndarray:
    """fp32 values -> e4m3 codes (uint8): nearest value, ties to the even
    code, |x| > 448 saturating to 448, NaN to 0x7F with the sign bit of x.
    Element by element (large arrays in pieces, which changes nothing)."""
    x = np.asarray(x32, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 20
    for i in range(0, flat.size, step):
        out[i:i + step] = _encode_piece(flat[i:i + step])
    return out.reshape(x.shape)


def _encode_piece(x32) -> np.ndarray:
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(x), 0x80, 0x00).astype(np.uint8)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(a - _POS[lo])
    d_hi = np.abs(_POS[hi] - a)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(a >= E4M3_MAX, np.uint8(0x7E), code)
    code = np.where(np.isnan(a), np.uint8(E4M3_NAN), code)
    return code | sign


def quantize(x, scale) -> np.ndarray:
    """Storage-dtype values x (torch or numpy, last axis any) and a scale
    (broadcast against x) -> e4m3 codes of x / scale, the quotient in fp32."""
    xf = x.float().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float32)
    sf = np.asarray(scale, dtype=np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (xf.astype(np.float32) / sf).astype(np.float32)
    return e4m3_encode(q)


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale):
    """The scatter of "LLM inference engine internals" (section 2.3: slot =
    block * block_size + offset; a negative slot is skipped) into uint8
    pools [NB, bs, Hkv, D], each token's K and V quantised per KV head.
    Returns new pools (numpy uint8)."""
    kc = np.array(key_cache, dtype=np.uint8, copy=True)
    vc = np.array(value_cache, dtype=np.uint8, copy=True)
    nb, bs, hkv, d = kc.shape
    ks = np.asarray(k_scale, dtype=np.float32).reshape(hkv, 1)
    vs = np.asarray(v_scale, dtype=np.float32).reshape(hkv, 1)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    kq = quantize(key, ks)          # [T, Hkv, D]
    vq = quantize(value, vs)
    for i, slot in enumerate(slots.tolist()):
        if slot < 0:
            continue
        kc[slot // bs, slot % bs] = kq[i]
        vc[slot // bs, slot % bs] = vq[i]
    return kc, vc


def dequantize(pool, scale) -> np.ndarray:
    """uint8 pool [NB, bs, Hkv, D] -> float64 values, code value * scale of
    its KV head (exact in float64)."""
    p = np.asarray(pool, dtype=np.uint8)
    s = np.asarray(scale, dtype=np.float32).astype(np.float64).reshape(1, 1, -1, 1)
    return e4m3_decode(p) * s


def decode_fp8(query, key_cache, value_cache, k_scale, v_scale, block_table, seq_lens,
               scale: float, seqs=None) -> np.ndarray:
    """Decode over an e4m3 pool: the decode oracle on the dequantised K and V."""
    return decode(query, dequantize(key_cache, k_scale), dequantize(value_cache, v_scale),
                  block_table, seq_lens, scale, seqs=seqs)


def multi_query_fp8(query, key_cache, value_cache, k_scale, v_scale, block_table, seq_lens,
                    scale: float, seqs=None) -> np.ndarray:
    """Multi-query (q_len new tokens, causal) over an e4m3 pool."""
    return multi_query(query, dequantize(key_cache, k_scale), dequantize(value_cache, v_scale),
                       block_table, seq_lens, scale, seqs=seqs)


def decode_shared_prefix_fp8(query, key_cache, value_cache, k_scale, v_scale, prefix_block_table,
                             prefix_lens, suffix_block_table, suffix_lens, group_size: int,
                             scale: float, seqs=None) -> np.ndarray:
    """Shared-prefix decode (groups of samples reading one prefix of whole
    blocks, then each its own blocks) over an e4m3 pool: the shared-prefix
    oracle of the paged_attention module on the dequantised K and V."""
    return decode_shared_prefix(query, dequantize(key_cache, k_scale), dequantize(value_cache, v_scale),
                                prefix_block_table, prefix_lens, suffix_block_table, suffix_lens,
                                group_size, scale, seqs=seqs)
