"""fp64 CPU oracle: paged decode attention, slot scatter, block copy, closed forms.

Test infrastructure only (see the package docstring): the product path never
imports this module.

Sources (four web pages on vLLM's PagedAttention; cited by title and section):
  [EI]  "LLM inference engine internals: PagedAttention, Continuous Batching and
        modern inference architecture" (ybb.press/ai-applications/9963)
  [IO]  "LLM inference optimisation in practice: from PagedAttention to
        Speculative Decoding" (ybb.press/ai-applications/10310)
  [PP]  "PagedAttention principle" article on tbr8.org (?p=14261)
  [VC]  "vLLM core concepts", course chapter 4 (5688vip.com)

Readings taken where the pages are silent or garbled (each is stated where it
is used below):
  * softmax runs over all cached tokens of one (sequence, query head); the
    pages' Python listing applies it to a single score, which is always 1;
  * the block table is indexed by the logical block number (the CUDA listing
    indexes it by the table length, a typo);
  * query head h reads KV head h // (num_heads / num_kv_heads);
  * seq_len counts every cached token the query attends to, including the
    token being decoded; seq_len = 0 gives a zero output row;
  * a negative slot means "no slot" and is skipped.
"""

from __future__ import annotations

import numpy as np
import torch


# ----------------------------------------------------------------------------
# helpers: storage dtype -> float64 (exact for fp32, fp16 and bf16)
# ----------------------------------------------------------------------------

def _to_f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _to_np_int(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def _pool_shape(cache) -> tuple[int, int, int, int]:
    nb, bs, hkv, d = tuple(cache.shape)
    return nb, bs, hkv, d


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def decode_one(q_s, key_cache, value_cache, table_row, seq_len: int,
               scale: float) -> np.ndarray:
    """Attention output of one sequence, float64 ``[num_heads, head_dim]``.

    Follows the paged-attention listing of [PP] §2.2 (kernel rework): walk the
    sequence's logical positions t = 0 .. seq_len-1, look up the physical
    block of logical block t // block_size in the block table, read slot
    t % block_size of that block from the pool laid out as
    [num_blocks, block_size, num_kv_heads, head_dim] ([PP] §2.2; the two-level
    addressing of [EI] §2.4), stop at seq_len (only the last block may be
    partly filled, [PP] §2.2 and [IO] §2.2), score = q . k * scale with
    scale = 1/sqrt(head_dim) in the pages, softmax over the scores of all
    positions, and output = sum_t softmax_t * v_t.

    The block table is indexed by the logical block number, as in [PP] §2.2
    (the CUDA listing of [EI] §2.4 indexes it by the table length: a typo).
    Query head h reads KV head h // G with G = num_heads / num_kv_heads; the
    pages name both head counts ([PP] §1, §2.2) but not the grouping.
    """
    q = _to_f64(q_s)                      # [H, D]
    H, D = q.shape
    nb, bs, hkv, d = _pool_shape(key_cache)
    if d != D:
        raise ValueError("head_dim mismatch")
    if H % hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = H // hkv
    L = int(seq_len)
    if L <= 0:
        return np.zeros((H, D), dtype=np.float64)
    row = _to_np_int(table_row)

    # per-token gather through the block table
    t = np.arange(L)
    phys = row[t // bs]
    off = t % bs
    if np.any(phys < 0) or np.any(phys >= nb):
        raise IndexError("block table entry outside the pool")
    kc = _to_f64(key_cache[torch.as_tensor(phys), torch.as_tensor(off)]
                 if isinstance(key_cache, torch.Tensor) else
                 np.asarray(key_cache)[phys, off])          # [L, Hkv, D]
    vc = _to_f64(value_cache[torch.as_tensor(phys), torch.as_tensor(off)]
                 if isinstance(value_cache, torch.Tensor) else
                 np.asarray(value_cache)[phys, off])

    out = np.empty((H, D), dtype=np.float64)
    for h in range(H):
        j = h // G
        scores = (kc[:, j, :] @ q[h]) * float(scale)        # [L]
        m = scores.max()
        w = np.exp(scores - m)
        out[h] = (w @ vc[:, j, :]) / w.sum()
    return out


def decode(query, key_cache, value_cache, block_table, seq_lens, scale: float,
           seqs=None) -> np.ndarray:
    """Paged decode attention for a batch, float64 ``[num_seqs, H, D]``.

    ``query`` is ``[num_seqs, num_heads, head_dim]``; ``block_table`` is
    ``[num_seqs, max_blocks_per_seq]``; ``seq_lens`` is ``[num_seqs]``.
    With ``seqs`` given, only those rows are computed (the others are NaN), so
    that large batches can be checked on a sample of sequences.
    """
    S, H, D = tuple(query.shape)
    lens = _to_np_int(seq_lens)
    bt = _to_np_int(block_table)
    out = np.full((S, H, D), np.nan, dtype=np.float64)
    rows = range(S) if seqs is None else seqs
    for s in rows:
        out[s] = decode_one(query[s], key_cache, value_cache, bt[s],
                            int(lens[s]), scale)
    return out


# ----------------------------------------------------------------------------
# several new tokens per sequence (speculative verification, chunked prefill)
# ----------------------------------------------------------------------------

def multi_query_one(q_s, key_cache, value_cache, table_row, seq_len: int,
                    scale: float) -> np.ndarray:
    """Attention outputs of the q_len newest tokens of one sequence, float64
    ``[q_len, num_heads, head_dim]``.

    The target model checks all of a draft model's candidate tokens in one
    forward pass over the cached prefix ([IO] §4.1-§4.2; [VC] §4.4.1;
    [EI] §5.2: the candidates' K/V live in the same blocks); a prefill cut
    into chunks does the same per chunk ([IO] §5.3). Reading taken: the
    q_len new tokens are the last q_len positions L-q_len .. L-1 of the
    sequence (their K/V already written to their slots), and new token j
    attends causally to positions 0 .. L-q_len+j. Each (token, head) is
    otherwise the decode of [PP] §2.2: gather through the block table,
    score = q . k * scale, softmax over the attended positions, weighted sum
    of V. A token with no attended position (L < q_len) gives a zero row.
    """
    q = _to_f64(q_s)                      # [q_len, H, D]
    Q, H, D = q.shape
    nb, bs, hkv, d = _pool_shape(key_cache)
    if d != D:
        raise ValueError("head_dim mismatch")
    if H % hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = H // hkv
    L = int(seq_len)
    out = np.zeros((Q, H, D), dtype=np.float64)
    if L <= 0:
        return out
    row = _to_np_int(table_row)
    t = np.arange(L)
    phys = row[t // bs]
    off = t % bs
    if np.any(phys < 0) or np.any(phys >= nb):
        raise IndexError("block table entry outside the pool")
    kc = _to_f64(key_cache[torch.as_tensor(phys), torch.as_tensor(off)]
                 if isinstance(key_cache, torch.Tensor) else
                 np.asarray(key_cache)[phys, off])          # [L, Hkv, D]
    vc = _to_f64(value_cache[torch.as_tensor(phys), torch.as_tensor(off)]
                 if isinstance(value_cache, torch.Tensor) else
                 np.asarray(value_cache)[phys, off])
    for j in range(Q):
        last = L - Q + j                  # the newest position token j sees
        if last < 0:
            continue
        for h in range(H):
            kv = h // G
            scores = (kc[:last + 1, kv, :] @ q[j, h]) * float(scale)
            w = np.exp(scores - scores.max())
            out[j, h] = (w @ vc[:last + 1, kv, :]) / w.sum()
    return out


def multi_query(query, key_cache, value_cache, block_table, seq_lens, scale: float,
                seqs=None) -> np.ndarray:
    """multi_query_one for a batch: ``query`` ``[num_seqs, q_len, H, D]`` ->
    float64 ``[num_seqs, q_len, H, D]``; rows not in ``seqs`` (if given) are NaN."""
    S, Q, H, D = tuple(query.shape)
    lens = _to_np_int(seq_lens)
    bt = _to_np_int(block_table)
    out = np.full((S, Q, H, D), np.nan, dtype=np.float64)
    rows = range(S) if seqs is None else seqs
    for s in rows:
        out[s] = multi_query_one(query[s], key_cache, value_cache, bt[s],
                                 int(lens[s]), scale)
    return out


# ----------------------------------------------------------------------------
# cache operations (bit copies in the storage dtype)
# ----------------------------------------------------------------------------

def _bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view of a tensor so that copies keep every bit (NaN payloads)."""
    itype = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}
    return t.view(itype[t.element_size()])


def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping):
    """Write each new token's K and V into its slot; returns new pools.

    The slot of a token is block * block_size + offset ([EI] §2.3, the block
    engine's append_slot: the offset is the token count modulo block_size in
    the sequence's last block, or 0 in a freshly taken block; growth as in
    [VC] §4.2.2). Here the slot is decoded back into (slot // block_size,
    slot % block_size) and the token's [num_kv_heads, head_dim] row is copied
    there. A negative slot means "no slot" (the page's append_slot returns
    nothing when the pool is exhausted) and writes nothing.
    """
    kc = key_cache.clone()
    vc = value_cache.clone()
    nb, bs, hkv, d = _pool_shape(kc)
    kb, vb = _bits(kc), _bits(vc)
    kin, vin = _bits(key.contiguous()), _bits(value.contiguous())
    slots = _to_np_int(slot_mapping)
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = int(slot) // bs, int(slot) % bs
        if blk >= nb:
            raise IndexError("slot outside the pool")
        kb[blk, off] = kin[i]
        vb[blk, off] = vin[i]
    return kc, vc


def copy_blocks(key_cache, value_cache, block_mapping):
    """Copy whole physical blocks (K and V) src -> dst; returns new pools.

    The copy-on-write step: a block shared by several sequences is copied
    before one of them writes to it ([VC] §4.2.2; [EI] §3.3, and the
    scheduler's blocks_to_copy output in [EI] §3.1; [PP] §5). The pages show
    blocks_to_copy only as an empty mapping; it is read here as a list of
    (src, dst) pairs with every read taken before any write (a snapshot).
    """
    kc = key_cache.clone()
    vc = value_cache.clone()
    snap_k, snap_v = _bits(key_cache.clone()), _bits(value_cache.clone())
    kb, vb = _bits(kc), _bits(vc)
    pairs = _to_np_int(block_mapping).reshape(-1, 2)
    for src, dst in pairs:
        kb[int(dst)] = snap_k[int(src)]
        vb[int(dst)] = snap_v[int(src)]
    return kc, vc


def decode_shared_prefix(query, key_cache, value_cache, prefix_block_table, prefix_lens,
                         suffix_block_table, suffix_lens, group_size: int, scale: float,
                         seqs=None) -> np.ndarray:
    """Decode for groups of ``group_size`` consecutive sequences sharing a
    prefix of whole blocks (the samples of one prompt share its blocks:
    [VC] §4.2.2, [EI] §3.3, [PP] §5): sequence s of group g = s // group_size
    has the block table prefix_block_table[g][:prefix_lens[g] / bs] followed
    by suffix_block_table[s], and length prefix_lens[g] + suffix_lens[s];
    the result is ``decode`` of those tables, float64 ``[S, H, D]``."""
    S = tuple(query.shape)[0]
    nb, bs, hkv, d = _pool_shape(key_cache)
    pt, pl = _to_np_int(prefix_block_table), _to_np_int(prefix_lens)
    st, sl = _to_np_int(suffix_block_table), _to_np_int(suffix_lens)
    width = pt.shape[1] + st.shape[1]
    table = np.zeros((S, width), dtype=np.int64)
    lens = np.zeros(S, dtype=np.int64)
    for s in range(S):
        g = s // group_size
        if pl[g] % bs != 0:
            raise ValueError("a shared prefix is made of whole blocks")
        npb = int(pl[g]) // bs
        row = list(pt[g, :npb]) + list(st[s])
        table[s, :len(row)] = row
        lens[s] = pl[g] + sl[s]
    return decode(query, key_cache, value_cache, table, lens, scale, seqs=seqs)


def swap_blocks(src_key, src_value, dst_key, dst_value, block_mapping):
    """Move whole blocks (K and V) from one pool to another; returns the new
    destination pools.

    Preemption by swapping: a sequence's blocks are copied from GPU memory to
    a CPU swap space and freed, and copied back (to any free GPU blocks) when
    it resumes ([EI] §3.2; the scheduler's blocks_to_swap_out and
    blocks_to_swap_in outputs in [EI] §3.1; the swap space of [VC] §4.2.4).
    Read here as a list of (source block, destination block) pairs between
    two pools of the same block layout; the source is not changed.
    """
    dk = dst_key.clone()
    dv = dst_value.clone()
    kb, vb = _bits(dk), _bits(dv)
    sk, sv = _bits(src_key), _bits(src_value)
    pairs = _to_np_int(block_mapping).reshape(-1, 2)
    for src, dst in pairs:
        kb[int(dst)] = sk[int(src)]
        vb[int(dst)] = sv[int(src)]
    return dk, dv


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def kv_cache_bytes(num_layers: int, seq_len: int, num_kv_heads: int,
                   head_dim: int, dtype_size: int = 2) -> int:
    """KV-cache bytes of one sequence: 2 (K and V) x layers x tokens x KV heads
    x head_dim x bytes per element ([PP] §1, the kv_cache_size formula)."""
    return 2 * num_layers * seq_len * num_kv_heads * head_dim * dtype_size


def block_bytes(num_layers: int, block_size: int, num_kv_heads: int,
                head_dim: int, dtype_size: int = 2) -> int:
    """Bytes of one physical block across all layers ([PP] §4.2, the
    kv_cache_per_block line of the block-count listing, and §7.3)."""
    return 2 * num_layers * block_size * num_kv_heads * head_dim * dtype_size


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks holding num_tokens tokens: the ceiling of num_tokens/block_size
    ([IO] §2.1, BlockTable.num_blocks; [PP] §3, BlockManager.allocate)."""
    return (num_tokens + block_size - 1) // block_size

