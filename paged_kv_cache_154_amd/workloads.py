"""Seeded synthetic inputs for paged decode attention (no attention arithmetic).

This module builds the inputs that both the HIP path and the CPU oracle read:
block tables, sequence lengths, queries, K/V pools, slot mappings and
copy-on-write pairs. It contains none of the method's arithmetic (no scores,
no softmax, no weighted sums); it only decides shapes, values and placement.

Shapes follow the pages' statement of the problem: query
``[num_seqs, num_heads, head_dim]``, pools ``[num_blocks, block_size,
num_kv_heads, head_dim]``, block tables ``[num_seqs, max_blocks_per_seq]``
int32, ``seq_lens`` int32, slot mappings int64 (slot = block * block_size +
offset), copy pairs int64 ``[num_pairs, 2]`` as (src, dst).

Randomness:
  * structure (lengths, order, placement) comes from
    ``numpy.random.default_rng(1540 + k)`` for workload k, drawn in the order
    lengths -> order shuffle -> physical placement;
  * values are N(0, 1) in float32, rounded to the storage dtype by torch;
    each value array (Q, K, V, new K, new V) has its own stream keyed by
    ``(1540 + k, array tag, chunk index)`` over fixed 4 Mi-element chunks, so
    it can be drawn on several threads and does not depend on the thread
    count;
  * placement: a random permutation of the pool's physical blocks is handed
    out in order to the logical blocks, sequence-major; blocks left over stay
    free;
  * fills: every slot that holds no token (the unused tail of each last block,
    free blocks, the slot a new token is about to be written to, the
    destination of a copy-on-write) holds NaN, so that any read of it shows
    up in the result; unused block-table entries point at a free (NaN) block.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 1540
_CHUNK = 1 << 22

_TAGS = {"q": 1, "k": 2, "v": 3, "new_k": 4, "new_v": 5}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, tag: str, n: int) -> np.ndarray:
    """n N(0,1) float32 draws from the stream (seed, tag), chunked."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        rng = np.random.default_rng([seed, _TAGS[tag], c])
        rng.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def _values(seed: int, tag: str, shape, dtype: torch.dtype) -> torch.Tensor:
    n = int(np.prod(shape))
    return torch.from_numpy(normal_f32(seed, tag, n)).reshape(shape).to(dtype)


@dataclass
class Workload:
    """One batch of decode inputs on the host (CPU tensors / numpy arrays)."""

    name: str
    seed: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    dtype: torch.dtype
    scale: float
    seq_lens: np.ndarray            # int32 [S]
    block_table: np.ndarray         # int32 [S, MB] (after any copy-on-write remap)
    query: torch.Tensor             # [S, H, D]; [S, q_len, H, D] when q_len > 1
    key_cache: torch.Tensor         # [NB, bs, Hkv, D], before this step's cache ops
    value_cache: torch.Tensor
    partition_size: int = 0         # 0: the library chooses
    new_key: torch.Tensor | None = None      # [T, Hkv, D]
    new_value: torch.Tensor | None = None
    slot_mapping: np.ndarray | None = None   # int64 [T]
    block_mapping: np.ndarray | None = None  # int64 [P, 2] (src, dst)
    block_table_before_cow: np.ndarray | None = None
    unique_blocks: int = 0          # physical blocks holding data or referenced
    info: dict = field(default_factory=dict)
    q_len: int = 1                  # new tokens per sequence (the last q_len positions)

    # -- shape helpers ----------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return torch.empty((), dtype=self.dtype).element_size()

    @property
    def num_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode reads: every cached token's K and
        V row for every KV head, once."""
        return self.num_tokens * 2 * self.num_kv_heads * self.head_dim * self.elem_bytes


def _place(rng, num_blocks: int, n_virtual: int):
    perm = rng.permutation(num_blocks).astype(np.int64)
    phys = perm[:n_virtual]
    free = perm[n_virtual:]
    poison = int(free[0]) if free.size else 0
    return phys, poison


def _assemble(*, name, seed, rng, H, Hkv, D, bs, dtype, seq_lens, tables_virtual,
              fill, num_blocks, max_blocks, new_positions=None,
              tables_virtual_before=None, cow_virtual_pairs=None,
              partition_size=0, q_len=1) -> Workload:
    """Turn a virtual block layout into concrete pools and tables.

    tables_virtual[s] lists the virtual block ids of sequence s in logical
    order; fill[v] is how many leading slots of virtual block v hold a cached
    token (drawn here). new_positions[s] (optional) is the logical position of
    the token that reshape_and_cache will write in this step.
    """
    S = len(seq_lens)
    n_virtual = len(fill)
    phys, poison = _place(rng, num_blocks, n_virtual)

    def table_of(tv):
        bt = np.full((S, max_blocks), poison, dtype=np.int32)
        for s, row in enumerate(tv):
            if len(row) > max_blocks:
                raise ValueError("sequence needs more blocks than max_blocks_per_seq")
            bt[s, :len(row)] = phys[np.asarray(row, dtype=np.int64)] if len(row) else []
        return bt

    block_table = table_of(tables_virtual)
    before = table_of(tables_virtual_before) if tables_virtual_before is not None else None

    query = _values(seed, "q", (S, H, D) if q_len == 1 else (S, q_len, H, D), dtype)

    fill = np.asarray(fill, dtype=np.int64)
    # flat slot of every cached token, virtual-block order, slot order
    starts = phys * bs
    flat = np.concatenate([starts[v] + np.arange(fill[v]) for v in range(n_virtual)]
                          ) if n_virtual else np.zeros(0, np.int64)
    n_fill = int(flat.size)
    key_cache = torch.full((num_blocks, bs, Hkv, D), float("nan"), dtype=dtype)
    value_cache = torch.full((num_blocks, bs, Hkv, D), float("nan"), dtype=dtype)
    idx = torch.from_numpy(flat)
    key_cache.view(num_blocks * bs, Hkv, D)[idx] = _values(seed, "k", (n_fill, Hkv, D), dtype)
    value_cache.view(num_blocks * bs, Hkv, D)[idx] = _values(seed, "v", (n_fill, Hkv, D), dtype)

    wl = Workload(name=name, seed=seed, num_heads=H, num_kv_heads=Hkv, head_dim=D,
                  block_size=bs, num_blocks=num_blocks, max_blocks_per_seq=max_blocks,
                  dtype=dtype, scale=1.0 / math.sqrt(D),
                  seq_lens=np.asarray(seq_lens, dtype=np.int32),
                  block_table=block_table, query=query, key_cache=key_cache,
                  value_cache=value_cache, partition_size=partition_size,
                  block_table_before_cow=before, unique_blocks=n_virtual, q_len=q_len)

    if new_positions is not None:
        # one position per sequence, or a list of them (q_len > 1), in order
        flat = [(s, int(pos)) for s, p_s in enumerate(new_positions)
                for pos in (p_s if isinstance(p_s, (list, tuple)) else [p_s])]
        T = len(flat)
        slots = np.empty(T, dtype=np.int64)
        for i, (s, pos) in enumerate(flat):
            lb, off = divmod(pos, bs)
            slots[i] = int(phys[tables_virtual[s][lb]]) * bs + off
        wl.slot_mapping = slots
        wl.new_key = _values(seed, "new_k", (T, Hkv, D), dtype)
        wl.new_value = _values(seed, "new_v", (T, Hkv, D), dtype)
    if cow_virtual_pairs is not None:
        wl.block_mapping = np.asarray([[phys[a], phys[b]] for a, b in cow_virtual_pairs],
                                      dtype=np.int64).reshape(-1, 2)
    return wl


def _plain_layout(seq_lens, bs, new_token: bool, q_len: int = 1):
    """Each sequence owns ceil(L/bs) private blocks, sequence-major. With
    new_token, positions L-q_len .. L-1 are left empty for this step's
    scatter."""
    tables, fill = [], []
    for L in seq_lens:
        L = int(L)
        stored = max(0, L - q_len) if (new_token and L > 0) else L
        nblk = (L + bs - 1) // bs
        row = []
        for i in range(nblk):
            row.append(len(fill))
            fill.append(min(bs, max(0, stored - i * bs)))
        tables.append(row)
    return tables, fill


def custom(seed: int, *, seq_lens, num_heads: int, num_kv_heads: int, head_dim: int,
           block_size: int, dtype: torch.dtype, num_blocks: int | None = None,
           max_blocks_per_seq: int | None = None, new_token: bool = False,
           partition_size: int = 0, name: str = "custom", q_len: int = 1) -> Workload:
    """A plain (unshared) paged batch with the given lengths. With q_len > 1
    each sequence has q_len new tokens (its last q_len positions): the query
    is [S, q_len, H, D], and with new_token their K/V come from the scatter."""
    rng = np.random.default_rng(seed)
    seq_lens = [int(x) for x in seq_lens]
    tables, fill = _plain_layout(seq_lens, block_size, new_token, q_len)
    need = len(fill)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(1.2 * need)) + 1
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max([len(r) for r in tables] + [1])
    if q_len == 1:
        newpos = [L - 1 for L in seq_lens] if new_token else None
    else:
        newpos = [list(range(L - q_len, L)) for L in seq_lens] if new_token else None
    if new_token and any(L < q_len for L in seq_lens):
        raise ValueError("new_token needs seq_len >= q_len")
    return _assemble(name=name, seed=seed, rng=rng, H=num_heads, Hkv=num_kv_heads,
                     D=head_dim, bs=block_size, dtype=dtype, seq_lens=seq_lens,
                     tables_virtual=tables, fill=fill, num_blocks=num_blocks,
                     max_blocks=max_blocks_per_seq, new_positions=newpos,
                     partition_size=partition_size, q_len=q_len)


# ----------------------------------------------------------------------------
# the five page-shaped workloads
# ----------------------------------------------------------------------------

def tiny() -> Workload:
    """4 sequences {1, 17, 33, 50}, 4 heads = 4 KV heads, head_dim 64, fp32,
    block_size 16, 32-block pool; the new token of each sequence (position
    L-1) is written by reshape_and_cache in the step. Lengths 17 and 33 put
    the new token at offset 0 of a fresh block, 50 at offset 1 of a partly
    filled one, and 1 gives the one-token case."""
    seed = SEED_BASE + 1
    rng = np.random.default_rng(seed)
    lens = [1, 17, 33, 50]
    tables, fill = _plain_layout(lens, 16, new_token=True)
    return _assemble(name="tiny_fp32", seed=seed, rng=rng, H=4, Hkv=4, D=64, bs=16,
                     dtype=torch.float32, seq_lens=lens, tables_virtual=tables,
                     fill=fill, num_blocks=32, max_blocks=4,
                     new_positions=[L - 1 for L in lens])


def llama3_8b(q_len: int = 1) -> Workload:
    """Llama-3-8B-shaped layer: 64 sequences, 32 q / 8 KV heads, head_dim 128,
    bf16, block_size 16, lengths uniform in [512, 4096], 20000-block pool,
    plus reshape_and_cache of each sequence's new token. With q_len > 1 the
    same lengths hold q_len new tokens each (the last q_len positions: a
    speculative verification step), written by the step's scatter."""
    seed = SEED_BASE + 2
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 4097, size=64).tolist()
    tables, fill = _plain_layout(lens, 16, new_token=True, q_len=q_len)
    newpos = ([L - 1 for L in lens] if q_len == 1 else
              [list(range(L - q_len, L)) for L in lens])
    return _assemble(name="llama3_8b_bf16" if q_len == 1 else f"llama3_8b_bf16_q{q_len}",
                     seed=seed, rng=rng, H=32, Hkv=8, D=128, bs=16, dtype=torch.bfloat16,
                     seq_lens=lens, tables_virtual=tables, fill=fill, num_blocks=20000,
                     max_blocks=256, new_positions=newpos, q_len=q_len)


def llama2_70b() -> Workload:
    """Llama-2-70B-shaped layer: 256 sequences, 64 q / 8 KV heads, head_dim
    128, fp16, block_size 32, lengths lognormal with median 1024 and sigma 1.0
    clipped to [32, 8192], pool 1.2x the blocks needed."""
    seed = SEED_BASE + 3
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(256)
    lens = np.clip(np.rint(np.exp(math.log(1024.0) + 1.0 * z)), 32, 8192).astype(int).tolist()
    tables, fill = _plain_layout(lens, 32, new_token=False)
    nb = math.ceil(1.2 * len(fill))
    return _assemble(name="llama2_70b_fp16", seed=seed, rng=rng, H=64, Hkv=8, D=128,
                     bs=32, dtype=torch.float16, seq_lens=lens, tables_virtual=tables,
                     fill=fill, num_blocks=nb, max_blocks=256)


def prefix_share(groups: int = 128, n: int = 3, prefix: int = 2048,
                 max_suffix: int = 512) -> Workload:
    """Parallel sampling: 128 prompt groups x 3 samples sharing a 2048-token
    prefix (the block-table entries of the three samples point at the same
    physical blocks), each sample with its own suffix of 0..512 tokens;
    32 q / 8 KV heads, head_dim 128, bf16, block_size 16.

    On fork, samples 1 and 2 of a group take a private copy of the last
    prefix block (copy-on-write); sample 0 keeps the original. The copy
    destinations hold NaN until copy_blocks runs. ``block_table`` is the
    table after the remap, ``block_table_before_cow`` the one before."""
    seed = SEED_BASE + 4
    rng = np.random.default_rng(seed)
    bs = 16
    suffix = rng.integers(0, max_suffix + 1, size=groups * n)
    lens = (prefix + suffix).tolist()
    npre = (prefix + bs - 1) // bs
    tables, before, fill, pairs = [], [], [], []
    for g in range(groups):
        pre = list(range(len(fill), len(fill) + npre))
        fill.extend([min(bs, prefix - i * bs) for i in range(npre)])
        cow = {}
        for i in range(1, n):
            cow[i] = len(fill)
            fill.append(0)
            pairs.append((pre[-1], cow[i]))
        for i in range(n):
            sl = int(suffix[g * n + i])
            nsb = (sl + bs - 1) // bs
            suf = list(range(len(fill), len(fill) + nsb))
            fill.extend([min(bs, sl - k * bs) for k in range(nsb)])
            row = pre[:-1] + [pre[-1] if i == 0 else cow[i]] + suf
            tables.append(row)
            before.append(pre + suf)
    nb = math.ceil(1.2 * len(fill))
    mb = (prefix + max_suffix + bs - 1) // bs
    wl = _assemble(name="prefix_share_bf16", seed=seed, rng=rng, H=32, Hkv=8, D=128,
                   bs=bs, dtype=torch.bfloat16, seq_lens=lens, tables_virtual=tables,
                   fill=fill, num_blocks=nb, max_blocks=mb,
                   tables_virtual_before=before, cow_virtual_pairs=pairs)
    wl.info.update(groups=groups, samples=n, prefix=prefix)
    return wl


def shared_prefix_tables(wl: Workload, group_size: int):
    """The batch's block tables split for shared-prefix decode: groups of
    group_size consecutive sequences; a group's prefix is the longest run of
    leading blocks that every member's table holds (and fills: at most the
    shortest member's whole blocks), the rest of each table its suffix.
    Returns prefix_table int32 [groups, max_prefix_blocks], prefix_lens int32
    [groups], suffix_table int32 [S, max_suffix_blocks], suffix_lens int32 [S]."""
    bs = wl.block_size
    S = wl.num_seqs
    if S % group_size:
        raise ValueError("the batch is not a whole number of groups")
    groups = S // group_size
    lens = wl.seq_lens.astype(np.int64)
    pre_rows, pre_lens, suf_rows, suf_lens = [], [], [], []
    for g in range(groups):
        members = range(g * group_size, (g + 1) * group_size)
        full = min(int(lens[s]) // bs for s in members)
        k = 0
        while k < full and len({int(wl.block_table[s, k]) for s in members}) == 1:
            k += 1
        pre_rows.append(wl.block_table[g * group_size, :k].tolist())
        pre_lens.append(k * bs)
        for s in members:
            nb = (int(lens[s]) + bs - 1) // bs
            suf_rows.append(wl.block_table[s, k:nb].tolist())
            suf_lens.append(int(lens[s]) - k * bs)
    wp = max([len(r) for r in pre_rows] + [1])
    ws = max([len(r) for r in suf_rows] + [1])
    pt = np.zeros((groups, wp), dtype=np.int32)
    st = np.zeros((S, ws), dtype=np.int32)
    for g, r in enumerate(pre_rows):
        pt[g, :len(r)] = r
    for s, r in enumerate(suf_rows):
        st[s, :len(r)] = r
    return pt, np.array(pre_lens, dtype=np.int32), st, np.array(suf_lens, dtype=np.int32)


def mixed_splitk() -> Workload:
    """Mixed batch: 16 sequences of 10000 tokens (20 turns x 500 tokens) and
    240 sequences uniform in [50, 2000], shuffled; 32 q / 8 KV heads,
    head_dim 128, bf16, block_size 8; 512-token sequence partitions."""
    seed = SEED_BASE + 5
    rng = np.random.default_rng(seed)
    short = rng.integers(50, 2001, size=240)
    lens = np.concatenate([np.full(16, 10000), short])
    order = rng.permutation(lens.size)
    lens = lens[order].tolist()
    tables, fill = _plain_layout(lens, 8, new_token=False)
    nb = math.ceil(1.2 * len(fill))
    return _assemble(name="mixed_splitk_bf16", seed=seed, rng=rng, H=32, Hkv=8, D=128,
                     bs=8, dtype=torch.bfloat16, seq_lens=lens, tables_virtual=tables,
                     fill=fill, num_blocks=nb, max_blocks=1250, partition_size=512)


CONFIGS = {1: tiny, 2: llama3_8b, 3: llama2_70b, 4: prefix_share, 5: mixed_splitk}


def make(config: int) -> Workload:
    return CONFIGS[config]()
