"""Paged KV-cache decode attention for AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``include/pagedkv.h``: it only turns
torch tensors (device memory) and the current HIP stream into the pointers
and sizes the library takes. Every step of the computation runs in the HIP
kernels of ``libpagedkv.so``; there is no Python or CPU fallback.

    paged_attn_decode(out, query, key_cache, value_cache, block_table,
                      seq_lens, scale, max_seq_len, partition_size=0,
                      workspace=None)
    paged_attn_multi_query(out, query, key_cache, value_cache, block_table,
                           seq_lens, scale, max_seq_len, partition_size=0,
                           workspace=None)
    reshape_and_cache(key, value, key_cache, value_cache, slot_mapping)
    copy_blocks(key_cache, value_cache, block_mapping)
    swap_blocks(src_key_cache, src_value_cache, dst_key_cache, dst_value_cache,
                block_mapping)      # GPU <-> pinned host pools

e4m3 KV cache (pools of uint8 codes, or torch.float8_e4m3fn; fp32 scales
``[num_kv_heads]`` for K and for V; the query bf16 or fp16):

    reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping,
                          k_scale, v_scale)
    paged_attn_decode_fp8(out, query, key_cache, value_cache, k_scale, v_scale,
                          block_table, seq_lens, scale, max_seq_len, ...)
    paged_attn_multi_query_fp8(...)   # query [num_seqs, q_len, num_heads, head_dim]

Shapes (all dense, on one GPU): query/out ``[num_seqs, num_heads,
head_dim]`` for decode, ``[num_seqs, q_len, num_heads, head_dim]`` for
the multi-query pass; pools ``[num_blocks, block_size, num_kv_heads, head_dim]``;
block_table int32 ``[num_seqs, max_blocks_per_seq]``; seq_lens int32
``[num_seqs]``; slot_mapping int64 ``[num_tokens]``; block_mapping int64
``[num_pairs, 2]``.
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import (PKV_BF16, PKV_E4M3, PKV_F16, PKV_F32, LIB_PATH, PagedKVError,  # noqa: F401
                   check, lib, status_string)

_DTYPE_CODE = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
               torch.uint8: PKV_E4M3, torch.float8_e4m3fn: PKV_E4M3}


def dtype_code(dtype: torch.dtype) -> int:
    try:
        return _DTYPE_CODE[dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {dtype}") from None


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpagedkv must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int | None:
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _torch_stream(t: torch.Tensor, stream):
    """The torch stream a call on ``t`` runs on: ``stream`` (a torch stream or
    a raw handle) or the current one. Buffers the binding allocates for a
    call are allocated on it, so the caching allocator does not hand them to
    other streams while the call's kernels may still use them."""
    if stream is None:
        return torch.cuda.current_stream(t.device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)), device=t.device)


def _zeroed_on(t: torch.Tensor, stream, nbytes: int) -> torch.Tensor:
    """A zero-filled uint8 device buffer allocated and cleared on the call's
    stream (the workspace's control area must be zero at its first use)."""
    with torch.cuda.stream(_torch_stream(t, stream)):
        return torch.zeros(nbytes, dtype=torch.uint8, device=t.device)


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def paged_attn_partition_tokens(num_seqs: int, num_kv_heads: int, block_size: int,
                                max_seq_len: int, partition_size: int = 0, q_len: int = 1,
                                num_heads: int | None = None, kv_dtype: int = PKV_BF16) -> int:
    """The partition length the attention calls use (partition_size 0: the
    library's choice for a pool of kv_dtype and q_len new tokens per
    sequence); num_heads defaults to num_kv_heads (only the query rows per KV
    head, q_len * num_heads / num_kv_heads, matter)."""
    H = num_kv_heads if num_heads is None else num_heads
    r = lib().paged_attn_partition_tokens(num_seqs, q_len, H, num_kv_heads, block_size, max_seq_len,
                                          partition_size, kv_dtype)
    if r < 0:
        raise PagedKVError(r, "paged_attn_partition_tokens")
    return r


def paged_attn_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                              block_size: int, max_seq_len: int, partition_size: int = 0) -> int:
    return int(lib().paged_attn_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                               block_size, max_seq_len, partition_size))


def paged_attn_multi_query_workspace_size(num_seqs: int, q_len: int, num_heads: int,
                                          num_kv_heads: int, head_dim: int, block_size: int,
                                          max_seq_len: int, partition_size: int = 0) -> int:
    return int(lib().paged_attn_multi_query_workspace_size(
        num_seqs, q_len, num_heads, num_kv_heads, head_dim, block_size, max_seq_len,
        partition_size))


def workspace_for(query: torch.Tensor, key_cache: torch.Tensor, max_seq_len: int,
                  partition_size: int = 0, stream=None) -> torch.Tensor | None:
    """A zero-filled device buffer big enough for paged_attn_decode (query
    ``[S, H, D]``) or paged_attn_multi_query (query ``[S, q_len, H, D]``) with
    these shapes, allocated on the call's stream. Every call leaves the
    workspace's control area zero again, so one buffer serves any number of
    later calls in order on that stream (graph replays included)."""
    if query.dim() == 3:
        S, H, D = query.shape
        Q = 1
    else:
        S, Q, H, D = query.shape
    NB, bs, Hkv, _ = key_cache.shape
    n = paged_attn_multi_query_workspace_size(S, Q, H, Hkv, D, bs, max_seq_len, partition_size)
    if n == 0:
        return None
    return _zeroed_on(query, stream, n)


def workspace_control_bytes(num_seqs: int, num_kv_heads: int, head_dim: int, block_size: int,
                            max_seq_len: int, partition_size: int = 0) -> int:
    """Bytes at the start of a decode / multi-query workspace that must be
    zero at its first use (the control area; include/pagedkv.h): 256, plus
    the arrival counts padded to 256 bytes when sequences are split (taken
    for the shortest partition choice, that of 16-bit pools at 9 to 16 query
    rows per KV head, so the size serves every call the workspace is sized
    for)."""
    P = paged_attn_partition_tokens(num_seqs, num_kv_heads, block_size, max_seq_len,
                                    partition_size, q_len=16)
    if P >= max_seq_len:
        return 256
    return 256 + (4 * min(num_seqs, 2048) * num_kv_heads + 255) // 256 * 256


def shared_prefix_control_bytes(num_groups: int, group_size: int, num_kv_heads: int,
                                head_dim: int, block_size: int, max_prefix_len: int,
                                max_suffix_len: int, partition_size: int = 0) -> int:
    """Bytes at the start of a shared-prefix workspace that must be zero at its
    first use: the prefix pass's control area, then the suffix pass's."""
    return (workspace_control_bytes(num_groups, num_kv_heads, head_dim, block_size,
                                    max_prefix_len, partition_size)
            + workspace_control_bytes(num_groups * group_size, num_kv_heads, head_dim, block_size,
                                      max_suffix_len, partition_size))


def _attention(name: str, out, query, key_cache, value_cache, block_table, seq_lens, scale,
               max_seq_len, partition_size, workspace, stream, k_scale=None,
               v_scale=None, events=None) -> torch.Tensor:
    multi = "multi_query" in name
    f8 = name.endswith("_fp8")
    want = 4 if multi else 3
    _require(query.dim() == want and out.shape == query.shape,
             "query/out must be [S, q_len, H, D]" if multi else "query/out must be [S, H, D]")
    _require(key_cache.dim() == 4 and value_cache.shape == key_cache.shape,
             "pools must be [num_blocks, block_size, num_kv_heads, head_dim]")
    _require(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32,
             "block_table and seq_lens must be int32")
    if f8:
        _require(dtype_code(key_cache.dtype) == PKV_E4M3 and key_cache.dtype == value_cache.dtype,
                 "e4m3 pools must be uint8 or float8_e4m3fn")
        _require(query.dtype in (torch.float16, torch.bfloat16), "the query must be fp16 or bf16")
        _require(k_scale is not None and v_scale is not None and k_scale.dtype == torch.float32
                 and v_scale.dtype == torch.float32
                 and k_scale.shape == v_scale.shape == (key_cache.shape[2],),
                 "k_scale and v_scale must be fp32 [num_kv_heads]")
    else:
        _require(query.dtype == key_cache.dtype == value_cache.dtype,
                 "query and pools share a dtype")
    if multi:
        S, Q, H, D = query.shape
    else:
        (S, H, D), Q = query.shape, 1
    NB, bs, Hkv, D2 = key_cache.shape
    _require(D2 == D, "head_dim of query and pools differ")
    _require(block_table.dim() == 2 and block_table.shape[0] == S and seq_lens.shape == (S,),
             "block_table must be [S, max_blocks] and seq_lens [S]")
    if workspace is None:
        workspace = workspace_for(query, key_cache, max_seq_len, partition_size, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if events is not None:
        # the same attention through paged_attn_timed: the launches set the
        # two events to the kernels' own start and end
        start, stop = events
        for ev in (start, stop):
            if ev.cuda_event == 0:          # created on first record
                ev.record(torch.cuda.current_stream(query.device))
        q_dt = dtype_code(query.dtype)
        st = lib().paged_attn_timed(
            _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
            _ptr(k_scale) if f8 else None, _ptr(v_scale) if f8 else None, _ptr(block_table),
            _ptr(seq_lens), S, Q, H, Hkv, D, bs, NB, block_table.shape[1], int(max_seq_len),
            float(scale), PKV_E4M3 if f8 else q_dt, q_dt, dtype_code(out.dtype), int(partition_size),
            _ptr(workspace), ws_bytes, _stream(query, stream), ctypes.c_void_p(start.cuda_event),
            ctypes.c_void_p(stop.cuda_event))
        check(st, "paged_attn_timed")
        return out
    head = [_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache)]
    if f8:
        head += [_ptr(k_scale), _ptr(v_scale)]
    head += [_ptr(block_table), _ptr(seq_lens), S]
    if multi:
        head.append(Q)
    # the 16-bit entry points take the KV dtype (= the query's), the e4m3 ones the query's
    st = getattr(lib(), name)(
        *head, H, Hkv, D, bs, NB, block_table.shape[1], int(max_seq_len), float(scale),
        dtype_code(query.dtype), dtype_code(out.dtype), int(partition_size), _ptr(workspace), ws_bytes,
        _stream(query, stream))
    check(st, name)
    return out


def paged_attn_decode(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, block_table: torch.Tensor,
                      seq_lens: torch.Tensor, scale: float, max_seq_len: int,
                      partition_size: int = 0, workspace: torch.Tensor | None = None,
                      stream=None, events=None) -> torch.Tensor:
    """Decode attention of one query token per sequence over the paged pool.

    ``workspace`` must hold ``paged_attn_workspace_size(...)`` bytes (the
    control area, zero before the first use and left zero by every call, and
    the split-K partials); later calls on the same stream can reuse it
    (``workspace_for`` makes one). With ``workspace=None`` a zeroed one is
    allocated by torch on the call's stream. ``events=(start, stop)`` (torch.cuda.Event(enable_timing=True))
    runs the same call through paged_attn_timed: the launches themselves set
    the events to the kernels' start and end (a measurement aid)."""
    return _attention("paged_attn_decode", out, query, key_cache, value_cache, block_table,
                      seq_lens, scale, max_seq_len, partition_size, workspace, stream,
                      events=events)


def paged_attn_decode_noalloc(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                              value_cache: torch.Tensor, block_table: torch.Tensor,
                              seq_lens: torch.Tensor, scale: float, max_seq_len: int,
                              partition_size: int = 0, stream=None) -> torch.Tensor:
    """paged_attn_decode with the library's static per-GPU scratch as the
    workspace: nothing is allocated, by the binding or the library (for code
    under graph capture and loops that must not allocate). Calls that may
    overlap on one GPU race on the shared scratch; a call that needs more
    than its 64 MiB raises PagedKVError (PKV_ERR_WORKSPACE)."""
    _require(query.dim() == 3 and out.shape == query.shape, "query/out must be [S, H, D]")
    _require(key_cache.dim() == 4 and value_cache.shape == key_cache.shape,
             "pools must be [num_blocks, block_size, num_kv_heads, head_dim]")
    _require(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32,
             "block_table and seq_lens must be int32")
    _require(query.dtype == key_cache.dtype == value_cache.dtype, "query and pools share a dtype")
    S, H, D = query.shape
    NB, bs, Hkv, D2 = key_cache.shape
    _require(D2 == D, "head_dim of query and pools differ")
    _require(block_table.dim() == 2 and block_table.shape[0] == S and seq_lens.shape == (S,),
             "block_table must be [S, max_blocks] and seq_lens [S]")
    st = lib().paged_attn_decode_noalloc(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_table),
        _ptr(seq_lens), S, H, Hkv, D, bs, NB, block_table.shape[1], int(max_seq_len), float(scale),
        dtype_code(query.dtype), dtype_code(out.dtype), int(partition_size), _stream(query, stream))
    check(st, "paged_attn_decode_noalloc")
    return out


def paged_attn_multi_query(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                           value_cache: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, scale: float, max_seq_len: int,
                           partition_size: int = 0, workspace: torch.Tensor | None = None,
                           stream=None, events=None) -> torch.Tensor:
    """Causal attention of the last ``q_len`` tokens of each sequence (query
    ``[S, q_len, H, D]``; their K/V already written to the pool): new token j
    sees positions ``0 .. seq_len - q_len + j``. ``q_len * (H / Hkv)`` must be
    at most 128 (the query rows of one KV head). Workspace rules as for
    paged_attn_decode, sized by ``paged_attn_multi_query_workspace_size``."""
    return _attention("paged_attn_multi_query", out, query, key_cache, value_cache,
                      block_table, seq_lens, scale, max_seq_len, partition_size, workspace,
                      stream, events=events)


def paged_attn_decode_fp8(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                          value_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                          block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                          max_seq_len: int, partition_size: int = 0,
                          workspace: torch.Tensor | None = None, stream=None,
                          events=None) -> torch.Tensor:
    """Decode over e4m3 pools: code * k_scale[kv head] and code * v_scale[kv head]
    stand for K and V. query bf16/fp16 [S, H, D]; out of the query's type or fp32."""
    return _attention("paged_attn_decode_fp8", out, query, key_cache, value_cache, block_table,
                      seq_lens, scale, max_seq_len, partition_size, workspace, stream,
                      k_scale, v_scale, events=events)


def paged_attn_multi_query_fp8(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                               value_cache: torch.Tensor, k_scale: torch.Tensor,
                               v_scale: torch.Tensor, block_table: torch.Tensor,
                               seq_lens: torch.Tensor, scale: float, max_seq_len: int,
                               partition_size: int = 0, workspace: torch.Tensor | None = None,
                               stream=None, events=None) -> torch.Tensor:
    """paged_attn_multi_query over e4m3 pools (query [S, q_len, H, D])."""
    return _attention("paged_attn_multi_query_fp8", out, query, key_cache, value_cache,
                      block_table, seq_lens, scale, max_seq_len, partition_size, workspace,
                      stream, k_scale, v_scale, events=events)


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                          value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                          k_scale: torch.Tensor, v_scale: torch.Tensor, stream=None) -> None:
    """Quantise each new token's K and V (fp32/fp16/bf16) into e4m3 codes of
    x / scale[kv head] at slot_mapping[i] of the uint8 pools."""
    _require(key.dim() == 3 and value.shape == key.shape, "key/value must be [T, Hkv, D]")
    _require(key_cache.dim() == 4 and value_cache.shape == key_cache.shape, "pool shape")
    _require(dtype_code(key_cache.dtype) == PKV_E4M3 and key_cache.dtype == value_cache.dtype,
             "e4m3 pools must be uint8 or float8_e4m3fn")
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (key.shape[0],),
             "slot_mapping must be int64 [T]")
    _require(key.dtype == value.dtype and key.dtype in (torch.float32, torch.float16,
                                                        torch.bfloat16), "key/value dtype")
    NB, bs, Hkv, D = key_cache.shape
    _require(tuple(key.shape[1:]) == (Hkv, D), "key rows must be [num_kv_heads, head_dim]")
    _require(k_scale.dtype == torch.float32 and v_scale.dtype == torch.float32
             and k_scale.shape == v_scale.shape == (Hkv,), "scales must be fp32 [num_kv_heads]")
    st = lib().reshape_and_cache_fp8(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                     _ptr(slot_mapping), _ptr(k_scale), _ptr(v_scale),
                                     key.shape[0], Hkv, D, bs, NB, dtype_code(key.dtype),
                                     _stream(key_cache, stream))
    check(st, "reshape_and_cache_fp8")


def paged_attn_decode_shared_prefix(out: torch.Tensor, query: torch.Tensor,
                                    key_cache: torch.Tensor, value_cache: torch.Tensor,
                                    prefix_block_table: torch.Tensor, prefix_lens: torch.Tensor,
                                    suffix_block_table: torch.Tensor, suffix_lens: torch.Tensor,
                                    group_size: int, scale: float, max_prefix_len: int,
                                    max_suffix_len: int, partition_size: int = 0,
                                    workspace: torch.Tensor | None = None,
                                    stream=None, k_scale: torch.Tensor | None = None,
                                    v_scale: torch.Tensor | None = None) -> torch.Tensor:
    """Decode for groups of group_size consecutive sequences that share a
    prefix of whole blocks: sequence s of group g attends over
    prefix_block_table[g] (prefix_lens[g] tokens) then suffix_block_table[s]
    (suffix_lens[s] tokens); each shared block is read once per group. With
    k_scale and v_scale (fp32 [num_kv_heads]) the pools hold e4m3 codes
    (paged_attn_decode_shared_prefix_fp8) and the query is fp16 or bf16."""
    f8 = k_scale is not None or v_scale is not None
    _require(query.dim() == 3 and out.shape == query.shape, "query/out must be [S, H, D]")
    _require(key_cache.dim() == 4 and value_cache.shape == key_cache.shape, "pool shape")
    if f8:
        _require(dtype_code(key_cache.dtype) == PKV_E4M3 and key_cache.dtype == value_cache.dtype,
                 "e4m3 pools must be uint8 or float8_e4m3fn")
        _require(query.dtype in (torch.float16, torch.bfloat16), "the query must be fp16 or bf16")
        _require(k_scale is not None and v_scale is not None and k_scale.dtype == torch.float32
                 and v_scale.dtype == torch.float32
                 and k_scale.shape == v_scale.shape == (key_cache.shape[2],),
                 "k_scale and v_scale must be fp32 [num_kv_heads]")
    else:
        _require(query.dtype == key_cache.dtype == value_cache.dtype, "query and pools share a dtype")
    for t in (prefix_block_table, prefix_lens, suffix_block_table, suffix_lens):
        _require(t.dtype == torch.int32, "tables and lengths must be int32")
    S, H, D = query.shape
    NB, bs, Hkv, D2 = key_cache.shape
    _require(D2 == D and group_size >= 1 and S % group_size == 0, "shapes / group size")
    G = S // group_size
    _require(prefix_block_table.dim() == 2 and prefix_block_table.shape[0] == G
             and prefix_lens.shape == (G,), "prefix table [groups, blocks], lens [groups]")
    _require(suffix_block_table.dim() == 2 and suffix_block_table.shape[0] == S
             and suffix_lens.shape == (S,), "suffix table [S, blocks], lens [S]")
    if workspace is None:
        n = int(lib().paged_attn_shared_prefix_workspace_size(G, group_size, H, Hkv, D, bs,
                                                              int(max_prefix_len),
                                                              int(max_suffix_len),
                                                              int(partition_size)))
        workspace = _zeroed_on(query, stream, max(n, 256))
    ws_bytes = workspace.numel() * workspace.element_size()
    name = "paged_attn_decode_shared_prefix_fp8" if f8 else "paged_attn_decode_shared_prefix"
    scales = [_ptr(k_scale), _ptr(v_scale)] if f8 else []
    st = getattr(lib(), name)(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), *scales, _ptr(prefix_block_table),
        _ptr(prefix_lens), G, group_size, prefix_block_table.shape[1], int(max_prefix_len),
        _ptr(suffix_block_table), _ptr(suffix_lens), suffix_block_table.shape[1],
        int(max_suffix_len), H, Hkv, D, bs, NB, float(scale), dtype_code(query.dtype),
        dtype_code(out.dtype), int(partition_size), _ptr(workspace), ws_bytes,
        _stream(query, stream))
    check(st, name)
    return out


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                      stream=None) -> None:
    """Write each new token's K and V into slot_mapping[i] of the pools."""
    _require(key.dim() == 3 and value.shape == key.shape, "key/value must be [T, Hkv, D]")
    _require(key_cache.dim() == 4 and value_cache.shape == key_cache.shape, "pool shape")
    _require(slot_mapping.dtype == torch.int64 and slot_mapping.shape == (key.shape[0],),
             "slot_mapping must be int64 [T]")
    _require(key.dtype == key_cache.dtype == value.dtype == value_cache.dtype, "dtypes differ")
    NB, bs, Hkv, D = key_cache.shape
    _require(tuple(key.shape[1:]) == (Hkv, D), "key rows must be [num_kv_heads, head_dim]")
    st = lib().reshape_and_cache(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                 _ptr(slot_mapping), key.shape[0], Hkv, D, bs, NB,
                                 dtype_code(key.dtype), _stream(key_cache, stream))
    check(st, "reshape_and_cache")


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor,
                block_mapping: torch.Tensor, stream=None) -> None:
    """Copy whole blocks src -> dst (K and V) for each row (src, dst)."""
    _require(key_cache.dim() == 4 and value_cache.shape == key_cache.shape, "pool shape")
    _require(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
             and block_mapping.shape[1] == 2, "block_mapping must be int64 [P, 2]")
    _require(key_cache.dtype == value_cache.dtype, "dtypes differ")
    NB, bs, Hkv, D = key_cache.shape
    st = lib().copy_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(block_mapping),
                           block_mapping.shape[0], NB, bs, Hkv, D, dtype_code(key_cache.dtype),
                           _stream(key_cache, stream))
    check(st, "copy_blocks")


def swap_blocks(src_key_cache: torch.Tensor, src_value_cache: torch.Tensor,
                dst_key_cache: torch.Tensor, dst_value_cache: torch.Tensor,
                block_mapping: torch.Tensor, stream=None) -> None:
    """Copy whole blocks src -> dst (K and V) between two pools, for each row
    (src, dst) of block_mapping: swapping out to pinned host pools
    (``pin_memory=True``) and back in. Pools on the GPU or in pinned host
    memory; the work runs on the stream of the GPU side."""
    _require(src_key_cache.dim() == 4 and src_value_cache.shape == src_key_cache.shape,
             "source pool shape")
    _require(dst_key_cache.dim() == 4 and dst_value_cache.shape == dst_key_cache.shape,
             "destination pool shape")
    _require(tuple(src_key_cache.shape[1:]) == tuple(dst_key_cache.shape[1:]),
             "pools differ in block layout")
    _require(src_key_cache.dtype == dst_key_cache.dtype == src_value_cache.dtype
             == dst_value_cache.dtype, "dtypes differ")
    _require(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
             and block_mapping.shape[1] == 2, "block_mapping must be int64 [P, 2]")
    for t in (src_key_cache, src_value_cache, dst_key_cache, dst_value_cache, block_mapping):
        _require(t.is_cuda or t.is_pinned(), "pools and mapping must be on the GPU or pinned")
    NBs, bs, Hkv, D = src_key_cache.shape
    gpu = next((t for t in (src_key_cache, dst_key_cache, block_mapping) if t.is_cuda), None)
    _require(gpu is not None or stream is not None, "give a stream when no pool is on the GPU")
    st = lib().swap_blocks(_ptr(src_key_cache), _ptr(src_value_cache), _ptr(dst_key_cache),
                           _ptr(dst_value_cache), _ptr(block_mapping), block_mapping.shape[0], NBs,
                           dst_key_cache.shape[0], bs, Hkv, D, dtype_code(src_key_cache.dtype),
                           _stream(gpu if gpu is not None else src_key_cache, stream))
    check(st, "swap_blocks")


def check_decode_inputs(block_table: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                        num_blocks: int, max_seq_len: int, stream=None) -> tuple[int, int]:
    """(bad block-table entries, bad lengths), counted on the device; waits
    for the call's stream."""
    ts = _torch_stream(block_table, stream)
    with torch.cuda.stream(ts):
        counts = torch.empty(2, dtype=torch.int32, device=block_table.device)
    S = block_table.shape[0]
    st = lib().pagedkv_check_decode_inputs(_ptr(block_table), _ptr(seq_lens), S, block_size,
                                           num_blocks, block_table.shape[1], max_seq_len,
                                           _ptr(counts), ts.cuda_stream)
    check(st, "pagedkv_check_decode_inputs")
    ts.synchronize()
    c = counts.cpu()
    return int(c[0]), int(c[1])


def check_cache_op_inputs(slot_mapping: torch.Tensor | None, block_mapping: torch.Tensor | None,
                          block_size: int, num_blocks: int,
                          stream=None) -> tuple[int, int, int, int]:
    """(slots outside the pool, repeated slots, pairs with an id outside the
    pool, pairs whose destination is a source or repeats), counted on the
    device for reshape_and_cache's slot_mapping (int64 [T]) and copy_blocks'
    block_mapping (int64 [P, 2]); either may be None. Waits for the call's
    stream."""
    ref = slot_mapping if slot_mapping is not None else block_mapping
    _require(ref is not None, "give slot_mapping or block_mapping")
    if slot_mapping is not None:
        _require(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1,
                 "slot_mapping must be int64 [T]")
    if block_mapping is not None:
        _require(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
                 and block_mapping.shape[1] == 2, "block_mapping must be int64 [P, 2]")
    ts = _torch_stream(ref, stream)
    with torch.cuda.stream(ts):
        counts = torch.empty(4, dtype=torch.int32, device=ref.device)
    T = 0 if slot_mapping is None else slot_mapping.shape[0]
    P = 0 if block_mapping is None else block_mapping.shape[0]
    st = lib().pagedkv_check_cache_op_inputs(_ptr(slot_mapping), T, int(block_size), int(num_blocks),
                                             _ptr(block_mapping), P, _ptr(counts), ts.cuda_stream)
    check(st, "pagedkv_check_cache_op_inputs")
    ts.synchronize()
    return tuple(int(x) for x in counts.cpu())


def stream_read(buf: torch.Tensor, sink: torch.Tensor, grid: int, stream=None) -> None:
    """Read ``buf`` once with the streaming-read kernel (measurement aid; see
    pagedkv_stream_read in include/pagedkv.h). ``sink`` is int32/uint32 with
    at least ``grid`` elements."""
    _require(buf.is_contiguous() and buf.numel() * buf.element_size() % 16 == 0,
             "buffer must be contiguous, a multiple of 16 bytes")
    _require(sink.numel() >= grid and sink.element_size() == 4, "sink needs grid 32-bit words")
    st = lib().pagedkv_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                   int(grid), _stream(buf, stream))
    check(st, "pagedkv_stream_read")

