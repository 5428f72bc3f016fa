"""Benchmark of the paged decode hot path on one MI355X.

One step = one layer's decode step of the Llama-2-70B-shaped batch (256
sequences, 64 query / 8 KV heads, head_dim 128, fp16 KV, block_size 32,
lengths lognormal with median 1024 clipped to [32, 8192], blocks placed at
random in a pool of 1.2x the blocks needed): paged_attn_decode over all
cached tokens. Steps rotate over ``--layers`` copies of the layer's pools
(same shapes and tables), so that a step never finds its K/V in the 256 MB
Infinity Cache or the L2 from the previous use of the same pool.

Prints one JSON line. ``value`` is KV GB/s: the algorithmic KV bytes a step
must read (every cached token's K and V rows, once) over the measured step
time. The roofline entry is for the decode call (one kernel: the split
sequences are merged by their last partition), its duration the kernel's own
start-to-end time from events its launch sets, on the stream the library
launches on. The same measurement of the Llama-3-8B-shaped step (64
sequences, 32 / 8 heads, bf16, block_size 16, lengths uniform in [512, 4096]:
reshape_and_cache of the 64 new tokens, then decode) rides along under the
key ``llama3_8b_bf16``; ``--workload llama3_8b_bf16`` makes it the headline.

The line also carries the streaming-read rate the same GPU reaches (the
library's stream-read kernel over a 4 GiB buffer, best of a few grid sizes)
and the decode call's share of it, and p10/p50/p90 of the decode call.
``--secondary`` adds the measurements the pages give context for: a
block-size sweep (8, 16, 32) of the Llama-3-8B lengths and paged vs
contiguous placement of the same blocks. ``--per-config`` adds every
page-shaped workload (the Llama-3-8B and Llama-2-70B layers, the
prefix-sharing batch and the mixed batch with split sequences): decode calls
timed cold, with p10/p50/p90, and the scatter and block copy of each step.
``--multi-query`` adds the verification pass of speculative decoding (q_len
2, 4 and 8 new tokens per sequence, causal) on the Llama-3-8B lengths, beside
decode; ``--q-len Q`` makes that pass, with its scatter of 64 x Q tokens, the
timed step itself (on the Llama-3-8B batch; the profile of it then covers
that pass alone). ``--kv-fp8`` times the e4m3 step of the Llama-3-8B batch.

    python bench.py [--steps K] [--warmup W] [--layers N] [--workload W] [--no-cpu-baseline]
                    [--secondary] [--per-config] [--multi-query] [--q-len Q] [--kv-fp8]
"""

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
METRIC = "paged decode attention: KV GB/s and % of HBM peak; sequences/s per layer"

# headline-able workloads: name -> (config number, description, lengths)
WORKLOADS = {
    "llama2_70b_fp16": (3, "Llama-2-70B-shaped single-layer decode",
                        "lognormal, median 1024, sigma 1.0, clipped to [32, 8192], seed 1543"),
    "llama3_8b_bf16": (2, "Llama-3-8B-shaped single-layer decode", "uniform [512, 4096], seed 1542"),
    "prefix_share_bf16": (4, "parallel-sampling batch, 128 prompts x 3 samples sharing a "
                             "2048-token prefix, plain decode of every sample",
                          "2048 + uniform [0, 512], seed 1544"),
    "mixed_splitk_bf16": (5, "mixed batch, 16 x 10000 + 240 x uniform [50, 2000] tokens, "
                             "block_size 8, 512-token partitions",
                          "16 x 10000 + 240 x uniform [50, 2000], shuffled, seed 1545"),
}


def kernel_source_hash():
    """sha256 of the decode kernel sources (as in the traffic profile), with
    their comments and blank lines left out: the measured traffic belongs to
    the code, which a change of comments leaves as it was."""
    h = hashlib.sha256()
    for f in ("decode.hip", "pagedkv_internal.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_154_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()


def measured_traffic(name="decode_llama3_8b_bf16"):
    """HBM bytes per attention call from the committed rocprofv3 counter runs
    of this workload, or None when there are none or the kernel sources
    changed after them."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    try:
        with open(path) as fh:
            doc = json.load(fh)
    except OSError:
        return None
    if doc.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return doc.get("traffic_bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def stream_read_peak(dev, gib=4, reps=8):
    """Best median streaming-read rate (GB/s) of the library's stream-read
    kernel over a buffer much larger than L2 and the Infinity Cache."""
    import torch

    import paged_kv_cache_154_amd as pkv
    buf = torch.empty(gib << 28, dtype=torch.float32, device=dev)
    buf.fill_(1.0)
    nbytes = buf.numel() * 4
    best = 0.0
    for grid in (2048, 4096, 8192, 16384):
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        pkv.stream_read(buf, sink, grid)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            pkv.stream_read(buf, sink, grid)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        rate = nbytes / (statistics.median(ts) * 1e-3) / 1e9
        log(f"stream read, grid {grid}: {rate:.0f} GB/s")
        best = max(best, rate)
    del buf
    return best


def time_decode(pkv, wl, dev, layers=2, calls=100, P=0, warm=20):
    """Median decode-call time (us) of a workload, the kernels' own start to
    end (events the launch sets): calls queued back to back (as in the timed
    steps) after `warm` untimed ones, rotating over layer copies of the
    pools. A workload with several new tokens per sequence runs the
    multi-query pass."""
    import torch
    attn = pkv.paged_attn_decode if wl.q_len == 1 else pkv.paged_attn_multi_query
    q = wl.query.to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    kc0, vc0 = wl.key_cache.to(dev), wl.value_cache.to(dev)
    if wl.new_key is not None:        # fill the slot this step's token occupies
        pkv.reshape_and_cache(wl.new_key.to(dev), wl.new_value.to(dev), kc0, vc0,
                              torch.from_numpy(wl.slot_mapping).to(dev))
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(layers - 1)]
    out = torch.empty(wl.query.shape, dtype=wl.dtype, device=dev)
    ws = pkv.workspace_for(q, kc0, wl.max_seq_len, P)
    for i in range(warm):
        kc, vc = pools[i % layers]
        attn(out, q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, P, ws)
    ev = _events(calls)
    torch.cuda.synchronize()
    for i in range(calls):
        kc, vc = pools[i % layers]
        attn(out, q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, P, ws, events=ev[i])
    torch.cuda.synchronize()
    del pools
    return statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)


def secondary(pkv, W, base, dev):
    """Block-size sweep and paged vs contiguous placement on the same lengths
    (context from the pages: bs 16 best; paged placement within a few
    percent of contiguous)."""
    import dataclasses

    import numpy as np
    import torch
    lens = base.seq_lens.tolist()
    out = {"block_size_sweep": {}, "placement": {}}
    for bs in (8, 16, 32):
        wl = W.custom(1542, seq_lens=lens, num_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=bs, dtype=torch.bfloat16)
        t = time_decode(pkv, wl, dev)
        out["block_size_sweep"][str(bs)] = {"decode_us": round(t, 1),
                                            "kv_GBps": round(wl.kv_bytes() / t / 1e3, 1)}
        log(f"block_size {bs}: {t:.1f} us")
        del wl
    # contiguous: relabel the blocks so each sequence's are consecutive
    wl = base
    order, seen = [], set()
    for s_ in range(wl.num_seqs):
        nb_ = (int(wl.seq_lens[s_]) + wl.block_size - 1) // wl.block_size
        for b_ in wl.block_table[s_, :nb_]:
            if int(b_) not in seen:
                seen.add(int(b_))
                order.append(int(b_))
    order = np.array(order + [b_ for b_ in range(wl.num_blocks) if b_ not in seen])
    newid = np.empty_like(order)
    newid[order] = np.arange(order.size)
    t_paged = time_decode(pkv, wl, dev)
    perm = torch.from_numpy(order)
    contig = dataclasses.replace(wl, key_cache=wl.key_cache[perm].contiguous(),
                                 value_cache=wl.value_cache[perm].contiguous(),
                                 block_table=newid[wl.block_table].astype(np.int32))
    t_contig = time_decode(pkv, contig, dev)
    out["placement"] = {"paged_us": round(t_paged, 1), "contiguous_us": round(t_contig, 1),
                        "paged_over_contiguous": round(t_paged / t_contig, 4)}
    log(f"placement: paged {t_paged:.1f} us, contiguous {t_contig:.1f} us")
    return out


def multi_query_rows(pkv, W, base, dev, q_lens=(2, 4, 8)):
    """The verification pass of speculative decoding on the Llama-3-8B-shaped
    lengths and placement of the decode step:
    q_len new tokens per sequence (their K/V scattered first), each KV head's
    blocks read once for all q_len x G query rows. Back-to-back medians beside
    decode of the same batch; KV GB/s over the same pool bytes."""
    import torch
    G = base.num_heads // base.num_kv_heads
    t_dec = time_decode(pkv, base, dev)
    rows = {"decode_us": round(t_dec, 1)}
    for Q in q_lens:
        if Q * G > 128:
            continue
        wl = W.llama3_8b(q_len=Q)
        t = time_decode(pkv, wl, dev)
        rows[f"q_len={Q}"] = {"us": round(t, 1), "kv_GBps": round(wl.kv_bytes() / t / 1e3, 1),
                              "over_decode": round(t / t_dec, 3),
                              "tokens_per_s": round(Q * wl.num_seqs / (t * 1e-6), 1)}
        log(f"multi-query q_len={Q}: {t:.1f} us (decode {t_dec:.1f} us)")
        del wl
        torch.cuda.empty_cache()
    return rows


def swap_rows(pkv, wl, dev, n_seqs=16, reps=20):
    """Preemption by swapping on the Llama-3-8B-shaped pools: the blocks of
    n_seqs sequences swapped out to pinned host pools and back in (one
    swap_blocks call each way, medians over reps), beside the host link's own
    rate: a contiguous device <-> pinned copy of the same bytes."""
    import torch
    bs = wl.block_size
    blocks = [int(b) for s_ in range(n_seqs)
              for b in wl.block_table[s_, :(int(wl.seq_lens[s_]) + bs - 1) // bs]]
    n = len(blocks)
    kc, vc = wl.key_cache.to(dev), wl.value_cache.to(dev)
    hk = torch.empty((n,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    out_map = torch.tensor([[b, i] for i, b in enumerate(blocks)], dtype=torch.int64, device=dev)
    in_map = torch.tensor([[i, b] for i, b in enumerate(blocks)], dtype=torch.int64, device=dev)
    nbytes = 2 * n * kc[0].numel() * kc.element_size()

    def med_us(fn):
        fn()
        ev = _events(reps)
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return statistics.median(_us(ev))

    t_out = med_us(lambda: pkv.swap_blocks(kc, vc, hk, hv, out_map))
    t_in = med_us(lambda: pkv.swap_blocks(hk, hv, kc, vc, in_map))
    dbuf = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    hbuf = torch.empty(nbytes // 2, dtype=torch.int16, pin_memory=True)
    t_d2h = med_us(lambda: hbuf.copy_(dbuf, non_blocking=True))
    t_h2d = med_us(lambda: dbuf.copy_(hbuf, non_blocking=True))
    log(f"swap {n} blocks ({nbytes / 1e6:.1f} MB): out {t_out:.0f} us, in {t_in:.0f} us; "
        f"link copies {t_d2h:.0f} / {t_h2d:.0f} us")
    del kc, vc, dbuf
    torch.cuda.empty_cache()
    return {"sequences": n_seqs, "blocks": n, "bytes": nbytes,
            "swap_out_us": round(t_out, 1), "swap_out_GBps": round(nbytes / t_out / 1e3, 2),
            "swap_in_us": round(t_in, 1), "swap_in_GBps": round(nbytes / t_in / 1e3, 2),
            "link_copy_d2h_GBps": round(nbytes / t_d2h / 1e3, 2),
            "link_copy_h2d_GBps": round(nbytes / t_h2d / 1e3, 2)}


def _events(n):
    import torch
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n)]


def _us(ev):
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def _pcts(xs):
    q = statistics.quantiles(xs, n=10)
    return round(q[0], 2), round(statistics.median(xs), 2), round(q[-1], 2)


def layout_stats(wl):
    """Slots the pool holds for the batch vs tokens it stores, and (when
    blocks are shared) logical vs distinct blocks and bytes."""
    import numpy as np
    bs = wl.block_size
    logical_blocks = int(sum((int(L) + bs - 1) // bs for L in wl.seq_lens))
    slots = []
    for s_, L in enumerate(wl.seq_lens.tolist()):
        t = np.arange(L, dtype=np.int64)
        slots.append(wl.block_table[s_, t // bs].astype(np.int64) * bs + t % bs)
    uniq_slots = int(np.unique(np.concatenate(slots)).size) if slots else 0
    return {
        "logical_blocks": logical_blocks,
        "distinct_blocks": int(wl.unique_blocks),
        "slot_utilisation": round(uniq_slots / max(1, wl.unique_blocks * bs), 4),
        "block_saving_from_sharing": round(1 - wl.unique_blocks / max(1, logical_blocks), 4),
        "kv_bytes_distinct": uniq_slots * 2 * wl.num_kv_heads * wl.head_dim * wl.elem_bytes,
    }


def per_config(pkv, W, dev, calls=200, warm=20):
    """Every page-shaped workload (configs 2-5): each decode call timed cold
    (a 1 GiB streaming read evicts L2 and the Infinity Cache before it,
    outside the events; a read, because a write flush leaves dirty lines
    whose write-back would be charged to the call) by the kernel's own start
    and end (events its launch sets, paged_attn_timed), median and p10/p90, a
    warm back-to-back mean, and the cache ops of the step (mean of
    back-to-back calls: one event pair per call would dwarf a few-us kernel)."""
    import torch
    fbuf = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    fsink = torch.empty(8192, dtype=torch.int32, device=dev)

    def flush():
        pkv.stream_read(fbuf, fsink, 8192)

    def mean_us(fn, n=50):
        fn()
        a, b = _events(1)[0]
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return round(a.elapsed_time(b) * 1e3 / n, 2)

    res = {}
    for c in (2, 3, 4, 5):
        log(f"config {c}: generating")
        wl = W.make(c)
        q = wl.query.to(dev)
        bt = torch.from_numpy(wl.block_table).to(dev)
        sl = torch.from_numpy(wl.seq_lens).to(dev)
        kc, vc = wl.key_cache.to(dev), wl.value_cache.to(dev)
        out = torch.empty(wl.query.shape, dtype=wl.dtype, device=dev)
        S, H, D = wl.query.shape
        row = {"workload": wl.name, "num_seqs": S, "num_heads": H, "num_kv_heads": wl.num_kv_heads,
               "head_dim": D, "block_size": wl.block_size, "tokens": wl.num_tokens,
               "kv_bytes": wl.kv_bytes(), **layout_stats(wl)}
        if wl.new_key is not None:
            nk, nv = wl.new_key.to(dev), wl.new_value.to(dev)
            slots = torch.from_numpy(wl.slot_mapping).to(dev)
            t = mean_us(lambda: pkv.reshape_and_cache(nk, nv, kc, vc, slots))
            nbytes = 4 * nk.numel() * nk.element_size()
            row["reshape_and_cache"] = {"mean_us": t, "bytes": nbytes}
        if wl.block_mapping is not None:
            bm = torch.from_numpy(wl.block_mapping).to(dev)
            t = mean_us(lambda: pkv.copy_blocks(kc, vc, bm))
            nbytes = 4 * bm.shape[0] * kc[0].numel() * kc.element_size()
            row["copy_blocks"] = {"mean_us": t, "bytes": nbytes, "pairs": int(bm.shape[0])}
        row["decode"] = {}
        for P in sorted({wl.partition_size, 0}):
            ws = pkv.workspace_for(q, kc, wl.max_seq_len, P)
            for _ in range(warm):
                pkv.paged_attn_decode(out, q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, P, ws)
            ev = _events(calls)
            for a, b in ev:
                flush()
                pkv.paged_attn_decode(out, q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, P, ws,
                                      events=(a, b))
            w0, w1 = _events(1)[0]
            w0.record()
            for _ in range(warm):
                pkv.paged_attn_decode(out, q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, P, ws)
            w1.record()
            torch.cuda.synchronize()
            p10, p50, p90 = _pcts(_us(ev))
            gbs = wl.kv_bytes() / p50 / 1e3
            part = pkv.paged_attn_partition_tokens(S, wl.num_kv_heads, wl.block_size,
                                                   wl.max_seq_len, P, num_heads=wl.num_heads,
                                                   kv_dtype=pkv.dtype_code(wl.dtype))
            row["decode"][f"partition_size={P}"] = {
                "partition_tokens": part, "cold_us_p10_p50_p90": [p10, p50, p90],
                "warm_mean_us": round(w0.elapsed_time(w1) * 1e3 / warm, 2),
                "kv_GBps": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
                "seqs_per_s": round(S / (p50 * 1e-6), 1)}
            log(f"config {c} P={P} ({part} tokens): cold median {p50:.1f} us, {gbs:.0f} GB/s")
        res[str(c)] = row
        del wl, q, bt, sl, kc, vc, out
        torch.cuda.empty_cache()
    del fbuf
    return res


def fp8_scales(pool):
    """A scale per KV head for an e4m3 cache: the largest finite magnitude of
    the 16-bit pool over 448 (a caller's calibration, outside the method)."""
    import torch
    a = torch.nan_to_num(pool.float().abs(), nan=0.0, posinf=0.0, neginf=0.0)
    return (a.amax(dim=(0, 1, 3)) / 448.0).clamp_min(1e-6).contiguous()


def prefix_share_rows(pkv, W, dev, calls=100, warm=10):
    """The prefix-sharing workload (128 groups x 3 samples, 2032 shared
    tokens per group after the copy-on-write step): decode of the batch and
    shared-prefix decode of the same batch (each group's shared blocks read
    once), each call timed cold after a 1 GiB streaming read, medians; GB/s
    on the logical bytes (every sample's whole context) and on the distinct
    bytes (shared blocks once). The same two calls over the pools stored as
    e4m3 codes (quantised once, a scale per KV head; half the bytes)."""
    import torch
    wl = W.make(4)
    kc, vc = wl.key_cache.to(dev), wl.value_cache.to(dev)
    pkv.copy_blocks(kc, vc, torch.from_numpy(wl.block_mapping).to(dev))
    q = wl.query.to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    pt, pl, st, sl2 = [torch.from_numpy(x).to(dev) for x in W.shared_prefix_tables(wl, 3)]
    out = torch.empty(wl.query.shape, dtype=wl.dtype, device=dev)
    ws = pkv.workspace_for(q, kc, wl.max_seq_len, 0)
    fbuf = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    fsink = torch.empty(8192, dtype=torch.int32, device=dev)
    mp, ms = int(pl.max()), int(sl2.max())
    n = pkv.lib().paged_attn_shared_prefix_workspace_size(128, 3, wl.num_heads, wl.num_kv_heads,
                                                          wl.head_dim, wl.block_size, mp, ms, 0)
    ws2 = torch.zeros(n, dtype=torch.uint8, device=dev)   # control areas zero at first use
    NB, bs, Hkv, D = kc.shape
    ks, vs = fp8_scales(kc), fp8_scales(vc)
    k8 = torch.empty(kc.shape, dtype=torch.uint8, device=dev)
    v8 = torch.empty_like(k8)
    pkv.reshape_and_cache_fp8(kc.view(-1, Hkv, D), vc.view(-1, Hkv, D), k8, v8,
                              torch.arange(NB * bs, dtype=torch.int64, device=dev), ks, vs)
    fns = {"decode": lambda: pkv.paged_attn_decode(out, q, kc, vc, bt, sl, wl.scale,
                                                   wl.max_seq_len, 0, ws),
           "shared_prefix": lambda: pkv.paged_attn_decode_shared_prefix(
               out, q, kc, vc, pt, pl, st, sl2, 3, wl.scale, mp, ms, 0, ws2),
           "decode_e4m3": lambda: pkv.paged_attn_decode_fp8(out, q, k8, v8, ks, vs, bt, sl, wl.scale,
                                                            wl.max_seq_len, 0, ws),
           "shared_prefix_e4m3": lambda: pkv.paged_attn_decode_shared_prefix(
               out, q, k8, v8, pt, pl, st, sl2, 3, wl.scale, mp, ms, 0, ws2, k_scale=ks, v_scale=vs)}
    logical = wl.kv_bytes()
    distinct = layout_stats(wl)["kv_bytes_distinct"]
    res = {"logical_kv_bytes": logical, "distinct_kv_bytes": distinct}
    for name, fn in fns.items():
        half = 2 if name.endswith("e4m3") else 1   # one byte per element
        for _ in range(warm):
            fn()
        ev = _events(calls)
        for a, b in ev:
            pkv.stream_read(fbuf, fsink, 8192)
            a.record()
            fn()
            b.record()
        w0, w1 = _events(1)[0]
        w0.record()
        for _ in range(warm):
            fn()
        w1.record()
        torch.cuda.synchronize()
        p10, p50, p90 = _pcts(_us(ev))
        res[name] = {"cold_us_p10_p50_p90": [p10, p50, p90],
                     "warm_mean_us": round(w0.elapsed_time(w1) * 1e3 / warm, 2),
                     "logical_GBps": round(logical / half / p50 / 1e3, 1),
                     "distinct_GBps": round(distinct / half / p50 / 1e3, 1)}
        log(f"prefix share, {name}: cold median {p50:.1f} us")
    res["speedup"] = round(res["decode"]["cold_us_p10_p50_p90"][1]
                           / res["shared_prefix"]["cold_us_p10_p50_p90"][1], 3)
    res["speedup_e4m3"] = round(res["decode_e4m3"]["cold_us_p10_p50_p90"][1]
                                / res["shared_prefix_e4m3"]["cold_us_p10_p50_p90"][1], 3)
    del kc, vc, k8, v8, fbuf
    torch.cuda.empty_cache()
    return res


def cpu_baseline_fp8(wl, ks, vs, n_seqs=8, budget_s=20.0):
    """The CPU oracle on the e4m3 step for a sample of the batch: the first
    n_seqs sequences' blocks quantised beforehand (not timed), then the timed
    oracle step: the quantising scatter of their new tokens and fp8 decode."""
    import numpy as np
    import torch

    from oracle import fp8_kv as F
    bs = wl.block_size
    Hkv = wl.num_kv_heads
    seqs = list(range(min(n_seqs, wl.num_seqs)))
    blocks = sorted({int(b) for s_ in seqs
                     for b in wl.block_table[s_, :(int(wl.seq_lens[s_]) + bs - 1) // bs]})
    remap = {b: i for i, b in enumerate(blocks)}
    idx = torch.tensor(blocks, dtype=torch.int64)
    k_s, v_s = ks.cpu().numpy(), vs.cpu().numpy()
    kq = F.quantize(wl.key_cache[idx], k_s.reshape(1, 1, Hkv, 1))
    vq = F.quantize(wl.value_cache[idx], v_s.reshape(1, 1, Hkv, 1))
    table = np.zeros_like(wl.block_table[:len(seqs)])
    for s_ in seqs:
        nb_ = (int(wl.seq_lens[s_]) + bs - 1) // bs
        table[s_, :nb_] = [remap[int(b)] for b in wl.block_table[s_, :nb_]]
    tok = [i for i, sl_ in enumerate(wl.slot_mapping.tolist()) if sl_ // bs in remap]
    slots = np.array([remap[wl.slot_mapping[i] // bs] * bs + wl.slot_mapping[i] % bs for i in tok])
    lens = wl.seq_lens[:len(seqs)]
    times = []
    while len(times) < 3 and sum(times) < budget_s:
        t0 = time.perf_counter()
        k2, v2 = F.reshape_and_cache_fp8(wl.new_key[tok], wl.new_value[tok], kq, vq, slots, k_s, v_s)
        attn = F.decode_fp8 if wl.q_len == 1 else F.multi_query_fp8
        attn(wl.query[:len(seqs)], k2, v2, k_s, v_s, table, lens, wl.scale)
        times.append(time.perf_counter() - t0)
        log(f"cpu oracle fp8 step {len(times)}: {times[-1]:.2f} s")
    t = statistics.median(times)
    nbytes = int(lens.astype(np.int64).sum()) * 2 * Hkv * wl.head_dim
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": (f"the e4m3 step for the first {len(seqs)} of the {wl.num_seqs} sequences "
                       f"({int(lens.sum())} tokens: oracle quantising scatter of their new tokens + "
                       f"fp64 decode over the dequantised codes), median of {len(times)} run(s), "
                       f"{t:.2f} s"),
            "seconds_per_step": round(t, 3)}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_step(wl):
    import oracle
    kc, vc = wl.key_cache, wl.value_cache
    if wl.slot_mapping is not None:
        kc, vc = oracle.reshape_and_cache(wl.new_key, wl.new_value, kc, vc, wl.slot_mapping)
    if wl.q_len == 1:
        oracle.decode(wl.query, kc, vc, wl.block_table, wl.seq_lens, wl.scale)
    else:
        oracle.multi_query(wl.query, kc, vc, wl.block_table, wl.seq_lens, wl.scale)


def cpu_baseline(wl, budget_s=20.0):
    """The CPU oracle on the same step (the scatter of the new tokens, when
    the step has them, and attention of every sequence), wall clock, median
    over up to 3 repeats within about budget_s seconds, on every host thread
    torch and NumPy use."""
    import torch
    times = []
    while len(times) < 3 and sum(times) < budget_s:
        t0 = time.perf_counter()
        _oracle_step(wl)
        times.append(time.perf_counter() - t0)
        log(f"cpu oracle step {len(times)}: {times[-1]:.2f} s")
    t = statistics.median(times)
    what = "decode" if wl.q_len == 1 else f"multi-query, q_len {wl.q_len}"
    scat = "oracle scatter of the new tokens + " if wl.slot_mapping is not None else ""
    return {"value": round(wl.kv_bytes() / t / 1e9, 4), "unit": "GB/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": (f"the whole step of the same workload ({wl.num_seqs} sequences, "
                       f"{wl.num_tokens} tokens: {scat}fp64 {what}), median of {len(times)} "
                       f"run(s), {t:.2f} s per step"),
            "cpu_model": cpu_model(),
            "seconds_per_step": round(t, 3),
            "seqs_per_s": round(wl.num_seqs / t, 3)}


def cpu_baseline_one_thread(wl, budget_s=15.0):
    """The same oracle step on one host thread (NumPy's BLAS and torch both
    limited to one), wall clock, median over up to 3 repeats within about
    budget_s seconds."""
    import torch
    from threadpoolctl import threadpool_limits
    prev = torch.get_num_threads()
    times = []
    try:
        torch.set_num_threads(1)
        with threadpool_limits(limits=1):
            while len(times) < 3 and sum(times) < budget_s:
                t0 = time.perf_counter()
                _oracle_step(wl)
                times.append(time.perf_counter() - t0)
                log(f"cpu oracle, 1 thread, {wl.name} step {len(times)}: {times[-1]:.2f} s")
    finally:
        torch.set_num_threads(prev)
    t = statistics.median(times)
    return {"workload": wl.name, "value": round(wl.kv_bytes() / t / 1e9, 4), "unit": "GB/s",
            "cores": 1, "seconds_per_step": round(t, 3), "runs": len(times),
            "seqs_per_s": round(wl.num_seqs / t, 3)}


def time_step(pkv, wl, dev, args, Q=1, fp8=False, P=None, layers_n=4):
    """The timed steps of one workload and their instrumented repeats.

    K steps with one event pair around them (events inside the steps would
    add their own dispatch latency to every step); then N = max(K, 100)
    more steps with the attention call's own kernel start and end (events
    its launch sets, paged_attn_timed) and events recorded around the call;
    then N attention calls back to back. N is at least 100 because the
    first few dozen calls after the GPU has been idle run up to 5% slower
    than the steady state the kernel's roofline is about. Returns the
    measurements (ms) and the workload's facts."""
    import torch
    S, H, D = wl.num_seqs, wl.num_heads, wl.head_dim
    NB, bs, Hkv, _ = wl.key_cache.shape
    P = wl.partition_size if P is None else P
    attn = pkv.paged_attn_decode if Q == 1 else pkv.paged_attn_multi_query
    attn_name = "paged_attn_decode" if Q == 1 else f"paged_attn_multi_query (q_len {Q})"
    q = wl.query.to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    has_new = wl.slot_mapping is not None
    if has_new:
        nk, nv = wl.new_key.to(dev), wl.new_value.to(dev)
        slots = torch.from_numpy(wl.slot_mapping).to(dev)
    kc0, vc0 = wl.key_cache.to(dev), wl.value_cache.to(dev)
    if wl.block_mapping is not None:
        # the copy-on-write of the fork (prefix-sharing batch), once, before
        # the steps: the copies' contents are what the remapped tables read
        pkv.copy_blocks(kc0, vc0, torch.from_numpy(wl.block_mapping).to(dev))
    ks = vs = None
    if fp8:
        # setup, not timed: a scale per KV head (largest magnitude / 448, the
        # caller's calibration) and every slot of the pools quantised
        ks, vs = fp8_scales(kc0), fp8_scales(vc0)
        k8 = torch.empty(kc0.shape, dtype=torch.uint8, device=dev)
        v8 = torch.empty_like(k8)
        pkv.reshape_and_cache_fp8(kc0.view(-1, Hkv, D), vc0.view(-1, Hkv, D), k8, v8,
                                  torch.arange(NB * bs, dtype=torch.int64, device=dev), ks, vs)
        del kc0, vc0
        kc0, vc0 = k8, v8
        attn_f8 = pkv.paged_attn_decode_fp8 if Q == 1 else pkv.paged_attn_multi_query_fp8
        attn_name = attn_name.replace("paged_attn_decode", "paged_attn_decode_fp8").replace(
            "paged_attn_multi_query", "paged_attn_multi_query_fp8")

        def scatter(kc, vc):
            pkv.reshape_and_cache_fp8(nk, nv, kc, vc, slots, ks, vs)

        def attend(kc, vc, events=None):
            attn_f8(out, q, kc, vc, ks, vs, bt, sl, wl.scale, wl.max_seq_len, P, ws, events=events)
    else:
        def scatter(kc, vc):
            pkv.reshape_and_cache(nk, nv, kc, vc, slots)

        def attend(kc, vc, events=None):
            attn(out, q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, P, ws, events=events)
    layers = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(layers_n - 1)]
    out = torch.empty(wl.query.shape, dtype=wl.dtype, device=dev)
    ws = pkv.workspace_for(q, kc0, wl.max_seq_len, P)
    part_tokens = pkv.paged_attn_partition_tokens(S, Hkv, bs, wl.max_seq_len, P, q_len=Q, num_heads=H,
                                                  kv_dtype=pkv.PKV_E4M3 if fp8 else pkv.dtype_code(wl.dtype))
    stream = torch.cuda.current_stream(dev)

    def step(i):
        kc, vc = layers[i % len(layers)]
        if has_new:
            scatter(kc, vc)
        attend(kc, vc)

    log(f"{wl.name}: warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_stop) / args.steps
    log(f"{wl.name}: {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall * 1e3 / args.steps:.1f})")

    n_inst = max(args.steps, 100)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_inst)]
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_inst)]
    for a, b in kev:   # HIP creates an event on its first record
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for i in range(n_inst):
        kc, vc = layers[i % len(layers)]
        if has_new:
            scatter(kc, vc)
        ev[i][0].record(stream)
        attend(kc, vc, kev[i])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in ev]
    ker_ms = [a.elapsed_time(b) for a, b in kev]
    ker_avg = sum(ker_ms) / len(ker_ms)
    log(f"{wl.name}: attention kernel avg {ker_avg * 1e3:.1f} us (median "
        f"{statistics.median(ker_ms) * 1e3:.1f}); with events around the call "
        f"{sum(dec_ms) / len(dec_ms) * 1e3:.1f} us")

    for i in range(args.warmup):
        kc, vc = layers[i % len(layers)]
        attend(kc, vc)
    b0 = torch.cuda.Event(enable_timing=True)
    b1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    b0.record(stream)
    for i in range(n_inst):
        kc, vc = layers[i % len(layers)]
        attend(kc, vc)
    b1.record(stream)
    torch.cuda.synchronize()
    dec_bb = b0.elapsed_time(b1) / n_inst
    log(f"{wl.name}: attention back to back: {dec_bb * 1e3:.1f} us per call")
    del layers, out, ws
    torch.cuda.empty_cache()
    kv = wl.kv_bytes() // (2 if fp8 else 1)      # e4m3: one byte per element
    return {"ms_step": ms_step, "dec_ms": dec_ms, "ker_ms": ker_ms, "ker_avg": ker_avg,
            "dec_bb": dec_bb, "kv": kv, "attn_name": attn_name, "part_tokens": part_tokens,
            "layers": layers_n, "scales": (ks, vs), "new_tokens": S * Q if has_new else 0}


def _pct3(xs):
    q = statistics.quantiles(xs, n=10) if len(xs) >= 2 else xs * 9
    return [round(q[0] * 1e3, 2), round(statistics.median(xs) * 1e3, 2), round(q[-1] * 1e3, 2)]


def step_summary(wl, m):
    """The per-workload figures of one time_step result."""
    kv = m["kv"]
    achieved = kv / (m["ker_avg"] * 1e-3) / 1e9
    return {
        "kv_GBps": round(kv / (m["ms_step"] * 1e-3) / 1e9, 2),
        "ms_per_step": round(m["ms_step"], 5),
        "pct_hbm_peak": round(100 * kv / (m["ms_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "seqs_per_s_per_layer": round(wl.num_seqs / (m["ms_step"] * 1e-3), 1),
        "decode_us": round(sum(m["dec_ms"]) / len(m["dec_ms"]) * 1e3, 2),
        "decode_us_p10_p50_p90": _pct3(m["dec_ms"]),
        "decode_kernel_us": round(m["ker_avg"] * 1e3, 2),
        "decode_kernel_us_p10_p50_p90": _pct3(m["ker_ms"]),
        "decode_us_back_to_back": round(m["dec_bb"] * 1e3, 2),
        "kv_GBps_back_to_back": round(kv / (m["dec_bb"] * 1e-3) / 1e9, 1),
        "kernel_frac_of_hbm_peak": round(achieved / HBM_PEAK_GBS, 4),
        "achieved_GBps": round(achieved, 2),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--workload", choices=list(WORKLOADS), default=None,
                    help="the headline workload (default: the Llama-2-70B-shaped layer; the "
                         "Llama-3-8B one for --q-len > 1 and --kv-fp8); the prefix-sharing and "
                         "mixed batches time their decode calls (for profiles)")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-peak", action="store_true",
                    help="skip measuring the streaming-read rate")
    ap.add_argument("--no-second-workload", action="store_true",
                    help="time the headline workload only")
    ap.add_argument("--secondary", action="store_true",
                    help="add the block-size sweep and the placement comparison")
    ap.add_argument("--q-len", type=int, default=1,
                    help="new tokens per sequence in the timed step: >1 times the "
                         "multi-query (speculative verification) pass instead of decode")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="an e4m3 KV cache (scales per KV head from the 16-bit pools): the "
                         "step is reshape_and_cache_fp8 + paged_attn_decode_fp8")
    ap.add_argument("--prefix-share", action="store_true",
                    help="also time the prefix-sharing batch: decode vs shared-prefix decode")
    ap.add_argument("--swap", action="store_true",
                    help="also time swap_blocks: 16 sequences' blocks to pinned host pools and "
                         "back, beside contiguous copies over the host link")
    ap.add_argument("--multi-query", action="store_true",
                    help="also time the multi-query (speculative verification) pass, "
                         "q_len 2, 4 and 8, on the same lengths")
    ap.add_argument("--per-config", action="store_true",
                    help="add cold-cache timings of every page-shaped workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (torch), 10 times: the "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sequences and KV heads are independent; see the sharding notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_154_amd as pkv
    from paged_kv_cache_154_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 1 GiB x 10")
        return
    Q = args.q_len
    fp8 = args.kv_fp8
    name = args.workload or ("llama3_8b_bf16" if (Q > 1 or fp8) else "llama2_70b_fp16")
    if name != "llama3_8b_bf16" and (Q > 1 or fp8):
        ap.error("--q-len > 1 and --kv-fp8 run on the Llama-3-8B-shaped batch")
    log(f"generating workload {name}")
    wl = W.llama3_8b(q_len=Q) if name == "llama3_8b_bf16" else W.make(WORKLOADS[name][0])
    m = time_step(pkv, wl, dev, args, Q=Q, fp8=fp8, P=args.partition_size, layers_n=args.layers)
    S, H, D = wl.num_seqs, wl.num_heads, wl.head_dim
    NB, bs, Hkv, _ = wl.key_cache.shape
    summ = step_summary(wl, m)
    kv = m["kv"]
    achieved = summ["achieved_GBps"]
    if name != "llama3_8b_bf16":
        workload = f"{name}: {WORKLOADS[name][1]}"
        lens = WORKLOADS[name][2]
        step_desc = "paged_attn_decode"
        if wl.block_mapping is not None:
            step_desc += " (after the fork's copy_blocks, done once before the steps)"
        profile = f"decode_{name}"
    else:
        workload = (("llama3_8b_e4m3" if fp8 else "llama3_8b_bf16")
                    + ("" if Q == 1 else f"_q{Q}") + ": Llama-3-8B-shaped single-layer "
                    + ("decode" if Q == 1 else f"verification of {Q} new tokens per sequence")
                    + (", e4m3 KV cache (a scale per KV head)" if fp8 else ""))
        lens = "uniform [512, 4096], seed 1542"
        step_desc = f"reshape_and_cache({m['new_tokens']} new tokens) + {m['attn_name']}"
        profile = (("decode" if Q == 1 else f"multi_query_q{Q}")
                   + ("_llama3_8b_e4m3" if fp8 else "_llama3_8b_bf16"))
    dtype = {torch.float16: "fp16", torch.bfloat16: "bf16", torch.float32: "fp32"}[wl.dtype]
    res = {
        "metric": METRIC,
        "value": summ["kv_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": summ["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"e4m3 KV, {dtype} query" if fp8 else dtype,
        "data": "synthetic",
        "config": {
            "workload": workload,
            "num_seqs": S, "num_heads": H, "num_kv_heads": Hkv, "head_dim": D,
            "block_size": bs, "num_blocks": NB, "seq_lens": lens,
            "tokens": wl.num_tokens, "kv_bytes_per_step": kv,
            "partition_tokens": m["part_tokens"], "layers_rotated": m["layers"],
            "step": step_desc,
        },
    }
    res.update({k: v for k, v in summ.items()
                if k not in ("kv_GBps", "ms_per_step", "kernel_frac_of_hbm_peak", "achieved_GBps")})
    res["roofline"] = {
        "bound": "hbm",
        "achieved": achieved,
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(profile),
        "kernel": f"{m['attn_name']} (decode_partition_kernel)",
        "duration": "mean of the kernel's own start-to-end time (events set by its launch, "
                    "hipExtLaunchKernel) over max(K, 100) more steps like the timed ones",
    }
    res["cpu_baseline"] = None
    ks, vs = m["scales"]
    second = None
    if name == "llama2_70b_fp16" and not args.no_second_workload:
        log("generating workload llama3_8b_bf16 (second line item)")
        second = W.llama3_8b()
        m2 = time_step(pkv, second, dev, args, layers_n=args.layers)
        s2 = step_summary(second, m2)
        res["llama3_8b_bf16"] = {
            "workload": "llama3_8b_bf16: Llama-3-8B-shaped single-layer decode (64 sequences, "
                        "32 / 8 heads, head_dim 128, bf16, block_size 16, lengths uniform "
                        "[512, 4096])",
            "step": f"reshape_and_cache({m2['new_tokens']} new tokens) + paged_attn_decode",
            "kv_bytes_per_step": m2["kv"], "partition_tokens": m2["part_tokens"], **s2,
            "roofline": {"bound": "hbm", "achieved": s2["achieved_GBps"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": s2["kernel_frac_of_hbm_peak"],
                         "traffic": measured_traffic("decode_llama3_8b_bf16")},
        }
    if not args.no_stream_peak:
        log("measuring the streaming-read rate")
        peak = stream_read_peak(dev)
        res["measured_stream_read_GBps"] = round(peak, 1)
        res["roofline"]["frac_of_measured_stream_read"] = round(achieved / peak, 4)
    if args.secondary or args.multi_query or args.swap or args.prefix_share or args.per_config:
        torch.cuda.empty_cache()
    base = second if second is not None else (wl if name == "llama3_8b_bf16" else None)
    if args.swap:
        res["swap"] = swap_rows(pkv, W.llama3_8b(), dev)
    if args.prefix_share:
        res["prefix_share"] = prefix_share_rows(pkv, W, dev)
    if args.secondary:
        res["secondary"] = secondary(pkv, W, base if base is not None else W.llama3_8b(), dev)
    if args.multi_query:
        res["multi_query"] = multi_query_rows(pkv, W, base if base is not None else W.llama3_8b(), dev)
    if args.per_config:
        res["per_config"] = per_config(pkv, W, dev)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same step")
        res["cpu_baseline"] = cpu_baseline_fp8(wl, ks, vs) if fp8 else cpu_baseline(wl)
        one = second if second is not None else (wl if (name == "llama3_8b_bf16" and not fp8) else None)
        if one is not None:
            res["cpu_baseline"]["one_thread"] = cpu_baseline_one_thread(one)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
