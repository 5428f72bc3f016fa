"""Benchmark of the paged decode hot path on one MI355X.

One step = one layer's decode step of the Llama-3-8B-shaped batch (64
sequences, 32 query / 8 KV heads, head_dim 128, bf16, block_size 16, lengths
uniform in [512, 4096], 20000-block pool): reshape_and_cache of the 64 new
tokens, then paged_attn_decode over all cached tokens. Steps rotate over
``--layers`` copies of the layer's pools (same shapes and tables), so that a
step never finds its K/V in the 256 MB Infinity Cache or the L2 from the
previous use of the same pool.

Prints one JSON line. ``value`` is KV GB/s: the algorithmic KV bytes a step
must read (every cached token's K and V rows, once) over the measured step
time. The roofline entry is for the decode call (partition kernel plus the
split-K merge kernel), timed with HIP events on the stream the library
launches on.

    python bench.py [--steps K] [--warmup W] [--layers N] [--no-cpu-baseline]
"""

import argparse
import hashlib
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


def kernel_source_hash():
    """sha256 of the decode kernel sources (as in the traffic profile)."""
    h = hashlib.sha256()
    for f in ("decode.hip", "pagedkv_internal.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_154_amd", "csrc", f)) as fh:
            h.update(fh.read().encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode call from the committed rocprofv3 counter runs,
    or None when the kernel sources changed after those runs."""
    path = os.path.join(ROOT, "profiles", "decode_llama3_8b_bf16_traffic.json")
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


def cpu_baseline(wl, budget_s=20.0):
    """The CPU oracle on the same step (scatter + decode of every sequence),
    wall clock, median over repeats within about budget_s seconds."""
    import torch

    import oracle
    times = []
    while len(times) < 3 and sum(times) < budget_s:
        t0 = time.perf_counter()
        kc, vc = oracle.reshape_and_cache(wl.new_key, wl.new_value, wl.key_cache,
                                          wl.value_cache, wl.slot_mapping)
        oracle.decode(wl.query, kc, vc, wl.block_table, wl.seq_lens, wl.scale)
        times.append(time.perf_counter() - t0)
        log(f"cpu oracle step {len(times)}: {times[-1]:.2f} s")
    t = statistics.median(times)
    return {"value": round(wl.kv_bytes() / t / 1e9, 4), "unit": "GB/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": (f"the whole step of the same workload ({wl.num_seqs} sequences, "
                       f"{wl.num_tokens} tokens: oracle scatter of the new tokens + fp64 "
                       f"decode), median of {len(times)} run(s), {t:.2f} s per step"),
            "seconds_per_step": round(t, 3),
            "seqs_per_s": round(wl.num_seqs / t, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    log("generating workload (Llama-3-8B-shaped layer)")
    wl = W.llama3_8b()
    P = wl.partition_size if args.partition_size is None else args.partition_size
    S, H, D = wl.query.shape
    NB, bs, Hkv, _ = wl.key_cache.shape

    q = wl.query.to(dev)
    bt = torch.from_numpy(wl.block_table).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    nk, nv = wl.new_key.to(dev), wl.new_value.to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    kc0, vc0 = wl.key_cache.to(dev), wl.value_cache.to(dev)
    layers = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(args.layers - 1)]
    out = torch.empty(S, H, D, dtype=wl.dtype, device=dev)
    ws = pkv.workspace_for(q, kc0, wl.max_seq_len, P)
    part_tokens = pkv.paged_attn_partition_tokens(S, Hkv, bs, wl.max_seq_len, P)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        kc, vc = layers[i % len(layers)]
        pkv.reshape_and_cache(nk, nv, kc, vc, slots)
        pkv.paged_attn_decode(out, q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, P, ws)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps, plus per-call events around each decode
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        kc, vc = layers[i % len(layers)]
        pkv.reshape_and_cache(nk, nv, kc, vc, slots)
        ev[i][0].record(stream)
        pkv.paged_attn_decode(out, q, kc, vc, bt, sl, wl.scale, wl.max_seq_len, P, ws)
        ev[i][1].record(stream)
    t_stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_stop) / args.steps
    dec_ms = [a.elapsed_time(b) for a, b in ev]
    dec_avg = sum(dec_ms) / len(dec_ms)
    log(f"{args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall * 1e3 / args.steps:.1f}), "
        f"decode call avg {dec_avg * 1e3:.1f} us, median {statistics.median(dec_ms) * 1e3:.1f} us")

    kv = wl.kv_bytes()
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = kv / (dec_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_bf16: Llama-3-8B-shaped single-layer decode",
            "num_seqs": S, "num_heads": H, "num_kv_heads": Hkv, "head_dim": D,
            "block_size": bs, "num_blocks": NB, "seq_lens": "uniform [512, 4096], seed 1542",
            "tokens": wl.num_tokens, "kv_bytes_per_step": kv,
            "partition_tokens": part_tokens, "layers_rotated": len(layers),
            "step": "reshape_and_cache(64 new tokens) + paged_attn_decode",
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seqs_per_s_per_layer": round(S / (ms_step * 1e-3), 1),
        "decode_us": round(dec_avg * 1e3, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": "paged_attn_decode (decode_partition_kernel + decode_reduce_kernel)",
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same step")
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
