"""Helpers shared by the GPU parity tests: device copies of a workload, the
max-abs error against the oracle with the output's own rounding taken off,
and bit views for bit-exact comparisons."""

import numpy as np
import torch

TOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 8e-3}
DEV = "cuda"


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def to_dev(wl):
    d = dict(q=wl.query.to(DEV), kc=wl.key_cache.to(DEV), vc=wl.value_cache.to(DEV),
             bt=torch.from_numpy(wl.block_table).to(DEV),
             sl=torch.from_numpy(wl.seq_lens).to(DEV))
    if wl.slot_mapping is not None:
        d["nk"] = wl.new_key.to(DEV)
        d["nv"] = wl.new_value.to(DEV)
        d["slots"] = torch.from_numpy(wl.slot_mapping).to(DEV)
    if wl.block_mapping is not None:
        d["pairs"] = torch.from_numpy(wl.block_mapping).to(DEV)
    return d


def max_err(gpu_out, ref, seqs=None):
    """Max-abs error. For a narrowed (fp16/bf16) output the final rounding to
    nearest-even of a value of magnitude |ref| may add up to half a unit in
    the last place of the output type; that share is taken off first, so the
    bar applies to the fp32-accumulated result in both cases."""
    g = gpu_out.detach().to("cpu", torch.float64).numpy()
    if seqs is not None:
        g, ref = g[seqs], ref[seqs]
    if not g.size:
        return 0.0
    err = np.abs(g - ref)
    mant = {torch.float16: 10, torch.bfloat16: 7}.get(gpu_out.dtype)
    if mant is not None:
        a = np.maximum(np.abs(ref), np.finfo(np.float64).tiny)
        half_ulp = np.exp2(np.floor(np.log2(a)) - mant - 1)
        err = np.maximum(err - half_ulp, 0.0)
    return float(err.max())


def bits(t):
    return t.view({2: torch.int16, 4: torch.int32}[t.element_size()])
