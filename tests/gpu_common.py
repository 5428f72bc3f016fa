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


# The fp32-accumulation bar for fp32 outputs, beside the per-dtype bars
# above: the kernels accumulate in fp32, and the observed error against the
# fp64 oracle is ~1e-6 or less; leaving out a single token of a sequence of
# 8192 tokens moves some output element by far more (test_oracle_sensitivity).
FP32_BAR = 2e-5


def assert_close(out, ref, kv_dtype, seqs=None, label=""):
    """max-abs error within the bar of the KV (or query) dtype, and, for an
    fp32 output, within FP32_BAR as well. Returns the error."""
    err = max_err(out, ref, seqs)
    n = "all" if seqs is None else len(seqs)
    say(f"{label} out={out.dtype} max_abs_err={err:.3g} on {n} seqs")
    assert err <= TOL[kv_dtype], (label, out.dtype, err)
    if out.dtype == torch.float32:
        assert err <= FP32_BAR, (label, err)
    return err


def poisoned_workspace(nbytes, ctl_bytes):
    """A workspace whose control area (the first ctl_bytes, which must be zero
    at first use) is zero and whose partials are 0xFF bytes (fp32 NaN)."""
    ws = torch.full((max(int(nbytes), int(ctl_bytes), 256),), 0xFF, dtype=torch.uint8, device=DEV)
    ws[:ctl_bytes].zero_()
    return ws


def repoison(ws, ctl_bytes, gen=None):
    """Partials overwritten (0xFF, or random bytes with a generator); the
    control area is left as the last call left it."""
    if gen is None:
        ws[ctl_bytes:].fill_(0xFF)
    else:
        ws[ctl_bytes:].copy_(torch.randint(0, 256, (ws.numel() - ctl_bytes,), generator=gen,
                                           device=DEV, dtype=torch.uint8))


def control_is_zero(ws, ctl_bytes):
    """Every call must leave the workspace's control area zero."""
    torch.cuda.synchronize()
    return bool((ws[:ctl_bytes] == 0).all())
