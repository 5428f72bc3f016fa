"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars: bit-exact for reshape_and_cache and copy_blocks; max-abs error on the
decode output at most 1e-5 (fp32 KV), 2e-3 (fp16 KV) or 8e-3 (bf16 KV),
with fp32 or KV-dtype output, and at most 2e-5 on every fp32 output (the
fp32-accumulation bar, tight enough to see one token left out of a sequence
of 8192); bitwise invariants (placement, NaN tails, copy-on-write remap,
run-to-run); split-K agreement. The full-size workloads are compared on every
sequence, with the workspace's partials poisoned (NaN) before each call and
its control area checked to be zero again after it.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_154_amd as pkv
from paged_kv_cache_154_amd import workloads as W
from gpu_common import (DEV, assert_close, bits, control_is_zero, poisoned_workspace, repoison, say,
                        to_dev)

pytestmark = pytest.mark.gpu


def gpu_step(wl, d, out_dtype=None, partition_size=None, table=None, workspace=None):
    """Cache ops of the step (scatter, copy-on-write), then decode."""
    if "slots" in d:
        pkv.reshape_and_cache(d["nk"], d["nv"], d["kc"], d["vc"], d["slots"])
    if "pairs" in d:
        pkv.copy_blocks(d["kc"], d["vc"], d["pairs"])
    out = torch.empty(wl.query.shape, dtype=out_dtype or wl.dtype, device=DEV)
    P = wl.partition_size if partition_size is None else partition_size
    pkv.paged_attn_decode(out, d["q"], d["kc"], d["vc"], d["bt"] if table is None else table,
                          d["sl"], wl.scale, wl.max_seq_len, P, workspace=workspace)
    torch.cuda.synchronize()
    return out


def ws_sizes(wl, P, max_seq_len=None):
    """(workspace bytes, control-area bytes) of a decode call on wl."""
    m = wl.max_seq_len if max_seq_len is None else max_seq_len
    n = pkv.paged_attn_workspace_size(wl.num_seqs, wl.num_heads, wl.num_kv_heads, wl.head_dim,
                                      wl.block_size, m, P)
    c = pkv.workspace_control_bytes(wl.num_seqs, wl.num_kv_heads, wl.head_dim, wl.block_size, m, P)
    return n, c


def oracle_step(wl, seqs=None):
    kc, vc = wl.key_cache, wl.value_cache
    if wl.slot_mapping is not None:
        kc, vc = oracle.reshape_and_cache(wl.new_key, wl.new_value, kc, vc, wl.slot_mapping)
    if wl.block_mapping is not None:
        kc, vc = oracle.copy_blocks(kc, vc, wl.block_mapping)
    out = oracle.decode(wl.query, kc, vc, wl.block_table, wl.seq_lens, wl.scale, seqs=seqs)
    return out, kc, vc


# ----------------------------------------------------------------------------
# small and medium shapes: every output element against the oracle
# ----------------------------------------------------------------------------

SMALL = [
    # id, dtype, D, bs, H, Hkv, lens, partition
    ("f32_d64_bs16_mha", torch.float32, 64, 16, 4, 4, [1, 17, 33, 50], 0),
    ("f32_d128_bs8_g2", torch.float32, 128, 8, 8, 4, [3, 8, 9, 129, 300], 0),
    ("f16_d128_bs16_g4", torch.float16, 128, 16, 32, 8, [1, 15, 16, 17, 31, 33, 200, 1000], 0),
    ("f16_d64_bs32_g8", torch.float16, 64, 32, 16, 2, [2, 31, 32, 33, 64, 513], 0),
    ("bf16_d128_bs16_g4", torch.bfloat16, 128, 16, 32, 8, [5, 16, 100, 511, 512, 513, 2000], 0),
    ("bf16_d128_bs8_g1", torch.bfloat16, 128, 8, 4, 4, [7, 8, 9, 77, 640], 0),
    ("bf16_d64_bs16_g16", torch.bfloat16, 64, 16, 16, 1, [1, 40, 300], 0),
    ("bf16_d128_bs32_g3", torch.bfloat16, 128, 32, 6, 2, [1, 95, 96, 97], 0),
    ("f16_d128_bs32_g8_split64", torch.float16, 128, 32, 64, 8, [32, 65, 300, 1029], 64),
    ("bf16_d128_bs8_g4_split128", torch.bfloat16, 128, 8, 32, 8, [8, 127, 128, 129, 1500], 128),
    ("f32_d64_bs16_split16", torch.float32, 64, 16, 4, 2, [1, 16, 17, 80], 16),
    ("bf16_d128_bs16_g4_split512", torch.bfloat16, 128, 16, 32, 8, [600, 1024, 1025, 3000], 512),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_match_oracle(case):
    name, dt, D, bs, H, Hkv, lens, P = case
    wl = W.custom(zlib.crc32(name.encode()) % 10000 + 100, seq_lens=lens, num_heads=H, num_kv_heads=Hkv,
                  head_dim=D, block_size=bs, dtype=dt, partition_size=P, new_token=True)
    ref, _, _ = oracle_step(wl)
    for out_dt in dict.fromkeys([dt, torch.float32]):
        say(f"{name} out={out_dt}")
        d = to_dev(wl)
        n, c = ws_sizes(wl, P)
        ws = poisoned_workspace(n, c)
        out = gpu_step(wl, d, out_dtype=out_dt, workspace=ws)
        assert control_is_zero(ws, c)
        assert torch.isfinite(out).all()
        assert_close(out, ref, dt, label=name)


def test_seq_len_one_is_the_v_row_bit_exact():
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        wl = W.custom(7, seq_lens=[1, 1, 1, 1], num_heads=8, num_kv_heads=2, head_dim=128,
                      block_size=16, dtype=dt)
        say(f"seq_len=1 {dt}")
        out = gpu_step(wl, to_dev(wl), out_dtype=dt).cpu()
        for s in range(4):
            vrow = wl.value_cache[int(wl.block_table[s, 0]), 0]      # [Hkv, D]
            for h in range(8):
                assert torch.equal(bits(out[s, h]), bits(vrow[h // 4])), (dt, s, h)


def test_zero_length_sequences_give_zero_rows():
    wl = W.custom(8, seq_lens=[0, 37, 0, 1], num_heads=8, num_kv_heads=8, head_dim=64,
                  block_size=8, dtype=torch.bfloat16)
    d = to_dev(wl)
    ref, _, _ = oracle_step(wl)
    for P in (0, 16):
        say(f"zero-length rows P={P}")
        out = gpu_step(wl, d, out_dtype=torch.float32, partition_size=P)
        assert torch.equal(out[0], torch.zeros_like(out[0]))
        assert torch.equal(out[2], torch.zeros_like(out[2]))
        assert_close(out, ref, torch.bfloat16, label=f"zero-length rows P={P}")


@pytest.mark.parametrize("P", [64, 0])
def test_max_seq_len_above_actual_lengths(P):
    """The launch is sized from the host bound; partitions past a sequence's
    end exit early."""
    wl = W.custom(9, seq_lens=[10, 300, 47], num_heads=16, num_kv_heads=4, head_dim=128,
                  block_size=16, dtype=torch.float16, max_blocks_per_seq=128)
    d = to_dev(wl)
    ref, _, _ = oracle_step(wl)
    out = torch.empty(wl.query.shape, dtype=torch.float32, device=DEV)
    say(f"max_seq_len 2048 over lengths <= 300, P={P}")
    pkv.paged_attn_decode(out, d["q"], d["kc"], d["vc"], d["bt"], d["sl"], wl.scale, 2048, P)
    torch.cuda.synchronize()
    assert_close(out, ref, torch.float16, label=f"max_seq_len bound P={P}")


@pytest.mark.parametrize("L,G,P", [(65536, 16, 64), (65536, 4, 64), (8192, 4, 16)])
def test_many_partitions_of_one_long_sequence(L, G, P):
    """One sequence split into hundreds or thousands of partitions: hundreds
    of arrivals at one (sequence, KV head) word, and a merge over them all."""
    wl = W.custom(16, seq_lens=[L], num_heads=G, num_kv_heads=1, head_dim=64,
                  block_size=16, dtype=torch.bfloat16)
    ref, _, _ = oracle_step(wl)
    say(f"one sequence of {L} tokens, G={G}, P={P}")
    n, c = ws_sizes(wl, P)
    ws = poisoned_workspace(n, c)
    out = gpu_step(wl, to_dev(wl), out_dtype=torch.float32, partition_size=P, workspace=ws)
    assert control_is_zero(ws, c)
    assert_close(out, ref, torch.bfloat16, label=f"L={L} P={P}")


# ----------------------------------------------------------------------------
# cache operations: bit-exact
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dt", [torch.float32, torch.float16, torch.bfloat16])
def test_reshape_and_cache_bit_exact(dt):
    NB, bs, Hkv, D = 40, 16, 4, 128
    g = torch.Generator().manual_seed(3)
    kc = torch.randn(NB, bs, Hkv, D, generator=g).to(dt)
    vc = torch.randn(NB, bs, Hkv, D, generator=g).to(dt)
    T = 50
    slots = torch.randperm(NB * bs, generator=g)[:T].to(torch.int64)
    slots[::7] = -1                                    # "no slot": skipped
    key = torch.randn(T, Hkv, D, generator=g).to(dt)
    value = torch.randn(T, Hkv, D, generator=g).to(dt)
    key[3, 1, 5] = float("nan")
    ek, ev = oracle.reshape_and_cache(key, value, kc, vc, slots.numpy())
    dk, dv = kc.to(DEV), vc.to(DEV)
    say(f"reshape_and_cache {dt}")
    pkv.reshape_and_cache(key.to(DEV), value.to(DEV), dk, dv, slots.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(bits(dk.cpu()), bits(ek)) and torch.equal(bits(dv.cpu()), bits(ev))


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16, torch.float32])
def test_copy_blocks_bit_exact(dt):
    NB, bs, Hkv, D = 64, 16, 8, 64
    g = torch.Generator().manual_seed(4)
    kc = torch.randn(NB, bs, Hkv, D, generator=g).to(dt)
    vc = torch.randn(NB, bs, Hkv, D, generator=g).to(dt)
    perm = torch.randperm(NB, generator=g)
    pairs = torch.stack([perm[:10], perm[10:20]], dim=1).to(torch.int64)   # disjoint src/dst
    pairs[3, 0] = pairs[0, 0]                       # one source copied twice
    ek, ev = oracle.copy_blocks(kc, vc, pairs.numpy())
    dk, dv = kc.to(DEV), vc.to(DEV)
    say(f"copy_blocks {dt}")
    pkv.copy_blocks(dk, dv, pairs.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(bits(dk.cpu()), bits(ek)) and torch.equal(bits(dv.cpu()), bits(ev))


def test_check_decode_inputs_counts_violations():
    bt = torch.tensor([[0, 5, 99, -3], [1, 2, 3, 4], [7, 1000, 0, 0]], dtype=torch.int32)
    sl = torch.tensor([40, 70, 17], dtype=torch.int32)     # 70 > max_seq_len 64
    say("check_decode_inputs")
    bad_blk, bad_len = pkv.check_decode_inputs(bt.to(DEV), sl.to(DEV), block_size=16,
                                               num_blocks=10, max_seq_len=64)
    # seq 0 uses 3 blocks: 99 is bad; seq 1 is clamped to 64 tokens = 4 blocks, all
    # good; seq 2 uses 2 blocks: 1000 is bad
    assert (bad_blk, bad_len) == (2, 1)


# ----------------------------------------------------------------------------
# invariants (bitwise)
# ----------------------------------------------------------------------------

def test_placement_permutation_is_bitwise_invariant():
    wl = W.custom(11, seq_lens=[33, 700, 129, 1], num_heads=32, num_kv_heads=8,
                  head_dim=128, block_size=16, dtype=torch.bfloat16)
    d = to_dev(wl)
    say("placement permutation")
    out = gpu_step(wl, d, out_dtype=torch.float32)
    perm = np.random.default_rng(1).permutation(wl.num_blocks)
    inv = torch.from_numpy(np.argsort(perm))
    d2 = dict(d)
    d2["kc"] = wl.key_cache[inv].to(DEV)
    d2["vc"] = wl.value_cache[inv].to(DEV)
    d2["bt"] = torch.from_numpy(perm[wl.block_table].astype(np.int32)).to(DEV)
    out2 = gpu_step(wl, d2, out_dtype=torch.float32)
    assert torch.equal(bits(out), bits(out2))


def test_unused_slots_are_never_read():
    """NaN in unused tail slots and free blocks vs zeros there: bitwise equal."""
    wl = W.custom(12, seq_lens=[1, 15, 17, 100, 250], num_heads=16, num_kv_heads=4,
                  head_dim=64, block_size=32, dtype=torch.float16)
    d = to_dev(wl)
    say("NaN tails")
    out = gpu_step(wl, d, out_dtype=torch.float32)
    d0 = dict(d)
    d0["kc"] = torch.nan_to_num(wl.key_cache, nan=0.0).to(DEV)
    d0["vc"] = torch.nan_to_num(wl.value_cache, nan=0.0).to(DEV)
    out0 = gpu_step(wl, d0, out_dtype=torch.float32)
    assert torch.isfinite(out).all()
    assert torch.equal(bits(out), bits(out0))


def test_run_to_run_determinism():
    wl = W.custom(13, seq_lens=[3000, 17, 1200], num_heads=32, num_kv_heads=8,
                  head_dim=128, block_size=16, dtype=torch.bfloat16)
    d = to_dev(wl)
    say("determinism")
    a = gpu_step(wl, d, out_dtype=torch.float32, partition_size=256)
    b = gpu_step(wl, d, out_dtype=torch.float32, partition_size=256)
    assert torch.equal(bits(a), bits(b))


def test_split_partitions_agree_with_unsplit():
    wl = W.custom(14, seq_lens=[2500, 513, 64, 4000], num_heads=32, num_kv_heads=8,
                  head_dim=128, block_size=16, dtype=torch.bfloat16)
    d = to_dev(wl)
    say("split-K agreement")
    whole = gpu_step(wl, d, out_dtype=torch.float32, partition_size=4096)
    for P in (64, 128, 512):
        part = gpu_step(wl, d, out_dtype=torch.float32, partition_size=P)
        rel = ((part - whole).abs().max() / whole.abs().max()).item()
        say(f"split P={P} rel={rel:.3g}")
        assert rel <= 1e-5


def test_copy_on_write_remap_is_bitwise_invariant():
    """Decode through the private copies made by copy_blocks equals decode
    through the shared original block."""
    wl = W.prefix_share(groups=4, n=3, prefix=256, max_suffix=100)
    d = to_dev(wl)
    say("copy-on-write remap")
    after = gpu_step(wl, d, out_dtype=torch.float32)            # copies, remapped table
    d2 = to_dev(wl)
    d2.pop("pairs")
    before_tbl = torch.from_numpy(wl.block_table_before_cow).to(DEV)
    before = gpu_step(wl, d2, out_dtype=torch.float32, table=before_tbl)
    assert torch.equal(bits(after), bits(before))


# ----------------------------------------------------------------------------
# the workspace and the persistent kernel's schedule
# ----------------------------------------------------------------------------

def _decode_into(wl, d, ws, P, out_dtype=torch.float32):
    out = torch.empty(wl.query.shape, dtype=out_dtype, device=DEV)
    pkv.paged_attn_decode(out, d["q"], d["kc"], d["vc"], d["bt"], d["sl"], wl.scale,
                          wl.max_seq_len, P, workspace=ws)
    torch.cuda.synchronize()
    return out


def test_one_workspace_serves_many_calls():
    """A workspace zeroed once serves calls of different shapes and
    partitions in turn: every call leaves the control area zero again, and
    the partials, overwritten with garbage before each call, are never read
    before they are written."""
    a = W.custom(21, seq_lens=[5, 700, 1300, 64, 2], num_heads=16, num_kv_heads=4, head_dim=128,
                 block_size=16, dtype=torch.bfloat16)
    b = W.custom(22, seq_lens=list(range(1, 301, 7)), num_heads=8, num_kv_heads=8, head_dim=64,
                 block_size=8, dtype=torch.float16)
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    runs = [(a, 64), (b, 0), (a, 0), (b, 32), (a, 64), (b, 16)]
    refs = {id(a): oracle_step(a)[0], id(b): oracle_step(b)[0]}
    devs = {id(a): to_dev(a), id(b): to_dev(b)}
    g = torch.Generator(device=DEV).manual_seed(5)
    ctl_max = max(ws_sizes(wl, P)[1] for wl, P in runs)
    for i, (wl, P) in enumerate(runs):
        need, ctl = ws_sizes(wl, P)
        assert need <= ws.numel()
        repoison(ws, ctl_max, gen=g if i % 2 else None)
        say(f"shared workspace: S={wl.num_seqs} P={P}")
        out = _decode_into(wl, devs[id(wl)], ws, P)
        assert control_is_zero(ws, ctl_max)
        assert_close(out, refs[id(wl)], wl.dtype, label=f"shared workspace S={wl.num_seqs} P={P}")


def test_graph_replays_match_the_oracle():
    """Decode captured into a HIP graph (through torch.cuda.graph) and
    replayed with new queries: every replay runs every item and merges every
    split sequence, because each launch leaves its workspace's control area
    zero for the next (a per-call tag decided on the host would be frozen in
    the graph)."""
    wl = W.custom(25, seq_lens=[3000, 17, 1200, 1, 0, 640, 2049, 96, 513], num_heads=32,
                  num_kv_heads=8, head_dim=128, block_size=16, dtype=torch.bfloat16)
    d = to_dev(wl)
    for P in (256, 0):
        n, c = ws_sizes(wl, P)
        ws = poisoned_workspace(n, c)
        out = torch.empty(wl.query.shape, dtype=torch.float32, device=DEV)
        q = d["q"].clone()

        def call():
            pkv.paged_attn_decode(out, q, d["kc"], d["vc"], d["bt"], d["sl"], wl.scale,
                                  wl.max_seq_len, P, workspace=ws)

        call()                          # eager first (occupancy figures cached)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        torch.cuda.synchronize()
        gen = torch.Generator().manual_seed(26 + P)
        for rep in range(3):
            qh = torch.randn(wl.query.shape, generator=gen).to(wl.dtype)
            q.copy_(qh.to(DEV))
            out.fill_(float("nan"))
            repoison(ws, c)
            torch.cuda.synchronize()
            say(f"graph replay {rep} P={P}")
            graph.replay()
            torch.cuda.synchronize()
            assert control_is_zero(ws, c)
            ref = oracle.decode(qh, wl.key_cache, wl.value_cache, wl.block_table, wl.seq_lens,
                                wl.scale)
            assert_close(out, ref, wl.dtype, label=f"graph replay {rep} P={P}")
        del graph


def test_call_on_a_side_stream_with_its_own_workspace():
    """A call on a stream other than the current one, with the workspace
    allocated by the binding (on that stream): memory taken on the current
    stream right after the call cannot be the call's workspace."""
    wl = W.custom(27, seq_lens=[4000, 3000, 2500, 1800], num_heads=32, num_kv_heads=8,
                  head_dim=128, block_size=16, dtype=torch.bfloat16)
    d = to_dev(wl)
    ref = oracle_step(wl)[0]
    side = torch.cuda.Stream()
    out = torch.empty(wl.query.shape, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    say("side stream call")
    pkv.paged_attn_decode(out, d["q"], d["kc"], d["vc"], d["bt"], d["sl"], wl.scale,
                          wl.max_seq_len, 256, stream=side)
    junk = [torch.full((1 << 20,), -1, dtype=torch.int32, device=DEV) for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert_close(out, ref, wl.dtype, label="side stream")


def test_check_cache_op_inputs_counts_violations():
    """The contract check of slot_mapping and block_mapping: slots outside the
    pool, repeated slots, pairs outside the pool, and destinations that are a
    source or repeat, counted as a plain loop over the lists counts them."""
    rng = np.random.default_rng(28)
    NB, bs = 60, 16
    T = 700                                   # several workgroups of 256 tokens
    slots = rng.permutation(NB * bs)[:T].astype(np.int64)
    slots[::50] = -1                          # no slot: not a violation
    slots[7] = NB * bs + 3                    # outside the pool
    slots[300] = slots[10]                    # repeats an earlier slot
    slots[650] = slots[299]                   # repeats across workgroups
    slots[651] = slots[650]                   # and again
    pairs = rng.integers(0, NB, size=(300, 2)).astype(np.int64)   # two workgroups of pairs
    pairs[3] = [5, NB]                        # destination outside the pool
    pairs[4] = [-1, 2]                        # source outside the pool

    def expect():
        seen = set()
        out_pool = dup = 0
        for x in slots.tolist():
            if x >= NB * bs:
                out_pool += 1
            elif x >= 0:
                dup += x in seen
                seen.add(x)
        ok = [(a, b) for a, b in pairs.tolist() if 0 <= a < NB and 0 <= b < NB]
        bad = len(pairs) - len(ok)
        srcs = {a for a, b in pairs.tolist()}
        overlap, dsts = 0, set()
        for a, b in pairs.tolist():
            if 0 <= a < NB and 0 <= b < NB:
                overlap += (b in srcs) or (b in dsts)
            dsts.add(b)
        return out_pool, dup, bad, overlap

    say("check_cache_op_inputs")
    got = pkv.check_cache_op_inputs(torch.from_numpy(slots).to(DEV), torch.from_numpy(pairs).to(DEV),
                                    bs, NB)
    assert got == expect(), (got, expect())
    assert got[1] >= 3 and got[3] > 0
    # clean lists: nothing to report
    clean = np.arange(0, NB * bs, 3, dtype=np.int64)
    cp = np.array([[0, 1], [0, 2], [3, 4]], dtype=np.int64)
    assert pkv.check_cache_op_inputs(torch.from_numpy(clean).to(DEV), torch.from_numpy(cp).to(DEV),
                                     bs, NB) == (0, 0, 0, 0)
    assert pkv.check_cache_op_inputs(None, torch.from_numpy(cp).to(DEV), bs, NB) == (0, 0, 0, 0)


def test_more_sequences_than_one_launch():
    """4500 sequences run as launches of at most 2048 (each with its own
    schedule); rows on both sides of each launch boundary are checked."""
    rng = np.random.default_rng(23)
    lens = rng.integers(1, 121, size=4500).tolist()
    lens[2047], lens[2048], lens[4095], lens[4096] = 300, 1, 0, 250
    wl = W.custom(23, seq_lens=lens, num_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                  dtype=torch.bfloat16)
    seqs = sorted(set([0, 1, 2046, 2047, 2048, 2049, 4094, 4095, 4096, 4097, 4499]
                      + rng.choice(4500, size=40, replace=False).tolist()))
    ref, _, _ = oracle_step(wl, seqs=seqs)
    d = to_dev(wl)
    for P in (0, 128):
        say(f"4500 sequences, P={P}")
        out = gpu_step(wl, d, out_dtype=torch.float32, partition_size=P)
        assert torch.isfinite(out).all()
        assert_close(out, ref, torch.bfloat16, seqs, label=f"4500 sequences P={P}")
        assert torch.equal(out[4095], torch.zeros_like(out[4095]))


FIRST_ITEM_CASES = [
    # id, lengths, partition: the first items of some workgroups are found
    # from the first 64 lengths alone, the others from the work list
    ("few_splits_in_first_64", [int(x) for x in np.r_[np.full(60, 200), [700, 1500, 30, 2100],
                                                        np.arange(36) * 61 + 900]], 512),
    ("unsplit_mixed_classes", [int(x) for x in (np.arange(80) * 37) % 1000 + 1], 1008),
    ("unsplit_with_empty", [0, 5, 1000, 999, 0] + [1000] * 70, 1008),
]


@pytest.mark.parametrize("case", FIRST_ITEM_CASES, ids=[c[0] for c in FIRST_ITEM_CASES])
def test_first_items_with_and_without_the_work_list(case):
    name, lens, P = case
    wl = W.custom(zlib.crc32(name.encode()) % 10000 + 300, seq_lens=lens, num_heads=32, num_kv_heads=8,
                  head_dim=128, block_size=16, dtype=torch.bfloat16, partition_size=P)
    ref, _, _ = oracle_step(wl)
    d = to_dev(wl)
    n, c = ws_sizes(wl, P)
    ws = poisoned_workspace(n, c)
    for call in range(2):
        say(f"{name} call {call}")
        repoison(ws, c)
        out = gpu_step(wl, d, out_dtype=torch.float32, workspace=ws)
        assert control_is_zero(ws, c)
        assert_close(out, ref, wl.dtype, label=name)


def test_schedule_order_does_not_change_results():
    """Reversing the batch changes every sequence's place in the schedule
    (and which workgroup runs it) but not its output bits."""
    wl = W.custom(24, seq_lens=[3000, 17, 1200, 1, 0, 640, 2049, 96], num_heads=32,
                  num_kv_heads=8, head_dim=128, block_size=16, dtype=torch.bfloat16)
    d = to_dev(wl)
    say("schedule order")
    out = gpu_step(wl, d, out_dtype=torch.float32, partition_size=512)
    r = torch.arange(wl.num_seqs - 1, -1, -1, device=DEV)
    d2 = dict(d, q=d["q"][r].contiguous(), bt=d["bt"][r].contiguous(), sl=d["sl"][r].contiguous())
    out2 = gpu_step(wl, d2, out_dtype=torch.float32, partition_size=512)
    assert torch.equal(bits(out[r]), bits(out2))


# ----------------------------------------------------------------------------
# the five page-shaped workloads at full size
# ----------------------------------------------------------------------------

_WORKLOADS = {}
_REFS = {}


def _workload(config):
    """Each full-size workload and its oracle result are made once per test
    session (one config held at a time)."""
    if config not in _WORKLOADS:
        _WORKLOADS.clear()
        _REFS.clear()
        _WORKLOADS[config] = W.make(config)
    return _WORKLOADS[config]


def _config_ref(config):
    if config not in _REFS:
        _REFS[config] = oracle_step(_workload(config))
    return _REFS[config]


# (config, partition_size): None is the workload's own launch (the library's
# choice, or 512-token partitions for the mixed batch); the other entry splits
# the same inputs differently.
CONFIG_RUNS = [(1, None), (1, 16), (2, None), (2, 1024), (3, None), (3, 512),
               (4, None), (4, 512), (5, None), (5, 0)]


@pytest.mark.parametrize("config,part", CONFIG_RUNS, ids=[f"cfg{c}-P{p}" for c, p in CONFIG_RUNS])
def test_config_parity(config, part):
    """Every sequence of the workload against the oracle, element by element,
    with both output types; the pools after the step's cache operations bit
    for bit."""
    wl = _workload(config)
    P = wl.partition_size if part is None else part
    say(f"config {config} {wl.name}: S={wl.num_seqs} tokens={wl.num_tokens} "
        f"max_len={wl.max_seq_len} P={P}")
    ref, ek, ev = _config_ref(config)
    n, c = ws_sizes(wl, P)
    for out_dt in (torch.float32, wl.dtype):
        d = to_dev(wl)
        ws = poisoned_workspace(n, c)
        out = gpu_step(wl, d, out_dtype=out_dt, partition_size=P, workspace=ws)
        assert control_is_zero(ws, c)
        if out_dt == torch.float32:
            # bit-exact cache ops over the whole pool
            assert torch.equal(bits(d["kc"].cpu()), bits(ek))
            assert torch.equal(bits(d["vc"].cpu()), bits(ev))
        assert torch.isfinite(out).all()
        assert_close(out, ref, wl.dtype, label=f"config {config} P={P}")
        del d, ws
