"""Plain CPU oracle for paged KV-cache decode attention (test infrastructure).

This package is test infrastructure. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the product
path (``paged_kv_cache_154_amd``) never does, and the two share no code.

Everything here is written from the four web pages on PagedAttention that the
package documentation names, in float64 for attention (exact conversion from
fp32/fp16/bf16 storage) and as bit copies for the cache operations.

Pins (checked by ``tests/test_oracle_*.py`` without a GPU):
  * ``decode``: contiguous scaled-dot-product attention from torch in float64
    on an independently gathered K/V, seq_len = 1 returns the V row, q = 0
    returns the mean of V, a dominant key selects its V row, GQA equals MHA
    with each KV head repeated, invariance under physical-block permutation
    and under re-packing at another block size, NaN in unused slots ignored.
  * ``reshape_and_cache``: the slot worked out from the block table of the
    three-level mapping example (PagedAttention principle, tbr8.org, §2.1)
    and the slot rule of the block engine (LLM inference engine internals,
    §2.3); every other byte unchanged.
  * ``copy_blocks``: destination equals the pre-call source, all else
    unchanged, and decode after a copy-on-write remap equals decode before.
  * ``decode_shared_prefix``: on the prefix-sharing batch, the tables it
    builds from each group's shared blocks and each sample's own blocks are
    the samples' block tables, so it equals ``decode`` of the batch; a group
    of one with an empty prefix is ``decode``.
  * ``swap_blocks``: destination blocks equal the source blocks, all else
    unchanged, the source untouched; swapping out and back in to other
    blocks, with the block table remapped, leaves decode unchanged; within
    one pool it is ``copy_blocks``.
  * ``multi_query`` (q_len new tokens per sequence): row j equals ``decode``
    of the sequence truncated to the positions it sees; one new token is
    decode; changing position p changes exactly the rows that see it.
  * closed forms: the printed KV-size, block-size and pool-sizing numbers.
  * ``fp8_kv`` (an e4m3 KV cache, LLM inference optimisation in practice,
    §6.2): the value table against its landmarks (smallest subnormal and
    normal, 1, 448, NaN) and torch's float8_e4m3fn for all 256 codes; the
    encoder against torch's rounding inside the range, every midpoint to the
    even code, saturation at 448, NaN and signed zero, a round trip of every
    finite code, the quotient formed in fp32; the scatter's placement and
    negative slots; attention over pools of small integers (exact in e4m3)
    equal to ``decode``, k_scale and v_scale acting as scalings; multi-query
    rows equal to decodes of their prefixes; shared-prefix decode equal to
    ``decode_fp8`` over the joined tables; planted mistakes (scales
    swapped or dividing, exponent bias 8, no subnormals, ties away from
    even, no saturation) each fail a pin.
No function here is "parity unpinned".
"""

from .paged_attention import (  # noqa: F401
    blocks_needed,
    block_bytes,
    copy_blocks,
    decode,
    decode_one,
    decode_shared_prefix,
    kv_cache_bytes,
    multi_query,
    multi_query_one,
    reshape_and_cache,
    swap_blocks,
)
from . import fp8_kv  # noqa: F401,E402
