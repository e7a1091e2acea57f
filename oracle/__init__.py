"""Reference oracle for paged-KV decode attention with split-sequence LSE merge.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, float64 CPU definition that
the HIP path is checked against.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it; the
product path (``paged_kv_cache_mla_amd``) never does, and this package imports nothing
from it.  The two share no code: the oracle re-derives the block layout, the address
resolution, the attention and the merge from their definitions.

Sources (cited by tag):
  [InplaceKVCache] "Physically Partitioned KVCache Format for CPU-GPU Load Balancing in MoE
                   Inference" -- §4.1 block-organised regions, §4.2 the CPU returns only its
                   partial output and normalisers and the GPU merges, §5.1 sequence-dimension
                   split with exact LSE merge, §5.2-5.3 Eq. 1-2 the share policy
                   (``oracle.share``), §6.1 exact attention with online softmax.
  [CrossPool]      "CrossPool: Efficient Multi-LLM Serving for Cold MoE Models through
                   KV-Cache and Weight Disaggregation" -- §3.1 paged KV interface over a
                   logical KV address space.
  [VAMP]           "Dynamic HBM Repartitioning for Multi-Turn MoE Serving" -- §IV-C, §V-A
                   reclaimed pages joining the free-block pool.

Parity pins: every function here is pinned on the CPU by
  ``tests/test_oracle_pins.py``    attention and merge (closed forms, invariants, brute force
                                   at 50 digits, a library special case), the layout reader
                                   against an element-wise writer, partition ranges, the
                                   per-partition partials against attention over dense slices,
                                   the address resolution against the element at each returned
                                   offset (planted mistakes must fail);
  ``tests/test_alloc_oracle.py``   the allocator model (published SplitMix64 outputs,
                                   exhaustive permutation counts);
  ``tests/test_share_policy.py``   the share policy (brute-force minimum of Eq. 1's step
                                   time, balance, limits, exact cost recovery, a line fit);
  ``tests/test_write_oracle.py``   the token writer (a loop-based statement of the layout,
                                   round trips through the reader, untouched elements);
  ``tests/test_sparse_oracle.py``  block selection (sub-table and masked statements along
                                   different routes; all blocks selected gives the dense case);
  ``tests/test_kvstore_cpu.py``    the placement-store model (token conservation, blocks
                                   neither lost nor duplicated, copies exactly the CPU-routed
                                   blocks).
None is "parity unpinned".
"""

from .bf16 import bf16_bits_to_f64
from .layout import Layout, block_elems, gather_sequence, token_k_offset
from .attention import attend, merge
from .partition import partition_count, partition_ranges
from .write import write_tokens
from .decode import decode_reference, decode_partials_reference, resolve_offsets_reference
from . import alloc
from . import share
from . import sparse

__all__ = [
    "bf16_bits_to_f64",
    "Layout",
    "block_elems",
    "gather_sequence",
    "token_k_offset",
    "attend",
    "merge",
    "partition_count",
    "partition_ranges",
    "write_tokens",
    "decode_reference",
    "decode_partials_reference",
    "resolve_offsets_reference",
    "alloc",
    "share",
    "sparse",
]
