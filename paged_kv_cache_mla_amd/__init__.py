"""Paged-KV decode attention with split-sequence LSE merge for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libkvattn.so`` (hand-written HIP kernels, see
``include/kvattn.h``); this package is its thin Python binding.  Importing the package
loads nothing; the first call loads the library and raises if it has not been built.
"""

from .api import (BF16, F32, DecodeStep, HostShare, KVStore, KvattnError, Pool,
                  ShareController, append_kv, block_bytes, decode_partial, host_partial,
                  merge_lse, partition_count, resolve_offsets, share_fit, share_optimum)

__all__ = ["BF16", "F32", "DecodeStep", "HostShare", "KVStore", "KvattnError", "Pool",
           "ShareController", "append_kv", "block_bytes", "decode_partial", "host_partial",
           "merge_lse", "partition_count", "resolve_offsets", "share_fit", "share_optimum"]
