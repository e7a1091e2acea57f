"""Partition bookkeeping of the sequence-dimension split (oracle; test infrastructure only).

[InplaceKVCache] §5.1 splits each sequence along its tokens, each engine covering a
disjoint token range over all heads.  Here the device-resident range [begin, L) is cut
into consecutive pieces of P tokens; the last piece may be short.
"""


def partition_count(ctx_len: int, begin: int, part_tokens: int) -> int:
    """ceil((L - begin) / P); 0 for an empty range; -1 for invalid arguments."""
    if ctx_len < 0 or begin < 0 or begin > ctx_len or part_tokens <= 0:
        return -1
    n = ctx_len - begin
    return -(-n // part_tokens)


def partition_ranges(ctx_len: int, begin: int, part_tokens: int):
    """List of (lo, hi) token ranges of the partitions, in order."""
    count = partition_count(ctx_len, begin, part_tokens)
    if count < 0:
        raise ValueError("invalid partition arguments")
    out = []
    for p in range(count):
        lo = begin + p * part_tokens
        out.append((lo, min(ctx_len, lo + part_tokens)))
    return out
