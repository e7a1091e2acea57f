"""Whole decode step of the oracle: resolve each sequence, attend, split, merge.

Test infrastructure only.  Built from `layout.gather_sequence` (logical -> physical
resolution, [CrossPool] §3.1), `attention.attend` / `attention.merge` (exact attention and
LSE merge, [InplaceKVCache] §5.1, §6.1) and `partition.partition_ranges` (sequence split).
"""

import numpy as np

from .attention import attend, merge
from .layout import ABSENT, Layout, gather_sequence, locate, token_k_offset
from .partition import partition_ranges


def _q_f64(q, layout: Layout):
    from .bf16 import bf16_bits_to_f64
    q = np.asarray(q)
    if q.dtype == np.uint16:
        return bf16_bits_to_f64(q)
    return q.astype(np.float64)


def decode_reference(layout: Layout, regions, region_blocks, table, ctx_lens, q, scale,
                     tok_begin=None, seqs=None):
    """Unsplit attention of each sequence b over its tokens [tok_begin[b], ctx_lens[b]).

    q [B, Hq, Dk] (uint16 bf16 bits or float32).  Returns o [B, Hq, Dv], lse [B, Hq] in
    float64 (rows not listed in `seqs` are left zero / -inf).
    """
    qf = _q_f64(q, layout)
    bsz, hq, _ = qf.shape
    o = np.zeros((bsz, hq, layout.head_dim_v))
    lse = np.full((bsz, hq), -np.inf)
    for b in (range(bsz) if seqs is None else seqs):
        lo = 0 if tok_begin is None else int(tok_begin[b])
        k, v = gather_sequence(layout, regions, region_blocks, table[b], lo, int(ctx_lens[b]))
        o[b], lse[b] = attend(qf[b], k, v, scale)
    return o, lse


def decode_partials_reference(layout: Layout, regions, region_blocks, table, ctx_lens, q,
                              scale, part_tokens, tok_begin=None, seqs=None):
    """Per-partition partials: list over b of (o [np_b, Hq, Dv], lse [np_b, Hq])."""
    qf = _q_f64(q, layout)
    out = []
    for b in (range(qf.shape[0]) if seqs is None else seqs):
        lo = 0 if tok_begin is None else int(tok_begin[b])
        os_, ls_ = [], []
        for p_lo, p_hi in partition_ranges(int(ctx_lens[b]), lo, int(part_tokens[b])):
            k, v = gather_sequence(layout, regions, region_blocks, table[b], p_lo, p_hi)
            o_p, l_p = attend(qf[b], k, v, scale)
            os_.append(o_p)
            ls_.append(l_p)
        hq = qf.shape[1]
        out.append((np.array(os_).reshape(len(os_), hq, layout.head_dim_v),
                    np.array(ls_).reshape(len(ls_), hq)))
    return out


def resolve_offsets_reference(layout: Layout, region_blocks, table, ctx_lens, max_tokens):
    """(region index, byte offset of K(h=0, t, 0)) for every (b, t); -1 where not resident."""
    from .layout import block_elems
    bsz = len(ctx_lens)
    region = np.full((bsz, max_tokens), -1, np.int32)
    offset = np.full((bsz, max_tokens), -1, np.int64)
    total = int(sum(region_blocks))
    bb = block_elems(layout) * layout.elem_bytes
    for b in range(bsz):
        for t in range(min(int(ctx_lens[b]), max_tokens)):
            pid = int(table[b][t // layout.block_size])
            if pid == ABSENT or pid < 0 or pid >= total:
                continue
            r, local = locate(pid, region_blocks)
            region[b, t] = r
            offset[b, t] = local * bb + token_k_offset(layout, t % layout.block_size) * layout.elem_bytes
    return region, offset
