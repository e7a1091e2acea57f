"""Block-level sparse decode (oracle; test infrastructure only).

[InplaceKVCache] §4.2 (sparse-selection compatibility): a block-level top-k selection is a set
of whole blocks of the format; attending the selection means attending exactly the tokens of
those blocks.

Two statements of the same thing, written independently so that each pins the other:
  * ``select_blocks`` builds the sub-table the library documents (selected full blocks in
    ascending logical order, then the partial last block if selected) and its length;
  * ``masked_reference`` attends the whole context with every token of an unselected block
    excluded from the softmax (its weight is zero), without any sub-table.
Selection entries < 0 are padding; an index outside the context or a repeat is flagged and
ignored.
"""

import numpy as np

from .attention import attend
from .layout import gather_sequence

BAD_SEQ = 2
BAD_SELECT = 4


def select_blocks(table_row, ctx_len, bs, sel, max_blocks):
    """(sub_row: list of physical ids, sub_len, flags)."""
    ctx_len = int(ctx_len)
    nb = -(-ctx_len // bs) if ctx_len >= 0 else -1
    if nb < 0 or nb > max_blocks:
        return [], 0, BAD_SEQ
    chosen, flags = set(), 0
    for s in sel:
        s = int(s)
        if s < 0:
            continue
        if s >= nb or s in chosen:
            flags |= BAD_SELECT
            continue
        chosen.add(s)
    last = nb - 1 if ctx_len % bs else -1
    full = sorted(j for j in chosen if j != last)
    row = [int(table_row[j]) for j in full]
    sub_len = len(full) * bs
    if last in chosen:
        row.append(int(table_row[last]))
        sub_len += ctx_len - last * bs
    return row, sub_len, flags


def masked_reference(layout, regions, region_blocks, table_row, ctx_len, sel, q, scale):
    """Attention of q [Hq, Dk] over the tokens of the selected blocks, as the full context
    with the other tokens given zero weight."""
    bs = layout.block_size
    k, v = gather_sequence(layout, regions, region_blocks, table_row, 0, int(ctx_len))
    nb = -(-int(ctx_len) // bs)
    keep_block = np.zeros(max(nb, 1), bool)
    for s in sel:
        if 0 <= int(s) < nb:
            keep_block[int(s)] = True
    keep = keep_block[np.arange(int(ctx_len)) // bs] if ctx_len else np.zeros(0, bool)
    return attend(np.asarray(q, np.float64), k[keep], v[keep], scale)
