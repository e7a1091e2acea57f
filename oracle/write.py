"""Writing new tokens into blocks (oracle; test infrastructure only).

[InplaceKVCache] §4.1: the block is the unit of write-time placement; §4.2: a new decode
token's key and value are written into the GPU's staging window at once.  The element
positions follow the block layout restated in ``oracle.layout`` (this library's choice):

  GQA block = [K part | V part], x = 16 // element bytes:
      K[t, h, c*x + u]  ->  element ((h * (Dk // x) + c) * bs + t) * x + u
      V[t, h, j]        ->  element Hkv * bs * Dk + (h * Dv + j) * bs + t
  MLA block:
      C[t, c*x + u]     ->  element (c * bs + t) * x + u

Values are passed in their storage form (uint16 bf16 bit patterns or float32) and stored
unchanged: a write is a pure placement.
"""

import numpy as np

from .layout import ABSENT, Layout, block_elems, locate


def write_tokens(layout: Layout, regions, region_blocks, table_row, t0: int, k, v=None):
    """Store tokens t0 .. t0 + n - 1 of one sequence.

    k: [n, Hkv, Dk] (MLA: [n, Dk]) and v: [n, Hkv, Dv] (MLA: None), in the regions' storage
    dtype.  `regions` (flat element arrays) are modified in place.  Every touched table
    entry must be a resident block.
    """
    bs, x = layout.block_size, layout.chunk
    dk, dv, hkv = layout.head_dim_k, layout.head_dim_v, layout.num_kv_heads
    nel = block_elems(layout)
    k = np.asarray(k)
    n = k.shape[0]
    for i in range(n):
        t = t0 + i
        pid = int(table_row[t // bs])
        if pid == ABSENT:
            raise ValueError(f"token {t}: logical block {t // bs} is not resident")
        r, local = locate(pid, region_blocks)
        blk = regions[r][local * nel:(local + 1) * nel]
        ts = t % bs
        if layout.latent:
            for d in range(dk):
                c, u = divmod(d, x)
                blk[(c * bs + ts) * x + u] = k[i, d]
            continue
        for h in range(hkv):
            for d in range(dk):
                c, u = divmod(d, x)
                blk[((h * (dk // x) + c) * bs + ts) * x + u] = k[i, h, d]
            for j in range(dv):
                blk[hkv * bs * dk + (h * dv + j) * bs + ts] = v[i, h, j]
