"""Block layout and logical-to-physical resolution (oracle; test infrastructure only).

The cache is a set of regions, each a flat array of elements holding whole blocks
([InplaceKVCache] §4.1: each region is organised in fixed-size blocks).  Physical block ids
run consecutively over the regions in order ([VAMP] §IV-C, §V-A: reclaimed HBM pages join
the same free-block pool as the base region).  A per-sequence block table maps logical
block i (tokens i*bs .. i*bs+bs-1) to a physical id ([CrossPool] §3.1: kernels see a logical
KV address space, physical pages are placed by the virtualiser).

The arrangement of elements inside a block is this library's own choice (the pages only
fix that blocks have a fixed size); it is restated here from its definition:

  e = element bytes (4 for f32, 2 for bf16), x = 16 // e, bs = block size.
  GQA block = [K part | V part]:
      K part viewed as [Hkv][Dk // x][bs][x]:  K[t, h, c*x + u] = Kpart[h, c, t, u]
      V part viewed as [Hkv][Dv][bs]:          V[t, h, j]       = Vpart[h, j, t]
  MLA block viewed as [Dk // x][bs][x]:        C[t, c*x + u]    = block[c, t, u]
      K = C, V = C[:, :Dv]  (one latent shared by all heads).
"""

from dataclasses import dataclass

import numpy as np

from .bf16 import bf16_bits_to_f64

ABSENT = -1


@dataclass(frozen=True)
class Layout:
    block_size: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    dtype: str  # "f32" or "bf16"
    latent: bool = False

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def chunk(self) -> int:
        """Elements per 16-byte chunk."""
        return 16 // self.elem_bytes


def block_elems(layout: Layout) -> int:
    """Elements in one block."""
    if layout.latent:
        return layout.block_size * layout.head_dim_k
    return layout.num_kv_heads * layout.block_size * (layout.head_dim_k + layout.head_dim_v)


def _to_f64(raw: np.ndarray, layout: Layout) -> np.ndarray:
    if layout.dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if raw.dtype != np.float32:
        raise TypeError(f"f32 layout expects float32 storage, got {raw.dtype}")
    return raw.astype(np.float64)


def unpack_block(layout: Layout, block: np.ndarray):
    """One block's flat element array -> (K [bs, Hkv, Dk], V [bs, Hkv, Dv]) as float64."""
    bs, hkv, dk, dv, x = (layout.block_size, layout.num_kv_heads, layout.head_dim_k,
                          layout.head_dim_v, layout.chunk)
    vals = _to_f64(block, layout)
    if layout.latent:
        c = vals.reshape(dk // x, bs, x).transpose(1, 0, 2).reshape(bs, dk)
        return c[:, None, :], c[:, None, :dv]
    kpart = vals[: hkv * bs * dk].reshape(hkv, dk // x, bs, x)
    vpart = vals[hkv * bs * dk:].reshape(hkv, dv, bs)
    k = kpart.transpose(2, 0, 1, 3).reshape(bs, hkv, dk)
    v = vpart.transpose(2, 0, 1)
    return k, v


def locate(block_id: int, region_blocks) -> tuple:
    """Physical id -> (region index, index of the block inside that region)."""
    first = 0
    for r, n in enumerate(region_blocks):
        if first <= block_id < first + n:
            return r, block_id - first
        first += n
    raise IndexError(f"block id {block_id} outside the pool of {first} blocks")


def gather_sequence(layout: Layout, regions, region_blocks, table_row, lo: int, hi: int):
    """Dense float64 K [hi-lo, Hkv, Dk] and V [hi-lo, Hkv, Dv] of logical tokens [lo, hi).

    `regions` are flat element arrays (uint16 bf16 bits or float32), region r holding
    region_blocks[r] blocks.  Every block touched must be resident (not ABSENT).
    """
    bs = layout.block_size
    nel = block_elems(layout)
    n = hi - lo
    k_out = np.empty((n, layout.num_kv_heads, layout.head_dim_k), np.float64)
    v_out = np.empty((n, layout.num_kv_heads, layout.head_dim_v), np.float64)
    if n <= 0:
        return k_out[:0], v_out[:0]
    for blk in range(lo // bs, (hi - 1) // bs + 1):
        pid = int(table_row[blk])
        if pid == ABSENT:
            raise ValueError(f"logical block {blk} is not resident")
        r, local = locate(pid, region_blocks)
        k, v = unpack_block(layout, regions[r][local * nel:(local + 1) * nel])
        t0 = max(lo, blk * bs)
        t1 = min(hi, (blk + 1) * bs)
        k_out[t0 - lo:t1 - lo] = k[t0 - blk * bs:t1 - blk * bs]
        v_out[t0 - lo:t1 - lo] = v[t0 - blk * bs:t1 - blk * bs]
    return k_out, v_out


def token_k_offset(layout: Layout, t_in_block: int) -> int:
    """Element offset, inside its block, of K(head 0, token t, dim 0) (MLA: C(t, 0))."""
    # Head 0 and dim 0 sit in chunk 0, whose bs token slots are consecutive x-element runs.
    return t_in_block * layout.chunk
