"""Workload definitions and seeded generators (random data, block tables, lengths).

Five workloads, shaped like the models the pages run (sizes of the full variants):
  tiny_fp32      batch 2, lengths 100 and 257, 4 q heads / 1 KV head, d 64, fp32, bs 16,
                 64-block pool, tables = first 7 + 17 entries of a seeded permutation,
                 each sequence cut into 2 partitions.
  gqa_32k        Qwen3-30B-A3B-shaped layer: batch 16 x 32768 tokens, 32 q / 4 KV heads,
                 d 128, bf16, bs 16, pool of exactly the 32768 needed blocks in a seeded
                 permutation, partitions of 512 tokens.
  split_128k     Mixtral-8x7B-shaped split decode: batch 4 x 131072, 32 q / 8 KV heads,
                 d 128, bf16, bs 16; the first fraction r of each sequence lives in a
                 separate host-side pool (its partial is computed elsewhere), the device
                 pool holds only [r*L, L).
  prefix_shared  64 sequences in 8 groups of 8 sharing their first 75% of blocks, lengths
                 16 * U{512..4096}, 16 q / 2 KV heads, d 256, bf16, bs 16, two disjoint
                 regions (base + reclaimed) with seeded interleaving of physical ids.  The
                 prefixes nest: every member other than its group's longest takes its first
                 floor(0.75 * nblocks) blocks from the longest member's table.
  mla_16k        DeepSeek-V2-Lite-shaped MLA: batch 32 x 16384, 16 heads on one 576-d
                 latent (value = first 512), bf16, bs 64, seeded tables, scale 1/sqrt(192).
Each has a "small" variant that the float64 oracle finishes in seconds while still
spanning several blocks / partitions with ragged tails.

Random streams: numpy PCG64 seeded with 1000 + workload number, split with SeedSequence
into independent streams for q, KV data, tables and lengths.  Normal samples are drawn in
float32 and rounded to bfloat16 (round to nearest, ties to even).
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

ABSENT = -1
CHUNK = 1 << 24  # normal samples drawn per call; fixed so results never depend on memory

WORKLOADS = {
    "tiny_fp32": 1,
    "gqa_32k": 2,
    "split_128k": 3,
    "prefix_shared": 4,
    "mla_16k": 5,
}


@dataclass
class Case:
    name: str
    variant: str
    seed: int
    # layout
    block_size: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    dtype: str                      # "f32" | "bf16"
    latent: bool
    # device pool contents: flat element arrays (uint16 bf16 bits or float32)
    regions: List[np.ndarray]
    region_blocks: List[int]
    table: np.ndarray               # int32 [B, max_blocks], ABSENT-padded
    ctx_lens: np.ndarray            # int32 [B]
    tok_begin: Optional[np.ndarray]  # int32 [B] or None (all zero)
    part_tokens: np.ndarray         # int32 [B]
    q: np.ndarray                   # [B, Hq, Dk] uint16 bits or float32
    num_q_heads: int
    scale: float
    # tokens [0, tok_begin) of each sequence held outside the device pool (split workload)
    ext_regions: Optional[List[np.ndarray]] = None
    ext_region_blocks: Optional[List[int]] = None
    ext_table: Optional[np.ndarray] = None
    info: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.table.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def elems_per_block(self) -> int:
        if self.latent:
            return self.block_size * self.head_dim_k
        return self.num_kv_heads * self.block_size * (self.head_dim_k + self.head_dim_v)

    def kv_bytes_per_token(self) -> int:
        """Bytes of K and V (or of the latent) one token occupies."""
        return self.elems_per_block() * self.elem_bytes // self.block_size

    def device_tokens(self) -> int:
        """Tokens each decode step reads from the device pool (algorithmic, each once)."""
        beg = np.zeros_like(self.ctx_lens) if self.tok_begin is None else self.tok_begin
        return int((self.ctx_lens.astype(np.int64) - beg).sum())


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def _normals(rng: np.random.Generator, n: int, dtype: str) -> np.ndarray:
    out = np.empty(n, np.uint16 if dtype == "bf16" else np.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        z = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = bf16_round_bits(z) if dtype == "bf16" else z
    return out


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def _nblocks(length: int, bs: int) -> int:
    return -(-length // bs)


def _finish(name, variant, seed, bs, hkv, dk, dv, dtype, latent, hq, scale, region_blocks,
            table, ctx_lens, tok_begin, part_tokens, rng_q, rng_kv, **extra):
    per_block = bs * dk if latent else hkv * bs * (dk + dv)
    regions = [_normals(rng_kv, n * per_block, dtype) for n in region_blocks]
    q = _normals(rng_q, len(ctx_lens) * hq * dk, dtype).reshape(len(ctx_lens), hq, dk)
    return Case(name=name, variant=variant, seed=seed, block_size=bs, num_kv_heads=hkv,
                head_dim_k=dk, head_dim_v=dv, dtype=dtype, latent=latent, regions=regions,
                region_blocks=list(region_blocks), table=table,
                ctx_lens=np.asarray(ctx_lens, np.int32),
                tok_begin=None if tok_begin is None else np.asarray(tok_begin, np.int32),
                part_tokens=np.asarray(part_tokens, np.int32), q=q, num_q_heads=hq,
                scale=float(scale), **extra)


def _permuted_tables(rng, lens, bs, max_blocks, total=None):
    """Tables that use every id of a pool of exactly the needed blocks, in random order."""
    nbs = [_nblocks(L, bs) for L in lens]
    need = sum(nbs)
    perm = rng.permutation(need if total is None else total).astype(np.int32)
    table = np.full((len(lens), max_blocks), ABSENT, np.int32)
    pos = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    return table, need


def _tiny_fp32(variant):
    seed = 1001
    rq, rkv, rtab, _ = _streams(seed)
    bs, lens = 16, [100, 257]
    perm = rtab.permutation(64).astype(np.int32)
    table = np.full((2, 17), ABSENT, np.int32)
    table[0, :7] = perm[:7]
    table[1, :17] = perm[7:24]
    # two partitions per sequence: P_b = bs * ceil(nblocks_b / 2)
    part = [bs * (-(-_nblocks(L, bs) // 2)) for L in lens]
    return _finish("tiny_fp32", variant, seed, bs, 1, 64, 64, "f32", False, 4, 1 / 8.0,
                   [64], table, lens, None, part, rq, rkv)


def _gqa_32k(variant):
    seed = 1002
    rq, rkv, rtab, _ = _streams(seed)
    bs = 16
    if variant == "full":
        lens = [32768] * 16
    else:
        lens = [2048, 1531, 17, 600]
    max_blocks = _nblocks(max(lens), bs)
    table, need = _permuted_tables(rtab, lens, bs, max_blocks)
    return _finish("gqa_32k", variant, seed, bs, 4, 128, 128, "bf16", False, 32,
                   1 / np.sqrt(128.0), [need], table, lens, None, [512] * len(lens), rq, rkv)


def _split_128k(variant, r=0.5):
    seed = 1003
    rq, rkv, rtab, _ = _streams(seed)
    bs = 16
    if variant == "full":
        lens = [131072] * 4
        begins = [int(r * L) for L in lens]
        part = 1024
    else:
        lens = [4096, 3000]
        begins = [int(r * L) for L in lens]   # 3000 * r need not be block aligned
        part = 512
    max_blocks = _nblocks(max(lens), bs)
    # device pool: blocks of [begin, L) -- a block straddling `begin` lives on both sides
    dev_first = [b // bs for b in begins]
    dev_n = [_nblocks(L, bs) - f for L, f in zip(lens, dev_first)]
    dperm = rtab.permutation(sum(dev_n)).astype(np.int32)
    table = np.full((len(lens), max_blocks), ABSENT, np.int32)
    pos = 0
    for b in range(len(lens)):
        table[b, dev_first[b]:dev_first[b] + dev_n[b]] = dperm[pos:pos + dev_n[b]]
        pos += dev_n[b]
    # host-side pool for [0, begin)
    host_n = [_nblocks(bg, bs) for bg in begins]
    hperm = rtab.permutation(sum(host_n)).astype(np.int32)
    ext_table = np.full((len(lens), max_blocks), ABSENT, np.int32)
    pos = 0
    for b in range(len(lens)):
        ext_table[b, :host_n[b]] = hperm[pos:pos + host_n[b]]
        pos += host_n[b]
    case = _finish("split_128k", variant, seed, bs, 8, 128, 128, "bf16", False, 32,
                   1 / np.sqrt(128.0), [sum(dev_n)], table, lens, begins,
                   [part] * len(lens), rq, rkv)
    per_block = case.elems_per_block()
    case.ext_regions = [_normals(rkv, sum(host_n) * per_block, "bf16")]
    case.ext_region_blocks = [sum(host_n)]
    case.ext_table = ext_table
    case.info["r"] = r
    return case


def _prefix_shared(variant):
    seed = 1004
    rq, rkv, rtab, rlen = _streams(seed)
    bs = 16
    if variant == "full":
        groups, lo, hi = 8, 512, 4096
    else:
        groups, lo, hi = 2, 20, 100
    per_group = 8
    lens = (16 * rlen.integers(lo, hi + 1, size=groups * per_group)).astype(np.int32)
    nbs = [_nblocks(int(L), bs) for L in lens]
    max_blocks = max(nbs)
    # nested prefixes: in each group the longest member (the lowest index among equals) owns
    # its whole table; every other member's first floor(0.75 * nblocks) blocks are the
    # leader's first blocks (shared, ref-counted), the rest of its table is private
    leaders, shared = [], []
    for g in range(groups):
        members = list(range(g * per_group, (g + 1) * per_group))
        lead = max(members, key=lambda m: (nbs[m], -m))
        leaders.append(lead)
        for m in members:
            shared.append(0 if m == lead else (3 * nbs[m]) // 4)
    total = sum(nbs[m] - shared[m] for m in range(len(lens)))
    ids = rtab.permutation(total).astype(np.int32)    # seeded interleave over both regions
    table = np.full((len(lens), max_blocks), ABSENT, np.int32)
    pos = 0
    for g in range(groups):
        lead = leaders[g]
        table[lead, :nbs[lead]] = ids[pos:pos + nbs[lead]]
        pos += nbs[lead]
        for m in range(g * per_group, (g + 1) * per_group):
            if m == lead:
                continue
            table[m, :shared[m]] = table[lead, :shared[m]]
            priv = nbs[m] - shared[m]
            table[m, shared[m]:nbs[m]] = ids[pos:pos + priv]
            pos += priv
    base = int(np.ceil(0.37 * total))
    case = _finish("prefix_shared", variant, seed, bs, 2, 256, 256, "bf16", False, 16,
                   1 / 16.0, [base, total - base], table, lens, None,
                   [512] * len(lens), rq, rkv)
    case.info["shared_blocks"] = shared     # per sequence: leading blocks taken from its leader
    case.info["leaders"] = leaders
    case.info["group_size"] = per_group
    return case


def _mla_16k(variant):
    seed = 1005
    rq, rkv, rtab, _ = _streams(seed)
    bs = 64
    if variant == "full":
        lens = [16384] * 32
        part = 512
    else:
        lens = [1000, 64, 333]
        part = 256
    max_blocks = _nblocks(max(lens), bs)
    table, need = _permuted_tables(rtab, lens, bs, max_blocks)
    return _finish("mla_16k", variant, seed, bs, 1, 576, 512, "bf16", True, 16,
                   1 / np.sqrt(192.0), [need], table, lens, None, [part] * len(lens), rq, rkv)


def gqa_case(block_size, num_kv_heads, head_dim, num_q_heads, lens, part_tokens,
             tok_begin=None, dtype: str = "bf16", seed: int = 1007) -> Case:
    """A per-head K/V (GQA) case of any geometry with the given context lengths, partition
    sizes and first tokens, over a pool of exactly the blocks needed, in random order."""
    rq, rkv, rtab, _ = _streams(seed)
    max_blocks = _nblocks(max(lens), block_size)
    table, need = _permuted_tables(rtab, lens, block_size, max_blocks)
    return _finish("gqa_custom", "small", seed, block_size, num_kv_heads, head_dim, head_dim,
                   dtype, False, num_q_heads, 1 / np.sqrt(float(head_dim)), [need], table, lens,
                   tok_begin, part_tokens, rq, rkv)


def mla_case(lens, part_tokens, tok_begin=None, seed: int = 1006, num_q_heads: int = 16) -> Case:
    """A latent-cache (MLA) case of the 16K layer's geometry (bs 64, Dk 576, Dv 512, up to 16
    heads) with the given context lengths, partition sizes and first tokens, over a pool of
    exactly the blocks needed, in random order."""
    rq, rkv, rtab, _ = _streams(seed)
    bs = 64
    max_blocks = _nblocks(max(lens), bs)
    table, need = _permuted_tables(rtab, lens, bs, max_blocks)
    return _finish("mla_custom", "small", seed, bs, 1, 576, 512, "bf16", True, num_q_heads,
                   1 / np.sqrt(192.0), [need], table, lens, tok_begin, part_tokens, rq, rkv)


def make_case(name: str, variant: str = "small", **kw) -> Case:
    """Build workload `name` ("tiny_fp32", "gqa_32k", "split_128k", "prefix_shared",
    "mla_16k") in variant "small" or "full"; split_128k takes r (default 0.5)."""
    if variant not in ("small", "full"):
        raise ValueError(variant)
    fn = {"tiny_fp32": _tiny_fp32, "gqa_32k": _gqa_32k, "split_128k": _split_128k,
          "prefix_shared": _prefix_shared, "mla_16k": _mla_16k}[name]
    return fn(variant, **kw)
