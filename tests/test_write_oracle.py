"""Pins of the oracle's token writer (``oracle.write_tokens``), CPU only.

The writer places new tokens' K/V in their blocks ([InplaceKVCache] §4.1, §4.2).  It is pinned
against a second, loop-based statement of the block layout (the element-wise scatter of the
layout pin test) and by round trips through the oracle's reader, and it must touch nothing but
the written tokens' elements.
"""

import numpy as np
import pytest

from oracle import Layout, bf16_bits_to_f64, block_elems, gather_sequence, write_tokens
from synth import bf16_round_bits
from tests.test_oracle_pins import _write_pool_elementwise


def _layouts():
    return [Layout(4, 3, 8, 8, "f32", False), Layout(8, 1, 24, 16, "f32", True),
            Layout(16, 2, 16, 16, "bf16", False), Layout(64, 1, 48, 32, "bf16", True)]


def _tokens(rng, layout, n):
    """Dense K [n, Hkv, Dk] and V [n, Hkv, Dv] in the storage dtype (V = leading latent
    columns for MLA)."""
    kf = rng.standard_normal((n, layout.num_kv_heads, layout.head_dim_k)).astype(np.float32)
    vf = (kf[:, :, :layout.head_dim_v] if layout.latent else
          rng.standard_normal((n, layout.num_kv_heads, layout.head_dim_v)).astype(np.float32))
    if layout.dtype == "bf16":
        return bf16_round_bits(kf), bf16_round_bits(vf)
    return kf, vf


def _widen(a, layout):
    return bf16_bits_to_f64(a) if layout.dtype == "bf16" else a.astype(np.float64)


@pytest.mark.parametrize("layout", _layouts(),
                         ids=lambda l: f"{l.dtype}-{'mla' if l.latent else 'gqa'}")
def test_writes_in_pieces_equal_elementwise_scatter(layout):
    rng = np.random.default_rng(11)
    n = 3 * layout.block_size + 5
    nblk = -(-n // layout.block_size)
    region_blocks = [2, nblk + 1]
    table = rng.permutation(sum(region_blocks))[:nblk].astype(np.int32)
    k, v = _tokens(rng, layout, n)
    # the loop-based scatter, on the values widened to float64 (NaN = never written)
    ref = _write_pool_elementwise(layout, _widen(k, layout), _widen(v, layout), table,
                                  region_blocks, np.float64)
    nel = block_elems(layout)
    store = np.uint16 if layout.dtype == "bf16" else np.float32
    fill = np.uint16(0x7FC1) if layout.dtype == "bf16" else np.float32(-7.25)
    regions = [np.full(nb * nel, fill, store) for nb in region_blocks]
    # pieces of random sizes, written out of order
    cuts = sorted(set(rng.integers(1, n, 5).tolist()) | {0, n})
    pieces = list(zip(cuts[:-1], cuts[1:]))
    rng.shuffle(pieces)
    for lo, hi in pieces:
        if layout.latent:
            write_tokens(layout, regions, region_blocks, table, lo, k[lo:hi, 0, :])
        else:
            write_tokens(layout, regions, region_blocks, table, lo, k[lo:hi], v[lo:hi])
    for r in range(len(regions)):
        written = ~np.isnan(ref[r])
        assert np.array_equal(_widen(regions[r][written], layout), ref[r][written])
        assert np.all(regions[r][~written] == fill)   # nothing else touched
    kk, vv = gather_sequence(layout, regions, region_blocks, table, 0, n)
    assert np.array_equal(kk, _widen(k, layout)) and np.array_equal(vv, _widen(v, layout))


# the random region bytes include signalling-NaN bf16 patterns outside the written tokens;
# widening them to float64 is exact (NaN stays NaN) but numpy reports the cast as invalid
@pytest.mark.filterwarnings("ignore:invalid value encountered in cast:RuntimeWarning")
def test_write_touches_only_its_tokens():
    layout = Layout(16, 2, 16, 16, "bf16", False)
    rng = np.random.default_rng(5)
    nel = block_elems(layout)
    regions = [rng.integers(0, 1 << 16, 6 * nel, dtype=np.uint16)]
    before = regions[0].copy()
    table = np.array([4, 1, 3], np.int32)
    k, v = _tokens(rng, layout, 2)
    write_tokens(layout, regions, [6], table, 15, k, v)   # tokens 15 (block 4) and 16 (block 1)
    changed = np.nonzero(regions[0] != before)[0]
    assert len(changed) <= 2 * 2 * (16 + 16)
    assert set((changed // nel).tolist()) <= {4, 1}
    kk, vv = gather_sequence(layout, regions, [6], table, 15, 17)
    assert np.array_equal(kk, _widen(k, layout)) and np.array_equal(vv, _widen(v, layout))
