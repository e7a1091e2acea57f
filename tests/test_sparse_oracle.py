"""Pins of the block-sparse oracle (``oracle.sparse``), CPU only.

[InplaceKVCache] §4.2: a block-level selection is a set of whole blocks.  The sub-table
statement (``select_blocks``) and the masked statement (``masked_reference``) are computed
along different routes and must agree; selecting every block must give back the dense case.
"""

import numpy as np
import pytest

import oracle
from oracle import Layout, block_elems, gather_sequence
from oracle.sparse import BAD_SELECT, masked_reference, select_blocks


def _case(rng, layout, ctx_len):
    nb = -(-ctx_len // layout.block_size)
    total = nb + 5
    nel = block_elems(layout)
    regions = [rng.standard_normal(total * nel).astype(np.float32)]
    table = rng.permutation(total)[:nb].astype(np.int32)
    q = rng.standard_normal((4, layout.head_dim_k))
    return regions, [total], table, q


@pytest.mark.parametrize("ctx_len", [64, 61, 1, 17])
def test_selecting_every_block_is_the_dense_case(ctx_len):
    rng = np.random.default_rng(ctx_len)
    layout = Layout(16, 2, 32, 32, "f32", False)
    regions, rb, table, q = _case(rng, layout, ctx_len)
    nb = len(table)
    sel = rng.permutation(nb)
    row, sub_len, flags = select_blocks(table, ctx_len, 16, sel, nb)
    assert flags == 0 and sub_len == ctx_len and row == [int(x) for x in table]
    o1, l1 = oracle.attend(q, *gather_sequence(layout, regions, rb, np.array(row), 0, sub_len), 0.3)
    o2, l2 = oracle.attend(q, *gather_sequence(layout, regions, rb, table, 0, ctx_len), 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("latent", [False, True])
def test_sub_table_route_equals_masked_route(seed, latent):
    rng = np.random.default_rng(100 + seed)
    layout = Layout(8, 1, 24, 16, "f32", True) if latent else Layout(16, 2, 32, 32, "f32", False)
    bs = layout.block_size
    ctx_len = int(rng.integers(1, 12 * bs))
    regions, rb, table, q = _case(rng, layout, ctx_len)
    nb = len(table)
    k = int(rng.integers(1, nb + 3))
    sel = rng.integers(-1, nb, k)                       # padding and repeats included
    row, sub_len, flags = select_blocks(table, ctx_len, bs, sel, nb)
    o_sub, l_sub = oracle.attend(q, *gather_sequence(layout, regions, rb, np.array(row, np.int32),
                                                     0, sub_len), 0.25)
    o_msk, l_msk = masked_reference(layout, regions, rb, table, ctx_len, sel, q, 0.25)
    assert np.max(np.abs(o_sub - o_msk)) <= 1e-12
    if np.all(np.isneginf(l_msk)):          # nothing selected: no weight on either route
        assert np.all(np.isneginf(l_sub))
    else:
        assert np.max(np.abs(l_sub - l_msk)) <= 1e-12
    # the order of the selection does not matter
    assert select_blocks(table, ctx_len, bs, sel[::-1], nb)[:2] == (row, sub_len)


def test_flags_and_padding():
    table = np.arange(10, 14, dtype=np.int32)
    row, sub_len, flags = select_blocks(table, 50, 16, [-1, 2, 2, 4, -7, 0], 4)
    assert row == [10, 12] and sub_len == 32 and flags == BAD_SELECT
    row, sub_len, flags = select_blocks(table, 50, 16, [3, 1], 4)      # partial block 3 last
    assert row == [11, 13] and sub_len == 16 + 2 and flags == 0
    assert select_blocks(table, 0, 16, [0], 4) == ([], 0, BAD_SELECT)
    assert select_blocks(table, 65, 16, [0], 4)[2] == 2                  # beyond max_blocks


def test_partial_block_must_come_last():
    """Placing the partial block anywhere but last reads the wrong tokens: the masked route
    tells the difference (a planted mistake in the sub-table order)."""
    rng = np.random.default_rng(9)
    layout = Layout(16, 2, 32, 32, "f32", False)
    ctx_len = 16 * 3 + 5
    regions, rb, table, q = _case(rng, layout, ctx_len)
    sel = [0, 3, 2]
    row, sub_len, _ = select_blocks(table, ctx_len, 16, sel, 4)
    wrong = [row[-1]] + row[:-1]
    o_bad, _ = oracle.attend(q, *gather_sequence(layout, regions, rb, np.array(wrong), 0, sub_len), 0.3)
    o_ref, _ = masked_reference(layout, regions, rb, table, ctx_len, sel, q, 0.3)
    assert np.max(np.abs(o_bad - o_ref)) > 1e-3
