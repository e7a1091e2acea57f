"""Run-time growth and shrinking of a block pool against the allocator model, host only.

[VAMP] §IV-C, §V-A: reclaimed pages join the free-block pool and are allocatable at once; the
remap also runs in reverse.  The library and ``oracle.alloc`` go through the same random
sequence of allocations, releases, added regions, grown and shrunk last regions; every table
and free count must agree.  Model pins: ids stay a partition of used and free blocks, and a
shrink never removes a used block.
"""

import random

import numpy as np
import pytest

from oracle import alloc as oa
from oracle.alloc import PoolError, PoolModel
from paged_kv_cache_mla_amd import _lib
from paged_kv_cache_mla_amd.api import KvattnError, Pool

FAKE = 0x7F0000000000
BS = 16


def _used(model):
    return sorted(i for i, r in enumerate(model.ref) if r > 0)


@pytest.mark.parametrize("seed", range(6))
def test_growth_and_shrink_match_model(seed):
    rng = random.Random(seed)
    n0 = rng.randrange(4, 40)
    lib = Pool(BS, 2, 64, 64, "bf16", False, [(FAKE, n0)], seed=seed)
    model = PoolModel(n0, seed, BS)
    live = []          # (library table, model table)
    next_base = FAKE + 0x100000000
    for step in range(300):
        op = rng.random()
        if op < 0.35:                                         # allocate a few sequences
            lens = [rng.randrange(0, 6 * BS) for _ in range(rng.randrange(1, 4))]
            st, t_lib, short = lib.block_table(lens, 6)
            try:
                t_mod = model.alloc(lens, 6)
                m_st = _lib.OK
            except PoolError as e:
                m_st = {"exhausted": _lib.E_POOL_EXHAUSTED, "inval": _lib.E_INVAL}[e.kind]
            assert st == m_st
            if st == _lib.OK:
                assert np.array_equal(t_lib, t_mod)
                live.append((t_lib, t_mod))
        elif op < 0.6 and live:                               # release one
            t_lib, t_mod = live.pop(rng.randrange(len(live)))
            assert lib.release(t_lib) == _lib.OK
            model.release(t_mod)
        elif op < 0.72 and lib.num_regions < _lib.MAX_REGIONS:  # add a region
            n = rng.randrange(1, 20)
            assert lib.add_region(next_base, n) == oa.add_region(model, n)
            next_base += 0x100000000
        elif op < 0.86:                                       # grow the last region
            sizes = getattr(model, "region_sizes", [model.total])
            n = sizes[-1] + rng.randrange(1, 12)
            lib.resize_last_region(n)
            oa.resize_last_region(model, n)
        else:                                                 # shrink the last region
            sizes = getattr(model, "region_sizes", [model.total])
            n = rng.randrange(0, sizes[-1] + 1)
            try:
                oa.resize_last_region(model, n)
                m_st = _lib.OK
            except PoolError as e:
                m_st = {"state": _lib.E_STATE, "inval": _lib.E_INVAL}[e.kind]
            if m_st == _lib.OK:
                lib.resize_last_region(n)
            else:
                with pytest.raises(KvattnError) as e:
                    lib.resize_last_region(n)
                assert e.value.status == m_st
        # model pins and agreement
        assert sorted(_used(model) + model.free) == list(range(model.total))
        assert lib.num_free == len(model.free)
        assert lib.num_regions == len(getattr(model, "region_sizes", [model.total]))


def test_added_blocks_are_handed_out_first_in_order():
    lib = Pool(BS, 2, 64, 64, "bf16", False, [(FAKE, 8)], seed=1)
    st, t, _ = lib.block_table([2 * BS], 2)
    assert st == _lib.OK
    first = lib.add_region(FAKE + 0x100000000, 5)
    assert first == 8
    st, t2, _ = lib.block_table([5 * BS], 5)
    assert list(t2[0]) == [8, 9, 10, 11, 12]
    lib.resize_last_region(7)                                 # grows: ids 13, 14
    st, t3, _ = lib.block_table([BS], 1)
    assert t3[0, 0] == 13
    with pytest.raises(KvattnError) as e:                     # 13 is in use
        lib.resize_last_region(5)
    assert e.value.status == _lib.E_STATE
    lib.release(t3)
    lib.release(t2)
    lib.resize_last_region(0)                                 # the added region goes away
    assert lib.num_regions == 1 and lib.num_free == 6
    with pytest.raises(KvattnError) as e:
        lib.resize_last_region(0)                             # never the only region
    assert e.value.status == _lib.E_INVAL


def test_add_region_validation():
    lib = Pool(BS, 2, 64, 64, "bf16", False, [(FAKE, 8)], seed=1)
    with pytest.raises(KvattnError):
        lib.add_region(FAKE + 8, 4)                           # misaligned
    with pytest.raises(KvattnError):
        lib.add_region(FAKE + 0x1000, 0)
    for i in range(_lib.MAX_REGIONS - 1):
        lib.add_region(FAKE + (i + 1) * 0x100000000, 1)
    with pytest.raises(KvattnError):
        lib.add_region(FAKE + 0x900000000, 1)                 # ninth region
