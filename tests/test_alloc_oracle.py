"""Pins of the oracle's model of the block pool (free-list order, sharing, all-or-nothing).

SplitMix64 is pinned by its published first outputs for seed 0; the Fisher-Yates shuffle
by exhaustive enumeration of its random choices (Durstenfeld's variant maps the n! choice
sequences one-to-one onto the n! permutations); the pool semantics by direct scenarios.
"""

import itertools

import numpy as np
import pytest

from oracle.alloc import PoolError, PoolModel, SplitMix64, shuffled_ids


def test_splitmix64_published_outputs_seed0():
    g = SplitMix64(0)
    assert [g.next() for _ in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                            0x06C45D188009454F]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_fisher_yates_choice_sequences_are_a_bijection(n):
    perms = set()
    ranges = [range(i + 1) for i in range(n - 1, 0, -1)]      # choices j_i in [0, i]
    for choice in itertools.product(*ranges):
        it = iter(choice)
        p = tuple(shuffled_ids(n, 0, draw=lambda i: next(it)))
        assert sorted(p) == list(range(n))
        perms.add(p)
    assert len(perms) == int(np.prod(range(1, n + 1)))


def test_seeded_shuffle_is_a_permutation_and_seed_dependent():
    a = shuffled_ids(1000, 7)
    b = shuffled_ids(1000, 8)
    assert sorted(a) == list(range(1000)) and a != b
    assert shuffled_ids(1000, 7) == a


def test_pool_model_share_release_exhaust():
    pm = PoolModel(20, seed=3, block_size=4)
    order = shuffled_ids(20, 3)
    t = pm.alloc([9, 8], max_blocks=4)               # 3 + 2 blocks
    assert t.tolist() == [order[0:3] + [-1], order[3:5] + [-1, -1]]
    t2 = pm.alloc([16, 12], max_blocks=4, share_src=[-1, 0], share_nblocks=[0, 2])
    assert t2[1, :2].tolist() == t2[0, :2].tolist()
    assert pm.ref[int(t2[0, 0])] == 2
    free_before = len(pm.free)
    with pytest.raises(PoolError) as e:
        pm.alloc([4 * 20], max_blocks=20)
    assert e.value.kind == "exhausted" and e.value.shortfall == 20 - free_before
    assert len(pm.free) == free_before
    pm.release(t2)
    with pytest.raises(PoolError) as e:
        pm.release(t2[:1])                         # private blocks of row 0 already free
    assert e.value.kind == "state"
    pm.release(t)
    assert len(pm.free) == 20 and all(r == 0 for r in pm.ref)
    # the most recently released block is handed out first
    last = int(t[1, 1])
    assert pm.alloc([1], max_blocks=1)[0, 0] == last


def test_pool_model_first_tok_and_explicit():
    pm = PoolModel(10, seed=1, block_size=16)
    t = pm.alloc([64], max_blocks=4, first_tok=[33])    # blocks 0, 1 absent
    assert t[0, :2].tolist() == [-1, -1] and (t[0, 2:] >= 0).all()
    with pytest.raises(PoolError) as e:
        pm.claim_explicit([16], np.array([[int(t[0, 2])]]))
    assert e.value.kind == "state"
    free_id = pm.free[0]
    got = pm.claim_explicit([32, 16], np.array([[free_id, -1], [free_id, -1]]))
    assert pm.ref[free_id] == 2 and free_id not in pm.free and got[1, 0] == free_id
    with pytest.raises(PoolError) as e:
        pm.claim_explicit([16], np.array([[10]]))
    assert e.value.kind == "range"
