"""Write-time placement store (kvattn_kvstore_*) against the oracle's model, host only.

Pins of the model itself (facts that follow from the contract, not restatements of it):
  * tokens are conserved: CPU view + GPU view lengths equal every token appended;
  * no block is lost or duplicated: the views' blocks and the pools' free lists partition the
    pools' ids;
  * a batch routed to the GPU copies nothing; copies are exactly the CPU-routed blocks;
  * the CPU view holds exactly the tokens each sequence's controller placed on the CPU.
Then the library must reproduce the model's views, copy lists and flags step by step.
Device and host addresses are fake: the plan calls never touch memory.
"""

import random

import numpy as np
import pytest

from oracle import share as osh
from oracle.alloc import PoolError, PoolModel
from oracle.kvstore import StoreModel
from paged_kv_cache_mla_amd import _lib
from paged_kv_cache_mla_amd.api import KvattnError, KVStore, Pool, ShareController

FAKE_DEV = 0x7F0000000000
FAKE_HOST = 0x7E0000000000
KIND = {"inval": _lib.E_INVAL, "exhausted": _lib.E_POOL_EXHAUSTED, "state": _lib.E_STATE}


def _pools(dev_blocks, host_blocks, seed, bs=16):
    dev = Pool(bs, 2, 64, 64, "bf16", False, [(FAKE_DEV, dev_blocks)], seed=seed)
    host = Pool(bs, 2, 64, 64, "bf16", False, [(FAKE_HOST, host_blocks)], seed=seed + 1)
    return dev, host, PoolModel(dev_blocks, seed, bs), PoolModel(host_blocks, seed + 1, bs)


def _controllers(rng, batch, with_ctl):
    lib, ora = [], []
    for b in range(batch):
        if not with_ctl[b]:
            lib.append(None)
            ora.append(None)
            continue
        A, B = rng.uniform(0.5, 3.0), rng.uniform(0.5, 3.0)
        C_cpu, C_gpu = rng.uniform(0, 400), rng.uniform(0, 400)
        lib.append(ShareController(A, B, C_cpu, C_gpu, window=8))
        ora.append(osh.Controller(A, B, C_cpu, C_gpu, 8))
    return lib, ora


def _same_views(store, model):
    for got, exp in zip(store.views(), model.views()):
        assert np.array_equal(got, exp)


def _model_invariants(model, appended, dev_total, host_total):
    gt, gl, ct, cl = model.views()
    assert np.array_equal(gl + cl, np.asarray(appended))
    dev_ids = [x for b in range(model.batch) for x in model.gpu[b] + model.win[b]]
    host_ids = [x for b in range(model.batch) for x in model.cpu[b]]
    assert sorted(dev_ids + model.dev.free) == list(range(dev_total))
    assert sorted(host_ids + model.host.free) == list(range(host_total))
    for b in range(model.batch):
        if model.ctl[b] is not None:
            assert cl[b] == model.ctl[b].c


@pytest.mark.parametrize("seed", range(6))
def test_store_matches_model_over_a_decode_run(seed):
    rng = random.Random(seed)
    batch, bs, D = rng.choice([1, 3, 5]), 16, rng.choice([32, 64, 256])
    max_blocks = 160
    dev_total, host_total = batch * max_blocks + 7, batch * max_blocks + 3
    dev, host, mdev, mhost = _pools(dev_total, host_total, 1000 + seed, bs)
    with_ctl = [rng.random() < 0.8 for _ in range(batch)]
    lctl, octl = _controllers(rng, batch, with_ctl)
    store = KVStore(dev, host, batch, D, max_blocks, lctl)
    model = StoreModel(mdev, mhost, batch, D, max_blocks, octl)
    prefill = [rng.randrange(0, 600) for _ in range(batch)]
    appended = list(prefill)
    assert store.reserve(prefill) == model.reserve(prefill)
    store.commit(prefill)
    model.commit(prefill)
    _same_views(store, model)
    changed, copies = store.place_prefill_plan()
    m_changed, m_copies = model.place_prefill()
    assert changed == m_changed and [tuple(c) for c in copies] == m_copies
    _same_views(store, model)
    _model_invariants(model, appended, dev_total, host_total)
    for step in range(1200):
        n_new = [1 if rng.random() < 0.9 else rng.randrange(0, 4) for _ in range(batch)]
        if rng.random() < 0.02:
            n_new = [rng.randrange(0, 70) for _ in range(batch)]     # a burst (chunked append)
        if max(g + n for g, n in zip(model.views()[1], n_new)) > max_blocks * bs - 2 * D:
            break
        assert store.reserve(n_new) == model.reserve(n_new)
        store.commit(n_new)
        model.commit(n_new)
        appended = [a + n for a, n in zip(appended, n_new)]
        if step % rng.choice([1, 1, 1, 5]) == 0:
            changed, copies = store.flush_plan()
            m_changed, m_copies = model.flush()
            assert changed == m_changed and [tuple(c) for c in copies] == m_copies
        _same_views(store, model)
    _model_invariants(model, appended, dev_total, host_total)
    # routed-to-GPU batches move nothing: every copy is a CPU block
    assert dev.num_free == len(mdev.free) and host.num_free == len(mhost.free)
    store.close()
    assert dev.num_free == dev_total and host.num_free == host_total


def _expect(status, fn, *args):
    with pytest.raises(KvattnError) as e:
        fn(*args)
    assert e.value.status == status


def test_store_errors_leave_state_unchanged():
    dev, host, mdev, mhost = _pools(10, 4, 7)
    lctl, octl = _controllers(random.Random(1), 2, [True, True])
    store = KVStore(dev, host, 2, 32, 8, lctl)
    model = StoreModel(mdev, mhost, 2, 32, 8, octl)
    # device exhaustion: 2 x 6 blocks > 10
    _expect(_lib.E_POOL_EXHAUSTED, store.reserve, [96, 96])
    with pytest.raises(PoolError):
        model.reserve([96, 96])
    _same_views(store, model)
    assert dev.num_free == 10
    # a GPU view beyond max_blocks
    _expect(_lib.E_INVAL, store.reserve, [8 * 16 + 1, 0])
    # commit beyond the reservation
    store.reserve([40, 40])
    model.reserve([40, 40])
    _expect(_lib.E_STATE, store.commit, [49, 1])
    store.commit([40, 40])
    model.commit([40, 40])
    _same_views(store, model)
    # flush before place_prefill: the controllers have not admitted yet
    _expect(_lib.E_STATE, store.flush_plan)
    # host pool too small for the worst case: 2 x 2 whole blocks to the CPU > 4? (= 4: fits)
    changed, copies = store.place_prefill_plan()
    m_changed, m_copies = model.place_prefill()
    assert [tuple(c) for c in copies] == m_copies
    _expect(_lib.E_STATE, store.place_prefill_plan)       # only once
    store.close()
    assert dev.num_free == 10 and host.num_free == 4


def test_host_pool_checks_exact_for_prefill_and_worst_case_for_flush():
    # no controller: the prefill needs no host block, even with a tiny host pool
    dev, host, _, _ = _pools(40, 3, 9)
    store = KVStore(dev, host, 1, 32, 40)
    store.reserve([100])
    store.commit([100])
    store.place_prefill_plan()
    assert store.views()[1][0] == 100
    # a flush of two pending batches could need 2 x 2 host blocks > 3
    store.reserve([64])
    store.commit([64])
    _expect(_lib.E_POOL_EXHAUSTED, store.flush_plan)
    assert store.views()[1][0] == 164
    # a controller that admits more than the host pool holds: refused before any change
    dev2, host2, _, _ = _pools(40, 3, 10)
    ctl = ShareController(0.0, 1.0)               # r = 1: the whole prefill to the CPU
    store2 = KVStore(dev2, host2, 1, 32, 40, [ctl])
    store2.reserve([100])
    store2.commit([100])
    _expect(_lib.E_POOL_EXHAUSTED, store2.place_prefill_plan)
    assert store2.views()[1][0] == 100 and host2.num_free == 3
    assert ctl.state()["placed_tokens"] == 0      # not admitted by the refused call


def test_store_create_validation():
    dev, host, _, _ = _pools(8, 8, 3)
    other = Pool(32, 2, 64, 64, "bf16", False, [(FAKE_HOST, 4)])
    _expect(_lib.E_INVAL, KVStore, dev, other, 1, 32, 4)      # layouts differ
    _expect(_lib.E_INVAL, KVStore, dev, host, 1, 24, 4)       # window not a block multiple
    _expect(_lib.E_INVAL, KVStore, dev, host, 0, 32, 4)
    _expect(_lib.E_INVAL, KVStore, dev, host, 1, 32, 0)
    s = KVStore(dev, host, 2, 32, 4)
    _expect(_lib.E_INVAL, s.reserve, [-1, 0])


def test_pool_freed_before_its_store_is_deferred():
    """kvattn_pool_free on a pool a store still holds defers the deletion until the store is
    freed (which still returns its blocks to that pool)."""
    dev, host, _, _ = _pools(16, 16, 21)
    store = KVStore(dev, host, 2, 32, 8)
    store.reserve([40, 7])
    store.commit([40, 7])
    dev.close()
    host.close()
    gt, gl, ct, cl = store.views()
    assert list(gl) == [40, 7]
    store.close()
