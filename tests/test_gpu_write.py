"""GPU tests of the write side through the C ABI: kvattn_append_kv against the oracle's token
writer, bit for bit (a write is a pure placement, so every byte must match)."""

import sys

import numpy as np
import pytest

import oracle
from oracle import Layout, block_elems

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU (run with -m 'not gpu' on CPU-only hosts)")
    from paged_kv_cache_mla_amd import _lib
    _lib.load()
    torch.cuda.set_device(0)


LAYOUTS = {
    "gqa_bf16": Layout(16, 4, 128, 128, "bf16", False),
    "tiny_f32": Layout(16, 1, 64, 64, "f32", False),
    "mla_bf16": Layout(64, 1, 576, 512, "bf16", True),
}


def _storage(layout):
    return np.uint16 if layout.dtype == "bf16" else np.float32


def _random_storage(rng, shape, layout):
    if layout.dtype == "bf16":
        from synth import bf16_round_bits
        return bf16_round_bits(rng.standard_normal(shape, dtype=np.float32))
    return rng.standard_normal(shape, dtype=np.float32)


def _dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t, dtype):
    a = t.cpu().numpy()
    return a.view(np.uint16) if dtype == np.uint16 else a


def _setup(layout, rng, batch, max_blocks, region_blocks):
    from paged_kv_cache_mla_amd.api import Pool
    nel = block_elems(layout)
    regions = [_random_storage(rng, n * nel, layout) for n in region_blocks]
    dev = [_dev(r) for r in regions]
    pool = Pool(layout.block_size, layout.num_kv_heads, layout.head_dim_k, layout.head_dim_v,
                layout.dtype, layout.latent, [(t.data_ptr(), n) for t, n in zip(dev, region_blocks)])
    perm = rng.permutation(sum(region_blocks)).astype(np.int32)
    table = perm[:batch * max_blocks].reshape(batch, max_blocks)
    return regions, dev, pool, table


@pytest.mark.parametrize("name", sorted(LAYOUTS))
@pytest.mark.parametrize("n_new", [1, 37, 200])
def test_append_matches_oracle_writer(name, n_new):
    """One token per sequence takes the per-token kernel; 37 and 200 the tile kernel (tiles of
    16 tokens for these GQA layouts, 32 for MLA); every byte must match the oracle's writer."""
    from paged_kv_cache_mla_amd.api import append_kv
    layout = LAYOUTS[name]
    _say(f"[append] {name} n_new={n_new}")
    rng = np.random.default_rng(100 * sorted(LAYOUTS).index(name) + n_new)
    batch = 5
    max_blocks = max(6, -(-(n_new + layout.block_size) // layout.block_size) + 1)
    region_blocks = [13, batch * max_blocks + 4 - 13]
    regions, dev, pool, table = _setup(layout, rng, batch, max_blocks, region_blocks)
    cap = max_blocks * layout.block_size
    pos = rng.integers(0, cap - n_new + 1, batch).astype(np.int32)
    pos[0] = cap - n_new                      # ends exactly at the last slot
    pos[1] = layout.block_size - 1            # starts one slot before a block boundary
    hkv = 1 if layout.latent else layout.num_kv_heads
    k = _random_storage(rng, (batch, n_new, hkv, layout.head_dim_k), layout)
    v = None if layout.latent else _random_storage(rng, (batch, n_new, hkv, layout.head_dim_v), layout)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    append_kv(pool, _dev(k), None if v is None else _dev(v), oracle_dtype(layout),
              _dev(table), max_blocks, _dev(pos), err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for b in range(batch):
        kb = k[b, :, 0, :] if layout.latent else k[b]
        oracle.write_tokens(layout, regions, region_blocks, table[b], int(pos[b]), kb,
                            None if v is None else v[b])
    for r, t in zip(regions, dev):
        assert np.array_equal(_host(t, _storage(layout)), r)


def oracle_dtype(layout):
    from paged_kv_cache_mla_amd import _lib
    return _lib.BF16 if layout.dtype == "bf16" else _lib.F32


@pytest.mark.parametrize("n_new", [4, 40])
def test_append_flags_absent_and_out_of_range_tokens_and_writes_the_rest(n_new):
    """Both kernels (4 tokens: per token; 40: tiles) flag and skip exactly the tokens whose
    index is negative or past the table, or whose block entry is not a valid id."""
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import append_kv
    layout = LAYOUTS["gqa_bf16"]
    rng = np.random.default_rng(3)
    bs = layout.block_size
    batch, max_blocks = 4, 8
    region_blocks = [batch * max_blocks]
    regions, dev, pool, table = _setup(layout, rng, batch, max_blocks, region_blocks)
    table = table.copy()
    table[1, 2] = -1                                   # ABSENT inside sequence 1's range
    pos = np.array([5, 2 * bs - 2, max_blocks * bs - 2,  # seq 2 runs past the table
                    -3], np.int32)                       # seq 3 starts before token 0
    k = _random_storage(rng, (batch, n_new, 4, 128), layout)
    v = _random_storage(rng, (batch, n_new, 4, 128), layout)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    append_kv(pool, _dev(k), _dev(v), _lib.BF16, _dev(table), max_blocks, _dev(pos), err)
    torch.cuda.synchronize()
    assert int(err.item()) == _lib.ERR_BAD_BLOCK | _lib.ERR_BAD_SEQ
    # expected: every token with an index in the table and a valid block is written
    for b in range(batch):
        for j in range(n_new):
            t = int(pos[b]) + j
            if t < 0 or t // bs >= max_blocks or table[b, t // bs] < 0:
                continue
            oracle.write_tokens(layout, regions, region_blocks, table[b], t, k[b, j:j + 1],
                                v[b, j:j + 1])
    assert np.array_equal(_host(dev[0], np.uint16), regions[0])


# ---------------------------------------------------------------- a decode session
SESSIONS = {
    # layout, hq, window D, prefill lengths, decode steps, check every
    "gqa": (Layout(16, 2, 128, 128, "bf16", False), 8, 64, [100, 37, 0], 300, 60),
    "mla": (Layout(64, 1, 576, 512, "bf16", True), 16, 128, [300, 64, 5], 300, 100),
}


@pytest.mark.parametrize("name", sorted(SESSIONS))
def test_decode_session_with_window_eviction_and_both_views(name):
    """Prefill and decode tokens are appended into the staging window; D-token batches are
    evicted to the GPU share or, copied to pinned host blocks, to the CPU share, as each
    sequence's share controller routes them.  At checkpoints the GPU view is decoded on the
    device and the CPU view on the host, and the merge matches the oracle's attention over
    every token appended so far; the two views hold exactly the appended tokens."""
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import (DecodeStep, KVStore, Pool, ShareController,
                                            append_kv, host_partial)
    layout, hq, D, prefill, steps, every = SESSIONS[name]
    _say(f"[session] {name}")
    rng = np.random.default_rng(77)
    B, bs = len(prefill), layout.block_size
    hkv = 1 if layout.latent else layout.num_kv_heads
    max_blocks = -(-(max(prefill) + steps) // bs) + D // bs + 2
    nel = block_elems(layout)
    dev_blocks, host_blocks = B * max_blocks + 3, B * max_blocks + 2
    dev_region = torch.zeros(dev_blocks * nel, dtype=torch.int16, device="cuda")
    host_region = torch.zeros(host_blocks * nel, dtype=torch.int16, pin_memory=True)
    args = (bs, layout.num_kv_heads, layout.head_dim_k, layout.head_dim_v, "bf16", layout.latent)
    dev_pool = Pool(*args, [(dev_region.data_ptr(), dev_blocks)], seed=5)
    host_pool = Pool(*args, [(host_region.data_ptr(), host_blocks)], seed=6)
    ctls = [ShareController(2.0, 1.0, 0.0, 0.0, window=4) for _ in range(B)]   # p = 1/3
    store = KVStore(dev_pool, host_pool, B, D, max_blocks, ctls)
    hist_k = [np.zeros((0, hkv, layout.head_dim_k), np.uint16) for _ in range(B)]
    hist_v = [np.zeros((0, hkv, layout.head_dim_v), np.uint16) for _ in range(B)]

    def tokens(n):
        k = _random_storage(rng, (n, hkv, layout.head_dim_k), layout)
        v = k[:, :, :layout.head_dim_v].copy() if layout.latent else \
            _random_storage(rng, (n, hkv, layout.head_dim_v), layout)
        return k, v

    def upload_views():
        gt, gl, ct, cl = store.views()
        return _dev(gt), gl, ct, cl

    def append(b_list, ks, vs, n, table_dev, gl):
        for b, k, v in zip(b_list, ks, vs):
            if n == 0:
                continue
            kd = _dev(k[None, :, 0, :] if layout.latent else k[None])
            vd = None if layout.latent else _dev(v[None])
            pos = torch.tensor([int(gl[b])], dtype=torch.int32, device="cuda")
            append_kv(dev_pool, kd, vd, _lib.BF16, table_dev[b:b + 1], max_blocks, pos, err)
            hist_k[b] = np.concatenate([hist_k[b], k])
            hist_v[b] = np.concatenate([hist_v[b], v])

    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # prefill: ragged lengths, one append per sequence, then placement
    store.reserve(prefill)
    table_dev, gl, ct, cl = upload_views()
    for b in range(B):
        k, v = tokens(prefill[b])
        append([b], [k], [v], prefill[b], table_dev, gl)
    store.commit(prefill)
    store.place_prefill()
    table_dev, gl, ct, cl = upload_views()
    cpu_batches = 0
    for step in range(1, steps + 1):
        if store.reserve(1):
            table_dev, gl, ct, cl = upload_views()
        kv = [tokens(1) for _ in range(B)]
        append(range(B), [k for k, _ in kv], [v for _, v in kv], 1, table_dev, gl)
        store.commit(1)
        if store.flush():
            cpu_batches += 1
        table_dev, gl, ct, cl = upload_views()
        if step % every and step != steps:
            continue
        torch.cuda.synchronize()        # appends and copies to host blocks done
        assert int(err.item()) == 0
        assert np.array_equal(gl + cl, [len(h) for h in hist_k])
        # the two views hold exactly the appended tokens (as a multiset of K rows)
        dev_np = dev_region.cpu().numpy().view(np.uint16)
        host_np = host_region.numpy().view(np.uint16)
        gt_host = table_dev.cpu().numpy()
        for b in range(B):
            kg, _ = oracle.gather_sequence(layout, [dev_np], [dev_blocks], gt_host[b], 0, int(gl[b]))
            kc, _ = oracle.gather_sequence(layout, [host_np], [host_blocks], ct[b], 0, int(cl[b]))
            got = np.concatenate([kg, kc]).reshape(len(hist_k[b]), -1)
            exp = oracle.bf16_bits_to_f64(hist_k[b]).reshape(len(hist_k[b]), -1)
            assert np.array_equal(got[np.lexsort(got.T[::-1])], exp[np.lexsort(exp.T[::-1])])
        # attention: GPU view on the device, CPU view on the host, merged on the device
        q = _random_storage(rng, (B, hq, layout.head_dim_k), layout)
        scale = 1.0 / np.sqrt(192.0 if layout.latent else layout.head_dim_k)
        ds = DecodeStep(dev_pool, gt_host, gl, [bs * 4] * B, hq, layout.head_dim_v,
                        group_parts=1)
        o_h, l_h = host_partial(bs, layout.num_kv_heads, layout.head_dim_k, layout.head_dim_v,
                                "bf16", layout.latent, [host_np], q, hq, scale, ct, cl,
                                n_threads=4)
        o, lse = ds.run(_dev(q), _lib.BF16, scale, torch.from_numpy(o_h).cuda(),
                        torch.from_numpy(l_h).cuda())
        torch.cuda.synchronize()
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        qf = oracle.bf16_bits_to_f64(q)
        for b in range(B):
            k64 = oracle.bf16_bits_to_f64(hist_k[b])
            v64 = oracle.bf16_bits_to_f64(hist_v[b])
            o_ref, lse_ref = oracle.attend(qf[b], k64, v64, scale)
            err_o = np.max(np.abs(o[b] - o_ref)) / np.max(np.abs(o_ref))
            assert err_o <= 2e-3, (step, b, err_o)
            assert np.max(np.abs(lse[b] - lse_ref)) <= 2e-3
        _say(f"[session] {name} step {step}: GPU view {list(gl)}, CPU view {list(cl)}")
    assert sum(cl) > 0 and cpu_batches > 0     # the CPU side was exercised
    store.close()


def test_flush_into_a_host_region_added_after_the_first_flush():
    """Every batch goes to the CPU share (p ~ 1).  The first flush fills the host pool's only
    region; a second pinned region is then added to the host pool, and the next flush must copy
    into it through the region's own device-mapped address.  The CPU view then holds exactly
    the appended tokens, in order."""
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import KVStore, Pool, ShareController, append_kv
    layout = Layout(16, 2, 64, 64, "bf16", False)
    rng = np.random.default_rng(91)
    B, bs, D, max_blocks = 2, 16, 32, 8
    nb = D // bs
    nel = block_elems(layout)
    dev_region = torch.zeros(B * max_blocks * nel, dtype=torch.int16, device="cuda")
    host_a = torch.zeros(B * nb * nel, dtype=torch.int16, pin_memory=True)   # one flush's room
    host_b = torch.zeros(B * nb * nel, dtype=torch.int16, pin_memory=True)
    args = (bs, 2, 64, 64, "bf16", False)
    dev_pool = Pool(*args, [(dev_region.data_ptr(), B * max_blocks)], seed=3)
    host_pool = Pool(*args, [(host_a.data_ptr(), B * nb)], seed=4)
    ctls = [ShareController(1e-6, 1.0, 0.0, 0.0, window=4) for _ in range(B)]
    store = KVStore(dev_pool, host_pool, B, D, max_blocks, ctls)
    store.place_prefill()                       # admits the controllers; nothing to place
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hist = [[] for _ in range(B)]

    def append_batch():
        store.reserve([D] * B)
        gt, gl, _, _ = store.views()
        table = _dev(gt)
        for b in range(B):
            k = _random_storage(rng, (D, 2, 64), layout)
            v = _random_storage(rng, (D, 2, 64), layout)
            pos = torch.tensor([int(gl[b])], dtype=torch.int32, device="cuda")
            append_kv(dev_pool, _dev(k[None]), _dev(v[None]), _lib.BF16, table[b:b + 1],
                      max_blocks, pos, err)
            hist[b].append((k, v))
        store.commit([D] * B)

    append_batch()
    store.flush()
    torch.cuda.synchronize()
    assert host_pool.num_free == 0
    first = host_pool.add_region(host_b.data_ptr(), B * nb)
    _say(f"[kvstore] host region added at id {first}")
    append_batch()
    store.flush()
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    _, gl, ct, cl = store.views()
    regions = [host_a.numpy().view(np.uint16), host_b.numpy().view(np.uint16)]
    for b in range(B):
        assert cl[b] == 2 * D and gl[b] == 0
        assert all(x >= first for x in ct[b, nb:2 * nb])     # the second batch is in the new region
        k, v = oracle.gather_sequence(layout, regions, [B * nb, B * nb], ct[b], 0, 2 * D)
        k_ref = np.concatenate([oracle.bf16_bits_to_f64(x[0]) for x in hist[b]])
        v_ref = np.concatenate([oracle.bf16_bits_to_f64(x[1]) for x in hist[b]])
        assert np.array_equal(k, k_ref) and np.array_equal(v, v_ref)
    store.close()
    host_pool.close()
    dev_pool.close()


def test_full_size_append_rebuilds_the_pool_byte_for_byte():
    """The 16 x 32K layer: every token of every sequence is read back out of the workload's
    pool, the device pool is cleared, and the tokens are appended again through the same
    tables (the tile kernel, one call per sequence).  The 1 GiB pool must come back byte for
    byte, and a decode of it must match the oracle on sampled sequences."""
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import append_kv
    from paged_kv_cache_mla_amd.session import DeviceCase
    from synth import bf16_round_bits, make_case
    from tests import oracle_cases as oc
    _say("[append-full] generating gqa_32k full")
    case = make_case("gqa_32k", "full")
    dc = DeviceCase(case)
    lay = oc.layout_of(case)
    for t in dc.regions:
        t.zero_()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b in range(case.batch):
        L = int(case.ctx_lens[b])
        k, v = oracle.gather_sequence(lay, case.regions, case.region_blocks, case.table[b], 0, L)
        kb = bf16_round_bits(k.astype(np.float32))      # exact: the values are bf16
        vb = bf16_round_bits(v.astype(np.float32))
        append_kv(dc.pool, _dev(kb[None]), _dev(vb[None]), _lib.BF16, dc.step.table_dev[b:b + 1],
                  case.max_blocks, pos, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for r, t in zip(case.regions, dc.regions):
        assert np.array_equal(_host(t, np.uint16), r)
    _say("[append-full] pool rebuilt byte for byte; decoding")
    o, lse = dc.run()
    torch.cuda.synchronize()
    seqs = [0, 11]
    o_ref, lse_ref = oc.full_reference(case, seqs)
    o = o.cpu().numpy()
    assert oc.out_error(case, o[seqs], o_ref[seqs]) <= oc.out_tol(case)
