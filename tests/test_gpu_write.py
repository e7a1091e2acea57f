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
@pytest.mark.parametrize("n_new", [1, 37])
def test_append_matches_oracle_writer(name, n_new):
    from paged_kv_cache_mla_amd.api import append_kv
    layout = LAYOUTS[name]
    _say(f"[append] {name} n_new={n_new}")
    rng = np.random.default_rng(100 * sorted(LAYOUTS).index(name) + n_new)
    batch, max_blocks = 5, 6
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


def test_append_flags_absent_and_out_of_range_tokens_and_writes_the_rest():
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import append_kv
    layout = LAYOUTS["gqa_bf16"]
    rng = np.random.default_rng(3)
    batch, max_blocks = 3, 4
    region_blocks = [batch * max_blocks]
    regions, dev, pool, table = _setup(layout, rng, batch, max_blocks, region_blocks)
    table = table.copy()
    table[1, 2] = -1                                   # ABSENT inside sequence 1's range
    bs = layout.block_size
    n_new = 4
    pos = np.array([5, 2 * bs - 2, max_blocks * bs - 2], np.int32)  # seq 2 runs past the table
    k = _random_storage(rng, (batch, n_new, 4, 128), layout)
    v = _random_storage(rng, (batch, n_new, 4, 128), layout)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    append_kv(pool, _dev(k), _dev(v), _lib.BF16, _dev(table), max_blocks, _dev(pos), err)
    torch.cuda.synchronize()
    assert int(err.item()) == _lib.ERR_BAD_BLOCK | _lib.ERR_BAD_SEQ
    # expected: every token whose block is valid is written, the others are not
    for b in range(batch):
        for j in range(n_new):
            t = int(pos[b]) + j
            if t // bs >= max_blocks or table[b, t // bs] < 0:
                continue
            oracle.write_tokens(layout, regions, region_blocks, table[b], t, k[b, j:j + 1],
                                v[b, j:j + 1])
    assert np.array_equal(_host(dev[0], np.uint16), regions[0])
