"""GPU tests of run-time pool growth over HIP virtual memory ([VAMP] §IV-C, §V-A): physical
pages move from an "expert weights" range into the KV pool's growth range and back, carrying
their contents; the pool grows over them (a new region, then an in-place resize of the last
one) and shrinks again; decodes over every region match the oracle, and a decode in flight is
not disturbed by growth."""

import ctypes
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

H2D, D2H = 1, 2


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
    torch.zeros(1, device="cuda")          # the HIP runtime is loaded and initialised


def _hip():
    from paged_kv_cache_mla_amd.session import _hip_runtime
    hip = _hip_runtime()
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    return hip


def _vmm(nbytes, chunk=0):
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import KvattnError, VMMRange
    try:
        return VMMRange(nbytes, chunk)
    except KvattnError as e:
        if e.status == _lib.E_UNSUPPORTED:
            pytest.skip("this device has no HIP virtual memory management")
        raise


def _put(hip, addr, arr):
    arr = np.ascontiguousarray(arr)
    assert hip.hipMemcpy(ctypes.c_void_p(addr), ctypes.c_void_p(arr.ctypes.data), arr.nbytes, H2D) == 0


def _get(hip, addr, nbytes):
    out = np.empty(nbytes, np.uint8)
    assert hip.hipMemcpy(ctypes.c_void_p(out.ctypes.data), ctypes.c_void_p(addr), nbytes, D2H) == 0
    return out


def test_mapped_pages_hold_data():
    hip = _hip()
    r = _vmm(8 << 20)
    g = r.granularity
    _say(f"[vmm] recommended granularity {g}")
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import KvattnError
    with pytest.raises(KvattnError) as e:
        _vmm(8 << 20, 1000)                      # not a multiple of the minimum granularity
    assert e.value.status == _lib.E_INVAL
    r.map_new(0, 2 * g)
    assert r.mapped_bytes == 2 * g
    data = np.random.default_rng(1).integers(0, 256, 2 * g, dtype=np.uint8)
    _put(hip, r.base, data)
    assert np.array_equal(_get(hip, r.base, 2 * g), data)
    r.close()


def test_move_carries_contents_and_reverses():
    hip = _hip()
    expert = _vmm(8 << 20)
    g = expert.granularity
    kv = _vmm(8 * g)
    expert.map_new(0, 4 * g)
    pattern = np.random.default_rng(2).integers(0, 256, 2 * g, dtype=np.uint8)
    _put(hip, expert.base + g, pattern)
    expert.move_to(g, kv, 0, 2 * g)
    assert expert.mapped_bytes == 2 * g and kv.mapped_bytes == 2 * g
    assert np.array_equal(_get(hip, kv.base, 2 * g), pattern)       # the pages moved
    kv.move_to(0, expert, g, 2 * g)                                 # and back
    assert np.array_equal(_get(hip, expert.base + g, 2 * g), pattern)
    assert kv.mapped_bytes == 0
    kv.close()
    expert.close()


def _bf16(rng, shape):
    from synth import bf16_round_bits
    return bf16_round_bits(rng.standard_normal(shape, dtype=np.float32))


def test_pool_grows_over_moved_pages_decodes_and_shrinks():
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import DecodeStep, Pool, append_kv
    rng = np.random.default_rng(5)
    bs, hkv, d, hq = 16, 2, 128, 8
    bb = hkv * bs * 2 * d * 2                                      # block bytes
    base_blocks = 64
    base = torch.zeros(base_blocks * bb // 2, dtype=torch.int16, device="cuda")
    pool = Pool(bs, hkv, d, d, "bf16", False, [(base.data_ptr(), base_blocks)], seed=3)
    # the remap unit ("expert group"): whole blocks and whole granules, here 2 MiB chunks
    unit = 2 << 20
    expert = _vmm(16 << 20, unit)
    assert expert.granularity == unit and unit % bb == 0
    g = unit
    per_g = g // bb
    kv = _vmm(8 * g, unit)
    expert.map_new(0, 6 * g)                                       # "expert weights"
    max_blocks = 40

    seqs = {}                                                       # name -> (table row, K, V)

    def admit(name, L):
        st, t, _ = pool.block_table([L], max_blocks)
        assert st == _lib.OK, (name, st)
        k = _bf16(rng, (L, hkv, d))
        v = _bf16(rng, (L, hkv, d))
        kd = torch.from_numpy(k.view(np.int16)[None]).cuda()
        vd = torch.from_numpy(v.view(np.int16)[None]).cuda()
        append_kv(pool, kd, vd, _lib.BF16, torch.from_numpy(t).cuda(), max_blocks,
                  torch.zeros(1, dtype=torch.int32, device="cuda"))
        seqs[name] = (t[0], k, v, L)

    def decode(names, q):
        table = np.stack([seqs[n][0] for n in names])
        lens = [seqs[n][3] for n in names]
        step = DecodeStep(pool, table, lens, [128] * len(names), hq, d)
        o, lse = step.run(torch.from_numpy(q.view(np.int16)).cuda(), _lib.BF16, 0.1)
        return o, lse

    def check(names, q, o, lse):
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        for i, n in enumerate(names):
            _, k, v, _ = seqs[n]
            o_ref, lse_ref = oracle.attend(oracle.bf16_bits_to_f64(q[i]), oracle.bf16_bits_to_f64(k),
                                           oracle.bf16_bits_to_f64(v), 0.1)
            assert np.max(np.abs(o[i] - o_ref)) / np.max(np.abs(o_ref)) <= 2e-3, n
            assert np.max(np.abs(lse[i] - lse_ref)) <= 2e-3, n

    # the base region fills up
    for i, L in enumerate([300, 500, 200]):                        # 19 + 32 + 13 = 64 blocks
        admit(f"a{i}", L)
    assert pool.num_free == 0
    st, _, short = pool.block_table([100], max_blocks)
    assert st == _lib.E_POOL_EXHAUSTED
    # growth 1: two granules of expert pages move into the KV range, a new region
    expert.move_to(0, kv, 0, 2 * g)
    first = pool.add_region(kv.base, 2 * per_g)
    assert first == base_blocks and pool.num_regions == 2
    admit("b0", min(400, 2 * per_g * bs))
    assert all(x >= base_blocks for x in seqs["b0"][0][:(-(-seqs["b0"][3] // bs))])
    # growth 2: one more granule, mapped right after, grows the region in place
    expert.move_to(2 * g, kv, 2 * g, g)
    pool.resize_last_region(3 * per_g)
    admit("c0", 250)
    names = ["a0", "a1", "a2", "b0", "c0"]
    q = _bf16(rng, (len(names), hq, d))
    o, lse = decode(names, q)
    torch.cuda.synchronize()
    _say(f"[growth] decoded {names} over {pool.num_regions} regions")
    check(names, q, o, lse)
    o_ab = o[:4].clone()
    # shrink: c0 leaves, the region returns to two granules, the third moves back
    pool.release(seqs.pop("c0")[0][None])
    pool.resize_last_region(2 * per_g)
    kv.move_to(2 * g, expert, 2 * g, g)
    assert kv.mapped_bytes == 2 * g
    o2, lse2 = decode(names[:4], q[:4])
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ab)                                   # the rest is untouched
    # growth while a decode is in flight: fresh pages, no synchronisation in between
    o3, _ = decode(names[:4], q[:4])                               # enqueued, not waited for
    kv.map_new(2 * g, g)
    pool.resize_last_region(3 * per_g)
    admit("d0", 180)
    o4, lse4 = decode(["d0"], q[:1])
    torch.cuda.synchronize()
    assert torch.equal(o3, o_ab)
    check(["d0"], q[:1], o4, lse4)
    del o, o2, o3, o4
    pool.close()
    kv.close()
    expert.close()
