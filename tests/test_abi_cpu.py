"""CPU tests of the C ABI: symbols, pool bookkeeping vs the oracle's model, validation.

No call here reaches a kernel: the pool is host-only, and every decode / merge call below
fails validation before anything is enqueued (fake device addresses are never touched).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from oracle.alloc import PoolError, PoolModel
from oracle.layout import Layout as OLayout, block_elems
from paged_kv_cache_mla_amd import _lib
from paged_kv_cache_mla_amd.api import Pool, block_bytes, partition_count

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kvattn.h")
FAKE = 0x7F0000000000  # 16-byte aligned fake device address (never dereferenced)
KIND = {"inval": _lib.E_INVAL, "exhausted": _lib.E_POOL_EXHAUSTED, "range": _lib.E_RANGE,
        "state": _lib.E_STATE}


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return sorted(set(re.findall(r"\b(kvattn_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert names == sorted(_lib._SIGNATURES)        # the binding covers exactly the header
    for name in names:
        assert hasattr(lib, name), name
    assert lib.kvattn_version().decode().startswith("kvattn")
    assert lib.kvattn_last_error() is not None


def _pool(total_or_regions, seed, bs=16, hkv=2, d=64, dtype="bf16", latent=False):
    regions = total_or_regions if isinstance(total_or_regions, list) else [total_or_regions]
    addrs = []
    base = FAKE
    for n in regions:
        addrs.append((base, n))
        base += 0x100000000
    return Pool(bs, hkv, d, d, dtype, latent, addrs, seed=seed)


def _model_call(model, fn, *args, **kw):
    try:
        return _lib.OK, getattr(model, fn)(*args, **kw), 0
    except PoolError as e:
        return KIND[e.kind], None, e.shortfall


@pytest.mark.parametrize("seed", [0, 1, 12345, 2 ** 63 + 5])
def test_initial_free_order_matches_oracle_shuffle(seed):
    pool = _pool([37, 64], seed, bs=4)
    model = PoolModel(101, seed, 4)
    st, table, _ = pool.block_table([4 * 101], max_blocks=101)
    assert st == _lib.OK
    assert table[0].tolist() == oracle.alloc.shuffled_ids(101, seed)
    assert table[0].tolist() == model.alloc([4 * 101], 101)[0].tolist()
    assert pool.num_free == 0


def test_pool_matches_model_over_random_operations():
    rng = np.random.default_rng(7)
    for trial in range(12):
        bs = int(rng.choice([1, 4, 16, 64]))
        total = int(rng.integers(1, 400))
        seed = int(rng.integers(0, 2 ** 63))
        split = int(rng.integers(0, total + 1))
        pool = _pool([split, total - split] if split not in (0, total) else [total], seed, bs=bs)
        model = PoolModel(total, seed, bs)
        live = []
        for step in range(40):
            op = rng.random()
            if op < 0.55 or not live:
                bsz = int(rng.integers(1, 6))
                mb = int(rng.integers(1, 12))
                ctx = rng.integers(0, mb * bs + 1, size=bsz)
                if rng.random() < 0.1:
                    ctx[0] = mb * bs + 1                       # too long -> E_INVAL
                first = None
                share_src = share_n = None
                if rng.random() < 0.3:
                    first = [int(rng.integers(0, c + 1)) for c in ctx]
                elif rng.random() < 0.5 and bsz > 1:
                    share_src = [-1] + [int(rng.integers(-1, b)) for b in range(1, bsz)]
                    share_n = [int(rng.integers(0, mb + 1)) for _ in range(bsz)]
                st, table, short = pool.block_table(ctx, mb, first, share_src, share_n)
                mst, mtable, mshort = _model_call(model, "alloc", ctx, mb, first, share_src, share_n)
                assert st == mst, (trial, step, _lib.load().kvattn_last_error())
                if st == _lib.OK:
                    assert np.array_equal(table, mtable)
                    live.append((ctx, table))
                elif st == _lib.E_POOL_EXHAUSTED:
                    assert short == mshort
            elif op < 0.85:
                ctx, table = live.pop(int(rng.integers(0, len(live))))
                assert pool.release(table) == _lib.OK
                model.release(table)
                if rng.random() < 0.3:                          # double release
                    assert pool.release(table) == _lib.E_STATE or not (table >= 0).any()
            else:
                # explicit claim of some currently free ids (plus maybe a used one)
                free_now = list(model.free)
                if not free_now:
                    continue
                k = int(rng.integers(1, min(len(free_now), 6) + 1))
                ids = rng.choice(free_now, size=k, replace=False)
                tab = np.full((2, k), -1, np.int32)
                tab[0] = ids
                tab[1, : k // 2] = ids[: k // 2]                    # shared references
                if rng.random() < 0.3 and live:
                    tab[0, 0] = live[0][1].reshape(-1)[live[0][1].reshape(-1) >= 0][0] \
                        if (live[0][1] >= 0).any() else tab[0, 0]
                ctx = [k * bs, (k // 2) * bs]
                st, table, _ = pool.block_table(ctx, k, explicit=tab)
                mst, mtab, _ = _model_call(model, "claim_explicit", ctx, tab)
                assert st == mst
                if st == _lib.OK:
                    live.append((np.array(ctx), tab))
            assert pool.num_free == len(model.free)
            for pid in range(total):
                assert pool.refcount(pid) == model.ref[pid]
            assert pool.shared_blocks == sum(1 for r in model.ref if r >= 2)


def test_exhaustion_is_all_or_nothing_and_reports_shortfall():
    pool = _pool(10, 3, bs=16)
    st, t1, _ = pool.block_table([16 * 6], max_blocks=8)
    assert st == _lib.OK and pool.num_free == 4
    st, t2, short = pool.block_table([16 * 3, 16 * 3], max_blocks=8)
    assert st == _lib.E_POOL_EXHAUSTED and short == 2 and pool.num_free == 4
    assert (t2 == -7).all()                                    # output untouched
    assert pool.release(t1) == _lib.OK and pool.num_free == 10


def test_explicit_table_errors():
    pool = _pool(8, 0, bs=16)
    st, _, _ = pool.block_table([32], 2, explicit=[[0, 8]])
    assert st == _lib.E_RANGE
    st, _, _ = pool.block_table([16], 2, explicit=[[0, 1]])       # entry past the end
    assert st == _lib.E_INVAL
    st, _, _ = pool.block_table([32, 16], 2, explicit=[[0, 1], [1, -1]])
    assert st == _lib.OK and pool.refcount(1) == 2 and pool.refcount(0) == 1
    st, _, _ = pool.block_table([16], 1, explicit=[[1]])
    assert st == _lib.E_STATE
    assert pool.release([[1, 1, 1]]) == _lib.E_STATE              # 3 drops, 2 refs
    assert pool.release([[9]]) == _lib.E_RANGE
    assert pool.release([[0, 1], [1, -1]]) == _lib.OK and pool.num_free == 8


def test_pool_alloc_validation(lib):
    lay = _lib.Layout(16, 2, 64, 64, _lib.BF16, 0)
    out = ctypes.c_void_p()
    regs = (_lib.Region * 2)()
    regs[0].base, regs[0].num_blocks = FAKE, 4
    regs[1].base, regs[1].num_blocks = FAKE + 8, 4                  # misaligned
    assert lib.kvattn_pool_alloc(ctypes.byref(lay), regs, 2, 0, ctypes.byref(out)) == _lib.E_INVAL
    regs[1].base = None
    assert lib.kvattn_pool_alloc(ctypes.byref(lay), regs, 2, 0, ctypes.byref(out)) == _lib.E_INVAL
    assert lib.kvattn_pool_alloc(ctypes.byref(lay), regs, 9, 0, ctypes.byref(out)) == _lib.E_INVAL
    for bad in [_lib.Layout(12, 2, 64, 64, _lib.BF16, 0), _lib.Layout(16, 0, 64, 64, _lib.BF16, 0),
                _lib.Layout(16, 2, 60, 64, _lib.BF16, 0), _lib.Layout(16, 2, 64, 64, 7, 0),
                _lib.Layout(16, 2, 576, 512, _lib.BF16, 1), _lib.Layout(16, 1, 512, 576, _lib.BF16, 1)]:
        assert lib.kvattn_block_bytes(ctypes.byref(bad)) == -1
        assert lib.kvattn_pool_alloc(ctypes.byref(bad), regs, 1, 0, ctypes.byref(out)) == _lib.E_INVAL


@pytest.mark.parametrize("shape", [(16, 4, 128, 128, "bf16", False), (16, 1, 64, 64, "f32", False),
                                   (64, 1, 576, 512, "bf16", True), (16, 2, 256, 256, "bf16", False)])
def test_block_bytes_match_oracle_layout(shape):
    bs, hkv, dk, dv, dt, lat = shape
    lay = OLayout(bs, hkv, dk, dv, dt, lat)
    assert block_bytes(bs, hkv, dk, dv, dt, lat) == block_elems(lay) * lay.elem_bytes


def test_partition_count_matches_oracle():
    for L in range(0, 300, 7):
        for beg in range(0, L + 2, 11):
            for P in (-1, 0, 1, 16, 48, 512):
                assert partition_count(L, beg, P) == oracle.partition_count(L, beg, P)


def _decode_call(lib, pool, **over):
    args = dict(q=FAKE, q_dtype=_lib.BF16, batch=2, hq=8, scale=0.1, table=FAKE, max_blocks=4,
                ctx=[64, 50], beg=None, part=[32, 32], seq=FAKE, max_parts=2, o=FAKE, lse=FAKE,
                nparts=FAKE, err=None, group_parts=1)
    args.update(over)
    arr = lambda v: None if v is None else np.ascontiguousarray(np.asarray(v, np.int32))  # noqa: E731
    ctx, beg, part = arr(args["ctx"]), arr(args["beg"]), arr(args["part"])
    p32 = lambda a: None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
    vp = lambda v: None if v is None else ctypes.c_void_p(v)  # noqa: E731
    return lib.kvattn_decode_partial(pool.handle, vp(args["q"]), args["q_dtype"], args["batch"],
                                     args["hq"], ctypes.c_float(args["scale"]), vp(args["table"]),
                                     args["max_blocks"], p32(ctx), p32(beg), p32(part),
                                     vp(args["seq"]), args["max_parts"], args["group_parts"],
                                     vp(args["o"]), vp(args["lse"]), vp(args["nparts"]),
                                     vp(args["err"]), None)


def test_decode_partial_validation_without_gpu(lib):
    pool = _pool(8, 0, bs=16, hkv=2, d=64)
    assert _decode_call(lib, pool, q=None) == _lib.E_INVAL
    assert _decode_call(lib, pool, q=FAKE + 4) == _lib.E_INVAL             # misaligned q
    assert _decode_call(lib, pool, q_dtype=_lib.F32) == _lib.E_UNSUPPORTED
    assert _decode_call(lib, pool, hq=7) == _lib.E_INVAL                    # not a multiple of Hkv
    assert _decode_call(lib, pool, hq=34) == _lib.E_UNSUPPORTED             # group 17 > 16
    assert _decode_call(lib, pool, part=[32, 24]) == _lib.E_INVAL           # not a block multiple
    assert _decode_call(lib, pool, part=[32, 0]) == _lib.E_INVAL
    assert _decode_call(lib, pool, ctx=[65, 50]) == _lib.E_INVAL            # > max_blocks * bs
    assert _decode_call(lib, pool, beg=[0, 51]) == _lib.E_INVAL             # begin past the end
    assert _decode_call(lib, pool, beg=[-1, 0]) == _lib.E_INVAL
    assert _decode_call(lib, pool, max_parts=1) == _lib.E_INVAL             # 2 partitions needed
    assert _decode_call(lib, pool, scale=float("nan")) == _lib.E_INVAL
    assert _decode_call(lib, pool, batch=0) == _lib.E_INVAL
    assert _decode_call(lib, pool, group_parts=-1) == _lib.E_INVAL
    assert _decode_call(lib, pool, group_parts=17) == _lib.E_INVAL          # > KVATTN_MAX_GROUP_PARTS
    p128 = _pool(8, 0, bs=16, hkv=2, d=128)
    assert _decode_call(lib, p128, group_parts=9) == _lib.E_UNSUPPORTED     # > 8 waves at d 128
    p256 = _pool(8, 0, bs=16, hkv=2, d=256)
    assert _decode_call(lib, p256, hq=32, group_parts=8) == _lib.E_UNSUPPORTED  # LDS > 64 KiB
    assert "64 KiB" in lib.kvattn_last_error().decode()
    pool3 = _pool(8, 0, bs=16, hkv=2, d=96)
    assert _decode_call(lib, pool3) == _lib.E_UNSUPPORTED                   # d 96 has no kernel
    mla = _pool(8, 0, bs=32, hkv=1, d=576, latent=False)
    assert mla.handle
    mla_bad = Pool(32, 1, 576, 512, "bf16", True, [(FAKE, 4)])
    assert _decode_call(lib, mla_bad, hq=16) == _lib.E_UNSUPPORTED          # latent needs bs 64
    assert "block" in lib.kvattn_last_error().decode()


def test_gather_probe_validation_without_gpu(lib):
    """kvattn_gather_probe validates like kvattn_decode_partial, and serves only the
    matrix-core GQA layout with 16-token blocks and the MLA layout."""
    vp = ctypes.c_void_p
    p32 = lambda v: np.ascontiguousarray(np.asarray(v, np.int32)).ctypes.data_as(  # noqa: E731
        ctypes.POINTER(ctypes.c_int32))

    def call(pool, xsum=FAKE, part=(32, 32), ctx=(64, 50), hq=8, g=1):
        return lib.kvattn_gather_probe(pool.handle, 2, hq, vp(FAKE), 4, p32(ctx), None,
                                       p32(part), vp(FAKE), g, None if xsum is None else vp(xsum),
                                       None, None)
    ok = _pool(8, 0, bs=16, hkv=2, d=128)
    assert call(ok, xsum=None) == _lib.E_INVAL
    assert call(ok, part=(32, 24)) == _lib.E_INVAL                          # not a block multiple
    assert call(ok, hq=7) == _lib.E_INVAL
    assert call(ok, g=-1) == _lib.E_INVAL
    assert call(_pool(8, 0, bs=16, hkv=2, d=128, dtype="f32")) == _lib.E_UNSUPPORTED
    assert call(_pool(8, 0, bs=32, hkv=2, d=128), ctx=(64, 50)) == _lib.E_UNSUPPORTED
    assert "block size 16" in lib.kvattn_last_error().decode()


def test_merge_validation_without_gpu(lib):
    vp = ctypes.c_void_p
    ok = dict(o=vp(FAKE), l=vp(FAKE), n=vp(FAKE), b=2, h=4, mp=3, dv=128, ox=None, lx=None,
              out=vp(FAKE), lout=None)

    def call(**over):
        a = dict(ok)
        a.update(over)
        return lib.kvattn_merge_lse(a["o"], a["l"], a["n"], a["b"], a["h"], a["mp"], a["dv"],
                                    a["ox"], a["lx"], a["out"], a["lout"], None)
    assert call(o=None) == _lib.E_INVAL
    assert call(ox=vp(FAKE)) == _lib.E_INVAL                                # lse_ext missing
    assert call(dv=130) == _lib.E_UNSUPPORTED
    assert call(dv=2048) == _lib.E_UNSUPPORTED
    assert call(mp=0) == _lib.E_INVAL
    assert call(out=vp(FAKE + 8)) == _lib.E_INVAL


def test_partition_count_edge_values(lib):
    assert lib.kvattn_partition_count(0, 0, 16) == 0
    assert lib.kvattn_partition_count(1, 0, 16) == 1
    assert lib.kvattn_partition_count(2 ** 31 - 1, 0, 1) == 2 ** 31 - 1
    assert lib.kvattn_partition_count(10, 11, 16) == -1


def test_append_validation_without_gpu(lib):
    vp = ctypes.c_void_p
    gqa = _pool(8, 0, bs=16, hkv=2, d=64)
    mla = Pool(64, 1, 576, 512, "bf16", True, [(FAKE, 4)])

    def call(pool, **over):
        a = dict(k=vp(FAKE), v=vp(FAKE), dt=_lib.BF16, b=2, n=1, t=vp(FAKE), mb=4, pos=vp(FAKE))
        a.update(over)
        return lib.kvattn_append_kv(pool.handle, a["k"], a["v"], a["dt"], a["b"], a["n"], a["t"],
                                    a["mb"], a["pos"], None, None)
    assert call(gqa, k=None) == _lib.E_INVAL
    assert call(gqa, v=None) == _lib.E_INVAL                  # V required for a GQA cache
    assert call(mla) == _lib.E_INVAL                          # no V for a latent cache
    assert call(gqa, dt=_lib.F32) == _lib.E_UNSUPPORTED
    assert call(gqa, k=vp(FAKE + 8)) == _lib.E_INVAL          # K must be 16-byte aligned
    assert call(gqa, v=vp(FAKE + 1)) == _lib.E_INVAL          # V element-aligned
    assert call(gqa, n=0) == _lib.E_INVAL
    assert call(gqa, b=0) == _lib.E_INVAL
    assert call(gqa, b=65536, n=65536) == _lib.E_INVAL        # 2^32 tokens in one launch
    assert call(gqa, t=None) == _lib.E_INVAL


def test_select_blocks_validation_without_gpu(lib):
    vp = ctypes.c_void_p

    def call(**over):
        a = dict(t=vp(FAKE), mb=64, c=vp(FAKE), bs=16, s=vp(FAKE), b=2, k=8, st=vp(FAKE), ms=8,
                 sl=vp(FAKE))
        a.update(over)
        return lib.kvattn_select_blocks(a["t"], a["mb"], a["c"], a["bs"], a["s"], a["b"], a["k"],
                                        a["st"], a["ms"], a["sl"], None, None)
    assert call(t=None) == _lib.E_INVAL
    assert call(sl=None) == _lib.E_INVAL
    assert call(k=0) == _lib.E_INVAL
    assert call(ms=7) == _lib.E_INVAL                         # sub-table narrower than k
    assert call(mb=65537) == _lib.E_INVAL                     # bitmap beyond its LDS budget
    assert call(mb=0) == _lib.E_INVAL
    assert call(bs=24) == _lib.E_INVAL
    assert call(bs=512) == _lib.E_INVAL
    assert call(b=0) == _lib.E_INVAL


# ---------------------------------------------------------------- the library's group_parts
def _choose(pool, hq, lens, part, beg=None, cus=256):
    from paged_kv_cache_mla_amd.api import choose_group_parts
    return choose_group_parts(pool, hq, lens, beg, [part] * len(lens), cus)


def test_choose_group_parts_reproduces_the_measured_sweeps():
    """group_parts = 0 picks, for 256 CUs, the best (or within 3% of the best) entry of every
    row of the decode-step sweeps measured on MI355X."""
    gqa = _pool(1, 0, bs=16, hkv=4, d=128)            # Qwen3-30B-A3B layer: 32 q / 4 KV heads
    for b, L, want in [(1, 32768, 1), (4, 32768, 1), (8, 32768, 8), (16, 8192, 1),
                       (16, 32768, 16), (4, 131072, 16), (64, 8192, 16)]:
        assert _choose(gqa, 32, [L] * b, 512) == want, (b, L)
    mix = _pool(1, 0, bs=16, hkv=8, d=128)            # Mixtral split layer, 1024-token partitions
    for r, want in [(0.25, 4), (0.5, 8), (0.75, 1)]:
        beg = int(r * 131072)
        assert _choose(mix, 32, [131072] * 4, 1024, [beg] * 4) == want, r
    mla = Pool(64, 1, 576, 512, "bf16", True, [(FAKE, 1)])
    for b, L, want in [(1, 65536, 1), (8, 16384, 1), (16, 16384, 2), (32, 16384, 4),
                       (64, 4096, 2), (64, 16384, 8), (128, 2048, 2)]:
        assert _choose(mla, 16, [L] * b, 512) == want, (b, L)
    f32 = _pool(1, 0, bs=16, hkv=4, d=128, dtype="f32")
    assert _choose(f32, 32, [8192] * 16, 512) == 2
    assert _choose(_pool(1, 0, bs=16, hkv=1, d=64, dtype="f32"), 4, [100, 257], 64) == 1


def test_choose_group_parts_respects_kernel_limits_and_shared_pools():
    d256 = _pool(200, 0, bs=16, hkv=2, d=256)          # 16 q / 2 KV heads, head dim 256
    lens = [16 * int(x) for x in np.random.default_rng(1).integers(512, 4097, 64)]
    g = _choose(d256, 16, lens, 512)
    assert g in (2, 4, 8)                               # 16 would need more than 64 KiB of LDS
    st, table, _ = d256.block_table([64, 64], 4, share_src=[-1, 0], share_nblocks=[0, 3])
    assert st == _lib.OK and d256.shared_blocks > 0
    assert _choose(d256, 16, lens, 512) <= 2            # shared blocks: cache-retaining loads
    with pytest.raises(Exception):
        _choose(d256, 15, lens, 512)                    # not a multiple of the KV heads
    assert _choose(_pool(1, 0, bs=16, hkv=2, d=128), 16, [64], 512, cus=0) >= 1  # no device
