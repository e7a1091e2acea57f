"""CPU tests of the decode plan (kvattn_decode_plan): sequences that hold the same token range
in the same blocks share one wave item ([VAMP] §II-A prefix reuse; [CrossPool] §3.1 paged
tables); every sequence's tokens are covered exactly once by the items it is a member of, its
partial slots run 0 .. nparts - 1 in token order ([InplaceKVCache] §5.1: any partition of the
tokens merges exactly), and the plan reads each shared range once.  No GPU: the planner is host
bookkeeping, and fake device addresses are never touched.
"""

import functools

import numpy as np
import pytest

from paged_kv_cache_mla_amd import _lib
from paged_kv_cache_mla_amd.api import Pool, decode_plan
from synth import make_case

FAKE = 0x7F0000000000
HEADER, ITEM = 8, 6


@functools.lru_cache(maxsize=None)
def _case(name, variant):
    """Cases are only read here: one build per (name, variant) for the whole module."""
    return make_case(name, variant)


def _pool_for(case):
    return Pool(case.block_size, case.num_kv_heads, case.head_dim_k, case.head_dim_v, case.dtype,
                case.latent, [(FAKE + (i << 32), n) for i, n in enumerate(case.region_blocks)])


def parse(plan, batch):
    hdr = plan[:HEADER]
    nparts = plan[HEADER:HEADER + batch]
    n_items = int(hdr[3])
    items = plan[HEADER + batch:HEADER + batch + ITEM * n_items].reshape(n_items, ITEM)
    members = plan[HEADER + batch + ITEM * n_items:].reshape(-1, 2)
    return hdr, nparts, items, members


def check_plan(plan, n_groups, max_parts, table, lens, begins, parts, bs, group, span=3):
    """The plan's invariants (raises AssertionError)."""
    batch = len(lens)
    hdr, nparts, items, members = parse(plan, batch)
    assert hdr[0] == 0x4E4C5031 and hdr[1] == batch and hdr[2] == n_groups
    assert hdr[3] == 4 * n_groups and hdr[4] == members.shape[0] and hdr[6] == group
    mpw = 16 // group
    assert hdr[7] == mpw and max_parts == max(1, int(nparts.max()))
    # a staged workgroup (mode 2): all four items mode 2 over one range, at least two of them
    # with sequences (the rest padding); modes 0 / 1 only in workgroups of independent waves
    for g in range(n_groups):
        gi = items[4 * g:4 * g + 4]
        if (gi[:, 5] == 2).any():
            assert (gi[:, 5] == 2).all() and (gi[:, :3] == gi[0, :3]).all(), g
            assert (gi[:, 3] > 0).sum() >= 2
        else:
            assert set(gi[:, 5].tolist()) <= {0, 1}
    covered = [[] for _ in range(batch)]       # (lo, hi, slot) per sequence
    for x, (seq, lo, hi, nmem, moff, shared) in enumerate(items):
        if nmem == 0:
            continue
        assert 1 <= nmem <= mpw and 0 <= lo < hi
        assert (hi - 1) // bs - lo // bs < 128                 # the wave's window of block ids
        mem = members[moff:moff + nmem]
        assert seq in mem[:, 0] or shared                      # the row read is a member's
        blocks = table[seq][lo // bs:(hi - 1) // bs + 1]
        assert (blocks >= 0).all()
        for m, slot in mem:
            assert np.array_equal(table[m][lo // bs:(hi - 1) // bs + 1], blocks), (x, m)
            assert lo >= begins[m] and hi <= lens[m]
            assert hi - lo <= span * parts[m]               # at most span partitions of tokens
            covered[m].append((lo, hi, slot))
    for b in range(batch):
        cov = sorted(covered[b])
        assert [s for _, _, s in cov] == list(range(len(cov))) == list(range(nparts[b]))
        pos = begins[b]
        for lo, hi, _ in cov:
            assert lo == pos
            pos = hi
        assert pos == lens[b]
    return items, members


def _case_arrays(case):
    begins = np.zeros(case.batch, np.int32) if case.tok_begin is None else case.tok_begin
    return case.table, case.ctx_lens, begins, case.part_tokens


@pytest.mark.parametrize("variant", ["small", "full"])
def test_prefix_pool_plan_covers_each_sequence_and_reads_shared_blocks_once(variant):
    case = _case("prefix_shared", variant)
    pool = _pool_for(case)
    table, lens, begins, parts = _case_arrays(case)
    plan, ng, mp = decode_plan(pool, case.num_q_heads, table, lens, begins, parts)
    group = case.num_q_heads // case.num_kv_heads
    items, members = check_plan(plan, ng, mp, table, lens, begins, parts, case.block_size, group)
    # tokens the plan reads per KV head: each item's range once per distinct (row, range)
    ranges = {(int(s), int(lo), int(hi)) for s, lo, hi, n, _, _ in items if n > 0}
    read = sum(hi - lo for _, lo, hi in ranges)
    bs = case.block_size
    keys = np.concatenate([table[b][np.arange(lens[b]) // bs].astype(np.int64) * bs + np.arange(lens[b]) % bs
                           for b in range(case.batch)])
    unique = np.unique(keys).size
    logical = int(lens.sum())
    # sharing is found block by block: the plan reads exactly the unique token slots
    assert read == unique, (read, unique, logical)
    assert read < 0.5 * logical
    if variant == "full":   # ranges of every kind: staged, two waves, one wave
        assert check_range_modes(items, members) == {1, 2, 3}
    check_range_modes(items, members)


def check_range_modes(items, members, stage_min=3):
    """Placement of a range's wave items by their number k: k >= stage_min, ceil(k / 4)
    staged workgroups of their own (mode 2), sizes within one; 2 <= k < stage_min, one
    workgroup, mode 1; k = 1, mode 0 (read once, streamed), shared or private."""
    by_range = {}
    for x, (s, lo, hi, n, off, mode) in enumerate(items):
        if n > 0:
            by_range.setdefault((s, lo, hi), []).append((x // 4, mode, n))
    kinds = set()
    for v in by_range.values():
        k = len(v)
        wgs = sorted({g for g, _, _ in v})
        modes = {m for _, m, _ in v}
        if k >= stage_min:
            assert modes == {2} and len(wgs) == -(-k // 4)
            sizes = [sum(1 for g, _, _ in v if g == w) for w in wgs]
            assert max(sizes) - min(sizes) <= 1
        elif k >= 2:
            assert modes == {1} and len(wgs) == 1
        else:
            assert modes == {0}
        kinds.add(min(k, stage_min))
    return kinds


@pytest.mark.parametrize("layout,stage_min", [("same", 99), ("stage", 2), ("stage", 4)])
def test_placement_switches_keep_items_and_slots(monkeypatch, layout, stage_min):
    """The tuning switches (KVATTN_PLAN_LAYOUT=same: no staged workgroup; KVATTN_PLAN_STAGE_MIN:
    the k from which a range is staged) change where the wave items run, not the items, their
    members or their slots."""
    case = _case("prefix_shared", "full")
    pool = _pool_for(case)
    table, lens, begins, parts = _case_arrays(case)
    group = case.num_q_heads // case.num_kv_heads
    plan_d, ng_d, mp_d = decode_plan(pool, case.num_q_heads, table, lens, begins, parts)
    items_d, members_d = check_plan(plan_d, ng_d, mp_d, table, lens, begins, parts,
                                    case.block_size, group)
    monkeypatch.setenv("KVATTN_PLAN_LAYOUT", layout)
    monkeypatch.setenv("KVATTN_PLAN_STAGE_MIN", str(stage_min))
    plan, ng, mp = decode_plan(pool, case.num_q_heads, table, lens, begins, parts)
    items, members = check_plan(plan, ng, mp, table, lens, begins, parts, case.block_size, group)
    check_range_modes(items, members, stage_min)
    assert mp == mp_d and ((items[:, 5] == 2).any() == (layout == "stage"))

    def entries(it, mem):
        return sorted((int(s), int(lo), int(hi), int(m), int(sl)) for s, lo, hi, n, off, _ in it
                      for m, sl in mem[off:off + n])
    assert entries(items, members) == entries(items_d, members_d)


def test_private_layer_plan_is_one_item_per_span():
    """Without shared blocks every item is private, one sequence, up to the window's
    partitions (3 partitions of 32 blocks in 127 block ids), partial counts as the span implies."""
    case = make_case("gqa_32k", "small")
    pool = _pool_for(case)
    table, lens, begins, parts = _case_arrays(case)
    plan, ng, mp = decode_plan(pool, case.num_q_heads, table, lens, begins, parts)
    items, _ = check_plan(plan, ng, mp, table, lens, begins, parts, 16, 8)
    assert (items[:, 5] == 0).all() and (items[items[:, 3] > 0, 3] == 1).all()
    hdr, nparts, _, _ = parse(plan, case.batch)
    for b in range(case.batch):
        npart = -(-int(lens[b]) // 512)
        assert nparts[b] == -(-npart // 3)
    plan2, ng2, mp2 = decode_plan(pool, case.num_q_heads, table, lens, begins, parts, span_parts=2)
    check_plan(plan2, ng2, mp2, table, lens, begins, parts, 16, 8, span=2)
    assert mp2 == -(-(-(-int(lens.max()) // 512)) // 2)


def test_sharing_needs_identical_blocks_and_ranges():
    """Sharing is decided block position by position: the same block id with the same token
    extent.  A differing block splits the run, a different start leaves only the first block
    apart, an invalid id stays private, and pieces are at most span_parts partitions long;
    groups of 1 .. 16 query heads per KV head (16 .. 1 sequences per wave item)."""
    bs = 16
    pool = Pool(bs, 2, 64, 64, "bf16", False, [(FAKE, 400)])
    rng = np.random.default_rng(3)
    ids = rng.permutation(400).astype(np.int32)
    mb = 40
    t = np.full((6, mb), -1, np.int32)
    t[0, :40] = ids[:40]
    t[1, :40] = ids[:40]                  # same as 0
    t[2, :40] = ids[:40]
    t[2, 5] = ids[100]                    # differs in partition 1 (blocks 4..7 at P = 64)
    t[3, :40] = ids[:40]                  # same blocks, different begin
    t[4, :30] = ids[:30]
    t[4, 30:40] = ids[200:210]            # shares blocks 0..29
    t[5, :40] = ids[300:340]
    t[5, 2] = 999                         # invalid id: private, flagged by the kernel
    lens = np.array([640, 640, 640, 600, 640, 640], np.int32)
    begins = np.array([0, 0, 0, 8, 0, 0], np.int32)
    parts = np.array([64] * 6, np.int32)
    for hq in (2, 6, 16, 32):
        group = hq // 2
        plan, ng, mp = decode_plan(pool, hq, t, lens, begins, parts, span_parts=3)
        items, members = check_plan(plan, ng, mp, t, lens, begins, parts, bs, group, span=3)
        mem_sets = {}
        for s, lo, hi, n, off, sh in items:
            if n:
                for m, _ in members[off:off + n]:
                    mem_sets.setdefault((int(s), int(lo), int(hi)), set()).add(int(m))
        together = {k: sorted(v) for k, v in mem_sets.items()}
        # block 5 of sequence 2 differs: [80, 96) is 0, 1, 4 only, and 2 shares 0's other
        # blocks; 3 shares the blocks but starts at token 8, so only its first block differs;
        # 4 shares blocks 0..29; 5 (an invalid id) shares nothing
        assert together[(0, 0, 16)] == [0, 1, 2, 4] and together[(3, 8, 16)] == [3]
        assert together[(0, 16, 80)] == [0, 1, 2, 3, 4]
        assert together[(0, 80, 96)] == [0, 1, 3, 4] and together[(2, 80, 96)] == [2]
        assert all(5 not in v or v == [5] for v in together.values())
        assert max(hi for (_, lo, hi), v in together.items() if 4 in v and len(v) > 1) == 30 * bs


def test_plan_errors():
    case = make_case("prefix_shared", "small")
    pool = _pool_for(case)
    table, lens, begins, parts = _case_arrays(case)
    with pytest.raises(_lib.KvattnError):
        decode_plan(pool, 15, table, lens, begins, parts)                  # heads not a multiple
    with pytest.raises(_lib.KvattnError):
        decode_plan(pool, 16, table, lens, begins, parts + 1)              # not a block multiple
    bad_beg = begins.copy()
    bad_beg[0] = lens[0] + 1
    with pytest.raises(_lib.KvattnError):
        decode_plan(pool, 16, table, lens, bad_beg, parts)
    with pytest.raises(_lib.KvattnError):          # pieces of 2 x 2064 tokens: > 127 blocks
        decode_plan(pool, 16, table, lens, begins, np.full_like(parts, 2064), span_parts=2)
    decode_plan(pool, 16, table, lens, begins, np.full_like(parts, 4096))   # 0: pieces fit
    mla = Pool(64, 1, 576, 512, "bf16", True, [(FAKE, 4)])
    with pytest.raises(_lib.KvattnError):
        decode_plan(mla, 16, np.zeros((1, 4), np.int32), [64], None, [64])
    # a buffer one entry short is refused
    lib = _lib.load()
    import ctypes
    plan, ng, mp = decode_plan(pool, 16, table, lens, begins, parts)
    n, g, m = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    t = np.ascontiguousarray(table)
    p32 = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))  # noqa: E731
    buf = np.zeros(plan.size - 1, np.int32)
    st = lib.kvattn_decode_plan(pool.handle, case.batch, 16, p32(t), t.shape[1], p32(lens),
                                p32(np.ascontiguousarray(begins)), p32(parts), 0, p32(buf),
                                buf.size, ctypes.byref(n), ctypes.byref(g), ctypes.byref(m))
    assert st == _lib.E_INVAL and n.value == plan.size


def test_decode_partial_plan_validation_without_gpu():
    """Argument checks of kvattn_decode_partial_plan, all before any launch."""
    import ctypes
    lib = _lib.load()
    case = make_case("prefix_shared", "small")
    pool = _pool_for(case)
    vp = ctypes.c_void_p

    def call(p=pool, q=FAKE, qd=_lib.BF16, batch=16, hq=16, plan=FAKE, ng=3, work=None, mp=4,
             o=FAKE, lse=FAKE, npart=FAKE):
        return lib.kvattn_decode_partial_plan(p.handle, vp(q) if q else None, qd, batch, hq,
                                              ctypes.c_float(0.1), vp(FAKE), 97,
                                              vp(plan) if plan else None, ng,
                                              vp(work) if work else None, mp,
                                              vp(o) if o else None, vp(lse), vp(npart), None, None)
    assert call(q=None) == _lib.E_INVAL
    assert call(plan=None) == _lib.E_INVAL
    assert call(q=FAKE + 4) == _lib.E_INVAL                  # q not 16-byte aligned
    assert call(work=FAKE + 4) == _lib.E_INVAL               # work counters not 8-byte aligned
    assert call(ng=-1) == _lib.E_INVAL
    assert call(mp=0) == _lib.E_INVAL
    assert call(hq=15) == _lib.E_INVAL
    assert call(qd=_lib.F32) == _lib.E_UNSUPPORTED
    mla = Pool(64, 1, 576, 512, "bf16", True, [(FAKE, 4)])
    assert call(p=mla) == _lib.E_UNSUPPORTED


def _random_pool_case(rng):
    """A random shared pool: sequences that take prefixes of random length from a few stems
    (some of them nested), then private blocks; random starts (some inside a block), ends,
    block size, group size and span; now and then an invalid id or an empty sequence."""
    bs = int(rng.choice([16, 32, 64]))
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 4, 6, 8, 16]))
    nseq = int(rng.integers(1, 24))
    nblk = int(rng.integers(1, 90))
    nstem = int(rng.integers(1, 4))
    pool_blocks = nstem * nblk + nseq * nblk + 4
    ids = rng.permutation(pool_blocks).astype(np.int32)
    stems = [ids[s * nblk:(s + 1) * nblk] for s in range(nstem)]
    pos = nstem * nblk
    table = np.full((nseq, nblk), -1, np.int32)
    lens = np.zeros(nseq, np.int32)
    begins = np.zeros(nseq, np.int32)
    for s in range(nseq):
        nb = int(rng.integers(1, nblk + 1))
        k = int(rng.integers(0, nb + 1))
        table[s, :k] = stems[int(rng.integers(0, nstem))][:k]
        table[s, k:nb] = ids[pos:pos + nb - k]
        pos += nb - k
        lens[s] = nb * bs - int(rng.integers(0, bs))
        r = rng.random()
        begins[s] = 0 if r < 0.6 else (int(rng.integers(0, lens[s] + 1)) if r < 0.95 else lens[s])
        if rng.random() < 0.1 and nb > 1:
            table[s, int(rng.integers(0, nb))] = pool_blocks + 7       # invalid: private
    parts = np.full(nseq, bs * int(rng.choice([1, 2, 4, 8])), np.int32)
    span = int(rng.integers(0, 4))
    while span > 0 and span * parts[0] // bs >= 128:
        span -= 1
    return bs, hkv, group, table, lens, begins, parts, span, pool_blocks


@pytest.mark.parametrize("seed", range(100))
def test_random_pools_plan_invariants(seed):
    """The plan invariants on random pools: coverage of every sequence's tokens exactly once,
    slots in token order, sharing only over identical blocks and extents, the window, the
    placement rules; and, where no id is invalid, exactly the unique token slots read."""
    rng = np.random.default_rng(5000 + seed)
    bs, hkv, group, table, lens, begins, parts, span, pool_blocks = _random_pool_case(rng)
    pool = Pool(bs, hkv, 64, 64, "bf16", False, [(FAKE, pool_blocks)])
    plan, ng, mp = decode_plan(pool, hkv * group, table, lens, begins, parts, span_parts=span)
    items, members = check_plan(plan, ng, mp, table, lens, begins, parts, bs, group,
                                span=span if span else 128)
    check_range_modes(items, members)
    # the header's bound on a plan's length: 8 + batch + 26 P (P: block positions)
    live = lens > begins
    positions = int(np.sum((lens[live] - 1) // bs - begins[live] // bs + 1))
    assert plan.size <= 8 + len(lens) + 26 * positions
    if not (table >= pool_blocks).any():
        # every distinct (position, block id, token extent) key is read once: blocks held with
        # the same extent are read once for all their holders, and a block two sequences hold
        # with different extents (a start or an end inside it) once per extent
        ranges = {(int(s), int(lo), int(hi)) for s, lo, hi, n, _, _ in items if n > 0}
        read = sum(hi - lo for _, lo, hi in ranges)
        keys = set()
        for b in range(len(lens)):
            for i in range(begins[b] // bs, (lens[b] - 1) // bs + 1 if lens[b] > begins[b] else 0):
                keys.add((i, int(table[b, i]), max(int(begins[b]), i * bs), min(int(lens[b]), (i + 1) * bs)))
        assert read == sum(hi - lo for _, _, lo, hi in keys), (read, len(keys))
        if (begins == 0).all():          # equal starts: shared blocks differ only in their last
            slots = set()                # block's extent, so at most one extra read per holder
            for b in range(len(lens)):
                t = np.arange(begins[b], lens[b])
                slots.update(zip(table[b][t // bs].tolist(), (t % bs).tolist()))
            assert len(slots) <= read <= len(slots) + bs * len(lens)


@pytest.mark.parametrize("seed", range(20))
def test_plan_does_not_depend_on_pool_size(seed):
    """The same tables planned over a pool just large enough and over one far larger than the
    plan (where the planner keys block ids through a hash map rather than an array over the
    pool) give the same plan, bit for bit."""
    rng = np.random.default_rng(8000 + seed)
    bs, hkv, group, table, lens, begins, parts, span, pool_blocks = _random_pool_case(rng)
    table = np.where(table >= pool_blocks, -5, table)       # no invalid ids: both pools hold all
    plans = []
    for nblocks in (pool_blocks, pool_blocks + 400_000):
        pool = Pool(bs, hkv, 64, 64, "bf16", False, [(FAKE, nblocks)])
        plans.append(decode_plan(pool, hkv * group, table, lens, begins, parts, span_parts=span))
    assert np.array_equal(plans[0][0], plans[1][0]) and plans[0][1:] == plans[1][1:]
