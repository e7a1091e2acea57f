"""GPU parity of the planned decode (kvattn_decode_plan + kvattn_decode_partial_plan + merge),
through the C ABI, against the float64 oracle.

Sequences that hold the same token range in the same blocks share one wave item, whose
columns carry several sequences' query heads ([VAMP] §II-A prefix reuse; [CrossPool] §3.1
paged tables); every sequence still gets its own partials, which merge to its attention
([InplaceKVCache] §5.1).  Tolerances as in test_gpu_parity: bf16 caches max |o - o_ref| /
max |o_ref| <= 2e-3, lse within 2e-3; each item's partial is checked against the oracle's
attention over its token range, element by element.
"""

import sys

import numpy as np
import pytest

import oracle
from synth import make_case
from synth.workloads import _normals, _streams
from tests import oracle_cases as oc
from tests.test_plan_cpu import parse

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


def _run_plan(case, span_parts=0, plan=True):
    from paged_kv_cache_mla_amd.session import DeviceCase
    dc = DeviceCase(case, plan=plan, span_parts=span_parts)
    o, lse = dc.run()
    torch.cuda.synchronize()
    return dc, o.cpu().numpy(), lse.cpu().numpy()


def _check_items(case, dc):
    """Every item's partial for every member equals the oracle's attention over the item's
    token range of that member; nparts equals the plan's counts."""
    plan = dc.step.plan
    hdr, nparts, items, members = parse(plan, case.batch)
    assert np.array_equal(dc.step.nparts.cpu().numpy(), nparts)
    o_part = dc.step.o_part.cpu().numpy()
    l_part = dc.step.lse_part.cpu().numpy()
    lay = oc.layout_of(case)
    qf = oc.q_f64(case)
    worst = 0.0
    for seq, lo, hi, nmem, moff, _ in items:
        for m, slot in members[moff:moff + nmem]:
            k, v = oracle.gather_sequence(lay, case.regions, case.region_blocks, case.table[m], lo, hi)
            o_ref, l_ref = oracle.attend(qf[m], k, v, case.scale)
            err = float(np.max(np.abs(o_part[m, :, slot] - o_ref))) / float(np.max(np.abs(o_ref)))
            worst = max(worst, err)
            assert err <= oc.out_tol(case), (m, slot, err)
            assert float(np.max(np.abs(l_part[m, :, slot] - l_ref))) <= oc.lse_tol(case)
    return worst


@pytest.mark.parametrize("span_parts", [0, 1, 2])
def test_prefix_pool_plan_matches_oracle(span_parts):
    case = make_case("prefix_shared", "small")
    _say(f"[plan] prefix_shared small, span_parts {span_parts}")
    dc, o, lse = _run_plan(case, span_parts)
    assert dc.step.plan is not None and int(dc.step.err.item()) == 0
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    worst = _check_items(case, dc)
    _say(f"[plan] out error {err:.3e}, worst item partial {worst:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)


def test_shared_pool_takes_the_plan_by_default_and_both_paths_agree():
    """A pool holding shared blocks runs the plan when group_parts is the library's choice;
    the per-sequence kernel on the same pool (group_parts given) agrees within rounding, and
    the plan path is bitwise deterministic."""
    from paged_kv_cache_mla_amd.session import DeviceCase
    case = make_case("prefix_shared", "small")
    auto = DeviceCase(case)
    assert auto.step.plan is not None
    o1, l1 = (t.clone() for t in auto.run())
    o2, l2 = auto.run()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    per_seq = DeviceCase(case, group_parts=2)
    assert per_seq.step.plan is None
    o3, l3 = per_seq.run()
    torch.cuda.synchronize()
    o_ref, _ = oc.full_reference(case)
    assert oc.out_error(case, o1.cpu().numpy(), o_ref) <= oc.out_tol(case)
    assert oc.out_error(case, o3.cpu().numpy(), o_ref) <= oc.out_tol(case)


def _custom_case(bs, hkv, d, hq, table, lens, begins, part, pool_blocks, seed=1011):
    """A bf16 per-head case over `pool_blocks` blocks of random data with the given table."""
    from synth.workloads import _finish
    rq, rkv, _, _ = _streams(seed)
    return _finish("plan_custom", "small", seed, bs, hkv, d, d, "bf16", False, hq,
                   1 / np.sqrt(float(d)), [pool_blocks], np.asarray(table, np.int32), lens,
                   begins, [part] * len(lens), rq, rkv)


def _sharing_table(rng, nseq, nblk, pool_blocks, bs):
    """Sequences over a common stock of blocks: each takes a prefix of a random length from
    one of two stems, then private blocks; one sequence also differs from its stem in one
    block inside the prefix."""
    ids = rng.permutation(pool_blocks).astype(np.int32)
    stems = [ids[:nblk], ids[nblk:2 * nblk]]
    pos = 2 * nblk
    t = np.full((nseq, nblk), -1, np.int32)
    for s in range(nseq):
        stem = stems[s % 2]
        k = int(rng.integers(0, nblk + 1))
        t[s, :k] = stem[:k]
        t[s, k:] = ids[pos:pos + nblk - k]
        pos += nblk - k
    t[2, 1] = ids[pos]
    return t


GEOMS = [(16, 2, 256, 16), (16, 4, 128, 32), (32, 2, 64, 2), (64, 1, 128, 16), (16, 2, 128, 6),
         (16, 1, 64, 16), (128, 2, 128, 4), (256, 2, 256, 16), (32, 1, 256, 6), (16, 4, 256, 8)]


@pytest.mark.parametrize("bs,hkv,d,hq", GEOMS, ids=[f"bs{g[0]}-hkv{g[1]}-d{g[2]}-hq{g[3]}" for g in GEOMS])
def test_plan_kernel_geometries_with_ragged_sharing(bs, hkv, d, hq):
    """Sharing of random prefix lengths from two stems, ragged ends and starts (one sequence
    starts inside a block), block sizes 16 .. 256, head dims 64 / 128 / 256, 1 .. 16 query
    heads per KV head (16 .. 1 sequences per wave item; at 6 heads per KV head, 4 of the 16
    columns carry no query, also where head dim 256 keeps Q^T in LDS)."""
    rng = np.random.default_rng(bs * 7 + d + hq)
    nseq, nblk = 9, 24
    pool_blocks = 2 * nblk + nseq * nblk + 8
    table = _sharing_table(rng, nseq, nblk, pool_blocks, bs)
    lens = [int(nblk * bs - rng.integers(0, bs)) for _ in range(nseq)]
    lens[4] = bs * 3 + 1
    begins = [0] * nseq
    begins[5] = bs // 2 + 1
    case = _custom_case(bs, hkv, d, hq, table, lens, begins, bs * 4, pool_blocks)
    for s in range(nseq):
        case.table[s, -(-lens[s] // bs):] = -1
    _say(f"[plan-geom] bs={bs} hkv={hkv} d={d} hq={hq}")
    dc, o, lse = _run_plan(case, span_parts=2)
    assert int(dc.step.err.item()) == 0
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    worst = _check_items(case, dc)
    _say(f"[plan-geom] out error {err:.3e}, worst item {worst:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)


def test_plan_with_invalid_ids_and_a_stale_header():
    """An invalid id inside a range is flagged and contributes nothing; a plan whose header
    does not match the call is refused by the kernel (flagged, nothing written)."""
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.session import DeviceCase
    case = make_case("prefix_shared", "small")
    dc = DeviceCase(case)
    bad = dc.table.copy()
    b = 0                     # the lowest sequence of its shared prefix: its row is the one read
    bad[b, 2] = sum(case.region_blocks) + 5
    dc.step.table_dev.copy_(torch.from_numpy(bad))
    o, lse = dc.run()
    torch.cuda.synchronize()
    assert int(dc.step.err.item()) & _lib.ERR_BAD_BLOCK
    assert np.isfinite(o.cpu().numpy()).all()
    # a plan for another batch size
    dc2 = DeviceCase(case)
    dc2.step.plan_dev[1] = case.batch + 1
    dc2.step.nparts.fill_(-5)
    dc2.step.partial(dc2.q, dc2.q_dtype, case.scale)
    torch.cuda.synchronize()
    assert int(dc2.step.err.item()) & _lib.ERR_BAD_SEQ
    assert (dc2.step.nparts.cpu().numpy() == -5).all()
    # buffers sized for fewer partials than the plan writes: refused the same way
    from paged_kv_cache_mla_amd.api import decode_partial_plan
    dc3 = DeviceCase(case)
    dc3.step.nparts.fill_(-5)
    st = dc3.step
    decode_partial_plan(st.pool, dc3.q, dc3.q_dtype, case.num_q_heads, case.scale, st.table_dev,
                        st.max_blocks, st.plan_dev, st.n_groups, st.max_parts - 1, st.o_part,
                        st.lse_part, st.nparts, st.err)
    torch.cuda.synchronize()
    assert int(st.err.item()) & _lib.ERR_BAD_SEQ
    assert (st.nparts.cpu().numpy() == -5).all()


def test_plan_relabelled_blocks_give_identical_bits():
    """Moving every physical block (and rewriting the tables) changes no output bit: the plan's
    items and their arithmetic depend on which blocks are equal, not on where they are."""
    case = make_case("prefix_shared", "small")
    _, o1, l1 = _run_plan(case)
    rng = np.random.default_rng(9)
    total = sum(case.region_blocks)
    perm = rng.permutation(total).astype(np.int32)
    flat = np.concatenate(case.regions)
    nel = case.elems_per_block()
    moved = np.empty_like(flat)
    for old in range(total):
        moved[perm[old] * nel:(perm[old] + 1) * nel] = flat[old * nel:(old + 1) * nel]
    c2 = make_case("prefix_shared", "small")
    c2.regions = [moved[:case.region_blocks[0] * nel], moved[case.region_blocks[0] * nel:]]
    c2.table = np.where(case.table >= 0, perm[np.maximum(case.table, 0)], -1).astype(np.int32)
    _, o2, l2 = _run_plan(c2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", ["prefix_shared", "gqa_32k"])
def test_claiming_launch_equals_one_unit_per_workgroup(name):
    """With work counters the workgroups take units as they finish (as many workgroups as the
    device holds); the result equals the one-unit-per-workgroup launch bit for bit, every
    step, and every launch leaves the counters at zero."""
    from paged_kv_cache_mla_amd.session import DeviceCase
    case = make_case(name, "small")
    fixed = DeviceCase(case, plan=True, claim=False)
    claim = DeviceCase(case, plan=True, claim=True)
    assert fixed.step.work is None and claim.step.work is not None
    o_f, l_f = (t.clone() for t in fixed.run())
    for step in range(4):
        o_c, l_c = claim.run()
        torch.cuda.synchronize()
        assert torch.equal(o_c, o_f) and torch.equal(l_c, l_f), step
        assert (claim.step.work.cpu().numpy() == 0).all(), step
    assert int(claim.step.err.item()) == 0
    o_ref, _ = oc.full_reference(case)
    assert oc.out_error(case, o_f.cpu().numpy(), o_ref) <= oc.out_tol(case)


def _one_row_case(nseq, length, begin, bs, hkv, d, hq, seed):
    """`nseq` sequences holding one table row over the same tokens [begin, length): every range
    has nseq sharers."""
    rng = np.random.default_rng(seed)
    nblk = -(-length // bs)
    pool_blocks = nblk + 6
    ids = rng.permutation(pool_blocks).astype(np.int32)
    table = np.tile(ids[:nblk], (nseq, 1))
    return _custom_case(bs, hkv, d, hq, table, [length] * nseq, [begin] * nseq, bs * 4,
                        pool_blocks, seed)


STAGED = [(256, 16, 2, 1237, 0), (128, 32, 4, 901, 21), (64, 16, 1, 2047, 5)]


@pytest.mark.parametrize("d,hq,hkv,length,begin", STAGED,
                         ids=[f"d{s[0]}-hq{s[1]}-hkv{s[2]}-L{s[3]}-b{s[4]}" for s in STAGED])
def test_staged_ranges_ignore_nan_in_unused_slots(d, hq, hkv, length, begin):
    """Eight sequences on one table row: every range has eight sharers, which at 8 or 16 query
    heads per KV head fill 4 or 8 wave items, so every range is staged (mode 2).  Every token
    slot outside [begin, length) holds a NaN bit pattern; the staged workgroups read whole
    32-token stages, and the lines of a tile or stage past the range load other tiles again,
    so those slots reach the waves and must get zero weight and zeroed V.  Ragged ends, a start
    inside a block, pairs not a multiple of the ring depth."""
    from tests.test_gpu_parity import _poison_unused_slots
    case = _poison_unused_slots(_one_row_case(8, length, begin, 16, hkv, d, hq, 1013 + d))
    _say(f"[staged] d={d} hq={hq} hkv={hkv} L={length} begin={begin}")
    dc, o, lse = _run_plan(case, span_parts=2)
    _, _, items, _ = parse(dc.step.plan, case.batch)
    assert (items[items[:, 3] > 0, 5] == 2).all()
    assert int(dc.step.err.item()) == 0
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    worst = _check_items(case, dc)
    _say(f"[staged] out error {err:.3e}, worst item {worst:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)


def test_staged_range_with_an_invalid_id_is_flagged():
    """A block id that turns invalid inside a staged range after the plan was made (the plan
    is built from the host table, the device table changes): KVATTN_ERR_BAD_BLOCK, finite
    output, the block's tokens contribute nothing to its range's partials, and every other
    partial still equals the oracle's."""
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.session import DeviceCase
    case = _one_row_case(8, 1500, 0, 16, 2, 256, 16, 1021)
    dc = DeviceCase(case, plan=True, span_parts=1)
    bad = dc.table.copy()
    bad[:, 40] = sum(case.region_blocks) + 3          # tokens [640, 656)
    dc.step.table_dev.copy_(torch.from_numpy(bad))
    o, lse = dc.run()
    torch.cuda.synchronize()
    assert int(dc.step.err.item()) & _lib.ERR_BAD_BLOCK
    assert np.isfinite(o.cpu().numpy()).all()
    hdr, nparts, items, members = parse(dc.step.plan, case.batch)
    o_part = dc.step.o_part.cpu().numpy()
    qf = oc.q_f64(case)
    lay = oc.layout_of(case)
    holding = 0
    for seq, lo, hi, nmem, moff, mode in items:
        if nmem == 0:
            continue
        assert mode == 2
        spans = [(lo, hi)]
        if lo < 656 and hi > 640:      # the range holds the invalid block: the rest of it
            spans = [(a, b) for a, b in ((lo, 640), (656, hi)) if b > a]
            holding += 1
        for m, slot in members[moff:moff + nmem]:
            parts = [oracle.gather_sequence(lay, case.regions, case.region_blocks, case.table[m], a, b)
                     for a, b in spans]
            k = np.concatenate([p[0] for p in parts])
            v = np.concatenate([p[1] for p in parts])
            o_ref, _ = oracle.attend(qf[m], k, v, case.scale)
            err = float(np.max(np.abs(o_part[m, :, slot] - o_ref))) / float(np.max(np.abs(o_ref)))
            assert err <= oc.out_tol(case), (m, slot, lo, hi, err)
    assert holding > 0


def test_claiming_launch_with_more_units_than_the_device_holds():
    """Units enough that claiming workgroups run several each: eight sequences on one table row
    (staged ranges) and sixteen private ones, 64-token pieces at head dim 256 (ring waves keep
    Q^T in the workgroup's LDS, which a staged unit before them used for its stages).  The
    claiming launch equals the one-unit launch bit for bit, leaves the counters at zero, and
    sampled sequences match the oracle."""
    from paged_kv_cache_mla_amd.session import DeviceCase
    bs, hkv, d, hq, L = 16, 2, 256, 16, 4096
    rng = np.random.default_rng(1051)
    nblk = L // bs
    pool_blocks = 17 * nblk + 6
    ids = rng.permutation(pool_blocks).astype(np.int32)
    table = np.concatenate([np.tile(ids[:nblk], (8, 1)),
                            ids[nblk:17 * nblk].reshape(16, nblk)]).astype(np.int32)
    case = _custom_case(bs, hkv, d, hq, table, [L] * 24, [0] * 24, 64, pool_blocks, 1051)
    fixed = DeviceCase(case, plan=True, span_parts=1)
    claim = DeviceCase(case, plan=True, span_parts=1, claim=True)
    units = fixed.step.n_groups * hkv
    _say(f"[claim] {units} units")
    assert units > 2 * 256
    _, _, items, _ = parse(fixed.step.plan, case.batch)
    assert (items[:, 5] == 2).any() and (items[:, 5] == 0).any()
    o_f, l_f = (t.clone() for t in fixed.run())
    for step in range(3):
        o_c, l_c = claim.run()
        torch.cuda.synchronize()
        assert torch.equal(o_c, o_f) and torch.equal(l_c, l_f), step
        assert (claim.step.work.cpu().numpy() == 0).all(), step
    assert int(claim.step.err.item()) == 0 and int(fixed.step.err.item()) == 0
    o = o_f.cpu().numpy()
    lay = oc.layout_of(case)
    qf = oc.q_f64(case)
    for b in (0, 5, 8, 23):
        k, v = oracle.gather_sequence(lay, case.regions, case.region_blocks, case.table[b], 0, L)
        o_ref, _ = oracle.attend(qf[b], k, v, case.scale)
        assert float(np.max(np.abs(o[b] - o_ref))) / float(np.max(np.abs(o_ref))) <= oc.out_tol(case), b


def test_plan_with_empty_sequences_and_an_empty_batch():
    """A sequence with no tokens (tok_begin = ctx_len) gets no wave item and no partial: its
    output is zero and its lse -inf, like the oracle's; the others are unaffected.  A batch
    with no tokens at all plans zero workgroups, and the launch only writes zero counts."""
    bs, hkv, d, hq = 16, 2, 128, 16
    rng = np.random.default_rng(77)
    nseq, nblk = 6, 20
    pool_blocks = 2 * nblk + nseq * nblk + 8
    table = _sharing_table(rng, nseq, nblk, pool_blocks, bs)
    lens = [nblk * bs - 3] * nseq
    begins = [0] * nseq
    begins[1] = lens[1]                 # empty at its end
    begins[4] = lens[4] = 5 * bs + 2     # empty inside a block
    for s in range(nseq):
        table[s, -(-lens[s] // bs):] = -1
    case = _custom_case(bs, hkv, d, hq, table, lens, begins, bs * 4, pool_blocks)
    dc, o, lse = _run_plan(case, span_parts=2)
    assert int(dc.step.err.item()) == 0
    nparts = dc.step.nparts.cpu().numpy()
    assert nparts[1] == 0 and nparts[4] == 0 and (np.delete(nparts, [1, 4]) > 0).all()
    o_ref, lse_ref = oc.full_reference(case)
    assert (o[[1, 4]] == 0).all() and np.isneginf(lse[[1, 4]]).all()
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)
    keep = np.delete(np.arange(nseq), [1, 4])
    assert float(np.max(np.abs(lse[keep] - lse_ref[keep]))) <= oc.lse_tol(case)
    # no tokens anywhere: an empty plan
    empty = _custom_case(bs, hkv, d, hq, table, lens, lens, bs * 4, pool_blocks)
    dc0, o0, lse0 = _run_plan(empty)
    assert dc0.step.n_groups == 0 and int(dc0.step.err.item()) == 0
    assert (dc0.step.nparts.cpu().numpy() == 0).all()
    assert (o0 == 0).all() and np.isneginf(lse0).all()


@pytest.mark.parametrize("seed", range(6))
def test_random_pools_plan_matches_oracle(seed):
    """Random small shared pools (stems of random prefix length, some sequences starting
    inside a block or empty, block sizes 16 / 32 / 64, head dims 64 / 128 / 256, 1 to 16 query
    heads per KV head, spans 0 to 3): every item's partial of every member and the merged
    output against the oracle."""
    rng = np.random.default_rng(9000 + seed)
    bs = int(rng.choice([16, 32, 64]))
    d = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2]))
    group = int(rng.choice([1, 2, 4, 8, 16]))
    nseq, nblk, nstem = int(rng.integers(2, 12)), int(rng.integers(2, 30)), int(rng.integers(1, 3))
    pool_blocks = nstem * nblk + nseq * nblk + 4
    ids = rng.permutation(pool_blocks).astype(np.int32)
    table = np.full((nseq, nblk), -1, np.int32)
    lens, begins, pos = [], [], nstem * nblk
    for s in range(nseq):
        nb = int(rng.integers(1, nblk + 1))
        k = int(rng.integers(0, nb + 1))
        stem = int(rng.integers(0, nstem))
        table[s, :k] = ids[stem * nblk:stem * nblk + k]
        table[s, k:nb] = ids[pos:pos + nb - k]
        pos += nb - k
        length = nb * bs - int(rng.integers(0, bs))
        r = rng.random()
        lens.append(length)
        begins.append(0 if r < 0.7 else (int(rng.integers(0, length + 1)) if r < 0.95 else length))
    parts = bs * int(rng.choice([1, 2, 4]))
    span = int(rng.integers(0, 4))
    case = _custom_case(bs, hkv, d, hkv * group, table, lens, begins, parts, pool_blocks, 1200 + seed)
    _say(f"[plan-rand] seed={seed} bs={bs} d={d} hkv={hkv} group={group} nseq={nseq} span={span}")
    dc, o, lse = _run_plan(case, span_parts=span)
    assert int(dc.step.err.item()) == 0
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    worst = _check_items(case, dc)
    _say(f"[plan-rand] out error {err:.3e}, worst item {worst:.3e}")
    assert err <= oc.out_tol(case)
    live = np.asarray(lens) > np.asarray(begins)
    assert float(np.max(np.abs(lse[live] - lse_ref[live]))) <= oc.lse_tol(case)
    assert np.isneginf(lse[~live]).all() and (o[~live] == 0).all()


@pytest.mark.parametrize("d,hq,hkv", [(256, 16, 2), (128, 32, 4)])
def test_shared_prefix_decode_session_with_appends(d, hq, hkv):
    """A serving loop over a pool with a shared prefix: eight sequences take the same first
    blocks from the pool's ref-counted block table, the prefix is written once and each
    sequence's own tokens through the append kernel, and each step appends one token to every
    sequence, builds a new plan (the shared ranges staged: eight sharers at eight heads per KV
    head fill four waves) and decodes; every step matches the oracle's attention over each
    sequence's whole history."""
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.api import DecodeStep, Pool, append_kv
    from synth import bf16_round_bits
    rng = np.random.default_rng(31 + d)
    B, bs, S, steps = 8, 16, 40, 3                     # S shared blocks (640 tokens)
    own = [int(x) for x in rng.integers(0, 90, B)]
    final = [S * bs + own[b] + steps for b in range(B)]
    max_blocks = -(-max(final) // bs)
    nblocks = S + B * (max_blocks - S) + 4
    nel = 2 * hkv * bs * d
    region = torch.zeros(nblocks * nel, dtype=torch.int16, device="cuda")
    pool = Pool(bs, hkv, d, d, "bf16", False, [(region.data_ptr(), nblocks)], seed=3)
    st, table, _ = pool.block_table(final, max_blocks, share_src=[-1] + [0] * (B - 1),
                                    share_nblocks=[0] + [S] * (B - 1))
    assert st == 0 and pool.shared_blocks > 0
    table_dev = torch.from_numpy(table).cuda()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")

    def tokens(n):
        k = bf16_round_bits(rng.standard_normal((n, hkv, d), dtype=np.float32))
        v = bf16_round_bits(rng.standard_normal((n, hkv, d), dtype=np.float32))
        return k, v

    def write(b, k, v, pos):
        kd = torch.from_numpy(k[None].view(np.int16)).cuda()
        vd = torch.from_numpy(v[None].view(np.int16)).cuda()
        p = torch.tensor([pos], dtype=torch.int32, device="cuda")
        append_kv(pool, kd, vd, _lib.BF16, table_dev[b:b + 1], max_blocks, p, err)

    pk, pv = tokens(S * bs)                            # the prefix, written once (by sequence 0)
    write(0, pk, pv, 0)
    hist = []
    for b in range(B):
        k, v = tokens(own[b])
        if own[b]:
            write(b, k, v, S * bs)
        hist.append([np.concatenate([pk, k]), np.concatenate([pv, v])])
    scale = 1.0 / np.sqrt(float(d))
    for step in range(steps):
        for b in range(B):
            k, v = tokens(1)
            write(b, k, v, len(hist[b][0]))
            hist[b] = [np.concatenate([hist[b][0], k]), np.concatenate([hist[b][1], v])]
        lens = np.array([len(h[0]) for h in hist], np.int32)
        cur = table.copy()
        for b in range(B):
            cur[b, -(-int(lens[b]) // bs):] = -1
        dstep = DecodeStep(pool, cur, lens, [bs * 4] * B, hq, d)
        assert dstep.plan is not None
        q = bf16_round_bits(rng.standard_normal((B, hq, d), dtype=np.float32))
        o, lse = dstep.run(torch.from_numpy(q.view(np.int16)).cuda(), _lib.BF16, scale)
        torch.cuda.synchronize()
        assert int(err.item()) == 0 and int(dstep.err.item()) == 0
        o, lse = o.cpu().numpy(), lse.cpu().numpy()
        _, _, items, _ = parse(dstep.plan, B)
        qf = oracle.bf16_bits_to_f64(q)
        worst = 0.0
        for b in range(B):
            o_ref, lse_ref = oracle.attend(qf[b], oracle.bf16_bits_to_f64(hist[b][0]),
                                           oracle.bf16_bits_to_f64(hist[b][1]), scale)
            e = float(np.max(np.abs(o[b] - o_ref))) / float(np.max(np.abs(o_ref)))
            worst = max(worst, e)
            assert e <= oc.BF16_REL_TOL, (step, b, e)
            assert float(np.max(np.abs(lse[b] - lse_ref))) <= oc.LSE_ABS_TOL, (step, b)
        _say(f"[session] d={d} step {step}: modes {sorted(set(items[items[:, 3] > 0, 5].tolist()))}, "
             f"worst {worst:.2e}")
        assert (items[:, 5] == 2).any()
