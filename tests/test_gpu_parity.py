"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Tolerances (written here, applied element by element): bf16 caches with fp32 accumulation
max |o_gpu - o_ref| / max |o_ref| <= 2e-3; fp32 caches max |o_gpu - o_ref| <= 1e-5; lse
within 2e-3 (bf16) / 1e-5 (fp32).  Partition counts and address resolution are compared
bit for bit, and relabelling physical blocks must leave the GPU output bitwise unchanged.
"""

import os
import sys

import numpy as np
import pytest

import oracle
from synth import make_case
from tests import oracle_cases as oc

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
    _lib.load()                      # fails loudly if the library is not built
    torch.cuda.set_device(0)


def _run(case, ext=None, group_parts=1):
    from paged_kv_cache_mla_amd.session import DeviceCase
    dc = DeviceCase(case, group_parts=group_parts)
    o_ext = lse_ext = None
    if ext is not None:
        o_ext = torch.from_numpy(ext[0].astype(np.float32)).cuda()
        lse_ext = torch.from_numpy(ext[1].astype(np.float32)).cuda()
    o, lse = dc.run(o_ext, lse_ext)
    torch.cuda.synchronize()
    return dc, o.cpu().numpy(), lse.cpu().numpy()


def _check_partials(case, dc, seqs=None, group_parts=1):
    parts = oc.grouped_partials(case, group_parts, seqs)
    nparts = dc.step.nparts.cpu().numpy()
    o_part = dc.step.o_part.cpu().numpy()
    l_part = dc.step.lse_part.cpu().numpy()
    for idx, b in enumerate(range(case.batch) if seqs is None else seqs):
        beg = 0 if case.tok_begin is None else int(case.tok_begin[b])
        count = oracle.partition_count(int(case.ctx_lens[b]), beg, int(case.part_tokens[b]))
        assert nparts[b] == -(-count // group_parts)
        po, pl = parts[idx]
        n = po.shape[0]
        if n == 0:
            continue
        ref_scale = float(np.max(np.abs(po))) if case.dtype == "bf16" else 1.0
        err = float(np.max(np.abs(o_part[b, :, :n, :].transpose(1, 0, 2) - po))) / ref_scale
        assert err <= oc.out_tol(case), (b, err)
        assert float(np.max(np.abs(l_part[b, :, :n].T - pl))) <= oc.lse_tol(case)


SMALL = ["tiny_fp32", "gqa_32k", "split_128k", "prefix_shared", "mla_16k"]


@pytest.mark.parametrize("name", SMALL)
def test_small_workload_matches_oracle(name):
    case = make_case(name, "small")
    _say(f"[parity] {name} small B={case.batch} L={case.ctx_lens.tolist()}")
    ext = oc.external_partial(case) if case.ext_regions is not None else None
    dc, o, lse = _run(case, ext)
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    _say(f"[parity] {name}: out error {err:.3e} (tol {oc.out_tol(case)})")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0
    _check_partials(case, dc)


GROUPED = [("gqa_32k", 2), ("gqa_32k", 3), ("gqa_32k", 4), ("gqa_32k", 8), ("gqa_32k", 16), ("prefix_shared", 4),
           ("prefix_shared", 7), ("split_128k", 4), ("mla_16k", 3), ("tiny_fp32", 2)]


@pytest.mark.parametrize("name,group_parts", GROUPED, ids=[f"{n}-g{g}" for n, g in GROUPED])
def test_grouped_partials_match_oracle(name, group_parts):
    """Partials of group_parts consecutive partitions merged on chip (one wave per partition
    and an LDS merge in the matrix-core kernel; an in-order walk elsewhere) equal the oracle's
    merge of those partitions' partials; the final output is unchanged."""
    case = make_case(name, "small")
    _say(f"[grouped] {name} group_parts={group_parts}")
    ext = oc.external_partial(case) if case.ext_regions is not None else None
    dc, o, lse = _run(case, ext, group_parts)
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    _say(f"[grouped] {name} g{group_parts}: out error {err:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0
    _check_partials(case, dc, group_parts=group_parts)


GEOMETRIES = [  # block size, KV heads, head dim, q heads, partition blocks, group_parts
    (32, 2, 128, 16, 2, 1), (32, 4, 64, 8, 3, 4), (64, 2, 64, 32, 2, 8),
    (64, 1, 256, 4, 1, 2), (128, 2, 128, 8, 1, 4), (256, 1, 128, 16, 1, 2),
    (256, 2, 256, 2, 1, 1), (16, 8, 64, 128, 4, 16)]


@pytest.mark.parametrize("bs,hkv,d,hq,pblocks,group_parts", GEOMETRIES,
                         ids=[f"bs{g[0]}-hkv{g[1]}-d{g[2]}-hq{g[3]}-g{g[5]}" for g in GEOMETRIES])
def test_matrix_core_kernel_block_sizes_and_head_dims(bs, hkv, d, hq, pblocks, group_parts):
    """The matrix-core GQA kernel at every block size it is built for (16 .. 256), head dims
    64 / 128 / 256 and 1 .. 16 query heads per KV head, with ragged lengths (one token, a
    partial last block, a start inside a block), against the oracle element by element."""
    from synth import gqa_case
    lens = [bs * 5 + 3, 1, bs * 11, 2 * bs - 1, bs * 3 + bs // 2]
    begin = [0, 0, bs // 2 + 1, 0, bs]
    case = gqa_case(bs, hkv, d, hq, lens, [bs * pblocks] * len(lens), tok_begin=begin)
    _say(f"[geometry] bs={bs} hkv={hkv} d={d} hq={hq} P={bs * pblocks} group_parts={group_parts}")
    dc, o, lse = _run(case, None, group_parts)
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    _say(f"[geometry] out error {err:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0
    _check_partials(case, dc, group_parts=group_parts)


EXTREMES = [  # lengths, tok_begin, group_parts
    ([131072, 100001], [0, 777], 16),     # 256 and 194 partitions, groups of 16
    ([512] * 255 + [7], None, 1),        # 256 sequences, one partition each
]


@pytest.mark.parametrize("lens,begin,group_parts", EXTREMES, ids=["long-128K-g16", "batch-256-g1"])
def test_extreme_launch_shapes(lens, begin, group_parts):
    """The Qwen3-30B-A3B GQA shape at the ends of its launch space: two 100K+ contexts in the
    largest groups (grids of few workgroups, long on-chip merges), and 256 short sequences
    (grids of many tiny workgroups), against the oracle."""
    from synth import gqa_case
    case = gqa_case(16, 4, 128, 32, lens, [512] * len(lens), tok_begin=begin, seed=1011)
    _say(f"[extreme] B={case.batch} max L={max(lens)} group_parts={group_parts}")
    dc, o, lse = _run(case, None, group_parts)
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    _say(f"[extreme] out error {err:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0


SMALL_BLOCKS = [  # block size, KV heads, head dim, q heads, dtype, group_parts
    (1, 2, 64, 8, "f32", 1), (2, 1, 128, 4, "bf16", 3), (4, 2, 64, 4, "f32", 2),
    (8, 4, 128, 16, "bf16", 4), (8, 1, 256, 16, "f32", 1), (64, 2, 64, 8, "f32", 2)]


@pytest.mark.parametrize("bs,hkv,d,hq,dtype,group_parts", SMALL_BLOCKS,
                         ids=[f"bs{g[0]}-d{g[2]}-{g[4]}-g{g[5]}" for g in SMALL_BLOCKS])
def test_generic_kernel_block_sizes(bs, hkv, d, hq, dtype, group_parts):
    """Block sizes below the matrix-core kernel's 16 tokens, and fp32 caches, go to the plain
    VALU kernel: block sizes 1 .. 8 and 64, head dims 64 .. 256, fp32 and bf16, against the
    oracle, partials included."""
    from synth import gqa_case
    lens = [37, 1, 130, 64 + 5]
    begin = [0, 0, 3, 16]
    pt = max(bs, 16) * 2
    case = gqa_case(bs, hkv, d, hq, lens, [pt] * len(lens), tok_begin=begin, dtype=dtype)
    _say(f"[generic] bs={bs} d={d} {dtype} hq={hq} hkv={hkv} group_parts={group_parts}")
    dc, o, lse = _run(case, None, group_parts)
    o_ref, lse_ref = oc.full_reference(case)
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0
    _check_partials(case, dc, group_parts=group_parts)


HEAD_COUNTS = [(1, "f32", 64), (3, "f32", 128), (5, "bf16", 64), (12, "f32", 256), (7, "bf16", 128)]


@pytest.mark.parametrize("group,dtype,d", HEAD_COUNTS, ids=[f"g{g}-{t}-d{d}" for g, t, d in HEAD_COUNTS])
def test_generic_kernel_head_counts(group, dtype, d):
    """The VALU kernel is built for 1, 2, 4, 8 or 16 query heads per KV head; other counts run
    in the next size up, with zero queries in the padding heads, which are never written.
    Counts 1, 3, 5, 7 and 12 (block size 8 for bf16, so that the VALU kernel serves it) against
    the oracle, partials included, with ragged lengths over a full 64-token chunk."""
    from synth import gqa_case
    bs = 16 if dtype == "f32" else 8
    hkv = 2
    lens = [37, 1, 200, 64 + 5]
    begin = [0, 0, 3, 16]
    case = gqa_case(bs, hkv, d, hkv * group, lens, [96] * len(lens), tok_begin=begin, dtype=dtype)
    _say(f"[generic heads] group={group} {dtype} d={d}")
    dc, o, lse = _run(case, None, 2)
    o_ref, lse_ref = oc.full_reference(case)
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0
    _check_partials(case, dc, group_parts=2)


@pytest.mark.parametrize("hq", [1, 5, 8])
def test_mla_fewer_heads(hq):
    """Latent-cache decode with fewer than the 16 heads an MFMA tile holds: the unused head
    columns are zero in the operands and never written."""
    from synth import mla_case
    case = mla_case([1000, 64, 333], [256] * 3, tok_begin=[0, 0, 70], num_q_heads=hq)
    _say(f"[mla heads] hq={hq}")
    dc, o, lse = _run(case, None, 2)
    o_ref, lse_ref = oc.full_reference(case)
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0
    _check_partials(case, dc, group_parts=2)


@pytest.mark.parametrize("group_parts", [1, 3])
def test_mla_split_with_external_partial(group_parts):
    """A latent-cache layer split as the pages split a sequence between engines: the oldest
    tokens [0, begin) are a partial computed elsewhere (the oracle's, here), the device decodes
    [begin, L) and the merge folds the external partial in (the 512-wide wave merge with an
    external term).  Split points on and inside block boundaries; the result must be the
    unsplit attention over [0, L)."""
    from synth import mla_case
    lens = [3000, 1000, 64 * 20 + 7, 700]
    begins = [1024, 512, 64 * 7 + 5, 699]
    case = mla_case(lens, [256] * len(lens))
    o_ref, lse_ref = oc.full_reference(case)            # the whole context, unsplit
    lay, qf = oc.layout_of(case), oc.q_f64(case)
    o_x = np.zeros((case.batch, case.num_q_heads, case.head_dim_v))
    l_x = np.zeros((case.batch, case.num_q_heads))
    for b, beg in enumerate(begins):
        k, v = oracle.gather_sequence(lay, case.regions, case.region_blocks, case.table[b], 0, beg)
        o_x[b], l_x[b] = oracle.attend(qf[b], k, v, case.scale)
    case.tok_begin = np.array(begins, np.int32)
    _say(f"[mla split] L={lens} begin={begins} group_parts={group_parts}")
    dc, o, lse = _run(case, (o_x, l_x), group_parts)
    err = oc.out_error(case, o, o_ref)
    _say(f"[mla split] out error {err:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0


def test_long_mla_groups_cross_block_id_windows():
    """Latent-cache groups longer than the 128 stages (64-token blocks) whose block ids the
    kernel holds in registers at a time: a group of 257 stages starting mid-block (two full
    windows and a one-stage window), a group of exactly 128 stages followed by a short one,
    and a short sequence, each against the oracle."""
    from synth import mla_case
    case = mla_case([20000, 64 * 130 + 5, 777], [8192, 4096, 512], tok_begin=[37, 0, 100])
    _say(f"[mla windows] L={case.ctx_lens.tolist()} P={case.part_tokens.tolist()} group_parts=2")
    dc, o, lse = _run(case, None, 2)
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    _say(f"[mla windows] out error {err:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0
    _check_partials(case, dc, group_parts=2)


@pytest.mark.parametrize("part,group_parts", [(640, 1), (192, 2), (128, 3)])
def test_mla_team_split_over_stage_counts(part, group_parts):
    """The latent-cache kernel gives a group's even 64-token stages to one team of waves and
    the odd ones to the other, and merges the two teams at the end.  Groups of 1 to 10 stages
    (so the second team has nothing, as many stages, or one fewer), starting at, just after
    and just before block boundaries, against the oracle and partial by partial."""
    from synth import mla_case
    lens = [1, 67, 191, 256, 300, 400, 448, 512, 542, 640]     # 1 .. 10 stages
    begin = [0, 3, 63, 10, 20, 100, 0, 0, 30, 0]
    case = mla_case(lens, [part] * len(lens), tok_begin=begin)
    _say(f"[mla teams] L={lens} begin={begin} P={part} group_parts={group_parts}")
    dc, o, lse = _run(case, None, group_parts)
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    _say(f"[mla teams] out error {err:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0
    _check_partials(case, dc, group_parts=group_parts)


def _poison_unused_slots(case):
    """A copy of `case` whose pool holds NaN bit patterns in every token slot that no
    sequence's range [tok_begin, L) uses: the tails of last blocks, the slots before
    tok_begin, and blocks no table names.  The oracle never reads those slots."""
    import dataclasses
    lay = oc.layout_of(case)
    bs, x = case.block_size, lay.chunk
    total = sum(case.region_blocks)
    used = np.zeros((total, bs), bool)
    for b in range(case.batch):
        beg = 0 if case.tok_begin is None else int(case.tok_begin[b])
        t = np.arange(beg, int(case.ctx_lens[b]))
        used[case.table[b, t // bs], t % bs] = True
    # token slot of every element of a block, from the block layout
    if case.latent:
        slot = np.broadcast_to(np.arange(bs)[None, :, None], (case.head_dim_k // x, bs, x)).ravel()
    else:
        hkv, dk, dv = case.num_kv_heads, case.head_dim_k, case.head_dim_v
        slot = np.concatenate([
            np.broadcast_to(np.arange(bs)[None, None, :, None], (hkv, dk // x, bs, x)).ravel(),
            np.broadcast_to(np.arange(bs)[None, None, :], (hkv, dv, bs)).ravel()])
    nan = np.uint16(0x7FC0) if case.dtype == "bf16" else np.float32(np.nan)
    regions, first = [], 0
    for reg, n in zip(case.regions, case.region_blocks):
        r = reg.copy().reshape(n, -1)
        for i in range(n):
            r[i, ~used[first + i][slot]] = nan
        regions.append(r.reshape(-1))
        first += n
    return dataclasses.replace(case, regions=regions)


@pytest.mark.parametrize("name,group_parts", [("gqa_32k", 1), ("gqa_32k", 3), ("gqa_32k", 16),
                                              ("mla_16k", 1), ("mla_16k", 3), ("split_128k", 4),
                                              ("tiny_fp32", 1)])
def test_nan_in_unused_token_slots_is_ignored(name, group_parts):
    """Token slots outside every sequence's range may hold anything (a slot never written, a
    stale block): NaN bit patterns there must not reach the output, although the kernels
    read whole tiles and give those tokens zero weight."""
    case = _poison_unused_slots(make_case(name, "small"))
    _say(f"[poison] {name} group_parts={group_parts}")
    ext = oc.external_partial(case) if case.ext_regions is not None else None
    dc, o, lse = _run(case, ext, group_parts)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    o_ref, lse_ref = oc.full_reference(case)
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)
    assert int(dc.step.err.item()) == 0


@pytest.mark.parametrize("name", ["gqa_32k", "prefix_shared", "split_128k"])
def test_generic_kernel_matches_oracle(name, monkeypatch):
    monkeypatch.setenv("KVATTN_FORCE_GENERIC", "1")
    case = make_case(name, "small")
    ext = oc.external_partial(case) if case.ext_regions is not None else None
    _, o, lse = _run(case, ext)
    o_ref, lse_ref = oc.full_reference(case)
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)


@pytest.mark.parametrize("name", ["gqa_32k", "mla_16k", "prefix_shared"])
def test_deterministic_bitwise(name):
    case = make_case(name, "small")
    from paged_kv_cache_mla_amd.session import DeviceCase
    dc = DeviceCase(case)
    o1, l1 = (t.clone() for t in dc.run())
    o2, l2 = dc.run()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_interleaved_steps_keep_their_own_buffers():
    """Two decode steps alive at once, their calls interleaved, with q passed as fresh tensors
    and changed in place between calls: each step reads and writes only its own buffers (the
    step object converts its fixed arguments once), and each result equals the oracle's for
    the q it was given."""
    from paged_kv_cache_mla_amd.session import DeviceCase
    ca, cb = make_case("gqa_32k", "small"), make_case("mla_16k", "small")
    da, db = DeviceCase(ca), DeviceCase(cb)
    ref_a = oc.full_reference(ca)
    ref_b = oc.full_reference(cb)
    qa0 = da.q.clone()
    qa_rev = da.q.flip(0).contiguous()
    ref_a_rev = oc.full_reference(_with_q(ca, np.ascontiguousarray(ca.q[::-1])))
    for i in range(3):
        if i == 0:
            q = qa0.clone()            # a fresh tensor
        else:
            da.q.copy_(qa_rev if i == 1 else qa0)   # the same tensor, changed in place
            q = da.q
        da.step.partial(q, da.q_dtype, ca.scale)
        db.run()
        da.step.merge()
        torch.cuda.synchronize()
        want_a = ref_a_rev if i == 1 else ref_a
        assert oc.out_error(ca, da.step.o_out.cpu().numpy(), want_a[0]) <= oc.out_tol(ca), i
        assert oc.out_error(cb, db.step.o_out.cpu().numpy(), ref_b[0]) <= oc.out_tol(cb), i
    assert int(da.step.err.item()) == 0 and int(db.step.err.item()) == 0


def _with_q(case, q):
    import copy
    c2 = copy.copy(case)
    c2.q = q
    return c2


def _relabelled(case, seed):
    """Same logical content, every physical block moved to a new random slot (across
    regions), tables rewritten accordingly."""
    import copy
    rng = np.random.default_rng(seed)
    total = sum(case.region_blocks)
    new_of_old = rng.permutation(total)
    per = case.elems_per_block()
    flat = np.concatenate(case.regions)
    moved = np.empty_like(flat)
    for old in range(total):
        new = new_of_old[old]
        moved[new * per:(new + 1) * per] = flat[old * per:(old + 1) * per]
    c2 = copy.copy(case)
    bounds = np.cumsum([0] + list(case.region_blocks))
    c2.regions = [moved[bounds[r] * per:bounds[r + 1] * per] for r in range(len(case.region_blocks))]
    t = case.table.copy()
    t[t >= 0] = new_of_old[t[t >= 0]]
    c2.table = t
    return c2


@pytest.mark.parametrize("name", ["gqa_32k", "prefix_shared", "mla_16k", "tiny_fp32"])
def test_physical_relabelling_is_bitwise_invisible(name):
    case = make_case(name, "small")
    _, o1, l1 = _run(case)
    _, o2, l2 = _run(_relabelled(case, 11))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _unshared(case):
    """Same logical content with every shared block given its own physical copy per table
    entry: the pool then holds no shared blocks."""
    import copy
    per = case.elems_per_block()
    flat = np.concatenate(case.regions)
    ids = case.table[case.table >= 0]
    c2 = copy.copy(case)
    c2.regions = [np.concatenate([flat[int(i) * per:(int(i) + 1) * per] for i in ids])]
    c2.region_blocks = [int(ids.size)]
    t = np.full_like(case.table, -1)
    t[case.table >= 0] = np.arange(ids.size, dtype=np.int32)
    c2.table = t
    return c2


def test_shared_and_unshared_prefix_give_bitwise_equal_output():
    """Pools with shared blocks are read with cache-retaining loads, others with streaming
    loads; the arithmetic is the same, so unsharing the prefixes changes no bit."""
    case = make_case("prefix_shared", "small")
    dc1, o1, l1 = _run(case)
    dc2, o2, l2 = _run(_unshared(case))
    assert dc1.pool.shared_blocks > 0 and dc2.pool.shared_blocks == 0
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", ["prefix_shared", "mla_16k", "split_128k", "tiny_fp32"])
def test_resolution_offsets_bitwise(name):
    from paged_kv_cache_mla_amd.api import resolve_offsets
    from paged_kv_cache_mla_amd.session import DeviceCase
    case = make_case(name, "small")
    dc = DeviceCase(case)
    max_tokens = case.max_blocks * case.block_size
    reg = torch.empty((case.batch, max_tokens), dtype=torch.int32, device="cuda")
    off = torch.empty((case.batch, max_tokens), dtype=torch.int64, device="cuda")
    ctx_dev = torch.from_numpy(case.ctx_lens).cuda()
    resolve_offsets(dc.pool, dc.step.table_dev, case.max_blocks, ctx_dev, max_tokens, reg, off)
    torch.cuda.synchronize()
    want_r, want_o = oracle.resolve_offsets_reference(oc.layout_of(case), case.region_blocks,
                                                      case.table, case.ctx_lens, max_tokens)
    assert np.array_equal(reg.cpu().numpy(), want_r)
    assert np.array_equal(off.cpu().numpy(), want_o)


def test_one_token_context_returns_value_exactly():
    case = make_case("gqa_32k", "small")
    case.ctx_lens = np.array([1, 16, 17, 600], np.int32)
    nb = [1, 1, 2, 38]
    t = case.table.copy()
    for b in range(case.batch):
        t[b, nb[b]:] = -1
    case.table = t
    dc, o, lse = _run(case)
    lay = oc.layout_of(case)
    k, v = oracle.gather_sequence(lay, case.regions, case.region_blocks, case.table[0], 0, 1)
    g = case.num_q_heads // case.num_kv_heads
    for h in range(case.num_q_heads):
        assert np.array_equal(o[0, h].astype(np.float64), v[0, h // g])      # bit-exact value
    o_ref, _ = oc.full_reference(case)
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)


def test_empty_device_range_returns_external_partial():
    case = make_case("split_128k", "small")
    case.tok_begin = case.ctx_lens.copy()             # the whole context lives elsewhere
    rng = np.random.default_rng(3)
    o_ext = rng.standard_normal((case.batch, case.num_q_heads, case.head_dim_v)).astype(np.float32)
    l_ext = rng.standard_normal((case.batch, case.num_q_heads)).astype(np.float32)
    dc, o, lse = _run(case, (o_ext, l_ext))
    assert (dc.step.nparts.cpu().numpy() == 0).all()
    assert np.allclose(o, o_ext, rtol=0, atol=1e-6) and np.allclose(lse, l_ext, rtol=0, atol=1e-6)


def test_invalid_block_id_is_flagged_not_read():
    from paged_kv_cache_mla_amd import _lib
    case = make_case("gqa_32k", "small")
    from paged_kv_cache_mla_amd.session import DeviceCase
    dc = DeviceCase(case)
    bad = dc.table.copy()
    bad[0, 3] = sum(case.region_blocks) + 5           # out of range inside sequence 0's span
    dc.step.table_dev.copy_(torch.from_numpy(bad))
    dc.run()
    torch.cuda.synchronize()
    assert int(dc.step.err.item()) & _lib.ERR_BAD_BLOCK


INVALID_PARTITIONS = [  # workload, sequence, first tokens made invalid, group_parts
    ("gqa_32k", 0, 512, 1), ("gqa_32k", 0, 1024, 4), ("gqa_32k", 0, 512, 2),
    ("mla_16k", 0, 256, 1), ("mla_16k", 0, 512, 3), ("tiny_fp32", 1, 144, 1)]


@pytest.mark.parametrize("name,b,ntok,group_parts", INVALID_PARTITIONS,
                         ids=[f"{n}-{t}-g{g}" for n, _, t, g in INVALID_PARTITIONS])
def test_partition_of_invalid_blocks_contributes_nothing(name, b, ntok, group_parts):
    """Every block of a sequence's first partitions (one or two waves' whole ranges) is an
    invalid id: the error bit is set, those blocks contribute nothing, no 0/0 reaches a
    partial (o = 0 beside lse = -inf), and the output is the attention over the remaining
    tokens."""
    from paged_kv_cache_mla_amd import _lib
    from paged_kv_cache_mla_amd.session import DeviceCase
    case = make_case(name, "small")
    good = case.table
    bad = good.copy()
    bad[b, :ntok // case.block_size] = sum(case.region_blocks) + 7
    _say(f"[invalid] {name} seq {b}: first {ntok} tokens in invalid blocks, group_parts {group_parts}")
    dc = DeviceCase(case, group_parts=group_parts)     # the pool admits only valid tables:
    dc.step.table_dev.copy_(torch.from_numpy(bad))     # the invalid ids go to the device copy
    o, lse = dc.run()
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert int(dc.step.err.item()) & _lib.ERR_BAD_BLOCK
    o_part = dc.step.o_part.cpu().numpy()
    l_part = dc.step.lse_part.cpu().numpy()
    n = int(dc.step.nparts.cpu().numpy()[b])
    assert np.isfinite(o_part[b, :, :n]).all()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    lay = oc.layout_of(case)
    k, v = oracle.gather_sequence(lay, case.regions, case.region_blocks, good[b], ntok,
                                  int(case.ctx_lens[b]))
    o_ref, lse_ref = oc.full_reference(case)
    o_ref[b], lse_ref[b] = oracle.attend(oc.q_f64(case)[b], k, v, case.scale)
    if group_parts == 1:
        dead = ntok // int(case.part_tokens[b])
        assert np.isneginf(l_part[b, :, :dead]).all() and (o_part[b, :, :dead] == 0).all()
    err = oc.out_error(case, o, o_ref)
    _say(f"[invalid] out error {err:.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)


# ---------------------------------------------------------------- full sizes, every sequence
FULL = [("gqa_32k", {}), ("mla_16k", {}), ("split_128k", {"r": 0.25}), ("split_128k", {"r": 0.5}),
        ("split_128k", {"r": 0.75}), ("prefix_shared", {})]


@pytest.mark.parametrize("name,kw", FULL, ids=[f"{n}-{k.get('r', '')}" for n, k in FULL])
def test_full_size_every_sequence(name, kw):
    """Full-size workloads in the launch configuration bench.py times (group_parts chosen by
    the library), every sequence and head against the oracle (the split layer's host share
    from the oracle too)."""
    _say(f"[full] generating {name} {kw}")
    case = make_case(name, "full", **kw)
    ext = oc.external_partial(case) if case.ext_regions is not None else None
    _say(f"[full] running {name} B={case.batch} device tokens={case.device_tokens()}")
    dc, o, lse = _run(case, ext, 0)
    group_parts = dc.step.group_parts
    _say(f"[full] {name} ran with group_parts {group_parts} (library choice)"
         + (f", from a plan of {dc.step.n_groups} workgroups" if dc.step.plan is not None else ""))
    assert int(dc.step.err.item()) == 0
    nparts = dc.step.nparts.cpu().numpy()
    if dc.step.plan is not None:          # a pool with shared blocks runs its plan
        from tests.test_plan_cpu import parse
        assert np.array_equal(nparts, parse(dc.step.plan, case.batch)[1])
    for b in range(case.batch if dc.step.plan is None else 0):
        beg = 0 if case.tok_begin is None else int(case.tok_begin[b])
        count = oracle.partition_count(int(case.ctx_lens[b]), beg, int(case.part_tokens[b]))
        assert nparts[b] == -(-count // group_parts)
    o_ref, lse_ref = oc.full_reference(case)
    err = oc.out_error(case, o, o_ref)
    # the worst (sequence, head) row against its own scale, reported beside the bound
    rows = np.max(np.abs(o.astype(np.float64) - o_ref), axis=2)
    if case.dtype == "bf16":
        rows = rows / np.max(np.abs(o_ref), axis=2)
    wb, wh = np.unravel_index(int(np.argmax(rows)), rows.shape)
    _say(f"[full] {name} {kw} all {case.batch} sequences: out error {err:.3e}, worst row "
         f"(b={wb}, h={wh}) {rows[wb, wh]:.3e}, lse error {float(np.max(np.abs(lse - lse_ref))):.3e}")
    assert err <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)


# ---------------------------------------------------------------- native host share, merged
HOST_THREADS = min(16, len(os.sched_getaffinity(0)))


def _split_step(case, group_parts):
    from paged_kv_cache_mla_amd.api import HostShare
    from paged_kv_cache_mla_amd.session import DeviceCase, SplitStep
    dc = DeviceCase(case, group_parts=group_parts)
    hs = HostShare(case.block_size, case.num_kv_heads, case.head_dim_k, case.head_dim_v,
                   case.dtype, case.latent, case.ext_regions, case.num_q_heads, case.scale,
                   case.ext_table, case.tok_begin, n_threads=HOST_THREADS)
    return dc, SplitStep(dc.step, dc.q, dc.q_dtype, case.scale, hs)


@pytest.mark.parametrize("variant,kw,seqs,group_parts", [
    ("small", {}, None, 1), ("small", {"r": 0.25}, None, 4),
    ("full", {"r": 0.5}, [0, 3], 8)])
def test_split_step_with_native_host_share(variant, kw, seqs, group_parts):
    """The CPU share computed by kvattn_host_partial while the device computes its own, then
    merged on the device straight from mapped host memory: every step of a back-to-back run
    with changing queries matches the oracle, and repeating a query repeats the bits."""
    import copy

    from synth.workloads import bf16_round_bits
    _say(f"[split-step] {variant} {kw} group_parts={group_parts}")
    case = make_case("split_128k", variant, **kw)
    dc, ss = _split_step(case, group_parts)
    # four steps back to back, each with its own q (both mapped buffers are used twice, so a
    # stale host partial would show), then the first q again
    rng = np.random.default_rng(7)
    qs = [case.q] + [bf16_round_bits(rng.standard_normal(case.q.shape, dtype=np.float32))
                     for _ in range(3)] + [case.q]
    outs = []
    for q in qs:
        dc.q.copy_(torch.from_numpy(q.view(np.int16)))
        o, lse = ss.run()
        outs.append((o.clone(), lse.clone()))
    torch.cuda.synchronize()
    assert int(dc.step.err.item()) == 0
    assert torch.equal(outs[-1][0], outs[0][0]) and torch.equal(outs[-1][1], outs[0][1])
    sel = list(range(case.batch)) if seqs is None else seqs
    for i, q in enumerate(qs[:-1] if variant == "small" else qs[:2]):
        c = copy.copy(case)
        c.q = q
        o_ref, lse_ref = oc.full_reference(c, seqs)
        o = outs[i][0].cpu().numpy()
        lse = outs[i][1].cpu().numpy()
        err = oc.out_error(case, o[sel], o_ref[sel])
        _say(f"[split-step] step {i} out error {err:.3e}")
        assert err <= oc.out_tol(case)
        assert float(np.max(np.abs(lse[sel] - lse_ref[sel]))) <= oc.lse_tol(case)


# ---------------------------------------------------------------- the two merge kernels
@pytest.mark.parametrize("dv,max_parts", [(64, 1), (64, 32), (128, 4), (128, 16), (128, 32),
                                          (256, 8), (256, 16), (256, 17), (512, 1), (512, 8),
                                          (512, 16), (512, 40)])
@pytest.mark.parametrize("ext", [False, True])
def test_merge_kernels_match_oracle_and_each_other(dv, max_parts, ext):
    """kvattn_merge_lse on random partials (counts from 0 to max_parts, -inf entries) against
    the oracle's float64 merge; narrow heads, and heads of 256 or 512 values with at most 16
    partials, take a wave kernel, the others the workgroup kernel, and forcing the workgroup
    kernel gives the same result within rounding.  Partials of no weight (lse = -inf) carry
    NaN outputs, which must be left out, not multiplied by zero."""
    import os
    from paged_kv_cache_mla_amd.api import merge_lse
    rng = np.random.default_rng(dv * 100 + max_parts + ext)
    B, hq = 5, 6
    o_part = rng.standard_normal((B, hq, max_parts, dv)).astype(np.float32)
    lse = (rng.standard_normal((B, hq, max_parts)) * 3).astype(np.float32)
    lse[rng.random(lse.shape) < 0.15] = -np.inf
    nparts = rng.integers(0, max_parts + 1, B).astype(np.int32)
    nparts[0], nparts[-1] = max_parts, 0
    o_x = rng.standard_normal((B, hq, dv)).astype(np.float32) if ext else None
    l_x = (rng.standard_normal((B, hq)) * 3).astype(np.float32) if ext else None
    if ext:
        l_x[1, 2] = -np.inf
    # a weightless partial's o may be anything: NaN there must not reach the output
    o_part[np.isneginf(lse)] = np.nan
    if ext:
        o_x[np.isneginf(l_x)] = np.nan
    dev = lambda a: None if a is None else torch.from_numpy(a).cuda()  # noqa: E731
    outs = {}
    for kernel in ("auto", "block"):
        if kernel == "block":
            os.environ["KVATTN_MERGE_KERNEL"] = "block"
        try:
            o = torch.empty((B, hq, dv), dtype=torch.float32, device="cuda")
            l = torch.empty((B, hq), dtype=torch.float32, device="cuda")
            merge_lse(dev(o_part), dev(lse), dev(nparts), B, hq, max_parts, dv, o, dev(o_x),
                      dev(l_x), l)
            torch.cuda.synchronize()
            outs[kernel] = (o.cpu().numpy(), l.cpu().numpy())
        finally:
            os.environ.pop("KVATTN_MERGE_KERNEL", None)
    # the oracle's convention for a partial of no weight: o = 0, lse = -inf
    o_part = np.where(np.isneginf(lse)[..., None], 0.0, o_part)
    if ext:
        o_x = np.where(np.isneginf(l_x)[..., None], 0.0, o_x)
    for b in range(B):
        parts_o = [o_part[b, :, p] for p in range(nparts[b])] + ([o_x[b]] if ext else [])
        parts_l = [lse[b, :, p] for p in range(nparts[b])] + ([l_x[b]] if ext else [])
        if not parts_o:
            o_ref, l_ref = np.zeros((hq, dv)), np.full(hq, -np.inf)
        else:
            o_ref, l_ref = oracle.merge(parts_o, parts_l)
        for kernel, (o, l) in outs.items():
            assert np.max(np.abs(o[b] - o_ref)) <= 1e-5 * max(1.0, np.max(np.abs(o_ref))), (kernel, b)
            fin = np.isfinite(l_ref)
            assert np.array_equal(np.isneginf(l[b]), ~fin), (kernel, b)
            assert np.max(np.abs(l[b][fin] - l_ref[fin]), initial=0.0) <= 1e-5, (kernel, b)
    assert np.max(np.abs(outs["auto"][0] - outs["block"][0])) <= 1e-6
