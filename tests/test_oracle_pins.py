"""Pins of the float64 oracle against facts fixed by mathematics and the pages.

Each test checks the oracle against something other than itself: IEEE bit patterns,
closed forms of softmax attention, exactness of the LSE merge ([InplaceKVCache] §5.1:
partials over disjoint ranges merge exactly), a 50-digit brute force, torch's own
attention routine, an element-by-element writer of the documented block layout, and the
per-token KV sizes implied by the KV tables of "Physically Partitioned KVCache Format for
CPU-GPU Load Balancing in MoE Inference" (Table 1, Table 2).
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle
from oracle.layout import Layout, gather_sequence, block_elems

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 widening
def test_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000, 0x4049], np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, -0.0,
            3.140625]
    got = oracle.bf16_bits_to_f64(bits)
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w
    assert math.copysign(1.0, got[5]) == -1.0


# ---------------------------------------------------------------- closed forms
def _rand_qkv(rng, n, hq, hkv, dk, dv):
    return (rng.standard_normal((hq, dk)), rng.standard_normal((n, hkv, dk)),
            rng.standard_normal((n, hkv, dv)))


def test_one_token_returns_value():
    rng = np.random.default_rng(1)
    q, k, v = _rand_qkv(rng, 1, 4, 2, 8, 6)
    o, lse = oracle.attend(q, k, v, 0.3)
    for h in range(4):
        kvh = h // 2
        assert np.array_equal(o[h], v[0, kvh])
        assert lse[h] == pytest.approx(0.3 * float(q[h] @ k[0, kvh]), abs=1e-15)


def test_identical_keys_give_mean_value():
    rng = np.random.default_rng(2)
    n = 37
    q, k, v = _rand_qkv(rng, n, 2, 1, 5, 3)
    k[:] = k[0]
    o, lse = oracle.attend(q, k, v, 0.7)
    for h in range(2):
        s = 0.7 * float(q[h] @ k[0, 0])
        assert np.allclose(o[h], v[:, 0].mean(axis=0), atol=1e-14, rtol=0)
        assert lse[h] == pytest.approx(s + math.log(n), abs=1e-13)


def test_zero_query_gives_mean_value():
    rng = np.random.default_rng(3)
    _, k, v = _rand_qkv(rng, 20, 4, 4, 8, 8)
    o, lse = oracle.attend(np.zeros((4, 8)), k, v, 1.0)
    for h in range(4):
        assert np.allclose(o[h], v[:, h].mean(axis=0), atol=1e-14, rtol=0)
        assert lse[h] == pytest.approx(math.log(20), abs=1e-14)


def test_two_tokens_sigmoid_form():
    rng = np.random.default_rng(4)
    q, k, v = _rand_qkv(rng, 2, 3, 1, 7, 4)
    o, lse = oracle.attend(q, k, v, 0.5)
    for h in range(3):
        s0 = 0.5 * float(q[h] @ k[0, 0])
        s1 = 0.5 * float(q[h] @ k[1, 0])
        sig = lambda x: 1.0 / (1.0 + math.exp(-x))  # noqa: E731
        want = sig(s0 - s1) * v[0, 0] + sig(s1 - s0) * v[1, 0]
        assert np.allclose(o[h], want, atol=1e-14, rtol=0)
        assert lse[h] == pytest.approx(np.logaddexp(s0, s1), abs=1e-14)


def test_empty_range_is_weightless():
    o, lse = oracle.attend(np.ones((2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 3)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    rng = np.random.default_rng(5)
    q, k, v = _rand_qkv(rng, 9, 2, 1, 4, 3)
    full = oracle.attend(q, k, v, 1.0)
    m = oracle.merge([o, full[0]], [lse, full[1]])
    assert np.allclose(m[0], full[0], atol=1e-15) and np.allclose(m[1], full[1], atol=1e-15)
    allempty = oracle.merge([o, o], [lse, lse])
    assert np.all(allempty[0] == 0) and np.all(np.isneginf(allempty[1]))


# ---------------------------------------------------------------- merge exactness
@pytest.mark.parametrize("seed", range(6))
def test_merge_of_any_split_equals_unsplit(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 300))
    hq, hkv = [(4, 1), (8, 2), (16, 16), (6, 3)][seed % 4]
    q, k, v = _rand_qkv(rng, n, hq, hkv, 16, 12)
    q *= 2.0                        # spread the scores so the partials differ in scale
    full_o, full_l = oracle.attend(q, k, v, 0.25)
    ncut = int(rng.integers(0, 8))
    cuts = sorted(rng.integers(0, n + 1, size=ncut).tolist())
    if seed % 2:
        cuts += [cuts[-1]] if cuts else [0]          # an empty partition
        cuts += [min(n, (cuts[-1] + 1))]             # and a one-token one
        cuts.sort()
    bounds = [0] + cuts + [n]
    os_, ls_ = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o_p, l_p = oracle.attend(q, k[a:b], v[a:b], 0.25)
        os_.append(o_p)
        ls_.append(l_p)
    order = rng.permutation(len(os_))                  # the merge is order-free
    o, l = oracle.merge([os_[i] for i in order], [ls_[i] for i in order])
    assert np.max(np.abs(o - full_o)) <= 1e-12
    assert np.max(np.abs(l - full_l)) <= 1e-12


# ---------------------------------------------------------------- 50-digit brute force
@pytest.mark.parametrize("seed", range(4))
def test_bruteforce_50_digits(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 9))
    dk = int(rng.integers(1, 9))
    dv = int(rng.integers(1, 9))
    q, k, v = _rand_qkv(rng, n, 2, 1, dk, dv)
    q *= 3.0
    scale = 0.37
    o, lse = oracle.attend(q, k, v, scale)
    mpmath.mp.dps = 50
    for h in range(2):
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(q[h, i])) * mpmath.mpf(float(k[t, 0, i]))
                                             for i in range(dk)) for t in range(n)]
        e = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(e)
        for j in range(dv):
            want = mpmath.fsum(e[t] * mpmath.mpf(float(v[t, 0, j])) for t in range(n)) / z
            assert abs(float(want) - o[h, j]) <= 1e-13 * max(1.0, abs(float(want)))
        assert abs(float(mpmath.log(z)) - lse[h]) <= 1e-13 * max(1.0, abs(float(mpmath.log(z))))


# ---------------------------------------------------------------- library special case
@pytest.mark.parametrize("shape", [(32, 4, 128, 128, 300), (16, 1, 576, 512, 200), (4, 1, 64, 64, 100)])
def test_matches_torch_sdpa_float64(shape):
    import torch
    hq, hkv, dk, dv, n = shape
    rng = np.random.default_rng(300 + hq)
    q, k, v = _rand_qkv(rng, n, hq, hkv, dk, dv)
    if dk == 576:                      # MLA: the value is the leading 512 latent columns
        v = k[:, :, :dv].copy()
    scale = 1.0 / math.sqrt(192.0 if dk == 576 else dk)
    o, _ = oracle.attend(q, k, v, scale)
    tq = torch.from_numpy(q)[None, :, None, :]                       # [1, Hq, 1, Dk]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]  # [1, Hkv, n, Dk]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, scale=scale, enable_gqa=hkv != hq)[0, :, 0, :].numpy()
    assert np.max(np.abs(ref - o)) <= 1e-12


# ---------------------------------------------------------------- block layout
def _scatter_elementwise(layout, regions, region_blocks, dense_k, dense_v, table_row):
    """Write one sequence's dense K/V into `regions` with the per-element offsets of the
    documented layout (a second, loop-based statement of it; the oracle reads with
    reshapes/transposes).  Values are stored as given (float32, or uint16 bf16 bits)."""
    bs, hkv, dk, dv, x = (layout.block_size, layout.num_kv_heads, layout.head_dim_k,
                          layout.head_dim_v, layout.chunk)
    nel = block_elems(layout)
    starts = np.cumsum([0] + list(region_blocks))
    for t in range(dense_k.shape[0]):
        pid = int(table_row[t // bs])
        r = int(np.searchsorted(starts, pid, side="right") - 1)
        base = (pid - starts[r]) * nel
        tt = t % bs
        for h in range(hkv):
            for i in range(dk):
                if layout.latent:
                    off = ((i // x) * bs + tt) * x + i % x
                else:
                    off = ((h * (dk // x) + i // x) * bs + tt) * x + i % x
                regions[r][base + off] = dense_k[t, h, i]
            if not layout.latent:
                for j in range(dv):
                    regions[r][base + hkv * bs * dk + (h * dv + j) * bs + tt] = dense_v[t, h, j]


def _write_pool_elementwise(layout, dense_k, dense_v, table_row, region_blocks, dtype):
    nel = block_elems(layout)
    # NaN (or NaN bf16 bit patterns) in every slot no token is written to
    fill = np.nan if np.issubdtype(np.dtype(dtype), np.floating) else 0x7FC1
    regions = [np.full(n * nel, fill, dtype) for n in region_blocks]
    _scatter_elementwise(layout, regions, region_blocks, dense_k, dense_v, table_row)
    return regions


@pytest.mark.parametrize("latent", [False, True])
def test_layout_gather_matches_elementwise_writer(latent):
    rng = np.random.default_rng(400 + latent)
    if latent:
        layout = Layout(8, 1, 24, 16, "f32", True)
    else:
        layout = Layout(4, 3, 8, 8, "f32", False)
    n = 29
    nblk = -(-n // layout.block_size)
    region_blocks = [3, nblk + 2]
    perm = rng.permutation(sum(region_blocks))[:nblk]
    dk = rng.standard_normal((n, layout.num_kv_heads, layout.head_dim_k)).astype(np.float32)
    if latent:
        dv = dk[:, :, :layout.head_dim_v]
    else:
        dv = rng.standard_normal((n, layout.num_kv_heads, layout.head_dim_v)).astype(np.float32)
    regions = _write_pool_elementwise(layout, dk, dv, perm, region_blocks, np.float32)
    for lo, hi in [(0, n), (3, 17), (28, 29), (5, 5)]:
        k, v = gather_sequence(layout, regions, region_blocks, perm, lo, hi)
        assert np.array_equal(k, dk[lo:hi].astype(np.float64))
        assert np.array_equal(v, dv[lo:hi].astype(np.float64))


def test_relabelling_physical_blocks_leaves_output_unchanged():
    rng = np.random.default_rng(500)
    layout = Layout(16, 2, 32, 32, "f32", False)
    nel = block_elems(layout)
    nblk, n = 12, 181
    pool = rng.standard_normal(nblk * nel).astype(np.float32)
    table = rng.permutation(nblk)[:12].astype(np.int32)
    q = rng.standard_normal((1, 8, 32)).astype(np.float32)
    o1, l1 = oracle.decode_reference(layout, [pool], [nblk], table[None], [n], q, 0.2)
    # move every block to a new physical slot and rewrite the table accordingly
    new_pos = rng.permutation(nblk)
    moved = np.empty_like(pool)
    for old in range(nblk):
        moved[new_pos[old] * nel:(new_pos[old] + 1) * nel] = pool[old * nel:(old + 1) * nel]
    o2, l2 = oracle.decode_reference(layout, [moved], [nblk], new_pos[table][None], [n], q, 0.2)
    assert np.max(np.abs(o1 - o2)) <= 1e-15 and np.max(np.abs(l1 - l2)) <= 1e-15


# ---------------------------------------------------------------- partitions
def test_partition_ranges_cover_exactly():
    for L in range(0, 70):
        for beg in range(0, L + 1, 3):
            for P in (1, 5, 16, 64):
                rs = oracle.partition_ranges(L, beg, P)
                assert len(rs) == oracle.partition_count(L, beg, P) == math.ceil((L - beg) / P)
                covered = [t for a, b in rs for t in range(a, b)]
                assert covered == list(range(beg, L))
                assert all(0 < b - a <= P for a, b in rs)
    assert oracle.partition_count(5, 6, 4) == -1
    assert oracle.partition_count(5, 0, 0) == -1


# ---------------------------------------------------------------- page-fixed sizes
def test_kv_bytes_per_token_match_page_tables():
    """The synthetic workloads' per-token KV bytes reproduce the pages' KV tables."""
    from synth import make_case
    g = json.load(open(os.path.join(GOLDEN, "kv_footprints.json")))
    # per-token bytes of one layer: MLA latent 576 bf16; GQA K+V of 4 (Qwen3) / 8 (Mixtral)
    # KV heads x 128 dims x bf16 -- taken from the workloads and the oracle's layout
    cases = {"DeepSeek-V2-Lite": make_case("mla_16k"), "Qwen3-30B-A3B": make_case("gqa_32k"),
             "Mixtral-8x7B": make_case("split_128k")}
    for model, case in cases.items():
        lay = Layout(case.block_size, case.num_kv_heads, case.head_dim_k, case.head_dim_v,
                     case.dtype, case.latent)
        per_tok = block_elems(lay) * lay.elem_bytes // lay.block_size
        assert per_tok == case.kv_bytes_per_token()
        layers = g["models"][model]["layers"]
        t1 = g["table1"]
        got = per_tok * layers * t1["tokens"] / t1["unit_bytes"]
        assert round(got, t1["decimals"]) == t1["kv"][model]
        t2 = g["table2"]
        got = per_tok * layers * t2["tokens"] / t2["unit_bytes"]
        assert abs(got - (t2["unpinned"][model] + t2["pinned"][model])) <= 0.011
        assert round(256 * 32 * per_tok * layers / 1e6) == t2["all_layers_256_entries_mb"][model]
        assert abs(1024 * 32 * per_tok / 1e6 - t2["one_layer_1024_entries_mb"][model]) <= 0.06


# ---------------------------------------------------------------- per-partition partials
def _pool_with_dense(layout, lens, region_blocks, rng, unique=False):
    """A pool over two regions holding `len(lens)` sequences written element by element, with
    the dense float64 K/V each sequence holds and its table (entries past the sequence ABSENT).
    With `unique`, every stored element is a distinct value (distinct bit pattern)."""
    bs, hkv, dk, dv = (layout.block_size, layout.num_kv_heads, layout.head_dim_k,
                       layout.head_dim_v)
    nbs = [-(-L // bs) for L in lens]
    max_blocks = max(nbs) + 2
    total = sum(region_blocks)
    ids = rng.permutation(total).astype(np.int32)
    table = np.full((len(lens), max_blocks), oracle.layout.ABSENT, np.int32)
    pos = 0
    for b, nb in enumerate(nbs):
        table[b, :nb] = ids[pos:pos + nb]
        pos += nb
    store = np.uint16 if layout.dtype == "bf16" else np.float32
    nel = block_elems(layout)
    regions = [np.full(n * nel, 0x7FC1 if store == np.uint16 else np.nan, store)
               for n in region_blocks]
    n_k = [L * hkv * dk for L in lens]
    n_v = [0 if layout.latent else L * hkv * dv for L in lens]
    need = sum(n_k) + sum(n_v)
    if layout.dtype == "bf16":
        # distinct finite positive and negative bf16 patterns (exponents 2^-61 .. 2^63)
        pool_bits = np.concatenate([np.arange(0x2100, 0x5F00), np.arange(0xA100, 0xDF00)])
        vals = (rng.choice(pool_bits, need, replace=False) if unique
                else rng.choice(pool_bits, need)).astype(np.uint16)
        widen = oracle.bf16_bits_to_f64
    else:
        vals = rng.standard_normal(need).astype(np.float32)
        if unique:
            assert len(np.unique(vals)) == need
        widen = lambda a: a.astype(np.float64)  # noqa: E731
    dense = []
    off = 0
    for b, L in enumerate(lens):
        k = vals[off:off + n_k[b]].reshape(L, hkv, dk)
        off += n_k[b]
        if layout.latent:
            v = k[:, :, :dv]
        else:
            v = vals[off:off + n_v[b]].reshape(L, hkv, dv)
            off += n_v[b]
        _scatter_elementwise(layout, regions, region_blocks, k, v, table[b])
        dense.append((k, widen(k), widen(v)))
    return regions, table, dense


PARTIAL_LAYOUTS = [Layout(4, 2, 8, 8, "f32", False), Layout(8, 1, 16, 16, "bf16", False),
                   Layout(8, 1, 24, 16, "bf16", True), Layout(4, 1, 32, 16, "f32", True)]


def _check_partials_against_dense(layout, partials, dense, q, scale, lens, begins, parts):
    """Each partition p of sequence b covers [beg + p*P, min(L, beg + (p+1)*P)) and its
    partial is the attention over exactly those dense tokens."""
    for b, (o_b, l_b) in enumerate(partials):
        L, beg, P = lens[b], begins[b], parts[b]
        count = -(-(L - beg) // P)
        assert o_b.shape[0] == count and l_b.shape[0] == count, b
        for p in range(count):
            lo, hi = beg + p * P, min(L, beg + (p + 1) * P)
            o_ref, l_ref = oracle.attend(q[b], dense[b][1][lo:hi], dense[b][2][lo:hi], scale)
            assert np.array_equal(o_b[p], o_ref), (b, p)
            assert np.array_equal(l_b[p], l_ref), (b, p)


@pytest.mark.parametrize("layout", PARTIAL_LAYOUTS,
                         ids=lambda l: f"{l.dtype}-{'mla' if l.latent else 'gqa'}")
def test_partials_are_attention_over_their_token_ranges(layout):
    """decode_partials_reference against attention over element-wise-written dense slices:
    a start inside the context (tok_begin != 0), short last partitions, a one-token range and
    an empty one; the merge of every sequence's partials equals the unsplit attention over
    [tok_begin, L) to 1e-12 ([InplaceKVCache] §5.1: the split is exact)."""
    rng = np.random.default_rng(600 + layout.block_size + 7 * layout.latent)
    bs = layout.block_size
    lens = [5 * bs + 3, 4 * bs, 2 * bs + 1, 3 * bs, 7]
    begins = [bs + 2, 0, 2 * bs, 3 * bs, 7]          # mid-block start, 0, one token, empty
    parts = [2 * bs, bs, bs, 2 * bs, bs]
    regions, table, dense = _pool_with_dense(layout, lens, [6, 40], rng)
    hq = 4 if not layout.latent else 3
    q = rng.standard_normal((len(lens), hq, layout.head_dim_k)).astype(np.float32)
    scale = 0.31
    partials = oracle.decode_partials_reference(layout, regions, [6, 40], table, lens, q, scale,
                                                parts, tok_begin=begins)
    qf = q.astype(np.float64)
    _check_partials_against_dense(layout, partials, dense, qf, scale, lens, begins, parts)
    unsplit = oracle.decode_reference(layout, regions, [6, 40], table, lens, q, scale,
                                      tok_begin=begins)
    for b, (o_b, l_b) in enumerate(partials):
        o_m, l_m = (oracle.merge(list(o_b), list(l_b)) if o_b.shape[0] else
                    (np.zeros_like(unsplit[0][b]), np.full(hq, -np.inf)))
        o_d, l_d = oracle.attend(qf[b], dense[b][1][begins[b]:], dense[b][2][begins[b]:], scale)
        assert np.max(np.abs(o_m - unsplit[0][b])) <= 1e-12
        assert np.max(np.abs(o_m - o_d)) <= 1e-12
        fin = np.isfinite(l_d)
        assert np.array_equal(np.isfinite(l_m), fin) and np.array_equal(np.isfinite(unsplit[1][b]), fin)
        assert np.max(np.abs(l_m[fin] - l_d[fin]), initial=0.0) <= 1e-12


def test_partials_pin_catches_a_dropped_begin():
    """A partial reference that ignored tok_begin (every range starting at 0) fails the pin."""
    layout = PARTIAL_LAYOUTS[0]
    rng = np.random.default_rng(610)
    lens, begins, parts = [23, 17], [5, 4], [8, 4]
    regions, table, dense = _pool_with_dense(layout, lens, [6, 40], rng)
    q = rng.standard_normal((2, 4, layout.head_dim_k)).astype(np.float32)
    wrong = oracle.decode_partials_reference(layout, regions, [6, 40], table, lens, q, 0.5, parts)
    with pytest.raises(AssertionError):
        _check_partials_against_dense(layout, wrong, dense, q.astype(np.float64), 0.5, lens,
                                      begins, parts)


# ---------------------------------------------------------------- address resolution
def _check_resolution(layout, regions, region_blocks, table, lens, dense, max_tokens,
                      resolve=None):
    """Every (b, t) of a resident block resolves to the region and byte offset at which the
    stored element K(h=0, t, 0) (MLA: C(t, 0)) sits; every other (b, t) gives -1 / -1."""
    resolve = resolve or oracle.resolve_offsets_reference
    region, offset = resolve(layout, region_blocks, table, lens, max_tokens)
    starts = np.cumsum([0] + list(region_blocks))
    e = layout.elem_bytes
    for b in range(len(lens)):
        for t in range(max_tokens):
            pid = int(table[b][t // layout.block_size]) if t // layout.block_size < table.shape[1] else -1
            resident = t < lens[b] and 0 <= pid < starts[-1]
            if not resident:
                assert region[b, t] == -1 and offset[b, t] == -1, (b, t)
                continue
            r = int(np.searchsorted(starts, pid, side="right") - 1)
            assert region[b, t] == r, (b, t)
            off = int(offset[b, t])
            assert off % e == 0 and 0 <= off < regions[r].nbytes, (b, t)
            got = regions[r].view(np.uint8)[off:off + e].view(regions[r].dtype)[0]
            want = dense[b][0][t, 0, 0]
            assert got.tobytes() == np.asarray(want, regions[r].dtype).tobytes(), (b, t)


RESOLVE_LAYOUTS = [Layout(4, 2, 8, 8, "f32", False), Layout(4, 3, 16, 16, "bf16", False),
                   Layout(8, 1, 24, 16, "bf16", True), Layout(2, 1, 8, 4, "f32", True),
                   Layout(16, 2, 8, 8, "bf16", False)]


def _resolve_case(layout, seed):
    rng = np.random.default_rng(seed)
    bs = layout.block_size
    lens = [3 * bs + 1, 2 * bs, 1, 4 * bs - 1]
    region_blocks = [5, 9]
    regions, table, dense = _pool_with_dense(layout, lens, region_blocks, rng, unique=True)
    table[3, 1] = oracle.layout.ABSENT               # a hole (not resident on this device)
    table[2, 1] = sum(region_blocks) + 3              # beyond the sequence: never resolved
    table[0, 2] = sum(region_blocks) + 1              # an invalid id inside the context
    max_tokens = table.shape[1] * bs
    return regions, region_blocks, table, lens, dense, max_tokens


@pytest.mark.parametrize("layout", RESOLVE_LAYOUTS,
                         ids=lambda l: f"bs{l.block_size}-{l.dtype}-{'mla' if l.latent else 'gqa'}")
def test_resolved_offsets_point_at_each_tokens_first_key(layout):
    """resolve_offsets_reference (with token_k_offset) over two regions, against an
    element-wise write of distinct values: the element at the returned (region, byte offset)
    is the token's K(h=0, t, 0), for every (b, t); -1 exactly past the context and for ABSENT
    or invalid entries ([CrossPool] §3.1: logical KV address -> physical page)."""
    regions, region_blocks, table, lens, dense, max_tokens = _resolve_case(layout, 620)
    _check_resolution(layout, regions, region_blocks, table, lens, dense, max_tokens)


@pytest.mark.parametrize("layout", RESOLVE_LAYOUTS[:3],
                         ids=lambda l: f"{l.dtype}-{'mla' if l.latent else 'gqa'}")
def test_resolution_pin_catches_a_wrong_token_offset(layout, monkeypatch):
    """With token_k_offset planted as t * Dk (tokens contiguous in K), the pin fails."""
    import oracle.decode as od
    regions, region_blocks, table, lens, dense, max_tokens = _resolve_case(layout, 621)
    monkeypatch.setattr(od, "token_k_offset", lambda lay, t: t * lay.head_dim_k)
    with pytest.raises(AssertionError):
        _check_resolution(layout, regions, region_blocks, table, lens, dense, max_tokens)
