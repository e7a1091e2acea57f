"""The native CPU share (kvattn_host_partial) against the float64 oracle.

Host code, so these run without a GPU.  Tolerances are those of the device path: fp32
caches max |o - o_ref| <= 1e-5 (lse likewise); bf16 caches max |o - o_ref| / max |o_ref| <=
2e-3 and lse within 2e-3.  The chunk partials are merged in a fixed order, so the result
must not depend on the thread count (bitwise).
"""

import numpy as np
import pytest

import oracle
from paged_kv_cache_mla_amd import _lib
from paged_kv_cache_mla_amd.api import KvattnError, host_partial
from synth import make_case
from tests import oracle_cases as oc


def _run(case, regions, region_blocks, table, tok_end, threads=0):
    return host_partial(case.block_size, case.num_kv_heads, case.head_dim_k, case.head_dim_v,
                        case.dtype, case.latent, regions, case.q, case.num_q_heads, case.scale,
                        table, tok_end, n_threads=threads)


@pytest.mark.parametrize("name", ["tiny_fp32", "gqa_32k", "prefix_shared", "mla_16k"])
def test_host_partial_over_whole_context_matches_oracle(name):
    case = make_case(name, "small")
    o, lse = _run(case, case.regions, case.region_blocks, case.table, case.ctx_lens)
    o_ref, lse_ref = oracle.decode_reference(oc.layout_of(case), case.regions, case.region_blocks,
                                             case.table, case.ctx_lens, case.q, case.scale)
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)


def test_host_partial_of_split_share_matches_oracle():
    """The split workload's host-side share [0, tok_begin) -- the partial the GPU merges."""
    case = make_case("split_128k", "small")
    o, lse = _run(case, case.ext_regions, case.ext_region_blocks, case.ext_table, case.tok_begin)
    o_ref, lse_ref = oc.external_partial(case)
    assert oc.out_error(case, o, o_ref) <= oc.out_tol(case)
    assert float(np.max(np.abs(lse - lse_ref))) <= oc.lse_tol(case)


def test_host_partial_prefix_lengths_and_empty_range():
    """Ragged token ends (mid-block, one token, zero tokens) over the same blocks."""
    case = make_case("gqa_32k", "small")
    ends = np.array([1, 17, 0, 599], np.int32)
    o, lse = _run(case, case.regions, case.region_blocks, case.table, ends)
    for b in range(case.batch):
        if ends[b] == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        k, v = oracle.gather_sequence(oc.layout_of(case), case.regions, case.region_blocks,
                                      case.table[b], 0, int(ends[b]))
        o_ref, lse_ref = oracle.attend(oc.q_f64(case)[b], k, v, case.scale)
        assert np.max(np.abs(o[b] - o_ref)) / np.max(np.abs(o_ref)) <= 2e-3
        assert np.max(np.abs(lse[b] - lse_ref)) <= 2e-3
    # one token: the value itself (bf16 widened exactly, weight 1)
    k, v = oracle.gather_sequence(oc.layout_of(case), case.regions, case.region_blocks,
                                  case.table[0], 0, 1)
    g = case.num_q_heads // case.num_kv_heads
    for h in range(case.num_q_heads):
        assert np.array_equal(o[0, h].astype(np.float64), v[0, h // g])


@pytest.mark.parametrize("name", ["gqa_32k", "mla_16k"])
def test_host_partial_independent_of_thread_count(name):
    case = make_case(name, "small")
    o1, l1 = _run(case, case.regions, case.region_blocks, case.table, case.ctx_lens, threads=1)
    o7, l7 = _run(case, case.regions, case.region_blocks, case.table, case.ctx_lens, threads=7)
    assert np.array_equal(o1, o7) and np.array_equal(l1, l7)


def test_host_partial_validation():
    case = make_case("gqa_32k", "small")
    bad = case.table.copy()
    bad[1, 2] = sum(case.region_blocks) + 3
    with pytest.raises(KvattnError) as e:
        _run(case, case.regions, case.region_blocks, bad, case.ctx_lens)
    assert e.value.status == _lib.E_RANGE
    with pytest.raises(KvattnError) as e:
        _run(case, case.regions, case.region_blocks, case.table,
             np.array([case.max_blocks * case.block_size + 1, 1, 1, 1], np.int32))
    assert e.value.status == _lib.E_INVAL


def test_host_partial_repeated_calls_changing_thread_counts_and_concurrent_callers():
    """The persistent workers: back-to-back calls with growing and shrinking worker counts, and
    two caller threads at once (calls are serialised inside the library), all give the same
    bits."""
    import threading

    case = make_case("split_128k", "small")
    ref = _run(case, case.ext_regions, case.ext_region_blocks, case.ext_table, case.tok_begin, 1)
    counts = [1, 7, 3, 12, 2, 8, 1, 16, 5] * 12
    for th in counts:
        o, lse = _run(case, case.ext_regions, case.ext_region_blocks, case.ext_table,
                      case.tok_begin, th)
        assert np.array_equal(o, ref[0]) and np.array_equal(lse, ref[1])
    bad = []

    def caller(seed):
        rng = np.random.default_rng(seed)
        for _ in range(40):
            o, lse = _run(case, case.ext_regions, case.ext_region_blocks, case.ext_table,
                          case.tok_begin, int(rng.integers(1, 9)))
            if not (np.array_equal(o, ref[0]) and np.array_equal(lse, ref[1])):
                bad.append(seed)

    ts = [threading.Thread(target=caller, args=(s,)) for s in (1, 2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad
